/*
 * kvq.h - C ABI of libkvq: entropy-coded KV-cache quantisation for AMD MI355X
 * (gfx950).  Write side: per-token key/value streams are Hadamard-rotated,
 * keys lose a windowed channel mean, every stream gets one affine grid
 * (scale, offset), symbols are assigned under a rate budget ("drift") and
 * rANS-coded into a container of exactly C bytes.  Read side: a fused kernel
 * decodes the containers at fixed stride and computes softmax(q K^T) V.
 *
 * The method is the one of "D-Quant: Driftable Entropy Coding for KV Cache
 * Quantization" (arXiv 2609.19880), cited below as [D-Quant].
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned and allocated by the caller
 *    (e.g. torch tensors' data_ptr()); all must be 16-byte aligned, else
 *    KVQ_EINVAL.  Scalars and small out-arrays are host memory.
 *  - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *    the default stream).  Argument errors return synchronously with nothing
 *    launched; a failed launch returns KVQ_EDEVICE; faults inside kernels
 *    surface at the caller's next synchronisation.
 *  - The library allocates no device memory on the encode/decode path; a
 *    plan owns only host-side tables.  There is no global error state.
 *  - Inputs must be finite; NaN/Inf input is undefined behaviour.
 *  - Layouts are row-major.  A "stream" is one token of one sequence:
 *    n = n_kv_heads * head_dim values ordered [kv_head][dim].  A "sequence"
 *    is one (layer, batch) cache; layers fold into the sequence count.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_EINVAL = -1,        /* bad argument, shape or alignment              */
  KVQ_EINFEASIBLE = -2,   /* container too small for n cheapest symbols    */
  KVQ_EUNSUPPORTED = -3,  /* valid but not implemented (e.g. head_dim)     */
  KVQ_EDEVICE = -4,       /* a HIP call or kernel launch failed            */
  KVQ_ENOMEM = -5,        /* host allocation failed                        */
  KVQ_EWORKSPACE = -6     /* workspace smaller than kvq_workspace_bytes()  */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* How a cache array stores the containers of one side (container_layout).
 * Either way a stream's container is the same C bytes ([D-Quant] §4.2 Eq. 3):
 * the 4-byte little-endian final state, the payload the decoder reads
 * forwards, zero padding.
 *   KVQ_LAYOUT_ROWS   [n_seqs, capacity, C]: token t of sequence s at byte
 *                     (s capacity + t) C, each container one row.
 *   KVQ_LAYOUT_TILES  [n_seqs, capacity64, Cp]: capacity64 = capacity rounded
 *                     up to a multiple of 64, Cp = C rounded up to a multiple
 *                     of 4 (the extra bytes are zero).  Flat token
 *                     g = s capacity64 + t: byte j of its container lies at
 *                     (g / 64) 64 Cp + (j / 4) 256 + (g mod 64) 4 + j mod 4,
 *                     i.e. dword k of the 64 containers of a tile side by
 *                     side, so that a wave reading dword k of 64 consecutive
 *                     tokens reads 256 contiguous bytes.  Decode attention
 *                     with 9-level V alphabets and the fixed-width
 *                     comparator take the row layout only. */
typedef enum { KVQ_LAYOUT_ROWS = 0, KVQ_LAYOUT_TILES = 1 } kvq_layout;

/* Configuration of one cache format ([D-Quant] §4.2, §4.4, §5.1: container
 * bytes, number of levels and the K/V split are free parameters; the page's
 * default is 331/231 bytes, 8/6 levels, alpha = 1.4, 2.26 bits per value). */
typedef struct {
  int32_t n_kv_heads;         /* Hkv >= 1                                     */
  int32_t head_dim;           /* d: power of two, 32..256                     */
  int32_t levels_k;           /* M_K in [2, 16]                               */
  int32_t levels_v;           /* M_V in [2, 16]                               */
  int32_t container_bytes_k;  /* C_K > 4 (4 bytes hold the final rANS state)  */
  int32_t container_bytes_v;  /* C_V > 4                                      */
  int32_t mean_window;        /* W: power of two; tokens per key-mean window  */
  double sharpen_alpha;       /* alpha >= 1; probabilities p^alpha ([D-Quant] §4.4) */
  int32_t container_layout;   /* kvq_layout of the cache arrays (0: rows)     */
} kvq_params;

/* Immutable plan: the integer rANS tables derived from the Gaussian
 * order-statistics model ([D-Quant] §4.2), the fixed-point rate tables and
 * the lambda grid of the drift solver (Appendix A, Algorithm 1).  Pure host
 * object; safe to share between threads. */
typedef struct kvq_plan kvq_plan;

/* Builds a plan.  Returns KVQ_EINVAL for out-of-range params,
 * KVQ_EINFEASIBLE if n * min_m r(m) exceeds 8C - 32 bits for K or V (Eq. 3:
 * even the cheapest symbol everywhere would not fit), KVQ_ENOMEM. */
kvq_status kvq_plan_create(const kvq_params* params, kvq_plan** out_plan);
void kvq_plan_destroy(kvq_plan* plan);

/* As kvq_plan_create, with non-affine reconstruction levels ([D-Quant]
 * Appendix A: a table entry carries the level v_m; Eqs. (7)-(9) hold for any
 * v_m).  values_k / values_v (nullable: v_m = m) hold levels_k / levels_v
 * levels in grid units; they are rounded to fp16, which is what is stored,
 * and must then rise strictly from 0 to levels - 1 (KVQ_EINVAL otherwise), so
 * the min-max fit of Eq. 4 is unchanged.  Nearest rounding, drift and the
 * least-squares refit use rec_m = o + s v_m, and the probability model's cells
 * are bounded by the midpoints of adjacent levels (symmetrised only for
 * symmetric levels).  Decode attention accepts non-affine plans when both
 * alphabets have at most 16 (keys) and 8 (values) levels; the fixed-width
 * comparator needs affine levels. */
kvq_status kvq_plan_create_levels(const kvq_params* params, const float* values_k,
                                  const float* values_v, kvq_plan** out_plan);

/* Copies one side's level values v_m as stored (16 floats; zero past levels). */
kvq_status kvq_plan_levels(const kvq_plan* plan, int side, float* values);

/* Copies one side's tables (side 0 = keys, 1 = values) to host arrays of at
 * least 16 entries: frequencies f_m (sum 256), cumulative c_m and the rates
 * r_fx[m] = rne((8 - log2 f_m) * 2^16).  Entries >= levels are zero. */
kvq_status kvq_plan_tables(const kvq_plan* plan, int side, uint16_t* freq,
                           uint16_t* cum, int32_t* rate_fx);

/* The probability model itself ([D-Quant] §4.2, §4.4): expected fraction of
 * each of `levels` symbols when n iid N(0,1) values are min-max normalised and
 * rounded to the nearest level, raised to alpha and renormalised (alpha = 1:
 * the plain model).  Writes `levels` doubles.  KVQ_EINVAL out of range. */
kvq_status kvq_model_probs(int32_t levels, int32_t n, double alpha, double* probs);

/* Copies the 512-entry lambda grid E[k] = fp32(2^(k/512)) to host memory. */
kvq_status kvq_plan_lambda_grid(const kvq_plan* plan, float* grid512);

/* Storage cost in bits per value ([D-Quant] §3.1: symbols and metadata).
 * metadata != 0 counts, per token-layer, two fp16 (scale, offset) pairs and
 * the INT8 key mean of n values plus its fp16 scale per W tokens:
 * 8 (C_K + C_V + 8 + (n + 2) / W) / (2 n).  metadata == 0: containers only.
 * With KVQ_LAYOUT_TILES the containers count at their stored size (C rounded
 * up to a multiple of 4). */
double kvq_bits_per_elem(const kvq_params* params, int metadata);

/* Container sizes for a budget in bits per value (metadata included):
 * total = floor(bpe 2n/8 - 8 - (n+2)/W) bytes split 331:562 between K and V
 * (the page's default split, §5.1), so 2.26 gives 331/231. */
kvq_status kvq_containers_for_budget(double bits_per_elem, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t mean_window,
                                     int32_t* c_k, int32_t* c_v);

/* Device workspace needed by kvq_decode_attention / kvq_decode_attention_ex
 * (op = 1) for n_seqs sequences of seq_len compressed tokens (seq_len >= 0;
 * the size also covers an uncompressed tail); op = 0 (encode) needs none and
 * reports 0. */
kvq_status kvq_workspace_bytes(const kvq_plan* plan, int op, int64_t n_seqs,
                               int64_t seq_len, int32_t n_q_heads, size_t* bytes);

/* Write side ([D-Quant] Figure 1, §4.2-§4.3, Appendix A Algorithm 1).
 *   k, v          [n_seqs, seq_len, Hkv, d] in `in_dtype` (fp32 or bf16)
 *   k_cont, v_cont out [n_seqs, seq_len, C_K] / [.., C_V] bytes in the plan's
 *                 container_layout (KVQ_LAYOUT_TILES: [n_seqs, seq_len rounded
 *                 up to 64, C rounded up to 4]); every container is exactly C
 *                 bytes: 4-byte little-endian final state, payload (read
 *                 forwards by the decoder), zero padding
 *   k_so, v_so    out [n_seqs, seq_len, 2] fp16 bits: (scale, offset)
 *   k_mean_q      out [n_seqs, seq_len/W, n] int8 key channel means
 *   k_mean_scale  out [n_seqs, seq_len/W] fp16 bits
 *   stats         nullable device uint64[8], ACCUMULATED (caller zeroes it):
 *                 [0] K streams whose first drift fell back to the cheapest
 *                 symbol, [1] same for the second drift, [2] K symbols that
 *                 differ from nearest rounding on the final grid, [3] K
 *                 streams that overran their container (always 0), [4..7] the
 *                 same for V.
 * seq_len must be a positive multiple of W.  Returns KVQ_EUNSUPPORTED unless
 * n = Hkv d is 64 times a power of two (64 .. 4096) and W >= 4.  Output is
 * deterministic and independent of launch geometry. */
kvq_status kvq_encode_streams(const kvq_plan* plan, const void* k, const void* v,
                              kvq_dtype in_dtype, int64_t n_seqs, int64_t seq_len,
                              uint8_t* k_cont, uint8_t* v_cont,
                              uint16_t* k_so, uint16_t* v_so,
                              int8_t* k_mean_q, uint16_t* k_mean_scale,
                              uint64_t* stats, void* hip_stream);

/* Streaming append ([D-Quant] §5.1 "Implementation details": the most recent
 * tokens stay uncompressed in bf16 and are compressed a window at a time).
 * Encodes n_tokens tokens per sequence, k, v [n_seqs, n_tokens, Hkv, d], into
 * rows [token_offset, token_offset + n_tokens) of cache arrays that hold
 * cache_capacity tokens per sequence (k_cont [n_seqs, cache_capacity, C_K],
 * k_mean_q [n_seqs, cache_capacity / W, n], ...); other rows are untouched.
 * n_tokens, token_offset and cache_capacity must be multiples of W
 * (KVQ_EINVAL otherwise, and for token_offset + n_tokens > cache_capacity).
 * Every key-mean window lies inside the appended tokens, so appending a
 * sequence window by window writes exactly the bytes kvq_encode_streams
 * writes for the whole sequence.  stats as for kvq_encode_streams. */
kvq_status kvq_encode_append(const kvq_plan* plan, const void* k, const void* v,
                             kvq_dtype in_dtype, int64_t n_seqs, int64_t n_tokens,
                             int64_t cache_capacity, int64_t token_offset,
                             uint8_t* k_cont, uint8_t* v_cont,
                             uint16_t* k_so, uint16_t* v_so,
                             int8_t* k_mean_q, uint16_t* k_mean_scale,
                             uint64_t* stats, void* hip_stream);

/* Read side ([D-Quant] §4.5 "Decoding", Appendix A Algorithm 2 and
 * Eqs. (7)-(9)): one decode query per sequence attends over all seq_len
 * cached tokens; query head h reads KV head h / (Hq / Hkv).
 *   q             [n_seqs, Hq, d] bf16
 *   k_cont ...    as written by kvq_encode_streams
 *   softmax_scale <= 0 selects 1/sqrt(d)
 *   out           [n_seqs, Hq, d] bf16 (round-to-nearest-even of out_f32)
 *   out_f32       nullable [n_seqs, Hq, d] fp32
 *   workspace     device memory of at least kvq_workspace_bytes(plan, 1, ...)
 * Results are deterministic for a given shape.  Returns KVQ_EUNSUPPORTED
 * unless d = 128, Hkv and Hq / Hkv are in {1, 2, 4, 8}, both alphabets have at
 * most 9 levels, W >= 64, seq_len is a multiple of 64, n_seqs <= 65535 and
 * seq_len * max(C_K, C_V) + 16 <= 2^31 - 1; KVQ_EWORKSPACE if the workspace
 * is too small.  Nothing is launched when an error is returned. */
kvq_status kvq_decode_attention(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                const uint8_t* k_cont, const uint8_t* v_cont,
                                const uint16_t* k_so, const uint16_t* v_so,
                                const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                void* out, float* out_f32,
                                void* workspace, size_t workspace_bytes,
                                void* hip_stream);

/* kvq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, whose role is taken
 * by a library-owned scratch array of KVQ_NOALLOC_SCRATCH_BYTES per GPU (a
 * static device array, held by every GPU the library runs on until the process
 * ends; its address is looked up once per device on the first call there).
 * The call allocates nothing and its kernels are those of kvq_decode_attention,
 * so results are identical.  Returns KVQ_EWORKSPACE, launching nothing, when
 * kvq_workspace_bytes(plan, 1, n_seqs, seq_len, n_q_heads) exceeds
 * KVQ_NOALLOC_SCRATCH_BYTES (72 MiB covers, for example, 512 sequences of 8192
 * tokens at 32/8 heads, or one of 131072 tokens at 64/8 heads), and KVQ_EDEVICE
 * if the array's address cannot be obtained.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  Nothing needs clearing between calls
 * (every byte read was written earlier in the same call). */
#define KVQ_NOALLOC_SCRATCH_BYTES (72ull << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                        const uint8_t* k_cont, const uint8_t* v_cont,
                                        const uint16_t* k_so, const uint16_t* v_so,
                                        const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                        int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                        void* out, float* out_f32, void* hip_stream);

/* Decode attention over a compressed prefix and an uncompressed bf16 tail
 * ([D-Quant] §5.1 "Implementation details": the most recent tokens are kept in
 * BF16; both parts join one softmax).  The query attends over
 *   * rows [0, n_tokens) of cache arrays holding cache_capacity tokens per
 *     sequence (n_tokens a multiple of W and of 64; may be 0, and then the
 *     cache pointers may be NULL), and
 *   * rows [0, res_len) of res_k, res_v [n_seqs, res_capacity, Hkv, d] bf16
 *     (res_len may be 0, and then res_k / res_v may be NULL),
 * with n_tokens + res_len >= 1.  The workspace is
 * kvq_workspace_bytes(plan, 1, n_seqs, n_tokens, n_q_heads).  Other arguments
 * and errors as for kvq_decode_attention, which is this call with
 * cache_capacity = n_tokens = seq_len and res_len = 0. */
kvq_status kvq_decode_attention_ex(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                   const uint8_t* k_cont, const uint8_t* v_cont,
                                   const uint16_t* k_so, const uint16_t* v_so,
                                   const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                   int64_t n_seqs, int64_t cache_capacity, int64_t n_tokens,
                                   const void* res_k, const void* res_v,
                                   int64_t res_capacity, int64_t res_len,
                                   float softmax_scale, void* out, float* out_f32,
                                   void* workspace, size_t workspace_bytes,
                                   void* hip_stream);

/* Fixed-width comparator ([D-Quant] Appendix B: same preprocessing, symbols
 * by nearest-level rounding instead of drift, no entropy coding).  Each symbol
 * takes b bits, b the smallest of 1, 2, 4, 8 with 2^b >= levels (the page
 * charges the ideal log2 M bits; no fixed width can hold every symbol in
 * that), so a stream is n b / 8 bytes: symbol i = 4c + r sits in byte r of
 * little-endian dword c / (8/b), bits b (c mod 8/b) .. + b.
 * kvq_fixed_width_container_bytes gives n b / 8 (KVQ_EINVAL unless n b is a
 * multiple of 32). */
kvq_status kvq_fixed_width_container_bytes(int32_t levels, int32_t n, int32_t* bytes);

/* Encodes like kvq_encode_streams (same tensors and layout) in the
 * fixed-width format; the plan's container sizes must equal the fixed-width
 * sizes of its alphabets (KVQ_EINVAL otherwise), e.g. 6/3 levels -> 512/256
 * bytes for n = 1024.  KVQ_EUNSUPPORTED unless n >= 1024 and (n/64) b is a
 * multiple of 32.  The plan's rANS tables are not used. */
kvq_status kvq_encode_fixed_width(const kvq_plan* plan, const void* k, const void* v,
                                  kvq_dtype in_dtype, int64_t n_seqs, int64_t seq_len,
                                  uint8_t* k_cont, uint8_t* v_cont,
                                  uint16_t* k_so, uint16_t* v_so,
                                  int8_t* k_mean_q, uint16_t* k_mean_scale,
                                  void* hip_stream);

/* Fused decode attention over fixed-width containers: arguments, workspace
 * and output as kvq_decode_attention.  KVQ_EUNSUPPORTED unless d = 128, Hkv
 * and Hq / Hkv are in {1, 2, 4, 8}, both alphabets have at most 8 levels,
 * (b_K, b_V) is (4, 2), (4, 4), (2, 2) or (2, 1), W >= 64 and seq_len is a
 * multiple of 64. */
kvq_status kvq_decode_attention_fixed_width(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                            const uint8_t* k_cont, const uint8_t* v_cont,
                                            const uint16_t* k_so, const uint16_t* v_so,
                                            const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                            int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                            void* out, float* out_f32,
                                            void* workspace, size_t workspace_bytes,
                                            void* hip_stream);

/* Decodes containers back to symbol indices (Appendix A, Algorithm 2); a
 * verification helper.  side 0 = K table, 1 = V table.
 *   cont      [n_streams, C] bytes in the plan's container_layout (with
 *             KVQ_LAYOUT_TILES, n_streams flat tokens of whole 64-token tiles,
 *             i.e. n_seqs times the padded capacity);
 *             symbols out [n_streams, n] uint8
 *   end_ok    nullable out [n_streams] uint32: 1 if the final state equals
 *             2^23 (a well-formed stream ends where the encoder started). */
kvq_status kvq_decode_symbols(const kvq_plan* plan, int side, const uint8_t* cont,
                              int64_t n_streams, uint8_t* symbols, uint32_t* end_ok,
                              void* hip_stream);

/* Diagnostics: per-kernel timing of the fused decode-attention kernel.
 * While enabled, every kvq_decode_attention call records a pair of HIP events
 * on its stream around that one kernel (the events are created on first use
 * and reused; up to 4096 launches are held between collects, later launches
 * are not timed).  kvq_timing_collect waits for the recorded events, returns
 * the summed milliseconds and the number of timed launches since the previous
 * collect, and clears them.  Not thread-safe; timing off by default. */
kvq_status kvq_timing_enable(int on);
kvq_status kvq_timing_collect(double* total_ms, int64_t* launches);

/* Static description of a status code. */
const char* kvq_status_str(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
