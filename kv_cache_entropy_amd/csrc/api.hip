// C ABI entry points that launch device work (the host-only entry points are
// in plan.cpp).  Argument checking happens here, before anything is enqueued.

#include <mutex>
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <climits>
#include <cstring>
#include <vector>

#include "device_common.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

// Split-K geometry of the decode attention: 64-token tiles; enough splits to
// give the chip about 2048 waves (each split is one wave).
// one_tile: every split holds one 64-token tile (the fused kernel for 8 query
// heads on more than 2 KV heads writes each head's partial output right after
// its tile, so it needs splits of one tile).
void split_geometry(int64_t S, int64_t T, int* nsplit, int64_t* tokens_per_split, bool one_tile = false) {
  const int64_t tiles = T / 64;
  if (tiles == 0) {
    *nsplit = 0;
    *tokens_per_split = 0;
    return;
  }
  if (one_tile) {
    *tokens_per_split = 64;
    *nsplit = int(tiles);
    return;
  }
  int64_t want = (2048 + S - 1) / S;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  const int64_t tiles_per = (tiles + want - 1) / want;
  *tokens_per_split = tiles_per * 64;
  *nsplit = int((tiles + tiles_per - 1) / tiles_per);
}

struct WsLayout {
  size_t qop, qscale, qsum, qmu, part, total;
};

// Decode-attention workspace: the fp16 query operand (hi + lo, 16 bytes per
// 4 channels of a query slot; slots padded to a multiple of 4 per KV head),
// per-head scale, sum and per-window mean terms, and the split partials.
bool one_tile_splits(int G, int hkv) { return G == 8 && hkv > 2; }

WsLayout ws_layout(const kvq_plan* plan, int64_t S, int64_t T, int Hq) {
  int nsplit;
  int64_t tps;
  const int d = plan->params.head_dim;
  const int hkv = plan->params.n_kv_heads;
  const int G = Hq / hkv > 0 ? Hq / hkv : 1;
  split_geometry(S, T, &nsplit, &tps, one_tile_splits(G, hkv));
  const int slots = ((G + 3) / 4) * 4;
  const int64_t nW = T / plan->params.mean_window;
  WsLayout w;
  w.qop = 0;
  w.qscale = round256(w.qop + size_t(S) * hkv * slots * (d / 4) * 16);
  w.qsum = round256(w.qscale + size_t(S) * Hq * 4);
  w.qmu = round256(w.qsum + size_t(S) * Hq * 4);
  w.part = round256(w.qmu + size_t(S) * Hq * nW * 4);
  // one more split per sequence holds the partials of an uncompressed residual
  w.total = round256(w.part + size_t(S) * (nsplit + 1) * Hq * (d + 4) * 4);
  return w;
}

kvq::EncTabs enc_tabs(const kvq_plan* plan, int side) {
  const kvq::SideTables& t = plan->side[side];
  kvq::EncTabs e;
  std::memset(&e, 0, sizeof(e));
  for (int m = 0; m < kvq::kMaxLevels; ++m) {
    e.rate_fx[m] = t.rate_fx[m];
    e.freq[m] = t.freq[m];
    e.cum[m] = t.cum[m];
    e.rcp[m] = t.rcp[m];
    e.rshift[m] = t.rshift[m];
    e.level[m] = t.level[m];
  }
  std::memcpy(e.lambda, plan->lambda_grid, sizeof(e.lambda));
  e.levels = t.levels;
  e.container_bytes = t.container_bytes;
  e.cheapest = t.cheapest;
  e.budget_fx = t.budget_fx;
  return e;
}

// Bits per symbol of the fixed-width comparator: the smallest of 1, 2, 4, 8
// that holds `levels` symbols (0 if none does).
int fw_bits(int levels) {
  for (int b = 1; b <= 8; b <<= 1)
    if ((1 << b) >= levels) return b;
  return 0;
}

// Streams per encode workgroup: the largest of 32/16/8/4 that divides the
// tokens per sequence (a workgroup's streams then lie in one sequence) and
// keeps the symbol and container staging under 56 KiB.
// Streams per encode workgroup: as many as fit (symbols staged at 4 bits,
// plus the container image) in 56 KiB of LDS, up to one per lane of a wave,
// since one lane per stream runs the rANS phase.
// Bytes a container of C bytes occupies in the cache, and a sequence's cache
// bytes, in the plan's layout (tiles: C rounded up to 4 bytes, the capacity
// to 64 tokens).
bool tiles(const kvq_params& P) { return P.container_layout == KVQ_LAYOUT_TILES; }
int stored_bytes(const kvq_params& P, int C) { return tiles(P) ? (C + 3) / 4 * 4 : C; }
int64_t seq_bytes(const kvq_params& P, int C, int64_t capacity) {
  return tiles(P) ? (capacity + 63) / 64 * 64 * stored_bytes(P, C) : capacity * C;
}

int pick_spw(int64_t tokens, int n, int C) {
  for (int spw = 64; spw >= 4; spw >>= 1)
    if (tokens % spw == 0 && size_t(spw) * (size_t(n) / 2 + size_t(C)) <= 56u * 1024u) return spw;
  return 0;
}

// Opt-in event timing of the fused attention kernel (diagnostics only).
struct KernelTimer {
  bool on = false;
  std::vector<hipEvent_t> start, stop;
  size_t used = 0;
  static constexpr size_t kMax = 4096;
};
KernelTimer g_timer;

bool timer_begin(hipStream_t stream, size_t* slot) {
  if (!g_timer.on || g_timer.used >= KernelTimer::kMax) return false;
  if (g_timer.used == g_timer.start.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return false;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return false;
    }
    g_timer.start.push_back(a);
    g_timer.stop.push_back(b);
  }
  *slot = g_timer.used;
  return hipEventRecord(g_timer.start[*slot], stream) == hipSuccess;
}

void timer_end(hipStream_t stream, size_t slot) {
  if (hipEventRecord(g_timer.stop[slot], stream) == hipSuccess) g_timer.used = slot + 1;
}

}  // namespace

extern "C" {

kvq_status kvq_timing_enable(int on) {
  g_timer.on = on != 0;
  return KVQ_OK;
}

kvq_status kvq_timing_collect(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return KVQ_EINVAL;
  double tot = 0.0;
  for (size_t i = 0; i < g_timer.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_timer.stop[i]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]) != hipSuccess)
      return KVQ_EDEVICE;
    tot += ms;
  }
  *total_ms = tot;
  *launches = int64_t(g_timer.used);
  g_timer.used = 0;
  return KVQ_OK;
}

kvq_status kvq_workspace_bytes(const kvq_plan* plan, int op, int64_t n_seqs, int64_t seq_len,
                               int32_t n_q_heads, size_t* bytes) {
  if (!plan || !bytes || n_seqs < 1 || seq_len < 0) return KVQ_EINVAL;
  if (op == 0) {
    *bytes = 0;
    return KVQ_OK;
  }
  if (op != 1 || n_q_heads < 1) return KVQ_EINVAL;
  *bytes = ws_layout(plan, n_seqs, seq_len, n_q_heads).total;
  return KVQ_OK;
}

}  // extern "C"

namespace {

// Encodes n_tokens tokens per sequence (k, v: [S, n_tokens, Hkv, d]) into
// cache rows [t_off, t_off + n_tokens) of arrays holding `capacity` tokens per
// sequence.  Every key-mean window is local to the tokens encoded with it.
kvq_status encode_impl(const kvq_plan* plan, const void* k, const void* v, kvq_dtype in_dtype,
                       int64_t n_seqs, int64_t n_tokens, int64_t capacity, int64_t t_off,
                       uint8_t* k_cont, uint8_t* v_cont, uint16_t* k_so, uint16_t* v_so,
                       int8_t* k_mean_q, uint16_t* k_mean_scale, uint64_t* stats, void* hip_stream,
                       bool fixed_width = false) {
  if (!plan || !k || !v || !k_cont || !v_cont || !k_so || !v_so || !k_mean_q || !k_mean_scale)
    return KVQ_EINVAL;
  if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return KVQ_EINVAL;
  const void* ptrs[] = {k, v, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale};
  for (const void* p : ptrs)
    if (!aligned16(p)) return KVQ_EINVAL;
  if (stats && (reinterpret_cast<uintptr_t>(stats) & 7u)) return KVQ_EINVAL;
  const kvq_params& P = plan->params;
  const int n = plan->n;
  const int W = P.mean_window;
  if (n_seqs < 1 || n_tokens < W || n_tokens % W) return KVQ_EINVAL;
  if (t_off < 0 || t_off % W || capacity % W || t_off + n_tokens > capacity) return KVQ_EINVAL;
  // one encoder instantiation per stream length: n = 64 * 2^k up to 4096
  if (n % 64 || n > 4096 || ((n / 64) & (n / 64 - 1)) || W < 4) return KVQ_EUNSUPPORTED;
  int fwb[2] = {0, 0};
  if (fixed_width) {
    if (!plan->side[0].affine || !plan->side[1].affine || tiles(P)) return KVQ_EUNSUPPORTED;
    fwb[0] = fw_bits(P.levels_k);
    fwb[1] = fw_bits(P.levels_v);
    for (int side = 0; side < 2; ++side) {
      const int C = side == 0 ? P.container_bytes_k : P.container_bytes_v;
      if (C != n * fwb[side] / 8) return KVQ_EINVAL;            // not the fixed-width size
      if (((n / 64) * fwb[side]) % 32 || n / 64 < 16) return KVQ_EUNSUPPORTED;
    }
  }
  const int64_t n_streams = n_seqs * n_tokens;
  const int spw_k = pick_spw(n_tokens, n, stored_bytes(P, P.container_bytes_k));
  const int spw_v = pick_spw(n_tokens, n, stored_bytes(P, P.container_bytes_v));
  if (!spw_k || !spw_v) return KVQ_EUNSUPPORTED;
  if (n_streams / 4 > int64_t(0x7FFFFFFF)) return KVQ_EUNSUPPORTED;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);

  kvq::KeyMeanArgs km;
  km.k = k;
  km.in_bf16 = in_dtype == KVQ_BF16;
  km.mean_q = k_mean_q;
  km.mean_scale = k_mean_scale;
  km.T = n_tokens;
  km.T_cap = capacity;
  km.t_off = t_off;
  km.W = W;
  km.n = n;
  km.d = P.head_dim;
  km.hscale = plan->hadamard_scale;
  if (kvq::launch_key_mean(km, n_seqs * (n_tokens / W), stream) != hipSuccess) return KVQ_EDEVICE;

  for (int side = 0; side < 2; ++side) {
    kvq::EncodeArgs ea;
    std::memset(&ea, 0, sizeof(ea));
    ea.x = side == 0 ? k : v;
    ea.in_bf16 = in_dtype == KVQ_BF16;
    ea.is_key = side == 0;
    ea.mean_q = k_mean_q;
    ea.mean_scale = k_mean_scale;
    ea.cont = side == 0 ? k_cont : v_cont;
    ea.so = side == 0 ? k_so : v_so;
    ea.stats = stats ? reinterpret_cast<unsigned long long*>(stats) + 4 * side : nullptr;
    ea.T = n_tokens;
    ea.T_cap = capacity;
    ea.t_off = t_off;
    ea.W = W;
    ea.n = n;
    ea.d = P.head_dim;
    ea.hscale = plan->hadamard_scale;
    ea.spw = side == 0 ? spw_k : spw_v;
    ea.fw_bits = fwb[side];
    const int C = side == 0 ? P.container_bytes_k : P.container_bytes_v;
    ea.tiles = tiles(P) ? 1 : 0;
    ea.cs = stored_bytes(P, C);
    ea.seq_bytes = seq_bytes(P, C, capacity);
    ea.tabs = enc_tabs(plan, side);
    if (kvq::launch_encode(ea, n_streams, stream) != hipSuccess) return KVQ_EDEVICE;
  }
  return KVQ_OK;
}

// Decode attention of one query per sequence over n_tokens compressed tokens
// (rows [0, n_tokens) of arrays holding `capacity` tokens per sequence) and
// res_len uncompressed bf16 tokens (rows [0, res_len) of res_k / res_v, which
// hold res_cap tokens per sequence).
kvq_status attention_impl(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                          const uint8_t* k_cont, const uint8_t* v_cont, const uint16_t* k_so,
                          const uint16_t* v_so, const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                          int64_t n_seqs, int64_t capacity, int64_t n_tokens, const void* res_k,
                          const void* res_v, int64_t res_cap, int64_t res_len, float softmax_scale,
                          void* out, float* out_f32, void* workspace, size_t workspace_bytes,
                          void* hip_stream, bool fixed_width = false) {
  if (!plan || !q || !out || !workspace) return KVQ_EINVAL;
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace)) return KVQ_EINVAL;
  if (out_f32 && !aligned16(out_f32)) return KVQ_EINVAL;
  const kvq_params& P = plan->params;
  const int Hkv = P.n_kv_heads, d = P.head_dim, W = P.mean_window;
  if (n_q_heads < 1 || n_q_heads % Hkv) return KVQ_EINVAL;
  if (n_seqs < 1 || n_tokens < 0 || n_tokens % W || res_len < 0 || n_tokens + res_len < 1)
    return KVQ_EINVAL;
  if (n_tokens > 0) {
    if (!k_cont || !v_cont || !k_so || !v_so || !k_mean_q || !k_mean_scale) return KVQ_EINVAL;
    const void* ptrs[] = {k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale};
    for (const void* p : ptrs)
      if (!aligned16(p)) return KVQ_EINVAL;
    if (capacity < n_tokens || capacity % W) return KVQ_EINVAL;
  }
  if (res_len > 0) {
    if (!res_k || !res_v || !aligned16(res_k) || !aligned16(res_v) || res_cap < res_len) return KVQ_EINVAL;
  }
  const int G = n_q_heads / Hkv;
  const int bk = fw_bits(P.levels_k), bv = fw_bits(P.levels_v);
  const bool affine = plan->side[0].affine && plan->side[1].affine;
  if (fixed_width) {
    if (P.container_bytes_k != plan->n * bk / 8 || P.container_bytes_v != plan->n * bv / 8) return KVQ_EINVAL;
    if (!affine) return KVQ_EUNSUPPORTED;
    if (n_tokens % 64 || W < 64 || !kvq::attention_fw_supported(n_q_heads, G, d, bk, bv, P.levels_k, P.levels_v))
      return KVQ_EUNSUPPORTED;
  } else if (n_tokens % 64 || !kvq::attention2_supported(n_q_heads, G, d, P.levels_k, P.levels_v, W, affine)) {
    return KVQ_EUNSUPPORTED;
  }
  // the tile layout is read by the split-wave kernel (V alphabets of up to 8 levels)
  if (tiles(P) && (fixed_width || P.levels_v > 8)) return KVQ_EUNSUPPORTED;
  if (n_seqs > 65535) return KVQ_EUNSUPPORTED;
  // the attention kernel addresses one sequence's containers with 32-bit offsets
  if (int64_t(n_tokens + 63) * std::max(stored_bytes(P, P.container_bytes_k), stored_bytes(P, P.container_bytes_v)) +
          16 > INT32_MAX)
    return KVQ_EUNSUPPORTED;
  const WsLayout wl = ws_layout(plan, n_seqs, n_tokens, n_q_heads);
  if (workspace_bytes < wl.total) return KVQ_EWORKSPACE;
  int nsplit;
  int64_t tps;
  split_geometry(n_seqs, n_tokens, &nsplit, &tps, one_tile_splits(G, Hkv));
  const int part_splits = nsplit + (res_len > 0 ? 1 : 0);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* qscale = reinterpret_cast<float*>(ws + wl.qscale);
  float* qsum = reinterpret_cast<float*>(ws + wl.qsum);
  float* qmu = reinterpret_cast<float*>(ws + wl.qmu);
  float* part = reinterpret_cast<float*>(ws + wl.part);
  const float tau = softmax_scale > 0.f ? softmax_scale : float(1.0 / std::sqrt(double(d)));

  if (n_tokens > 0) {
    kvq::Prologue2Args pa;
    pa.q = static_cast<const uint16_t*>(q);
    pa.mean_q = k_mean_q;
    pa.mean_scale = k_mean_scale;
    pa.qop = reinterpret_cast<uint16_t*>(ws + wl.qop);
    pa.qscale = qscale;
    pa.qsum = qsum;
    pa.qmu = qmu;
    pa.nW = n_tokens / W;
    pa.nW_cap = capacity / W;
    pa.Hq = n_q_heads;
    pa.G = G;
    pa.n = plan->n;
    pa.hscale = plan->hadamard_scale;
    if (kvq::launch_prologue2(pa, n_seqs, stream) != hipSuccess) return KVQ_EDEVICE;

    kvq::Attn2Args aa;
    std::memset(&aa, 0, sizeof(aa));
    aa.k_cont = k_cont;
    aa.v_cont = v_cont;
    aa.k_so = k_so;
    aa.v_so = v_so;
    aa.qop = reinterpret_cast<const uint4*>(ws + wl.qop);
    aa.qscale = qscale;
    aa.qsum = qsum;
    aa.qmu = qmu;
    aa.part = part;
    aa.T = n_tokens;
    aa.T_cap = capacity;
    aa.tokens_per_split = tps;
    aa.nW = n_tokens / W;
    aa.nsplit = nsplit;
    aa.part_splits = part_splits;
    aa.log2W = 0;
    while ((1 << aa.log2W) < W) ++aa.log2W;
    aa.CK = P.container_bytes_k;
    aa.CV = P.container_bytes_v;
    aa.tiles = tiles(P) ? 1 : 0;
    aa.CKs = stored_bytes(P, P.container_bytes_k);
    aa.CVs = stored_bytes(P, P.container_bytes_v);
    aa.seq_bytes_k = seq_bytes(P, P.container_bytes_k, capacity);
    aa.seq_bytes_v = seq_bytes(P, P.container_bytes_v, capacity);
    aa.tau = tau;
    aa.Mk = P.levels_k;
    aa.Mv = P.levels_v;
    for (int m = 0; m < kvq::kMaxLevels; ++m) {
      aa.fk[m] = plan->side[0].freq[m];
      aa.ck[m] = plan->side[0].cum[m];
      aa.hbk[m] = plan->side[0].fp16_hi[m];
      aa.fv[m] = plan->side[1].freq[m];
      aa.cv[m] = plan->side[1].cum[m];
      aa.hbv[m] = plan->side[1].fp16_hi[m];
      aa.lvk[m] = plan->side[0].fp16_bits[m];
      aa.lbv[m] = plan->side[1].fp16_lo[m];
      if (aa.lbv[m]) aa.v_lo_nonzero = 1;
    }
    for (int z = 0; z < 256; ++z) {
      const uint32_t dk = plan->side[0].dec[z];
      aa.tabk[z] = (dk & 0xFFFFu) | (plan->side[0].fp16_bits[(dk >> 16) & 0xFFu] << 16);
      // integer value levels (zero fp16 low bytes): the level's fp16 high byte in
      // place of its index, so the product needs no lookup
      const uint32_t dv = plan->side[1].dec[z];
      aa.tabv[z] = aa.v_lo_nonzero ? dv : (dv & 0xFFFFu) | (plan->side[1].fp16_hi[(dv >> 16) & 0xFFu] << 16);
    }
    size_t slot = 0;
    const bool timed = timer_begin(stream, &slot);
    const hipError_t e = fixed_width ? kvq::launch_attention_fw(aa, n_seqs, n_q_heads, G, bk, bv, stream)
                                     : kvq::launch_attention2(aa, n_seqs, n_q_heads, G, stream);
    if (e != hipSuccess) return KVQ_EDEVICE;
    if (timed) timer_end(stream, slot);
  }
  if (res_len > 0) {
    kvq::ResidualArgs ra;
    ra.q = static_cast<const uint16_t*>(q);
    ra.k = static_cast<const uint16_t*>(res_k);
    ra.v = static_cast<const uint16_t*>(res_v);
    ra.part = part;
    ra.R = res_len;
    ra.R_cap = res_cap;
    ra.nsplit_total = part_splits;
    ra.split = nsplit;
    ra.Hq = n_q_heads;
    ra.G = G;
    ra.d = d;
    ra.tau = tau;
    ra.hscale = plan->hadamard_scale;
    if (kvq::launch_residual(ra, n_seqs, stream) != hipSuccess) return KVQ_EDEVICE;
  }

  kvq::CombineArgs ca;
  ca.part = part;
  ca.out = static_cast<uint16_t*>(out);
  ca.out_f32 = out_f32;
  ca.nsplit = part_splits;
  ca.Hq = n_q_heads;
  ca.d = d;
  ca.hscale = plan->hadamard_scale;
  if (kvq::launch_combine(ca, n_seqs, stream) != hipSuccess) return KVQ_EDEVICE;
  return KVQ_OK;
}

// Scratch of kvq_decode_attention_noalloc: one array per GPU the library runs
// on, held until the process ends.  In host code `noalloc_scratch_arr` only
// names the symbol; its device address, one per device, comes from
// hipGetSymbolAddress with that device current, on the entry point's first
// call there, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(KVQ_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t noalloc_scratch_arr[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

bool noalloc_scratch(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch_arr)) != hipSuccess || !p) return false;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return true;
}

}  // namespace

extern "C" {

kvq_status kvq_encode_streams(const kvq_plan* plan, const void* k, const void* v,
                              kvq_dtype in_dtype, int64_t n_seqs, int64_t seq_len,
                              uint8_t* k_cont, uint8_t* v_cont, uint16_t* k_so, uint16_t* v_so,
                              int8_t* k_mean_q, uint16_t* k_mean_scale, uint64_t* stats,
                              void* hip_stream) {
  return encode_impl(plan, k, v, in_dtype, n_seqs, seq_len, seq_len, 0, k_cont, v_cont, k_so, v_so,
                     k_mean_q, k_mean_scale, stats, hip_stream);
}

kvq_status kvq_encode_append(const kvq_plan* plan, const void* k, const void* v,
                             kvq_dtype in_dtype, int64_t n_seqs, int64_t n_tokens,
                             int64_t cache_capacity, int64_t token_offset,
                             uint8_t* k_cont, uint8_t* v_cont, uint16_t* k_so, uint16_t* v_so,
                             int8_t* k_mean_q, uint16_t* k_mean_scale, uint64_t* stats,
                             void* hip_stream) {
  return encode_impl(plan, k, v, in_dtype, n_seqs, n_tokens, cache_capacity, token_offset, k_cont,
                     v_cont, k_so, v_so, k_mean_q, k_mean_scale, stats, hip_stream);
}

kvq_status kvq_decode_attention(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                const uint8_t* k_cont, const uint8_t* v_cont,
                                const uint16_t* k_so, const uint16_t* v_so,
                                const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                void* out, float* out_f32, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
  if (seq_len < 1) return KVQ_EINVAL;
  return attention_impl(plan, q, n_q_heads, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, n_seqs,
                        seq_len, seq_len, nullptr, nullptr, 0, 0, softmax_scale, out, out_f32, workspace,
                        workspace_bytes, hip_stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                        const uint8_t* k_cont, const uint8_t* v_cont,
                                        const uint16_t* k_so, const uint16_t* v_so,
                                        const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                        int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                        void* out, float* out_f32, void* hip_stream) {
  if (!plan || seq_len < 1 || n_seqs < 1 || n_q_heads < 1) return KVQ_EINVAL;
  size_t need = 0;
  const kvq_status st = kvq_workspace_bytes(plan, 1, n_seqs, seq_len, n_q_heads, &need);
  if (st != KVQ_OK) return st;
  if (need > kNoAllocScratchBytes) return KVQ_EWORKSPACE;
  void* ws = nullptr;
  if (!noalloc_scratch(&ws)) return KVQ_EDEVICE;
  return attention_impl(plan, q, n_q_heads, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, n_seqs,
                        seq_len, seq_len, nullptr, nullptr, 0, 0, softmax_scale, out, out_f32, ws,
                        kNoAllocScratchBytes, hip_stream);
}

kvq_status kvq_decode_attention_ex(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                   const uint8_t* k_cont, const uint8_t* v_cont,
                                   const uint16_t* k_so, const uint16_t* v_so,
                                   const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                   int64_t n_seqs, int64_t cache_capacity, int64_t n_tokens,
                                   const void* res_k, const void* res_v, int64_t res_capacity,
                                   int64_t res_len, float softmax_scale, void* out, float* out_f32,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  return attention_impl(plan, q, n_q_heads, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, n_seqs,
                        cache_capacity, n_tokens, res_k, res_v, res_capacity, res_len, softmax_scale, out,
                        out_f32, workspace, workspace_bytes, hip_stream);
}

kvq_status kvq_fixed_width_container_bytes(int32_t levels, int32_t n, int32_t* bytes) {
  if (!bytes || levels < 2 || levels > 256 || n < 1) return KVQ_EINVAL;
  const int b = fw_bits(levels);
  if ((int64_t(n) * b) % 32) return KVQ_EINVAL;
  *bytes = n * b / 8;
  return KVQ_OK;
}

kvq_status kvq_encode_fixed_width(const kvq_plan* plan, const void* k, const void* v,
                                  kvq_dtype in_dtype, int64_t n_seqs, int64_t seq_len,
                                  uint8_t* k_cont, uint8_t* v_cont, uint16_t* k_so, uint16_t* v_so,
                                  int8_t* k_mean_q, uint16_t* k_mean_scale, void* hip_stream) {
  return encode_impl(plan, k, v, in_dtype, n_seqs, seq_len, seq_len, 0, k_cont, v_cont, k_so, v_so,
                     k_mean_q, k_mean_scale, nullptr, hip_stream, true);
}

kvq_status kvq_decode_attention_fixed_width(const kvq_plan* plan, const void* q, int32_t n_q_heads,
                                            const uint8_t* k_cont, const uint8_t* v_cont,
                                            const uint16_t* k_so, const uint16_t* v_so,
                                            const int8_t* k_mean_q, const uint16_t* k_mean_scale,
                                            int64_t n_seqs, int64_t seq_len, float softmax_scale,
                                            void* out, float* out_f32, void* workspace,
                                            size_t workspace_bytes, void* hip_stream) {
  if (seq_len < 1) return KVQ_EINVAL;
  return attention_impl(plan, q, n_q_heads, k_cont, v_cont, k_so, v_so, k_mean_q, k_mean_scale, n_seqs,
                        seq_len, seq_len, nullptr, nullptr, 0, 0, softmax_scale, out, out_f32, workspace,
                        workspace_bytes, hip_stream, true);
}

kvq_status kvq_decode_symbols(const kvq_plan* plan, int side, const uint8_t* cont,
                              int64_t n_streams, uint8_t* symbols, uint32_t* end_ok,
                              void* hip_stream) {
  if (!plan || (side != 0 && side != 1) || !cont || !symbols || n_streams < 1) return KVQ_EINVAL;
  if (!aligned16(cont) || !aligned16(symbols) || (end_ok && !aligned16(end_ok))) return KVQ_EINVAL;
  if (tiles(plan->params) && n_streams % 64) return KVQ_EINVAL;     // whole 64-token tiles
  kvq::DecSymArgs a;
  a.cont = cont;
  a.n_streams = n_streams;
  a.C = plan->side[side].container_bytes;
  a.tiles = tiles(plan->params) ? 1 : 0;
  a.cs = stored_bytes(plan->params, a.C);
  a.n = plan->n;
  a.sym = symbols;
  a.end_ok = end_ok;
  std::memcpy(a.dec, plan->side[side].dec, sizeof(a.dec));
  if (kvq::launch_decode_symbols(a, static_cast<hipStream_t>(hip_stream)) != hipSuccess)
    return KVQ_EDEVICE;
  return KVQ_OK;
}

}  // extern "C"
