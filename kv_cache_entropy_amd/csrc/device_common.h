// Device-side helpers and the argument blocks passed by value to kernels.
#ifndef KVQ_DEVICE_COMMON_H_
#define KVQ_DEVICE_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

// ----------------------------------------------------------------- encoder
struct KeyMeanArgs {
  const void* k;              // [S, T, n] (the tokens being encoded)
  int in_bf16;
  int8_t* mean_q;             // [S, T_cap / W, n]
  uint16_t* mean_scale;       // [S, T_cap / W]
  int64_t T;                  // tokens per sequence in k
  int64_t T_cap;              // tokens per sequence in the cache arrays
  int64_t t_off;              // cache position of k's first token (multiple of W)
  int W, n, d;
  float hscale;
};

struct EncTabs {
  uint32_t rate_fx[kMaxLevels];
  uint32_t freq[kMaxLevels];
  uint32_t cum[kMaxLevels];
  uint32_t rcp[kMaxLevels];
  uint32_t rshift[kMaxLevels];
  float level[kMaxLevels];     // reconstruction levels v_m (grid units)
  float lambda[kLambdaGrid];
  int levels;
  int container_bytes;
  uint32_t cheapest;
  uint64_t budget_fx;
};

struct EncodeArgs {
  const void* x;               // [S, T, n]
  int in_bf16;
  int is_key;
  const int8_t* mean_q;        // [S, T_cap / W, n]
  const uint16_t* mean_scale;  // [S, T_cap / W]
  uint8_t* cont;               // [S, T_cap, C]
  uint16_t* so;                // [S, T_cap, 2]
  unsigned long long* stats;   // already offset to the side's 4 counters
  int64_t T;                   // tokens per sequence in x (a multiple of spw)
  int64_t T_cap;               // tokens per sequence in the cache arrays
  int64_t t_off;               // cache position of x's first token
  int W, n, d;
  float hscale;
  int spw;                     // streams per workgroup (multiple of 4)
  int fw_bits;                 // 0: rANS + drift; 1/2/4/8: fixed-width comparator
  int tiles;                   // KVQ_LAYOUT_TILES: dword k of a 64-token tile's containers side by side
  int cs;                      // bytes a container occupies in the cache (C, or C rounded up to 4)
  int64_t seq_bytes;           // cache bytes per sequence (tiles: capacity rounded up to 64, times cs)
  EncTabs tabs;
};

struct EncShared {
  float lambda[kLambdaGrid];
  float level[kMaxLevels];
  uint32_t rate_fx[kMaxLevels];
  float rate_f[kMaxLevels];
  uint4 coder[kMaxLevels];    // per symbol: (f, c, reciprocal, shift), one 16-byte read
  uint32_t cheapest;
  uint64_t budget_fx;
};

// ----------------------------------------------------------------- decoder
struct DecSymArgs {
  const uint8_t* cont;
  int64_t n_streams;
  int C, n;
  uint8_t* sym;
  uint32_t* end_ok;
  int tiles;                   // KVQ_LAYOUT_TILES (n_streams is then a multiple of 64)
  int cs;                      // bytes a container occupies (C, or C rounded up to 4)
  uint32_t dec[256];
};

struct Prologue2Args {
  const uint16_t* q;          // bf16 [S, Hq, 128]
  const int8_t* mean_q;       // [S, nW, n]
  const uint16_t* mean_scale; // [S, nW]
  uint16_t* qop;              // fp16 MFMA operand [S][Hkv][ngm][32][4][hi 4, lo 4]
  float* qscale;              // [S, Hq]: 2^-e undoing the operand scaling
  float* qsum;                // [S, Hq]
  float* qmu;                 // [S, Hq, nW]
  int64_t nW;                 // windows attended per sequence
  int64_t nW_cap;             // windows per sequence in the mean arrays
  int Hq, G, n;
  float hscale;
};

struct Attn2Args {
  const uint8_t* k_cont;
  const uint8_t* v_cont;
  const uint16_t* k_so;
  const uint16_t* v_so;
  const uint4* qop;
  const float* qscale;
  const float* qsum;
  const float* qmu;
  float* part;                // [S, nsplit (+1 residual), Hq, 128 + 4]
  int64_t T;                  // tokens attended per sequence
  int64_t T_cap;              // tokens per sequence in the cache arrays
  int64_t tokens_per_split;
  int64_t nW;
  int nsplit, log2W, CK, CV;
  int part_splits;             // splits per sequence in `part` (nsplit, +1 with a residual)
  float tau;
  int Mk, Mv;
  uint32_t fk[kMaxLevels], ck[kMaxLevels], hbk[kMaxLevels];
  uint32_t fv[kMaxLevels], cv[kMaxLevels], hbv[kMaxLevels];
  uint32_t lvk[kMaxLevels];   // fp16 bits of the key levels
  uint32_t lbv[kMaxLevels];   // low bytes of the fp16 value levels (0 when affine)
  int v_lo_nonzero;           // some value level has a nonzero low byte
  int tiles;                   // KVQ_LAYOUT_TILES containers (split-wave kernel only)
  int CKs, CVs;                // bytes a container occupies (C, or C rounded up to 4)
  int64_t seq_bytes_k, seq_bytes_v;   // cache bytes per sequence
  // decode-table entries of the fused kernels, slot z = state mod 256: f | (z - c) << 8
  // in the low half; the high half holds the fp16 bits of the key level (K) or,
  // for V, the level's fp16 high byte when every value level is an integer
  // (v_lo_nonzero == 0), else the level index
  uint32_t tabk[256], tabv[256];
};

// The uncompressed tail of every sequence (the most recent tokens, kept in
// bf16) as one more split of partials.
struct ResidualArgs {
  const uint16_t* q;          // bf16 [S, Hq, d]
  const uint16_t* k;          // bf16 [S, R_cap, Hkv, d]
  const uint16_t* v;
  float* part;                // [S, nsplit_total, Hq, d + 4]; this writes split `split`
  int64_t R, R_cap;
  int nsplit_total, split, Hq, G, d;
  float tau, hscale;
};

struct CombineArgs {
  const float* part;
  uint16_t* out;              // bf16 [S, Hq, d]
  float* out_f32;             // nullable
  int nsplit, Hq, d;
  float hscale;
};

// ----------------------------------------------------------------- helpers
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_min(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fminf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ inline int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Loads NPL consecutive values (fp32 or bf16) starting at element `off`.
template <int NPL>
__device__ inline void load_values(const void* base, int in_bf16, int64_t off, float (&v)[NPL]) {
  if (in_bf16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if constexpr (NPL % 8 == 0) {
#pragma unroll
      for (int c = 0; c < NPL / 8; ++c) {
        const uint4 w = reinterpret_cast<const uint4*>(p)[c];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[c * 8 + 2 * k] = __uint_as_float(ws[k] << 16);
          v[c * 8 + 2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPL; ++i) v[i] = bf16_bits_to_f32(p[i]);
    }
  } else {
    const float* p = static_cast<const float*>(base) + off;
    if constexpr (NPL % 4 == 0) {
#pragma unroll
      for (int c = 0; c < NPL / 4; ++c) {
        const float4 w = reinterpret_cast<const float4*>(p)[c];
        v[4 * c] = w.x;
        v[4 * c + 1] = w.y;
        v[4 * c + 2] = w.z;
        v[4 * c + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NPL; ++i) v[i] = p[i];
    }
  }
}

// Per-head orthonormal Sylvester Hadamard on values distributed NPL per lane
// (lane holds global indices lane*NPL .. lane*NPL+NPL-1).  Stage h pairs i and
// i + h (bit h of i clear) into (a + b, a - b); then everything is scaled by
// fp32(1/sqrt(d)).
template <int NPL>
__device__ inline void fwht_lanes(float (&v)[NPL], int d, int lane, float scale) {
#pragma unroll
  for (int h = 1; h < NPL; h <<= 1) {
    if (h < d) {
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if (!(i & h)) {
          const float a = v[i], b = v[i + h];
          v[i] = __fadd_rn(a, b);
          v[i + h] = __fsub_rn(a, b);
        }
      }
    }
  }
  for (int h = NPL; h < d; h <<= 1) {
    const int lx = h / NPL;
    const bool upper = (lane & lx) != 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float p = __shfl_xor(v[i], lx, 64);
      v[i] = upper ? __fsub_rn(p, v[i]) : __fadd_rn(v[i], p);
    }
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = __fmul_rn(v[i], scale);
}


hipError_t launch_key_mean(const KeyMeanArgs& a, int64_t n_windows, hipStream_t stream);
hipError_t launch_encode(const EncodeArgs& a, int64_t n_streams, hipStream_t stream);
hipError_t launch_decode_symbols(const DecSymArgs& a, hipStream_t stream);
hipError_t launch_prologue2(const Prologue2Args& a, int64_t S, hipStream_t stream);
hipError_t launch_attention2(const Attn2Args& a, int64_t S, int Hq, int G, hipStream_t stream);
bool attention2_supported(int Hq, int G, int d, int levels_k, int levels_v, int window, bool affine);
hipError_t launch_combine(const CombineArgs& a, int64_t S, hipStream_t stream);
hipError_t launch_residual(const ResidualArgs& a, int64_t S, hipStream_t stream);
bool attention_fw_supported(int Hq, int G, int d, int bk, int bv, int levels_k, int levels_v);
hipError_t launch_attention_fw(const Attn2Args& a, int64_t S, int Hq, int G, int bk, int bv,
                               hipStream_t stream);

}  // namespace kvq

#endif  // KVQ_DEVICE_COMMON_H_
