// Fused decode attention over entropy-coded containers, tuned for gfx950.
//
// [D-Quant] §4.5 "Decoding": the kernel is token-centric - every stream is
// decoded exactly once and its levels feed all query heads of the current KV
// head.  Appendix A, Algorithm 2 gives the per-symbol decoder; Eqs. (8)-(9)
// let the contractions run on the raw levels with the affine terms applied
// afterwards.
//
// The kernels handle a token range of one sequence in 64-token tiles, lane
// t <-> token t0 + t:
//   * QK^T: every 4 decoded K levels of a lane form the B operand of a
//     v_mfma_f32_4x4x4f16 block (16 blocks of 4 tokens); the A operand is the
//     rotated query of 4 heads, split into fp16 hi + lo parts after a
//     power-of-two scaling, so each lane ends with its own token's logits.
//   * PV: V levels go to a [channel][token] LDS chunk; the contraction over
//     tokens is again 4x4x4 MFMA blocks (16 channel groups x 4 heads) with the
//     softmax weights (hi + lo) as A.
//   * Online softmax per query head across tiles; the per-token scale folds
//     into the weights and the per-token offset into a separate sum (Eq. 9).
// attention5_kernel (V alphabets of up to 8 levels) decodes K and V in the two
// waves of a pair, eight pairs per workgroup sharing replicated decode tables
// in LDS; its layout is described above its definition.
// attention2_kernel is the single-wave form for 9-level V alphabets: 8-byte
// decode-table entries (lo = f | fp16 level high byte << 24, hi = z - c, one
// v_mad_u32_u24 per symbol), a 64-byte ring per lane refilled by 16-byte loads
// two 16-symbol blocks ahead, and an fp16 V chunk.

#include <type_traits>
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.h"

namespace kvq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;             // head_dim handled by this kernel
constexpr int kRingStride = 68;     // bytes per lane ring: 64 + 4 to spread LDS banks
constexpr int kChunkStride = 136;   // bytes per channel row of the V chunk: 64 fp16 + pad
constexpr uint32_t kNoChunk = 0xFFFFFFFFu;

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ inline half4_t as_half4(uint32_t a, uint32_t b) {
  union {
    uint2 u;
    half4_t h;
  } c;
  c.u = make_uint2(a, b);
  return c.h;
}

// -------------------------------------------------------------------- ring
struct Ring {
  const uint8_t* g;     // 16-byte aligned global base of the lane's frame
  uint32_t P;           // frame position of the next unread byte
  uint32_t F;           // frame position of the next chunk to fetch
  uint32_t lim;         // frame position one past the container's last byte
  uint32_t last;        // frame position of the container's last chunk
  uint4 pend[2];        // chunks in flight
  uint32_t ppos[2];     // their frame positions (kNoChunk: nothing to write)
};

__device__ inline void ring_write(uint8_t* ring_lane, uint32_t pos, const uint4& d) {
  uint32_t* w = reinterpret_cast<uint32_t*>(ring_lane + (pos & 63u));
  w[0] = d.x;
  w[1] = d.y;
  w[2] = d.z;
  w[3] = d.w;
}

// Starts a container: fills the ring with the first 64 frame bytes (chunks
// past the container are never fetched, so no load leaves the array) and
// reads the 4-byte little-endian initial state.
__device__ inline uint32_t ring_start(Ring& r, uint8_t* ring_lane, const uint8_t* cont_row, uint32_t C) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(cont_row);
  const uint32_t off0 = uint32_t(a & 15u);
  r.g = reinterpret_cast<const uint8_t*>(a - off0);
  r.lim = off0 + C;
  r.last = (r.lim - 1u) & ~15u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (uint32_t(16 * q) < r.lim) {
      const uint4 d = *reinterpret_cast<const uint4*>(r.g + 16 * q);
      ring_write(ring_lane, 16u * q, d);
    }
  }
  r.F = 64;
  r.ppos[0] = r.ppos[1] = kNoChunk;
  const uint32_t x = uint32_t(ring_lane[(off0) & 63u]) | (uint32_t(ring_lane[(off0 + 1) & 63u]) << 8) |
                     (uint32_t(ring_lane[(off0 + 2) & 63u]) << 16) | (uint32_t(ring_lane[(off0 + 3) & 63u]) << 24);
  r.P = off0 + 4;
  return x;
}

// Once per 16 symbols, slot s alternating: write the chunk fetched two
// blocks ago, then fetch the next chunk if the lane is within 48 bytes of
// the fetch front.  Every lane issues exactly one load per block (a re-load of
// the container's last chunk when nothing is needed) so the outstanding-load
// count is uniform.  Invariants (at most one byte per symbol): the bytes of
// the coming 16 symbols are written before they are read, and a chunk never
// overwrites bytes not yet consumed.
template <int S>
__device__ inline void ring_block(Ring& r, uint8_t* ring_lane) {
  if (r.ppos[S] != kNoChunk) ring_write(ring_lane, r.ppos[S], r.pend[S]);
  const bool real = (r.F < r.lim) && (r.F - r.P <= 48u);
  const uint32_t pos = real ? r.F : r.last;
  r.pend[S] = *reinterpret_cast<const uint4*>(r.g + pos);
  r.ppos[S] = real ? pos : kNoChunk;
  r.F += real ? 16u : 0u;
}

// One symbol of Algorithm 2.  Returns the low table word (fp16 level in the
// upper half).  The next container byte is read before it is known whether it
// is needed, so the update is branch-free.
__device__ inline uint32_t dec_step(uint32_t& x, Ring& r, const uint2* tab, const uint8_t* ring_lane) {
  const uint32_t b = ring_lane[r.P & 63u];
  const uint2 e = tab[x & 0xFFu];
  x = __umul24(e.x, x >> 8) + e.y;
  const bool renorm = x < kStateLow;
  x = renorm ? ((x << 8) | b) : x;
  r.P += renorm ? 1u : 0u;
  return e.x;
}

__device__ inline float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ inline float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Wave-wide reductions in VALU only: DPP within rows of 16 lanes, then the
// gfx950 row and half-wave swaps; the result is taken from lane 0 so that it
// is exactly uniform (the partial sums are combined in lane-dependent order).
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline float swap_rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float r = __uint_as_float(a[0]) + __uint_as_float(a[1]);    // own + partner row
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(r), __float_as_uint(r), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);             // own + partner half
}
// The max runs on order-preserving integer keys of the (finite) floats: an
// integer max takes its DPP operand directly, where fmaxf would first quiet
// both operands.  Lanes without a DPP source would keep INT_MIN, the max's
// identity (every pattern used here is a full permutation).
template <int CTRL>
__device__ inline int dpp_max_i(int v) {
  const int o = __builtin_amdgcn_update_dpp(int(0x80000000), v, CTRL, 0xF, 0xF, false);
  return v > o ? v : o;
}
__device__ inline int swap_rows_max_i(int v) {
  const auto a = __builtin_amdgcn_permlane16_swap(uint32_t(v), uint32_t(v), false, false);
  const int r = int(a[0]) > int(a[1]) ? int(a[0]) : int(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(uint32_t(r), uint32_t(r), false, false);
  return int(b[0]) > int(b[1]) ? int(b[0]) : int(b[1]);
}
__device__ inline int float_key(int b) { return b ^ ((b >> 31) & 0x7FFFFFFF); }
__device__ inline float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);      // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);      // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);     // row_ror:4
  v += dpp_f<0x128>(v);     // row_ror:8
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(swap_rows_sum(v))));
}
__device__ inline float wave_max_dpp(float v) {
  int k = float_key(__float_as_int(v));
  k = dpp_max_i<0xB1>(k);
  k = dpp_max_i<0x4E>(k);
  k = dpp_max_i<0x124>(k);
  k = dpp_max_i<0x128>(k);
  return __int_as_float(float_key(__builtin_amdgcn_readfirstlane(swap_rows_max_i(k))));
}

// Reduce-scatter of N per-lane values (N a power of two, at most 16) over the
// wave: each halving stage pairs lanes that differ in one bit of the lane
// index (quad xor 1 and 2, then row rotations by 4 and 8, which flip bit 2 and
// bit 3 of a row position); a lane keeps the half of its values selected by
// that bit and adds the partner's copy of the same half.  After log2 N stages
// a lane holds one value; the remaining row stages and the two row swaps sum
// it over the wave.  Lane l ends with the wave total of value
// sum_k bit_k(l) * (N >> (k + 1)), k < log2 N.
template <int N>
__device__ inline float wave_sum_scatter(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 16 && (N & (N - 1)) == 0, "N must be a power of two up to 16");
  int c = N;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool hi = ((lane >> k) & 1) != 0;
    if (c > 1) {
      const int h = c / 2;
#pragma unroll
      for (int j = 0; j < N / 2; ++j) {
        if (j < h) {
          // the empty asm keeps the two selects as selects of values (not one
          // dynamically indexed read of v)
          float lo_v = v[j], hi_v = v[j + h];
          asm("" : "+v"(lo_v), "+v"(hi_v));
          const float keep = hi ? hi_v : lo_v;
          const float send = hi ? lo_v : hi_v;
          const float got = k == 0 ? dpp_f<0xB1>(send) : k == 1 ? dpp_f<0x4E>(send)
                                                         : k == 2 ? dpp_f<0x124>(send) : dpp_f<0x128>(send);
          v[j] = keep + got;
        }
      }
      c = h;
    } else {
      const float got = k == 0 ? dpp_f<0xB1>(v[0]) : k == 1 ? dpp_f<0x4E>(v[0])
                                                   : k == 2 ? dpp_f<0x124>(v[0]) : dpp_f<0x128>(v[0]);
      v[0] += got;
    }
  }
  return swap_rows_sum(v[0]);
}

// ------------------------------------------------------------------ prologue
// The query terms of one query slot v of KV head g: slot v < G is query head
// g G + v; slots up to the next multiple of 4 are zero padding.  The chunk-0
// wave writes the MFMA A operand (rotated query scaled by 2^e so that max |q|
// is in [2^7, 2^8), split into fp16 hi + lo), the inverse scale and
// sum_j q_rot_j.  Returns the rotated query (lane holds j = 2 lane, 2 lane + 1)
// and its scale 2^e in up_out.
__device__ inline void prologue_query(const Prologue2Args& a, int64_t s, int g, int v, int64_t chunk, int lane,
                                      float (&q)[2], float* up_out = nullptr) {
  const int hkv = a.Hq / a.G;
  const int ngm = (a.G + 3) / 4;
  const bool real = v < a.G;
  const int h = g * a.G + v;
  q[0] = q[1] = 0.f;
  if (real) {
    const uint16_t* qp = a.q + (s * a.Hq + h) * kD + lane * 2;
    q[0] = bf16_bits_to_f32(qp[0]);
    q[1] = bf16_bits_to_f32(qp[1]);
  }
  fwht_lanes<2>(q, kD, lane, a.hscale);
  const float amax = wave_max_f(fmaxf(fabsf(q[0]), fabsf(q[1])));
  int e = 0;
  if (amax > 0.f) {
    int ex;
    frexpf(amax, &ex);                  // amax in [2^(ex-1), 2^ex)
    e = 8 - ex;
  }
  const float up = ldexpf(1.0f, e);
  if (up_out) *up_out = up;
  // operand layout: [s][g][gm][c = j/4][n][hi0..3 lo0..3]
  const int gm = v / 4, n = v % 4;
  uint16_t* op = a.qop + ((((s * hkv + g) * ngm + gm) * 32) * 4) * 8;
#pragma unroll
  for (int i = 0; i < 2 && chunk == 0; ++i) {
    const int j = lane * 2 + i;
    const float qs = q[i] * up;
    const __half hi = __float2half_rn(qs);
    const __half lo = __float2half_rn(qs - __half2float(hi));
    const int c = j / 4, k = j % 4;
    op[(c * 4 + n) * 8 + k] = __half_as_ushort(hi);
    op[(c * 4 + n) * 8 + 4 + k] = __half_as_ushort(lo);
  }
  if (!real) return;
  const float qs = wave_sum_f(q[0] + q[1]);
  if (lane == 0 && chunk == 0) {
    a.qsum[s * a.Hq + h] = qs;
    a.qscale[s * a.Hq + h] = ldexpf(1.0f, -e);
  }
}

// sum_j q_rot_j mu_w,j of NH query heads for window w (its 128 int8 means of
// KV head g, read as 16-byte vectors: rows are 16-byte aligned, since the base
// is and n is a multiple of 128).  mu_w,j = RN(mu_q sc) is formed once and
// shared by the heads; each head's sum runs in j order.
template <int NH>
__device__ inline void prologue_qmu(const Prologue2Args& a, int64_t s, int g, int64_t w, const float* qsh,
                                    float (&acc)[NH]) {
  const float sc = h2f(a.mean_scale[s * a.nW_cap + w]);
  const uint4* mq = reinterpret_cast<const uint4*>(a.mean_q + (s * a.nW_cap + w) * a.n + int64_t(g) * kD);
#pragma unroll
  for (int v = 0; v < NH; ++v) acc[v] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 v4 = mq[c];
    const uint32_t wd[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float mu = __fmul_rn(float(int8_t(wd[k / 4] >> (8 * (k % 4)))), sc);
#pragma unroll
      for (int v = 0; v < NH; ++v) acc[v] = __fadd_rn(acc[v], __fmul_rn(qsh[v * kD + 16 * c + k], mu));
    }
  }
}

// One wave per (sequence, KV head, query slot v, chunk of 64 key-mean
// windows): the query terms of slot v, and sum_j q_rot_j mu_w,j for the
// windows w of the chunk, one per lane (a long context has thousands of
// windows per head, spread over chunks, so the windows' loads are
// independent).
__global__ __launch_bounds__(64) void prologue2_kernel(Prologue2Args a) {
  const int lane = threadIdx.x;
  const int ngm = (a.G + 3) / 4;
  const int v = int(blockIdx.x % unsigned(ngm * 4));           // query slot in [0, NGM*4)
  const int64_t chunk = blockIdx.x / unsigned(ngm * 4);        // windows [64 chunk, 64 chunk + 64)
  const int g = blockIdx.y;
  const int64_t s = blockIdx.z;
  float q[2];
  prologue_query(a, s, g, v, chunk, lane, q);
  if (v >= a.G) return;
  __shared__ float qsh[kD];
  qsh[2 * lane] = q[0];
  qsh[2 * lane + 1] = q[1];
  __syncthreads();
  const int64_t w = chunk * 64 + lane;
  if (w < a.nW) {
    float acc[1];
    prologue_qmu<1>(a, s, g, w, qsh, acc);
    a.qmu[(s * a.Hq + g * a.G + v) * a.nW + w] = acc[0];
  }
}

// ----------------------------------------------------------------- attention
template <int G, int HKV>
__global__ __launch_bounds__(64, 2) void attention2_kernel(Attn2Args a) {
  constexpr int HQ = G * HKV;
  constexpr int NGM = (G + 3) / 4;       // groups of 4 query heads per KV head
  constexpr int NW = (G < 4 ? 4 : G);    // weight rows written per KV head
  __shared__ uint2 tabK[256], tabV[256];
  __shared__ __align__(16) uint8_t ring[64 * kRingStride];
  __shared__ __align__(16) uint8_t vch[64 * kChunkStride];
  __shared__ __align__(16) uint16_t wts[2][NW][64];   // [hi/lo][head][token]
  __shared__ float runM[HQ], runL[HQ], runZ[HQ];
  __shared__ float affS[HQ], affQ[HQ], affM[HQ];   // per tile: query scale, sum q, sum q mu

  const int lane = threadIdx.x;
  const int64_t s = blockIdx.y;
  const int split = blockIdx.x;
  uint8_t* const my_ring = ring + lane * kRingStride;

  // decode tables
  for (int z = lane; z < 256; z += 64) {
    uint32_t mk = 0, mv = 0;
    for (int m = 1; m < a.Mk; ++m) mk = (uint32_t(z) >= a.ck[m]) ? uint32_t(m) : mk;
    for (int m = 1; m < a.Mv; ++m) mv = (uint32_t(z) >= a.cv[m]) ? uint32_t(m) : mv;
    tabK[z] = make_uint2(a.fk[mk] | (a.hbk[mk] << 24), uint32_t(z) - a.ck[mk]);
    tabV[z] = make_uint2(a.fv[mv] | (a.hbv[mv] << 24), uint32_t(z) - a.cv[mv]);
  }
  for (int h = lane; h < HQ; h += 64) {
    runM[h] = -__builtin_inff();
    runL[h] = 0.f;
    runZ[h] = 0.f;
  }
  __syncthreads();

  float4_t O[HKV][2][NGM];
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int m = 0; m < NGM; ++m) O[g][c][m] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t tb = int64_t(split) * a.tokens_per_split;
  const int64_t te = tb + a.tokens_per_split < a.T ? tb + a.tokens_per_split : a.T;
  const uint4* qop = a.qop + s * (HKV * NGM * 32 * 4);
  const float* qscale = a.qscale + s * HQ;
  const float* qsum = a.qsum + s * HQ;
  const float* qmu = a.qmu + s * HQ * a.nW;
  const int qn = lane & 3;   // A-operand row = query slot within a group of 4

  for (int64_t t0 = tb; t0 < te; t0 += 64) {
    const int64_t row = s * a.T_cap + t0 + lane;
    const float sk = h2f(a.k_so[2 * row]), ok = h2f(a.k_so[2 * row + 1]);
    // the 64-token tile lies in one key-mean window (W >= 64, tiles aligned)
    const int64_t w = t0 >> a.log2W;
    for (int h = lane; h < HQ; h += 64) {
      affS[h] = qscale[h];
      affQ[h] = qsum[h];
      affM[h] = qmu[h * a.nW + w];
    }
    __syncthreads();
    float logit[HKV][NGM][4];

    // ------------------------------------------------------------ keys
    Ring r;
    uint32_t x = ring_start(r, my_ring, a.k_cont + row * a.CK, uint32_t(a.CK));
#pragma unroll
    for (int g = 0; g < HKV; ++g) {
      float4_t D[NGM];
#pragma unroll
      for (int m = 0; m < NGM; ++m) D[m] = float4_t{0.f, 0.f, 0.f, 0.f};
      const uint4* qg = qop + g * (NGM * 32 * 4) + qn;
      // A operands one channel quad ahead (explicit double buffer keeps the
      // register footprint small)
      uint4 qa[NGM];
#pragma unroll
      for (int m = 0; m < NGM; ++m) qa[m] = qg[(m * 32) * 4];
#pragma unroll 1
      for (int blk = 0; blk < 8; ++blk) {
        if (blk & 1) ring_block<1>(r, my_ring); else ring_block<0>(r, my_ring);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int c = blk * 4 + cc;                  // channel quad within the head
          const int cn = c + 1 < 32 ? c + 1 : 31;
          uint4 qb[NGM];
#pragma unroll
          for (int m = 0; m < NGM; ++m) qb[m] = qg[(m * 32 + cn) * 4];
          const uint32_t e0 = dec_step(x, r, tabK, my_ring);
          const uint32_t e1 = dec_step(x, r, tabK, my_ring);
          const uint32_t e2 = dec_step(x, r, tabK, my_ring);
          const uint32_t e3 = dec_step(x, r, tabK, my_ring);
          const half4_t B = as_half4(__builtin_amdgcn_perm(e1, e0, 0x07060302u),
                                     __builtin_amdgcn_perm(e3, e2, 0x07060302u));
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(qa[m].x, qa[m].y), B, D[m], 0, 0, 0);
            D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(qa[m].z, qa[m].w), B, D[m], 0, 0, 0);
            qa[m] = qb[m];
          }
        }
      }
#pragma unroll
      for (int m = 0; m < NGM; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = m * 4 + i;
          if (v < G) {
            const int h = g * G + v;
            logit[g][m][i] = a.tau * (sk * (D[m][i] * affS[h]) + ok * affQ[h] + affM[h]);
          } else {
            logit[g][m][i] = 0.f;
          }
        }
    }

    // ------------------------------------------------------------ values
    const float sv = h2f(a.v_so[2 * row]), ov = h2f(a.v_so[2 * row + 1]);
    x = ring_start(r, my_ring, a.v_cont + row * a.CV, uint32_t(a.CV));
#pragma unroll
    for (int g = 0; g < HKV; ++g) {
      // online softmax of this KV head's query heads over the tile
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int m = v / 4, i = v % 4;
        float whi = 0.f, wlo = 0.f;
        if (v < G) {
          const int h = g * G + v;
          const float lg = logit[g][m][i];
          const float tmax = wave_max_f(lg);
          const float Mo = runM[h], Lo = runL[h], Zo = runZ[h];
          const float Mn = fmaxf(Mo, tmax);
          const float al = __expf(Mo - Mn);
          const float p = __expf(lg - Mn);
          const float ls = wave_sum_f(p);
          const float zs = wave_sum_f(p * ov);
          __syncthreads();
          runM[h] = Mn;
          runL[h] = Lo * al + ls;
          runZ[h] = Zo * al + zs;
#pragma unroll
          for (int c = 0; c < 2; ++c) O[g][c][m][i] *= al;
          const float wt = p * sv;
          const __half hh = __float2half_rn(wt);
          whi = wt;
          wlo = wt - __half2float(hh);
        }
        wts[0][v][lane] = __half_as_ushort(__float2half_rn(whi));
        wts[1][v][lane] = __half_as_ushort(__float2half_rn(wlo));
      }
      for (int c = 0; c < 2; ++c) {
        // decode 64 channels of this KV head into the [channel][token] chunk
#pragma unroll 1
        for (int blk = 0; blk < 4; ++blk) {
          if (blk & 1) ring_block<1>(r, my_ring); else ring_block<0>(r, my_ring);
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int j = blk * 16 + jj;
            const uint32_t e = dec_step(x, r, tabV, my_ring);
            *reinterpret_cast<uint16_t*>(vch + j * kChunkStride + 2 * lane) = uint16_t(e >> 16);
          }
        }
        __syncthreads();
        // PV over the 64 tokens, 4 at a time
#pragma unroll 2
        for (int tq = 0; tq < 16; ++tq) {
          const uint2 bb = *reinterpret_cast<const uint2*>(vch + lane * kChunkStride + 8 * tq);
          const half4_t B = as_half4(bb.x, bb.y);
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            const uint2 ah = *reinterpret_cast<const uint2*>(&wts[0][m * 4 + qn][4 * tq]);
            const uint2 al = *reinterpret_cast<const uint2*>(&wts[1][m * 4 + qn][4 * tq]);
            O[g][c][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(ah.x, ah.y), B, O[g][c][m], 0, 0, 0);
            O[g][c][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(al.x, al.y), B, O[g][c][m], 0, 0, 0);
          }
        }
        __syncthreads();
      }
    }
  }

  // partials: lane holds channel c*64 + lane of every query head
  float* P = a.part + (s * a.part_splits + split) * int64_t(HQ) * (kD + 4);
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int m = 0; m < NGM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = m * 4 + i;
        if (v < G) {
          const int h = g * G + v;
#pragma unroll
          for (int c = 0; c < 2; ++c) P[h * (kD + 4) + c * 64 + lane] = O[g][c][m][i];
          if (lane == 0) {
            P[h * (kD + 4) + kD] = runM[h];
            P[h * (kD + 4) + kD + 1] = runL[h];
            P[h * (kD + 4) + kD + 2] = runZ[h];
          }
        }
      }
}


// ------------------------------------------- LDS rings and decode tables
// Decode-table entries are 32-bit: f | (z - c) << 8 | payload, the payload
// being the fp16 bits of the level (K) or, in bits 16..23, the level's fp16
// high byte (V with integer levels) or its index (other V levels).  Replicated tables put replica r of a slot at a bank of its own, and
// lane l reads replica l mod R.
// A lane's ring holds container bytes [16 rows of 4]: frame byte p sits in
// row (p / 4) mod 16, byte p mod 4 of the lane's own dword of that row, so the
// lanes of a wave never share a bank in ring reads and writes.  Row 16 repeats
// row 0 so that two consecutive rows can be read with one ds_read2.  The
// decoder reads the 8-byte window holding the next 4 bytes once per 4 symbols
// and takes its bytes with v_perm.
constexpr int kChunk8Stride = 68;     // bytes per channel row of the int8 V chunk
constexpr uint32_t kRingBytes = 17u * 256u;

__device__ inline void wave_lds_fence() {
  // LDS instructions of one wave execute in order; this only keeps the
  // compiler from moving LDS accesses across the point.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Hides a value's known bits from the optimiser, so that an or with it stays
// an or (one v_and_or_b32) and a product stays a product (byte-select operands).
__device__ inline uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Container bytes are fetched with raw buffer loads on a resource spanning the
// wave's sequence; a lane with nothing to fetch passes an offset past the end,
// which loads zeros without touching memory, so every lane issues the same
// loads and the outstanding-load count stays static.
constexpr uint32_t kNoLoad = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t seq_rsrc(const uint8_t* seq_base, uint32_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(seq_base);
  const uint32_t mis = uint32_t(a & 15u);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(seq_base - mis), 0, int(bytes + mis),
                                           0x00020000);
}

__device__ inline uint4 load_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// The 16-byte chunk at frame position F of a lane's container in the tile
// layout: its four dwords lie 256 bytes apart (dword k of the tile's 64
// containers side by side), so the wave's four loads each read 256
// contiguous bytes.  off = the lane's dword offset + 64 F; kNoLoad stays out
// of range for all four.
__device__ inline uint4 load_chunk_tiles(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return make_uint4(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0),
                    __builtin_amdgcn_raw_buffer_load_b32(rs, off + 256u, 0, 0),
                    __builtin_amdgcn_raw_buffer_load_b32(rs, off + 512u, 0, 0),
                    __builtin_amdgcn_raw_buffer_load_b32(rs, off + 768u, 0, 0));
}

// Positions in a lane's stream are kept in bits (8 per byte), so that the
// decode step's shift amounts add up to the bytes consumed directly.
struct Ring5 {
  uint32_t fo;          // buffer offset of the lane's 16-byte aligned frame
  uint32_t off;         // LDS offset of the lane's dword in row 0 of its ring
  uint32_t P;           // frame position of the next unread byte, in bits
  uint32_t F;           // frame position of the next chunk to fetch, in bits
  uint32_t lim;         // frame position one past the container's last byte, in bits
  uint4 pend[2];        // chunks in flight
  uint32_t ppos[2];     // their frame positions in bits (kNoChunk: nothing to write)
};

template <int RS>
__device__ inline uint32_t ring5_row(uint32_t pos, uint32_t off) {
  // row (pos / 32) mod 16 at a pitch of 2^RS bytes: one bit-field extract and
  // one shift-add (opaque keeps the compiler from turning the extract into a
  // shift and a mask)
  return (opaque(__builtin_amdgcn_ubfe(pos, 5u, 4u)) << RS) + off;
}

// Writes the 16-byte chunk at frame position pos (bits; a multiple of 128, so
// its four rows do not wrap), and row 16 with it when it lands on row 0.
template <int RS>
__device__ inline void ring5_write(uint8_t* lds, uint32_t off, uint32_t pos, const uint4& d) {
  constexpr int R = 1 << (RS - 2);            // dwords per ring row
  uint32_t* w = reinterpret_cast<uint32_t*>(lds + ring5_row<RS>(pos, off));
  w[0] = d.x;
  w[R] = d.y;
  w[2 * R] = d.z;
  w[3 * R] = d.w;
  if ((pos & 511u) == 0u) w[16 * R] = d.x;
}

// Bytes P .. P+3 of the stream as a little-endian dword (P's 8-byte window,
// shifted by P mod 4 bytes).
template <int RS>
__device__ inline uint32_t ring5_window(const Ring5& r, const uint8_t* lds) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(lds + ring5_row<RS>(r.P, r.off));
  return __builtin_amdgcn_alignbit(w[1 << (RS - 2)], w[0], r.P);
}

// The same bytes big-endian: byte P in bits 24..31, as the decode step
// shifts them into the state from the top.
template <int RS>
__device__ inline uint32_t ring5_window_be(const Ring5& r, const uint8_t* lds) {
  const uint32_t le = ring5_window<RS>(r, lds);
  return __builtin_amdgcn_perm(le, le, 0x00010203u);
}

// Starts a container (cont_off: its byte offset in the sequence's buffer
// resource): fills the ring with the first 64 frame bytes (chunks past the
// container are not fetched) and reads the 4-byte little-endian initial state.
// TL: the tile layout, cont_off the lane's dword-0 offset (frames start at 0).
template <int RS, bool TL = false>
__device__ inline uint32_t ring5_start(Ring5& r, uint8_t* lds, __amdgpu_buffer_rsrc_t rs, uint32_t cont_off,
                                       uint32_t C) {
  const uint32_t off0 = TL ? 0u : cont_off & 15u;
  r.fo = cont_off - off0;
  r.lim = 8u * (off0 + C);
  uint4 d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d[q] = TL ? load_chunk_tiles(rs, 128u * q < r.lim ? r.fo + 1024u * q : kNoLoad)
              : load_chunk(rs, 128u * q < r.lim ? r.fo + 16u * q : kNoLoad);
#pragma unroll
  for (int q = 0; q < 4; ++q) ring5_write<RS>(lds, r.off, 128u * q, d[q]);
  r.F = 512u;
  r.ppos[0] = r.ppos[1] = kNoChunk;
  r.P = 8u * off0;
  const uint32_t x = ring5_window<RS>(r, lds);
  r.P += 32u;
  return x;
}

// Once per 16 symbols, slot S alternating: write the chunk fetched two blocks
// ago, then fetch the next chunk if the lane is within 48 bytes of the fetch
// front.  Invariants (at most one byte per symbol): the bytes of the coming 16
// symbols are written before they are read, and a chunk never overwrites
// bytes not yet consumed.
template <int S, int RS, bool TL = false>
__device__ inline void ring5_block(Ring5& r, uint8_t* lds, __amdgpu_buffer_rsrc_t rs) {
  if (r.ppos[S] != kNoChunk) ring5_write<RS>(lds, r.off, r.ppos[S], r.pend[S]);
  const bool real = (r.F < r.lim) && (r.F - r.P <= 384u);
  r.pend[S] = TL ? load_chunk_tiles(rs, real ? r.fo + 8u * r.F : kNoLoad)
                 : load_chunk(rs, real ? r.fo + (r.F >> 3) : kNoLoad);
  r.ppos[S] = real ? r.F : kNoChunk;
  r.F += real ? 128u : 0u;
}

// One symbol of Algorithm 2: x = f (x >> 8) + z - c, then at most one byte
// shifted in.  xw holds the state in its high half and the next stream bytes,
// big-endian, in its low half, so the byte shift-in is one 64-bit shift by 8
// or 0 bits that also moves the window on; the shift amount (bits consumed)
// is returned in sh.  Reads no LDS besides the table; returns the table entry.
// PERM: the table slot is row x mod 256 of the interleaved table region at
// TAB, so the address is one v_perm: byte 0 from the lane's replica offset
// toff, byte 1 the state's low byte, bytes 2..3 zero; TAB is an immediate.
// Otherwise slot z holds its replicas contiguously (toff = table base + the
// lane's replica offset) and the address is a shift and an and-or.
template <bool PERM, uint32_t SLOT_SHIFT, uint32_t TAB>
__device__ inline uint32_t dec5_step(uint64_t& xw, uint32_t& sh, const uint8_t* lds, uint32_t toff) {
  constexpr uint32_t mask = 0xFFu << SLOT_SHIFT;
  const uint32_t x = uint32_t(xw >> 32);
  const uint32_t addr = PERM ? __builtin_amdgcn_perm(x, toff, 0x0C0C0400u) + TAB
                             : (((x << SLOT_SHIFT) & mask) | toff);
  const uint32_t e = *reinterpret_cast<const uint32_t*>(lds + addr);
  const uint32_t m = opaque(__umul24(e & 0xFFu, x >> 8));
  const uint32_t x1 = m + ((e >> 8) & 0xFFu);
  // opaque: a shift by a selected amount, not a select between two shifts
  sh = opaque(x1 < kStateLow ? 8u : 0u);
  xw = ((uint64_t(x1) << 32) | uint32_t(xw)) << sh;
  return e;
}

// Four symbols from the window at the lane's position; advances the position
// by the bits they consumed.
template <bool PERM, uint32_t SLOT_SHIFT, uint32_t TAB, int RS>
__device__ inline void dec5_group(uint32_t& x, Ring5& r, const uint8_t* lds, uint32_t toff, uint32_t (&e)[4]) {
  uint64_t xw = (uint64_t(x) << 32) | ring5_window_be<RS>(r, lds);
  uint32_t sh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = dec5_step<PERM, SLOT_SHIFT, TAB>(xw, sh[i], lds, toff);
  x = uint32_t(xw >> 32);
  r.P = r.P + sh[0] + sh[1] + sh[2] + sh[3];
}

// dec5_group for the V wave: each symbol's level byte goes to its row of the
// level chunk, one symbol late, so that every byte store follows the next
// symbol's table read (LDS instructions of a wave run in order; a store
// queued ahead of a read would lengthen the decode chain).  row0 is the
// address of the group's first symbol in its row; epend carries the pending
// entry (skipped before the first symbol of a run, flushed by the caller).
template <bool PERM, uint32_t SLOT_SHIFT, uint32_t TAB, int RS>
__device__ inline void dec5_group_v(uint32_t& x, Ring5& r, const uint8_t* lds, uint32_t toff, uint8_t* row0,
                                    uint32_t& epend, bool first) {
  uint64_t xw = (uint64_t(x) << 32) | ring5_window_be<RS>(r, lds);
  uint32_t sh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = dec5_step<PERM, SLOT_SHIFT, TAB>(xw, sh[i], lds, toff);
    if (!(first && i == 0)) row0[(i - 1) * kChunk8Stride] = uint8_t(epend >> 16);
    epend = e;
  }
  x = uint32_t(xw >> 32);
  r.P = r.P + sh[0] + sh[1] + sh[2] + sh[3];
}

// 4x4x4 MFMA whose A operand is broadcast from block `abid` to all 16 blocks.
// The builtin needs the block as a literal; callers pass a value that is a
// constant after unrolling, so the switch folds to one instruction.
__device__ __attribute__((always_inline)) inline float4_t mfma_bcast_a(half4_t a, half4_t b, float4_t c,
                                                                       int abid) {
#define KVQ_MFMA_BCAST_CASE(i) \
  case i:                      \
    return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, i, 0);
  switch (abid) {
    KVQ_MFMA_BCAST_CASE(0) KVQ_MFMA_BCAST_CASE(1) KVQ_MFMA_BCAST_CASE(2) KVQ_MFMA_BCAST_CASE(3)
    KVQ_MFMA_BCAST_CASE(4) KVQ_MFMA_BCAST_CASE(5) KVQ_MFMA_BCAST_CASE(6) KVQ_MFMA_BCAST_CASE(7)
    KVQ_MFMA_BCAST_CASE(8) KVQ_MFMA_BCAST_CASE(9) KVQ_MFMA_BCAST_CASE(10) KVQ_MFMA_BCAST_CASE(11)
    KVQ_MFMA_BCAST_CASE(12) KVQ_MFMA_BCAST_CASE(13) KVQ_MFMA_BCAST_CASE(14)
    default:
      return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, 15, 0);
  }
#undef KVQ_MFMA_BCAST_CASE
}

// The query terms with one wave per (sequence, KV head, chunk of 64 key-mean
// windows) for all G <= 4 query heads of the KV head: sum_j q_rot_j mu_w,j
// for the chunk's windows is a [4 heads x 128] x [128 x 64 windows] product
// on 4x4x4 MFMA blocks.  Lane 4 b + n holds window 64 chunk + 4 b + n: its
// 128 int8 means are the B operand (4 per k-step, exact in fp16); the A
// operand, the rotated query scaled by 2^e and split into fp16 hi + lo, is
// broadcast from the block that holds the k-step (set t, block b: k-step
// 16 t + b, lane 4 b + m: head slot m).  The products are exact in fp32 and
// accumulate in fp32; the sum is then scaled by the window's mean scale and
// 2^-e.  Slots v >= G are zero.
template <int G>
__global__ __launch_bounds__(64) void prologue_mfma_kernel(Prologue2Args a) {
  const int lane = threadIdx.x;
  const int64_t chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int64_t s = blockIdx.z;
  __shared__ float qsh[4][kD];
  __shared__ float upsh[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float q[2], up;
    prologue_query(a, s, g, v, chunk, lane, q, &up);
    qsh[v][2 * lane] = q[0];
    qsh[v][2 * lane + 1] = q[1];
    if (lane == 0) upsh[v] = up;
  }
  __syncthreads();
  // A operand sets: lane 4 b + m, k-step c = 16 t + b of head slot m
  const int m = lane & 3, b = lane >> 2;
  const float upm = upsh[m];
  uint32_t ahi[2][2], alo[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float4 qv = *reinterpret_cast<const float4*>(&qsh[m][4 * (16 * t + b)]);
    const float qs[4] = {qv.x * upm, qv.y * upm, qv.z * upm, qv.w * upm};   // exact: a power of two
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const __half hi = __float2half_rn(qs[k]);
      hb[k] = __half_as_ushort(hi);
      lb[k] = __half_as_ushort(__float2half_rn(qs[k] - __half2float(hi)));
    }
    ahi[t][0] = hb[0] | (hb[1] << 16);
    ahi[t][1] = hb[2] | (hb[3] << 16);
    alo[t][0] = lb[0] | (lb[1] << 16);
    alo[t][1] = lb[2] | (lb[3] << 16);
  }
  // B operand: the lane's window (zero past the windows attended)
  const int64_t w = chunk * 64 + lane;
  uint4 mv[8];
  float sc = 0.f;
  if (w < a.nW) {
    sc = h2f(a.mean_scale[s * a.nW_cap + w]);
    const uint4* mq = reinterpret_cast<const uint4*>(a.mean_q + (s * a.nW_cap + w) * a.n + int64_t(g) * kD);
#pragma unroll
    for (int c = 0; c < 8; ++c) mv[c] = mq[c];
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) mv[c] = uint4{0u, 0u, 0u, 0u};
  }
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v off = {_Float16(1152.0f), _Float16(1152.0f)};
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    const uint32_t d = c % 4 == 0 ? mv[c / 4].x : c % 4 == 1 ? mv[c / 4].y : c % 4 == 2 ? mv[c / 4].z : mv[c / 4].w;
    // int8 x -> fp16: the bits 0x6400 | (x + 128) are 1024 + x + 128; minus 1152
    const uint32_t u = d ^ 0x80808080u;
    const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - off;
    const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - off;
    const half4_t B = {lo.x, lo.y, hi.x, hi.y};
    acc = mfma_bcast_a(as_half4(ahi[c / 16][0], ahi[c / 16][1]), B, acc, c % 16);
    acc = mfma_bcast_a(as_half4(alo[c / 16][0], alo[c / 16][1]), B, acc, c % 16);
  }
  if (w < a.nW) {
#pragma unroll
    for (int v = 0; v < G; ++v)
      a.qmu[(s * a.Hq + g * G + v) * a.nW + w] = acc[v] * (sc / upsh[v]);
  }
}

// PV over the 64 tokens of a tile for 64 channels: the int8 level indices of
// the [channel][token] chunk become fp16 through v_perm lookups (high bytes;
// with LO also the low bytes of non-integer levels) and are contracted on
// 4x4x4 MFMA blocks with the softmax weights (hi + lo parts) as A.
template <int NGM, bool LO>
__device__ inline void pv_half(const uint8_t* vch, int lane, int qn, const uint16_t* wv, const uint16_t* wv_lo,
                               uint32_t lutHi, uint32_t lutLo, uint32_t lutHi2, uint32_t lutLo2,
                               float4_t (&O)[NGM]) {
#pragma unroll 2
  for (int tq = 0; tq < 16; ++tq) {
    const uint32_t idx = *reinterpret_cast<const uint32_t*>(vch + lane * kChunk8Stride + 4 * tq);
    const uint32_t hb = __builtin_amdgcn_perm(lutHi, lutLo, idx);
    const uint32_t lb = LO ? __builtin_amdgcn_perm(lutHi2, lutLo2, idx) : 0u;
    const half4_t B = as_half4(__builtin_amdgcn_perm(hb, lb, 0x05010400u),
                               __builtin_amdgcn_perm(hb, lb, 0x07030602u));
#pragma unroll
    for (int m = 0; m < NGM; ++m) {
      const uint2 ah = *reinterpret_cast<const uint2*>(wv + (m * 4 + qn) * 64 + 4 * tq);
      const uint2 al = *reinterpret_cast<const uint2*>(wv_lo + (m * 4 + qn) * 64 + 4 * tq);
      O[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(ah.x, ah.y), B, O[m], 0, 0, 0);
      O[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(al.x, al.y), B, O[m], 0, 0, 0);
    }
  }
}

// -------------------------------- attention, K and V decode in separate waves
// The two waves of a pair share one split (token range of one sequence): the
// K wave decodes the K stream of (tile, KV head), contracts it with the query,
// runs the online softmax and stores the head's weights; the V wave decodes
// the V stream of the same (tile, head) and contracts it with those weights.
// Each wave runs one decode chain, and a CU holds 16 waves (8 pairs, 4 waves
// per SIMD), so each SIMD interleaves four independent chains.
//
// Steps are (tile, head) in order.  The waves of a pair hand steps over
// through two LDS counters (pair_wait / pair_post), never through a
// workgroup barrier, so pairs do not wait for one another: the K wave stores
// step s's weights once the V wave has posted that it finished step s - 1,
// then posts s + 1; the V wave decodes the first half of step s (with at most
// 4 pairs per workgroup, both halves) before it waits for that post.
//
// LDS map: per pair (VCH: [64 ch][68] V level bytes of a half step; WTS: one
// step's [hi/lo][NW][64] fp16 weights; ALV: the step's rescale factors, a grow
// flag and the two counters; RUN: running max, sums and the tile's affine
// terms), then the pairs' rings (K ring 2p, V ring 2p + 1, 17 rows of 64
// dwords), then the K and V decode tables with REPS replicas (16, 8 or 4, the
// most that fit) - or, when it fits, the interleaved layout (PERM) below.
constexpr int kPairs = 8;

template <int G, int HKV>
struct Lay5 {
  static constexpr int HQ = G * HKV;
  static constexpr int NW = ((G + 3) / 4) * 4;
  static constexpr uint32_t VCH = 0;
  static constexpr uint32_t WTS = 64u * kChunk8Stride;
  static constexpr uint32_t WTS_BUF = 2u * NW * 64u * 2u;        // fp16 hi and lo weights of one step
  static constexpr uint32_t ALV = WTS + WTS_BUF;                   // [16] f32 (NW factors, flag at 15)
  static constexpr uint32_t RUN = ALV + 64u;                       // 6 x [HQ] f32
  static constexpr uint32_t SIZE = (RUN + 6u * HQ * 4u + 15u) & ~15u;
  static constexpr uint32_t RINGS = (kPairs * SIZE + 255u) & ~255u;
  static constexpr uint32_t RING_END = RINGS + 2u * kPairs * kRingBytes;
  static constexpr uint32_t tab_end(uint32_t reps) {
    return ((RING_END + 1024u * reps - 1u) / (1024u * reps) * (1024u * reps)) + 2u * 1024u * reps;
  }
  static constexpr uint32_t REPS = tab_end(16) <= 163840u ? 16u : tab_end(8) <= 163840u ? 8u : 4u;
  static constexpr uint32_t TAB_BYTES = 256u * REPS * 4u;
  static constexpr uint32_t TABK = (RING_END + TAB_BYTES - 1u) / TAB_BYTES * TAB_BYTES;
  static constexpr uint32_t TABV = TABK + TAB_BYTES;
  static constexpr uint32_t TOTAL = TABV + TAB_BYTES;
  static constexpr uint32_t SLOT_SHIFT = REPS == 16u ? 6u : REPS == 8u ? 5u : 4u;
  static_assert(TOTAL <= 163840u, "exceeds the LDS of a CU");

  // Interleaved layout (PERM), when it fits: decode-table slot z is row z
  // (256 bytes) of a 64 KiB region at P_TAB - K replica r at byte 4 r, V
  // replica r at 64 + 4 r (16 each) - so a lookup address is one v_perm;
  // bytes 128..255 of the rows hold 7 rings (row pitch 512 bytes, lanes
  // 0..31 and 32..63 in two consecutive table rows); the other 9 rings follow
  // in 512-byte rows shared by two rings (one at bytes 0 and 256, one at 128
  // and 384), and the free half of the last of them holds each pair's running
  // max, sums and rescale factors, 128 bytes apiece (HQ <= 32).
  static constexpr uint32_t P_AFF = WTS + WTS_BUF;            // per pair: VCH, WTS, affine terms
  static constexpr uint32_t P_SIZE = (P_AFF + 3u * HQ * 4u + 15u) & ~15u;
  static constexpr uint32_t P_TAB = (kPairs * P_SIZE + 255u) & ~255u;
  static constexpr uint32_t P_RING_BYTES = 17u * 512u;
  static constexpr int P_RINGS_IN_TAB = 7;
  static constexpr uint32_t P_RINGS = P_TAB + 65536u;
  static constexpr int P_PAIRS = (2 * kPairs - P_RINGS_IN_TAB + 1) / 2;
  static constexpr uint32_t P_TOTAL = P_RINGS + uint32_t(P_PAIRS) * P_RING_BYTES;
  // piece k (128 bytes) of the free half of the last ring block
  static constexpr uint32_t piece(int k) {
    return P_RINGS + uint32_t(P_PAIRS - 1) * P_RING_BYTES + uint32_t(k >> 1) * 512u + uint32_t(k & 1) * 256u + 128u;
  }
  static constexpr bool PERM = NW == 4 && HQ <= 32 && (2 * kPairs - P_RINGS_IN_TAB) % 2 == 1 &&
                               4 * kPairs <= 34 && P_TOTAL <= 163840u && P_TAB <= 65535u;
  static constexpr uint32_t LDS_BYTES = PERM ? P_TOTAL : TOTAL;
  static constexpr int RS = PERM ? 9 : 8;
  // pair p's rescale factors: [16] f32 (NW <= 8 factors, the flag at 15);
  // dwords 12 and 13 hold the pair's hand-off counters
  static constexpr uint32_t alv_off(int p) { return PERM ? piece(4 * p + 3) : uint32_t(p) * SIZE + ALV; }
  static constexpr uint32_t READY = 12u * 4u, DONE = 13u * 4u;
};

// Hand-off between the two waves of a pair through two LDS step counters,
// so that pairs never wait for one another (a workgroup barrier would hold
// every pair to the slowest one at each step).  The K wave posts `ready` =
// j + 1 once the weights of its step j are in LDS; the V wave posts `done` =
// j + 1 once it has read them.  Only LDS accesses are ordered around the
// counters: container loads in flight stay in flight.  A waiting wave polls
// once per 256-clock sleep, so that its polls take little issue time from the
// waves that share its SIMD.  The wait is bounded (2^20 polls, far beyond any
// step) so that no wave can spin for ever; both waves of a pair run the same
// step sequence, so the bound is never reached in a correct run.
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ void pair_wait(const uint32_t* counter, uint32_t want) {
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= want) break;
    __builtin_amdgcn_s_sleep(4);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void pair_post(uint32_t* counter, uint32_t value, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if (lane == 0) __hip_atomic_store(counter, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// In a full workgroup the waves of pairs p and p ^ 4 share a SIMD (wave w
// runs on SIMD w mod 4).  Issue favours the older waves, so without a
// correction pairs 0..3 run ahead and finish well before pairs 4..7, which
// then finish the launch with half the waves on each SIMD.  Once per step
// each wave compares its pair's progress with the other pair's (the same
// counter kind: ready for K waves, done for V waves) and takes the higher
// issue priority while its pair is behind, so the two pairs finish together.
// This changes only the order of issue, never what is computed.
__device__ __forceinline__ void balance_issue(uint32_t mine, const uint32_t* other) {
  const uint32_t theirs =
      __builtin_amdgcn_readfirstlane(__hip_atomic_load(other, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  if (mine < theirs)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// pv_half for integer V levels (every fp16 level has a zero low byte): the
// chunk holds the levels' fp16 high bytes (the V table entries carry them in
// place of the level index), and two v_perms place them over zero low bytes.
template <int NGM>
__device__ inline void pv_half_int(const uint8_t* vch, int lane, int qn, const uint16_t* wv, const uint16_t* wv_lo,
                                   float4_t (&O)[NGM]) {
  // 4 columns per batch: every LDS load of the batch first, then the
  // lookups and products
#pragma unroll
  for (int t0 = 0; t0 < 16; t0 += 4) {
    uint32_t idx[4];
    uint2 ah[4][NGM], al[4][NGM];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      idx[u] = *reinterpret_cast<const uint32_t*>(vch + lane * kChunk8Stride + 4 * (t0 + u));
#pragma unroll
      for (int m = 0; m < NGM; ++m) {
        ah[u][m] = *reinterpret_cast<const uint2*>(wv + (m * 4 + qn) * 64 + 4 * (t0 + u));
        al[u][m] = *reinterpret_cast<const uint2*>(wv_lo + (m * 4 + qn) * 64 + 4 * (t0 + u));
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t hb = idx[u];
      const half4_t B =
          as_half4(__builtin_amdgcn_perm(0u, hb, 0x010C000Cu), __builtin_amdgcn_perm(0u, hb, 0x030C020Cu));
#pragma unroll
      for (int m = 0; m < NGM; ++m) {
        O[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(ah[u][m].x, ah[u][m].y), B, O[m], 0, 0, 0);
        O[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(al[u][m].x, al[u][m].y), B, O[m], 0, 0, 0);
      }
    }
  }
}

// TL: containers in the tile layout (KVQ_LAYOUT_TILES), rows otherwise.
template <int G, int HKV, bool TL>
__global__ __launch_bounds__(128 * kPairs, 1) void attention5_kernel(Attn2Args a, int64_t S) {
  using Lay = Lay5<G, HKV>;
  constexpr int HQ = Lay::HQ;
  constexpr int NGM = (G + 3) / 4;
  constexpr int NW = Lay::NW;
  constexpr bool PERM = Lay::PERM;
  constexpr int RS = Lay::RS;
  constexpr uint32_t TAB = PERM ? Lay::P_TAB : 0u;
  // 8 query heads on more than 2 KV heads: the accumulators of all heads would
  // not fit the registers, so every split holds one tile (the host sets that
  // geometry) and the V wave writes each head's output right after its step.
  constexpr bool PERHEAD = G == 8 && HKV > 2;
  __shared__ __align__(16) uint8_t lds[Lay::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves 0 .. np-1 decode K, waves np .. 2np-1 decode V (pair w mod np), so
  // that every SIMD (wave index mod 4) hosts K and V waves alike
  const int np = int(blockDim.x >> 7);
  const bool kwave = w < np;
  const int pw = kwave ? w : w - np;  // pair within the workgroup

  // Decode tables: entry idx of the replicated table is the host's entry for
  // slot idx / NREP (one load from the kernel arguments).
  constexpr uint32_t NREP = PERM ? 16u : Lay::REPS;
#pragma unroll 4
  for (int idx = tid; idx < 256 * int(NREP); idx += int(blockDim.x)) {
    const uint32_t z = uint32_t(idx) / NREP;
    const uint32_t ek = a.tabk[z], ev = a.tabv[z];
    if (PERM) {
      const uint32_t row = Lay::P_TAB + z * 256u + (uint32_t(idx) % NREP) * 4u;
      *reinterpret_cast<uint32_t*>(lds + row) = ek;
      *reinterpret_cast<uint32_t*>(lds + row + 64u) = ev;
    } else {
      reinterpret_cast<uint32_t*>(lds + Lay::TABK)[idx] = ek;
      reinterpret_cast<uint32_t*>(lds + Lay::TABV)[idx] = ev;
    }
  }
  if (tid < int(blockDim.x >> 7)) {
    *reinterpret_cast<uint32_t*>(lds + Lay::alv_off(tid) + Lay::READY) = 0u;
    *reinterpret_cast<uint32_t*>(lds + Lay::alv_off(tid) + Lay::DONE) = 0u;
  }
  __syncthreads();

  // lane offset of ring i (2 pw + stream)
  auto ring_off = [&](int i) -> uint32_t {
    if (PERM) {
      const uint32_t lane_off = uint32_t(lane >> 5) * 256u + uint32_t(lane & 31) * 4u;
      if (i < Lay::P_RINGS_IN_TAB) return Lay::P_TAB + uint32_t(i) * Lay::P_RING_BYTES + 128u + lane_off;
      const int j = i - Lay::P_RINGS_IN_TAB;
      return Lay::P_RINGS + uint32_t(j / 2) * Lay::P_RING_BYTES + uint32_t(j % 2) * 128u + lane_off;
    }
    return Lay::RINGS + uint32_t(i) * kRingBytes + uint32_t(lane) * 4u;
  };

  const int64_t gp = int64_t(blockIdx.x) * (blockDim.x >> 7) + pw;
  if (gp >= S * a.nsplit) return;          // no split for this pair
  const int64_t s = gp / a.nsplit;
  const int split = int(gp - s * a.nsplit);

  uint8_t* const mine = lds + uint32_t(pw) * (PERM ? Lay::P_SIZE : Lay::SIZE);
  uint8_t* const vch = mine + Lay::VCH;
  uint16_t* const wts = reinterpret_cast<uint16_t*>(mine + Lay::WTS);
  float* const alv = reinterpret_cast<float*>(lds + Lay::alv_off(pw));
  uint32_t* const ready = reinterpret_cast<uint32_t*>(lds + Lay::alv_off(pw) + Lay::READY);
  uint32_t* const done = reinterpret_cast<uint32_t*>(lds + Lay::alv_off(pw) + Lay::DONE);
  // the other pair on this wave's SIMD (full workgroups only)
  const bool balance = np == kPairs;
  const uint32_t* const other_ready =
      reinterpret_cast<const uint32_t*>(lds + Lay::alv_off(pw ^ (kPairs / 2)) + Lay::READY);
  const uint32_t* const other_done =
      reinterpret_cast<const uint32_t*>(lds + Lay::alv_off(pw ^ (kPairs / 2)) + Lay::DONE);
  uint32_t step = 0;                  // steps of this wave so far (tile i, KV head g)
  float* const runM = reinterpret_cast<float*>(PERM ? lds + Lay::piece(4 * pw) : mine + Lay::RUN);
  float* const runL = PERM ? reinterpret_cast<float*>(lds + Lay::piece(4 * pw + 1)) : runM + HQ;
  float* const runZ = PERM ? reinterpret_cast<float*>(lds + Lay::piece(4 * pw + 2)) : runL + HQ;
  float* const affS = PERM ? reinterpret_cast<float*>(mine + Lay::P_AFF) : runZ + HQ;
  float* const affQ = affS + HQ;
  float* const affM = affQ + HQ;

  const int64_t tb = int64_t(split) * a.tokens_per_split;
  const int64_t te = tb + a.tokens_per_split < a.T ? tb + a.tokens_per_split : a.T;
  const int64_t NT = (te - tb) / 64;
  float* P = a.part + (s * a.part_splits + split) * int64_t(HQ) * (kD + 4);
  const int qn = lane & 3;

  if (kwave) {
    // ------------------------------------------------------------ K wave
    for (int h = lane; h < HQ; h += 64) {
      runM[h] = -__builtin_inff();
      runL[h] = 0.f;
      runZ[h] = 0.f;
    }
    float* sum_slot = runL;
    {
      int idx = 0;
#pragma unroll
      for (int b = 0, w2 = G; w2 >= 1; ++b, w2 >>= 1) idx += ((lane >> b) & 1) * w2;
      sum_slot = ((idx & 1) ? runZ : runL) + (idx >> 1);
    }
    const uint32_t toffK = opaque(PERM ? uint32_t(lane % 16) * 4u : Lay::TABK + uint32_t(lane % Lay::REPS) * 4u);
    Ring5 rk;
    rk.off = opaque(ring_off(2 * pw));
    wave_lds_fence();

    const uint4* qop = a.qop + s * (HKV * NGM * 32 * 4);
    const float* qscale = a.qscale + s * HQ;
    const float* qsum = a.qsum + s * HQ;
    const float* qmu = a.qmu + s * HQ * a.nW;
    const int qc0 = 16 * ((lane >> 2) >> 3) + ((lane >> 2) & 7);
    constexpr bool kQPrefetch = NGM == 1;
    uint4 qnx[NGM][2];
#pragma unroll
    for (int m = 0; m < NGM; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t) qnx[m][t] = kQPrefetch ? qop[(m * 32 + qc0 + 8 * t) * 4 + qn] : uint4{};

    const uint8_t* const kseq = a.k_cont + s * (TL ? a.seq_bytes_k : a.T_cap * a.CK);
    const __amdgpu_buffer_rsrc_t rsK = seq_rsrc(kseq, uint32_t(a.T * (TL ? a.CKs : a.CK)));
    const uint32_t misK = uint32_t(reinterpret_cast<uintptr_t>(kseq) & 15u);
    uint32_t xk = 0;
    float sk = 0.f, ok = 0.f, svK = 0.f, ovK = 0.f;
    for (int64_t i = 0; i < NT; ++i) {
      const int64_t tK = tb + 64 * i;
#pragma unroll 1
      for (int g = 0; g < HKV; ++g) {
        if (balance) balance_issue(step, other_ready);
        if (g == 0) {
          const int64_t row = s * a.T_cap + tK + lane;
          xk = ring5_start<RS, TL>(
              rk, lds, rsK,
              TL ? misK + uint32_t(tK) * uint32_t(a.CKs) + uint32_t(lane) * 4u
                 : misK + uint32_t(tK + lane) * uint32_t(a.CK),
              uint32_t(a.CK));
          sk = h2f(a.k_so[2 * row]);
          ok = h2f(a.k_so[2 * row + 1]);
          svK = h2f(a.v_so[2 * row]);
          ovK = h2f(a.v_so[2 * row + 1]);
          const int64_t wdx = tK >> a.log2W;
          // logits are kept in log2 units: tau log2(e) folds into the affine terms
          const float tl = a.tau * 1.4426950408889634f;
          for (int h = lane; h < HQ; h += 64) {
            affS[h] = tl * qscale[h];
            affQ[h] = tl * qsum[h];
            affM[h] = tl * qmu[h * a.nW + wdx];
          }
          wave_lds_fence();
        }
        float4_t D[NGM];
#pragma unroll
        for (int m = 0; m < NGM; ++m) D[m] = float4_t{0.f, 0.f, 0.f, 0.f};
        uint4 qh[NGM][2];
        {
          const int gn = kQPrefetch ? (g + 1 < HKV ? g + 1 : 0) : g;
          const uint4* qg = qop + gn * (NGM * 32 * 4) + qn;
#pragma unroll
          for (int m = 0; m < NGM; ++m)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              if (kQPrefetch) {
                qh[m][t] = qnx[m][t];
                qnx[m][t] = qg[(m * 32 + qc0 + 8 * t) * 4];
              } else {
                qh[m][t] = qg[(m * 32 + qc0 + 8 * t) * 4];
              }
            }
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
            for (int bh = 0; bh < 2; ++bh) {
              if (bh == 1) ring5_block<1, RS, TL>(rk, lds, rsK);
              else ring5_block<0, RS, TL>(rk, lds, rsK);
#pragma unroll
              for (int cc = 0; cc < 4; ++cc) {
                uint32_t e[4];
                dec5_group<PERM, Lay::SLOT_SHIFT, TAB, RS>(xk, rk, lds, toffK, e);
                const half4_t B = as_half4(__builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                                           __builtin_amdgcn_perm(e[3], e[2], 0x07060302u));
#pragma unroll
                for (int m = 0; m < NGM; ++m) {
                  D[m] = mfma_bcast_a(as_half4(qh[m][0].x, qh[m][0].y), B, D[m], 8 * ch + 4 * bh + cc);
                  D[m] = mfma_bcast_a(as_half4(qh[m][0].z, qh[m][0].w), B, D[m], 8 * ch + 4 * bh + cc);
                }
              }
              if (bh == 1) {
#pragma unroll
                for (int m = 0; m < NGM; ++m) {
                  const uint4 t = qh[m][0];
                  qh[m][0] = qh[m][1];
                  qh[m][1] = t;
                }
              }
            }
        }
        // logits -> online softmax (lazy running maximum) -> weights of this step
        float sums[2 * G];
        uint32_t wbits[NW];             // fp16 hi (low half) and lo (high half) weight
        float alf[NW];
        bool grew = false;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          const int m = v / 4, ii = v % 4;
          float whi = 0.f, wlo = 0.f, alh = 1.f;
          if (v < G) {
            const int h = g * G + v;
            const float lg = __builtin_fmaf(sk, D[m][ii] * affS[h], __builtin_fmaf(ok, affQ[h], affM[h]));
            float Mr = runM[h];
            if (__builtin_amdgcn_ballot_w64(lg > Mr) != 0) {
              const float Mn = fmaxf(Mr, wave_max_dpp(lg));
              alh = __builtin_amdgcn_exp2f(Mr - Mn);
              runL[h] *= alh;
              runZ[h] *= alh;
              grew = true;
              Mr = Mn;
              runM[h] = Mn;
            }
            const float p = __builtin_amdgcn_exp2f(lg - Mr);
            sums[2 * v] = p;
            sums[2 * v + 1] = p * ovK;
            const float wt = p * svK;
            const __half hh = __float2half_rn(wt);
            whi = wt;
            wlo = wt - __half2float(hh);
          }
          wbits[v] = uint32_t(__half_as_ushort(__float2half_rn(whi))) |
                     (uint32_t(__half_as_ushort(__float2half_rn(wlo))) << 16);
          alf[v] = alh;
        }
        const float tot = wave_sum_scatter<2 * G>(sums, lane);
        if (lane < 2 * G) atomicAdd(sum_slot + g * G, tot);
        // one weight buffer per pair: free once the V wave has finished the
        // previous step (it decodes the first half of its next step meanwhile)
        pair_wait(done, step);
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          wts[v * 64 + lane] = uint16_t(wbits[v]);
          wts[NW * 64 + v * 64 + lane] = uint16_t(wbits[v] >> 16);
          if (lane == 0) alv[v] = alf[v];
        }
        if (lane == 0) alv[15] = grew ? 1.f : 0.f;
        pair_post(ready, ++step, lane);
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int v = 0; v < G; ++v)
      for (int g = 0; g < HKV; ++g) {
        const int h = g * G + v;
        if (lane == 0) {
          P[h * (kD + 4) + kD] = runM[h] * 0.6931471805599453f;      // back to natural log units
          P[h * (kD + 4) + kD + 1] = runL[h];
          P[h * (kD + 4) + kD + 2] = runZ[h];
        }
      }
    return;
  }

  // -------------------------------------------------------------- V wave
  const uint32_t toffV = opaque(PERM ? 64u + uint32_t(lane % 16) * 4u : Lay::TABV + uint32_t(lane % Lay::REPS) * 4u);
  Ring5 rv;
  rv.off = opaque(ring_off(2 * pw + 1));
  // fp16 bytes of the V levels as v_perm lookups (non-integer levels only:
  // for integer levels the decoded entries already hold the high bytes)
  const uint32_t lutLo = a.hbv[0] | (a.hbv[1] << 8) | (a.hbv[2] << 16) | (a.hbv[3] << 24);
  const uint32_t lutHi = a.hbv[4] | (a.hbv[5] << 8) | (a.hbv[6] << 16) | (a.hbv[7] << 24);
  const uint32_t lutLo2 = a.lbv[0] | (a.lbv[1] << 8) | (a.lbv[2] << 16) | (a.lbv[3] << 24);
  const uint32_t lutHi2 = a.lbv[4] | (a.lbv[5] << 8) | (a.lbv[6] << 16) | (a.lbv[7] << 24);
  const bool lo_levels = a.v_lo_nonzero != 0;
  // A workgroup of at most 4 pairs leaves pairs 4..7's areas unused: there
  // the V wave keeps the second half of a step in pair pw + 4's VCH area and
  // decodes a whole step before it needs the step's weights.
  constexpr uint32_t kVch2 = uint32_t(kPairs / 2) * (PERM ? Lay::P_SIZE : Lay::SIZE);
  const bool two_vch = blockDim.x <= 128u * (kPairs / 2);
  // Output accumulators, rotated once per step so that V's head is O[0]; after
  // NT HKV steps O[j] holds KV head j again.
  float4_t O[HKV][2][NGM];
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int m = 0; m < NGM; ++m) O[g][c][m] = float4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* const vseq = a.v_cont + s * (TL ? a.seq_bytes_v : a.T_cap * a.CV);
  const __amdgpu_buffer_rsrc_t rsV = seq_rsrc(vseq, uint32_t(a.T * (TL ? a.CVs : a.CV)));
  const uint32_t misV = uint32_t(reinterpret_cast<uintptr_t>(vseq) & 15u);
  uint32_t xv = 0;
  if constexpr (PERHEAD) {
    for (int64_t i = 0; i < NT; ++i) {                  // NT == 1
      const int64_t tV = tb + 64 * i;
#pragma unroll 1
      for (int g = 0; g < HKV; ++g) {
        if (balance) balance_issue(step, other_done);
        if (g == 0) xv = ring5_start<RS, TL>(rv, lds, rsV,
                                             TL ? misV + uint32_t(tV) * uint32_t(a.CVs) + uint32_t(lane) * 4u
                                                : misV + uint32_t(tV + lane) * uint32_t(a.CV),
                                             uint32_t(a.CV));
        const uint16_t* const wv = wts;
        const uint16_t* const wv_lo = wv + NW * 64;
        float4_t Oc[2][NGM];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int m = 0; m < NGM; ++m) Oc[c][m] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
#pragma unroll 1
          for (int b2 = 0; b2 < 2; ++b2) {
            uint32_t epend = 0;
#pragma unroll
            for (int bh = 0; bh < 2; ++bh) {
              const int b4 = 2 * b2 + bh;
              if (bh == 1) ring5_block<1, RS, TL>(rv, lds, rsV);
              else ring5_block<0, RS, TL>(rv, lds, rsV);
#pragma unroll
              for (int cc = 0; cc < 4; ++cc)
                dec5_group_v<PERM, Lay::SLOT_SHIFT, TAB, RS>(xv, rv, lds, toffV,
                                                             vch + (b4 * 16 + cc * 4) * kChunk8Stride + lane, epend,
                                                             bh == 0 && cc == 0);
            }
            vch[(b2 * 32 + 31) * kChunk8Stride + lane] = uint8_t(epend >> 16);
          }
          if (ch == 0) pair_wait(ready, step + 1u);     // the K wave's weights of (i, g)
          wave_lds_fence();
          if (lo_levels)
            pv_half<NGM, true>(vch, lane, qn, wv, wv_lo, lutHi, lutLo, lutHi2, lutLo2, Oc[ch]);
          else
            pv_half_int<NGM>(vch, lane, qn, wv, wv_lo, Oc[ch]);
          wave_lds_fence();
        }
        pair_post(done, ++step, lane);
        // the split's only tile: this head's accumulators are final
#pragma unroll
        for (int m = 0; m < NGM; ++m)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int v = m * 4 + ii;
            if (v < G) {
              const int h = g * G + v;
#pragma unroll
              for (int c = 0; c < 2; ++c) P[h * (kD + 4) + c * 64 + lane] = Oc[c][m][ii];
            }
          }
      }
    }
    return;
  }
  for (int64_t i = 0; i < NT; ++i) {
    const int64_t tV = tb + 64 * i;
#pragma unroll 1
    for (int g = 0; g < HKV; ++g) {
      if (balance) balance_issue(step, other_done);
      if (g == 0) xv = ring5_start<RS, TL>(rv, lds, rsV,
                                             TL ? misV + uint32_t(tV) * uint32_t(a.CVs) + uint32_t(lane) * 4u
                                                : misV + uint32_t(tV + lane) * uint32_t(a.CV),
                                             uint32_t(a.CV));
      const uint16_t* const wv = wts;
      const uint16_t* const wv_lo = wv + NW * 64;
      auto rescale = [&]() {
        if (alv[15] != 0.f) {
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int m = 0; m < NGM; ++m)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) O[0][c][m][ii] *= alv[m * 4 + ii];
        }
      };
      auto pv = [&](const uint8_t* vc, int ch) {
        wave_lds_fence();
        if (lo_levels)
          pv_half<NGM, true>(vc, lane, qn, wv, wv_lo, lutHi, lutLo, lutHi2, lutLo2, O[0][ch]);
        else
          pv_half_int<NGM>(vc, lane, qn, wv, wv_lo, O[0][ch]);
        wave_lds_fence();
      };
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        uint8_t* const vc = vch + (ch == 1 && two_vch ? kVch2 : 0u);
#pragma unroll 1
        for (int b2 = 0; b2 < 2; ++b2) {
          uint32_t epend = 0;
#pragma unroll
          for (int bh = 0; bh < 2; ++bh) {
            const int b4 = 2 * b2 + bh;
            if (bh == 1) ring5_block<1, RS, TL>(rv, lds, rsV);
            else ring5_block<0, RS, TL>(rv, lds, rsV);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
              dec5_group_v<PERM, Lay::SLOT_SHIFT, TAB, RS>(xv, rv, lds, toffV,
                                                           vc + (b4 * 16 + cc * 4) * kChunk8Stride + lane, epend,
                                                           bh == 0 && cc == 0);
          }
          vc[(b2 * 32 + 31) * kChunk8Stride + lane] = uint8_t(epend >> 16);
        }
        if (two_vch) {
          // both halves decoded before the step's weights are needed
          if (ch == 1) {
            pair_wait(ready, step + 1u);                // the K wave's weights of (i, g)
            rescale();
            pv(vch, 0);
            pv(vch + kVch2, 1);
          }
        } else {
          if (ch == 0) {
            pair_wait(ready, step + 1u);                // the K wave's weights of (i, g)
            rescale();
          }
          pv(vch, ch);
        }
      }
      pair_post(done, ++step, lane);
      // rotate: the next step's head becomes O[0]
      if (HKV > 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            const float4_t t = O[0][c][m];
#pragma unroll
            for (int j = 0; j + 1 < HKV; ++j) O[j][c][m] = O[j + 1][c][m];
            O[HKV - 1][c][m] = t;
          }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int m = 0; m < NGM; ++m)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int v = m * 4 + ii;
        if (v < G) {
          const int h = g * G + v;
#pragma unroll
          for (int c = 0; c < 2; ++c) P[h * (kD + 4) + c * 64 + lane] = O[g][c][m][ii];
        }
      }
}

// ------------------------------------------------ fixed-width comparator
// [D-Quant] Appendix B compares the entropy-coded container with fixed-width
// symbols at the same preprocessing.  Symbol i = 4c + r of a stream sits in
// byte r of dword c / (8/B), bits B (c mod 8/B) .. + B, so the 4 symbols of
// channel quad c are (dword >> shift) & mask with one symbol per byte, and a
// KV head's 128 symbols are 4 B contiguous dwords at a fixed offset.  Same
// contractions and softmax as the entropy-coded kernels (one wave per split,
// K head g then V head g); the decoder is a shift and a mask per 4 symbols.
template <int N>
__device__ inline uint32_t dword_of(const uint4 (&v)[N], int i) {
  const uint4 q = v[i / 4];
  return (i % 4 == 0) ? q.x : (i % 4 == 1) ? q.y : (i % 4 == 2) ? q.z : q.w;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, fully unrolled.
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F& f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      StaticFor<B + 1, E>::run(f);
    }
  }
};

// One lane's K and V bit vectors of KV head g of token t, and the head's query
// operand in the broadcast layout (register r holds channel quad 16 r + the
// lane's MFMA block).
template <int KQ, int VQ, int NGM>
__device__ __forceinline__ void fw_fetch(uint4 (&kd)[KQ], uint4 (&vd)[VQ], uint4 (&qd)[NGM][2],
                                         const Attn2Args& a, int64_t s, int64_t t, int g, int lane,
                                         const uint4* qop, int qn) {
  const int64_t rw = s * a.T_cap + t + lane;
  const uint4* kr = reinterpret_cast<const uint4*>(a.k_cont + rw * a.CK) + g * KQ;
  const uint4* vr = reinterpret_cast<const uint4*>(a.v_cont + rw * a.CV) + g * VQ;
#pragma unroll
  for (int j = 0; j < KQ; ++j) kd[j] = kr[j];
#pragma unroll
  for (int j = 0; j < VQ; ++j) vd[j] = vr[j];
  const uint4* qg = qop + g * (NGM * 32 * 4) + qn;
#pragma unroll
  for (int m = 0; m < NGM; ++m)
#pragma unroll
    for (int r = 0; r < 2; ++r) qd[m][r] = qg[(m * 32 + 16 * r + (lane >> 2)) * 4];
}

template <int G, int HKV, int BK, int BV>
__global__ __launch_bounds__(64) void attention_fw_kernel(Attn2Args a) {
  constexpr int HQ = G * HKV;
  constexpr int NGM = (G + 3) / 4;
  constexpr int NW = NGM * 4;
  constexpr int KW = 128 * BK / 32, VW = 128 * BV / 32;    // dwords per head
  constexpr int KPER = 8 / BK, VPER = 8 / BV;              // channel quads per dword
  constexpr uint32_t KMASK = ((1u << BK) - 1u) * 0x01010101u;
  constexpr uint32_t VMASK = ((1u << BV) - 1u) * 0x01010101u;
  __shared__ __align__(16) uint8_t vch[64 * kChunk8Stride];
  __shared__ __align__(16) uint16_t wts[2][NW][64];       // [hi/lo][slot][token]
  __shared__ float runM[HQ], runL[HQ], runZ[HQ];
  __shared__ float affS[HQ], affQ[HQ], affM[HQ];

  const int lane = threadIdx.x;
  const int64_t s = blockIdx.y;
  const int split = blockIdx.x;
  for (int h = lane; h < HQ; h += 64) {
    runM[h] = -__builtin_inff();
    runL[h] = 0.f;
    runZ[h] = 0.f;
  }
  for (int i = lane; i < 2 * NW * 64; i += 64) (&wts[0][0][0])[i] = 0;
  const uint32_t lutLoK = a.hbk[0] | (a.hbk[1] << 8) | (a.hbk[2] << 16) | (a.hbk[3] << 24);
  const uint32_t lutHiK = a.hbk[4] | (a.hbk[5] << 8) | (a.hbk[6] << 16) | (a.hbk[7] << 24);
  const uint32_t lutLoV = a.hbv[0] | (a.hbv[1] << 8) | (a.hbv[2] << 16) | (a.hbv[3] << 24);
  const uint32_t lutHiV = a.hbv[4] | (a.hbv[5] << 8) | (a.hbv[6] << 16) | (a.hbv[7] << 24);
  wave_lds_fence();

  // Output accumulators, rotated once per head step (as in the entropy-coded
  // kernel) so the loop over heads needs no register indexing: during head g's
  // step O[0] holds head g, and after the last head O[j] holds head j again.
  float4_t O[HKV][2][NGM];
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int m = 0; m < NGM; ++m) O[g][c][m] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t tb = int64_t(split) * a.tokens_per_split;
  const int64_t te = tb + a.tokens_per_split < a.T ? tb + a.tokens_per_split : a.T;
  const uint4* qop = a.qop + s * (HKV * NGM * 32 * 4);
  const float* qscale = a.qscale + s * HQ;
  const float* qsum = a.qsum + s * HQ;
  const float* qmu = a.qmu + s * HQ * a.nW;
  const int qn = lane & 3;

  // Per head, one lane's whole K and V bit vectors (KW and VW dwords) and the
  // query operand are registers, fetched one head ahead (the next tile's first
  // head after the last), so no load is waited for inside a head.  The query
  // operand of channel quad c lives in register c / 16 of the lanes of MFMA
  // block c mod 16, which the QK^T MFMA broadcasts to all blocks (CBSZ = 4).
  // With two MFMA groups the prefetch would not fit the registers: the head's
  // own loads are issued at its start instead.
  constexpr bool kPre = NGM == 1;
  constexpr int KQ = KW / 4, VQ = VW / 4;                  // uint4 per head
  uint4 kn[KQ], vn[VQ], qn4[NGM][2];
  if (kPre) fw_fetch<KQ, VQ, NGM>(kn, vn, qn4, a, s, tb, 0, lane, qop, qn);

  for (int64_t t0 = tb; t0 < te; t0 += 64) {
    const int64_t row = s * a.T_cap + t0 + lane;
    const float sk = h2f(a.k_so[2 * row]), ok = h2f(a.k_so[2 * row + 1]);
    const float sv = h2f(a.v_so[2 * row]), ov = h2f(a.v_so[2 * row + 1]);
    const int64_t wdx = t0 >> a.log2W;
    for (int h = lane; h < HQ; h += 64) {
      affS[h] = qscale[h];
      affQ[h] = qsum[h];
      affM[h] = qmu[h * a.nW + wdx];
    }
    wave_lds_fence();
#pragma unroll 1
    for (int g = 0; g < HKV; ++g) {
      uint4 kc[KQ], vc[VQ], qh[NGM][2];
      if (kPre) {
#pragma unroll
        for (int j = 0; j < KQ; ++j) kc[j] = kn[j];
#pragma unroll
        for (int j = 0; j < VQ; ++j) vc[j] = vn[j];
#pragma unroll
        for (int m = 0; m < NGM; ++m) {
          qh[m][0] = qn4[m][0];
          qh[m][1] = qn4[m][1];
        }
        // the next head of this tile, else the next tile's first (the last
        // head of the last tile refetches the current tile: in bounds, unused)
        const bool last = g + 1 == HKV;
        const int64_t tn = last && t0 + 64 < te ? t0 + 64 : t0;
        fw_fetch<KQ, VQ, NGM>(kn, vn, qn4, a, s, tn, last ? 0 : g + 1, lane, qop, qn);
      } else {
        fw_fetch<KQ, VQ, NGM>(kc, vc, qh, a, s, t0, g, lane, qop, qn);
      }
      // ---- QK^T on the K levels of head g, one MFMA pair per channel quad
      float4_t D[NGM];
#pragma unroll
      for (int m = 0; m < NGM; ++m) D[m] = float4_t{0.f, 0.f, 0.f, 0.f};
      // (a compile-time loop: the quad's dword, shift, register and MFMA block
      // are all constants)
      auto qk_quad = [&](auto cq) __attribute__((always_inline)) {
        constexpr int c = decltype(cq)::value;
        const uint32_t sym = (dword_of(kc, c / KPER) >> (BK * (c % KPER))) & KMASK;
        const uint32_t hb = __builtin_amdgcn_perm(lutHiK, lutLoK, sym);
        const half4_t B = as_half4(__builtin_amdgcn_perm(0u, hb, 0x010C000Cu),
                                   __builtin_amdgcn_perm(0u, hb, 0x030C020Cu));
#pragma unroll
        for (int m = 0; m < NGM; ++m) {
          const uint4 q4 = qh[m][c / 16];
          D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(q4.x, q4.y), B, D[m], 4, c % 16, 0);
          D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(q4.z, q4.w), B, D[m], 4, c % 16, 0);
        }
      };
      StaticFor<0, 32>::run(qk_quad);
      // ---- online softmax of this KV head's query heads over the tile
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int m = v / 4, ii = v % 4;
        float whi = 0.f, wlo = 0.f;
        if (v < G) {
          const int h = g * G + v;
          const float lg = a.tau * (sk * (D[m][ii] * affS[h]) + ok * affQ[h] + affM[h]);
          const float tmax = wave_max_dpp(lg);
          const float Mo = runM[h], Lo = runL[h], Zo = runZ[h];
          const float Mn = fmaxf(Mo, tmax);
          const float al = __expf(Mo - Mn);
          const float p = __expf(lg - Mn);
          const float ls = wave_sum_dpp(p);
          const float zs = wave_sum_dpp(p * ov);
          runM[h] = Mn;
          runL[h] = Lo * al + ls;
          runZ[h] = Zo * al + zs;
#pragma unroll
          for (int c = 0; c < 2; ++c) O[0][c][m][ii] *= al;
          const float wt = p * sv;
          const __half hh = __float2half_rn(wt);
          whi = wt;
          wlo = wt - __half2float(hh);
        }
        wts[0][v][lane] = __half_as_ushort(__float2half_rn(whi));
        wts[1][v][lane] = __half_as_ushort(__float2half_rn(wlo));
      }
      // ---- V levels of head g, 64 channels at a time, then PV
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        wave_lds_fence();
#pragma unroll
        for (int cq = 0; cq < 16; ++cq) {
          const int c = ch * 16 + cq;
          const uint32_t sym = (dword_of(vc, c / VPER) >> (BV * (c % VPER))) & VMASK;
          uint8_t* col = vch + (4 * cq) * kChunk8Stride + lane;
          col[0] = uint8_t(sym);
          col[kChunk8Stride] = uint8_t(sym >> 8);
          col[2 * kChunk8Stride] = uint8_t(sym >> 16);
          col[3 * kChunk8Stride] = uint8_t(sym >> 24);
        }
        wave_lds_fence();
#pragma unroll 2
        for (int tq = 0; tq < 16; ++tq) {
          const uint32_t idx = *reinterpret_cast<const uint32_t*>(vch + lane * kChunk8Stride + 4 * tq);
          const uint32_t hb = __builtin_amdgcn_perm(lutHiV, lutLoV, idx);
          const half4_t B = as_half4(__builtin_amdgcn_perm(0u, hb, 0x010C000Cu),
                                     __builtin_amdgcn_perm(0u, hb, 0x030C020Cu));
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            const uint2 ah = *reinterpret_cast<const uint2*>(&wts[0][m * 4 + qn][4 * tq]);
            const uint2 al = *reinterpret_cast<const uint2*>(&wts[1][m * 4 + qn][4 * tq]);
            O[0][ch][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(ah.x, ah.y), B, O[0][ch][m], 0, 0, 0);
            O[0][ch][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(al.x, al.y), B, O[0][ch][m], 0, 0, 0);
          }
        }
      }
      wave_lds_fence();
      // rotate: the next head's accumulators become O[0]
      if (HKV > 1) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            const float4_t t = O[0][c][m];
#pragma unroll
            for (int j = 0; j + 1 < HKV; ++j) O[j][c][m] = O[j + 1][c][m];
            O[HKV - 1][c][m] = t;
          }
      }
    }
  }

  float* P = a.part + (s * a.part_splits + split) * int64_t(HQ) * (kD + 4);
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int m = 0; m < NGM; ++m)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int v = m * 4 + ii;
        if (v < G) {
          const int h = g * G + v;
#pragma unroll
          for (int c = 0; c < 2; ++c) P[h * (kD + 4) + c * 64 + lane] = O[g][c][m][ii];
          if (lane == 0) {
            P[h * (kD + 4) + kD] = runM[h];
            P[h * (kD + 4) + kD + 1] = runL[h];
            P[h * (kD + 4) + kD + 2] = runZ[h];
          }
        }
      }
}

}  // namespace

hipError_t launch_prologue2(const Prologue2Args& a, int64_t S, hipStream_t stream) {
  const int ngm = (a.G + 3) / 4;
  const int hkv = a.Hq / a.G;
  const int64_t chunks = (a.nW + 63) / 64;
  if (chunks * ngm * 4 > int64_t(0x7FFFFFFF)) return hipErrorInvalidValue;
  // up to 4 query heads per KV head and at least 4 such waves per CU: one wave
  // for all of them, the window sums on MFMA; otherwise one wave per query
  // slot (more, shorter waves)
  if (a.G <= 4 && S * hkv * chunks >= 1024) {
    const dim3 grid{unsigned(chunks), unsigned(hkv), unsigned(S)};
    if (a.G == 1) hipLaunchKernelGGL(prologue_mfma_kernel<1>, grid, dim3(64), 0, stream, a);
    else if (a.G == 2) hipLaunchKernelGGL(prologue_mfma_kernel<2>, grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL(prologue_mfma_kernel<4>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(prologue2_kernel, dim3(unsigned(chunks * ngm * 4), unsigned(hkv), unsigned(S)), dim3(64), 0,
                     stream, a);
  return hipGetLastError();
}

bool attention2_supported(int Hq, int G, int d, int levels_k, int levels_v, int window, bool affine) {
  const int hkv = Hq / G;
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  const bool h_ok = hkv == 1 || hkv == 2 || hkv == 4 || hkv == 8;
  if (d != kD || !g_ok || !h_ok || window < 64) return false;
  // the split-wave kernel takes any key levels and up to 8 value levels; the
  // single-wave one (9 value levels) needs integer levels
  if (levels_v <= 8) return true;
  return affine && levels_k <= 9 && levels_v <= 9;
}

template <int G, int HKV>
static hipError_t launch_attn2_t(const Attn2Args& a, int64_t S, hipStream_t stream) {
  // the split-wave kernel keeps V levels as bytes (fp16 high byte or, for
  // non-integer levels, an index into an 8-entry lookup), so it serves V
  // alphabets of up to 8 levels
  if (a.Mv <= 8) {
    // 8 query heads on more than 2 KV heads need splits of one tile
    if (G == 8 && HKV > 2 && a.tokens_per_split != 64) return hipErrorInvalidValue;
    const int64_t pairs = S * a.nsplit;
    constexpr int64_t kCUs = 256;
    int64_t ppw = (pairs + kCUs - 1) / kCUs;
    ppw = ppw < 1 ? 1 : (ppw > kPairs ? kPairs : ppw);
    const dim3 grid(unsigned((pairs + ppw - 1) / ppw)), block(unsigned(128 * ppw));
    if (a.tiles)
      hipLaunchKernelGGL((attention5_kernel<G, HKV, true>), grid, block, 0, stream, a, S);
    else
      hipLaunchKernelGGL((attention5_kernel<G, HKV, false>), grid, block, 0, stream, a, S);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((attention2_kernel<G, HKV>), dim3(a.nsplit, unsigned(S)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_attn2_g(const Attn2Args& a, int64_t S, int hkv, hipStream_t stream) {
  switch (hkv) {
    case 1: return launch_attn2_t<G, 1>(a, S, stream);
    case 2: return launch_attn2_t<G, 2>(a, S, stream);
    case 4: return launch_attn2_t<G, 4>(a, S, stream);
    case 8: return launch_attn2_t<G, 8>(a, S, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention2(const Attn2Args& a, int64_t S, int Hq, int G, hipStream_t stream) {
  const int hkv = Hq / G;
  switch (G) {
    case 1: return launch_attn2_g<1>(a, S, hkv, stream);
    case 2: return launch_attn2_g<2>(a, S, hkv, stream);
    case 4: return launch_attn2_g<4>(a, S, hkv, stream);
    case 8: return launch_attn2_g<8>(a, S, hkv, stream);
  }
  return hipErrorInvalidValue;
}

template <int G, int HKV>
static hipError_t launch_fw_t(const Attn2Args& a, int64_t S, int bk, int bv, hipStream_t stream) {
  const dim3 grid(a.nsplit, unsigned(S));
  if (bk == 4 && bv == 2)
    hipLaunchKernelGGL((attention_fw_kernel<G, HKV, 4, 2>), grid, dim3(64), 0, stream, a);
  else if (bk == 4 && bv == 4)
    hipLaunchKernelGGL((attention_fw_kernel<G, HKV, 4, 4>), grid, dim3(64), 0, stream, a);
  else if (bk == 2 && bv == 2)
    hipLaunchKernelGGL((attention_fw_kernel<G, HKV, 2, 2>), grid, dim3(64), 0, stream, a);
  else if (bk == 2 && bv == 1)
    hipLaunchKernelGGL((attention_fw_kernel<G, HKV, 2, 1>), grid, dim3(64), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int G>
static hipError_t launch_fw_g(const Attn2Args& a, int64_t S, int hkv, int bk, int bv, hipStream_t stream) {
  switch (hkv) {
    case 1: return launch_fw_t<G, 1>(a, S, bk, bv, stream);
    case 2: return launch_fw_t<G, 2>(a, S, bk, bv, stream);
    case 4: return launch_fw_t<G, 4>(a, S, bk, bv, stream);
    case 8: return launch_fw_t<G, 8>(a, S, bk, bv, stream);
  }
  return hipErrorInvalidValue;
}

bool attention_fw_supported(int Hq, int G, int d, int bk, int bv, int levels_k, int levels_v) {
  const int hkv = Hq / G;
  const bool widths = (bk == 4 && (bv == 2 || bv == 4)) || (bk == 2 && (bv == 2 || bv == 1));
  return d == kD && (G == 1 || G == 2 || G == 4 || G == 8) && (hkv == 1 || hkv == 2 || hkv == 4 || hkv == 8) &&
         widths && levels_k <= 8 && levels_v <= 8;
}

hipError_t launch_attention_fw(const Attn2Args& a, int64_t S, int Hq, int G, int bk, int bv,
                               hipStream_t stream) {
  const int hkv = Hq / G;
  switch (G) {
    case 1: return launch_fw_g<1>(a, S, hkv, bk, bv, stream);
    case 2: return launch_fw_g<2>(a, S, hkv, bk, bv, stream);
    case 4: return launch_fw_g<4>(a, S, hkv, bk, bv, stream);
    case 8: return launch_fw_g<8>(a, S, hkv, bk, bv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
