// Fused decode attention over entropy-coded containers, tuned for gfx950.
//
// [D-Quant] §4.5 "Decoding": the kernel is token-centric - every stream is
// decoded exactly once and its levels feed all query heads of the current KV
// head.  Appendix A, Algorithm 2 gives the per-symbol decoder; Eqs. (8)-(9)
// let the contractions run on the raw levels with the affine terms applied
// afterwards.
//
// Layout of one workgroup (a single wave, 64 lanes) handling a token range of
// one sequence in 64-token tiles, lane t <-> token t0 + t:
//   * Container bytes reach the decoder through a 64-byte ring per lane in
//     LDS, refilled with 16-byte aligned global loads issued two 16-symbol
//     blocks before they are needed (a lane consumes at most one byte per
//     symbol), so only 4 KiB of LDS per wave holds compressed bytes.
//   * The 256-entry decode table lives in LDS as 8-byte entries:
//       lo = f | fp16(level) high byte << 24   (bits 8..23 clear)
//       hi = z - c
//     so one v_mad_u32_u24 performs x = f (x >> 8) + z - c, and the fp16 level
//     (levels 0..8 have a zero low byte) sits in the upper half of lo.
//   * QK^T: every 4 decoded K levels of a lane form the B operand of a
//     v_mfma_f32_4x4x4f16 block (16 blocks of 4 tokens); the A operand is the
//     rotated query of 4 heads, split into fp16 hi + lo parts after a
//     power-of-two scaling, so each lane ends with its own token's logits.
//   * PV: V levels are written as fp16 into a [64 channels][64 tokens] LDS
//     chunk; the contraction over tokens is again 4x4x4 MFMA blocks (16
//     channel groups x 4 heads) with the softmax weights (hi + lo) as A.
//   * Online softmax per query head across tiles; the per-token scale folds
//     into the weights and the per-token offset into a separate sum (Eq. 9).

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

// ------------------------------------------------------------------ prologue
// One wave per (sequence, KV head, query slot v): slot v < G is query head
// g G + v; slots up to the next multiple of 4 are zero padding.  Writes the
// MFMA A operand (rotated query scaled by 2^e so that max |q| is in
// [2^7, 2^8), split into fp16 hi + lo), the inverse scale, sum_j q_rot_j and
// sum_j q_rot_j mu_w,j for every key-mean window w.
__global__ __launch_bounds__(64) void prologue2_kernel(Prologue2Args a) {
  const int lane = threadIdx.x;
  const int v = blockIdx.x;          // query slot in [0, NGM*4)
  const int g = blockIdx.y;
  const int64_t s = blockIdx.z;
  const int hkv = a.Hq / a.G;
  const int ngm = (a.G + 3) / 4;
  const bool real = v < a.G;
  const int h = g * a.G + v;
  float q[2] = {0.f, 0.f};
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
  // operand layout: [s][g][gm][c = j/4][n][hi0..3 lo0..3]
  const int gm = v / 4, n = v % 4;
  uint16_t* op = a.qop + ((((s * hkv + g) * ngm + gm) * 32) * 4) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
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
  if (lane == 0) {
    a.qsum[s * a.Hq + h] = qs;
    a.qscale[s * a.Hq + h] = ldexpf(1.0f, -e);
  }
  for (int64_t w = 0; w < a.nW; ++w) {
    const float sc = h2f(a.mean_scale[s * a.nW + w]);
    const int8_t* mq = a.mean_q + (s * a.nW + w) * a.n + int64_t(g) * kD + lane * 2;
    float acc = q[0] * __fmul_rn(float(mq[0]), sc) + q[1] * __fmul_rn(float(mq[1]), sc);
    acc = wave_sum_f(acc);
    if (lane == 0) a.qmu[(s * a.Hq + h) * a.nW + w] = acc;
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
    const int64_t row = s * a.T + t0 + lane;
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
  float* P = a.part + (s * a.nsplit + split) * int64_t(HQ) * (kD + 4);
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


// ----------------------------------------------------------- attention (v3)
// Two decode chains per lane: while the K stream of (tile i, KV head g) is
// decoded and contracted with the query, the V stream of the head before it
// in (tile, head) order is decoded into the int8 transpose chunk and
// contracted with that head's softmax weights.  Only one head group of logits
// is live at a time.  The first iteration's V work and the last iteration's K
// work are dummies on valid containers (zero weights, discarded logits).
constexpr int kChunk8Stride = 68;   // bytes per channel row of the int8 V chunk

template <int G, int HKV>
__global__ __launch_bounds__(64, 2) void attention3_kernel(Attn2Args a) {
  constexpr int HQ = G * HKV;
  constexpr int NGM = (G + 3) / 4;
  constexpr int NW = NGM * 4;
  __shared__ uint2 tabK[256], tabV[256];
  __shared__ __align__(16) uint8_t ringK[64 * kRingStride];
  __shared__ __align__(16) uint8_t ringV[64 * kRingStride];
  __shared__ __align__(16) uint8_t vch[64 * kChunk8Stride];
  __shared__ __align__(16) uint16_t wts[2][2][NW][64];   // [buffer][hi/lo][slot][token]
  __shared__ float runM[HQ], runL[HQ], runZ[HQ];
  __shared__ float affS[HQ], affQ[HQ], affM[HQ];

  const int lane = threadIdx.x;
  const int64_t s = blockIdx.y;
  const int split = blockIdx.x;
  uint8_t* const rK = ringK + lane * kRingStride;
  uint8_t* const rV = ringV + lane * kRingStride;

  for (int z = lane; z < 256; z += 64) {
    uint32_t mk = 0, mv = 0;
    for (int m = 1; m < a.Mk; ++m) mk = (uint32_t(z) >= a.ck[m]) ? uint32_t(m) : mk;
    for (int m = 1; m < a.Mv; ++m) mv = (uint32_t(z) >= a.cv[m]) ? uint32_t(m) : mv;
    tabK[z] = make_uint2(a.fk[mk] | (a.hbk[mk] << 24), uint32_t(z) - a.ck[mk]);
    tabV[z] = make_uint2(a.fv[mv] | (mv << 24), uint32_t(z) - a.cv[mv]);   // V: level index
  }
  for (int h = lane; h < HQ; h += 64) {
    runM[h] = -__builtin_inff();
    runL[h] = 0.f;
    runZ[h] = 0.f;
  }
  for (int i = lane; i < 2 * 2 * NW * 64; i += 64) (&wts[0][0][0][0])[i] = 0;
  __syncthreads();

  // fp16 high bytes of levels 0..7 as a v_perm lookup (low byte is zero)
  const uint32_t lutLo = a.hbv[0] | (a.hbv[1] << 8) | (a.hbv[2] << 16) | (a.hbv[3] << 24);
  const uint32_t lutHi = a.hbv[4] | (a.hbv[5] << 8) | (a.hbv[6] << 16) | (a.hbv[7] << 24);

  float4_t O[HKV][2][NGM];
#pragma unroll
  for (int g = 0; g < HKV; ++g)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int m = 0; m < NGM; ++m) O[g][c][m] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t tb = int64_t(split) * a.tokens_per_split;
  const int64_t te = tb + a.tokens_per_split < a.T ? tb + a.tokens_per_split : a.T;
  const int64_t NT = (te - tb) / 64;
  const uint4* qop = a.qop + s * (HKV * NGM * 32 * 4);
  const float* qscale = a.qscale + s * HQ;
  const float* qsum = a.qsum + s * HQ;
  const float* qmu = a.qmu + s * HQ * a.nW;
  const int qn = lane & 3;

  Ring rk, rv;
  uint32_t xk = 0, xv = 0;
  float sk = 0.f, ok = 0.f, svK = 0.f, ovK = 0.f;

  for (int64_t i = 0; i <= NT; ++i) {
    const bool kreal = i < NT;
    const int64_t tK = tb + 64 * (kreal ? i : NT - 1);        // K tile (clamped dummy)
#pragma unroll
    for (int g = 0; g < HKV; ++g) {
      if (!kreal && g > 0) break;
      // ---- stream starts
      if (g == 0) {
        const int64_t row = s * a.T + tK + lane;
        xk = ring_start(rk, rK, a.k_cont + row * a.CK, uint32_t(a.CK));
        sk = h2f(a.k_so[2 * row]);
        ok = h2f(a.k_so[2 * row + 1]);
        svK = h2f(a.v_so[2 * row]);
        ovK = h2f(a.v_so[2 * row + 1]);
        const int64_t w = tK >> a.log2W;
        __syncthreads();
        for (int h = lane; h < HQ; h += 64) {
          affS[h] = qscale[h];
          affQ[h] = qsum[h];
          affM[h] = qmu[h * a.nW + w];
        }
        __syncthreads();
      }
      const int vg = (g + HKV - 1) % HKV;                      // V's KV head this iteration
      if (vg == 0 || (i == 0 && g == 0)) {                     // V starts a container
        // (the very first iteration always starts one: its V work is the
        // dummy on tile 0, and the ring must point at valid memory)
        const int64_t vt = (g == 0) ? i - 1 : i;               // V's tile (-1: dummy on tile 0)
        const int64_t tV = tb + 64 * (vt < 0 ? 0 : (vt >= NT ? NT - 1 : vt));
        xv = ring_start(rv, rV, a.v_cont + (s * a.T + tV + lane) * a.CV, uint32_t(a.CV));
      }
      const uint16_t* wv = &wts[(i * HKV + g + 1) & 1][0][0][0];   // weights of V's head
      const uint16_t* wv_lo = wv + NW * 64;

      float4_t D[NGM];
#pragma unroll
      for (int m = 0; m < NGM; ++m) D[m] = float4_t{0.f, 0.f, 0.f, 0.f};
      const uint4* qg = qop + g * (NGM * 32 * 4) + qn;
      uint4 qa[NGM];
#pragma unroll
      for (int m = 0; m < NGM; ++m) qa[m] = qg[(m * 32) * 4];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll 1
        for (int b4 = 0; b4 < 4; ++b4) {
          const int blk = ch * 4 + b4;
          if (b4 & 1) {
            ring_block<1>(rk, rK);
            ring_block<1>(rv, rV);
          } else {
            ring_block<0>(rk, rK);
            ring_block<0>(rv, rV);
          }
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const int c = blk * 4 + cc;
            const int cn = c + 1 < 32 ? c + 1 : 31;
            uint4 qb[NGM];
#pragma unroll
            for (int m = 0; m < NGM; ++m) qb[m] = qg[(m * 32 + cn) * 4];
            uint32_t e[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              e[r] = dec_step(xk, rk, tabK, rK);
              const uint32_t ev = dec_step(xv, rv, tabV, rV);
              vch[(b4 * 16 + cc * 4 + r) * kChunk8Stride + lane] = uint8_t(ev >> 24);
            }
            const half4_t B = as_half4(__builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                                       __builtin_amdgcn_perm(e[3], e[2], 0x07060302u));
#pragma unroll
            for (int m = 0; m < NGM; ++m) {
              D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(qa[m].x, qa[m].y), B, D[m], 0, 0, 0);
              D[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(qa[m].z, qa[m].w), B, D[m], 0, 0, 0);
              qa[m] = qb[m];
            }
          }
        }
        // PV of V's head for the 64 channels of this half
        __syncthreads();
#pragma unroll 2
        for (int tq = 0; tq < 16; ++tq) {
          const uint32_t idx = *reinterpret_cast<const uint32_t*>(vch + lane * kChunk8Stride + 4 * tq);
          const uint32_t hb = __builtin_amdgcn_perm(lutHi, lutLo, idx);
          const half4_t B = as_half4(__builtin_amdgcn_perm(0u, hb, 0x010C000Cu),
                                     __builtin_amdgcn_perm(0u, hb, 0x030C020Cu));
#pragma unroll
          for (int m = 0; m < NGM; ++m) {
            const uint2 ah = *reinterpret_cast<const uint2*>(wv + (m * 4 + qn) * 64 + 4 * tq);
            const uint2 al = *reinterpret_cast<const uint2*>(wv_lo + (m * 4 + qn) * 64 + 4 * tq);
            O[vg][ch][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(ah.x, ah.y), B, O[vg][ch][m], 0, 0, 0);
            O[vg][ch][m] = __builtin_amdgcn_mfma_f32_4x4x4f16(as_half4(al.x, al.y), B, O[vg][ch][m], 0, 0, 0);
          }
        }
        __syncthreads();
      }
      // ---- K head g done: logits -> online softmax -> weights for the next iteration
      if (kreal) {
        uint16_t* wk = &wts[(i * HKV + g) & 1][0][0][0];
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          const int m = v / 4, ii = v % 4;
          float whi = 0.f, wlo = 0.f;
          if (v < G) {
            const int h = g * G + v;
            const float lg = a.tau * (sk * (D[m][ii] * affS[h]) + ok * affQ[h] + affM[h]);
            const float tmax = wave_max_f(lg);
            const float Mo = runM[h], Lo = runL[h], Zo = runZ[h];
            const float Mn = fmaxf(Mo, tmax);
            const float al = __expf(Mo - Mn);
            const float p = __expf(lg - Mn);
            const float ls = wave_sum_f(p);
            const float zs = wave_sum_f(p * ovK);
            __syncthreads();
            runM[h] = Mn;
            runL[h] = Lo * al + ls;
            runZ[h] = Zo * al + zs;
#pragma unroll
            for (int c = 0; c < 2; ++c) O[g][c][m][ii] *= al;
            const float wt = p * svK;
            const __half hh = __float2half_rn(wt);
            whi = wt;
            wlo = wt - __half2float(hh);
          }
          wk[v * 64 + lane] = __half_as_ushort(__float2half_rn(whi));
          wk[NW * 64 + v * 64 + lane] = __half_as_ushort(__float2half_rn(wlo));
        }
        __syncthreads();
      }
    }
  }

  float* P = a.part + (s * a.nsplit + split) * int64_t(HQ) * (kD + 4);
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
  hipLaunchKernelGGL(prologue2_kernel, dim3(ngm * 4, a.Hq / a.G, unsigned(S)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

bool attention2_supported(int Hq, int G, int d, int levels_k, int levels_v, int window) {
  const int hkv = Hq / G;
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  const bool h_ok = hkv == 1 || hkv == 2 || hkv == 4 || hkv == 8;
  return d == kD && g_ok && h_ok && levels_k <= 9 && levels_v <= 9 && window >= 64;
}

template <int G, int HKV>
static hipError_t launch_attn2_t(const Attn2Args& a, int64_t S, hipStream_t stream) {
  // the interleaved kernel keeps V levels as int8 and maps them to fp16 with
  // an 8-entry lookup, so it serves V alphabets of up to 8 levels
  if (a.Mv <= 8)
    hipLaunchKernelGGL((attention3_kernel<G, HKV>), dim3(a.nsplit, unsigned(S)), dim3(64), 0, stream, a);
  else
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

}  // namespace kvq
