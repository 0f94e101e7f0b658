// Read side: container decoding and fused decode attention.
//
// [D-Quant] Appendix A, Algorithm 2: the state is read little-endian from the
// first four bytes; each step looks up T[z] for z = x mod 256, which gives the
// symbol (the reconstruction level), f and z - c; x = f floor(x / 256) + z - c;
// while x < 2^23 one more byte is shifted in.  Eqs. (7)-(9): the affine
// parameters fold into the contractions, q.k_t = s_t sum_j q_j m_tj +
// o_t sum_j q_j + sum_j q_j mu_j and sum_t a_t v_t = sum_t (a_t s_t) m_t +
// sum_t a_t o_t, so decoded levels are consumed without dequantising.  §4.5
// "Decoding": the kernel is token-centric, every stream is decoded exactly once
// and feeds all query heads of each KV head in turn.
//
// This file holds the standalone container decoder and the split combine of
// decode attention (the prologue and the fused kernel are in attention.hip):
//   combine   merges the splits by log-sum-exp, rotates back (H is symmetric
//             and orthonormal) and writes bf16 / fp32.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.h"

namespace kvq {
namespace {

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// ----------------------------------------------------------------- symbols
__global__ __launch_bounds__(256) void decode_symbols_kernel(DecSymArgs a) {
  __shared__ uint32_t tab[256];
  tab[threadIdx.x] = a.dec[threadIdx.x];
  __syncthreads();
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= a.n_streams) return;
  // byte j of the stream: row layout s C + j; tile layout, dword j / 4 of the
  // 64 containers of a tile side by side
  const uint8_t* const p = a.tiles ? a.cont + (s >> 6) * 64 * int64_t(a.cs) + (s & 63) * 4 : a.cont + s * a.C;
  auto at = [&](int j) -> uint32_t { return a.tiles ? p[(j >> 2) * 256 + (j & 3)] : p[j]; };
  uint32_t x = at(0) | (at(1) << 8) | (at(2) << 16) | (at(3) << 24);
  int ptr = 4;
  uint8_t* out = a.sym + s * a.n;
  for (int i = 0; i < a.n; ++i) {
    const uint32_t e = tab[x & 0xFFu];
    out[i] = uint8_t(e >> 16);
    x = (e & 0xFFu) * (x >> 8) + ((e >> 8) & 0xFFu);
    // a well-formed stream needs at most one byte per symbol; the bound keeps
    // malformed input from looping
    for (int r = 0; r < 2 && x < kStateLow; ++r) {
      const uint32_t b = ptr < a.C ? at(ptr) : 0u;
      x = (x << 8) | b;
      ++ptr;
    }
  }
  if (a.end_ok) a.end_ok[s] = (x == kStateLow) ? 1u : 0u;
}

// ----------------------------------------------------------------- combine
// One workgroup per (query head, sequence).  Its waves share the splits: each
// merges a contiguous range of at most kCombineChunk splits per round (the
// maxima, sums and weights spread over the lanes, the partial outputs of the
// whole round loaded before any is used, so that a round costs one memory
// latency), then wave 0 merges the waves' results through LDS, undoes the
// rotation and stores.  A single long sequence has thousands of splits: then a
// first pass (FINAL = false, one workgroup per (query head, sequence, group of
// `group` splits)) merges each group into the group's first slot, in place (a
// group is read only by its own workgroup), and the final pass merges those
// slots, `group` apart.
constexpr int kCombineMaxWaves = 16;
constexpr int kCombineChunk = 16;          // splits per wave and round
constexpr int kCombineGroup = 64;          // splits per first-pass workgroup
constexpr int kCombineTwoPass = 128;       // split counts above this take two passes

template <int NPL, bool FINAL>
__global__ __launch_bounds__(64 * kCombineMaxWaves) void combine_kernel(CombineArgs a, int group) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const int h = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int stride = a.d + 4;
  const int64_t sp = int64_t(a.Hq) * stride;
  // the splits this workgroup merges: cnt slots, `step` apart, from `first`
  const int first = FINAL ? 0 : int(blockIdx.z) * group;
  const int step = FINAL ? group : 1;
  const int cnt = FINAL ? (a.nsplit + group - 1) / group
                        : (a.nsplit - first < group ? a.nsplit - first : group);
  const float* P = a.part + (s * a.nsplit + first) * sp + int64_t(h) * stride;
  const int per = (cnt + nwv - 1) / nwv;
  const int kb = wv * per;
  const int ke = kb + per < cnt ? kb + per : cnt;
  // with one round of splits (the common case) the maximum comes from that
  // round's own loads; otherwise from a pass over the splits' maxima first
  const bool one_round = ke - kb <= kCombineChunk;
  float Mx = -__builtin_inff();
  if (!one_round) {
    for (int k = kb + lane; k < ke; k += 64) Mx = fmaxf(Mx, P[int64_t(k) * step * sp + a.d]);
    Mx = wave_max(Mx);
  }
  float L = 0.f, Z = 0.f;
  float acc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
  if (one_round || Mx > -__builtin_inff()) {
    for (int k0 = kb; k0 < ke; k0 += kCombineChunk) {
      const int kn = ke - k0 < kCombineChunk ? ke - k0 : kCombineChunk;
      // every load of the round first: lane j < kn the max and sums of split
      // k0 + j, each lane its NPL channels of the kn partial outputs
      float mk = -__builtin_inff(), lk = 0.f, zk = 0.f;
      if (lane < kn) {
        const float* Pk = P + int64_t(k0 + lane) * step * sp;
        mk = Pk[a.d];
        lk = Pk[a.d + 1];
        zk = Pk[a.d + 2];
      }
      float v[kCombineChunk][NPL];
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j)
#pragma unroll
        for (int i = 0; i < NPL; ++i)
          v[j][i] = j < kn ? P[int64_t(k0 + j) * step * sp + lane * NPL + i] : 0.f;
      if (one_round) {
        Mx = wave_max(mk);
        if (!(Mx > -__builtin_inff())) break;           // no split holds a token
      }
      const float sck = lane < kn ? __expf(mk - Mx) : 0.f;
      L += wave_sum_f32(sck * lk);
      Z += wave_sum_f32(sck * zk);
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        const float sc = __shfl(sck, j, 64);            // 0 past kn
#pragma unroll
        for (int i = 0; i < NPL; ++i) acc[i] += sc * v[j][i];
      }
    }
  }
  float M = Mx;
  if (nwv > 1) {
    __shared__ float red[kCombineMaxWaves][64 * NPL + 4];
    if (lane == 0) {
      red[wv][64 * NPL] = Mx;
      red[wv][64 * NPL + 1] = L;
      red[wv][64 * NPL + 2] = Z;
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) red[wv][lane * NPL + i] = acc[i];
    __syncthreads();
    if (wv != 0) return;
    M = -__builtin_inff();
    for (int w = 0; w < nwv; ++w) M = fmaxf(M, red[w][64 * NPL]);
    L = 0.f;
    Z = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
    for (int w = 0; w < nwv; ++w) {
      const float sc = __expf(red[w][64 * NPL] - M);     // 0 for a wave without splits
      L += sc * red[w][64 * NPL + 1];
      Z += sc * red[w][64 * NPL + 2];
#pragma unroll
      for (int i = 0; i < NPL; ++i) acc[i] += sc * red[w][lane * NPL + i];
    }
  }
  if (!FINAL) {
    // the merged partial replaces the group's first slot (already read)
    float* Q = const_cast<float*>(P);
#pragma unroll
    for (int i = 0; i < NPL; ++i) Q[lane * NPL + i] = acc[i];
    if (lane == 0) {
      Q[a.d] = M;
      Q[a.d + 1] = L;
      Q[a.d + 2] = Z;
    }
    return;
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[i] = (acc[i] + Z) * inv;
  fwht_lanes<NPL>(acc, a.d, lane, a.hscale);
  const int64_t ob = (s * a.Hq + h) * a.d + lane * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    // round to nearest even into bf16
    const uint32_t u = __float_as_uint(acc[i]);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    a.out[ob + i] = uint16_t(r >> 16);
    if (a.out_f32) a.out_f32[ob + i] = acc[i];
  }
}

// Few splits (at most kCombineChunk): one wave per (query head, sequence)
// merges all of them in one round, kCombineHeads heads per workgroup and no
// LDS, so that the launch's many small workgroups are not held back by the
// multi-wave kernel's reduction buffer (8 KiB per workgroup) and run in
// fewer rounds.  Same arithmetic as one wave of combine_kernel in one round.
constexpr int kCombineHeads = 8;

template <int NPL>
__global__ __launch_bounds__(64 * kCombineHeads) void combine_heads_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int h = int(blockIdx.x) * kCombineHeads + int(threadIdx.x >> 6);
  if (h >= a.Hq) return;
  const int64_t s = blockIdx.y;
  const int stride = a.d + 4;
  const int64_t sp = int64_t(a.Hq) * stride;
  const int kn = a.nsplit;                            // <= kCombineChunk
  const float* P = a.part + s * a.nsplit * sp + int64_t(h) * stride;
  float mk = -__builtin_inff(), lk = 0.f, zk = 0.f;
  if (lane < kn) {
    const float* Pk = P + int64_t(lane) * sp;
    mk = Pk[a.d];
    lk = Pk[a.d + 1];
    zk = Pk[a.d + 2];
  }
  float v[kCombineChunk][NPL];
#pragma unroll
  for (int j = 0; j < kCombineChunk; ++j)
#pragma unroll
    for (int i = 0; i < NPL; ++i) v[j][i] = j < kn ? P[int64_t(j) * sp + lane * NPL + i] : 0.f;
  const float M = wave_max(mk);
  float acc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
  float L = 0.f, Z = 0.f;
  if (M > -__builtin_inff()) {
    const float sck = lane < kn ? __expf(mk - M) : 0.f;
    L = wave_sum_f32(sck * lk);
    Z = wave_sum_f32(sck * zk);
#pragma unroll
    for (int j = 0; j < kCombineChunk; ++j) {
      const float sc = __shfl(sck, j, 64);            // 0 past kn
#pragma unroll
      for (int i = 0; i < NPL; ++i) acc[i] += sc * v[j][i];
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[i] = (acc[i] + Z) * inv;
  fwht_lanes<NPL>(acc, a.d, lane, a.hscale);
  const int64_t ob = (s * a.Hq + h) * a.d + lane * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const uint32_t u = __float_as_uint(acc[i]);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    a.out[ob + i] = uint16_t(r >> 16);
    if (a.out_f32) a.out_f32[ob + i] = acc[i];
  }
}

// ---------------------------------------------------------------- residual
// The most recent tokens of every sequence kept uncompressed in bf16
// ([D-Quant] §5.1 "Implementation details") join the same softmax as one more
// split of partials.  One wave per (KV head, sequence): per 64-token chunk,
// lane t gets the logits of token t for the G query heads, the chunk's
// max / sum update the running softmax state, and lane j then accumulates
// channels 2j, 2j+1 of sum_t p_t v_t.  The accumulator is rotated (orthonormal
// Hadamard, its own inverse) so that it matches the rotated partials of the
// compressed splits; the offset sum Z is zero.
//
// The logits are a [4 heads x 128] x [128 x 64 tokens] product per group of 4
// query heads on bf16 4x4x4 MFMA blocks: block b, column n is token 4 b + n
// (the lane's own token), whose key row supplies the B operand 4 channels per
// k-step straight from its bf16 pairs; the query is the A operand, broadcast
// from the block that holds the k-step (k-step c in block c mod 16, slot
// c / 16).  Products of bf16 values are exact in fp32 and accumulate in fp32.
// The result of block b is the lane's 4 heads' logits.
constexpr int kResMaxG = 8;

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float res_f4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4_t as_bf16x4(uint32_t lo, uint32_t hi) {
  const uint2 u = {lo, hi};
  return __builtin_bit_cast(bf16x4_t, u);
}

// bf16 4x4x4 MFMA with the A operand broadcast from block `abid` (a literal
// after unrolling, so the switch folds to one instruction).
__device__ __attribute__((always_inline)) inline res_f4_t mfma_bf16_bcast(bf16x4_t a, bf16x4_t b, res_f4_t c,
                                                                          int abid) {
#define KVQ_RES_MFMA_CASE(i) \
  case i:                    \
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 4, i, 0);
  switch (abid) {
    KVQ_RES_MFMA_CASE(0) KVQ_RES_MFMA_CASE(1) KVQ_RES_MFMA_CASE(2) KVQ_RES_MFMA_CASE(3)
    KVQ_RES_MFMA_CASE(4) KVQ_RES_MFMA_CASE(5) KVQ_RES_MFMA_CASE(6) KVQ_RES_MFMA_CASE(7)
    KVQ_RES_MFMA_CASE(8) KVQ_RES_MFMA_CASE(9) KVQ_RES_MFMA_CASE(10) KVQ_RES_MFMA_CASE(11)
    KVQ_RES_MFMA_CASE(12) KVQ_RES_MFMA_CASE(13) KVQ_RES_MFMA_CASE(14)
    default:
      return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 4, 15, 0);
  }
#undef KVQ_RES_MFMA_CASE
}

__global__ __launch_bounds__(64) void residual_kernel(ResidualArgs a) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int G = a.G, d = a.d;                 // d == 128: two channels per lane
  const int hkv = a.Hq / G;
  __shared__ float ps[kResMaxG][64];
  // half a chunk's value rows, token t at (t mod 32) kResRow bytes (16 bytes
  // of padding per row spread the lanes' 16-byte stores over the banks); half
  // a chunk keeps the workgroup's LDS small enough for 12 waves per CU
  constexpr int kResRow = 272;
  __shared__ __align__(16) uint8_t vst[32 * kResRow];
  // A operands: query head 4 m + (lane & 3), channels 4 c .. 4 c + 3 of
  // k-steps c = lane / 4 and lane / 4 + 16 (zero for head slots >= G)
  uint2 qa[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int h = 4 * m + (lane & 3), c = (lane >> 2) + 16 * i;
      qa[m][i] = h < G ? *reinterpret_cast<const uint2*>(a.q + (s * a.Hq + g * G + h) * d + 4 * c) : uint2{0u, 0u};
    }
  float M[kResMaxG], L[kResMaxG], acc[kResMaxG][2];
#pragma unroll
  for (int h = 0; h < kResMaxG; ++h) {
    M[h] = -__builtin_inff();
    L[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }
  const int64_t row_stride = int64_t(hkv) * d;          // elements per token
  const uint16_t* kb = a.k + (s * a.R_cap) * row_stride + int64_t(g) * d;
  const uint16_t* vb = a.v + (s * a.R_cap) * row_stride + int64_t(g) * d;
  for (int64_t t0 = 0; t0 < a.R; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool live = t < a.R;
    // the token's 128 key values as 16 independent 16-byte loads (zero past the tail)
    uint4 kv[16];
    if (live) {
      const uint4* kr = reinterpret_cast<const uint4*>(kb + t * row_stride);
#pragma unroll
      for (int c = 0; c < 16; ++c) kv[c] = kr[c];
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) kv[c] = uint4{0u, 0u, 0u, 0u};
    }
    res_f4_t D[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const bf16x4_t B = (c & 1) ? as_bf16x4(kv[c >> 1].z, kv[c >> 1].w) : as_bf16x4(kv[c >> 1].x, kv[c >> 1].y);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (4 * m < G) D[m] = mfma_bf16_bcast(as_bf16x4(qa[m][c >> 4].x, qa[m][c >> 4].y), B, D[m], c & 15);
    }
    float lg[kResMaxG];
#pragma unroll
    for (int h = 0; h < kResMaxG; ++h) lg[h] = D[h >> 2][h & 3];
    // the token's value row, loaded like its key row (in flight during the
    // softmax) and staged in LDS, so that the products below read value rows
    // from LDS instead of waiting on memory 8 rows at a time
    uint4 vv[16];
    if (live) {
      const uint4* vr = reinterpret_cast<const uint4*>(vb + t * row_stride);
#pragma unroll
      for (int c = 0; c < 16; ++c) vv[c] = vr[c];
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) vv[c] = uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kResMaxG; ++h) {
      if (h < G) {
        const float l = live ? lg[h] * a.tau : -__builtin_inff();
        const float mx = fmaxf(M[h], wave_max(l));
        const float al = __expf(M[h] - mx);             // 0 on the first chunk
        const float p = live ? __expf(l - mx) : 0.f;
        L[h] = L[h] * al + wave_sum_f32(p);
        M[h] = mx;
        acc[h][0] *= al;
        acc[h][1] *= al;
        ps[h][lane] = p;
      }
    }
    const int tn = int(a.R - t0 < 64 ? a.R - t0 : 64);
    for (int hb = 0; hb < tn; hb += 32) {
      if ((lane >> 5) == (hb >> 5)) {
#pragma unroll
        for (int c = 0; c < 16; ++c) *reinterpret_cast<uint4*>(vst + (lane & 31) * kResRow + 16 * c) = vv[c];
      }
      __syncthreads();
      const int he = tn < hb + 32 ? tn : hb + 32;
      for (int u0 = hb; u0 < he; u0 += 8) {
        uint32_t two[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          two[e] = *reinterpret_cast<const uint32_t*>(vst + ((u0 + e) & 31) * kResRow + 4 * lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v0 = __uint_as_float(two[e] << 16), v1 = __uint_as_float(two[e] & 0xFFFF0000u);
#pragma unroll
          for (int h = 0; h < kResMaxG; ++h)
            if (h < G && u0 + e < he) {
              acc[h][0] += ps[h][u0 + e] * v0;
              acc[h][1] += ps[h][u0 + e] * v1;
            }
        }
      }
      __syncthreads();
    }
  }
  const int stride = d + 4;
#pragma unroll
  for (int h = 0; h < kResMaxG; ++h) {
    if (h < G) {
      float o[2] = {acc[h][0], acc[h][1]};
      fwht_lanes<2>(o, d, lane, a.hscale);
      float* P = a.part + ((s * a.nsplit_total + a.split) * a.Hq + g * G + h) * int64_t(stride);
      P[2 * lane] = o[0];
      P[2 * lane + 1] = o[1];
      if (lane == 0) {
        P[d] = M[h];
        P[d + 1] = L[h];
        P[d + 2] = 0.f;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_symbols(const DecSymArgs& a, hipStream_t stream) {
  const unsigned blocks = unsigned((a.n_streams + 255) / 256);
  hipLaunchKernelGGL(decode_symbols_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int NPL>
static hipError_t launch_combine_t(const CombineArgs& a, int64_t S, hipStream_t stream) {
  if (a.nsplit <= kCombineChunk) {
    const dim3 grid(unsigned((a.Hq + kCombineHeads - 1) / kCombineHeads), unsigned(S));
    hipLaunchKernelGGL((combine_heads_kernel<NPL>), grid, dim3(64 * kCombineHeads), 0, stream, a);
    return hipGetLastError();
  }
  int group = 1;
  if (a.nsplit > kCombineTwoPass) {
    group = kCombineGroup;
    const dim3 grid1(a.Hq, unsigned(S), unsigned((a.nsplit + group - 1) / group));
    hipLaunchKernelGGL((combine_kernel<NPL, false>), grid1, dim3(64 * (kCombineGroup / kCombineChunk)), 0, stream,
                       a, group);
  }
  // one round of kCombineChunk merged slots per wave, up to 16 waves per
  // (query head, sequence)
  const int slots = (a.nsplit + group - 1) / group;
  int waves = (slots + kCombineChunk - 1) / kCombineChunk;
  waves = waves < 1 ? 1 : (waves > kCombineMaxWaves ? kCombineMaxWaves : waves);
  hipLaunchKernelGGL((combine_kernel<NPL, true>), dim3(a.Hq, unsigned(S)), dim3(64 * waves), 0, stream, a, group);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int64_t S, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_combine_t<1>(a, S, stream);
    case 128: return launch_combine_t<2>(a, S, stream);
    case 256: return launch_combine_t<4>(a, S, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_residual(const ResidualArgs& a, int64_t S, hipStream_t stream) {
  if (a.d != 128 || a.G < 1 || a.G > kResMaxG) return hipErrorInvalidValue;
  hipLaunchKernelGGL(residual_kernel, dim3(unsigned(a.Hq / a.G), unsigned(S)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvq
