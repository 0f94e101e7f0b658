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
// Decode attention runs as three launches on the caller's stream:
//   prologue  q_rot = H q per head, sum_j q_rot_j, and sum_j q_rot_j mu_w,j
//             for every key-mean window w;
//   attention split-K over tokens: each workgroup owns a token range, decodes
//             the K containers of 64-token tiles, forms logits, keeps an
//             online softmax, decodes the V containers and accumulates PV;
//   combine   merges the splits by log-sum-exp, rotates back (H is symmetric
//             and orthonormal) and writes bf16 / fp32.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.h"

namespace kvq {
namespace {

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// One step of Algorithm 2 on a container staged in LDS.  `pend` is the last
// byte of the lane's container: reads never leave it, whatever the bytes.
__device__ inline uint32_t decode_step(const uint32_t* tab, const uint8_t* cont, uint32_t& x,
                                       uint32_t& ptr, uint32_t pend) {
  const uint32_t e = tab[x & 0xFFu];
  x = (e & 0xFFu) * (x >> 8) + ((e >> 8) & 0xFFu);
  const uint32_t b = cont[ptr < pend ? ptr : pend];
  if (x < kStateLow) {
    x = (x << 8) | b;
    ++ptr;
  }
  return (e >> 16) & 0xFFu;
}

// ----------------------------------------------------------------- symbols
__global__ __launch_bounds__(256) void decode_symbols_kernel(DecSymArgs a) {
  __shared__ uint32_t tab[256];
  tab[threadIdx.x] = a.dec[threadIdx.x];
  __syncthreads();
  const int64_t s = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (s >= a.n_streams) return;
  const uint8_t* p = a.cont + s * a.C;
  uint32_t x = uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24);
  int ptr = 4;
  uint8_t* out = a.sym + s * a.n;
  for (int i = 0; i < a.n; ++i) {
    const uint32_t e = tab[x & 0xFFu];
    out[i] = uint8_t(e >> 16);
    x = (e & 0xFFu) * (x >> 8) + ((e >> 8) & 0xFFu);
    // a well-formed stream needs at most one byte per symbol; the bound keeps
    // malformed input from looping
    for (int r = 0; r < 2 && x < kStateLow; ++r) {
      const uint32_t b = ptr < a.C ? p[ptr] : 0u;
      x = (x << 8) | b;
      ++ptr;
    }
  }
  if (a.end_ok) a.end_ok[s] = (x == kStateLow) ? 1u : 0u;
}

// ----------------------------------------------------------------- prologue
// One wave per (sequence, query head); lane holds d/64 consecutive channels.
template <int NPL>
__global__ __launch_bounds__(64) void prologue_kernel(PrologueArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int g = h / a.G;
  float v[NPL];
  const uint16_t* qp = a.q + (s * a.Hq + h) * a.d + lane * NPL;
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = bf16_bits_to_f32(qp[i]);
  fwht_lanes<NPL>(v, a.d, lane, a.hscale);
  float* qr = a.qrot + (s * a.Hq + h) * a.d + lane * NPL;
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    qr[i] = v[i];
    part += v[i];
  }
  part = wave_sum_f32(part);
  if (lane == 0) a.qsum[s * a.Hq + h] = part;
  for (int64_t w = 0; w < a.nW; ++w) {
    const float sc = h2f(a.mean_scale[s * a.nW + w]);
    const int8_t* mq = a.mean_q + (s * a.nW + w) * a.n + int64_t(g) * a.d + lane * NPL;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc += v[i] * __fmul_rn(float(mq[i]), sc);
    acc = wave_sum_f32(acc);
    if (lane == 0) a.qmu[(s * a.Hq + h) * a.nW + w] = acc;
  }
}

// ----------------------------------------------------------------- attention
// One wave per (split, sequence); 64-token tiles, one token per lane.
template <int G, int HKV, int D>
__global__ __launch_bounds__(64) void attention_kernel(AttnArgs a) {
  constexpr int HQ = G * HKV;
  constexpr int CPL = D / 64;
  __shared__ uint32_t tabK[256], tabV[256];
  __shared__ uint8_t symV[64][D + 4];
  __shared__ float wts[G][64];
  __shared__ float runM[HQ], runL[HQ], runZ[HQ];
  extern __shared__ __align__(16) uint8_t cont[];
  const int lane = threadIdx.x;
  const int64_t s = blockIdx.y;
  const int split = blockIdx.x;
  for (int i = lane; i < 256; i += 64) {
    tabK[i] = a.deck[i];
    tabV[i] = a.decv[i];
  }
  for (int h = lane; h < HQ; h += 64) {
    runM[h] = -__builtin_inff();
    runL[h] = 0.f;
    runZ[h] = 0.f;
  }
  __syncthreads();
  float o[HQ][CPL];
#pragma unroll
  for (int h = 0; h < HQ; ++h)
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[h][c] = 0.f;
  const int64_t tb = int64_t(split) * a.tokens_per_split;
  const int64_t te = tb + a.tokens_per_split < a.T ? tb + a.tokens_per_split : a.T;
  const float* qrot = a.qrot + s * HQ * D;
  const float* qsum = a.qsum + s * HQ;
  const float* qmu = a.qmu + s * HQ * a.nW;
  for (int64_t t0 = tb; t0 < te; t0 += 64) {
    const int64_t t = t0 + lane;
    const int64_t row = s * a.T + t;
    // ---- keys: stage the tile's containers, decode, logits
    {
      const uint4* src = reinterpret_cast<const uint4*>(a.k_cont + (s * a.T + t0) * a.CK);
      uint4* dst = reinterpret_cast<uint4*>(cont);
      for (int i = lane; i < 4 * a.CK; i += 64) dst[i] = src[i];
    }
    __syncthreads();
    const uint32_t base = uint32_t(lane) * a.CK;
    uint32_t x = uint32_t(cont[base]) | (uint32_t(cont[base + 1]) << 8) |
                 (uint32_t(cont[base + 2]) << 16) | (uint32_t(cont[base + 3]) << 24);
    uint32_t ptr = base + 4;
    uint32_t pend = base + a.CK - 1;
    const float sk = h2f(a.k_so[2 * row]), ok = h2f(a.k_so[2 * row + 1]);
    const int64_t w = t / a.W;
    float logit[HQ];
#pragma unroll
    for (int g = 0; g < HKV; ++g) {
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      for (int j = 0; j < D; ++j) {
        const float mf = float(decode_step(tabK, cont, x, ptr, pend));
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(qrot[(g * G + h) * D + j], mf, acc[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int hh = g * G + h;
        logit[hh] = a.tau * (sk * acc[h] + ok * qsum[hh] + qmu[hh * a.nW + w]);
      }
    }
    __syncthreads();
    // ---- online softmax over the tile
    const float sv = h2f(a.v_so[2 * row]), ov = h2f(a.v_so[2 * row + 1]);
    float pw[HQ];
#pragma unroll
    for (int h = 0; h < HQ; ++h) {
      const float mt = wave_max(logit[h]);
      const float Mo = runM[h];
      const float Mn = fmaxf(Mo, mt);
      const float al = __expf(Mo - Mn);
      const float p = __expf(logit[h] - Mn);
      const float ls = wave_sum_f32(p);
      const float zs = wave_sum_f32(p * ov);
      pw[h] = p * sv;
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[h][c] *= al;
      const float Lo = runL[h], Zo = runZ[h];
      __syncthreads();
      runM[h] = Mn;
      runL[h] = Lo * al + ls;
      runZ[h] = Zo * al + zs;
    }
    // ---- values: stage, decode one KV head at a time, PV via an LDS transpose
    {
      const uint4* src = reinterpret_cast<const uint4*>(a.v_cont + (s * a.T + t0) * a.CV);
      uint4* dst = reinterpret_cast<uint4*>(cont);
      for (int i = lane; i < 4 * a.CV; i += 64) dst[i] = src[i];
    }
    __syncthreads();
    const uint32_t vbase = uint32_t(lane) * a.CV;
    x = uint32_t(cont[vbase]) | (uint32_t(cont[vbase + 1]) << 8) |
        (uint32_t(cont[vbase + 2]) << 16) | (uint32_t(cont[vbase + 3]) << 24);
    ptr = vbase + 4;
    pend = vbase + a.CV - 1;
#pragma unroll
    for (int g = 0; g < HKV; ++g) {
      for (int j = 0; j < D; ++j) symV[lane][j] = uint8_t(decode_step(tabV, cont, x, ptr, pend));
#pragma unroll
      for (int h = 0; h < G; ++h) wts[h][lane] = pw[g * G + h];
      __syncthreads();
      for (int tt = 0; tt < 64; ++tt) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const float mv = float(symV[tt][lane + 64 * c]);
#pragma unroll
          for (int h = 0; h < G; ++h) o[g * G + h][c] = fmaf(wts[h][tt], mv, o[g * G + h][c]);
        }
      }
      __syncthreads();
    }
  }
  float* P = a.part + (s * a.nsplit + split) * int64_t(HQ) * (D + 4);
#pragma unroll
  for (int h = 0; h < HQ; ++h) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) P[h * (D + 4) + lane + 64 * c] = o[h][c];
    if (lane == 0) {
      P[h * (D + 4) + D] = runM[h];
      P[h * (D + 4) + D + 1] = runL[h];
      P[h * (D + 4) + D + 2] = runZ[h];
    }
  }
}

// ----------------------------------------------------------------- combine
template <int NPL>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int64_t s = blockIdx.y;
  const int stride = a.d + 4;
  const float* P = a.part + (s * a.nsplit) * int64_t(a.Hq) * stride + int64_t(h) * stride;
  const int64_t sp = int64_t(a.Hq) * stride;
  float Mx = -__builtin_inff();
  for (int k = 0; k < a.nsplit; ++k) Mx = fmaxf(Mx, P[k * sp + a.d]);
  float L = 0.f, Z = 0.f;
  float acc[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[i] = 0.f;
  for (int k = 0; k < a.nsplit; ++k) {
    const float sc = __expf(P[k * sp + a.d] - Mx);
    L += sc * P[k * sp + a.d + 1];
    Z += sc * P[k * sp + a.d + 2];
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc[i] += sc * P[k * sp + lane * NPL + i];
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

}  // namespace

hipError_t launch_decode_symbols(const DecSymArgs& a, hipStream_t stream) {
  const unsigned blocks = unsigned((a.n_streams + 255) / 256);
  hipLaunchKernelGGL(decode_symbols_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, int64_t S, hipStream_t stream) {
  const dim3 grid(a.Hq, unsigned(S));
  switch (a.d) {
    case 64: hipLaunchKernelGGL(prologue_kernel<1>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(prologue_kernel<2>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(prologue_kernel<4>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G, int HKV, int D>
static hipError_t launch_attn_t(const AttnArgs& a, int64_t S, hipStream_t stream) {
  const size_t lds = size_t(64) * size_t(a.CK > a.CV ? a.CK : a.CV);
  hipLaunchKernelGGL((attention_kernel<G, HKV, D>), dim3(a.nsplit, unsigned(S)), dim3(64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int64_t S, int Hq, int G, int d, hipStream_t stream) {
  const int hkv = Hq / G;
  if (d == 128 && G == 1 && hkv == 1) return launch_attn_t<1, 1, 128>(a, S, stream);
  if (d == 128 && G == 4 && hkv == 8) return launch_attn_t<4, 8, 128>(a, S, stream);
  if (d == 128 && G == 8 && hkv == 8) return launch_attn_t<8, 8, 128>(a, S, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineArgs& a, int64_t S, hipStream_t stream) {
  const dim3 grid(a.Hq, unsigned(S));
  switch (a.d) {
    case 64: hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<2>, grid, dim3(64), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(combine_kernel<4>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool attention_supported(int Hq, int G, int d) {
  const int hkv = Hq / G;
  return d == 128 && ((G == 1 && hkv == 1) || (G == 4 && hkv == 8) || (G == 8 && hkv == 8));
}

}  // namespace kvq
