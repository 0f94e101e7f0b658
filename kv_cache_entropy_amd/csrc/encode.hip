// Write side: windowed key channel mean and the per-stream encoder.
//
// [D-Quant] Figure 1 / §4.2: every head of a token's key (value) vector is
// Hadamard-rotated; keys subtract a windowed channel-wise mean; each stream
// (all KV heads of one token) gets one affine grid (Eq. 4).  §4.3 / Appendix
// A, Algorithm 1: symbols are assigned by a Lagrangian drift under the
// container budget (Eqs. 5-6), (s, o) are refitted by least squares, rounded
// to FP16 and the drift repeated on that grid; the symbols are rANS-coded
// (Eq. 2) backwards into a C-byte container (Eq. 3).  §4.5 "Encoding": one
// wavefront per stream keeps the values on chip throughout; distortions are
// recomputed on the fly for the M levels at every bisection step and the code
// length is reduced across the wavefront.
//
// Every floating-point step is one IEEE operation rounded to nearest-even
// (explicit __f*_rn / __d*_rn intrinsics, no contraction) and every float
// reduction has a fixed order, so containers are bit-identical to a plain CPU
// evaluation of the same steps.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "device_common.h"

namespace kvq {
namespace {

// ---------------------------------------------------------------------------
// Windowed key channel mean: one workgroup per (sequence, window); thread t
// owns channels 4t..4t+3.  mu = (fp32 running sum over the window's tokens in
// order, from +0) * (1/W); INT8 with one fp16 scale: sc = fp16(max|mu| / 127),
// mu_q = clamp(rne(mu / sc), -127, 127).
__global__ __launch_bounds__(1024) void key_mean_kernel(KeyMeanArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t nW = a.T / a.W;
  const int64_t seq = blockIdx.x / nW;
  const int64_t win = blockIdx.x % nW;
  const int j0 = tid * 4;
  const bool active = j0 < a.n;   // the block is rounded up to whole waves
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int tt = 0; tt < a.W; ++tt) {
    const int64_t row = (seq * a.T + win * a.W + tt) * a.n;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) load_values<4>(a.k, a.in_bf16, row + j0, v);
    fwht_lanes<4>(v, a.d, lane, a.hscale);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __fadd_rn(acc[i], v[i]);
  }
  const float invW = 1.0f / float(a.W);   // exact: W is a power of two
  float mu[4];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mu[i] = __fmul_rn(acc[i], invW);
    amax = fmaxf(amax, fabsf(mu[i]));
  }
  __shared__ float red[16];
  amax = wave_max(amax);
  if (lane == 0) red[tid >> 6] = amax;
  __syncthreads();
  const int nwaves = (blockDim.x + 63) >> 6;
  amax = red[0];
  for (int w = 1; w < nwaves; ++w) amax = fmaxf(amax, red[w]);
  const __half sc16 = __float2half_rn(__fdiv_rn(amax, 127.0f));
  const float sc = __half2float(sc16);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int qv = 0;
    if (sc != 0.f) {
      float r = rintf(__fdiv_rn(mu[i], sc));
      r = fminf(fmaxf(r, -127.f), 127.f);
      qv = int(r);
    }
    packed |= (uint32_t(qv) & 0xFFu) << (8 * i);
  }
  const int64_t orow = seq * (a.T_cap / a.W) + a.t_off / a.W + win;
  if (active) *reinterpret_cast<uint32_t*>(a.mean_q + orow * a.n + j0) = packed;
  if (tid == 0) a.mean_scale[orow] = __half_as_ushort(sc16);
}

// Wave-wide integer sum in VALU only (DPP within rows of 16 lanes, then the
// gfx950 row and half-wave swaps): no LDS round trips on the drift's
// per-step critical path.  Integer addition, so the order does not matter.
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
__device__ inline uint32_t wave_sum_u32_dpp(uint32_t v) {
  v += dpp_u32<0xB1>(v);      // quad_perm [1,0,3,2]
  v += dpp_u32<0x4E>(v);      // quad_perm [2,3,0,1]
  v += dpp_u32<0x124>(v);     // row_ror:4
  v += dpp_u32<0x128>(v);     // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t r = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(r, r, false, false);
  return __builtin_amdgcn_readfirstlane(b[0] + b[1]);
}

// Wave-wide max / min of finite floats, in VALU only, on order-preserving
// integer keys (sign-folded bit patterns): the result is the same value
// whatever the reduction order.  Lanes a DPP pattern leaves without a source
// would keep the identity (every pattern used is a full permutation).
__device__ inline int float_key(int b) { return b ^ ((b >> 31) & 0x7FFFFFFF); }
template <int CTRL, bool MAX>
__device__ inline int dpp_ext(int v) {
  const int o = __builtin_amdgcn_update_dpp(MAX ? int(0x80000000) : int(0x7FFFFFFF), v, CTRL, 0xF, 0xF, false);
  return MAX ? (v > o ? v : o) : (v < o ? v : o);
}
template <bool MAX>
__device__ inline float wave_ext_dpp(float x) {
  int k = float_key(__float_as_int(x));
  k = dpp_ext<0xB1, MAX>(k);
  k = dpp_ext<0x4E, MAX>(k);
  k = dpp_ext<0x124, MAX>(k);
  k = dpp_ext<0x128, MAX>(k);
  const auto a = __builtin_amdgcn_permlane16_swap(uint32_t(k), uint32_t(k), false, false);
  const int r = MAX ? (int(a[0]) > int(a[1]) ? int(a[0]) : int(a[1])) : (int(a[0]) < int(a[1]) ? int(a[0]) : int(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(uint32_t(r), uint32_t(r), false, false);
  const int t = MAX ? (int(b[0]) > int(b[1]) ? int(b[0]) : int(b[1])) : (int(b[0]) < int(b[1]) ? int(b[0]) : int(b[1]));
  return __int_as_float(float_key(__builtin_amdgcn_readfirstlane(t)));
}

// ---------------------------------------------------------------------------
// Drift (Algorithm 1) for the stream held NPL values per lane by one wave.
// Returns true if the encoder fell back to the cheapest symbol everywhere.
// If near != nullptr, the nearest-level (lambda -> 0) assignment is returned.
//
// With at most MC levels the distortions D_im = (x_i - rec_m)^2 are computed
// once and kept in registers: they do not depend on lambda, so each bisection
// step only adds lambda r_m and takes the argmin.  The values are the same
// roundings as recomputing them, so the result is identical.
template <int NPL, int MC>
__device__ bool drift(const float (&x)[NPL], float s, float o, const EncShared& sh,
                      int levels, uint8_t (&m)[NPL], uint8_t (*near)[NPL]) {
  // distortions, their range over all (i, level), and the nearest levels
  float dmax = 0.f, dmin = __builtin_inff();
  float Dc[MC][NPL];
  float bestD[NPL];
  uint32_t bl[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) { bestD[i] = __builtin_inff(); bl[i] = 0; }
#pragma unroll
  for (int l = 0; l < MC; ++l) {
    if (l < levels) {
      const float rec = __fadd_rn(o, __fmul_rn(s, sh.level[l]));
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float dl = __fsub_rn(x[i], rec);
        const float D = __fmul_rn(dl, dl);
        Dc[l][i] = D;
        dmax = fmaxf(dmax, D);
        dmin = fminf(dmin, D);
        const bool lt = D < bestD[i];
        bestD[i] = lt ? D : bestD[i];
        bl[i] = lt ? uint32_t(l) : bl[i];
      }
    }
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) (*near)[i] = uint8_t(bl[i]);
  }
  dmax = wave_ext_dpp<true>(dmax);
  dmin = wave_ext_dpp<false>(dmin);
  const float y = __fmul_rn(__fsub_rn(dmax, dmin), 8.0f);
  const uint8_t cheap = uint8_t(sh.cheapest);
  if (!(y > 0.f)) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m[i] = cheap;
    return false;
  }
  int e;
  const float fr = frexpf(y, &e);
  const int hi0 = (fr == 0.5f) ? e - 1 : e;
  int lo = 512 * (hi0 - 40), hi = 512 * hi0;
  bool moved = false;
#pragma unroll
  for (int i = 0; i < NPL; ++i) m[i] = cheap;
  uint32_t cur[NPL];
  for (int step = 0; step <= 12; ++step) {
    int u;
    if (step < 12) {
      u = (lo + hi) >> 1;              // lo + hi is always even: exact
    } else {
      if (moved) break;
      u = hi;                          // never feasible inside: try 2^hi
    }
    const float lam = ldexpf(sh.lambda[u & 511], u >> 9);
    float best[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) { best[i] = __builtin_inff(); cur[i] = 0; }
#pragma unroll
    for (int l = 0; l < MC; ++l) {
      if (l < levels) {
        const float lr = __fmul_rn(lam, sh.rate_f[l]);
#pragma unroll
        for (int i = 0; i < NPL; ++i) {
          const float obj = __fadd_rn(Dc[l][i], lr);
          const bool lt = obj < best[i];
          best[i] = lt ? obj : best[i];
          cur[i] = lt ? uint32_t(l) : cur[i];
        }
      }
    }
    uint32_t R = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) R += sh.rate_fx[cur[i]];
    R = wave_sum_u32_dpp(R);
    const bool ok = uint64_t(R) <= sh.budget_fx;
    if (step < 12) {
      if (ok) {
        hi = u;
        moved = true;
#pragma unroll
        for (int i = 0; i < NPL; ++i) m[i] = uint8_t(cur[i]);
      } else {
        lo = u;
      }
    } else {
      if (!ok) return true;            // fallback: cheapest level everywhere
#pragma unroll
      for (int i = 0; i < NPL; ++i) m[i] = uint8_t(cur[i]);
    }
  }
  return false;
}

// drift for an alphabet of exactly MC levels: the same result, with the argmin
// of each value taken as the minimum of its MC objectives (three-operand
// minimums) and then the lowest level whose objective equals it - the level a
// scan with strict < keeps - in fewer instructions than the scan.
template <int NPL, int MC>
__device__ bool drift_exact(const float (&x)[NPL], float s, float o, const EncShared& sh,
                      int levels, uint8_t (&m)[NPL], uint8_t (*near)[NPL]) {
  // distortions, their range over all (i, level), and the nearest levels
  float dmax = 0.f, dmin = __builtin_inff();
  float Dc[MC][NPL];
  float bestD[NPL];
  uint32_t bl[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) { bestD[i] = __builtin_inff(); bl[i] = 0; }
  (void)levels;                         // == MC
#pragma unroll
  for (int l = 0; l < MC; ++l) {
    const float rec = __fadd_rn(o, __fmul_rn(s, sh.level[l]));
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float dl = __fsub_rn(x[i], rec);
      const float D = __fmul_rn(dl, dl);
      Dc[l][i] = D;
      dmax = fmaxf(dmax, D);
      dmin = fminf(dmin, D);
      const bool lt = D < bestD[i];
      bestD[i] = lt ? D : bestD[i];
      bl[i] = lt ? uint32_t(l) : bl[i];
    }
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) (*near)[i] = uint8_t(bl[i]);
  }
  dmax = wave_ext_dpp<true>(dmax);
  dmin = wave_ext_dpp<false>(dmin);
  const float y = __fmul_rn(__fsub_rn(dmax, dmin), 8.0f);
  const uint8_t cheap = uint8_t(sh.cheapest);
  if (!(y > 0.f)) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m[i] = cheap;
    return false;
  }
  int e;
  const float fr = frexpf(y, &e);
  const int hi0 = (fr == 0.5f) ? e - 1 : e;
  int lo = 512 * (hi0 - 40), hi = 512 * hi0;
  bool moved = false;
#pragma unroll
  for (int i = 0; i < NPL; ++i) m[i] = cheap;
  uint32_t cur[NPL];
  for (int step = 0; step <= 12; ++step) {
    int u;
    if (step < 12) {
      u = (lo + hi) >> 1;              // lo + hi is always even: exact
    } else {
      if (moved) break;
      u = hi;                          // never feasible inside: try 2^hi
    }
    const float lam = ldexpf(sh.lambda[u & 511], u >> 9);
    float lr[MC];
#pragma unroll
    for (int l = 0; l < MC; ++l) lr[l] = __fmul_rn(lam, sh.rate_f[l]);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      float obj[MC];
#pragma unroll
      for (int l = 0; l < MC; ++l) obj[l] = __fadd_rn(Dc[l][i], lr[l]);
      // sums, never signalling NaNs: the minimums need no canonicalisation;
      // a NaN objective never equals the minimum, as it never beats one
      float best = obj[0];
#pragma unroll
      for (int l = 1; l < MC; ++l) best = __builtin_fminf(best, obj[l]);
      uint32_t c = 0;
#pragma unroll
      for (int l = MC - 1; l >= 0; --l) c = obj[l] == best ? uint32_t(l) : c;
      cur[i] = c;
    }
    uint32_t R = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) R += sh.rate_fx[cur[i]];
    R = wave_sum_u32_dpp(R);
    const bool ok = uint64_t(R) <= sh.budget_fx;
    if (step < 12) {
      if (ok) {
        hi = u;
        moved = true;
#pragma unroll
        for (int i = 0; i < NPL; ++i) m[i] = uint8_t(cur[i]);
      } else {
        lo = u;
      }
    } else {
      if (!ok) return true;            // fallback: cheapest level everywhere
#pragma unroll
      for (int i = 0; i < NPL; ++i) m[i] = uint8_t(cur[i]);
    }
  }
  return false;
}

// The same without the cache, for alphabets above MC levels.
template <int NPL>
__device__ bool drift_large(const float (&x)[NPL], float s, float o, const EncShared& sh,
                            int levels, uint8_t (&m)[NPL], uint8_t (*near)[NPL]) {
  // range of the distortion over all (i, level) and the nearest levels
  float dmax = 0.f, dmin = __builtin_inff();
  float bestD[NPL];
  uint8_t bl[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) { bestD[i] = __builtin_inff(); bl[i] = 0; }
  for (int l = 0; l < levels; ++l) {
    const float rec = __fadd_rn(o, __fmul_rn(s, sh.level[l]));
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float dl = __fsub_rn(x[i], rec);
      const float D = __fmul_rn(dl, dl);
      dmax = fmaxf(dmax, D);
      dmin = fminf(dmin, D);
      if (D < bestD[i]) { bestD[i] = D; bl[i] = uint8_t(l); }
    }
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) (*near)[i] = bl[i];
  }
  dmax = wave_ext_dpp<true>(dmax);
  dmin = wave_ext_dpp<false>(dmin);
  const float y = __fmul_rn(__fsub_rn(dmax, dmin), 8.0f);
  const uint8_t cheap = uint8_t(sh.cheapest);
  if (!(y > 0.f)) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) m[i] = cheap;
    return false;
  }
  int e;
  const float fr = frexpf(y, &e);
  const int hi0 = (fr == 0.5f) ? e - 1 : e;
  int lo = 512 * (hi0 - 40), hi = 512 * hi0;
  bool moved = false;
#pragma unroll
  for (int i = 0; i < NPL; ++i) m[i] = cheap;
  uint8_t cur[NPL];
  for (int step = 0; step <= 12; ++step) {
    int u;
    if (step < 12) {
      u = (lo + hi) >> 1;              // lo + hi is always even: exact
    } else {
      if (moved) break;
      u = hi;                          // never feasible inside: try 2^hi
    }
    const float lam = ldexpf(sh.lambda[u & 511], u >> 9);
    float best[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) { best[i] = __builtin_inff(); cur[i] = 0; }
    for (int l = 0; l < levels; ++l) {
      const float rec = __fadd_rn(o, __fmul_rn(s, sh.level[l]));
      const float lr = __fmul_rn(lam, sh.rate_f[l]);
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const float dl = __fsub_rn(x[i], rec);
        const float obj = __fadd_rn(__fmul_rn(dl, dl), lr);
        if (obj < best[i]) { best[i] = obj; cur[i] = uint8_t(l); }
      }
    }
    uint32_t R = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) R += sh.rate_fx[cur[i]];
    R = wave_sum_u32_dpp(R);
    const bool ok = uint64_t(R) <= sh.budget_fx;
    if (step < 12) {
      if (ok) {
        hi = u;
        moved = true;
#pragma unroll
        for (int i = 0; i < NPL; ++i) m[i] = cur[i];
      } else {
        lo = u;
      }
    } else {
      if (!ok) return true;            // fallback: cheapest level everywhere
#pragma unroll
      for (int i = 0; i < NPL; ++i) m[i] = cur[i];
    }
  }
  return false;
}

// Nearest level of every value (lowest index on ties): the lambda -> 0
// assignment, used alone by the fixed-width comparator.
template <int NPL>
__device__ void nearest(const float (&x)[NPL], float s, float o, int levels, const float* lev,
                        uint8_t (&m)[NPL]) {
  float bestD[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) { bestD[i] = __builtin_inff(); m[i] = 0; }
  for (int l = 0; l < levels; ++l) {
    const float rec = __fadd_rn(o, __fmul_rn(s, lev[l]));
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const float dl = __fsub_rn(x[i], rec);
      const float D = __fmul_rn(dl, dl);
      if (D < bestD[i]) { bestD[i] = D; m[i] = uint8_t(l); }
    }
  }
}

// Fixed-width container layout ([D-Quant] Appendix B comparator): symbol
// i = 4c + r in byte r of dword c / (8/b), bits b (c mod 8/b) .. + b.  A lane's
// NPL consecutive symbols fill NPL b / 32 whole dwords when NPL is a multiple
// of 32 / b, which the host checks.
template <int NPL, int B>
__device__ void fw_pack_lane(const uint8_t (&m)[NPL], uint32_t* img_words, int lane) {
  constexpr int per = 8 / B;                   // groups of 4 per dword
  constexpr int words = NPL * B / 32;
  static_assert(NPL * B % 32 == 0, "a lane must fill whole dwords");
#pragma unroll
  for (int q = 0; q < words; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < per; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int li = (q * per + k) * 4 + r;    // lane-local symbol index
        w |= uint32_t(m[li]) << (8 * r + B * k);
      }
    img_words[lane * words + q] = w;
  }
}

// Least-squares refit on [1, v_m] in float64 with the fixed summation order
// (chunk per lane in increasing index from +0, then xor-butterfly 32..1) for
// every sum, the guard, and rounding to fp16 through fp32.  With affine levels
// the level sums and den are exact integers.
template <int NPL>
__device__ void refit(const float (&x)[NPL], const uint8_t (&m)[NPL], float s, float o, int n,
                      const float* lev, __half& s16, __half& o16) {
  double px = 0.0, pmx = 0.0, p1 = 0.0, p2 = 0.0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const double xd = double(x[i]);
    const double vd = double(lev[m[i]]);
    px = __dadd_rn(px, xd);
    pmx = __dadd_rn(pmx, __dmul_rn(vd, xd));
    p1 = __dadd_rn(p1, vd);
    p2 = __dadd_rn(p2, __dmul_rn(vd, vd));
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    px = __dadd_rn(px, __shfl_xor(px, k, 64));
    pmx = __dadd_rn(pmx, __shfl_xor(pmx, k, 64));
    p1 = __dadd_rn(p1, __shfl_xor(p1, k, 64));
    p2 = __dadd_rn(p2, __shfl_xor(p2, k, 64));
  }
  const double nd = double(n), S1d = p1;
  const double den = __dsub_rn(__dmul_rn(nd, p2), __dmul_rn(S1d, S1d));
  double sn, on;
  if (den == 0.0) {
    sn = double(s);
    on = __ddiv_rn(__dsub_rn(px, __dmul_rn(sn, S1d)), nd);
  } else {
    sn = __ddiv_rn(__dsub_rn(__dmul_rn(nd, pmx), __dmul_rn(S1d, px)), den);
    on = __ddiv_rn(__dsub_rn(px, __dmul_rn(sn, S1d)), nd);
  }
  if (!(sn >= 0.0) || !isfinite(sn) || !isfinite(on)) {
    sn = double(s);
    on = double(o);
  }
  s16 = __float2half_rn(float(sn));
  o16 = __float2half_rn(float(on));
}

// rANS encoder of one stream (one lane): symbols sym[0..n) packed two per
// byte (symbol i in nibble i mod 2 of byte i / 2), from the last to the first;
// pushed bytes are written downwards from img[C-1], then moved to follow the
// 4-byte state.  Returns false if the stream would overrun.  The symbols are
// read eight at a time and each symbol's coder entry is one 16-byte LDS read,
// so only the state update is on the dependent chain.
__device__ bool rans_encode_lane(const uint8_t* sym, int n, uint8_t* img, int C, const EncShared& sh) {
  uint32_t x = kStateLow;
  int k = 0;
  bool ok = true;
  const uint32_t* sym8 = reinterpret_cast<const uint32_t*>(sym);    // n is a multiple of 8
  for (int i8 = n / 8 - 1; i8 >= 0; --i8) {
    const uint32_t s8 = sym8[i8];
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      const uint4 e = sh.coder[(s8 >> (4 * j)) & 0xFu];
      const uint32_t f = e.x;
      // Branch-free renormalisation: the low byte is always stored at the
      // next push position and only counted when it is pushed (an uncounted
      // byte is overwritten by the next push, or lies outside the payload
      // that the tail below keeps).  At most one byte per symbol: afterwards
      // x < f 2^23.
      const bool rn = x >= (f << 23);
      img[C - 1 - k] = uint8_t(x & 0xFF);
      ok = ok && !(rn && k >= C - 4);
      k += (rn && k < C - 4) ? 1 : 0;
      x = rn ? (x >> 8) : x;
      // q = x / f (exact; see the planner), q < 2^23 and f < 2^8, so the
      // product is a 24-bit multiply
      const uint32_t q = e.z ? (__umulhi(x, e.z) >> e.w) : (x >> e.w);
      x = (q << 8) + (x - __umul24(q, f)) + e.y;
    }
  }
  img[0] = uint8_t(x);
  img[1] = uint8_t(x >> 8);
  img[2] = uint8_t(x >> 16);
  img[3] = uint8_t(x >> 24);
  for (int j = 0; j < k; ++j) img[4 + j] = img[C - k + j];
  for (int j = 4 + k; j < C; ++j) img[j] = 0;
  return ok;
}

// One workgroup = 4 waves = SPW streams of one side.  Each wave runs
// Algorithm 1 on SPW/4 streams in turn (values stay in registers); then SPW
// lanes rANS-code the streams from LDS and the workgroup copies the SPW
// contiguous containers out with dword stores.
// Alphabets up to this size keep the drift distortions in registers (for
// streams of up to 16 values per lane: 128 registers).
constexpr int kDriftCache = 8;

// ML > 0: the alphabet has exactly ML levels (the cached drift in its exact
// form); 0: any alphabet.
template <int NPL, int FWB, int ML = 0>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
  constexpr bool FW = FWB != 0;
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ EncShared sh;
  __shared__ uint32_t so_sh[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int SPW = a.spw;
  const int n = a.n, C = a.tabs.container_bytes, M = a.tabs.levels;
  const int CS = a.cs;                         // a container's bytes in the image and the cache
  uint8_t* sym = dyn;                          // [SPW][n / 2]: two 4-bit symbols per byte
  uint8_t* img = dyn + size_t(SPW) * (n / 2);  // [SPW][CS]
  for (int i = tid; i < 512; i += 256) sh.lambda[i] = a.tabs.lambda[i];
  if (tid < kMaxLevels) {
    sh.level[tid] = a.tabs.level[tid];
    sh.rate_fx[tid] = a.tabs.rate_fx[tid];
    sh.rate_f[tid] = float(a.tabs.rate_fx[tid]) * (1.0f / 65536.0f);
    sh.coder[tid] = uint4{a.tabs.freq[tid], a.tabs.cum[tid], a.tabs.rcp[tid], a.tabs.rshift[tid]};
  }
  if (tid == 0) {
    sh.cheapest = a.tabs.cheapest;
    sh.budget_fx = a.tabs.budget_fx;
  }
  __syncthreads();
  const int64_t stream0 = int64_t(blockIdx.x) * SPW;
  const int per_wave = SPW / 4;
  uint32_t fb1 = 0, fb2 = 0, changed = 0;
  for (int js = 0; js < per_wave; ++js) {
    const int sl = wave * per_wave + js;
    const int64_t st = stream0 + sl;
    float x[NPL];
    load_values<NPL>(a.x, a.in_bf16, st * n + int64_t(lane) * NPL, x);
    fwht_lanes<NPL>(x, a.d, lane, a.hscale);
    if (a.is_key) {
      const int64_t seq = st / a.T, t = st % a.T;
      const int64_t row = seq * (a.T_cap / a.W) + (a.t_off + t) / a.W;
      const float sc = __half2float(__ushort_as_half(a.mean_scale[row]));
      const int8_t* mq = a.mean_q + row * n + int64_t(lane) * NPL;
#pragma unroll
      for (int i = 0; i < NPL; ++i) x[i] = __fsub_rn(x[i], __fmul_rn(float(mq[i]), sc));
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
    mn = __fadd_rn(wave_ext_dpp<false>(mn), 0.0f);     // a negative zero becomes +0
    mx = __fadd_rn(wave_ext_dpp<true>(mx), 0.0f);
    const float s = __fdiv_rn(__fsub_rn(mx, mn), float(M - 1));
    const float o = mn;
    uint8_t m[NPL];
    __half s16, o16;
    if constexpr (FW) {
      nearest<NPL>(x, s, o, M, sh.level, m);
      refit<NPL>(x, m, s, o, n, sh.level, s16, o16);
      nearest<NPL>(x, __half2float(s16), __half2float(o16), M, sh.level, m);
      if constexpr (FW) fw_pack_lane<NPL, FWB>(m, reinterpret_cast<uint32_t*>(img + size_t(sl) * CS), lane);
    } else {
      uint8_t near[NPL];
      if constexpr (ML > 0) {
        fb1 += drift_exact<NPL, ML>(x, s, o, sh, M, m, nullptr) ? 1u : 0u;
        refit<NPL>(x, m, s, o, n, sh.level, s16, o16);
        fb2 += drift_exact<NPL, ML>(x, __half2float(s16), __half2float(o16), sh, M, m, &near) ? 1u : 0u;
      } else if (NPL * kDriftCache <= 128 && M <= kDriftCache) {
        constexpr int MC = NPL * kDriftCache <= 128 ? kDriftCache : 1;
        fb1 += drift<NPL, MC>(x, s, o, sh, M, m, nullptr) ? 1u : 0u;
        refit<NPL>(x, m, s, o, n, sh.level, s16, o16);
        fb2 += drift<NPL, MC>(x, __half2float(s16), __half2float(o16), sh, M, m, &near) ? 1u : 0u;
      } else {
        fb1 += drift_large<NPL>(x, s, o, sh, M, m, nullptr) ? 1u : 0u;
        refit<NPL>(x, m, s, o, n, sh.level, s16, o16);
        fb2 += drift_large<NPL>(x, __half2float(s16), __half2float(o16), sh, M, m, &near) ? 1u : 0u;
      }
      uint32_t ch = 0;
#pragma unroll
      for (int i = 0; i < NPL; ++i) ch += (m[i] != near[i]) ? 1u : 0u;
      changed += wave_sum_u32(ch);
      // symbols i = lane NPL + idx, two per byte (levels <= 16)
      if constexpr (NPL >= 2) {
        uint8_t* dst = sym + size_t(sl) * (n / 2) + size_t(lane) * (NPL / 2);
#pragma unroll
        for (int b = 0; b < NPL / 2; ++b) dst[b] = uint8_t(m[2 * b] | (m[2 * b + 1] << 4));
      } else {
        const uint32_t odd = __shfl_xor(uint32_t(m[0]), 1, 64);
        if (!(lane & 1)) sym[size_t(sl) * (n / 2) + size_t(lane / 2)] = uint8_t(m[0] | (odd << 4));
      }
    }
    if (lane == 0) so_sh[sl] = uint32_t(__half_as_ushort(s16)) | (uint32_t(__half_as_ushort(o16)) << 16);
  }
  __syncthreads();
  // the SPW streams lie in one sequence (T is a multiple of SPW): their cache
  // rows are contiguous from ost0
  const int64_t seq0 = stream0 / a.T;
  const int64_t ost0 = seq0 * a.T_cap + a.t_off + (stream0 - seq0 * a.T);
  uint32_t overrun = 0;
  if (tid < SPW) {
    if constexpr (!FW) {
      overrun = rans_encode_lane(sym + size_t(tid) * (n / 2), n, img + size_t(tid) * CS, C, sh) ? 0u : 1u;
      for (int j = C; j < CS; ++j) img[size_t(tid) * CS + j] = 0;
    }
    reinterpret_cast<uint32_t*>(a.so)[ost0 + tid] = so_sh[tid];
  }
  __syncthreads();
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(img);
  if (a.tiles) {
    // dword k of cache token t at (t / 64) 64 CS + k 256 + (t mod 64) 4 in its
    // sequence; consecutive threads take consecutive tokens of one dword k
    const int dps = CS / 4;
    const int64_t t0 = a.t_off + (stream0 - seq0 * a.T);
    uint8_t* const seqb = a.cont + seq0 * a.seq_bytes;
    for (int i = tid; i < SPW * dps; i += 256) {
      const int j = i % SPW, kd = i / SPW;
      const int64_t t = t0 + j;
      *reinterpret_cast<uint32_t*>(seqb + (t >> 6) * (64 * int64_t(CS)) + int64_t(kd) * 256 + (t & 63) * 4) =
          ssrc[j * dps + kd];
    }
  } else {
    // SPW * C is a multiple of 4 (SPW is a multiple of 4); ost0 * C is a
    // multiple of 4 because ost0 is a multiple of SPW
    const int nwords = SPW * C / 4;
    uint32_t* gdst = reinterpret_cast<uint32_t*>(a.cont + ost0 * C);
    for (int i = tid; i < nwords; i += 256) gdst[i] = ssrc[i];
  }
  if (a.stats) {
    if (lane == 0) {
      if (fb1) atomicAdd(a.stats + 0, (unsigned long long)fb1);
      if (fb2) atomicAdd(a.stats + 1, (unsigned long long)fb2);
      if (changed) atomicAdd(a.stats + 2, (unsigned long long)changed);
    }
    if (overrun) atomicAdd(a.stats + 3, 1ull);
  }
}

}  // namespace

hipError_t launch_key_mean(const KeyMeanArgs& a, int64_t n_windows, hipStream_t stream) {
  const int threads = ((a.n / 4 + 63) / 64) * 64;
  hipLaunchKernelGGL(key_mean_kernel, dim3(unsigned(n_windows)), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, int64_t n_streams, hipStream_t stream) {
  const size_t lds = size_t(a.spw) * (size_t(a.n) / 2 + size_t(a.cs));
  const dim3 grid(unsigned(n_streams / a.spw)), block(256);
  if (a.fw_bits) {
    const int key = (a.n / 64) * 16 + a.fw_bits;
    switch (key) {
      case 16 * 16 + 2: hipLaunchKernelGGL((encode_kernel<16, 2>), grid, block, lds, stream, a); break;
      case 16 * 16 + 4: hipLaunchKernelGGL((encode_kernel<16, 4>), grid, block, lds, stream, a); break;
      case 16 * 16 + 8: hipLaunchKernelGGL((encode_kernel<16, 8>), grid, block, lds, stream, a); break;
      case 32 * 16 + 1: hipLaunchKernelGGL((encode_kernel<32, 1>), grid, block, lds, stream, a); break;
      case 32 * 16 + 2: hipLaunchKernelGGL((encode_kernel<32, 2>), grid, block, lds, stream, a); break;
      case 32 * 16 + 4: hipLaunchKernelGGL((encode_kernel<32, 4>), grid, block, lds, stream, a); break;
      case 32 * 16 + 8: hipLaunchKernelGGL((encode_kernel<32, 8>), grid, block, lds, stream, a); break;
      case 64 * 16 + 1: hipLaunchKernelGGL((encode_kernel<64, 1>), grid, block, lds, stream, a); break;
      case 64 * 16 + 2: hipLaunchKernelGGL((encode_kernel<64, 2>), grid, block, lds, stream, a); break;
      case 64 * 16 + 4: hipLaunchKernelGGL((encode_kernel<64, 4>), grid, block, lds, stream, a); break;
      case 64 * 16 + 8: hipLaunchKernelGGL((encode_kernel<64, 8>), grid, block, lds, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // the exact-size drift for the 8- and 6-level alphabets (their objectives
  // fit the registers up to 16 values per lane)
  const int L = a.tabs.levels;
  if ((L == 8 || L == 6) && a.n / 64 <= 16) {
    const int key = (a.n / 64) * 16 + L;
    switch (key) {
      case 1 * 16 + 8: hipLaunchKernelGGL((encode_kernel<1, 0, 8>), grid, block, lds, stream, a); break;
      case 1 * 16 + 6: hipLaunchKernelGGL((encode_kernel<1, 0, 6>), grid, block, lds, stream, a); break;
      case 2 * 16 + 8: hipLaunchKernelGGL((encode_kernel<2, 0, 8>), grid, block, lds, stream, a); break;
      case 2 * 16 + 6: hipLaunchKernelGGL((encode_kernel<2, 0, 6>), grid, block, lds, stream, a); break;
      case 4 * 16 + 8: hipLaunchKernelGGL((encode_kernel<4, 0, 8>), grid, block, lds, stream, a); break;
      case 4 * 16 + 6: hipLaunchKernelGGL((encode_kernel<4, 0, 6>), grid, block, lds, stream, a); break;
      case 8 * 16 + 8: hipLaunchKernelGGL((encode_kernel<8, 0, 8>), grid, block, lds, stream, a); break;
      case 8 * 16 + 6: hipLaunchKernelGGL((encode_kernel<8, 0, 6>), grid, block, lds, stream, a); break;
      case 16 * 16 + 8: hipLaunchKernelGGL((encode_kernel<16, 0, 8>), grid, block, lds, stream, a); break;
      case 16 * 16 + 6: hipLaunchKernelGGL((encode_kernel<16, 0, 6>), grid, block, lds, stream, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.n / 64) {
    case 1: hipLaunchKernelGGL((encode_kernel<1, 0>), grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL((encode_kernel<2, 0>), grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((encode_kernel<4, 0>), grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((encode_kernel<8, 0>), grid, block, lds, stream, a); break;
    case 16: hipLaunchKernelGGL((encode_kernel<16, 0>), grid, block, lds, stream, a); break;
    case 32: hipLaunchKernelGGL((encode_kernel<32, 0>), grid, block, lds, stream, a); break;
    case 64: hipLaunchKernelGGL((encode_kernel<64, 0>), grid, block, lds, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvq
