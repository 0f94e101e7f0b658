// Host planner: builds the coding tables of a cache format.
//
// [D-Quant] §4.2: the entropy model is derived analytically from Gaussian
// order statistics (no calibration) and, by affine invariance of min-max
// normalised positions, one table serves every token and layer.  §4.4: the
// probabilities are sharpened, p'_m ~ p_m^alpha.  §3.1: integer frequencies
// f_m summing to 2^p with p = 8.  Appendix A, Algorithm 1: rates
// r_m = -log2(f_m / sum f) and the budget B = 8C - sigma (Eq. 3).
//
// The model is p_m(M, n): the expected share of level m when n iid N(0,1)
// values are min-max normalised (Eq. 4) and rounded to the nearest of M
// levels; the minimum always takes level 0, the maximum level M-1, and the
// n-2 others are N(0,1) truncated to (min, max).  It is integrated over the
// joint density of (min, max) by nested Gauss-Legendre quadrature.

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvq_internal.h"

namespace {

constexpr int kQuadNodes = 512;
constexpr double kQuadLo = -9.0, kQuadHi = 9.0;

// Gauss-Legendre nodes and weights on [-1, 1] by Newton iteration on P_N.
void gauss_legendre(int N, std::vector<double>& x, std::vector<double>& w) {
  x.assign(N, 0.0);
  w.assign(N, 0.0);
  const double pi = std::acos(-1.0);
  for (int i = 0; i < (N + 1) / 2; ++i) {
    double z = std::cos(pi * (i + 0.75) / (N + 0.5));
    double pp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p1 = 1.0, p2 = 0.0;
      for (int j = 1; j <= N; ++j) {
        double p3 = p2;
        p2 = p1;
        p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
      }
      pp = N * (z * p1 - p2) / (z * z - 1.0);
      double z1 = z;
      z = z1 - p1 / pp;
      if (std::fabs(z - z1) < 1e-16) break;
    }
    x[i] = -z;
    x[N - 1 - i] = z;
    w[i] = w[N - 1 - i] = 2.0 / ((1.0 - z * z) * pp * pp);
  }
}

double Phi(double v) { return 0.5 * std::erfc(-v / std::sqrt(2.0)); }
double phi(double v) { return std::exp(-0.5 * v * v) / std::sqrt(2.0 * std::acos(-1.0)); }

// IEEE binary16 of a float, round to nearest even (subnormals kept).
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const int exp = int((x >> 23) & 0xFFu);
  uint32_t mant = x & 0x7FFFFFu;
  if (exp == 0xFF) return uint16_t(sign | 0x7C00u | (mant ? 0x200u : 0u));
  const int e = exp - 127 + 15;
  if (e >= 31) return uint16_t(sign | 0x7C00u);
  if (e <= 0) {
    if (e < -10) return uint16_t(sign);
    mant |= 0x800000u;
    const int shift = 14 - e;
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return uint16_t(sign | h);
  }
  uint32_t h = (uint32_t(e) << 10) | (mant >> 13);
  const uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return uint16_t(sign | h);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16;
  const int exp = (h >> 10) & 0x1F;
  const uint32_t mant = h & 0x3FFu;
  float v;
  if (exp == 0) {
    v = std::ldexp(float(mant), -24);
  } else if (exp == 31) {
    v = mant ? std::nanf("") : INFINITY;
  } else {
    v = std::ldexp(float(mant | 0x400u), exp - 25);
  }
  uint32_t b;
  std::memcpy(&b, &v, 4);
  b |= sign;
  std::memcpy(&v, &b, 4);
  return v;
}

// p_m(M, n).  mids[m] (m = 0..M-2) bound the nearest-rounding cells in grid
// units ((v_m + v_{m+1}) / 2; m + 1/2 for affine levels).  Symmetrised when the
// levels are symmetric (then p_m = p_{M-1-m} holds exactly for the normal law).
std::vector<double> order_stat_probs(int M, int n, const std::vector<double>& mids, bool symmetric) {
  std::vector<double> p(M, 0.0);
  p[0] += 1.0;
  p[M - 1] += 1.0;
  if (n > 2) {
    std::vector<double> t, w;
    gauss_legendre(kQuadNodes, t, w);
    std::vector<double> acc(M, 0.0);
    for (int i = 0; i < kQuadNodes; ++i) {
      const double a = 0.5 * (kQuadHi - kQuadLo) * t[i] + 0.5 * (kQuadHi + kQuadLo);
      const double wa = 0.5 * (kQuadHi - kQuadLo) * w[i];
      const double half = 0.5 * (kQuadHi - a);
      const double Fa = Phi(a), pa = phi(a);
      for (int k = 0; k < kQuadNodes; ++k) {
        const double b = half * t[k] + 0.5 * (kQuadHi + a);
        const double wb = half * w[k];
        double G = 1.0 - Fa - Phi(-b);           // Phi(b) - Phi(a)
        if (G < 0.0) G = 0.0;
        const double dens = double(n) * double(n - 1) * pa * phi(b) * std::pow(G, double(n - 3));
        const double wt = wa * wb * dens;
        if (wt == 0.0) continue;
        const double width = b - a;
        for (int m = 0; m < M; ++m) {
          const double lo_u = m > 0 ? mids[m - 1] : -0.5;
          const double hi_u = m < M - 1 ? mids[m] : M - 0.5;
          double lo = a + width * (lo_u / (M - 1));
          double hi = a + width * (hi_u / (M - 1));
          lo = std::min(std::max(lo, a), b);
          hi = std::min(std::max(hi, a), b);
          acc[m] += wt * (Phi(hi) - Phi(lo));
        }
      }
    }
    for (int m = 0; m < M; ++m) p[m] += double(n - 2) * acc[m];
  }
  for (int m = 0; m < M; ++m) p[m] /= double(n);
  if (!symmetric) return p;
  std::vector<double> sym(M);
  for (int m = 0; m < M; ++m) sym[m] = (p[m] + p[M - 1 - m]) / 2.0;
  return sym;
}

// Integer frequencies: f = max(1, floor(256 q)); missing units to the largest
// remainders 256 q - f (ties: lower index); any excess taken from the largest
// f (ties: lower index).
bool integer_table(const std::vector<double>& q, uint32_t* f) {
  const int M = int(q.size());
  std::vector<double> raw(M);
  long sum = 0;
  for (int m = 0; m < M; ++m) {
    raw[m] = q[m] * 256.0;
    double fl = std::floor(raw[m]);
    f[m] = fl < 1.0 ? 1u : uint32_t(fl);
    sum += f[m];
  }
  long missing = 256 - sum;
  if (missing > 0) {
    std::vector<int> order(M);
    for (int m = 0; m < M; ++m) order[m] = m;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      return (raw[a] - f[a]) > (raw[b] - f[b]);
    });
    for (long u = 0; u < missing; ++u) f[order[u]] += 1;
  }
  while (sum > 256) {
    int best = 0;
    for (int m = 1; m < M; ++m)
      if (f[m] > f[best]) best = m;
    f[best] -= 1;
    --sum;
  }
  long tot = 0;
  for (int m = 0; m < M; ++m) {
    if (f[m] < 1) return false;
    tot += f[m];
  }
  return tot == 256;
}

// Level values as stored (fp16): v_m = m, or the caller's values rounded to
// fp16, which must rise strictly from 0 to levels - 1.
bool level_values(int levels, const float* values, kvq::SideTables& s) {
  s.affine = 1;
  for (int m = 0; m < levels; ++m) {
    const uint16_t h = f32_to_f16(values ? values[m] : float(m));
    s.fp16_bits[m] = h;
    s.fp16_hi[m] = h >> 8;
    s.fp16_lo[m] = h & 0xFFu;
    s.level[m] = f16_to_f32(h);
    if (!std::isfinite(s.level[m])) return false;
    if (s.level[m] != float(m)) s.affine = 0;
  }
  if (s.level[0] != 0.f || s.level[levels - 1] != float(levels - 1)) return false;
  for (int m = 1; m < levels; ++m)
    if (!(s.level[m] > s.level[m - 1])) return false;
  return true;
}

bool build_side(int levels, int n, double alpha, int container_bytes, const float* values,
                kvq::SideTables& s) {
  std::memset(&s, 0, sizeof(s));
  s.levels = levels;
  s.container_bytes = container_bytes;
  if (!level_values(levels, values, s)) return false;
  std::vector<double> mids(levels - 1);
  bool symmetric = true;
  for (int m = 0; m + 1 < levels; ++m) mids[m] = 0.5 * (double(s.level[m]) + double(s.level[m + 1]));
  for (int m = 0; m < levels; ++m)
    if (double(s.level[m]) + double(s.level[levels - 1 - m]) != double(levels - 1)) symmetric = false;
  std::vector<double> p = order_stat_probs(levels, n, mids, symmetric);
  std::vector<double> q(levels);
  double tot = 0.0;
  for (int m = 0; m < levels; ++m) {
    q[m] = std::pow(p[m], alpha);
    tot += q[m];
  }
  for (int m = 0; m < levels; ++m) q[m] /= tot;
  if (!integer_table(q, s.freq)) return false;
  uint32_t c = 0;
  for (int m = 0; m < levels; ++m) {
    s.cum[m] = c;
    c += s.freq[m];
    s.rate_fx[m] = uint32_t(std::nearbyint((8.0 - std::log2(double(s.freq[m]))) * 65536.0));
    // x / f for x < 2^31: with k = floor(log2 f) and rcp = ceil(2^(32+k) / f)
    // (< 2^32 unless f is a power of two), umulhi(x, rcp) >> k is exact
    // because the rounding excess x (rcp - 2^(32+k)/f) / 2^(32+k) < 2^-(k+1)
    // stays below 1/f.
    uint32_t f = s.freq[m];
    uint32_t k = 0;
    while ((2u << k) <= f) ++k;
    if ((f & (f - 1)) == 0) {
      s.rcp[m] = 0;
      s.rshift[m] = k;
    } else {
      unsigned __int128 num = (unsigned __int128)1 << (32 + k);
      s.rcp[m] = uint32_t((num + f - 1) / f);
      s.rshift[m] = k;
    }
  }
  for (int m = 0; m < levels; ++m)
    for (uint32_t z = s.cum[m]; z < s.cum[m] + s.freq[m]; ++z)
      s.dec[z] = s.freq[m] | ((z - s.cum[m]) << 8) | (uint32_t(m) << 16);
  uint32_t cheap = 0;
  for (int m = 1; m < levels; ++m)
    if (s.rate_fx[m] < s.rate_fx[cheap]) cheap = m;
  s.cheapest = cheap;
  s.budget_fx = uint64_t(8 * container_bytes - 32) << kvq::kRateFracBits;
  return true;
}

}  // namespace

extern "C" {

kvq_status kvq_plan_create(const kvq_params* params, kvq_plan** out_plan) {
  return kvq_plan_create_levels(params, nullptr, nullptr, out_plan);
}

kvq_status kvq_plan_create_levels(const kvq_params* params, const float* values_k,
                                  const float* values_v, kvq_plan** out_plan) {
  if (!params || !out_plan) return KVQ_EINVAL;
  *out_plan = nullptr;
  const kvq_params& p = *params;
  auto pow2 = [](int v) { return v > 0 && (v & (v - 1)) == 0; };
  if (p.n_kv_heads < 1 || !pow2(p.head_dim) || p.head_dim < 32 || p.head_dim > 256)
    return KVQ_EINVAL;
  const long n = long(p.n_kv_heads) * p.head_dim;
  if (n > 4096) return KVQ_EINVAL;
  if (p.levels_k < 2 || p.levels_k > kvq::kMaxLevels || p.levels_v < 2 || p.levels_v > kvq::kMaxLevels)
    return KVQ_EINVAL;
  if (p.container_bytes_k <= 4 || p.container_bytes_v <= 4 ||
      p.container_bytes_k > 65536 || p.container_bytes_v > 65536)
    return KVQ_EINVAL;
  if (!pow2(p.mean_window)) return KVQ_EINVAL;
  if (p.container_layout != KVQ_LAYOUT_ROWS && p.container_layout != KVQ_LAYOUT_TILES) return KVQ_EINVAL;
  if (!(p.sharpen_alpha >= 1.0) || !(p.sharpen_alpha <= 16.0)) return KVQ_EINVAL;
  kvq_plan* plan = new (std::nothrow) kvq_plan;
  if (!plan) return KVQ_ENOMEM;
  plan->params = p;
  plan->n = int(n);
  if (!build_side(p.levels_k, int(n), p.sharpen_alpha, p.container_bytes_k, values_k, plan->side[0]) ||
      !build_side(p.levels_v, int(n), p.sharpen_alpha, p.container_bytes_v, values_v, plan->side[1])) {
    delete plan;
    return KVQ_EINVAL;
  }
  for (int s = 0; s < 2; ++s) {
    const kvq::SideTables& t = plan->side[s];
    if (uint64_t(n) * t.rate_fx[t.cheapest] > t.budget_fx) {
      delete plan;
      return KVQ_EINFEASIBLE;
    }
  }
  for (int k = 0; k < kvq::kLambdaGrid; ++k)
    plan->lambda_grid[k] = float(exp2l((long double)k / 512.0L));
  plan->hadamard_scale = float(1.0 / std::sqrt(double(p.head_dim)));
  *out_plan = plan;
  return KVQ_OK;
}

void kvq_plan_destroy(kvq_plan* plan) { delete plan; }

kvq_status kvq_plan_tables(const kvq_plan* plan, int side, uint16_t* freq, uint16_t* cum,
                           int32_t* rate_fx) {
  if (!plan || (side != 0 && side != 1)) return KVQ_EINVAL;
  const kvq::SideTables& t = plan->side[side];
  for (int m = 0; m < kvq::kMaxLevels; ++m) {
    const bool live = m < t.levels;
    if (freq) freq[m] = live ? uint16_t(t.freq[m]) : 0;
    if (cum) cum[m] = live ? uint16_t(t.cum[m]) : 0;
    if (rate_fx) rate_fx[m] = live ? int32_t(t.rate_fx[m]) : 0;
  }
  return KVQ_OK;
}

kvq_status kvq_plan_levels(const kvq_plan* plan, int side, float* values) {
  if (!plan || (side != 0 && side != 1) || !values) return KVQ_EINVAL;
  const kvq::SideTables& t = plan->side[side];
  for (int m = 0; m < kvq::kMaxLevels; ++m) values[m] = m < t.levels ? t.level[m] : 0.f;
  return KVQ_OK;
}

kvq_status kvq_plan_lambda_grid(const kvq_plan* plan, float* grid512) {
  if (!plan || !grid512) return KVQ_EINVAL;
  std::memcpy(grid512, plan->lambda_grid, sizeof(plan->lambda_grid));
  return KVQ_OK;
}

kvq_status kvq_model_probs(int32_t levels, int32_t n, double alpha, double* probs) {
  if (!probs || levels < 2 || levels > kvq::kMaxLevels || n < 2 || n > 4096) return KVQ_EINVAL;
  if (!(alpha >= 1.0) || !(alpha <= 16.0)) return KVQ_EINVAL;
  std::vector<double> mids(levels - 1);
  for (int m = 0; m + 1 < levels; ++m) mids[m] = m + 0.5;
  const std::vector<double> p = order_stat_probs(levels, n, mids, true);
  double tot = 0.0;
  for (int m = 0; m < levels; ++m) tot += std::pow(p[m], alpha);
  for (int m = 0; m < levels; ++m) probs[m] = std::pow(p[m], alpha) / tot;
  return KVQ_OK;
}

double kvq_bits_per_elem(const kvq_params* p, int metadata) {
  if (!p) return -1.0;
  const double n = double(p->n_kv_heads) * p->head_dim;
  const bool tiles = p->container_layout == KVQ_LAYOUT_TILES;
  const auto stored = [tiles](int32_t c) { return double(tiles ? (c + 3) / 4 * 4 : c); };
  double bytes = stored(p->container_bytes_k) + stored(p->container_bytes_v);
  if (metadata) bytes += 2 * (2 + 2) + (n + 2) / double(p->mean_window);
  return 8.0 * bytes / (2.0 * n);
}

kvq_status kvq_containers_for_budget(double bpe, int32_t n_kv_heads, int32_t head_dim,
                                     int32_t mean_window, int32_t* c_k, int32_t* c_v) {
  if (!c_k || !c_v || n_kv_heads < 1 || head_dim < 1 || mean_window < 1 || !(bpe > 0)) return KVQ_EINVAL;
  const double n = double(n_kv_heads) * head_dim;
  const double total = std::floor(bpe * 2.0 * n / 8.0 - (8.0 + (n + 2.0) / mean_window));
  if (total < 10) return KVQ_EINFEASIBLE;
  const double ck = std::nearbyint(total * 331.0 / 562.0);   // ties to even
  *c_k = int32_t(ck);
  *c_v = int32_t(total - ck);
  return KVQ_OK;
}

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EINFEASIBLE: return "container too small for the cheapest symbols";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_EDEVICE: return "HIP device error";
    case KVQ_ENOMEM: return "out of host memory";
    case KVQ_EWORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

}  // extern "C"
