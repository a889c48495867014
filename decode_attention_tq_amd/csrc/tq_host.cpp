// Host-only parts of the C ABI: the Lloyd-Max codebooks (Gaussian and
// sphere-exact) and the seeded rotation / projection matrices. Plain C++17, no
// HIP calls.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq.h"
#include "tq_internal.h"

namespace {

// ---- Gaussian Lloyd-Max (ai-accelerate.xyz TurboQuant article, section
// "TurboQuantの仕組み", step 1: optimal scalar quantizer of a near-Gaussian
// coordinate). Lloyd's fixed point for N(0,1).

double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }
double pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI); }

// Phi^-1(p) by bisection on the monotone upper tail (no closed form needed).
double inv_cdf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (1.0 - upper_tail(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

// Round a double to the nearest float16 value (ties to even), returned as double.
double round_to_half(double x) {
  if (x == 0.0 || !std::isfinite(x)) return x;
  const double ax = std::fabs(x);
  int e;
  std::frexp(ax, &e);            // ax in [2^(e-1), 2^e)
  int ulp_exp = (e - 1) - 10;    // 10 fraction bits
  if (ulp_exp < -24) ulp_exp = -24;  // subnormal spacing
  const double ulp = std::ldexp(1.0, ulp_exp);
  const double r = std::nearbyint(ax / ulp) * ulp;   // default rounding: to nearest even
  return std::copysign(r, x);
}

void lloyd_max(int levels, double* c) {
  for (int i = 0; i < levels; ++i) c[i] = inv_cdf((i + 0.5) / levels);
  std::vector<double> t(levels + 1), nc(levels);
  for (int it = 0; it < 200000; ++it) {
    t[0] = -INFINITY;
    t[levels] = INFINITY;
    for (int i = 1; i < levels; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0;
    for (int i = 0; i < levels; ++i) {
      const double p = upper_tail(t[i]) - upper_tail(t[i + 1]);
      nc[i] = (pdf(t[i]) - pdf(t[i + 1])) / p;
      delta = std::fmax(delta, std::fabs(nc[i] - c[i]));
    }
    for (int i = 0; i < levels; ++i) c[i] = nc[i];
    if (delta < 1e-14) break;
  }
  std::vector<double> s(c, c + levels);
  for (int i = 0; i < levels; ++i) c[i] = 0.5 * (s[i] - s[levels - 1 - i]);
}

// ---- sphere-exact Lloyd-Max: the law of one coordinate u of a uniform unit
// vector in d dimensions, density (1 - u^2)^((d-3)/2) / B(1/2, (d-1)/2) on
// [-1, 1], so (1 + u)/2 ~ Beta((d-1)/2, (d-1)/2). Same iteration and standard
// units (z = u sqrt(d)) as the Gaussian one.

// Regularized incomplete beta I_x(a, b): the continued fraction of DLMF 8.17.22
// (coefficients d_{2m+1} = -(a+m)(a+b+m)x / ((a+2m)(a+2m+1)),
// d_{2m} = m(b-m)x / ((a+2m-1)(a+2m))) evaluated by the modified Lentz method,
// on the side of the symmetry I_x(a,b) = 1 - I_{1-x}(b,a) where it converges fast.
double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  if (x > (a + 1.0) / (a + b + 2.0)) return 1.0 - inc_beta(b, a, 1.0 - x);
  const double ln_pre = a * std::log(x) + b * std::log1p(-x) - std::log(a) -
                        (std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b));
  const double tiny = 1e-300;
  // f = 1 / (1 + d1 / (1 + d2 / (1 + ...)))
  double f = tiny, C = f, D = 0.0;
  for (int j = 1; j < 100000; ++j) {
    double aj;
    if (j == 1) {
      aj = 1.0;
    } else {
      const int n = j - 1;   // coefficient d_n
      const int m = n / 2;
      aj = (n % 2 == 1) ? -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1))
                        : m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    }
    D = 1.0 + aj * D;
    if (std::fabs(D) < tiny) D = tiny;
    C = 1.0 + aj / C;
    if (std::fabs(C) < tiny) C = tiny;
    D = 1.0 / D;
    const double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < 1e-16) break;
  }
  return std::exp(ln_pre) * f;
}

double sphere_cdf(double u, int d) {
  const double al = 0.5 * (d - 1);
  return inc_beta(al, al, std::fmin(std::fmax(0.5 * (1.0 + u), 0.0), 1.0));
}

// int_a^b u f(u) du = ((1 - a^2)^(k+1) - (1 - b^2)^(k+1)) / (2 (k+1) B(1/2, k+1)), k = (d-3)/2
double sphere_partial_mean(double a, double b, int d) {
  const double k = 0.5 * (d - 3);
  const double lb = std::lgamma(0.5) + std::lgamma(k + 1.0) - std::lgamma(k + 1.5);
  auto g = [&](double u) {
    const double v = 1.0 - u * u;
    return v <= 0.0 ? 0.0 : std::exp((k + 1.0) * std::log(v) - lb);
  };
  return (g(a) - g(b)) / (2.0 * (k + 1.0));
}

void lloyd_max_sphere(int levels, int d, double* c) {
  const double sd = std::sqrt((double)d);
  // start at the quantiles (i + 1/2) / L of the law (bisection on the CDF)
  for (int i = 0; i < levels; ++i) {
    const double p = (i + 0.5) / levels;
    double lo = -1.0, hi = 1.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (sphere_cdf(mid, d) < p) lo = mid; else hi = mid;
    }
    c[i] = sd * 0.5 * (lo + hi);
  }
  std::vector<double> t(levels + 1), nc(levels);
  for (int it = 0; it < 200000; ++it) {
    t[0] = -1.0;
    t[levels] = 1.0;
    for (int i = 1; i < levels; ++i) t[i] = std::fmin(std::fmax(0.5 * (c[i - 1] + c[i]) / sd, -1.0), 1.0);
    double delta = 0.0;
    for (int i = 0; i < levels; ++i) {
      const double p = sphere_cdf(t[i + 1], d) - sphere_cdf(t[i], d);
      nc[i] = sd * sphere_partial_mean(t[i], t[i + 1], d) / p;
      delta = std::fmax(delta, std::fabs(nc[i] - c[i]));
    }
    for (int i = 0; i < levels; ++i) c[i] = nc[i];
    if (delta < 1e-14) break;
  }
  std::vector<double> s(c, c + levels);
  for (int i = 0; i < levels; ++i) c[i] = 0.5 * (s[i] - s[levels - 1 - i]);
}

// ---- seeded stream: SplitMix64 (Steele, Lea, Flood 2014; Vigna's finalizer)
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return ((double)(next() >> 11) + 0.5) * 0x1.0p-53; }
};

// d*d normals, row-major; Box-Muller pairs (cos first, then sin).
void gaussian(uint64_t seed, int d, std::vector<double>& g) {
  SplitMix64 rng{seed};
  const int n = d * d;
  g.resize(n);
  for (int k = 0; k < n; k += 2) {
    const double u1 = rng.uniform(), u2 = rng.uniform();
    const double r = std::sqrt(-2.0 * std::log(u1));
    g[k] = r * std::cos(2.0 * M_PI * u2);
    if (k + 1 < n) g[k + 1] = r * std::sin(2.0 * M_PI * u2);
  }
}

// Q * diag(sign(diag R)) of the Householder QR of the row-major d x d matrix a.
void haar_from_gaussian(int d, std::vector<double>& a, std::vector<double>& q) {
  std::vector<double> vs((size_t)d * d, 0.0);   // Householder vectors, column k in vs[k*d ..]
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += a[(size_t)i * d + k] * a[(size_t)i * d + k];
    const double norm = std::sqrt(norm2);
    double* v = &vs[(size_t)k * d];
    if (k == d - 1 || norm == 0.0) {
      rdiag[k] = a[(size_t)k * d + k];
      continue;                                  // identity reflector
    }
    const double x0 = a[(size_t)k * d + k];
    const double alpha = x0 >= 0.0 ? -norm : norm;   // R_kk after the reflection
    for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (int i = k; i < d; ++i) vn2 += v[i] * v[i];
    const double vn = std::sqrt(vn2);
    for (int i = k; i < d; ++i) v[i] /= vn;
    // A[k:, k:] -= 2 v (v^T A[k:, k:])
    for (int j = k; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * a[(size_t)i * d + j];
      for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= 2.0 * v[i] * s;
    }
    rdiag[k] = alpha;
  }
  // Q = H_0 H_1 ... H_{d-2}: apply the reflectors to I from the last one back.
  q.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 2; k >= 0; --k) {
    const double* v = &vs[(size_t)k * d];
    double vv = 0.0;
    for (int i = k; i < d; ++i) vv += v[i] * v[i];
    if (vv == 0.0) continue;
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * q[(size_t)i * d + j];
      for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= 2.0 * v[i] * s;
    }
  }
  // sign fix: column k times sign(R_kk), sign(0) = +1
  for (int k = 0; k < d; ++k) {
    if (rdiag[k] < 0.0)
      for (int i = 0; i < d; ++i) q[(size_t)i * d + k] = -q[(size_t)i * d + k];
  }
}

}  // namespace

namespace tq {

// Midpoints of neighbouring centroids; adding +0.0 turns a -0.0 midpoint into +0.0.
void thresholds_from_centroids(const float* c, int levels, float* t) {
  for (int i = 0; i + 1 < levels; ++i) t[i] = (float)(0.5 * ((double)c[i] + (double)c[i + 1])) + 0.0f;
}

}  // namespace tq

extern "C" int tq_make_codebook(int32_t bits, int32_t d, float* centroids, float* thresholds) {
  if (centroids == nullptr || bits < 1 || bits > 4 || d <= 0) return TQ_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != tq::kD && d != 256) return TQ_ERR_UNSUPPORTED;
  const int L = 1 << bits;
  double c[16];
  lloyd_max(L, c);
  double c16[16];
  for (int i = 0; i < L; ++i) c16[i] = round_to_half(c[i]);
  for (int i = 0; i < L; ++i) centroids[i] = (float)c16[i];
  if (thresholds != nullptr) {
    for (int i = 0; i + 1 < L; ++i) thresholds[i] = (float)(0.5 * (c16[i] + c16[i + 1]));
    thresholds[L / 2 - 1] = 0.0f;
  }
  return TQ_OK;
}

extern "C" int tq_make_codebook_sphere(int32_t bits, int32_t d, float* centroids, float* thresholds) {
  if (centroids == nullptr || bits < 1 || bits > 4 || d < 3 || d > 65536) return TQ_ERR_INVALID_ARGUMENT;
  const int L = 1 << bits;
  double c[16];
  lloyd_max_sphere(L, d, c);
  double c16[16];
  for (int i = 0; i < L; ++i) c16[i] = round_to_half(c[i]);
  for (int i = 0; i < L; ++i) centroids[i] = (float)c16[i];
  if (thresholds != nullptr) {
    for (int i = 0; i + 1 < L; ++i) thresholds[i] = (float)(0.5 * (c16[i] + c16[i + 1]));
    thresholds[L / 2 - 1] = 0.0f;
  }
  return TQ_OK;
}

extern "C" int tq_make_rotation(uint64_t seed, int32_t d, int32_t kind, float* out) {
  if (out == nullptr || d <= 0 || (kind != TQ_MAT_HAAR && kind != TQ_MAT_GAUSSIAN && kind != TQ_MAT_HADAMARD))
    return TQ_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != tq::kD && d != 256) return TQ_ERR_UNSUPPORTED;
  if (kind == TQ_MAT_HADAMARD) {
    // H D / sqrt(d): H[i][j] = (-1)^popcount(i & j), s_j from the top bit of output j+1
    SplitMix64 sm{seed};
    std::vector<double> sgn(d);
    for (int j = 0; j < d; ++j) sgn[j] = (sm.next() >> 63) ? -1.0 : 1.0;
    const double inv = 1.0 / std::sqrt((double)d);
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j)
        out[i * d + j] = (float)(((__builtin_popcount((unsigned)(i & j)) & 1) ? -inv : inv) * sgn[j]);
    return TQ_OK;
  }
  std::vector<double> g;
  gaussian(seed, d, g);
  if (kind == TQ_MAT_GAUSSIAN) {
    for (int i = 0; i < d * d; ++i) out[i] = (float)g[i];
    return TQ_OK;
  }
  std::vector<double> q;
  haar_from_gaussian(d, g, q);
  for (int i = 0; i < d * d; ++i) out[i] = (float)q[i];
  return TQ_OK;
}
