// Host-side codec construction for libtq: counter-based Gaussian draws, Haar rotation by
// Householder QR, Gaussian sketch, Lloyd-Max codebook for the rotated-coordinate law.
//
// Sources (page title, section):
//   7minutos.es TurboQuant walkthrough, "Etapa 1 (PolarQuant)": y = R x with R a random
//   orthogonal matrix; a rotated coordinate u_i of a unit vector satisfies
//   u_i^2 ~ Beta(1/2, (d-1)/2); the Lloyd-Max levels (boundaries at midpoints, levels at cell
//   means) depend only on (d, bits) and are computed once.
//   Same walkthrough, "Etapa 2 (Corrección Residual)": the projection S is random Gaussian.
//   TurboESM summary, section 2.B: one rotation per layer and head.
//
// Generators: SplitMix64 (Steele, Lea, Flood 2014), output k of stream `seed` is
// mix(seed + (k+1) * 0x9E3779B97F4A7C15); Box-Muller (1958) on outputs 2j, 2j+1 with
// u1 = 1 - (x >> 11) 2^-53 and u2 = (x >> 11) 2^-53.  Haar matrices: QR with the signs of
// diag(R) folded into Q (Mezzadri 2007).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {

static inline uint64_t splitmix64_at(uint64_t seed, uint64_t k) {
  uint64_t z = seed + (k + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline double to_unit(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

void gaussian_fill(uint64_t seed, int64_t count, double *out) {
  const double two_pi = 2.0 * M_PI;
  for (int64_t j = 0; 2 * j < count; ++j) {
    const double u1 = 1.0 - to_unit(splitmix64_at(seed, 2 * j));
    const double u2 = to_unit(splitmix64_at(seed, 2 * j + 1));
    const double rho = std::sqrt(-2.0 * std::log(u1));
    const double ang = two_pi * u2;
    out[2 * j] = rho * std::cos(ang);
    if (2 * j + 1 < count) out[2 * j + 1] = rho * std::sin(ang);
  }
}

// Householder QR of the row-major d x d matrix a (overwritten); q receives the orthogonal
// factor with the signs of R's diagonal folded in, so that q is the unique QR factor whose
// R has a positive diagonal.
static void haar_from_gaussian(int d, std::vector<double> &a, std::vector<double> &q) {
  std::vector<double> vs((size_t)d * d, 0.0);  // Householder vectors, row k holds v_k
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += a[(size_t)i * d + k] * a[(size_t)i * d + k];
    nrm = std::sqrt(nrm);
    const double x0 = a[(size_t)k * d + k];
    const double alpha = (x0 >= 0.0) ? -nrm : nrm;  // R_kk
    double *v = &vs[(size_t)k * d];
    for (int i = k; i < d; ++i) v[i] = a[(size_t)i * d + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    rdiag[k] = alpha;
    if (vn == 0.0) continue;  // column already reduced: H_k = I
    const double inv = 2.0 / vn;
    for (int j = k; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * a[(size_t)i * d + j];
      s *= inv;
      for (int i = k; i < d; ++i) a[(size_t)i * d + j] -= s * v[i];
    }
  }
  // Q = H_0 H_1 ... H_{d-1}; build by applying the reflectors to I from the right end.
  q.assign((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double *v = &vs[(size_t)k * d];
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    if (vn == 0.0) continue;
    const double inv = 2.0 / vn;
    for (int j = 0; j < d; ++j) {  // q <- H_k q
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * q[(size_t)i * d + j];
      s *= inv;
      for (int i = k; i < d; ++i) q[(size_t)i * d + j] -= s * v[i];
    }
  }
  // fold sign(R_kk) into column k of Q
  for (int k = 0; k < d; ++k) {
    if (rdiag[k] < 0.0)
      for (int i = 0; i < d; ++i) q[(size_t)i * d + k] = -q[(size_t)i * d + k];
  }
}

void haar_rotation64(uint64_t seed, int d, std::vector<double> &q) {
  std::vector<double> a((size_t)d * d);
  gaussian_fill(seed, (int64_t)d * d, a.data());
  haar_from_gaussian(d, a, q);
}

// ------------------------------------------------------------------------ Lloyd-Max

// Gauss-Legendre nodes and weights on [-1, 1] by Newton iteration on P_n.
static void gauss_legendre(int n, std::vector<double> &x, std::vector<double> &w) {
  x.resize(n);
  w.resize(n);
  for (int i = 0; i < (n + 1) / 2; ++i) {
    double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = z;
      for (int k = 2; k <= n; ++k) {
        const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
        p0 = p1;
        p1 = p2;
      }
      dp = n * (z * p1 - p0) / (z * z - 1.0);
      const double dz = p1 / dp;
      z -= dz;
      if (std::fabs(dz) < 1e-17) break;
    }
    x[i] = -z;
    x[n - 1 - i] = z;
    w[i] = w[n - 1 - i] = 2.0 / ((1.0 - z * z) * dp * dp);
  }
}

struct BetaCoordLaw {
  int d;
  double logc;
  std::vector<double> gx, gw;
  explicit BetaCoordLaw(int d_) : d(d_) {
    // 1 / B(1/2, (d-1)/2) = Gamma(d/2) / (Gamma(1/2) Gamma((d-1)/2))
    logc = std::lgamma(0.5 * d) - std::lgamma(0.5) - std::lgamma(0.5 * (d - 1));
    gauss_legendre(48, gx, gw);
  }
  double density(double x) const {
    const double t = 1.0 - x * x;
    if (t <= 0.0) return 0.0;
    return std::exp(logc + 0.5 * (d - 3) * std::log(t));
  }
  // mass and first moment of [a, b], split into panels for the steep tails at large d
  void cell(double a, double b, double &mass, double &mom) const {
    const int panels = 16;
    mass = 0.0;
    mom = 0.0;
    const double h = (b - a) / panels;
    for (int p = 0; p < panels; ++p) {
      const double lo = a + p * h, hi = (p + 1 == panels) ? b : a + (p + 1) * h;
      const double half = 0.5 * (hi - lo), mid = 0.5 * (hi + lo);
      double pm = 0.0, pq = 0.0;
      for (size_t i = 0; i < gx.size(); ++i) {
        const double x = mid + half * gx[i];
        const double f = density(x) * gw[i];
        pm += f;
        pq += f * x;
      }
      mass += pm * half;
      mom += pq * half;
    }
  }
};

int lloyd_max_codebook(int d, int bits, std::vector<double> &c, std::vector<double> &t) {
  const int L = 1 << bits;
  BetaCoordLaw law(d);
  c.resize(L);
  const double span = std::fmin(2.0 / std::sqrt((double)d), 0.9);
  for (int j = 0; j < L; ++j) c[j] = span * (2.0 * j + 1.0 - L) / L;
  std::vector<double> nc(L);
  double best = INFINITY;
  int since = 0;
  bool done = false;
  for (int it = 0; it < 400000 && !done; ++it) {
    double maxc = 0.0, step = 0.0;
    for (int j = 0; j < L; ++j) {
      const double a = (j == 0) ? -1.0 : 0.5 * (c[j - 1] + c[j]);
      const double b = (j == L - 1) ? 1.0 : 0.5 * (c[j] + c[j + 1]);
      double mass, mom;
      law.cell(a, b, mass, mom);
      nc[j] = mom / mass;
    }
    for (int j = 0; j < L; ++j) {
      maxc = std::fmax(maxc, std::fabs(nc[j]));
      step = std::fmax(step, std::fabs(nc[j] - c[j]));
    }
    c = nc;
    step /= maxc;
    if (step <= 1e-14) done = true;
    else if (step < best) { best = step; since = 0; }
    else if (best <= 1e-12 && ++since >= 200) done = true;
  }
  if (!done) return TQ_EINVAL;
  std::vector<double> sym(L);
  for (int j = 0; j < L; ++j) sym[j] = 0.5 * (c[j] - c[L - 1 - j]);
  c = sym;
  t.resize(L - 1);
  for (int j = 0; j + 1 < L; ++j) t[j] = 0.5 * (c[j] + c[j + 1]);
  return TQ_OK;
}

// Law of a polar node's angle psi = atan2(r_b, r_a) on [0, pi/2] when each child holds k
// coordinates of a uniform unit vector (hada.io TurboQuant page, "PolarQuant: um novo 'ângulo'
// para compressão": the angles' law is known and concentrated): r_a^2 / (r_a^2 + r_b^2) is
// Beta(k/2, k/2), so psi has density 2 / B(k/2, k/2) sin^(k-1) psi cos^(k-1) psi (uniform for
// k = 1).
struct AngleLaw {
  int k;
  double logc;
  std::vector<double> gx, gw;
  explicit AngleLaw(int k_) : k(k_) {
    logc = std::log(2.0) + std::lgamma((double)k) - 2.0 * std::lgamma(0.5 * k);
    gauss_legendre(48, gx, gw);
  }
  double density(double p) const {
    if (k == 1) return 2.0 / M_PI;
    const double sc = std::sin(p) * std::cos(p);
    if (sc <= 0.0) return 0.0;
    return std::exp(logc + (k - 1) * std::log(sc));
  }
  void cell(double a, double b, double &mass, double &mom) const {
    const int panels = 16;
    mass = 0.0;
    mom = 0.0;
    const double h = (b - a) / panels;
    for (int p = 0; p < panels; ++p) {
      const double lo = a + p * h, hi = (p + 1 == panels) ? b : a + (p + 1) * h;
      const double half = 0.5 * (hi - lo), mid = 0.5 * (hi + lo);
      double pm = 0.0, pq = 0.0;
      for (size_t i = 0; i < gx.size(); ++i) {
        const double x = mid + half * gx[i];
        const double f = density(x) * gw[i];
        pm += f;
        pq += f * x;
      }
      mass += pm * half;
      mom += pq * half;
    }
  }
};

// Lloyd-Max levels of AngleLaw(k) with L levels, ascending in [0, pi/2], symmetric about pi/4.
// k = 1: the uniform law's equal cells.  Otherwise the law's quantiles (j + 1/2) / L start the
// iteration, so every cell holds mass however concentrated the law is.
int polar_angle_levels(int k, int L, std::vector<double> &c) {
  const double half = 0.5 * M_PI;
  c.resize(L);
  if (k == 1) {
    for (int j = 0; j < L; ++j) c[j] = (j + 0.5) * half / L;
    return TQ_OK;
  }
  AngleLaw law(k);
  for (int j = 0; j < L; ++j) {
    const double target = (j + 0.5) / L;
    double lo = 0.0, hi = half;
    for (int it = 0; it < 64; ++it) {
      const double mid = 0.5 * (lo + hi);
      double mass, mom;
      law.cell(0.0, mid, mass, mom);
      (mass < target ? lo : hi) = mid;
    }
    c[j] = 0.5 * (lo + hi);
  }
  std::vector<double> nc(L);
  double best = INFINITY;
  int since = 0;
  bool done = false;
  for (int it = 0; it < 400000 && !done; ++it) {
    double maxc = 0.0, step = 0.0;
    for (int j = 0; j < L; ++j) {
      const double a = (j == 0) ? 0.0 : 0.5 * (c[j - 1] + c[j]);
      const double b = (j == L - 1) ? half : 0.5 * (c[j] + c[j + 1]);
      double mass, mom;
      law.cell(a, b, mass, mom);
      nc[j] = mass > 0.0 ? mom / mass : c[j];
    }
    for (int j = 0; j < L; ++j) {
      maxc = std::fmax(maxc, std::fabs(nc[j]));
      step = std::fmax(step, std::fabs(nc[j] - c[j]));
    }
    c = nc;
    step /= maxc;
    if (step <= 1e-13) done = true;
    else if (step < best) { best = step; since = 0; }
    else if (best <= 1e-11 && ++since >= 200) done = true;
  }
  if (!done) return TQ_EINVAL;
  std::vector<double> sym(L);
  for (int j = 0; j < L; ++j) sym[j] = 0.5 * (c[j] + (half - c[L - 1 - j]));
  c = sym;
  return TQ_OK;
}

}  // namespace tq

// ------------------------------------------------------------------------ C ABI

extern "C" int tq_calibrate_codebook(const float *host_u, int64_t n, int32_t bits, const float *host_init,
                                     int32_t max_iter, int32_t m, float *host_centroids, float *host_thresholds,
                                     float *host_ebar, float *host_resid_scale) {
  if (!host_u || !host_init || !host_centroids || !host_thresholds || !host_ebar) return TQ_EINVAL;
  if (n < 1 || bits < 1 || bits > 8 || max_iter < 1 || m < 1) return TQ_EINVAL;
  const int L = 1 << bits;
  std::vector<double> lv(L), sum(L), t(L - 1);
  std::vector<int64_t> cnt(L);
  for (int j = 0; j < L; ++j) lv[j] = host_init[j];
  for (int j = 0; j + 1 < L; ++j)
    if (!(lv[j] <= lv[j + 1])) return TQ_EINVAL;  // ascending (and not NaN)
  // the cell of u: the number of midpoints t_j with u >= t_j (binary search)
  auto cell = [&](double u) {
    int lo = 0, hi = L - 1;  // answer in [lo, hi]
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;  // is u >= t[mid - 1]?
      if (u >= t[mid - 1]) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  auto midpoints = [&]() {
    for (int j = 0; j + 1 < L; ++j) t[j] = 0.5 * (lv[j] + lv[j + 1]);
  };
  for (int it = 0; it < max_iter; ++it) {
    midpoints();
    std::fill(sum.begin(), sum.end(), 0.0);
    std::fill(cnt.begin(), cnt.end(), 0);
    for (int64_t i = 0; i < n; ++i) {
      const double u = host_u[i];
      const int c = cell(u);
      sum[c] += u;
      ++cnt[c];
    }
    double moved = 0.0, big = 0.0;
    for (int j = 0; j < L; ++j) {
      const double nv = cnt[j] ? sum[j] / (double)cnt[j] : lv[j];
      moved = std::fmax(moved, std::fabs(nv - lv[j]));
      lv[j] = nv;
      big = std::fmax(big, std::fabs(nv));
    }
    if (moved <= 1e-12 * big) break;
  }
  midpoints();
  double e = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double u = host_u[i];
    e += std::fabs(u - lv[cell(u)]);
  }
  for (int j = 0; j < L; ++j) host_centroids[j] = (float)lv[j];
  for (int j = 0; j + 1 < L; ++j) host_thresholds[j] = (float)t[j];
  const double ebar = e / (double)n;
  *host_ebar = (float)ebar;
  if (host_resid_scale) *host_resid_scale = (float)(ebar * (double)m / std::sqrt(M_PI / 2.0));
  return TQ_OK;
}

extern "C" int tq_make_rotation(uint64_t seed, int32_t d, float *host_out) {
  if (!host_out) return TQ_EINVAL;
  if (d < 3 || d > 1024) return TQ_EUNSUPPORTED;
  std::vector<double> q;
  tq::haar_rotation64(seed, d, q);
  for (size_t i = 0; i < q.size(); ++i) host_out[i] = (float)q[i];
  return TQ_OK;
}

extern "C" int tq_make_head_rotations(uint64_t seed_pi, const uint64_t *host_basis_seeds,
                                      int32_t n_rot, int32_t d, float *host_out) {
  if (!host_out || !host_basis_seeds || n_rot < 1) return TQ_EINVAL;
  if (d < 3 || d > 1024) return TQ_EUNSUPPORTED;
  std::vector<double> pi, b;
  tq::haar_rotation64(seed_pi, d, pi);
  for (int r = 0; r < n_rot; ++r) {
    tq::haar_rotation64(host_basis_seeds[r], d, b);
    float *o = host_out + (size_t)r * d * d;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int k = 0; k < d; ++k) s += pi[(size_t)i * d + k] * b[(size_t)k * d + j];
        o[(size_t)i * d + j] = (float)s;
      }
  }
  return TQ_OK;
}

extern "C" int tq_make_sketch(uint64_t seed, int32_t m, int32_t d, float *host_out) {
  if (!host_out || m < 1 || d < 1) return TQ_EINVAL;
  std::vector<double> g((size_t)m * d);
  tq::gaussian_fill(seed, (int64_t)m * d, g.data());
  for (size_t i = 0; i < g.size(); ++i) host_out[i] = (float)g[i];
  return TQ_OK;
}

extern "C" int tq_make_codebook(int32_t d, int32_t bits, float *host_centroids,
                                float *host_thresholds) {
  if (!host_centroids || !host_thresholds) return TQ_EINVAL;
  if (d < 3 || bits < 1 || bits > 8) return TQ_EUNSUPPORTED;
  std::vector<double> c, t;
  const int st = tq::lloyd_max_codebook(d, bits, c, t);
  if (st != TQ_OK) return st;
  for (size_t j = 0; j < c.size(); ++j) host_centroids[j] = (float)c[j];
  for (size_t j = 0; j < t.size(); ++j) host_thresholds[j] = (float)t[j];
  return TQ_OK;
}

extern "C" int tq_make_polar_tables(int32_t d, int32_t ab, float *host_tables) {
  if (!host_tables) return TQ_EINVAL;
  int levels = 0;
  while ((1 << levels) < d) ++levels;
  // more than 16 levels per table would make the Lloyd iteration (linear convergence, many
  // levels) take minutes; the device codec uses 2 to 4 angle bits
  if (d < 4 || (1 << levels) != d || d > 1024 || ab < 1 || ab > 4) return TQ_EINVAL;
  const int n = 1 << ab;
  for (int l = 1; l <= levels; ++l) {
    std::vector<double> c;
    const int st = tq::polar_angle_levels(1 << (l - 1), n, c);
    if (st != TQ_OK) return st;
    float *tab = host_tables + (int64_t)(l - 1) * 4 * n;
    for (int j = 0; j < 4 * n; ++j) tab[j] = 0.0f;
    for (int j = 0; j < n; ++j) {
      tab[j] = (float)std::cos(c[j]);
      tab[n + j] = (float)std::sin(c[j]);
    }
    for (int j = 0; j + 1 < n; ++j) {
      const double t = 0.5 * (c[j] + c[j + 1]);
      const double ct = std::cos(t), sn = std::sin(t);
      tab[2 * n + j] = (float)(ct * ct);
      tab[3 * n + j] = (float)(sn * sn);
    }
  }
  return TQ_OK;
}

extern "C" const char *tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_EALIGN: return "misaligned pointer or stride";
    case TQ_EWORKSPACE: return "workspace missing or too small";
    case TQ_EHIP: return "HIP launch failed";
    case TQ_ESCRATCH: return "the call needs more scratch memory than the library's static maximum";
    default: return "unknown status";
  }
}

extern "C" const char *tq_version(void) { return "libtq 0.1 (gfx950)"; }
