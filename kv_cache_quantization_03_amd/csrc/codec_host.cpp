// Host-side codec construction: seeded signs and Gaussian matrix, Lloyd-Max
// codebook for the post-rotation coordinate law, and the upload of the device
// tables.  Runs once per codec; nothing here is on the per-token path.
//
// Pages: 「谷歌 TurboQuant 深度拆解」 第二部分 (rotation -> known coordinate law ->
// optimal scalar quantizer without per-block constants; QJL Gaussian
// projection) and 第六部分 (the coordinate density);
// 「TurboQuant 学习路径」 二.2 (Gaussian JL matrix, random signs D of the FJLT)
// and 三.4 (Lloyd-Max).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "tq_internal.h"

namespace tq {

namespace {

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output i of the stream seeded
// with s0 is mix(s0 + (i+1) * golden).
inline uint64_t splitmix64_at(uint64_t s0, uint64_t i) {
  uint64_t z = s0 + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr uint64_t kTagSigns = 1, kTagGauss = 2;

// ---- sphere coordinate law -------------------------------------------------
// f(x) = C (1-x²)^α on [-1,1], α = (d-3)/2, C = Γ(d/2) / (√π Γ((d-1)/2)).
// CDF through J_α(t) = ∫_0^t (1-x²)^α dx with the reduction formula
//   J_α = [t (1-t²)^α + 2α J_{α-1}] / (2α + 1),
// started at J_{-1/2}(t) = asin t (d even) or J_0(t) = t (d odd).
struct SphereLaw {
  int d;
  double alpha, C;
  explicit SphereLaw(int d_) : d(d_) {
    alpha = (d - 3) / 2.0;
    C = std::exp(std::lgamma(d / 2.0) - 0.5 * std::log(M_PI) - std::lgamma((d - 1) / 2.0));
  }
  double J(double t) const {  // t in [0, 1]
    const bool even = (d % 2) == 0;
    double a = even ? -0.5 : 0.0;
    double j = even ? std::asin(t) : t;
    const double u = 1.0 - t * t;
    while (a < alpha - 1e-9) {
      a += 1.0;
      j = (t * std::pow(u, a) + 2.0 * a * j) / (2.0 * a + 1.0);
    }
    return j;
  }
  double cdf(double t) const {
    if (t <= -1.0) return 0.0;
    if (t >= 1.0) return 1.0;
    const double v = C * J(std::fabs(t));
    return t >= 0 ? 0.5 + v : 0.5 - v;
  }
  // ∫_lo^hi x f(x) dx = C/(2(α+1)) [(1-lo²)^(α+1) - (1-hi²)^(α+1)]
  double first_moment(double lo, double hi) const {
    const double a1 = alpha + 1.0;
    auto g = [&](double x) {
      const double u = 1.0 - x * x;
      return u <= 0 ? 0.0 : std::pow(u, a1);
    };
    return C / (2.0 * a1) * (g(lo) - g(hi));
  }
};

// Lloyd-Max: boundaries at midpoints, centroids at conditional means, codebook
// kept symmetric; start from evenly spaced levels in ±2/sqrt(d).  The density is
// log-concave, so the fixed point is unique and the start does not matter.
int lloyd_max(int d, int b, std::vector<double>* cent, std::vector<double>* bnd) {
  const int L = 1 << b;
  SphereLaw law(d);
  std::vector<double> c(L), nc(L), edges(L + 1);
  const double sd = std::sqrt(static_cast<double>(d));
  for (int k = 0; k < L; ++k) c[k] = ((2.0 * k + 1.0) / L - 1.0) * 2.0 / sd;
  int it = 0;
  for (it = 1; it <= 20000; ++it) {
    edges[0] = -1.0;
    edges[L] = 1.0;
    for (int k = 1; k < L; ++k) edges[k] = 0.5 * (c[k - 1] + c[k]);
    for (int k = 0; k < L; ++k) {
      const double mass = law.cdf(edges[k + 1]) - law.cdf(edges[k]);
      nc[k] = law.first_moment(edges[k], edges[k + 1]) / mass;
    }
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double v = 0.5 * (nc[k] - nc[L - 1 - k]);
      delta = std::fmax(delta, std::fabs(v - c[k]));
      c[k] = v;
    }
    if (delta * sd < 1e-13) break;
  }
  cent->assign(c.begin(), c.end());
  bnd->resize(L - 1);
  for (int k = 0; k + 1 < L; ++k) (*bnd)[k] = 0.5 * (c[k] + c[k + 1]);
  return it;
}

// ---- recursive polar angle laws ---------------------------------------------
// Level 1 angles are uniform on [0, 2π).  For level l > 1 with n = 2^(l-1),
// sin²θ ~ Beta(n/2, n/2): f(θ) = 2/B(n/2, n/2) (sin θ cos θ)^(n-1) on [0, π/2].
// With x = -cos 2θ, (sin θ cos θ)^(n-1) dθ ∝ (1 - x²)^((n-2)/2) dx: x follows
// the coordinate law of a unit vector in n + 1 dimensions, so the CDF is
// SphereLaw(n + 1).cdf(-cos 2θ).  The first moment ∫ θ f(θ) dθ is integrated
// with composite Gauss-Legendre (16 nodes, nodes by Newton on P_16).
struct GaussLegendre16 {
  double x[16], w[16];
  GaussLegendre16() {
    const int n = 16;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5)), pp = 0;
      for (int it = 0; it < 100; ++it) {
        double p1 = 1, p2 = 0;
        for (int j = 1; j <= n; ++j) {
          const double p3 = p2;
          p2 = p1;
          p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
        }
        pp = n * (z * p1 - p2) / (z * z - 1.0);
        const double z1 = z;
        z = z1 - p1 / pp;
        if (std::fabs(z - z1) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * pp * pp);
    }
  }
};

struct PolarLaw {
  int n;
  double logC;
  SphereLaw x_law;
  explicit PolarLaw(int level) : n(1 << (level - 1)), x_law(n + 1) {
    logC = std::log(2.0) - (2.0 * std::lgamma(n / 2.0) - std::lgamma(static_cast<double>(n)));
  }
  double density(double t) const {
    const double sc = std::sin(t) * std::cos(t);
    return sc <= 0 ? 0.0 : std::exp(logC + (n - 1) * std::log(sc));
  }
  double cdf(double t) const {
    if (t <= 0) return 0.0;
    if (t >= M_PI / 2) return 1.0;
    return x_law.cdf(-std::cos(2.0 * t));
  }
  double first_moment(double lo, double hi) const {
    static const GaussLegendre16 gl;
    constexpr int kPanels = 64;
    const double h = (hi - lo) / kPanels;
    double acc = 0;
    for (int p = 0; p < kPanels; ++p) {
      const double a = lo + p * h, mid = a + 0.5 * h;
      for (int i = 0; i < 16; ++i) {
        const double t = mid + 0.5 * h * gl.x[i];
        acc += 0.5 * h * gl.w[i] * t * density(t);
      }
    }
    return acc;
  }
};

// Codebook of one level's angle: level 1 the uniform quantizer of the circle;
// level > 1 Lloyd-Max on f, kept symmetric about π/4 (f is log-concave there,
// so the fixed point is unique).
int polar_lloyd_max(int level, int b, std::vector<double>* cent, std::vector<double>* bnd) {
  const int L = 1 << b;
  cent->assign(L, 0.0);
  bnd->assign(L - 1, 0.0);
  if (level == 1) {
    const double step = 2.0 * M_PI / L;
    for (int k = 0; k < L; ++k) (*cent)[k] = (k + 0.5) * step;
    for (int k = 1; k < L; ++k) (*bnd)[k - 1] = k * step;
    return 0;
  }
  PolarLaw law(level);
  const double w = std::fmin(M_PI / 4, 2.0 / std::sqrt(static_cast<double>(law.n)));
  std::vector<double> c(L), nc(L), edges(L + 1);
  for (int k = 0; k < L; ++k) c[k] = M_PI / 4 + ((2.0 * k + 1.0) / L - 1.0) * w;
  int it = 0;
  for (it = 1; it <= 5000; ++it) {
    edges[0] = 0.0;
    edges[L] = M_PI / 2;
    for (int k = 1; k < L; ++k) edges[k] = 0.5 * (c[k - 1] + c[k]);
    for (int k = 0; k < L; ++k)
      nc[k] = law.first_moment(edges[k], edges[k + 1]) / (law.cdf(edges[k + 1]) - law.cdf(edges[k]));
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double v = 0.5 * (nc[k] + (M_PI / 2 - nc[L - 1 - k]));
      delta = std::fmax(delta, std::fabs(v - c[k]));
      c[k] = v;
    }
    if (delta < 1e-13) break;
  }
  *cent = c;
  for (int k = 0; k + 1 < L; ++k) (*bnd)[k] = 0.5 * (c[k] + c[k + 1]);
  return it;
}

}  // namespace

tq_status_t build_polar_tables(int d, int bits, int m, uint64_t seed, HostTables* out) {
  if (d != 64 && d != 128 && d != 256) {
    set_error("the recursive polar stage is built for head_dim 64, 128 or 256");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  tq_status_t st = build_host_tables(d, bits, m, seed, out);
  if (st != TQ_SUCCESS) return st;
  try {
    out->polar = true;
    const int levels = d == 64 ? 6 : d == 128 ? 7 : 8;  // log2 d
    out->pcent.resize(levels);
    out->pbound.resize(levels);
    out->piters.resize(levels);
    for (int l = 1; l <= levels; ++l) out->piters[l - 1] = polar_lloyd_max(l, out->b, &out->pcent[l - 1], &out->pbound[l - 1]);
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed while building codec tables");
    return TQ_ERROR_OUT_OF_MEMORY;
  }
  return TQ_SUCCESS;
}

tq_status_t build_mse_tables(int d, int bits, uint64_t seed, HostTables* out) {
  if (bits < 2 || bits > 3) {
    set_error("an MSE-only codec takes bits 2 or 3 (all bits to the Lloyd-Max code)");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  // the two-stage tables of bits + 1 carry the b = bits codebook and D; S is dropped
  tq_status_t st = build_host_tables(d, bits + 1, 0, seed, out);
  if (st != TQ_SUCCESS) return st;
  out->bits = bits;
  out->m = 0;
  out->S.clear();
  out->S.shrink_to_fit();
  return TQ_SUCCESS;
}

bool supported_dim(int d) {
  return d == 64 || d == 128 || d == 256 || d == 512 || d == 1024 || d == 1536;
}

tq_status_t build_host_tables(int d, int bits, int m, uint64_t seed, HostTables* out) {
  if (d <= 0 || bits <= 0 || m < 0) {
    set_error("head_dim, bits must be > 0 and qjl_dim >= 0");
    return TQ_ERROR_INVALID_VALUE;
  }
  if (m == 0) m = d;
  if (!supported_dim(d)) {
    set_error("head_dim must be one of 64, 128, 256, 512, 1024, 1536");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if (bits < 2 || bits > 4) {
    set_error("bits must be 2, 3 or 4 (b = bits-1 Lloyd-Max bits + 1 QJL bit)");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  if (m != d) {
    set_error("qjl_dim must be 0 or equal to head_dim");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  try {
    out->d = d;
    out->bits = bits;
    out->b = bits - 1;
    out->m = m;
    out->seed = seed;
    // D_j = +1 iff the top bit of word(seed ^ 1, j) is clear.
    out->D.resize(d);
    const uint64_t s1 = seed ^ kTagSigns;
    for (int j = 0; j < d; ++j) out->D[j] = (splitmix64_at(s1, j) >> 63) ? -1.0f : 1.0f;
    // S row-major, entry k = i*d + j; pair k/2 draws two words; Box–Muller
    // (Box & Muller 1958) cosine for even k, sine for odd k; rounded to fp32.
    const size_t n = static_cast<size_t>(m) * d;
    out->S.resize(n);
    const uint64_t s2 = seed ^ kTagGauss;
    for (size_t pr = 0; pr < n / 2; ++pr) {
      const uint64_t w1 = splitmix64_at(s2, 2 * pr), w2 = splitmix64_at(s2, 2 * pr + 1);
      const double u1 = (static_cast<double>(w1 >> 11) + 1.0) * 0x1p-53;
      const double u2 = static_cast<double>(w2 >> 11) * 0x1p-53;
      const double rad = std::sqrt(-2.0 * std::log(u1));
      const double ang = 2.0 * M_PI * u2;
      out->S[2 * pr] = static_cast<float>(rad * std::cos(ang));
      out->S[2 * pr + 1] = static_cast<float>(rad * std::sin(ang));
    }
    out->iterations = lloyd_max(d, out->b, &out->centroids, &out->bounds);
  } catch (const std::bad_alloc&) {
    set_error("host allocation failed while building codec tables");
    return TQ_ERROR_OUT_OF_MEMORY;
  }
  return TQ_SUCCESS;
}

}  // namespace tq

using tq::set_error;

extern "C" tq_status_t tq_codec_build_host(int32_t head_dim, int32_t bits, int32_t qjl_dim,
                                           uint64_t seed, float* D_out, float* S_out,
                                           double* centroids, double* bounds, int32_t* iterations) {
  tq::clear_error();
  tq::HostTables t;
  tq_status_t st = tq::build_host_tables(head_dim, bits, qjl_dim, seed, &t);
  if (st != TQ_SUCCESS) return st;
  if (D_out) std::memcpy(D_out, t.D.data(), t.D.size() * sizeof(float));
  if (S_out) std::memcpy(S_out, t.S.data(), t.S.size() * sizeof(float));
  if (centroids) std::memcpy(centroids, t.centroids.data(), t.centroids.size() * sizeof(double));
  if (bounds) std::memcpy(bounds, t.bounds.data(), t.bounds.size() * sizeof(double));
  if (iterations) *iterations = t.iterations;
  return TQ_SUCCESS;
}

namespace {

// Bit-plane expansion of the codebook: with x_i = 2 bit_i - 1 a symmetric
// codebook is c(idx) = Σ_{odd |T|} α_T Π_{i∈T} x_i.  For b <= 3 the odd subsets
// are the single bits and (b = 3) the triple, whose product is 2·parity - 1.
// So c(idx) = bias + Σ_P coef_P · plane_P(idx) with planes
// {bit0, .., bit_{b-1}} (+ parity for b = 3).
void plane_expansion(const std::vector<double>& c, int b, float* coef, float* bias, int* n_planes) {
  const int L = 1 << b;
  auto alpha = [&](unsigned mask) {
    double acc = 0;
    for (int idx = 0; idx < L; ++idx) {
      double s = 1;
      for (int i = 0; i < b; ++i)
        if (mask >> i & 1) s *= 2.0 * ((idx >> i) & 1) - 1.0;
      acc += c[idx] * s;
    }
    return acc / L;
  };
  double bsum = 0;
  int np = 0;
  for (int i = 0; i < b; ++i) {
    const double a = alpha(1u << i);
    coef[np++] = static_cast<float>(2 * a);
    bsum += a;
  }
  if (b == 3) {
    const double a = alpha(7u);
    coef[np++] = static_cast<float>(2 * a);
    bsum += a;
  }
  for (int k = np; k < 4; ++k) coef[k] = 0.f;
  *bias = static_cast<float>(-bsum);
  *n_planes = np;
}

// v <- Hᵀ v for the codec's Hadamard matrix: Sylvester (symmetric) for
// d = 2^k, H12 ⊗ H_{d/12} for d = 12 * 2^k (Hᵀ = H12ᵀ ⊗ H_{d/12}).
void fwht_inplace(double* v, int n) {
  for (int h = 1; h < n; h <<= 1)
    for (int i = 0; i < n; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        const double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

void apply_hadamard_transposed(double* v, int d) {
  if ((d & (d - 1)) == 0) {
    fwht_inplace(v, d);
    return;
  }
  const int n = d / 12;
  for (int a = 0; a < 12; ++a) fwht_inplace(v + a * n, n);
  std::vector<double> t(12);
  for (int j = 0; j < n; ++j) {
    for (int b = 0; b < 12; ++b) {
      double acc = 0;
      for (int a = 0; a < 12; ++a) acc += tq::paley12(a, b) * v[a * n + j];
      t[b] = acc;
    }
    for (int b = 0; b < 12; ++b) v[b * n + j] = t[b];
  }
}

}  // namespace

namespace {
enum Stage { kTwoStage, kPolar, kMseOnly };

tq_status_t codec_create(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed, Stage stage,
                         tq_codec_t* out) {
  const bool polar = stage == kPolar;
  tq::clear_error();
  if (!out) {
    set_error("out is NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  *out = nullptr;
  tq_codec_s* c = new (std::nothrow) tq_codec_s();
  if (!c) {
    set_error("host allocation failed");
    return TQ_ERROR_OUT_OF_MEMORY;
  }
  tq_status_t st = polar               ? tq::build_polar_tables(head_dim, bits, qjl_dim, seed, &c->host)
                   : stage == kMseOnly ? tq::build_mse_tables(head_dim, bits, seed, &c->host)
                                       : tq::build_host_tables(head_dim, bits, qjl_dim, seed, &c->host);
  if (st != TQ_SUCCESS) {
    delete c;
    return st;
  }
  if (polar) {
    c->polar = true;
    tq::PolarParams& pp = c->pol;
    pp.levels = static_cast<int>(c->host.pcent.size());
    pp.nl = 1 << c->host.b;
    for (int l = 0; l < tq::kPolarMaxLevels; ++l)
      for (int k = 0; k < 16; ++k) {
        const bool in = l < pp.levels && k < pp.nl;
        pp.cosc[l][k] = in ? static_cast<float>(std::cos(c->host.pcent[l][k])) : 0.f;
        pp.sinc[l][k] = in ? static_cast<float>(std::sin(c->host.pcent[l][k])) : 0.f;
        pp.bound[l][k] = in && k + 1 < pp.nl ? static_cast<float>(c->host.pbound[l][k]) : INFINITY;
        const double bt = in && k + 1 < pp.nl ? c->host.pbound[l][k] : 0.0;
        const double cb = std::cos(bt), sb = std::sin(bt);
        pp.bcs[l][k] = l == 0 ? float2{static_cast<float>(cb), static_cast<float>(sb)}
                              : float2{static_cast<float>(cb * cb), static_cast<float>(sb * sb)};
      }
  }
  const auto& h = c->host;
  tq::DevParams& p = c->prm;
  std::memset(&p, 0, sizeof(p));
  for (size_t k = 0; k < h.centroids.size(); ++k) p.cent[k] = static_cast<float>(h.centroids[k]);
  for (size_t k = 0; k < h.bounds.size(); ++k) p.bound[k] = static_cast<float>(h.bounds[k]);
  for (size_t k = h.bounds.size(); k < 8; ++k) p.bound[k] = INFINITY;
  plane_expansion(h.centroids, h.b, p.plane_coef, &p.plane_bias, &p.n_planes);
  c->qjl = h.m > 0;
  p.qjl_kappa = c->qjl ? static_cast<float>(std::sqrt(M_PI / 2.0) / h.m) : 0.f;
  p.inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(h.d)));
  p.d = h.d;
  p.b = h.b;
  p.m = h.m;
  p.code_words = h.b * h.d / 32;
  p.sign_words = h.m / 32;

  if (hipGetDevice(&c->device) != hipSuccess) {
    set_error(std::string("hipGetDevice failed: ") + hipGetErrorString(hipGetLastError()));
    delete c;
    return TQ_ERROR_HIP;
  }
  const size_t nS = static_cast<size_t>(h.m) * h.d;
  const bool with16 = h.m == h.d && h.d % 128 == 0;  // fp16 split of S for the matrix-core projections
  const size_t bytes = (2 * nS + h.d) * sizeof(float) + (with16 ? 2 * nS * sizeof(_Float16) : 0);
  hipError_t e = hipMalloc(&c->dev_block, bytes);
  if (e != hipSuccess) {
    set_error(std::string("hipMalloc of codec tables failed: ") + hipGetErrorString(e));
    (void)hipGetLastError();
    delete c;
    return e == hipErrorOutOfMemory ? TQ_ERROR_OUT_OF_MEMORY : TQ_ERROR_HIP;
  }
  c->dS = static_cast<float*>(c->dev_block);
  c->dMt = c->dS + nS;
  c->dD = c->dMt + nS;
  if (nS == 0) c->dS = c->dMt = nullptr;  // MSE-only: no projection
  c->dS16 = with16 ? reinterpret_cast<_Float16*>(c->dD + h.d) : nullptr;
  // M = S R, row by row in fp64: M[i][j] = (Hᵀ S[i,:])[j] D[j] / sqrt(d); stored transposed.
  std::vector<float> Mt(nS);
  {
    std::vector<double> v(h.d);
    const double inv = 1.0 / std::sqrt(static_cast<double>(h.d));
    for (int i = 0; i < h.m; ++i) {
      for (int j = 0; j < h.d; ++j) v[j] = h.S[static_cast<size_t>(i) * h.d + j];
      apply_hadamard_transposed(v.data(), h.d);
      for (int j = 0; j < h.d; ++j) Mt[static_cast<size_t>(j) * h.m + i] = static_cast<float>(v[j] * h.D[j] * inv);
    }
  }
  {
    double mx = 0.0;
    for (int i = 0; i < h.m; ++i) {
      double ss = 0.0;
      for (int j = 0; j < h.d; ++j) {
        const double x = Mt[static_cast<size_t>(j) * h.m + i];
        ss += x * x;
      }
      mx = std::max(mx, std::sqrt(ss));
    }
    p.mrow_bound = std::nextafter(static_cast<float>(mx * (1.0 + 1e-6)), INFINITY);
  }
  e = hipSuccess;
  if (nS > 0) e = hipMemcpy(c->dS, h.S.data(), nS * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess && nS > 0) e = hipMemcpy(c->dMt, Mt.data(), nS * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->dD, h.D.data(), h.d * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess && with16) {
    // S = hi + lo: hi = fp16(S) (round to nearest even), lo = fp16(S - hi)
    std::vector<_Float16> s16(2 * nS);
    for (size_t i = 0; i < nS; ++i) {
      const float sv = h.S[i];
      const _Float16 hi = static_cast<_Float16>(sv);
      s16[i] = hi;
      s16[nS + i] = static_cast<_Float16>(sv - static_cast<float>(hi));
    }
    e = hipMemcpy(c->dS16, s16.data(), 2 * nS * sizeof(_Float16), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    set_error(std::string("uploading codec tables failed: ") + hipGetErrorString(e));
    (void)hipFree(c->dev_block);
    delete c;
    return TQ_ERROR_HIP;
  }
  *out = c;
  return TQ_SUCCESS;
}

}  // namespace

extern "C" tq_status_t tq_codec_create(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed,
                                       tq_codec_t* out) {
  return codec_create(head_dim, bits, qjl_dim, seed, kTwoStage, out);
}

extern "C" tq_status_t tq_codec_create_mse(int32_t head_dim, int32_t bits, uint64_t seed, tq_codec_t* out) {
  return codec_create(head_dim, bits, 0, seed, kMseOnly, out);
}

extern "C" tq_status_t tq_codec_create_polar(int32_t head_dim, int32_t bits, int32_t qjl_dim, uint64_t seed,
                                             tq_codec_t* out) {
  return codec_create(head_dim, bits, qjl_dim, seed, kPolar, out);
}

extern "C" tq_status_t tq_codec_create_vblock(int32_t head_dim, int32_t bits, int32_t mse_only, uint64_t seed,
                                              tq_codec_t* out) {
  tq::clear_error();
  if (out) *out = nullptr;
  if (head_dim != 128) {
    set_error("the 32-row block layout is built for head_dim 128");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  const tq_status_t st = codec_create(head_dim, bits, 0, seed, mse_only ? kMseOnly : kTwoStage, out);
  if (st == TQ_SUCCESS) (*out)->vblock = true;
  return st;
}

extern "C" tq_status_t tq_polar_book_host(int32_t head_dim, int32_t bits, int32_t level, double* centroids,
                                          double* bounds, int32_t* iterations) {
  tq::clear_error();
  if ((head_dim != 64 && head_dim != 128 && head_dim != 256) || bits < 2 || bits > 4) {
    set_error("the recursive polar stage is built for head_dim 64, 128 or 256 and bits 2, 3 or 4");
    return TQ_ERROR_NOT_SUPPORTED;
  }
  const int levels = head_dim == 64 ? 6 : head_dim == 128 ? 7 : 8;
  if (level < 1 || level > levels) {
    set_error("level must be in 1..log2(head_dim)");
    return TQ_ERROR_INVALID_VALUE;
  }
  std::vector<double> c, t;
  const int it = tq::polar_lloyd_max(level, bits - 1, &c, &t);
  if (centroids) std::memcpy(centroids, c.data(), c.size() * sizeof(double));
  if (bounds) std::memcpy(bounds, t.data(), t.size() * sizeof(double));
  if (iterations) *iterations = it;
  return TQ_SUCCESS;
}

extern "C" tq_status_t tq_codec_destroy(tq_codec_t c) {
  tq::clear_error();
  if (!c) {
    set_error("codec is NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  int cur = 0;
  (void)hipGetDevice(&cur);
  if (cur != c->device) (void)hipSetDevice(c->device);
  hipError_t e = c->dev_block ? hipFree(c->dev_block) : hipSuccess;
  if (cur != c->device) (void)hipSetDevice(cur);
  delete c;
  if (e != hipSuccess) {
    set_error(std::string("hipFree failed: ") + hipGetErrorString(e));
    return TQ_ERROR_HIP;
  }
  return TQ_SUCCESS;
}

extern "C" tq_status_t tq_codec_info(tq_codec_t c, tq_codec_info_t* info) {
  tq::clear_error();
  if (!c || !info) {
    set_error("codec or info is NULL");
    return TQ_ERROR_INVALID_VALUE;
  }
  std::memset(info, 0, sizeof(*info));
  const auto& h = c->host;
  info->head_dim = h.d;
  info->bits = h.bits;
  info->mse_bits = h.b;
  info->qjl_dim = h.m;
  info->code_words = c->prm.code_words;
  info->sign_words = c->prm.sign_words;
  info->record_bytes = 4 * (c->prm.code_words + c->prm.sign_words) + (c->qjl ? 8 : 4);
  info->lloyd_max_iterations = h.iterations;
  info->stage1 = c->polar ? 1 : 0;
  info->layout = c->vblock ? 1 : 0;
  info->seed = h.seed;
  for (size_t k = 0; k < h.centroids.size(); ++k) info->centroids[k] = h.centroids[k];
  for (size_t k = 0; k < h.bounds.size(); ++k) info->bounds[k] = h.bounds[k];
  return TQ_SUCCESS;
}
