// Seeded synthetic workload generator for the predictor-guided sparse FFN.
//
// This file builds inputs only: weights, biases, firing probabilities, the
// hot-first storage order and token vectors. It holds none of the method's
// arithmetic (no predictor, threshold, compaction, activation or projection)
// and is shared, as input data, by the CPU oracle and the GPU library alike.
//
// Every random value is keyed by (seed, tensor tag, layer, ORIGINAL row id,
// element block), so a row holds the same bits whatever storage order it is
// written in.  Counter-based RNG: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11).  Gaussians: Box-Muller
// in double.  Inverse normal CDF: Wichura, "Algorithm AS 241: the percentage
// points of the normal distribution", Applied Statistics 37 (1988), PPND16.
//
// Workload model (PowerInfer pages: power-law neuron activation, a few hot
// neurons fire for most inputs and many cold ones fire input-dependently):
//   p_i = clamp(C * k_i^-s, lo, hi), k = a seeded random permutation of 1..f,
//   C chosen by bisection so that mean(p) equals the target activity;
//   bias b_i = PhiInv(p_i) * ||stored row_i||_2, so that for x ~ N(0, I) the
//   pre-activation w_i.x + b_i is positive with probability exactly p_i.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- Philox4x32-10
struct P4 { uint32_t v[4]; };

inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

inline P4 philox4x32_10(P4 ctr, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;   // round multipliers
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;   // Weyl key increments
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(M0, ctr.v[0], &hi0, &lo0);
    mulhilo32(M1, ctr.v[2], &hi1, &lo1);
    P4 n;
    n.v[0] = hi1 ^ ctr.v[1] ^ k0;
    n.v[1] = lo1;
    n.v[2] = hi0 ^ ctr.v[3] ^ k1;
    n.v[3] = lo0;
    ctr = n;
    k0 += W0;
    k1 += W1;
  }
  return ctr;
}

// 53-bit uniform in the open interval (0, 1) and the half-open [0, 1).
inline double u53_open(uint32_t a, uint32_t b) {
  uint64_t m = (((uint64_t)a << 32) | b) >> 11;
  return ((double)m + 0.5) * 0x1.0p-53;
}
inline double u53_half(uint32_t a, uint32_t b) {
  uint64_t m = (((uint64_t)a << 32) | b) >> 11;
  return (double)m * 0x1.0p-53;
}

// Two standard normals from one Philox block (Box-Muller).
inline void box_muller(const P4& r, double* z0, double* z1) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = u53_open(r.v[0], r.v[1]);
  double u2 = u53_half(r.v[2], r.v[3]);
  double rad = std::sqrt(-2.0 * std::log(u1));
  *z0 = rad * std::cos(two_pi * u2);
  *z1 = rad * std::sin(two_pi * u2);
}

// ------------------------------------------------------ double -> IEEE binary16
// Round-to-nearest-even, with subnormals, overflow to infinity and NaN.
inline uint16_t f64_to_f16_bits(double x) {
  uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00u;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);  // rounds past 65504
  if (a < 0x1.0p-14) {                                   // subnormal range
    double q = std::nearbyint(a * 0x1.0p24);             // exact scaling, RNE
    return (uint16_t)(sign | (uint16_t)q);               // q == 1024 -> min normal
  }
  int e;
  double m = std::frexp(a, &e);          // a = m * 2^e, m in [0.5, 1)
  double q = std::nearbyint(m * 2048.0); // 11 significant bits, RNE
  int exp = e - 1;                       // a = (q/1024) * 2^exp
  if (q >= 2048.0) { q = 1024.0; exp += 1; }
  if (exp > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((exp + 15) << 10) | (uint16_t)((uint32_t)q - 1024u));
}

inline double f16_bits_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

template <typename F>
void parallel_rows(int64_t n, int nthreads, F&& fn) {
  if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
  if (n < 64 || nthreads == 1) { fn(0, n); return; }
  nthreads = (int)std::min<int64_t>(nthreads, n);
  std::vector<std::thread> th;
  int64_t chunk = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    int64_t a = t * chunk, b = std::min(n, a + chunk);
    if (a >= b) break;
    th.emplace_back([=, &fn] { fn(a, b); });
  }
  for (auto& x : th) x.join();
}

// --------------------------------------------------------------- AS 241 PPND16
double ppnd16(double p) {
  const double split1 = 0.425, split2 = 5.0, const1 = 0.180625, const2 = 1.6;
  static const double a[8] = {3.3871328727963666080e0, 1.3314166789178437745e+2,
                              1.9715909503065514427e+3, 1.3731693765509461125e+4,
                              4.5921953931549871457e+4, 6.7265770927008700853e+4,
                              3.3430575583588128105e+4, 2.5090809287301226727e+3};
  static const double b[8] = {1.0, 4.2313330701600911252e+1, 6.8718700749205790830e+2,
                              5.3941960214247511077e+3, 2.1213794301586595867e+4,
                              3.9307895800092710610e+4, 2.8729085735721942674e+4,
                              5.2264952788528545610e+3};
  static const double c[8] = {1.42343711074968357734e0, 4.63033784615654529590e0,
                              5.76949722146069140550e0, 3.64784832476320460504e0,
                              1.27045825245236838258e0, 2.41780725177450611770e-1,
                              2.27238449892691845833e-2, 7.74545014278341407640e-4};
  static const double d[8] = {1.0, 2.05319162663775882187e0, 1.67638483018380384940e0,
                              6.89767334985100004550e-1, 1.48103976427480074590e-1,
                              1.51986665636164571966e-2, 5.47593808499534494600e-4,
                              1.05075007164441684324e-9};
  static const double e[8] = {6.65790464350110377720e0, 5.46378491116411436990e0,
                              1.78482653991729133580e0, 2.96560571828504891230e-1,
                              2.65321895265761230930e-2, 1.24266094738807843860e-3,
                              2.71155556874348757815e-5, 2.01033439929228813265e-7};
  static const double f[8] = {1.0, 5.99832206555887937690e-1, 1.36929880922735805310e-1,
                              1.48753612908506148525e-2, 7.86869131145613259100e-4,
                              1.84631831751005468180e-5, 1.42151175831644588870e-7,
                              2.04426310338993978564e-15};
  auto horner = [](const double* k, double r) {
    double acc = k[7];
    for (int i = 6; i >= 0; --i) acc = acc * r + k[i];
    return acc;
  };
  if (!(p > 0.0 && p < 1.0)) {
    if (p == 0.0) return -INFINITY;
    if (p == 1.0) return INFINITY;
    return NAN;
  }
  double q = p - 0.5;
  if (std::fabs(q) <= split1) {
    double r = const1 - q * q;
    return q * horner(a, r) / horner(b, r);
  }
  double r = q < 0.0 ? p : 1.0 - p;
  r = std::sqrt(-std::log(r));
  double val;
  if (r <= split2) {
    r -= const2;
    val = horner(c, r) / horner(d, r);
  } else {
    r -= split2;
    val = horner(e, r) / horner(f, r);
  }
  return q < 0.0 ? -val : val;
}

}  // namespace

extern "C" {

int pg_version(void) { return 1; }

// Raw Philox4x32-10 block (exposed for known-answer tests).
void pg_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  P4 c{{ctr[0], ctr[1], ctr[2], ctr[3]}};
  P4 r = philox4x32_10(c, key[0], key[1]);
  std::memcpy(out, r.v, sizeof(r.v));
}

double pg_ndtri(double p) { return ppnd16(p); }

void pg_ndtri_vec(const double* p, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = ppnd16(p[i]);
}

void pg_f64_to_f16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16_bits(x[i]);
}

// mean over k = 1..f of clamp(C * k^-s, lo, hi)
static double zipf_mean(double C, int64_t f, double s, double lo, double hi) {
  double acc = 0.0;
  for (int64_t k = 1; k <= f; ++k) acc += std::min(hi, std::max(lo, C * std::pow((double)k, -s)));
  return acc / (double)f;
}

// Bisection for the Zipf constant C with mean(p) = target.
double pg_zipf_constant(int64_t f, double s, double lo, double hi, double target) {
  double a = 0.0, b = hi * std::pow((double)f, s) * 2.0;
  for (int it = 0; it < 200; ++it) {
    double m = 0.5 * (a + b);
    if (zipf_mean(m, f, s, lo, hi) < target) a = m; else b = m;
    if (b - a <= 1e-15 * b) break;
  }
  return 0.5 * (a + b);
}

// Seeded random rank order: rank[i] in 1..f for original neuron i.
void pg_zipf_ranks(uint32_t seed, uint32_t tag, uint32_t layer, int64_t f, int32_t* rank_out) {
  std::vector<std::pair<uint64_t, int32_t>> keys((size_t)f);
  for (int64_t i = 0; i < f; ++i) {
    P4 c{{(uint32_t)i, 0u, layer, 0u}};
    P4 r = philox4x32_10(c, seed, tag);
    keys[(size_t)i] = {((uint64_t)r.v[0] << 32) | r.v[1], (int32_t)i};
  }
  std::sort(keys.begin(), keys.end());
  for (int64_t pos = 0; pos < f; ++pos) rank_out[keys[(size_t)pos].second] = (int32_t)(pos + 1);
}

// Firing probabilities p[i] for original neuron i, and the constant C used.
double pg_zipf_probs(uint32_t seed, uint32_t tag, uint32_t layer, int64_t f, double s, double lo,
                     double hi, double target, double* p_out) {
  std::vector<int32_t> rank((size_t)f);
  pg_zipf_ranks(seed, tag, layer, f, rank.data());
  double C = pg_zipf_constant(f, s, lo, hi, target);
  for (int64_t i = 0; i < f; ++i)
    p_out[i] = std::min(hi, std::max(lo, C * std::pow((double)rank[(size_t)i], -s)));
  return C;
}

// Hot-first storage order: perm[slot] = original id, p descending, ties by id ascending.
void pg_hot_first_perm(const double* p, int64_t f, int32_t* perm) {
  std::vector<int32_t> ids((size_t)f);
  std::iota(ids.begin(), ids.end(), 0);
  std::stable_sort(ids.begin(), ids.end(), [p](int32_t a, int32_t b) { return p[a] > p[b]; });
  std::memcpy(perm, ids.data(), sizeof(int32_t) * (size_t)f);
}

// Gaussian rows N(0, stddev^2), rounded to the storage type.
//   dtype 0: float32, dtype 1: binary16 bits, dtype 2: float64.
// Output row j holds the row keyed by row_ids[j] (or j if row_ids is NULL).
void pg_gaussian_rows(uint32_t seed, uint32_t tag, uint32_t layer, const int32_t* row_ids,
                      int64_t nrows, int64_t ncols, double stddev, int dtype, void* out,
                      int nthreads) {
  parallel_rows(nrows, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t j = r0; j < r1; ++j) {
      uint32_t rid = row_ids ? (uint32_t)row_ids[j] : (uint32_t)j;
      for (int64_t blk = 0; 2 * blk < ncols; ++blk) {
        P4 c{{(uint32_t)blk, rid, layer, 0u}};
        P4 r = philox4x32_10(c, seed, tag);
        double z[2];
        box_muller(r, &z[0], &z[1]);
        for (int h = 0; h < 2; ++h) {
          int64_t col = 2 * blk + h;
          if (col >= ncols) break;
          double v = z[h] * stddev;
          int64_t o = j * ncols + col;
          if (dtype == 0) ((float*)out)[o] = (float)v;
          else if (dtype == 1) ((uint16_t*)out)[o] = f64_to_f16_bits(v);
          else ((double*)out)[o] = v;
        }
      }
    }
  });
}

// Uniform random bytes per row (Q4_0 nibble storage: every nibble uniform on 0..15).
void pg_random_bytes_rows(uint32_t seed, uint32_t tag, uint32_t layer, const int32_t* row_ids,
                          int64_t nrows, int64_t nbytes, uint8_t* out, int nthreads) {
  parallel_rows(nrows, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t j = r0; j < r1; ++j) {
      uint32_t rid = row_ids ? (uint32_t)row_ids[j] : (uint32_t)j;
      for (int64_t blk = 0; 16 * blk < nbytes; ++blk) {
        P4 c{{(uint32_t)blk, rid, layer, 1u}};
        P4 r = philox4x32_10(c, seed, tag);
        uint8_t bytes[16];
        std::memcpy(bytes, r.v, 16);
        int64_t n = std::min<int64_t>(16, nbytes - 16 * blk);
        std::memcpy(out + j * nbytes + 16 * blk, bytes, (size_t)n);
      }
    }
  });
}

// Q4_0 block scales: binary16(mult * |N(0, stddev^2)|), one per 32 weights.
void pg_q4_scales_rows(uint32_t seed, uint32_t tag, uint32_t layer, const int32_t* row_ids,
                       int64_t nrows, int64_t nblocks, double stddev, double mult, uint16_t* out,
                       int nthreads) {
  parallel_rows(nrows, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t j = r0; j < r1; ++j) {
      uint32_t rid = row_ids ? (uint32_t)row_ids[j] : (uint32_t)j;
      for (int64_t blk = 0; 2 * blk < nblocks; ++blk) {
        P4 c{{(uint32_t)blk, rid, layer, 2u}};
        P4 r = philox4x32_10(c, seed, tag);
        double z[2];
        box_muller(r, &z[0], &z[1]);
        for (int h = 0; h < 2; ++h) {
          int64_t b = 2 * blk + h;
          if (b >= nblocks) break;
          out[j * nblocks + b] = f64_to_f16_bits(mult * std::fabs(z[h] * stddev));
        }
      }
    }
  });
}

// Euclidean norms (double) of stored rows, used only to place the bias:
//   dtype 0 float32 rows, 1 binary16 rows, 3 Q4_0 rows (nibbles [rows][ncols/2],
//   scales [rows][ncols/32]; a block's squared norm is scale^2 * sum (q-8)^2).
void pg_row_norms(const void* rows, const uint16_t* scales, int64_t nrows, int64_t ncols, int dtype,
                  double* out, int nthreads) {
  parallel_rows(nrows, nthreads, [&](int64_t r0, int64_t r1) {
    for (int64_t j = r0; j < r1; ++j) {
      double acc = 0.0;
      if (dtype == 0) {
        const float* w = (const float*)rows + j * ncols;
        for (int64_t k = 0; k < ncols; ++k) acc += (double)w[k] * (double)w[k];
      } else if (dtype == 1) {
        const uint16_t* w = (const uint16_t*)rows + j * ncols;
        for (int64_t k = 0; k < ncols; ++k) {
          double v = f16_bits_to_f64(w[k]);
          acc += v * v;
        }
      } else {
        const uint8_t* nib = (const uint8_t*)rows + j * (ncols / 2);
        const uint16_t* sc = scales + j * (ncols / 32);
        for (int64_t b = 0; b < ncols / 32; ++b) {
          int64_t sq = 0;
          for (int k = 0; k < 16; ++k) {
            int lo = nib[16 * b + k] & 15, hi = nib[16 * b + k] >> 4;
            sq += (int64_t)(lo - 8) * (lo - 8) + (int64_t)(hi - 8) * (hi - 8);
          }
          double s = f16_bits_to_f64(sc[b]);
          acc += s * s * (double)sq;
        }
      }
      out[j] = std::sqrt(acc);
    }
  });
}

}  // extern "C"
