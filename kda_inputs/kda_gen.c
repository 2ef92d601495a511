/*
 * Seeded synthetic input generators for the KDA recurrence tests and benches.
 *
 * This file is test infrastructure shared by the fp64 oracle side and the HIP
 * side: it produces the *inputs* both consume and contains none of the
 * method's arithmetic (no decay, no delta rule, no chunking).
 *
 * Random source: Philox4x32-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11).  Every element is a pure function of (seed, stream id, element
 * index), so results do not depend on the thread count or on which slice of a
 * tensor is generated.
 *
 * Normal deviates: Box-Muller (1958) on two 24-bit uniforms in (0,1), with
 * fp32 log/sqrt/sincos; uniforms for U(lo,hi) use 53 bits.
 * Elements 2m and 2m+1 share one Philox block: r*cos(theta), r*sin(theta).
 *
 * Rounding to the stored dtype is round-to-nearest-even, done once from fp64
 * (no double rounding through fp32 for bf16).
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define KDAGEN_F32 0
#define KDAGEN_BF16 1
#define KDAGEN_F64 2

#define KDAGEN_NORMAL 0         /* N(0, scale^2)                                  */
#define KDAGEN_UNIT_NORMAL 1    /* N(0,1) vector per (token, head), L2-normalised */
#define KDAGEN_UNIFORM 2        /* U(lo, hi)                                      */
#define KDAGEN_SIGMOID_NORMAL 3 /* 1/(1+exp(-z)), z ~ N(0,1)                      */

/* ---- Philox4x32-10 ---------------------------------------------------- */
static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void kdagen_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(M0, c0, &hi0, &lo0);
    mulhilo32(M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += W0; k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* One Philox block for (seed, stream, block index). */
static inline void block(uint64_t seed, uint32_t stream, uint64_t idx, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), stream, 0x4B444131u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  kdagen_philox4x32_10(ctr, key, out);
}

/* 53-bit uniform strictly inside (0,1). */
static inline double u53(uint32_t hi, uint32_t lo) {
  uint64_t m = (((uint64_t)hi << 32) | lo) >> 11;
  return ((double)m + 0.5) * (1.0 / 9007199254740992.0);
}

/* 24-bit uniform strictly inside (0,1), fp32. */
static inline float u24(uint32_t x) { return ((float)(x >> 8) + 0.5f) * (1.0f / 16777216.0f); }

/* Box-Muller pair from one Philox block (fp32 transcendentals). */
static inline void bm_pair(const uint32_t x[4], double* z0, double* z1) {
  float r = sqrtf(-2.0f * logf(u24(x[0])));
  float s, c;
  sincosf(6.2831853071795864769f * u24(x[2]), &s, &c);
  *z0 = (double)(r * c);
  *z1 = (double)(r * s);
}

static inline double normal_at(uint64_t seed, uint32_t stream, uint64_t e) {
  uint32_t x[4];
  double z0, z1;
  block(seed, stream, e >> 1, x);
  bm_pair(x, &z0, &z1);
  return (e & 1) ? z1 : z0;
}

static inline double uniform_at(uint64_t seed, uint32_t stream, uint64_t e) {
  uint32_t x[4];
  block(seed, stream, e >> 1, x);
  return (e & 1) ? u53(x[2], x[3]) : u53(x[0], x[1]);
}

/* ---- rounding --------------------------------------------------------- */
/* Round an fp64 value to the nearest bf16 (ties to even); returns the bits.
   Rounds the fp64 significand to 8 bits directly (no double rounding through
   fp32), then narrows exactly.  Valid for |x| in bf16's normal range and 0. */
uint16_t kdagen_bf16_rne(double x) {
  if (x != x) return 0x7FC0u;
  uint64_t b;
  memcpy(&b, &x, 8);
  const uint64_t drop = 45; /* 52 fraction bits -> 7 */
  uint64_t lsb = (b >> drop) & 1u;
  b += ((1ull << (drop - 1)) - 1u) + lsb;
  b &= ~((1ull << drop) - 1u);
  double y;
  memcpy(&y, &b, 8);
  float f = (float)y; /* exact */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static inline void store(void* out, int dtype, int64_t i, double x) {
  if (dtype == KDAGEN_BF16) {
    ((uint16_t*)out)[i] = kdagen_bf16_rne(x);
  } else if (dtype == KDAGEN_F32) {
    ((float*)out)[i] = (float)x;
  } else {
    ((double*)out)[i] = x;
  }
}

/* Both Box-Muller outputs of block m: elements 2m (cos) and 2m+1 (sin). */
static inline void normal_pair(uint64_t seed, uint32_t stream, uint64_t m, double* z0, double* z1) {
  uint32_t x[4];
  block(seed, stream, m, x);
  bm_pair(x, z0, z1);
}

/* Raw draws for elements [e0, e0+n) of a stream into buf (n <= 1024). */
static void draws(uint64_t seed, uint32_t stream, int kind, uint64_t e0, int n, double* buf) {
  uint64_t e = e0;
  int i = 0;
  if ((e & 1) && i < n) { /* odd start: second half of a pair */
    buf[i++] = (kind == KDAGEN_UNIFORM) ? uniform_at(seed, stream, e) : normal_at(seed, stream, e);
    ++e;
  }
  for (; i + 1 < n; i += 2, e += 2) {
    if (kind == KDAGEN_UNIFORM) {
      uint32_t x[4];
      block(seed, stream, e >> 1, x);
      buf[i] = u53(x[0], x[1]);
      buf[i + 1] = u53(x[2], x[3]);
    } else {
      normal_pair(seed, stream, e >> 1, &buf[i], &buf[i + 1]);
    }
  }
  if (i < n) buf[i] = (kind == KDAGEN_UNIFORM) ? uniform_at(seed, stream, e) : normal_at(seed, stream, e);
}

/*
 * Fill rows [t0, t0+nt) of a logical [T, H, D] tensor (token-major, head,
 * channel).  Element (t, h, c) has index e = (t*H + h)*D + c in stream
 * `stream`.  `out` receives nt*H*D values of `dtype`, row t0 first.
 * kind/scale/lo/hi select the distribution (see KDAGEN_* above).
 */
int kdagen_fill(uint64_t seed, uint32_t stream, int kind, double scale, double lo, double hi,
                int64_t t0, int64_t nt, int32_t H, int32_t D, int dtype, void* out, int nthreads) {
  if (nt < 0 || H <= 0 || D <= 0 || D > 1024 || !out) return 1;
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  const int64_t rows = nt * (int64_t)H;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t rr = 0; rr < rows; ++rr) {
    int64_t t = t0 + rr / H;
    int64_t h = rr % H;
    uint64_t base = (uint64_t)((t * H + h) * (int64_t)D);
    int64_t ob = rr * D;
    double buf[1024];
    draws(seed, stream, kind == KDAGEN_UNIFORM ? KDAGEN_UNIFORM : KDAGEN_NORMAL, base, D, buf);
    if (kind == KDAGEN_UNIT_NORMAL) {
      double ss = 0.0;
      for (int c = 0; c < D; ++c) ss += buf[c] * buf[c];
      double inv = 1.0 / sqrt(ss);
      for (int c = 0; c < D; ++c) store(out, dtype, ob + c, buf[c] * inv);
    } else {
      for (int c = 0; c < D; ++c) {
        double x;
        if (kind == KDAGEN_NORMAL) {
          x = scale * buf[c];
        } else if (kind == KDAGEN_UNIFORM) {
          x = lo + (hi - lo) * buf[c];
        } else {
          x = 1.0 / (1.0 + exp(-buf[c]));
        }
        store(out, dtype, ob + c, x);
      }
    }
  }
  return 0;
}

/* Raw fp64 uniforms in (0,1) for elements [first, first+n) of a stream. */
int kdagen_uniform(uint64_t seed, uint32_t stream, uint64_t first, int64_t n, double* out) {
  if (n < 0 || !out) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = uniform_at(seed, stream, first + (uint64_t)i);
  return 0;
}

/* Raw fp64 standard normals for elements [first, first+n) of a stream. */
int kdagen_normal(uint64_t seed, uint32_t stream, uint64_t first, int64_t n, double* out) {
  if (n < 0 || !out) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(seed, stream, first + (uint64_t)i);
  return 0;
}
