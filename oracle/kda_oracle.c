/*
 * kda_oracle.c -- fp64, token-by-token CPU oracle for the KDA gated
 * delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  The
 * product path (the HIP library) never links, loads or calls it, and it shares
 * no code, header, table or helper with that path.
 *
 * What it computes (plain definition, no chunking, no blocking):
 *
 *   Page "Kimi K3 -- Lesson 01 - Architecture map" (gentlecold.top),
 *   section "两种 Attention，两种状态": each KDA head keeps a state
 *   S in R^(d_k x d_v).  For every token the old state is first decayed by a
 *   per-channel forget gate Diag(alpha_t), then the delta rule writes
 *   (k_t, v_t) with strength beta_t, then q_t reads the *updated* state:
 *
 *       S'   = Diag(alpha_t) S_{t-1}                (rows = key channels)
 *       u_t  = v_t - S'^T k_t                       (delta-rule residual)
 *       S_t  = S' + beta_t k_t u_t^T
 *       o_t  = S_t^T q_t
 *
 *   i.e. S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   the affine per-token form S_t = M_t S_{t-1} + b_t of page "KIMI K3 경량
 *   복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app), section 1.3.
 *   The extracted formula on the first page places Diag(alpha_t) inside the
 *   bracket; the prose of the same section (decay first, then write, then
 *   read) fixes the order used here.  See the "exact write" pin in the tests,
 *   which separates the two readings.
 *
 *   Gate input: by default `gate` holds log(alpha) and alpha = exp(gate) in
 *   fp64; with gate_is_alpha != 0 it holds alpha itself (used by the exact
 *   rational brute-force pins).
 *
 *   Checkpoints: page "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx),
 *   sections "La solution" and "Le fonctionnement du prefill": the recurrent
 *   state is persisted only at some hash-block ends.  A checkpoint at absolute
 *   position P is the state after P tokens; here it is emitted right after
 *   the token at absolute position P-1 is processed.  The oracle accepts any
 *   P with start < P <= start+len (alignment is the library's policy).
 *
 * Inputs are read in their stored dtype (fp32, bf16 bits, or fp64) and
 * widened exactly to fp64; all arithmetic is fp64.
 *
 * KDA_ORACLE_MUTANT (compile-time) plants one deliberate mistake so that the
 * pin tests can show they catch it; the default build defines none.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2

static inline double ld(const void* p, int dtype, int64_t i) {
  if (dtype == OR_F64) return ((const double*)p)[i];
#if KDA_ORACLE_MUTANT == 11
  /* mistake: fp32 inputs truncated to their upper 16 bits */
  if (dtype == OR_F32) {
    uint32_t w;
    memcpy(&w, (const float*)p + i, 4);
    w &= 0xffff0000u;
    float t;
    memcpy(&t, &w, 4);
    return (double)t;
  }
#else
  if (dtype == OR_F32) return (double)((const float*)p)[i];
#endif
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
#if KDA_ORACLE_MUTANT == 9
  u ^= 0x10000u; /* mistake: lowest mantissa bit of a bf16 input flipped */
#endif
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int kda_oracle_mutant(void) { return KDA_ORACLE_MUTANT; }

/* One (sequence, head) pair: the token loop.  Compiled twice (Haswell-class
   AVX2/FMA and baseline x86-64) and picked at load time by the CPU, so the
   library runs on any x86-64 host; the arithmetic is the same plain loops
   either way (the wider clone may contract a*b+c into one FMA). */
__attribute__((target_clones("arch=haswell", "default")))
static void run_pair(int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t gate_is_alpha,
                     const void* q, const void* k, const void* v, const void* gate,
                     const void* beta, const double* s0, double* o, double* s_final,
                     const int64_t* ckpt_pos, double* ckpt_out, int32_t n_sel, int32_t s,
                     int32_t hs, int32_t h, int64_t bos, int64_t len, int64_t st, int32_t m,
                     int32_t m_end, double* S, double* u, double* a, double* kk, double* qq) {
  const int64_t SD = (int64_t)dk * dv;
  if (s0)
    memcpy(S, s0 + ((int64_t)s * n_sel + hs) * SD, sizeof(double) * SD);
  else
    memset(S, 0, sizeof(double) * SD);

  for (int64_t t = 0; t < len; ++t) {
    const int64_t row = (bos + t) * H + h; /* (token, head) row index */
    const double b = ld(beta, in_dtype, row);
    for (int32_t c = 0; c < dk; ++c) {
      const double gv = ld(gate, in_dtype, row * dk + c);
      a[c] = gate_is_alpha ? gv : exp(gv);
      kk[c] = ld(k, in_dtype, row * dk + c);
      qq[c] = ld(q, in_dtype, row * dk + c);
    }
    for (int32_t j = 0; j < dv; ++j) u[j] = ld(v, in_dtype, row * dv + j);

#if KDA_ORACLE_MUTANT == 2
    /* mistake: read before this token's update */
    if (o) {
      double* orow = o + ((bos + t) * n_sel + hs) * dv;
      for (int32_t j = 0; j < dv; ++j) orow[j] = 0.0;
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) orow[j] += S[c * dv + j] * qq[c];
    }
#endif

#if KDA_ORACLE_MUTANT == 5
    /* mistake: literal bracket reading, decay only inside the erase term:
       S <- S - beta k (k^T Diag(a) S) + beta k v^T */
    for (int32_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int32_t c = 0; c < dk; ++c) acc += kk[c] * a[c] * S[c * dv + j];
      u[j] -= acc;
    }
#else
    /* S' = Diag(alpha) S: scale row c (key channel c) by alpha_c */
#if KDA_ORACLE_MUTANT == 1 || KDA_ORACLE_MUTANT == 8
    /* mistake: decay dropped here (mutant 8 applies it after the write) */
#else
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];
#endif
    /* u = v - S'^T k */
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j)
#if KDA_ORACLE_MUTANT == 3
        u[j] += S[c * dv + j] * kk[c]; /* mistake: sign of the residual */
#else
        u[j] -= S[c * dv + j] * kk[c];
#endif
#endif
    /* S = S' + beta k u^T */
    for (int32_t c = 0; c < dk; ++c) {
#if KDA_ORACLE_MUTANT == 7
      const double bk = kk[c]; /* mistake: beta dropped from the write */
#else
      const double bk = b * kk[c];
#endif
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] += bk * u[j];
    }
#if KDA_ORACLE_MUTANT == 8
    /* mistake: decay applied after the delta-rule write */
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];
#endif
    /* o = S^T q (read after write) */
#if KDA_ORACLE_MUTANT != 2
    if (o) {
      double* orow = o + ((bos + t) * n_sel + hs) * dv;
      for (int32_t j = 0; j < dv; ++j) orow[j] = 0.0;
#if KDA_ORACLE_MUTANT == 4
      /* mistake: the state is read with the key instead of the query */
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) orow[j] += S[c * dv + j] * kk[c];
#else
      for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j) orow[j] += S[c * dv + j] * qq[c];
#endif
    }
#endif
    /* checkpoint: state after P tokens */
#if KDA_ORACLE_MUTANT == 6
    const int64_t p_now = st + t + 2; /* mistake: off by one token */
#else
    const int64_t p_now = st + t + 1;
#endif
    if (m < m_end && ckpt_pos[m] == p_now) {
      memcpy(ckpt_out + ((int64_t)m * n_sel + hs) * SD, S, sizeof(double) * SD);
      ++m;
    }
  }
  if (s_final) memcpy(s_final + ((int64_t)s * n_sel + hs) * SD, S, sizeof(double) * SD);
}

/*
 * Layouts (T = cu_seqlens[num_seqs]):
 *   q, k, gate : [T][H][dk]     v : [T][H][dv]     beta : [T][H]
 *   s0         : [num_seqs][n_sel][dk][dv] fp64, or NULL for S_0 = 0
 *   o          : [T][n_sel][dv] fp64, or NULL
 *   s_final    : [num_seqs][n_sel][dk][dv] fp64, or NULL
 *   ckpt_cu    : [num_seqs+1] CSR offsets into ckpt_pos (NULL => none)
 *   ckpt_pos   : absolute positions, strictly increasing per sequence
 *   ckpt_out   : [ckpt_cu[num_seqs]][n_sel][dk][dv] fp64
 *   heads      : [n_sel] head indices to run, or NULL for all H heads
 *   start_pos  : [num_seqs] absolute position of each sequence's first token
 *                (NULL => 0); only used to match checkpoint positions.
 * Returns 0, or a nonzero code for malformed arguments.
 */
int kda_oracle_run(int32_t H, int32_t dk, int32_t dv, int32_t num_seqs, const int64_t* cu_seqlens,
                   const int64_t* start_pos, int32_t in_dtype, int32_t gate_is_alpha, const void* q,
                   const void* k, const void* v, const void* gate, const void* beta, const double* s0,
                   double* o, double* s_final, const int32_t* ckpt_cu, const int64_t* ckpt_pos,
                   double* ckpt_out, const int32_t* heads, int32_t n_sel, int32_t num_threads) {
  if (H <= 0 || dk <= 0 || dv <= 0 || num_seqs < 0 || !cu_seqlens) return 1;
  if (!q || !k || !v || !gate || !beta) return 1;
  if (heads == NULL) n_sel = H;
  if (n_sel <= 0) return 1;
  for (int32_t i = 0; i < n_sel && heads; ++i)
    if (heads[i] < 0 || heads[i] >= H) return 2;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return 3;
    if (!ckpt_cu) continue;
    int64_t st = start_pos ? start_pos[s] : 0;
    int64_t len = cu_seqlens[s + 1] - cu_seqlens[s];
    for (int32_t m = ckpt_cu[s]; m < ckpt_cu[s + 1]; ++m) {
      if (ckpt_pos[m] <= st || ckpt_pos[m] > st + len) return 4;
      if (m > ckpt_cu[s] && ckpt_pos[m] <= ckpt_pos[m - 1]) return 4;
    }
    if (ckpt_out == NULL && ckpt_cu[s + 1] > ckpt_cu[s]) return 1;
  }
  if (num_threads <= 0) num_threads = omp_get_max_threads();
  const int64_t SD = (int64_t)dk * dv;
  const int64_t pairs = (int64_t)num_seqs * n_sel;

#pragma omp parallel num_threads(num_threads)
  {
    double* S = (double*)malloc(sizeof(double) * SD);
    double* u = (double*)malloc(sizeof(double) * dv);
    double* a = (double*)malloc(sizeof(double) * dk);
    double* kk = (double*)malloc(sizeof(double) * dk);
    double* qq = (double*)malloc(sizeof(double) * dk);
#pragma omp for schedule(dynamic, 1)
    for (int64_t pr = 0; pr < pairs; ++pr) {
      const int32_t s = (int32_t)(pr / n_sel);
      const int32_t hs = (int32_t)(pr % n_sel);
#if KDA_ORACLE_MUTANT == 10
      const int32_t h = heads ? heads[0] : hs; /* mistake: first selected head for all */
#else
      const int32_t h = heads ? heads[hs] : hs;
#endif
      const int64_t bos = cu_seqlens[s], len = cu_seqlens[s + 1] - bos;
      const int64_t st = start_pos ? start_pos[s] : 0;
      const int32_t m = ckpt_cu ? ckpt_cu[s] : 0;
      const int32_t m_end = ckpt_cu ? ckpt_cu[s + 1] : 0;

      run_pair(H, dk, dv, in_dtype, gate_is_alpha, q, k, v, gate, beta, s0, o, s_final, ckpt_pos,
               ckpt_out, n_sel, s, hs, h, bos, len, st, m, m_end, S, u, a, kk, qq);
    }
    free(S);
    free(u);
    free(a);
    free(kk);
    free(qq);
  }
  return 0;
}
