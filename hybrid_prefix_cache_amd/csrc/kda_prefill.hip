// kda_prefill.hip -- chunk-parallel KDA prefill for gfx950.
//
// Method: page "Kimi K3 -- Lesson 01 - Architecture map" (gentlecold.top),
// section "两种 Attention，两种状态" (the per-token recurrence; prefill runs
// chunk-parallel with the state carried between chunks), and page "KIMI K3
// 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app), section 1.3 (a
// token segment collapses to one affine map, so chunks may be processed in
// parallel as long as their order is kept).  Checkpoint stores: page "Cache
// de préfixe hybride KDA–MLA" (mkdocs.reaper.mx), sections "La solution" and
// "Le fonctionnement du prefill".
//
// Chunk form (derived from the per-token steps; C = 64 tokens, entering state
// S0, G_r = inclusive prefix sum of g inside the chunk, e_r = exp(G_r)):
//   Kt = K*e, Kh = K/e, Qt = Q*e, Kend = K*(e_C/e)
//   A  = strictLower(Kt Kh^T) ; Aq = lowerIncl(Qt Kh^T)
//   T  = (I + diag(beta) A)^-1 diag(beta)
//   Keff = T Kt
//   W = T V - Keff S0 ; O = Qt S0 + Aq W ; S_C = diag(e_C) S0 + Kend^T W
// (O = (Qt - Aq Keff) S0 + Aq T V: the query side of each token sees the
// state entering the chunk plus the chunk's own corrected values W.)
// Everything left of "W =" is independent of the state and is computed by
// `prep_kernel` for all (chunk, head) pairs at once; `scan_kernel` walks the
// chunks of one (sequence, head, 16-column slab of d_v) in order, keeping its
// slab of S in fp32 registers.  Column j of S depends only on column j of v,
// which is what allows the d_v split.  A partial final chunk is padded with
// zero rows (k = q = v = g = beta = 0), which leave the state unchanged.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ---------------------------------------------------------------------------
// metadata fill: copy a kernel-argument payload into the workspace
// ---------------------------------------------------------------------------
__global__ void meta_fill_kernel(MetaFillArgs a) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(a.dst);
  for (uint32_t i = threadIdx.x; i < a.nwords; i += blockDim.x) dst[i] = a.words[i];
}

// ---------------------------------------------------------------------------
// shared helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
  u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = bf16_to_f32(v[j]);
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float* x) {
  u16x4 v = *reinterpret_cast<const u16x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = bf16_to_f32(v[j]);
}
__device__ __forceinline__ void load4(const float* p, float* x) {
  float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* x) {
  u16x8 v;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = f32_to_bf16(x[j]);
  *reinterpret_cast<u16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = float4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<float4*>(p + 4) = float4{x[4], x[5], x[6], x[7]};
}

// Largest s with seqs[s].chunk_begin <= chunk: the sequence owning `chunk`
// (zero-length sequences share their successor's chunk_begin).
// Offsets (in Op elements) of the pieces of one (chunk, head) block.  Every
// piece is stored fragment-major (see frag_off) as the scan's MFMA operand:
// Keff, Qt, T, Aq by token rows, KendT by channel rows.
template <int D> struct InterOff {
  static constexpr int kKeff = 0;
  static constexpr int kQt = 64 * D;
  static constexpr int kKendT = 128 * D;
  static constexpr int kT = 192 * D;
  static constexpr int kAq = 192 * D + 64 * 64;
  static constexpr int kGammaElems = 192 * D + 2 * 64 * 64;  // fp32 gamma starts here
};

// ---------------------------------------------------------------------------
// prep: state-independent part of every (chunk, head)
// ---------------------------------------------------------------------------

// LDS plan of the fp32-input prep: operands are read element-wise, so no
// transposed copies; T is formed in place of the inverse.
template <int D> struct PrepLayout {
  static constexpr int LDK = D + (D == 128 ? 0 : 4);  // [64][D] tiles
  static constexpr int LDF = 65;                      // fp32 solve tiles [64][65]
  static constexpr int kTile = 64 * LDK * 4;
  static constexpr int kKt = 0;
  static constexpr int kKh = kKt + kTile;
  static constexpr int kQt = kKh + kTile;
  static constexpr int kR0 = kQt + kTile;
  static constexpr int kR0Bytes = (64 * D * 4 > 2 * 64 * LDF * 4) ? 64 * D * 4 : 2 * 64 * LDF * 4;
  static constexpr int kY = kR0 + kR0Bytes;     // fp32 [3][16][17]
  static constexpr int kBeta = kY + 3 * 16 * 17 * 4;  // fp32 [64]
  static constexpr int kEM = kBeta + 64 * 4;          // fp32 [D]: exp(G_31) per channel
  static constexpr int kBytes = kEM + D * 4;
  static_assert(kBytes <= 160 * 1024, "prep LDS budget");
};

template <int D, typename Op>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
  static_assert(sizeof(Op) == 4, "bf16 inputs are prepared by prep2_kernel");
  using LY = PrepLayout<D>;
  using OT = OpT<Op>;
  constexpr int LDK = LY::LDK, LDF = LY::LDF;
  constexpr int KK = OT::kK;
  extern __shared__ __align__(16) uint8_t smem[];
  Op* Kt = reinterpret_cast<Op*>(smem + LY::kKt);
  Op* Kh = reinterpret_cast<Op*>(smem + LY::kKh);
  Op* Qt = reinterpret_cast<Op*>(smem + LY::kQt);
  float* Gm = reinterpret_cast<float*>(smem + LY::kR0);  // [64][D] prefix sums
  float* Lm = Gm;                                         // [64][LDF] diag(beta) A
  float* Ti = Gm + 64 * LDF;                              // [64][LDF] inverse, then T (fp32)
  float* Y = reinterpret_cast<float*>(smem + LY::kY);
  float* beta_s = reinterpret_cast<float*>(smem + LY::kBeta);
  float* em_s = reinterpret_cast<float*>(smem + LY::kEM);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // chunks in reverse dispatch order (see prep2_kernel)
  const int wchunk = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, H = a.H;
  const int chunk = a.chunk0 + wchunk;
  const SeqEntry se = seq_at(a, find_seq_in(a, chunk));
  const int lc = chunk - se.chunk_begin;
  const int64_t row0 = se.row_begin + 64LL * lc;
  const int len = min(64, se.len - 64 * lc);
  const Op* gq = reinterpret_cast<const Op*>(a.q);
  const Op* gk = reinterpret_cast<const Op*>(a.k);
  const Op* gg = reinterpret_cast<const Op*>(a.g);
  const Op* gb = reinterpret_cast<const Op*>(a.beta);
  Op* out = reinterpret_cast<Op*>(a.inter + ((int64_t)wchunk * H + h) * a.blk_bytes);
  using IO = InterOff<D>;
  constexpr int CG = D / 8;

  // ---- phase 1: gates -> LDS, inclusive prefix sum over tokens -------------
  for (int it = tid; it < 64 * CG; it += 256) {
    const int r = it / CG, cg = it % CG;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r < len) load8(gg + ((row0 + r) * H + h) * D + 8 * cg, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) Gm[r * D + 8 * cg + j] = x[j];
  }
  if (tid < 64) beta_s[tid] = tid < len ? load_as_f(gb + (row0 + tid) * H + h) : 0.f;
  __syncthreads();
  {
    constexpr int PARTS = 256 / D, TPP = 64 / PARTS;
    const int c = tid % D, part = tid / D;
    float run = 0.f;
    for (int i = 0; i < TPP; ++i) {
      const int r = part * TPP + i;
      run += Gm[r * D + c];
      Gm[r * D + c] = run;
    }
    __syncthreads();
    float off = 0.f;
    for (int p = 0; p < part; ++p) off += Gm[(p * TPP + TPP - 1) * D + c];
    __syncthreads();
    if (part > 0)
      for (int i = 0; i < TPP; ++i) Gm[(part * TPP + i) * D + c] += off;
    __syncthreads();
  }

  // ---- phase 2: decayed tiles ------------------------------------------------
  // The Gram tiles (LDS) take the mid-chunk prefix G_31 as reference:
  // Kt' = K exp(G - G_31), Kh' = K exp(G_31 - G), Qt' = Q exp(G - G_31)
  // (exp(G_i - G_j) K_i K_j per channel as with any reference, each factor
  // within exp(+-(half a chunk of gates))).  The workspace pieces keep the
  // chunk-start reference, where every factor is at most 1: Qt = Q exp(G),
  // Kend = K exp(G_C - G); Keff = T Kt' diag(exp(G_31)) (phase 5).
  for (int it = tid; it < 64 * CG; it += 256) {
    const int r = it / CG, cg = it % CG, c0 = 8 * cg;
    float kx[8] = {0, 0, 0, 0, 0, 0, 0, 0}, qx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r < len) {
      load8(gk + ((row0 + r) * H + h) * D + c0, kx);
      load8(gq + ((row0 + r) * H + h) * D + c0, qx);
    }
    float kt[8], kh[8], qt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float G = Gm[r * D + c0 + j], GC = Gm[63 * D + c0 + j], GM = Gm[31 * D + c0 + j];
      const float e = __expf(G - GM), ei = __expf(GM - G), eci = __expf(GC - G);
      kt[j] = kx[j] * e;
      kh[j] = kx[j] * ei;
      qt[j] = qx[j] * e;
      out[IO::kKendT + frag_off<KK>(c0 + j, r, 64)] = OT::from_f(kx[j] * eci);
      out[IO::kQt + frag_off<KK>(r, c0 + j, D)] = OT::from_f(qx[j] * __expf(G));
    }
    store8(Kt + r * LDK + c0, kt);
    store8(Kh + r * LDK + c0, kh);
    store8(Qt + r * LDK + c0, qt);
  }
  if (tid < D) {
    float* gamma = reinterpret_cast<float*>(out + IO::kGammaElems);
    gamma[tid] = __expf(Gm[63 * D + tid]);
    em_s[tid] = __expf(Gm[31 * D + tid]);
  }
  __syncthreads();

  // ---- phase 3: Gram matrices on MFMA ----------------------------------------
  // waves 0,1 -> A (Kt Kh^T), waves 2,3 -> Aq (Qt Kh^T); each takes two block
  // rows {0,3} or {1,2} of the lower triangle (5 tiles per wave).
  {
    const int gram = wave >> 1;
    const Op* Aop = gram == 0 ? Kt : Qt;
    for (int pass = 0; pass < 2; ++pass) {
      const int mt = (wave & 1) ? (pass ? 2 : 1) : (pass ? 3 : 0);
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 acc = zero4();
        if (nt <= mt) tile_mma<Op>(acc, Aop, LDK, 16 * mt, Kh, LDK, 16 * nt, 0, D, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * mt + acc_row(lane, r), j = 16 * nt + acc_col(lane);
          if (gram == 0)
            Lm[i * LDF + j] = (j < i) ? beta_s[i] * acc[r] : 0.f;
          else
            out[IO::kAq + frag_off<KK>(i, j, 64)] = OT::from_f((j <= i) ? acc[r] : 0.f);
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 4: T = (I + L)^-1 diag(beta), blocked 16x16 forward substitution
  if (lane < 16) {  // diagonal blocks: wave w inverts block w, lane j owns column j
    const int j = lane, b0 = 16 * wave;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= Lm[(b0 + i) * LDF + b0 + m] * x[m];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ti[(b0 + i) * LDF + b0 + j] = x[i];
  }
  __syncthreads();
  // block row ar: X_ab = -N_a * sum_{c=b}^{ar-1} L_ac X_cb  (b < ar)
  for (int ar = 1; ar < 4; ++ar) {
    for (int it = tid; it < ar * 256; it += 256) {
      const int b = it >> 8, i = (it >> 4) & 15, j = it & 15;
      float acc = 0.f;
      for (int c = b; c < ar; ++c)
#pragma unroll
        for (int m = 0; m < 16; ++m)
          acc += Lm[(16 * ar + i) * LDF + 16 * c + m] * Ti[(16 * c + m) * LDF + 16 * b + j];
      Y[(b * 16 + i) * 17 + j] = acc;
    }
    __syncthreads();
    for (int it = tid; it < ar * 256; it += 256) {
      const int b = it >> 8, i = (it >> 4) & 15, j = it & 15;
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m)
        acc += Ti[(16 * ar + i) * LDF + 16 * ar + m] * Y[(b * 16 + m) * 17 + j];
      Ti[(16 * ar + i) * LDF + 16 * b + j] = -acc;
    }
    __syncthreads();
  }
  for (int it = tid; it < 64 * 64; it += 256) {
    const int i = it >> 6, j = it & 63;
    const float t = (j <= i) ? Ti[i * LDF + j] * beta_s[j] : 0.f;
    Ti[i * LDF + j] = t;
    out[IO::kT + frag_off<KK>(i, j, 64)] = OT::from_f(t);
  }
  __syncthreads();

  // ---- phase 5: Keff = T Kt (wave w: rows 16w..16w+15) ------------------------
  {
    const int mt = wave;
    const int ke = min(64, ((16 * (mt + 1) + KK - 1) / KK) * KK);  // T is lower triangular
    for (int nt = 0; nt < D / 16; ++nt) {
      f32x4 acc = zero4();
      tile_mma_kn(acc, Ti, LDF, 16 * mt, reinterpret_cast<const float*>(Kt), LDK, 16 * nt, 0, ke, lane);
      const float em = em_s[16 * nt + acc_col(lane)];  // back to the chunk-start reference
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * mt + acc_row(lane, r), j = 16 * nt + acc_col(lane);
        out[IO::kKeff + frag_off<KK>(i, j, D)] = OT::from_f(acc[r] * em);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// prep for bf16 inputs: one (chunk, head) pair per 256-thread workgroup
// ---------------------------------------------------------------------------
// The workgroup (4 waves) owns an LDS region of at most 80 KB whose parts are
// reused phase by phase:
//   RA : Kt | Kh (decayed keys)  ->  L | Tinv (fp32 solve)  ->  T (bf16)
//   RQ : Qt (decayed queries)
//   RT : prefix partials  ->  Kt^T (keys, token-contiguous)
// so two workgroups share a CU and their phases interleave on the SIMDs (two
// independent workgroups beat one workgroup holding both pairs in lockstep).
// Element-wise work maps thread -> (channel pair, run of tokens), giving
// 256-byte coalesced loads and a register prefix sum; products are formed
// transposed (M = channels) so results reach global memory as 8-byte runs.
template <int D> struct Prep2Layout {
  static constexpr int NP = D / 2;             // channel pairs
  static constexpr int TPARTS = 256 / NP;      // token runs
  static constexpr int TPP = 64 / TPARTS;      // tokens per run
  static constexpr int LDK = D + 8;            // [64][D] bf16 tiles
  static constexpr int LDC = 64 + 8;           // [*][64] bf16 tiles
  static constexpr int LDF = 68;               // fp32 [64][68] (16-byte rows)
  static constexpr int kTileK = 64 * LDK * 2;
  static constexpr int kRA = 0;
  static constexpr int kRABytes = (2 * kTileK > 2 * 64 * LDF * 4) ? 2 * kTileK : 2 * 64 * LDF * 4;
  static constexpr int kRQ = kRA + kRABytes;
  static constexpr int kRT = kRQ + kTileK;
  static constexpr int kRTBytes = (D * LDC * 2 > TPARTS * D * 4) ? D * LDC * 2 : TPARTS * D * 4;
  static constexpr int kBeta = kRT + kRTBytes;  // fp32 beta[64]
  static constexpr int kBytes = kBeta + 64 * 4;
  static_assert(kBytes <= 80 * 1024, "two workgroups must fit in one CU's LDS");
  static_assert(kRQ % 16 == 0 && kRT % 16 == 0 && kBytes % 16 == 0, "align");
  // the workspace Qt staged in the Qt' region: 64 * D / 8 units of 16 bytes,
  // 16 bytes of padding after every 16 units
  static_assert(64 * D * 2 + 64 * D * 2 / 16 <= kTileK, "Qt staging fits the Qt' region");
};

__device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }

template <int D> struct Prep2In {
  static constexpr int TPP = Prep2Layout<D>::TPP;
  // channel pair c0, c0+1 of tokens r0 .. r0+TPP-1, as loaded: rows at or past
  // `len` hold a copy of the chunk's first row and are zeroed where consumed
  // (selecting here would make the issuing thread wait for every load)
  uint32_t k[TPP], q[TPP], g[TPP];
  uint16_t beta;  // token t (threads t < 64), same convention
  int len;        // valid rows of the chunk
};

// Element `off` (32-bit, in elements) of a uniform base pointer, so that the
// access is addressed as scalar base + 32-bit vector offset.
template <typename T>
__device__ __forceinline__ T* at32(T* base, uint32_t off) {
  using B = typename std::conditional<std::is_const<T>::value, const uint8_t, uint8_t>::type;
  return reinterpret_cast<T*>(reinterpret_cast<B*>(base) + off * (uint32_t)sizeof(T));
}

// Global inputs of one (chunk, head) pair into registers: thread -> channel
// pair cp, token run tp (4-byte loads, 256-byte coalesced per token).
template <int D>
__device__ __forceinline__ void prep2_load(const PrepArgs& a, int pair, int t, Prep2In<D>& x) {
  using LY = Prep2Layout<D>;
  constexpr int NP = LY::NP, TPP = LY::TPP;
  // pair is uniform: the sequence table is read through the constant address
  // space so that the lookup stays on the scalar unit (a vector load here
  // would wait on every store still in flight; the table is not written
  // while the kernel runs)
  const int H = a.H;
  const int wchunk = __builtin_amdgcn_readfirstlane(pair / H);
  const int h = __builtin_amdgcn_readfirstlane(pair - wchunk * H);
  const int chunk = a.chunk0 + wchunk;
  const SeqEntry se = seq_at(a, find_seq_in(a, chunk));
  const int lc = chunk - se.chunk_begin;
  const int64_t row0 = se.row_begin + 64LL * lc;
  const int len = min(64, se.len - 64 * lc);
  const int c0 = 2 * (t % NP), r0 = (t / NP) * TPP;
  // uniform row base, then 32-bit per-thread offsets (the host bounds
  // 64 * H * D well below 2^31)
  const int64_t rb = (row0 * H + h) * D;
  const uint16_t* gq = reinterpret_cast<const uint16_t*>(a.q) + rb;
  const uint16_t* gk = reinterpret_cast<const uint16_t*>(a.k) + rb;
  const uint16_t* gg = reinterpret_cast<const uint16_t*>(a.g) + rb;
  const uint16_t* gb = reinterpret_cast<const uint16_t*>(a.beta) + row0 * H + h;
  const uint32_t HD = (uint32_t)(H * D);
#pragma unroll
  for (int i = 0; i < TPP; ++i) {
    const int r = r0 + i;
    const uint32_t off = (r < len ? (uint32_t)r : 0u) * HD + (uint32_t)c0;
    x.k[i] = *reinterpret_cast<const uint32_t*>(at32(gk, off));
    x.q[i] = *reinterpret_cast<const uint32_t*>(at32(gq, off));
    x.g[i] = *reinterpret_cast<const uint32_t*>(at32(gg, off));
  }
  const int tb = (t & 63) < len ? (t & 63) : 0;
  x.beta = *at32(gb, (uint32_t)(tb * H));
  x.len = len;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// low halves / high halves of two packed bf16 pairs: (a.lo, b.lo), (a.hi, b.hi)
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Persistent: the grid holds as many workgroups as fit on the device at once
// and each walks the pairs with a stride of the grid size.  The kernel is
// bound by instruction issue (one (chunk, head) pair is a few thousand vector
// instructions per wave), so every phase is written to keep that count low:
// wave-uniform control flow, 32-bit store offsets from a scalar base, results
// produced in the orientation in which they are stored (4 or 8 contiguous
// elements per lane), gates accumulated in base-2 units for v_exp_f32.
template <int D>
__global__ __launch_bounds__(256) void prep2_kernel(PrepArgs a, int total_pairs) {
  using LY = Prep2Layout<D>;
  using IO = InterOff<D>;
  constexpr int NP = LY::NP, TPP = LY::TPP, LDK = LY::LDK, LDC = LY::LDC, LDF = LY::LDF;
  constexpr float kLog2e = 1.4426950408889634f;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* base = smem;
  uint16_t* Kt = reinterpret_cast<uint16_t*>(base + LY::kRA);
  uint16_t* Kh = Kt + 64 * LDK;
  float* Lm = reinterpret_cast<float*>(base + LY::kRA);
  float* Ti = Lm + 64 * LDF;
  uint16_t* Tb = reinterpret_cast<uint16_t*>(base + LY::kRA);  // inside L's region
  uint16_t* Qt = reinterpret_cast<uint16_t*>(base + LY::kRQ);
  float* partial = reinterpret_cast<float*>(base + LY::kRT);
  uint16_t* KtT = reinterpret_cast<uint16_t*>(base + LY::kRT);
  float* beta_s = reinterpret_cast<float*>(base + LY::kBeta);

  // Pairs are taken in reverse order: the scan reads chunks first to last, so
  // the blocks written last (the earliest chunks) are the ones still resident
  // in the memory-side cache when it starts, instead of the ones evicted first.
  // The inputs of the next pair are loaded into registers once the current
  // pair's have been consumed (after the decayed tiles), so their latency
  // hides behind the Gram, inverse and product phases.
  Prep2In<D> in;
  if ((int)blockIdx.x < total_pairs) prep2_load<D>(a, total_pairs - 1 - (int)blockIdx.x, threadIdx.x, in);
  for (int it = blockIdx.x; it < total_pairs; it += gridDim.x) {
  // The thread index is made opaque per iteration so that the compiler derives
  // the many per-thread LDS and global offsets inside the loop instead of
  // hoisting them all out of it, which would keep them live in registers.
  int t_opaque = threadIdx.x;
  __asm__ volatile("" : "+v"(t_opaque));
  const int t = t_opaque;
  const int lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int cp = t % NP, tp = t / NP, c0 = 2 * cp, r0 = tp * TPP;
  const int pair = total_pairs - 1 - it;
  const int len = in.len;
  if (len < 64) {  // rows past the chunk end read as zeros (uniform, rare)
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      const bool ok = r0 + i < len;
      in.k[i] = ok ? in.k[i] : 0u;
      in.q[i] = ok ? in.q[i] : 0u;
      in.g[i] = ok ? in.g[i] : 0u;
    }
  }
  const int H = a.H;
  const int wchunk = pair / H, h = pair - (pair / H) * H;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.inter + ((int64_t)wchunk * H + h) * a.blk_bytes);
  if (it != (int)blockIdx.x) __syncthreads();  // the previous pair is done with LDS
  if (t < 64) beta_s[t] = t < len ? bf16_to_f32(in.beta) : 0.f;

  // ---- B: inclusive prefix sum of g * log2(e) over tokens --------------------
  float G0[TPP], G1[TPP];
  {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      s0 = fmaf(bf_lo(in.g[i]), kLog2e, s0);
      s1 = fmaf(bf_hi(in.g[i]), kLog2e, s1);
      G0[i] = s0;
      G1[i] = s1;
    }
    *reinterpret_cast<float2*>(partial + tp * D + c0) = float2{s0, s1};
  }
  __syncthreads();
  // gc: the chunk total; gm: the prefix through token 31 (mid-chunk reference)
  float gc0 = 0.f, gc1 = 0.f, off0 = 0.f, off1 = 0.f, gm0 = 0.f, gm1 = 0.f;
#pragma unroll
  for (int p = 0; p < LY::TPARTS; ++p) {
    const float2 v = *reinterpret_cast<const float2*>(partial + p * D + c0);
    if (p < tp) { off0 += v.x; off1 += v.y; }
    if (p < LY::TPARTS / 2) { gm0 += v.x; gm1 += v.y; }
    gc0 += v.x;
    gc1 += v.y;
  }
  __syncthreads();  // partials are overwritten by Kt^T below

  // workspace Qt of this thread's channel pair, rows r0 .. r0+TPP-1: staged
  // through LDS after the Gram products (see phase E)
  uint32_t qs[TPP];

  // ---- C: decayed tiles --------------------------------------------------------
  // The Gram tiles (LDS) are decayed relative to the mid-chunk prefix G_31:
  // Kt' = K exp(G - G_31), Kh' = K exp(G_31 - G), Qt' = Q exp(G - G_31), whose
  // products over a channel equal exp(G_i - G_j) K_i K_j as with any other
  // reference, while each factor stays within exp(+-(half a chunk of gates)).
  // The state-side pieces keep the chunk-start reference, where every factor
  // is at most 1: Kt = K exp(G) (Kt^T, for Keff), Qt = Q exp(G) (workspace),
  // Kend = K exp(G_C - G) (workspace).
  {
    const float eC0 = __builtin_amdgcn_exp2f(gc0), eC1 = __builtin_amdgcn_exp2f(gc1);
    const float eM0 = __builtin_amdgcn_exp2f(gm0), eM1 = __builtin_amdgcn_exp2f(gm1);
    const float eCM0 = __builtin_amdgcn_exp2f(gc0 - gm0), eCM1 = __builtin_amdgcn_exp2f(gc1 - gm1);
    uint32_t ktT0[TPP / 2], ktT1[TPP / 2], ke0[TPP / 2], ke1[TPP / 2];
#pragma unroll
    for (int i = 0; i < TPP; i += 2) {
      uint32_t kt2[2], ke2[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = r0 + i + u;
        const float Ga = G0[i + u] + off0 - gm0, Gb = G1[i + u] + off1 - gm1;
        const float e0 = __builtin_amdgcn_exp2f(Ga), e1 = __builtin_amdgcn_exp2f(Gb);
        const float i0 = __builtin_amdgcn_exp2f(-Ga), i1 = __builtin_amdgcn_exp2f(-Gb);
        const float k0 = bf_lo(in.k[i + u]), k1 = bf_hi(in.k[i + u]);
        const float q0 = bf_lo(in.q[i + u]), q1 = bf_hi(in.q[i + u]);
        const float kt0 = k0 * e0, kt1 = k1 * e1, kh0 = k0 * i0, kh1 = k1 * i1;
        const float qt0 = q0 * e0, qt1 = q1 * e1;
        kt2[u] = pack_bf16x2(kt0 * eM0, kt1 * eM1);
        ke2[u] = pack_bf16x2(kh0 * eCM0, kh1 * eCM1);
        *reinterpret_cast<uint32_t*>(Kt + r * LDK + c0) = pack_bf16x2(kt0, kt1);
        *reinterpret_cast<uint32_t*>(Kh + r * LDK + c0) = pack_bf16x2(kh0, kh1);
        *reinterpret_cast<uint32_t*>(Qt + r * LDK + c0) = pack_bf16x2(qt0, qt1);
        qs[i + u] = pack_bf16x2(qt0 * eM0, qt1 * eM1);
      }
      ktT0[i / 2] = lo_halves(kt2[0], kt2[1]);
      ktT1[i / 2] = hi_halves(kt2[0], kt2[1]);
      ke0[i / 2] = lo_halves(ke2[0], ke2[1]);
      ke1[i / 2] = hi_halves(ke2[0], ke2[1]);
    }
    // token-contiguous runs: Kt^T rows c0, c0+1 in LDS; Kend^T rows in global
#pragma unroll
    for (int v = 0; v < TPP / 8; ++v) {
      const u32x4_t a0 = {ktT0[4 * v], ktT0[4 * v + 1], ktT0[4 * v + 2], ktT0[4 * v + 3]};
      const u32x4_t a1 = {ktT1[4 * v], ktT1[4 * v + 1], ktT1[4 * v + 2], ktT1[4 * v + 3]};
      *reinterpret_cast<u32x4_t*>(KtT + c0 * LDC + r0 + 8 * v) = a0;
      *reinterpret_cast<u32x4_t*>(KtT + (c0 + 1) * LDC + r0 + 8 * v) = a1;
      const u32x4_t b0 = {ke0[4 * v], ke0[4 * v + 1], ke0[4 * v + 2], ke0[4 * v + 3]};
      const u32x4_t b1 = {ke1[4 * v], ke1[4 * v + 1], ke1[4 * v + 2], ke1[4 * v + 3]};
      *reinterpret_cast<u32x4_t*>(at32(out, IO::kKendT + frag_off<32>(c0, r0 + 8 * v, 64))) = b0;
      *reinterpret_cast<u32x4_t*>(at32(out, IO::kKendT + frag_off<32>(c0 + 1, r0 + 8 * v, 64))) = b1;
    }
    if (tp == 0)
      *reinterpret_cast<float2*>(at32(reinterpret_cast<float*>(out + IO::kGammaElems), c0)) = float2{eC0, eC1};
  }
  // this pair's inputs are consumed: load the next pair's into the same
  // registers (beta has been staged in LDS at the top of the iteration)
  if (it + (int)gridDim.x < total_pairs) prep2_load<D>(a, pair - (int)gridDim.x, t, in);
  __syncthreads();

  // ---- D: Gram matrices, formed transposed (M = key token j, N = token i) ---
  // so that a lane holds 4 consecutive columns j of one row i.  Waves 0,1:
  // A = Kt' Kh'^T -> L = diag(beta) strictLower(A) (fp32, LDS); waves 2,3:
  // Aq = lowerIncl(Qt' Kh'^T) (bf16, to the workspace).  Each wave takes row
  // blocks {0,3} or {1,2} (5 lower tiles; the upper tiles of Aq inside
  // fragments the scan reads are written as zeros).  Products right of the
  // diagonal are computed and discarded by selects: with strong decay they
  // may overflow, which the selects keep out of the results.
  {
    const int gram = wv >> 1;
    const uint16_t* Bop = gram == 0 ? Kt : Qt;
    constexpr int NKD = D / 32;
    f32x4 acc[2][4];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int nt = (wv & 1) ? (pass ? 2 : 1) : (pass ? 3 : 0);  // row block of i
      Frag<uint16_t> bf[NKD];
#pragma unroll
      for (int k = 0; k < NKD; ++k) bf[k] = frag<uint16_t>(Bop, LDK, 16 * nt, 32 * k, lane);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {  // column block of j
        acc[pass][mt] = zero4();
        if (mt <= nt) {
#pragma unroll
          for (int k = 0; k < NKD; ++k) mfma(acc[pass][mt], frag<uint16_t>(Kh, LDK, 16 * mt, 32 * k, lane), bf[k]);
        }
      }
    }
    __syncthreads();  // Kt/Kh are overwritten by L below; Qt' is free
    // workspace Qt -> the Qt' region, in the workspace's fragment-major order
    // with 16 bytes of padding after every 256 (so that the 16 units one
    // instruction writes, 256 bytes apart, fall in different banks)
#pragma unroll
    for (int i = 0; i < TPP; ++i) {
      const int e = frag_off<32>(r0 + i, c0, D);  // element; its 16-byte unit is e / 8
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(Qt) + 2 * e + 16 * (e >> 7)) = qs[i];
    }
    const int jq = 4 * (lane >> 4);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int nt = (wv & 1) ? (pass ? 2 : 1) : (pass ? 3 : 0);
      const int i = 16 * nt + (lane & 15);
      if (gram == 0) {
        const float bi = beta_s[i];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mt <= nt) {
            const int j0 = 16 * mt + jq;
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (j0 + r < i) ? bi * acc[pass][mt][r] : 0.f;
            *reinterpret_cast<f32x4*>(Lm + i * LDF + j0) = v;
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (nt < 2 && mt >= 2) continue;  // a zero fragment the scan never reads
          const int j0 = 16 * mt + jq;
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = (j0 + r <= i) ? acc[pass][mt][r] : 0.f;
          *reinterpret_cast<u16x4*>(at32(out, IO::kAq + frag_off<32>(i, j0, 64))) =
              pack_bf16x4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
  __syncthreads();

  // ---- E: Tinv = (I + L)^-1 by 16x16 blocks, then T = Tinv diag(beta) -------
  // 1) wave 0 inverts the four diagonal blocks at once: lane = 16*block + column
  //    runs the column's forward substitution;
  // 2) 32x32 merges on fp32 MFMA: X10 = -N1 (L10 N0), X32 = -N3 (L32 N2);
  // 3) 64x64 merge: Y = L[32:64, 0:32] Inv_A, X = -Inv_B Y, where
  //    Inv_A = [[N0, 0], [X10, N1]] and Inv_B = [[N2, 0], [X32, N3]].
  if (wv == 0) {
    const int b0 = 16 * (lane >> 4), j = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc -= Lm[(b0 + i) * LDF + b0 + m] * x[m];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ti[(b0 + i) * LDF + b0 + j] = x[i];
  } else {
    // meanwhile waves 1..3 store the staged workspace Qt: 16-byte units in
    // order, 1 KB of contiguous workspace per wave instruction
    constexpr int kUnits = 64 * D / 8;
    const uint8_t* stage = reinterpret_cast<const uint8_t*>(Qt);
#pragma unroll
    for (int k = 0; k < (kUnits + 191) / 192; ++k) {
      const int u = 192 * k + (t - 64);
      if (u < kUnits)
        *reinterpret_cast<u32x4_t*>(at32(out, IO::kQt + 8 * u)) =
            *reinterpret_cast<const u32x4_t*>(stage + 16 * u + 16 * (u >> 4));
    }
  }
  __syncthreads();
  // C tile (16x16) -> Ti block (row block rb, col block cb), optionally negated
  auto put = [&](const f32x4& v, int rb, int cb, float sgn) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Ti[(16 * rb + acc_row(lane, r)) * LDF + 16 * cb + acc_col(lane)] = sgn * v[r];
  };
  if (wv < 2) {  // level 1: wave 0 -> X10, wave 1 -> X32 (Y staged in place)
    const int a0 = wv == 0 ? 1 : 3, b0 = a0 - 1;
    f32x4 y = zero4();
    tile_mma_kn(y, Lm, LDF, 16 * a0, Ti, LDF, 16 * b0, 16 * b0, 16 * b0 + 16, lane);  // L_ab N_b
    put(y, a0, b0, 1.f);
    f32x4 xx = zero4();
    tile_mma_kn(xx, Ti, LDF, 16 * a0, Ti, LDF, 16 * b0, 16 * a0, 16 * a0 + 16, lane);  // N_a Y
    put(xx, a0, b0, -1.f);  // reads of Y finished: the MFMA inputs are in registers
  }
  __syncthreads();
  {  // level 2, Y = C Inv_A: wave w -> block (2 + (w >> 1), w & 1)
    const int ra = 2 + (wv >> 1), cb = wv & 1;
    f32x4 y = zero4();
    // Y_{ra,cb} = sum_{c = cb}^{1} L_{ra,c} Inv_A[c][cb]
    tile_mma_kn(y, Lm, LDF, 16 * ra, Ti, LDF, 16 * cb, 16 * cb, 32, lane);
    put(y, ra, cb, 1.f);
  }
  __syncthreads();
  {  // X = -Inv_B Y: X_{ra,cb} = -sum_{c = 2}^{ra} Inv_B[ra][c] Y_{c,cb}
    const int ra = 2 + (wv >> 1), cb = wv & 1;
    f32x4 xx = zero4();
    tile_mma_kn(xx, Ti, LDF, 16 * ra, Ti, LDF, 16 * cb, 32, 16 * ra + 16, lane);
    __syncthreads();  // every wave has read its Y blocks
    put(xx, ra, cb, -1.f);
  }
  __syncthreads();
  {
    // T[i][j] = Tinv[i][j] beta_j (j <= i), as bf16: thread -> row i = t / 4,
    // columns 16 (t % 4) .. + 15, written as two 32-byte runs to LDS (inside
    // L's region, which no longer holds anything live) and to the workspace
    // (fragment-major, 16-byte runs of 8 columns).
    const int rv = t >> 2, g16 = 16 * (t & 3);
    uint32_t rowp[8];
    {
      const float* src = Ti + rv * LDF + g16;
#pragma unroll
      for (int m = 0; m < 16; m += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + m);
        const f32x4 b = *reinterpret_cast<const f32x4*>(beta_s + g16 + m);
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (g16 + m + r <= rv) ? x[r] * b[r] : 0.f;
        rowp[m / 2] = pack_bf16x2(y[0], y[1]);
        rowp[m / 2 + 1] = pack_bf16x2(y[2], y[3]);
      }
    }
    static_assert(64 * LDC * 2 <= 64 * LDF * 4, "T fits inside L's region, clear of Tinv");
    uint16_t* tr = Tb + rv * LDC + g16;
    const u32x4_t r0v = {rowp[0], rowp[1], rowp[2], rowp[3]}, r1v = {rowp[4], rowp[5], rowp[6], rowp[7]};
    *reinterpret_cast<u32x4_t*>(tr) = r0v;
    *reinterpret_cast<u32x4_t*>(tr + 8) = r1v;
    // rows 0..31 are zero right of column 31: the scan never reads those two
    // fragments, so they are not written
    if (rv >= 32 || g16 < 32) {
      *reinterpret_cast<u32x4_t*>(at32(out, IO::kT + frag_off<32>(rv, g16, 64))) = r0v;
      *reinterpret_cast<u32x4_t*>(at32(out, IO::kT + frag_off<32>(rv, g16 + 8, 64))) = r1v;
    }
  }
  __syncthreads();

  // ---- F: Keff = T Kt, formed transposed (M = channels) so that each lane
  // holds 4 consecutive channels of one token, an 8-byte run of the
  // workspace copy.  T is lower triangular: tokens of row blocks 0, 1 only
  // need k < 32.
  constexpr int MTW = D / 64;  // channel tiles per wave
#pragma unroll
  for (int u = 0; u < MTW; ++u) {
    const int mt = MTW * wv + u;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int ke = nt < 2 ? 32 : 64;
      f32x4 acc = zero4();
      tile_mma<uint16_t>(acc, KtT, LDC, 16 * mt, Tb, LDC, 16 * nt, 0, ke, lane);
      const int tok = 16 * nt + acc_col(lane), ch = 16 * mt + acc_row(lane, 0);
      *reinterpret_cast<u16x4*>(at32(out, IO::kKeff + frag_off<32>(tok, ch, D))) =
          pack_bf16x4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
  }
}

// ---------------------------------------------------------------------------
// scan: the state-dependent chain, chunk after chunk
// ---------------------------------------------------------------------------

constexpr int kBV = 16;  // value columns per slab

// Workgroup id -> (pair, slab): the NS slabs of one (sequence, head) pair get
// ids congruent modulo 8, so they are dispatched to the same XCD and share its
// L2 for the pair's chunk intermediates.
template <int D, int NH> struct ScanGrid {
  static constexpr int NS = D / (kBV * NH);
  __host__ __device__ static int grid(int npairs) { return 8 * NS * ((npairs + 7) / 8); }
};

// Scan workgroup: 8 waves on one (sequence, head, slab of 16*NH value columns).
//   waves 0-3 ("W"): rows 16w..16w+15 of W = T V - Keff S          -> LDS
//   waves 4-7 ("O"): the same rows of O, formed transposed,
//                    O^T = S^T Qt^T (before W is ready) + W^T Aq^T (after),
//                    stored as 4-column runs
//   every wave that owns an S tile (rows 16w..16w+15) applies
//                    S <- diag(gamma_C) S + Kend^T W
//   (the O waves read the same W fragments for both of their products).
// Each operand fragment feeds NH MFMAs (one per 16-column half), so a wider
// slab (NH = 2) halves the L2 traffic per column at twice the work per wave.
// Operands of chunk n+PF are loaded into registers while chunk n computes.
template <int D, typename Op, int NH> struct ChunkOps {
  static constexpr int KK = OpT<Op>::kK, NKD = D / KK, NKC = 64 / KK;
  Frag<Op> fa[NKC];  // W waves: T rows; O waves: Aq rows
  Frag<Op> fb[NKD];  // W waves: Keff rows; O waves: Qt rows
  Frag<Op> fe[NKC];  // Kend^T rows of the wave's S tile
  f32x4 gam;         // gamma_C of the 4 S rows this lane holds
  // 2*NH V values of this thread, kept in the input encoding until used
  typename std::conditional<sizeof(Op) == 2,
                            typename std::conditional<NH == 1, uint32_t, u32x2_t>::type,
                            typename std::conditional<NH == 1, u32x2_t, u32x4_t>::type>::type vraw;
};

struct ScanCtx {
  const uint8_t* inter;
  int64_t blk_bytes;
  const void* v;
  int H, h, c0, wv, lane, vt, vc;
  bool is_o, owns_s;
  int64_t row_begin;
  int len, chunk_begin;
};

// The operand loads of a future chunk are split in three groups issued at
// different points of the current chunk, so the memory pipeline drains while
// the waves compute instead of stalling them all at the top of the chunk.
template <int D, typename Op>
__device__ __forceinline__ const Op* chunk_block(const ScanCtx& c, int n) {
  // chunk_begin is relative to the window's first chunk
  return reinterpret_cast<const Op*>(c.inter +
                                     ((int64_t)(c.chunk_begin + n) * c.H + c.h) * c.blk_bytes);
}

template <int D, typename Op, int NH>
__device__ __forceinline__ void load_ops_a(ChunkOps<D, Op, NH>& f, const ScanCtx& c, int n) {
  using CO = ChunkOps<D, Op, NH>;
  using IO = InterOff<D>;
  const Op* pa = chunk_block<D, Op>(c, n) + (c.is_o ? IO::kAq : IO::kT);
  // T and Aq are lower triangular: a row tile's fragments right of its
  // diagonal block are zero and are neither loaded nor multiplied
#pragma unroll
  for (int i = 0; i < CO::NKC; ++i)
    if (i * CO::KK <= 16 * (c.wv & 3) + 15) f.fa[i] = frag_fm<Op>(pa, c.wv & 3, i, 64, c.lane);
}

template <int D, typename Op, int NH>
__device__ __forceinline__ void load_ops_b(ChunkOps<D, Op, NH>& f, const ScanCtx& c, int n) {
  using CO = ChunkOps<D, Op, NH>;
  using IO = InterOff<D>;
  const Op* pb = chunk_block<D, Op>(c, n) + (c.is_o ? IO::kQt : IO::kKeff);
#pragma unroll
  for (int i = 0; i < CO::NKD; ++i) f.fb[i] = frag_fm<Op>(pb, c.wv & 3, i, D, c.lane);
}

template <int D, typename Op, int NH>
__device__ __forceinline__ void load_ops_c(ChunkOps<D, Op, NH>& f, const ScanCtx& c, int n) {
  using CO = ChunkOps<D, Op, NH>;
  using IO = InterOff<D>;
  const Op* blk = chunk_block<D, Op>(c, n);
  {  // unconditional (a wave without an S tile reads a valid row it ignores)
    const int srow = min(16 * c.wv, D - 16);
#pragma unroll
    for (int i = 0; i < CO::NKC; ++i) f.fe[i] = frag_fm<Op>(blk + IO::kKendT, srow >> 4, i, 64, c.lane);
    const float* gam = reinterpret_cast<const float*>(blk + IO::kGammaElems);
    f.gam = *reinterpret_cast<const f32x4*>(gam + srow + 4 * (c.lane >> 4));
  }
  const int len = min(64, c.len - 64 * n);
  using VR = decltype(f.vraw);
  const Op* vp = reinterpret_cast<const Op*>(c.v) +
                 ((c.row_begin + 64LL * n + min(c.vt, len - 1)) * c.H + c.h) * D + c.c0 + c.vc;
  f.vraw = *reinterpret_cast<const VR*>(vp);  // rows past the chunk end are zeroed at use
}

// Issued in the same group order as inside the chunk loop, with scheduling
// fences, so that the wait counts the compiler derives at the loop entry
// match the steady state (an interleaved prologue forces needlessly deep
// waits on the first iterations of every unrolled group).
template <int D, typename Op, int NH>
__device__ __forceinline__ void load_ops(ChunkOps<D, Op, NH>& f, const ScanCtx& c, int n) {
  load_ops_a<D, Op, NH>(f, c, n);
  __builtin_amdgcn_sched_barrier(0);
  load_ops_b<D, Op, NH>(f, c, n);
  __builtin_amdgcn_sched_barrier(0);
  load_ops_c<D, Op, NH>(f, c, n);
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, typename Op, int NH>
__global__ __launch_bounds__(512) void scan_kernel(ScanArgs a) {
  using OT = OpT<Op>;
  using CO = ChunkOps<D, Op, NH>;
  constexpr int BW = 16 * NH, NS = D / BW, KK = OT::kK;
  // chunks of operands prefetched ahead (bf16: two, 157 registers; three
  // took 194 and were no faster)
  constexpr int PF = sizeof(Op) == 2 ? 2 : 1;
  // bf16: the few LDS operand fragments of a product are read up front (fp32
  // has 8x as many fragments; they are read as the products go)
  constexpr bool kBatchLds = sizeof(Op) == 2;
  constexpr int PAD = 16 / (int)sizeof(Op);
  constexpr int LDS_ = D + PAD, LDW = 64 + PAD;
  __shared__ __align__(16) Op Sb[BW * LDS_];  // S^T slab [col][row]
  __shared__ __align__(16) Op Wb[BW * LDW];   // W^T [col][token]
  __shared__ __align__(16) Op Vb[BW * LDW];   // V^T [col][token]

  const int L = blockIdx.x;
  const int xcd = L & 7, slab = (L >> 3) % NS, blk = L / (8 * NS);
  const int p = blk * 8 + xcd;
  if (p >= a.npairs) return;
  const int H = a.H, h = p % H;
  const SeqEntry se = a.inline_meta ? a.iseq.e[a.iseq.order[p / H]] : load_seq((ConstSeqPtr)(a.seqs), a.order[p / H]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches per role
  ScanCtx c;
  c.inter = a.inter;
  c.blk_bytes = a.blk_bytes;
  c.v = a.v;
  c.H = H;
  c.h = h;
  c.c0 = slab * BW;
  c.wv = wv;
  c.lane = lane;
  c.vt = tid >> 3;            // V tile: token
  c.vc = (tid & 7) * 2 * NH;  // V tile: first of 2*NH columns
  c.is_o = wv >= 4;
  c.owns_s = 16 * wv < D;
  c.row_begin = se.row_begin;
  c.len = se.len;
  c.chunk_begin = se.chunk_begin - a.c0;
  const int rt = wv & 3;
  const int64_t hoff = (int64_t)h * D * D;
  const int nchunks = (se.len + 63) / 64;
  // the sequence's chunks inside this window: [n_lo, n_hi)
  const int n_lo = max(a.c0 - se.chunk_begin, 0);
  const int n_hi = min(a.c0 + a.nch - se.chunk_begin, nchunks);

  // this wave's S tiles: rows 16*wv + 4*(lane/16) + r, column c0 + 16*j + lane%16;
  // the entering state is the sequence's (first window) or the carried one
  f32x4 S[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) S[j] = zero4();
  const float* s_src = n_lo > 0 ? a.carry_in + hoff
                       : se.state_in >= 0 ? reinterpret_cast<const float*>(a.pool + se.state_in * a.page_bytes) + hoff
                                          : nullptr;
  if (c.owns_s && s_src) {
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[j][r] = s_src[(16 * wv + acc_row(lane, r)) * D + c.c0 + 16 * j + acc_col(lane)];
  }
  auto s_to_lds = [&]() {
    if (c.owns_s) {
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        Op* d = Sb + (16 * j + acc_col(lane)) * LDS_ + 16 * wv + acc_row(lane, 0);
        if constexpr (sizeof(Op) == 2)
          *reinterpret_cast<u16x4*>(d) = pack_bf16x4(S[j][0], S[j][1], S[j][2], S[j][3]);
        else
          *reinterpret_cast<f32x4*>(d) = S[j];
      }
    }
  };
  auto s_store_to = [&](float* dst) {
    if (c.owns_s) {
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(16 * wv + acc_row(lane, r)) * D + c.c0 + 16 * j + acc_col(lane)] = S[j][r];
    }
  };
  auto s_store = [&](int page) { s_store_to(reinterpret_cast<float*>(a.pool + page * a.page_bytes) + hoff); };

  // The chunk loop is reachable only through the operand prologue, which is
  // issued after the state loads.  The wait counts inside the loop are derived
  // from every path into it: a path on which the state loads were the latest
  // memory operations (no prologue) made the loop's first use of S wait for
  // nearly every load in flight, on every iteration (3% of the scan's time).
  if (n_hi > n_lo) {
  __builtin_amdgcn_sched_barrier(0);
  CO f0, f1, f2;
  load_ops<D, Op, NH>(f0, c, n_lo);
  if (PF >= 2) load_ops<D, Op, NH>(f1, c, min(n_lo + 1, n_hi - 1));
  s_to_lds();

  int nck = se.ckpt_begin;
  // read through the constant address space: a vector load here would wait
  // for every operand load in flight
  const ConstCkptPtr ck = (ConstCkptPtr)(a.ckpts);
  auto ck_pos = [&](int i) -> int64_t { return a.inline_meta ? a.ick.e[i].pos : ck[i].pos; };
  auto ck_page = [&](int i) -> int { return a.inline_meta ? a.ick.e[i].page : ck[i].page; };
  // checkpoints at or before the window's first token belong to earlier windows
  while (nck < se.ckpt_end && ck_pos(nck) <= se.start_pos + 64LL * n_lo) ++nck;
  int64_t next_pos = nck < se.ckpt_end ? ck_pos(nck) : -1;

  auto step = [&](CO& cur, CO& pre, int n) {
    const int nf = min(n + PF, n_hi - 1);  // chunk whose operands are prefetched (inside the window)
    load_ops_a<D, Op, NH>(pre, c, nf);
    __builtin_amdgcn_sched_barrier(0);
    const int len = min(64, se.len - 64 * n);
    {  // V tile -> Vb (transposed), rows past the chunk end as zeros
      const bool live = c.vt < len;
#pragma unroll
      for (int j = 0; j < 2 * NH; ++j) {
        Op x;
        if constexpr (sizeof(Op) == 2) {
          if constexpr (NH == 1) x = (uint16_t)(cur.vraw >> (16 * j));
          else x = (uint16_t)(cur.vraw[j >> 1] >> (16 * (j & 1)));
        } else {
          x = __uint_as_float(cur.vraw[j]);
        }
        Vb[(c.vc + j) * LDW + c.vt] = live ? x : Op(0);
      }
    }
    __syncthreads();  // Vb and Sb ready
    load_ops_b<D, Op, NH>(pre, c, nf);
    __builtin_amdgcn_sched_barrier(0);

    // Each product reads its LDS operands (V^T and the bf16 copy of S) into
    // registers before the first MFMA, and accumulates in independent halves
    // that are summed at the end: the chains are then as short as the
    // matrix-core dependency allows instead of one LDS round trip per MFMA.
    f32x4 OQ[NH];  // O waves: S^T Qt^T, completed after the barrier
    if (!c.is_o) {
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        f32x4 U = zero4(), X0 = zero4(), X1 = zero4();
        if constexpr (kBatchLds) {
          Frag<Op> vf[CO::NKC], sf[CO::NKD];
#pragma unroll
          for (int i = 0; i < CO::NKC; ++i)
            if (i * KK <= 16 * rt + 15) vf[i] = frag<Op>(Vb, LDW, 16 * j, i * KK, lane);
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i) sf[i] = frag<Op>(Sb, LDS_, 16 * j, i * KK, lane);
#pragma unroll
          for (int i = 0; i < CO::NKC; ++i)
            if (i * KK <= 16 * rt + 15) mfma(U, cur.fa[i], vf[i]);
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i) mfma(i < CO::NKD / 2 ? X0 : X1, cur.fb[i], sf[i]);
        } else {
#pragma unroll
          for (int i = 0; i < CO::NKC; ++i)
            if (i * KK <= 16 * rt + 15) mfma(U, cur.fa[i], frag<Op>(Vb, LDW, 16 * j, i * KK, lane));
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i)
            mfma(i < CO::NKD / 2 ? X0 : X1, cur.fb[i], frag<Op>(Sb, LDS_, 16 * j, i * KK, lane));
        }
        const f32x4 Wv = U - X0 - X1;
        Op* wdst = Wb + (16 * j + acc_col(lane)) * LDW + 16 * rt + acc_row(lane, 0);
        if constexpr (sizeof(Op) == 2)
          *reinterpret_cast<u16x4*>(wdst) = pack_bf16x4(Wv[0], Wv[1], Wv[2], Wv[3]);
        else
          *reinterpret_cast<f32x4*>(wdst) = Wv;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        // O^T[col = 16j + 4*(lane/16) + r][token = 16*rt + lane%16], first part
        f32x4 OB0 = zero4(), OB1 = zero4();
        if constexpr (kBatchLds) {
          Frag<Op> sf[CO::NKD];
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i) sf[i] = frag<Op>(Sb, LDS_, 16 * j, i * KK, lane);
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i) mfma(i < CO::NKD / 2 ? OB0 : OB1, sf[i], cur.fb[i]);
        } else {
#pragma unroll
          for (int i = 0; i < CO::NKD; ++i)
            mfma(i < CO::NKD / 2 ? OB0 : OB1, frag<Op>(Sb, LDS_, 16 * j, i * KK, lane), cur.fb[i]);
        }
        OQ[j] = OB0 + OB1;
      }
    }
    __syncthreads();  // Wb ready; every wave is done reading Sb and Vb
    load_ops_c<D, Op, NH>(pre, c, nf);
    __builtin_amdgcn_sched_barrier(0);

    // S <- diag(gamma_C) S + Kend^T W on the waves that own an S tile;
    // O^T += W^T Aq^T on the O waves, then the O store
    const int tok = 16 * rt + acc_col(lane);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if (!c.owns_s && !c.is_o) continue;
      // bf16: the W fragments are read once for both products; fp32 (8x as
      // many fragments) reads them as the products go
      Frag<Op> wf[kBatchLds ? CO::NKC : 1];
      auto wfrag = [&](int i) { return kBatchLds ? wf[i] : frag<Op>(Wb, LDW, 16 * j, i * KK, lane); };
      if constexpr (kBatchLds) {
#pragma unroll
        for (int i = 0; i < CO::NKC; ++i) wf[i] = frag<Op>(Wb, LDW, 16 * j, i * KK, lane);
      }
      if (c.owns_s) {
        S[j] *= cur.gam;
#pragma unroll
        for (int i = 0; i < CO::NKC; ++i) mfma(S[j], cur.fe[i], wfrag(i));
      }
      if (c.is_o) {
        f32x4 OA = zero4();
#pragma unroll
        for (int i = 0; i < CO::NKC; ++i)
          if (i * KK <= 16 * rt + 15) mfma(OA, wfrag(i), cur.fa[i]);
        const f32x4 OT4 = OA + OQ[j];
        if (tok < len) {
          const int64_t base =
              ((c.row_begin + 64LL * n + tok) * H + h) * D + c.c0 + 16 * j + acc_row(lane, 0);
          if (a.out_bf16)
            *reinterpret_cast<u16x4*>(reinterpret_cast<uint16_t*>(a.o) + base) =
                pack_bf16x4(OT4[0], OT4[1], OT4[2], OT4[3]);
          else
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + base) = OT4;
        }
      }
    }
    if (se.start_pos + 64LL * n + len == next_pos) {
      s_store(ck_page(nck));
      ++nck;
      next_pos = nck < se.ckpt_end ? ck_pos(nck) : -1;
    }
    s_to_lds();
  };

  int n = n_lo;
  if constexpr (PF == 2) {
    for (; n + 3 <= n_hi; n += 3) {
      step(f0, f2, n);
      step(f1, f0, n + 1);
      step(f2, f1, n + 2);
    }
    if (n < n_hi) step(f0, f2, n);
    if (n + 1 < n_hi) step(f1, f0, n + 1);
  } else {
    for (; n + 2 <= n_hi; n += 2) {
      step(f0, f1, n);
      step(f1, f0, n + 1);
    }
    if (n < n_hi) step(f0, f1, n);
  }
  (void)f2;
  }
  if (n_hi < nchunks) s_store_to(a.carry_out + hoff);  // continues in the next window
  else if (se.state_out >= 0) s_store(se.state_out);
}

// ---------------------------------------------------------------------------
// host-side launch wrappers (called from kda_api.cpp)
// ---------------------------------------------------------------------------
hipError_t launch_meta_fill(const MetaFillArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(meta_fill_kernel, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, typename Op>
static hipError_t launch_prep_t(const PrepArgs& a, int total_chunks, hipStream_t st) {
  using LY = PrepLayout<D>;
  // Opt in to more than 64 KiB of dynamic LDS (best effort; the launch reports
  // any real failure).
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&prep_kernel<D, Op>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, LY::kBytes);
  hipLaunchKernelGGL((prep_kernel<D, Op>), dim3(total_chunks, a.H), dim3(256), LY::kBytes, st, a);
  return hipGetLastError();
}

template <int D, typename Op, int NH>
static hipError_t launch_scan_t(const ScanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((scan_kernel<D, Op, NH>), dim3(ScanGrid<D, NH>::grid(a.npairs)), dim3(512), 0,
                     st, a);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device; calls from
// several host threads may race to fill an entry, all with the same value).
static int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
static hipError_t launch_prep2_t(const PrepArgs& a, int total_chunks, hipStream_t st) {
  constexpr int kBytes = Prep2Layout<D>::kBytes;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&prep2_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kBytes);
  const int pairs = total_chunks * a.H;
  // two workgroups per CU fit (LDS); one grid-sized wave of them walks all pairs
  const int grid = (int)std::min<int64_t>(pairs, 2LL * device_cu_count());
  hipLaunchKernelGGL((prep2_kernel<D>), dim3(grid), dim3(256), kBytes, st, a, pairs);
  return hipGetLastError();
}

hipError_t launch_prep(int D, bool bf16, const PrepArgs& a, int total_chunks, hipStream_t st) {
  if (bf16) return D == 128 ? launch_prep2_t<128>(a, total_chunks, st) : launch_prep2_t<64>(a, total_chunks, st);
  return D == 128 ? launch_prep_t<128, float>(a, total_chunks, st) : launch_prep_t<64, float>(a, total_chunks, st);
}

// Slab width: 32 value columns when that still gives every CU a slab (fewer,
// wider slabs halve the L2 traffic per column), else 16.
int scan_slab_halves(int D, int npairs) {
  const char* env = getenv("KDA_SCAN_SLAB");
  if (env && (env[0] == '1' || env[0] == '2')) return env[0] - '0';
  return (long long)npairs * (D / 32) >= 256 ? 2 : 1;
}

hipError_t launch_scan(int D, bool bf16, const ScanArgs& a, hipStream_t st) {
  const int nh = scan_slab_halves(D, a.npairs);
  if (D == 128) {
    if (bf16) return nh == 2 ? launch_scan_t<128, uint16_t, 2>(a, st) : launch_scan_t<128, uint16_t, 1>(a, st);
    return nh == 2 ? launch_scan_t<128, float, 2>(a, st) : launch_scan_t<128, float, 1>(a, st);
  }
  if (bf16) return nh == 2 ? launch_scan_t<64, uint16_t, 2>(a, st) : launch_scan_t<64, uint16_t, 1>(a, st);
  return nh == 2 ? launch_scan_t<64, float, 2>(a, st) : launch_scan_t<64, float, 1>(a, st);
}


}  // namespace kda
