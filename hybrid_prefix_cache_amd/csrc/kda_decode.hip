// kda_decode.hip -- single-token KDA state update, one workgroup per
// (request, head), gfx950.
//
// Method: page "Kimi K3 -- Lesson 01 - Architecture map" (gentlecold.top),
// section "两种 Attention，两种状态": decode keeps only the state S at the
// current position and applies one token: decay the rows of S by
// alpha = exp(g), delta-rule write with beta, k, v, then read o = S^T q.
// Page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
// section 2.1: the step reads the fixed-size state, not the history, so it is
// a pure stream over the state: 64 KiB in and 64 KiB out per (request, head)
// at d = 128.
//
// Layout: the state of (page, head) is fp32 [d_k][d_v] row-major.  Thread t
// holds VPT rows x 4 columns: column quad cq = t % (D/4), row group
// rg = t / (D/4), rows rg + i * (D / VPT).  One wave instruction therefore
// moves whole consecutive 512-byte rows (d = 128), and each thread keeps only
// a few vectors between its loads and its stores, so the loads and stores of
// many waves interleave finely; state accesses are non-temporal.  Measured on
// the 256 x 32 x d=128 step, this shape (1024 threads, 4 rows per thread,
// registers capped so two workgroups share a CU) streams ~15% faster than one
// holding 16 rows per thread with ordinary loads.  The two column sums over
// rows (S'^T k and S^T q) use lane shuffles inside a wave, then one LDS
// exchange across the waves.
//
// The same kernel applies K tokens per request in one launch (speculative
// verification, page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제", sections
// 6.4/6.5: a target-verify path keeps every intermediate state, indexed per
// token, so that rejected draft tokens roll back): the state stays in registers from token to token
// and the state after token t is written to page_out[r*K + t]; a plain
// decode step is K = 1.  The reduction scratch alternates between two buffers
// by token parity, so consecutive tokens need no extra barrier.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int D> struct DecodeShape {
  static constexpr int VPT = D == 128 ? 4 : 2;  // rows per thread
  static constexpr int NQ = D / 4;              // column quads per row
  static constexpr int NT = D / VPT * NQ;       // threads: 1024 at d = 128, 512 at d = 64
  static constexpr int NW = NT / 64;            // waves
  static constexpr int RS = D / VPT;            // row stride between a thread's rows
};

__device__ __forceinline__ float in_f(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float in_f(float x) { return x; }

// Inputs of one token that a thread reads (its rows' g, k, q; the v column
// quad of the threads that form u; beta), raw.
template <int D, typename In> struct TokIn {
  In g[DecodeShape<D>::VPT], k[DecodeShape<D>::VPT], q[DecodeShape<D>::VPT];
  In v[4];
  In beta;
};

// MULTI (K > 1, speculative verification): the inputs of token t+1 are loaded
// while token t is applied.  That needs more than the 64 registers that let
// two 1024-thread workgroups share a CU, so a single-token step (MULTI false)
// keeps its loads where they are used and the 64-register shape.
template <int D, typename In, bool MULTI>
__global__ __launch_bounds__(DecodeShape<D>::NT, MULTI ? 4 : 8) void decode_kernel(DecodeArgs a) {
  using SH = DecodeShape<D>;
  constexpr int VPT = SH::VPT, NQ = SH::NQ, NW = SH::NW, RS = SH::RS;
  __shared__ f32x4 red[2][NW][NQ];
  __shared__ f32x4 sh_u[2][NQ];

  const int r = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cq = tid % NQ, rg = tid / NQ, c0 = 4 * cq;
  const int K = a.K;
  const int pin = a.page_in[r];
  bool ok = pin >= 0 && pin < a.num_pages;
  for (int t = 0; t < K; ++t) {
    const int po = a.page_out[r * K + t];
    ok = ok && po >= 0 && po < a.num_pages;
  }
  if (!ok) {  // a bad page index: touch no state, make this request's outputs loudly wrong
    for (int t = 0; t < K; ++t) {
      if (tid < D) {
        const int64_t oi = ((int64_t)(r * K + t) * a.H + h) * D + tid;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = 0x7fc0u;
        else reinterpret_cast<float*>(a.o)[oi] = __builtin_nanf("");
      }
    }
    return;
  }
  const int64_t hoff = (int64_t)h * D * D;
  const float* src = reinterpret_cast<const float*>(a.pool + pin * a.page_bytes) + hoff;
  f32x4 s[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (rg + i * RS) * D + c0));
  // sum over the row groups inside a wave: lanes that differ above the column-quad bits
  auto wave_sum = [&](f32x4 x) {
#pragma unroll
    for (int m = NQ; m < 64; m <<= 1) {
      x.x += __shfl_xor(x.x, m); x.y += __shfl_xor(x.y, m);
      x.z += __shfl_xor(x.z, m); x.w += __shfl_xor(x.w, m);
    }
    return x;
  };
  auto load_tok = [&](int t, TokIn<D, In>& x) {
    const int64_t row = (int64_t)(r * K + t) * a.H + h;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t c = row * D + rg + i * RS;
      x.g[i] = reinterpret_cast<const In*>(a.g)[c];
      x.k[i] = reinterpret_cast<const In*>(a.k)[c];
      x.q[i] = reinterpret_cast<const In*>(a.q)[c];
    }
    if (tid < NQ) {
#pragma unroll
      for (int j = 0; j < 4; ++j) x.v[j] = reinterpret_cast<const In*>(a.v)[row * D + 4 * tid + j];
    }
    x.beta = reinterpret_cast<const In*>(a.beta)[row];
  };
  TokIn<D, In> cur, nxt;  // MULTI: this token's inputs and the next token's
  if constexpr (MULTI) load_tok(0, cur);
  for (int t = 0; t < K; ++t) {
    const int par = t & 1;
    const int64_t row = (int64_t)(r * K + t) * a.H + h;  // (token, head) input row
    const In* gq = reinterpret_cast<const In*>(a.q) + row * D;
    const In* gk = reinterpret_cast<const In*>(a.k) + row * D;
    const In* gv = reinterpret_cast<const In*>(a.v) + row * D;
    const In* gg = reinterpret_cast<const In*>(a.g) + row * D;
    if constexpr (MULTI) {
      if (t + 1 < K) load_tok(t + 1, nxt);
    }
    float kr[VPT], qr[VPT];
    f32x4 p = zero4();
#pragma unroll
    for (int i = 0; i < VPT; ++i) {  // S' = diag(alpha) S ; partial S'^T k over this thread's rows
      const int c = rg + i * RS;
      float ac;
      if constexpr (MULTI) {
        ac = __expf(in_f(cur.g[i]));
        kr[i] = in_f(cur.k[i]);
        qr[i] = in_f(cur.q[i]);
      } else {
        ac = __expf(in_f(gg[c]));
        kr[i] = in_f(gk[c]);
        qr[i] = in_f(gq[c]);
      }
      s[i] *= ac;
      p += s[i] * kr[i];
    }
    p = wave_sum(p);
    if (lane < NQ) red[par][wv][cq] = p;
    __syncthreads();
    if (tid < NQ) {
      f32x4 acc = red[par][0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) acc += red[par][w][tid];
      const int c = 4 * tid;
      if constexpr (MULTI) {
        const TokIn<D, In>& x = cur;
        sh_u[par][tid] = f32x4{in_f(x.v[0]) - acc.x, in_f(x.v[1]) - acc.y, in_f(x.v[2]) - acc.z,
                               in_f(x.v[3]) - acc.w};  // u = v - S'^T k
      } else {
        sh_u[par][tid] = f32x4{in_f(gv[c]) - acc.x, in_f(gv[c + 1]) - acc.y, in_f(gv[c + 2]) - acc.z,
                               in_f(gv[c + 3]) - acc.w};  // u = v - S'^T k
      }
    }
    __syncthreads();
    const f32x4 u = sh_u[par][cq];
    float beta;
    if constexpr (MULTI) beta = in_f(cur.beta);
    else beta = in_f(reinterpret_cast<const In*>(a.beta)[row]);
    float* dst = reinterpret_cast<float*>(a.pool + a.page_out[r * K + t] * a.page_bytes) + hoff;
    f32x4 pq = zero4();
#pragma unroll
    for (int i = 0; i < VPT; ++i) {  // S = S' + beta k u^T ; partial S^T q
      s[i] += u * (beta * kr[i]);
      __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(dst + (rg + i * RS) * D + c0));
      pq += s[i] * qr[i];
    }
    pq = wave_sum(pq);
    if (lane < NQ) red[par][wv][cq] = pq;  // this buffer's first sum was read before the last barrier
    __syncthreads();
    if (tid < NQ) {
      f32x4 acc = red[par][0][tid];
#pragma unroll
      for (int w = 1; w < NW; ++w) acc += red[par][w][tid];
      const int64_t oi = row * D + 4 * tid;
      if (a.out_bf16)
        *reinterpret_cast<u16x4*>(reinterpret_cast<uint16_t*>(a.o) + oi) = pack_bf16x4(acc.x, acc.y, acc.z, acc.w);
      else
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.o) + oi) = acc;
    }
    if constexpr (MULTI) cur = nxt;
  }
}

template <int D, typename In>
static void launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.n * (unsigned)a.H), block(DecodeShape<D>::NT);
  if (a.K > 1) hipLaunchKernelGGL((decode_kernel<D, In, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((decode_kernel<D, In, false>), grid, block, 0, st, a);
}

hipError_t launch_decode(int D, bool bf16, const DecodeArgs& a, hipStream_t st) {
  if (D == 128) {
    if (bf16) launch_decode_t<128, uint16_t>(a, st);
    else launch_decode_t<128, float>(a, st);
  } else {
    if (bf16) launch_decode_t<64, uint16_t>(a, st);
    else launch_decode_t<64, float>(a, st);
  }
  return hipGetLastError();
}

}  // namespace kda
