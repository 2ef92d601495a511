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
// Layout: the state of (page, head) is fp32 [d_k][d_v] row-major.  A workgroup
// of 256 threads holds the whole state in registers: thread t owns four value
// columns (one 16-byte vector per row) of D / RG rows, RG = 256 / (D / 4) row
// groups.  Each wave therefore reads/writes whole 512-byte row segments.
// Two cross-row-group reductions (S'^T k and S^T q) go through LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {


template <int D, typename In>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;        // 16-byte column groups per row
  constexpr int RG = 256 / CG;     // row groups
  constexpr int RPT = D / RG;      // rows per thread
  __shared__ float red[RG][D];
  __shared__ float sh_u[D];
  __shared__ float sh_k[D], sh_q[D], sh_a[D];

  const int r = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int64_t row = (int64_t)r * a.H + h;  // (request, head) input row
  const In* gq = reinterpret_cast<const In*>(a.q) + row * D;
  const In* gk = reinterpret_cast<const In*>(a.k) + row * D;
  const In* gv = reinterpret_cast<const In*>(a.v) + row * D;
  const In* gg = reinterpret_cast<const In*>(a.g) + row * D;
  const int pin = a.page_in[r], pout = a.page_out[r];
  const bool ok = pin >= 0 && pin < a.num_pages && pout >= 0 && pout < a.num_pages;

  if (!ok) {  // bad page index: touch no state, make the output loudly wrong
    for (int j = tid; j < D; j += 256) {
      const int64_t oi = row * D + j;
      if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = 0x7fc0u;
      else reinterpret_cast<float*>(a.o)[oi] = __builtin_nanf("");
    }
    return;
  }
  for (int c = tid; c < D; c += 256) {
    sh_k[c] = load_as_f(gk + c);
    sh_q[c] = load_as_f(gq + c);
    sh_a[c] = __expf(load_as_f(gg + c));
  }
  const float beta = load_as_f(reinterpret_cast<const In*>(a.beta) + row);
  const int64_t hoff = (int64_t)h * D * D;
  const float* src = reinterpret_cast<const float*>(a.pool + pin * a.page_bytes) + hoff;
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = *reinterpret_cast<const float4*>(src + (rg * RPT + i) * D + 4 * cg);
  __syncthreads();

  // S' = diag(a) S ; partial (S'^T k) over this thread's rows
  float4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg * RPT + i;
    const float ac = sh_a[c], kc = sh_k[c];
    s[i].x *= ac; s[i].y *= ac; s[i].z *= ac; s[i].w *= ac;
    part.x += s[i].x * kc; part.y += s[i].y * kc; part.z += s[i].z * kc; part.w += s[i].w * kc;
  }
  *reinterpret_cast<float4*>(&red[rg][4 * cg]) = part;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) acc += red[g2][tid];
    sh_u[tid] = load_as_f(gv + tid) - acc;  // u = v - S'^T k
  }
  __syncthreads();

  // S = S' + beta k u^T ; partial (S^T q)
  const float4 u = *reinterpret_cast<const float4*>(&sh_u[4 * cg]);
  float4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int c = rg * RPT + i;
    const float bk = beta * sh_k[c], qc = sh_q[c];
    s[i].x += bk * u.x; s[i].y += bk * u.y; s[i].z += bk * u.z; s[i].w += bk * u.w;
    po.x += s[i].x * qc; po.y += s[i].y * qc; po.z += s[i].z * qc; po.w += s[i].w * qc;
  }
  float* dst = reinterpret_cast<float*>(a.pool + pout * a.page_bytes) + hoff;
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    *reinterpret_cast<float4*>(dst + (rg * RPT + i) * D + 4 * cg) = s[i];
  *reinterpret_cast<float4*>(&red[rg][4 * cg]) = po;  // red reads finished before the last barrier
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) acc += red[g2][tid];
    const int64_t oi = row * D + tid;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(acc);
    else reinterpret_cast<float*>(a.o)[oi] = acc;
  }
}

hipError_t launch_decode(int D, bool bf16, const DecodeArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.n * (unsigned)a.H), block(256);
  if (D == 128) {
    if (bf16) hipLaunchKernelGGL((decode_kernel<128, uint16_t>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<128, float>), grid, block, 0, st, a);
  } else {
    if (bf16) hipLaunchKernelGGL((decode_kernel<64, uint16_t>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<64, float>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace kda
