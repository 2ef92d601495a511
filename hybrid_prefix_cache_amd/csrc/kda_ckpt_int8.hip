// kda_ckpt_int8.hip -- int8 compressed checkpoints: quantise on write,
// dequantise once on restore, gfx950.
//
// Page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
// section 5.3 (Compressed Checkpoint): a cached recurrent state may be held as
// int8 with per-channel parameters; a hit dequantises it once into a fresh
// active slot and decoding continues at full precision, so quantisation error
// is not re-applied token after token.  Section 6.6.2 (Int8CheckpointStore):
// one scale per d_k index from the max-abs over d_v, symmetric quantisation.
//
// Per head of a compressed page: int8 q[d][d] (row i = d_k index), then fp32
// scale[d]; scale_i = max_j |S_ij| / 127, q_ij = clamp(rne(S_ij / scale_i),
// -127, 127) (0 when scale_i == 0), restore S~_ij = q_ij * scale_i.  The
// quotient is the IEEE fp32 division, so the codes are a fixed function of the
// fp32 state; the kernel reaches the same codes with a reciprocal multiply and
// falls back to the division only where the two could round differently.
//
// A 256-thread workgroup covers 256 / (d/4) rows of one head per pass: each
// thread holds one 16-byte vector of a row, the row max-abs is a DPP
// reduction over the d/4 lanes of the row, and each thread writes its 4 codes
// as one 4-byte store (a row of codes is one 128-byte line at d = 128).  Both
// directions are HBM streams; state accesses are non-temporal.  The write is
// read-dominated (4 bytes in per byte out), so each quantising thread keeps
// four rows' loads in flight (measured: 147 -> 121 us for 256 pages of
// 32 heads), and its codes and scales are stored non-temporally (cold
// source pages: 118 -> 111 us).  The restore reads a compressed page that is usually cold (not
// in the memory-side cache): each restoring thread loads two rows' codes and
// scales before its first store (256 pages of 32 heads, cold: one row 133 us,
// two rows 106 us, four rows 114 us).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int D> struct QuantShape {
  static constexpr int LPR = D / 4;       // lanes per row
  static constexpr int RPW = 256 / LPR;   // rows per workgroup pass
  static constexpr int WPH = D / RPW;     // restore workgroups per head
  static constexpr int QRPT = 4;          // rows per quantising thread
  static constexpr int QWPH = WPH / QRPT; // quantise workgroups per head
  static constexpr int RRPT = 2;          // rows per restoring thread
  static constexpr int RWPH = WPH / RRPT; // restore workgroups per head
  static_assert(QWPH >= 1 && RWPH >= 1, "rows per thread");
};

__device__ __forceinline__ uint32_t code_of(float x, float scale) {
  const float r = scale > 0.f ? fminf(fmaxf(rintf(x / scale), -127.f), 127.f) : 0.f;
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

// The same code with one multiply instead of a division.  q = x * rcp(scale)
// differs from the correctly rounded quotient RN(x / scale) by less than
// 3e-5 for |x / scale| <= 127 (v_rcp_f32 is within 1 ulp, the product adds half
// an ulp, RN(x / scale) half an ulp), and round-to-nearest-even changes value
// only at half-integers; so when the fraction of q is more than 2^-14 away
// from 1/2 both quotients round to the same integer.  `amb` is set otherwise
// (about one element in 8,000, and for scale 0 or non-finite, where q is NaN);
// the caller then recomputes the row's codes with the division.
__device__ __forceinline__ uint32_t code_fast(float x, float inv, bool& amb) {
  const float q = x * inv;
  amb |= !(fabsf(__builtin_amdgcn_fractf(q) - 0.5f) > 0x1p-14f);
  const float r = __builtin_amdgcn_fmed3f(rintf(q), -127.f, 127.f);
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

// RN(m / 127) without a division: q1 = m * RN(1/127), then one correction
// step with the exact remainder fma(-q1, 127, m).  Checked equal to the IEEE
// quotient for every non-negative finite fp32 m (all 2^31 - 2^23 of them,
// denormals included) by an exhaustive host-side comparison.
__device__ __forceinline__ float div127(float m) {
  constexpr float kR = 1.0f / 127.0f;
  const float q1 = m * kR;
  const float e = __builtin_fmaf(-q1, 127.0f, m);
  return __builtin_fmaf(e, kR, q1);
}

// Maximum over the LPR lanes that hold one row (LPR = 16 or 32, aligned):
// rotations by 1, 2, 4, 8 inside each 16-lane DPP row, then one exchange with
// the other half for 32-lane rows.
template <int LPR>
__device__ __forceinline__ uint32_t row_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));  // row_ror:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  if constexpr (LPR == 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  static_assert(LPR == 16 || LPR == 32, "rows of 16 or 32 lanes");
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void quant_kernel(QuantArgs a) {
  using QS = QuantShape<D>;
  constexpr int RPT = QS::QRPT;
  const int per_pair = a.H * QS::QWPH;
  const int pair = blockIdx.x / per_pair, rem = blockIdx.x % per_pair;
  if (pair >= a.npairs) return;
  const int h = rem / QS::QWPH, row0 = (rem % QS::QWPH) * QS::RPW * RPT + threadIdx.x / QS::LPR;
  const int c = (threadIdx.x % QS::LPR) * 4;
  const float* base = reinterpret_cast<const float*>(a.pool + a.src[pair] * a.page_bytes) +
                      (int64_t)h * D * D;
  f32x4 x[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k)
    x[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + (row0 + k * QS::RPW) * D + c));
  uint8_t* qh = a.qpool + a.dst[pair] * a.qpage_bytes + (int64_t)h * int8_head_bytes(D);
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int row = row0 + k * QS::RPW;
    // max |x| over the row: on the magnitude bit patterns, whose unsigned order
    // is the order of the magnitudes (a NaN compares above everything)
    uint32_t mu = max(max(__float_as_uint(x[k].x) & 0x7fffffffu, __float_as_uint(x[k].y) & 0x7fffffffu),
                      max(__float_as_uint(x[k].z) & 0x7fffffffu, __float_as_uint(x[k].w) & 0x7fffffffu));
    const float m = __uint_as_float(row_max<QS::LPR>(mu));
    const float scale = div127(m);  // m / 127, correctly rounded
    const float inv = __builtin_amdgcn_rcpf(scale);
    bool amb = false;
    uint32_t packed = code_fast(x[k].x, inv, amb) | (code_fast(x[k].y, inv, amb) << 8) |
                      (code_fast(x[k].z, inv, amb) << 16) | (code_fast(x[k].w, inv, amb) << 24);
    if (__builtin_expect(amb, 0))
      packed = code_of(x[k].x, scale) | (code_of(x[k].y, scale) << 8) | (code_of(x[k].z, scale) << 16) |
               (code_of(x[k].w, scale) << 24);
    // non-temporal: a checkpoint is read back only at a later hit
    __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(qh + row * D + c));
    if (threadIdx.x % QS::LPR == 0)
      __builtin_nontemporal_store(scale, reinterpret_cast<float*>(qh + (int64_t)D * D + 4 * row));
  }
}

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(QuantArgs a) {
  using QS = QuantShape<D>;
  constexpr int RPT = QS::RRPT;
  const int per_pair = a.H * QS::RWPH;
  const int pair = blockIdx.x / per_pair, rem = blockIdx.x % per_pair;
  if (pair >= a.npairs) return;
  const int h = rem / QS::RWPH, row0 = (rem % QS::RWPH) * QS::RPW * RPT + threadIdx.x / QS::LPR;
  const int c = (threadIdx.x % QS::LPR) * 4;
  const uint8_t* qh = a.qpool + a.src[pair] * a.qpage_bytes + (int64_t)h * int8_head_bytes(D);
  uint32_t packed[RPT];
  float scale[RPT];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int row = row0 + k * QS::RPW;
    packed[k] = *reinterpret_cast<const uint32_t*>(qh + row * D + c);
    scale[k] = *reinterpret_cast<const float*>(qh + (int64_t)D * D + 4 * row);
  }
  float* dst = reinterpret_cast<float*>(a.pool + a.dst[pair] * a.page_bytes) + (int64_t)h * D * D + c;
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    f32x4 y;
    y.x = (float)(int8_t)(packed[k] & 0xffu) * scale[k];
    y.y = (float)(int8_t)((packed[k] >> 8) & 0xffu) * scale[k];
    y.z = (float)(int8_t)((packed[k] >> 16) & 0xffu) * scale[k];
    y.w = (float)(int8_t)(packed[k] >> 24) * scale[k];
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(dst + (row0 + k * QS::RPW) * D));
  }
}

hipError_t launch_quant(int D, const QuantArgs& a, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL(quant_kernel<128>, dim3(a.npairs * a.H * QuantShape<128>::QWPH), dim3(256), 0,
                       st, a);
  else
    hipLaunchKernelGGL(quant_kernel<64>, dim3(a.npairs * a.H * QuantShape<64>::QWPH), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

hipError_t launch_dequant(int D, const QuantArgs& a, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL(dequant_kernel<128>, dim3(a.npairs * a.H * QuantShape<128>::RWPH), dim3(256),
                       0, st, a);
  else
    hipLaunchKernelGGL(dequant_kernel<64>, dim3(a.npairs * a.H * QuantShape<64>::RWPH), dim3(256), 0,
                       st, a);
  return hipGetLastError();
}

}  // namespace kda
