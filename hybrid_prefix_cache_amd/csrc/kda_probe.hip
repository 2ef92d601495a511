// kda_probe.hip -- peak probes for the roofline denominators of the benchmark
// (measurement only: built into libkda_probe.so, not part of libkda's API).
//
//   int kda_probe_mfma_bf16(float* out, int blocks, int iters, void* stream)
//       `blocks` workgroups of 256 threads; every wave runs `iters` rounds of
//       16 independent v_mfma_f32_16x16x32_bf16 (16x16x32 products, 16,384 flop
//       each): blocks * 4 * iters * 16 * 16384 flop.  out: blocks * 256 floats
//       (device), written so that the products cannot be elided.
//   int kda_probe_copy(void* dst, const void* src, int64_t bytes, void* stream)
//       dst[0, bytes) = src[0, bytes): one 16-byte non-temporal load and store
//       per thread, one 256-thread workgroup per 4 KiB; bytes a multiple of
//       4 KiB, both pointers 16-byte aligned.
//   int kda_probe_fill(void* dst, int64_t bytes, uint32_t word, void* stream)
//       every 32-bit word of dst[0, bytes) = word (one 16-byte non-temporal
//       store per thread); bytes a multiple of 4 KiB, dst 16-byte aligned.
// Each returns the hipError_t of its launch (0 on success); work is enqueued
// on `stream` and timed by the caller.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 16;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters) {
  const int tid = threadIdx.x;
  // operands that depend on the lane, so nothing folds at compile time
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * (float)((tid + i) & 15));
    b[i] = static_cast<__bf16>(0.002f * (float)((tid * 3 + i) & 7));
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(int64_t)blockIdx.x * 256 + tid] = s;
}

// One 16-byte vector per thread and many small workgroups: the loads and
// stores of different waves interleave finely (the fastest of the shapes
// tried for the library's page copy); non-temporal, the data is touched once.
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void fill_kernel(u32x4* __restrict__ dst, uint32_t word) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const u32x4 w = {word, word, word, word};
  __builtin_nontemporal_store(w, dst + i);
}

}  // namespace

extern "C" int kda_probe_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

extern "C" int kda_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || bytes % 4096 || bytes / 4096 > INT32_MAX ||
      ((uintptr_t)dst | (uintptr_t)src) % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)(bytes / 4096)), dim3(256), 0, (hipStream_t)stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src));
  return (int)hipGetLastError();
}

extern "C" int kda_probe_fill(void* dst, int64_t bytes, uint32_t word, void* stream) {
  if (!dst || bytes <= 0 || bytes % 4096 || bytes / 4096 > INT32_MAX || (uintptr_t)dst % 16)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)(bytes / 4096)), dim3(256), 0, (hipStream_t)stream,
                     static_cast<u32x4*>(dst), word);
  return (int)hipGetLastError();
}
