// kda_copy.hip -- batched page copy for checkpoint write / restore, gfx950.
//
// Page "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx), section "Le
// fonctionnement du prefill": checkpoints are read-only; a prefix hit copies
// the checkpoint into the request's private state, and new checkpoints are
// written to fresh slots.  Both directions are the same operation here: copy
// the state bytes (num_heads * d_k * d_v * 4) of one page to another.  Page
// padding is not touched.
//
// One workgroup moves one 64 KiB piece (one head at d = 128) of one page
// pair with 16-byte loads, all loads issued before the stores.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(CopyArgs a) {
  const int pair = blockIdx.x / a.pieces, piece = blockIdx.x % a.pieces;
  if (pair >= a.npairs) return;
  const int64_t off = (int64_t)piece * kPieceBytes;
  const int64_t nbytes = min((int64_t)kPieceBytes, a.state_bytes - off);
  const u32x4* s = reinterpret_cast<const u32x4*>(a.pool + a.src[pair] * a.page_bytes + off);
  u32x4* d = reinterpret_cast<u32x4*>(a.pool + a.dst[pair] * a.page_bytes + off);
  const int nvec = (int)(nbytes >> 4);
  constexpr int kUnroll = kPieceBytes / 16 / 256;  // 16 vectors per thread
  u32x4 buf[kUnroll];
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int idx = threadIdx.x + i * 256;
    if (idx < nvec) buf[i] = __builtin_nontemporal_load(s + idx);
  }
#pragma unroll
  for (int i = 0; i < kUnroll; ++i) {
    const int idx = threadIdx.x + i * 256;
    if (idx < nvec) __builtin_nontemporal_store(buf[i], d + idx);
  }
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)a.npairs * (unsigned)a.pieces), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace kda
