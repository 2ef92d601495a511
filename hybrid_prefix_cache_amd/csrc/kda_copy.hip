// kda_copy.hip -- batched page copy for checkpoint write / restore, gfx950.
//
// Page "Cache de préfixe hybride KDA–MLA" (mkdocs.reaper.mx), section "Le
// fonctionnement du prefill": checkpoints are read-only; a prefix hit copies
// the checkpoint into the request's private state, and new checkpoints are
// written to fresh slots.  Both directions are the same operation here: copy
// the state bytes (num_heads * d_k * d_v * 4) of one page to another.  Page
// padding is not touched.
//
// One workgroup moves one 4 KiB piece of one page pair, one 16-byte
// non-temporal load and store per thread.  Measured on 256 x 2 MiB pages, this
// finest split streams fastest (~6.5 TB/s): many small workgroups keep the
// loads and stores of different waves interleaved, where a thread that first
// loads 16 vectors and then stores them leaves the memory system bursty
// (~5.4 TB/s).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(CopyArgs a) {
  static_assert(kPieceBytes == 256 * 16, "one vector per thread");
  const int pair = blockIdx.x / a.pieces, piece = blockIdx.x % a.pieces;
  if (pair >= a.npairs) return;
  const int64_t off = (int64_t)piece * kPieceBytes + 16 * (int64_t)threadIdx.x;
  if (off >= a.state_bytes) return;  // state bytes are a multiple of 16
  const u32x4* s = reinterpret_cast<const u32x4*>(a.pool + a.src[pair] * a.page_bytes + off);
  u32x4* d = reinterpret_cast<u32x4*>(a.pool + a.dst[pair] * a.page_bytes + off);
  __builtin_nontemporal_store(__builtin_nontemporal_load(s), d);
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)a.npairs * (unsigned)a.pieces), dim3(256), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace kda
