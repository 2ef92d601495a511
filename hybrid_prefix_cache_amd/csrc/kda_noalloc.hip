// kda_noalloc.hip -- chunked prefill for callers that cannot allocate device
// memory: the workspace is a fixed static device array of this library.
//
// The array lives in the code object (one copy per GPU, allocated when the
// library's code object is loaded on that device and held until the process
// ends).  Host code never passes the array's name to a kernel: the name is a
// host-side stand-in.  The device address is resolved once per device with
// hipGetSymbolAddress and that address is what the prefill receives as its
// workspace.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace kda {
void host_set_error(const char* msg);
}

namespace {

static_assert(KDA_PREFILL_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[KDA_PREFILL_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved

kda_status fail_msg(kda_status st, const char* msg) {
  kda::host_set_error(msg);
  return st;
}

// Device address of the current device's scratch array (resolved on the first
// call on that device, with that device current).
kda_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_msg(KDA_ERR_HIP, "kda_prefill_chunked_noalloc: no current device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail_msg(KDA_ERR_HIP, "kda_prefill_chunked_noalloc: device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char buf[256];
      snprintf(buf, sizeof(buf), "kda_prefill_chunked_noalloc: hipGetSymbolAddress: %s",
               hipGetErrorString(e));
      return fail_msg(KDA_ERR_HIP, buf);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_prefill_chunked_noalloc(
    const kda_pool* pool, const void* q, const void* k, const void* v, const void* g,
    const void* beta, kda_dtype in_dtype, void* o, kda_dtype out_dtype, int32_t num_seqs,
    const int64_t* cu_seqlens, const int64_t* start_pos, const int32_t* state_in_page,
    const int32_t* state_out_page, const int32_t* ckpt_cu, const int64_t* ckpt_pos,
    const int32_t* ckpt_page, int32_t chunk_size, int32_t hash_block, void* stream) {
  // full validation first (host only); the scratch address is resolved only
  // for a call that passes it and fits the array
  return kda::prefill_impl(pool, q, k, v, g, beta, in_dtype, o, out_dtype, num_seqs, cu_seqlens,
                           start_pos, state_in_page, state_out_page, ckpt_cu, ckpt_pos, ckpt_page,
                           chunk_size, hash_block, nullptr, (size_t)KDA_PREFILL_SCRATCH_BYTES,
                           scratch_ptr, stream);
}
