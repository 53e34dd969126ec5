// rpa_forward_noalloc: ragged paged attention for callers that cannot
// allocate device memory.  The work list and the split-KV partials of a call
// live in one file-scope device array, `scratch`, that the library holds
// until the process ends (one copy per GPU, at that GPU's own address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "rpa.h"
#include "rpa_scratch.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;   // RPA_NOALLOC_SCRATCH_BYTES in rpa.h
static_assert(kScratchBytes == RPA_NOALLOC_SCRATCH_BYTES, "scratch size and its documented value");

// The device array.  Host code never passes `scratch` itself to a kernel or a
// copy (in host code it names a host-side stand-in): it uses the device
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the
// first call made on that device and kept.
int scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return RPA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[device] == nullptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return RPA_ERR_HIP;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return RPA_OK;
}

}  // namespace

extern "C" int rpa_forward_noalloc(rpa_ctx* ctx, const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* cu_q_lens, const int32_t* kv_lens,
                                   int32_t num_seqs, int32_t window, float scale, void* out, void* stream) {
  // host checks first; the scratch address is looked up (on the context's
  // device, current at that point) only for a call that launches work
  return rpa::forward_scratch(ctx, q, k_pages, v_pages, page_table, cu_q_lens, kv_lens, num_seqs, window, scale,
                              out, stream, scratch_address, kScratchBytes);
}
