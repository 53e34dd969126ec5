// rpa_probe_e4m3: the fp8 decode kernel's byte conversion on its own, so
// that its lane layout and exactness can be checked against a reference
// decoding of all 256 E4M3 bytes.  Each thread converts 8 bytes with the
// same device function the decode kernel uses.
#include "rpa_device.h"

namespace rpa {

constexpr int kE4m3Threads = 256;

__global__ void __launch_bounds__(kE4m3Threads)
probe_e4m3_kernel(const uint8_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kE4m3Threads + threadIdx.x;
  if (i >= n8) return;
  *reinterpret_cast<u32x4*>(dst + i * 8) = e4m3x8_to_bf16x8(load8(src + i * 8));
}

}  // namespace rpa

extern "C" int rpa_probe_e4m3(const void* src, void* dst, int64_t count, void* stream) {
  if (src == nullptr || dst == nullptr || count < 8 || count % 8 != 0 || count > (int64_t(1) << 30))
    return RPA_ERR_INVALID_ARG;
  const int64_t n8 = count / 8;
  const int blocks = static_cast<int>((n8 + rpa::kE4m3Threads - 1) / rpa::kE4m3Threads);
  hipLaunchKernelGGL(rpa::probe_e4m3_kernel, dim3(blocks), dim3(rpa::kE4m3Threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src), static_cast<uint16_t*>(dst),
                     n8);
  return hipGetLastError() == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}
