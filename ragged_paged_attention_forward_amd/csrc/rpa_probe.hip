// Measured-peak probes: what this device actually sustains for the two
// resources that bound the attention kernels, so that a kernel's throughput
// can be read against a measured ceiling as well as against the published
// one.
//
//  * rpa_probe_read -- a plain streaming read: every workgroup reads one
//    contiguous slice with 16-byte loads, several per thread in flight, and
//    folds the words into one value per thread (written to `sink`, so that
//    the loads are not removed).  Nothing of the attention method is
//    involved; it is the best case for moving the same number of bytes from
//    HBM into the compute units.
//
//  * rpa_probe_mfma -- independent chains of v_mfma_f32_32x32x16_bf16 (the
//    prefill kernel's instruction) on every wave, with operands in registers:
//    the matrix-core throughput at whatever clock the device holds under that
//    load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpa.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 512;   // 8 waves: two per SIMD
constexpr int kMfmaChains = 4;      // independent accumulators per wave

// THREADS threads per workgroup, each with UNROLL 16-byte loads in flight.
template <int THREADS, int UNROLL>
__global__ void __launch_bounds__(THREADS)
probe_read_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t per_wg, uint32_t* __restrict__ sink) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per_wg;
  const int64_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
  uint32_t acc = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += static_cast<int64_t>(THREADS) * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t j = i + static_cast<int64_t>(u) * THREADS;
      v[u] = j < b1 ? src[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[static_cast<int64_t>(blockIdx.x) * THREADS + threadIdx.x] = acc;
}

template <int THREADS, int UNROLL>
hipError_t launch_read(const void* src, int64_t n16, int32_t workgroups, void* sink, hipStream_t stream) {
  const int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL((probe_read_kernel<THREADS, UNROLL>), dim3(workgroups), dim3(THREADS), 0, stream,
                     static_cast<const u32x4*>(src), n16, per_wg, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

__global__ void __launch_bounds__(kMfmaThreads)
probe_mfma_kernel(int iterations, float* __restrict__ sink) {
  const float x = static_cast<float>(threadIdx.x & 7) * 0.125f;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(x + 0.0625f * e);
    b[e] = static_cast<__bf16>(0.5f - 0.03125f * e);
  }
  f32x16 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) c[k] = f32x16{};
  for (int i = 0; i < iterations; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) s += c[k][0] + c[k][15];
  sink[static_cast<int64_t>(blockIdx.x) * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" int rpa_probe_read(const void* src, int64_t bytes, int32_t workgroups, int32_t threads,
                              int32_t loads_in_flight, void* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes < 16 || bytes % 16 != 0 || workgroups < 1 ||
      workgroups > 65536)
    return RPA_ERR_INVALID_ARG;
  const int64_t n16 = bytes / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int key = threads * 100 + loads_in_flight;
  switch (key) {
    case 25604: e = launch_read<256, 4>(src, n16, workgroups, sink, s); break;
    case 25608: e = launch_read<256, 8>(src, n16, workgroups, sink, s); break;
    case 25616: e = launch_read<256, 16>(src, n16, workgroups, sink, s); break;
    case 25632: e = launch_read<256, 32>(src, n16, workgroups, sink, s); break;
    case 102404: e = launch_read<1024, 4>(src, n16, workgroups, sink, s); break;
    case 102408: e = launch_read<1024, 8>(src, n16, workgroups, sink, s); break;
    case 102416: e = launch_read<1024, 16>(src, n16, workgroups, sink, s); break;
    default: return RPA_ERR_INVALID_ARG;
  }
  return e == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}

extern "C" int rpa_probe_mfma(int32_t workgroups, int32_t iterations, void* sink, void* stream) {
  if (sink == nullptr || workgroups < 1 || workgroups > 65536 || iterations < 1) return RPA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                     iterations, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? RPA_OK : RPA_ERR_HIP;
}
