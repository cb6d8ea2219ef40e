// measure.hip -- the achievable-bandwidth probe: one plain streaming read of a
// device buffer with 128-bit non-temporal loads, the access pattern of the
// decode kernels' weight streams, and nothing else.  The decode step's speed
// is weight bytes over time [P3 "Flint: 125 tokens a second is what 2.5B
// active parameters buy at 273 GB/s", "Checking 125 tokens a second":
// bandwidth = bytes read per token x tokens per second], so this read sets
// the practical ceiling that the roofline fractions are read against.
#include "flint_common.h"
#include "flint_device.h"

namespace flint {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

// Every word read is folded into acc, which is stored only if it equals a key
// the compiler cannot know, so no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint4* __restrict__ p, uint64_t n16,
                                                               uint32_t key, uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = ld_nt_u4(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld_nt_u4(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) out[0] = acc;
}

}  // namespace
}  // namespace flint

using namespace flint;

extern "C" int32_t flint_stream_read(const void* src, size_t bytes, uint32_t* out, void* stream) {
  if (!src || !out) return FLINT_E_NULL;
  if (bytes < 16 || bytes % 16) return FLINT_E_DIMS;
  if (((uintptr_t)src & 15) || ((uintptr_t)out & 3)) return FLINT_E_ALIGN;
  int32_t st;
  if ((st = api_check_device())) return st;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return api_hip_fail(e);
  // eight workgroups of four waves per compute unit: enough loads in flight
  // to cover the memory latency
  const int grid = (cus > 0 ? cus : 256) * 8;
  k_stream_read<<<grid, kProbeThreads, 0, (hipStream_t)stream>>>(static_cast<const uint4*>(src), bytes / 16,
                                                                 0x9E3779B9u, out);
  e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}
