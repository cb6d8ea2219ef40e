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

constexpr int kProbeThreads = 512;
constexpr int kProbeDepth = 8;  // 8 KB pieces a workgroup keeps in flight

// Each workgroup reads whole 8 KB pieces (one 16-byte load a thread a
// piece), pieces b, b + G, b + 2 G, ... for workgroup b of G, eight at a time:
// consecutive pieces go to consecutive workgroups and so to the XCDs in turn.
// This reads about 15% faster than a grid-stride loop of 4 KB per workgroup
// (one workgroup per compute unit, or eight of 256 threads).  Every word read
// is folded into acc, which is stored only if it equals a key the compiler
// cannot know, so no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint4* __restrict__ p, uint64_t n16,
                                                               uint32_t key, uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const uint64_t np = n16 / kProbeThreads, G = gridDim.x;  // whole pieces
  uint64_t k = blockIdx.x;
  for (; k + (kProbeDepth - 1) * G < np; k += kProbeDepth * G) {
    uint4 v[kProbeDepth];
#pragma unroll
    for (int u = 0; u < kProbeDepth; ++u) v[u] = ld_nt_u4(p + (k + u * G) * kProbeThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kProbeDepth; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; k < np; k += G) {
    const uint4 v = ld_nt_u4(p + k * kProbeThreads + threadIdx.x);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the part past the last whole piece
  for (uint64_t i = np * kProbeThreads + (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n16;
       i += G * kProbeThreads) {
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
  // one workgroup of eight waves per compute unit, eight pieces in flight
  const int grid = cus > 0 ? cus : 256;
  k_stream_read<<<grid, kProbeThreads, 0, (hipStream_t)stream>>>(static_cast<const uint4*>(src), bytes / 16,
                                                                 0x9E3779B9u, out);
  e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}
