// Streaming-read reference kernel (pa_probe.h): reads a buffer once with the decode kernels' 16-byte
// non-temporal lane loads, a ring of 4 wave loads in flight per wave, each wave a contiguous slice.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeDepth = 4;

__global__ __launch_bounds__(64) void stream_read_kernel(const uint4* buf, int64_t chunks, uint32_t* sink) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t w = blockIdx.x, n = gridDim.x;
  // a wave's slice: whole 1 KB wave loads (64 lanes x 16 bytes)
  const int64_t loads = chunks / 64;
  const int64_t l0 = w * loads / n, l1 = (w + 1) * loads / n;
  const u32x4* p = reinterpret_cast<const u32x4*>(buf) + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  int64_t l = l0;
  for (; l + kProbeDepth <= l1; l += kProbeDepth) {
    u32x4 x[kProbeDepth];
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) x[d] = __builtin_nontemporal_load(p + (l + d) * 64);
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) acc ^= x[d];
  }
  for (; l < l1; ++l) acc ^= __builtin_nontemporal_load(p + l * 64);
  if (w == n - 1) {  // the tail past the last whole wave load
    for (int64_t c = loads * 64 + threadIdx.x; c < chunks; c += 64) acc ^= __builtin_nontemporal_load(p - threadIdx.x + c);
  }
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) v ^= __shfl_xor(v, d);
  if (threadIdx.x == 0) sink[w] = v;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t chunks, int num_waves, uint32_t* sink, hipStream_t s,
                              KernelTiming tm) {
  hipExtLaunchKernelGGL(stream_read_kernel, dim3((unsigned)num_waves), dim3(64), 0, s, tm.start, tm.stop, 0,
                        static_cast<const uint4*>(buf), chunks, sink);
  return hipGetLastError();
}

}  // namespace pa
