// tq_calib: a plain streaming read of device memory, the on-box ceiling the
// codec's read-dominated kernels are measured against (besides the vendor's
// 8 TB/s).  Grid-stride 16-byte non-temporal loads, eight in flight per
// thread, folded into one xor per thread so that no load is dead; the last
// thread-group's xor lands in `sink`.

#include "tq_device.h"

namespace tq {

typedef uint32_t u32x4_c __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_c* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  constexpr int U = 8;
  int64_t i = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  u32x4_c acc = {0u, 0u, 0u, 0u};
  for (; i + 256 * (U - 1) < n16; i += stride) {
    u32x4_c v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + 256 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) sink[0] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const int64_t n16 = bytes / 16;
  hipLaunchKernelGGL(stream_read_kernel, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_c*>(src), n16, sink);
  return (int)hipGetLastError();
}

}  // namespace tq
