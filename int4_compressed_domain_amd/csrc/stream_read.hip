// Streaming-read probe: the HBM read rate a plain kernel reaches on this GPU, the practical
// peak that the decode's achieved rate is set against. Not part of the method.
// Each workgroup reads one contiguous chunk of the buffer; every thread keeps 8 16-byte loads
// in flight (a wavefront reads 1 KB per load instruction) and stores one value, so the loads
// cannot be dropped. (Of the layouts tried on MI355X this one read fastest: 6.2 TB/s on 2 GiB.)
#include "tq_device.h"
#include "tq_internal.h"

namespace {

constexpr int U = 8;  // loads in flight per thread

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * 256 < b1; i += U * 256) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = src[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += 256) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

hipError_t tq_launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, st,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}
