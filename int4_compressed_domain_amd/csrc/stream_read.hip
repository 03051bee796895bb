// Streaming-read probe: the HBM read rate a plain kernel reaches on this GPU, the practical
// peak that the decode's achieved rate is set against. Not part of the method, and built
// into a library of its own (libtq_probe.so, include/tq_probe.h).
// Each workgroup of 1024 threads reads one contiguous chunk of the buffer; every thread keeps
// U = 4 16-byte non-temporal loads in flight (a wavefront reads 1 KB per load instruction),
// one workgroup per compute unit, and stores one value, so the loads cannot be dropped. Of
// the layouts tried on MI355X (4/8/16 loads in flight, 256/512/1024 threads, 1-16 workgroups
// per CU, with and without the non-temporal hint) this one read fastest.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"
#include "../../include/tq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int U = 4;      // loads in flight per thread
constexpr int NT = 1024;  // threads per workgroup

__global__ __launch_bounds__(NT) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * NT < b1; i += U * NT) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(src + i + u * NT);
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < b1; i += NT) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(size_t)blockIdx.x * NT + threadIdx.x] = acc;
}

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

}  // namespace

extern "C" int tq_stream_read_probe(const void* buf, size_t bytes, void* sink, size_t sink_bytes,
                                    void* stream) {
  if (bytes == 0) return TQ_OK;
  if (!buf || !sink || bytes % 16 != 0) return TQ_EINVAL;
  const int blocks = num_cus();
  if (sink_bytes < (size_t)blocks * NT * sizeof(uint32_t)) return TQ_ENOSPC;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(NT), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_EDEVICE;
}
