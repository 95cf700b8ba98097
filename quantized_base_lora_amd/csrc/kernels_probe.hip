// Measurement kernel: a plain streaming read, the HBM ceiling the path's
// kernels are compared with (no dequantization, no arithmetic beyond an XOR
// per word, no stores but one word per thread).
#include "common.h"
#include "device.h"

namespace ql {
namespace {

constexpr int SR_BLOCKS = 256, SR_THREADS = 256, SR_UNR = 8;

// thread t reads 16-byte words t, t + T, t + 2T, ... (T the grid's threads),
// SR_UNR loads in flight; words past the end read zero
__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const uint4* __restrict__ p, int64_t nwords,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t T = (int64_t)SR_BLOCKS * SR_THREADS;
  const int64_t t0 = (int64_t)blockIdx.x * SR_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t i = t0; i < nwords; i += SR_UNR * T) {
    uint4 v[SR_UNR];
#pragma unroll
    for (int u = 0; u < SR_UNR; ++u) {
      const int64_t w = i + u * T;
      v[u] = w < nwords ? p[w] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < SR_UNR; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[t0] = acc;
}

}  // namespace

static_assert(SR_BLOCKS * SR_THREADS == QL_STREAM_READ_THREADS, "grid of the stream read");

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(SR_BLOCKS), dim3(SR_THREADS), 0, s,
                     reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace ql
