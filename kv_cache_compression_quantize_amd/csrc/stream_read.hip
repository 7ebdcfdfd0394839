// Plain device read stream: the practical ceiling of HBM reads on this part,
// measured with the same toolchain and launch style as the method's kernels
// (a measurement helper beside them, not a step of the method).
#include <algorithm>

#include "internal.h"

namespace aqkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Every 16-byte chunk of the buffer is read once (four loads in flight per
// lane, grid-stride); the xor of everything read goes to *sink by one
// vector-memory atomic per block, so no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const uint4 *__restrict__ p, int64_t n,
                                                                   uint32_t *__restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0u;
    for (int wv = 0; wv < kReadThreads / 64; ++wv) a ^= part[wv];
    atomicXor(sink, a);
  }
}

}  // namespace
}  // namespace aqkv

extern "C" aqkv_status aqkv_read_stream(const void *data, size_t bytes, uint32_t *sink, void *stream) {
  if (!sink || (bytes > 0 && !data)) return AQKV_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(data) % 16 || bytes % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return AQKV_ERR_ALIGN;
  if (bytes == 0) return AQKV_OK;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  // eight blocks of 256 lanes per compute unit: enough loads in flight to cover HBM latency
  const int64_t want = 256 * 8;
  const int64_t blocks = std::min<int64_t>(want, (n + aqkv::kReadThreads - 1) / aqkv::kReadThreads);
  aqkv::read_stream_kernel<<<static_cast<unsigned>(blocks), aqkv::kReadThreads, 0,
                             static_cast<hipStream_t>(stream)>>>(static_cast<const uint4 *>(data), n, sink);
  return hipGetLastError() == hipSuccess ? AQKV_OK : AQKV_ERR_HIP;
}
