// Plain device read stream: the practical ceiling of HBM reads on this part,
// measured with the same toolchain and launch style as the method's kernels
// (a measurement helper beside them, not a step of the method).
#include <algorithm>

#include "internal.h"

namespace aqkv {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Every 16-byte chunk of the buffer is read once (eight loads in flight per
// lane, grid-stride); a lane stores the xor of what it read to *sink only if it
// is all ones, so no load can be dropped and almost no lane stores (a store or
// atomic per block cost up to 18 % of the rate at this grid).
__global__ __launch_bounds__(kReadThreads) void read_stream_kernel(const uint4 *__restrict__ p, int64_t n,
                                                                   uint32_t *__restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = stream_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = stream_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0xFFFFFFFFu) *sink = acc;
}

}  // namespace
}  // namespace aqkv

extern "C" aqkv_status aqkv_read_stream(const void *data, size_t bytes, uint32_t *sink, void *stream) {
  if (!sink || (bytes > 0 && !data)) return AQKV_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(data) % 16 || bytes % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return AQKV_ERR_ALIGN;
  if (bytes == 0) return AQKV_OK;
  const int64_t n = static_cast<int64_t>(bytes / 16);
  // 32 blocks of 256 lanes per compute unit (four rounds of full occupancy), eight
  // non-temporal 16-byte loads in flight per lane: the fastest of the shapes measured
  // (1024-8192 blocks, 4 or 8 loads, plain or non-temporal)
  const int64_t want = 256 * 32;
  const int64_t blocks = std::min<int64_t>(want, (n + aqkv::kReadThreads - 1) / aqkv::kReadThreads);
  aqkv::read_stream_kernel<<<static_cast<unsigned>(blocks), aqkv::kReadThreads, 0,
                             static_cast<hipStream_t>(stream)>>>(static_cast<const uint4 *>(data), n, sink);
  return hipGetLastError() == hipSuccess ? AQKV_OK : AQKV_ERR_HIP;
}
