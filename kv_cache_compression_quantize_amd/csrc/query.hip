// Query preparation.
//
// prepare_query (TurboQuant article §六: the query is forward-rotated, q Pi^T,
// and pre-sketched, q S^T, once per query; both are reused for every cached
// token).  A tiny GEMV: each block takes one query vector (staged in LDS) and
// kRowsPerBlock output rows of the stacked [Pi; S]; sixteen neighbouring lanes
// share a row, each reading every sixteenth element (so a row is read as one
// contiguous span), and reduce by shuffles.  All of a lane's loads are issued
// before the first is used, so a block costs about one memory round trip.

#include "internal.h"

namespace aqkv {
namespace {

constexpr int kQThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerBlock = 64;

template <int D>
__global__ __launch_bounds__(kQThreads) void prepare_query_kernel(QueryJob job, int chunks) {
  __shared__ float qs[D];
  const int64_t n = blockIdx.x / chunks;
  const int chunk = static_cast<int>(blockIdx.x % chunks);
  const int m = job.m;
  const int d_rot = job.q_rot ? D : 0;
  const int rows = d_rot + m;
  const int sub = threadIdx.x % kLanesPerRow, grp = threadIdx.x / kLanesPerRow;
  constexpr int kGroups = kQThreads / kLanesPerRow;
  constexpr int kIter = kRowsPerBlock / kGroups;
  constexpr int kPer = D / kLanesPerRow;
  float a[kIter][kPer];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int row = chunk * kRowsPerBlock + it * kGroups + grp;
    const float *src = row < d_rot ? job.rotation + static_cast<int64_t>(row) * D
                                   : job.sketch + static_cast<int64_t>(row - d_rot) * D;
#pragma unroll
    for (int i = 0; i < kPer; ++i) a[it][i] = row < rows ? src[sub + kLanesPerRow * i] : 0.0f;
  }
  // the matrix rows are in flight while the query is staged
  for (int k = threadIdx.x; k < D; k += kQThreads) {
    if (job.dtype == AQKV_BF16)
      qs[k] = bf16_to_f32(static_cast<const uint16_t *>(job.q)[n * D + k]);
    else
      qs[k] = static_cast<const float *>(job.q)[n * D + k];
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int row = chunk * kRowsPerBlock + it * kGroups + grp;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) acc = fmaf(a[it][i], qs[sub + kLanesPerRow * i], acc);
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kLanesPerRow);
    if (sub == 0 && row < rows) {
      if (row < d_rot)
        job.q_rot[n * D + row] = acc;
      else
        job.q_sketch[n * m + (row - d_rot)] = acc;
    }
  }
}

}  // namespace

hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream) {
  const int rows = (job.q_rot ? job.d : 0) + job.m;
  const int chunks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const unsigned grid = static_cast<unsigned>(job.n_q * chunks);
  switch (job.d) {
    case 64: prepare_query_kernel<64><<<grid, kQThreads, 0, stream>>>(job, chunks); break;
    case 128: prepare_query_kernel<128><<<grid, kQThreads, 0, stream>>>(job, chunks); break;
    default: prepare_query_kernel<256><<<grid, kQThreads, 0, stream>>>(job, chunks); break;
  }
  return hipGetLastError();
}

}  // namespace aqkv
