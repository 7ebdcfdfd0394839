// Query preparation (TurboQuant article §六: the query is forward-rotated,
// q Pi^T, and pre-sketched, q S^T, once per query; both are reused for every
// cached token): one block per (query vector, 64 rows of [Pi; S]), the GEMV of
// query_rows.h.  All of a lane's loads are issued before the first is used,
// so a block costs about one memory round trip.

#include "internal.h"
#include "query_rows.h"

namespace aqkv {
namespace {

template <int D>
__global__ __launch_bounds__(QueryRows<D>::kThreads) void prepare_query_kernel(QueryJob job, int chunks) {
  __shared__ float qs[D];
  const int64_t n = blockIdx.x / chunks;
  const int chunk = static_cast<int>(blockIdx.x % chunks);
  const int d_rot = job.q_rot ? D : 0;
  const int rows = d_rot + job.m;
  QueryRows<D> qr;
  qr.load(job.rotation, job.sketch, d_rot, rows, chunk);
  // the matrix rows are in flight while the query is staged
  for (int k = threadIdx.x; k < D; k += QueryRows<D>::kThreads) {
    if (job.dtype == AQKV_BF16)
      qs[k] = bf16_to_f32(static_cast<const uint16_t *>(job.q)[n * D + k]);
    else
      qs[k] = static_cast<const float *>(job.q)[n * D + k];
  }
  __syncthreads();
  qr.apply(qs, d_rot, rows, chunk, job.q_rot ? job.q_rot + n * D : nullptr, job.q_sketch + n * job.m);
}

}  // namespace

hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream) {
  const int rows = (job.q_rot ? job.d : 0) + job.m;
  const int chunks = (rows + 63) / 64;
  const unsigned grid = static_cast<unsigned>(job.n_q * chunks);
  switch (job.d) {
    case 64: prepare_query_kernel<64><<<grid, 256, 0, stream>>>(job, chunks); break;
    case 128: prepare_query_kernel<128><<<grid, 256, 0, stream>>>(job, chunks); break;
    default: prepare_query_kernel<256><<<grid, 256, 0, stream>>>(job, chunks); break;
  }
  return hipGetLastError();
}

}  // namespace aqkv
