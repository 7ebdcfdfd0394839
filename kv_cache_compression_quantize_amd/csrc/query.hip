// Query preparation.
//
// prepare_query (TurboQuant article §六: the query is forward-rotated, q Pi^T,
// and pre-sketched, q S^T, once per query; both are reused for every cached
// token): one block per query vector, the vector staged in LDS, one thread per
// output row.  This is a tiny GEMV and is latency-bound.

#include "internal.h"

namespace aqkv {
namespace {

__global__ __launch_bounds__(256) void prepare_query_kernel(QueryJob job) {
  extern __shared__ float qs[];
  const int64_t n = blockIdx.x;
  const int d = job.d, m = job.m;
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    if (job.dtype == AQKV_BF16)
      qs[k] = bf16_to_f32(static_cast<const uint16_t *>(job.q)[n * d + k]);
    else
      qs[k] = static_cast<const float *>(job.q)[n * d + k];
  }
  __syncthreads();
  if (job.q_rot) {
    for (int j = threadIdx.x; j < d; j += blockDim.x) {
      const float *row = job.rotation + static_cast<int64_t>(j) * d;
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(row[k], qs[k], acc);
      job.q_rot[n * d + j] = acc;
    }
  }
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    const float *row = job.sketch + static_cast<int64_t>(i) * d;
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = fmaf(row[k], qs[k], acc);
    job.q_sketch[n * m + i] = acc;
  }
}

}  // namespace

hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream) {
  prepare_query_kernel<<<job.n_q, 256, job.d * sizeof(float), stream>>>(job);
  return hipGetLastError();
}

}  // namespace aqkv
