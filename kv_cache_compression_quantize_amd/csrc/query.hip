// Query preparation and the per-layer projection used by key quantisation.
//
// prepare_query (TurboQuant article §六: the query is forward-rotated, q Pi^T,
// and pre-sketched, q S^T, once per query; both are reused for every cached
// token): one block per query vector, the vector staged in LDS, one thread per
// output row.  This is a tiny GEMV and is latency-bound.
//
// make_projection: P = S Pi^T ([m][d]).  With Pi orthogonal the QJL residual
// sketch satisfies S r = S Pi^T (Pi r) = n * P e, where e = y - c[idx] is the
// residual in rotated unit-sphere coordinates, so the key kernel can sketch
// the residual without first rotating the reconstruction back (one d x m
// product per key instead of a d x d and a d x m one).
#include "internal.h"

namespace aqkv {
namespace {

__global__ __launch_bounds__(256) void make_projection_kernel(const float *__restrict__ sketch,
                                                              const float *__restrict__ rotation,
                                                              float *__restrict__ proj, int m, int d) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(m) * d) return;
  const int i = static_cast<int>(idx / d), j = static_cast<int>(idx % d);
  const float *srow = sketch + static_cast<int64_t>(i) * d;
  const float *prow = rotation + static_cast<int64_t>(j) * d;
  float acc = 0.0f;
  for (int k = 0; k < d; ++k) acc = fmaf(srow[k], prow[k], acc);
  proj[idx] = acc;
}

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

hipError_t launch_make_projection(const float *sketch, const float *rotation, float *proj, int m, int d,
                                  hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(m) * d;
  make_projection_kernel<<<(total + 255) / 256, 256, 0, stream>>>(sketch, rotation, proj, m, d);
  return hipGetLastError();
}

hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream) {
  prepare_query_kernel<<<job.n_q, 256, job.d * sizeof(float), stream>>>(job);
  return hipGetLastError();
}

}  // namespace aqkv
