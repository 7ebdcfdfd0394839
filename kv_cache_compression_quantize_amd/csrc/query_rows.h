// The GEMV that rotates and sketches a query (TurboQuant article §六: the
// query is forward-rotated and pre-sketched once, both reused for every
// cached token), shared by query preparation and the top-K selection query.
// A block of 256 threads takes 64 output rows of the stacked [Pi; S] (rows
// below d_rot are Pi's, the rest S's) for one query vector staged in LDS;
// sixteen neighbouring lanes share a row, each reading every sixteenth element
// (so a row is read as one contiguous span), and reduce by shuffles.  The rows
// are loaded first (load), so they are in flight while the caller stages the
// query, then contracted (apply).
#pragma once

#include "internal.h"

namespace aqkv {

template <int D>
struct QueryRows {
  static constexpr int kThreads = 256;
  static constexpr int kLanes = 16;                // lanes per row
  static constexpr int kRows = 64;                 // output rows per block
  static constexpr int kGroups = kThreads / kLanes;
  static constexpr int kIter = kRows / kGroups;
  static constexpr int kPer = D / kLanes;
  float a[kIter][kPer];

  __device__ __forceinline__ int row_of(int chunk, int it) const {
    return chunk * kRows + it * kGroups + static_cast<int>(threadIdx.x) / kLanes;
  }
  // rows chunk * 64 .. + 63 of [rotation (d_rot rows); sketch], zero past `rows`
  __device__ __forceinline__ void load(const float *rotation, const float *sketch, int d_rot, int rows, int chunk) {
    const int sub = threadIdx.x % kLanes;
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int row = row_of(chunk, it);
      const float *src = row < d_rot ? rotation + static_cast<int64_t>(row) * D
                                     : sketch + static_cast<int64_t>(row - d_rot) * D;
#pragma unroll
      for (int i = 0; i < kPer; ++i) a[it][i] = row < rows ? src[sub + kLanes * i] : 0.0f;
    }
  }
  // the rows times qs (LDS, D floats): row r < d_rot to q_rot[r], the others to q_sk[r - d_rot]
  __device__ __forceinline__ void apply(const float *qs, int d_rot, int rows, int chunk, float *q_rot,
                                        float *q_sk) const {
    const int sub = threadIdx.x % kLanes;
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int row = row_of(chunk, it);
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc = fmaf(a[it][i], qs[sub + kLanes * i], acc);
#pragma unroll
      for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kLanes);
      if (sub == 0 && row < rows) {
        if (row < d_rot)
          q_rot[row] = acc;
        else
          q_sk[row - d_rot] = acc;
      }
    }
  }
};

}  // namespace aqkv
