// Exact attention over the recent-token window (TurboQuant article §六: the
// latest tokens stay at full precision in a ring buffer while the older
// history is served by the compressed path; attention covers both with one
// softmax).
//
// One block per kv slot computes, for each of its g query heads, the exact
// logits <q, k_t> * softmax_scale of the window's tokens (log2 units, fp32
// accumulation), their maximum M, L = sum 2^(logit - M) and
// acc = sum 2^(logit - M) v_t, and writes them as one more partial beside the
// compressed path's split partials, so the split combine merges both.  The
// window is small (at most 1024 tokens): its logits stay in LDS, every row is
// read twice from L2 at most, and the pass is a latency-bound side job.
#include "internal.h"

namespace aqkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float x, float *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// 8 consecutive elements of a row as fp32 (one 16-byte load for bf16, two for fp32)
template <bool BF16>
__device__ __forceinline__ void load8(const char *row, int c, float (&x)[8]) {
  if constexpr (BF16) {
    const uint4 u = reinterpret_cast<const uint4 *>(row)[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4 a = reinterpret_cast<const float4 *>(row)[2 * c];
    const float4 b = reinterpret_cast<const float4 *>(row)[2 * c + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void window_partial_kernel(WindowJob job) {
  extern __shared__ float smem[];                  // q [g][D], then p [g][n_window]
  __shared__ float red[4];
  __shared__ float part[kThreads];
  constexpr int kElt = BF16 ? 2 : 4;
  const int G = job.g, nw = job.n_window, tid = threadIdx.x;
  float *qs = smem;
  float *pw = smem + G * D;
  const int64_t slot = blockIdx.x;
  const int64_t b = slot / job.heads, h = slot % job.heads;
  for (int i = tid; i < G * D; i += kThreads) qs[i] = job.q[slot * G * D + i];
  __syncthreads();

  // 1. logits of every (head, token), log2 units
  const float lscale = job.softmax_scale * kLog2e;
  const char *kb = static_cast<const char *>(job.k) + (b * job.k_bs + h * job.k_hs) * kElt;
  for (int t = tid; t < nw; t += kThreads) {
    const char *row = kb + t * job.k_ts * kElt;
    float s[kMaxQPerKv];
#pragma unroll
    for (int g = 0; g < kMaxQPerKv; ++g) s[g] = 0.0f;
    for (int c = 0; c < D / 8; ++c) {
      float x[8];
      load8<BF16>(row, c, x);
#pragma unroll
      for (int g = 0; g < kMaxQPerKv; ++g) {
        if (g >= G) break;
        const float *qg = qs + g * D + 8 * c;
#pragma unroll
        for (int j = 0; j < 8; ++j) s[g] = fmaf(qg[j], x[j], s[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < kMaxQPerKv; ++g)
      if (g < G) pw[g * nw + t] = s[g] * lscale;
  }
  __syncthreads();

  // 2. per head: M, the weights 2^(logit - M) in place, L
  constexpr int P = kThreads / D;                  // threads per channel in the value sum
  const int j = tid % D, ph = tid / D;
  const char *vb = static_cast<const char *>(job.v) + (b * job.v_bs + h * job.v_hs) * kElt;
  for (int g = 0; g < G; ++g) {
    float mx = -INFINITY;
    for (int t = tid; t < nw; t += kThreads) mx = fmaxf(mx, pw[g * nw + t]);
    const float M = block_max(mx, red);
    float l = 0.0f;
    for (int t = tid; t < nw; t += kThreads) {
      const float p = __builtin_amdgcn_exp2f(pw[g * nw + t] - M);
      pw[g * nw + t] = p;
      l += p;
    }
    const float L = block_sum(l, red);             // its barriers also publish the weights

    // 3. acc[j] = sum_t p_t v_t[j]: P threads per channel, every P-th token each
    float o = 0.0f;
    for (int t = ph; t < nw; t += P) {
      const char *row = vb + t * job.v_ts * kElt;
      float v;
      if constexpr (BF16) v = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(row)[j]) << 16);
      else v = reinterpret_cast<const float *>(row)[j];
      o = fmaf(pw[g * nw + t], v, o);
    }
    part[tid] = o;
    __syncthreads();
    const int64_t ph_idx = (slot * G + g) * job.part_stride + job.part_index;
    if (ph == 0) {
      float sum = 0.0f;
      for (int k = 0; k < P; ++k) sum += part[k * D + j];
      job.part_acc[ph_idx * D + j] = nw > 0 ? sum : 0.0f;
    }
    if (tid == 0) {
      job.part_ml[ph_idx * 2 + 0] = nw > 0 ? M : 0.0f;
      job.part_ml[ph_idx * 2 + 1] = nw > 0 ? L : 0.0f;   // 0 = empty part
    }
    __syncthreads();                               // part[] and red[] reused by the next head
  }
}

template <int D>
hipError_t launch_d(const WindowJob &job, hipStream_t stream) {
  const size_t smem = sizeof(float) * static_cast<size_t>(job.g) * (D + job.n_window);
  auto kern = job.dtype == AQKV_BF16 ? window_partial_kernel<D, true> : window_partial_kernel<D, false>;
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  kern<<<static_cast<unsigned>(job.n_slots), kThreads, smem, stream>>>(job);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_window_partial(const WindowJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
