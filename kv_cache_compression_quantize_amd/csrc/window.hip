// Attention over the recent-token window, merged with the compressed path
// (TurboQuant article §六: the latest tokens stay at full precision in a ring
// buffer while the older history is served by the compressed path; attention
// covers both with one softmax).
//
// This replaces the split combine when a window is given: one block per query
// head computes the window's exact logits <q, k_t> * softmax_scale (log2
// units, fp32 accumulation), its maximum, weights and weighted value sum, and
// merges them with the decoder's split partials into the output.  The window
// is small (at most 1024 tokens): its logits stay in LDS; rows are read as
// 16-byte pieces by several lanes at once (8 lanes per key row for the logits,
// one lane per 8 channels of a value row for the sum).
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

// 8 consecutive elements (chunk c) of a row as fp32: one 16-byte load for
// bf16, two for fp32
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
__global__ __launch_bounds__(kThreads) void combine_window_kernel(DecodeJob job, WindowJob wj) {
  constexpr int kElt = BF16 ? 2 : 4;
  constexpr int CH = D / 8;                        // 8-channel chunks of a row
  constexpr int CPL = CH / 8;                      // chunks per lane: 8 lanes share a token's logit
  constexpr int TP = kThreads / CH;                // token phases of the value sum
  __shared__ float qs[D];
  __shared__ float pw[kMaxWindow];
  __shared__ float part[TP * D];
  __shared__ float red[4];
  __shared__ float wts[1024];
  const int tid = threadIdx.x, nw = wj.n_window, G = wj.g;
  const int64_t head = blockIdx.x, slot = head / G;
  const int64_t b = slot / wj.heads, h = slot % wj.heads;
  for (int i = tid; i < D; i += kThreads) qs[i] = wj.q[head * D + i];
  __syncthreads();

  // 1. window logits (log2 units): 8 lanes per token, summed over the 8 lanes
  const float lscale = wj.softmax_scale * kLog2e;
  const char *kb = static_cast<const char *>(wj.k) + (b * wj.k_bs + h * wj.k_hs) * kElt;
  const int lt = tid / 8, pl = tid % 8;
  for (int t0 = 0; t0 < nw; t0 += kThreads / 8) {
    const int t = t0 + lt;
    float x[CPL][8];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[c][j] = 0.0f;
    if (t < nw) {
      const char *row = kb + t * wj.k_ts * kElt;
#pragma unroll
      for (int c = 0; c < CPL; ++c) load8<BF16>(row, pl * CPL + c, x[c]);
    }
    const float *qp = qs + pl * CPL * 8;
    float sg = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) sg = fmaf(qp[8 * c + j], x[c][j], sg);
    sg += __shfl_xor(sg, 1);
    sg += __shfl_xor(sg, 2);
    sg += __shfl_xor(sg, 4);
    if (pl == 0 && t < nw) pw[t] = sg * lscale;
  }
  __syncthreads();

  // 2. the window's maximum, weights 2^(logit - Mw) in place, their sum
  float mx = -INFINITY;
  for (int t = tid; t < nw; t += kThreads) mx = fmaxf(mx, pw[t]);
  const float Mw = block_max(mx, red);
  float l = 0.0f;
  for (int t = tid; t < nw; t += kThreads) {
    const float p = __builtin_amdgcn_exp2f(pw[t] - Mw);
    pw[t] = p;
    l += p;
  }
  const float Lw = block_sum(l, red);              // its barriers also publish the weights

  // 3. the maximum over the window and the non-empty split partials
  const int ns = job.part_stride;
  const float *ml = job.part_ml + head * ns * 2;
  const float *acc = job.part_acc + head * ns * D;
  float ms = -INFINITY;
  for (int i = tid; i < ns; i += kThreads)
    if (ml[2 * i + 1] > 0.0f) ms = fmaxf(ms, ml[2 * i]);
  const float M = fmaxf(block_max(ms, red), nw > 0 ? Mw : -INFINITY);
  const float ww = nw > 0 ? __builtin_amdgcn_exp2f(Mw - M) : 0.0f;   // the window's weight

  // 4. out[j] = (ww sum_t p_t v_t[j] + sum_i w_i acc_i[j]) / (ww Lw + sum_i w_i l_i):
  //    each thread 8 channels of every TP-th window token, then of every TP-th split
  const int tp = tid / CH, ck = tid % CH;
  const char *vb = static_cast<const char *>(wj.v) + (b * wj.v_bs + h * wj.v_hs) * kElt;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.0f;
#pragma unroll 4
  for (int t = tp; t < nw; t += TP) {
    float x[8];
    load8<BF16>(vb + t * wj.v_ts * kElt, ck, x);
    const float p = pw[t] * ww;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = fmaf(p, x[j], o[j]);
  }
  float lsum = tid == 0 ? Lw * ww : 0.0f;
  for (int c0 = 0; c0 < ns; c0 += 1024) {
    const int cn = min(1024, ns - c0);
    __syncthreads();                               // the previous chunk's weights are consumed
    for (int i = tid; i < cn; i += kThreads) {
      const float li = ml[2 * (c0 + i) + 1];
      const float wi = li > 0.0f ? __builtin_amdgcn_exp2f(ml[2 * (c0 + i)] - M) : 0.0f;
      wts[i] = wi;
      lsum = fmaf(li, wi, lsum);
    }
    __syncthreads();
    for (int i = tp; i < cn; i += TP) {
      const float4 *ap = reinterpret_cast<const float4 *>(acc + static_cast<int64_t>(c0 + i) * D + 8 * ck);
      const float4 u = ap[0], v = ap[1];
      const float wi = wts[i];
      o[0] = fmaf(wi, u.x, o[0]);
      o[1] = fmaf(wi, u.y, o[1]);
      o[2] = fmaf(wi, u.z, o[2]);
      o[3] = fmaf(wi, u.w, o[3]);
      o[4] = fmaf(wi, v.x, o[4]);
      o[5] = fmaf(wi, v.y, o[5]);
      o[6] = fmaf(wi, v.z, o[6]);
      o[7] = fmaf(wi, v.w, o[7]);
    }
  }
  const float L = block_sum(lsum, red);
#pragma unroll
  for (int j = 0; j < 8; ++j) part[tp * D + 8 * ck + j] = o[j];
  __syncthreads();
  if (tid < D) {
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < TP; ++k) sum += part[k * D + tid];
    job.out[head * D + tid] = L > 0.0f ? sum / L : 0.0f;
  }
}

template <int D>
hipError_t launch_d(const DecodeJob &job, const WindowJob &wj, hipStream_t stream) {
  auto kern = wj.dtype == AQKV_BF16 ? combine_window_kernel<D, true> : combine_window_kernel<D, false>;
  kern<<<static_cast<unsigned>(job.n_slots * job.g), kThreads, 0, stream>>>(job, wj);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_window(const DecodeJob &job, const WindowJob &wj, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, wj, stream);
    case 128: return launch_d<128>(job, wj, stream);
    default: return launch_d<256>(job, wj, stream);
  }
}

}  // namespace aqkv
