// Decode attention on the packed cache (TurboQuant article §五 estimator, §六
// fused decode attention with online softmax; A-QJL pure-QJL keys).
//
// Split-K over the sequence: block (split, slot) walks its token range in
// chunks of 256 tokens and keeps, for each of the G query heads that share the
// slot's kv head, the running maximum, the running sum and the un-normalised
// output.  Per chunk:
//   A. one thread per token decodes its code planes and sign row and scores
//      all G heads against the query-side vectors held in LDS:
//        s = n <q_rot, c[idx]> + sqrt(pi/2)/m * gamma * <q_sk, +-1>;
//   B. one wave per head updates the online softmax (base-2 exponentials);
//   C. one thread per (head, channel) accumulates p * (code * scale + min)
//      from the chunk's value rows staged in LDS.
// A second kernel merges the per-split partials.  No fp key is formed.
#include <math.h>

#include "internal.h"

namespace aqkv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;
constexpr float kLog2e = 1.4426950408889634f;

// bit of element j (0..31) in a 32-bit bit-row word: 8 (j % 4) + j / 4
__device__ __forceinline__ int word_bit(int j) { return 8 * (j & 3) + (j >> 2); }

template <int D, int W, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeJob job) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int m = job.m, vb = job.vb;
  constexpr int kGroups = D / 32;
  const int vwords = D * vb / 32;                // value code words per row
  float *qr = reinterpret_cast<float *>(smem);                   // [G][D]
  float *qs = qr + (W > 0 ? G * D : 0);                          // [G][m]
  float *sc = qs + G * m;                                        // [G][kChunk]
  float *vsc = sc + G * kChunk;                                  // [kChunk][kGroups]
  float *vmn = vsc + kChunk * kGroups;                           // [kChunk][kGroups]
  float *stat = vmn + kChunk * kGroups;                          // [G][3]: max, sum, factor
  uint32_t *vcw = reinterpret_cast<uint32_t *>(stat + 4 * G);    // [kChunk][vwords]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slot = blockIdx.x / job.n_split;
  const int split = static_cast<int>(blockIdx.x % job.n_split);
  const int64_t t_begin = static_cast<int64_t>(split) * job.split_tokens;
  const int64_t t_end = min<int64_t>(job.context, t_begin + job.split_tokens);
  const int64_t head0 = slot * G;                 // first global query head of this slot
  const float kappa = 1.2533141373155003f / static_cast<float>(m);   // sqrt(pi/2) / m
  const float lscale = job.softmax_scale * kLog2e;

  for (int i = tid; i < G * D && W > 0; i += kThreads) qr[i] = job.q_rot[head0 * D + i];
  for (int i = tid; i < G * m; i += kThreads) qs[i] = job.q_sketch[head0 * m + i];
  if (tid < G) {
    stat[4 * tid + 0] = -INFINITY;
    stat[4 * tid + 1] = 0.0f;
    stat[4 * tid + 2] = 0.0f;
  }
  float cen[W > 0 ? (1 << W) : 1];
#pragma unroll
  for (int i = 0; i < (W > 0 ? (1 << W) : 0); ++i) cen[i] = job.centroids[i];

  constexpr int kPairs = (G * D + kThreads - 1) / kThreads;
  float acc[kPairs];
#pragma unroll
  for (int i = 0; i < kPairs; ++i) acc[i] = 0.0f;
  __syncthreads();

  const int code_bytes = W * D / 8, sign_bytes = m / 8;
  for (int64_t c0 = t_begin; c0 < t_end; c0 += kChunk) {
    const int64_t t = c0 + tid;
    const bool valid = t < t_end;
    const int64_t row = slot * job.capacity + t;

    // stage this thread's share of the chunk's value-code blocks (whole 32-token
    // blocks: a block's words hold codes of all its tokens); past the end -> 0
    const bool block_valid = c0 + (tid & ~31) < t_end;
    for (int i = 0; i < vwords; ++i)
      vcw[tid * vwords + i] = block_valid ? reinterpret_cast<const uint32_t *>(job.vcodes + rec_row(row, D * vb / 8, job.rec))[i] : 0u;
    const bool sf = job.sf != 0;   // half side information (else fp32)
    for (int i = 0; i < kGroups; ++i) {
      const uint8_t *side = job.vside + rec_row(row & ~int64_t(31), 0, job.rec);
      vsc[tid * kGroups + i] = valid ? load_side(side, side_index(i, static_cast<int>(row & 31), 0), sf) : 0.0f;
      vmn[tid * kGroups + i] = valid ? load_side(side, side_index(i, static_cast<int>(row & 31), 1), sf) : 0.0f;
    }

    // A. scores
    float s_acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s_acc[g] = 0.0f;
    if (valid) {
      const int64_t rb = rec_row(row & ~int64_t(31), 0, job.rec), ri = row & 31;
      const float n = load_side(job.norm + rb, ri, sf);
      const float gamma = W > 0 ? load_side(job.rnorm + rb, ri, sf) : n;
      float mse[G], qjl[G];
#pragma unroll
      for (int g = 0; g < G; ++g) { mse[g] = 0.0f; qjl[g] = 0.0f; }
      if constexpr (W > 0) {
        const uint32_t *cw = reinterpret_cast<const uint32_t *>(job.codes + rec_row(row, code_bytes, job.rec));
        for (int wi = 0; wi < D / 32; ++wi) {
          uint32_t pl[W];
#pragma unroll
          for (int p = 0; p < W; ++p) pl[p] = cw[p * (D / 32) + wi];
          float cv[32];
#pragma unroll
          for (int l = 0; l < 32; ++l) {
            int idx = 0;
#pragma unroll
            for (int p = 0; p < W; ++p) idx |= static_cast<int>((pl[p] >> word_bit(l)) & 1u) << p;
            float v = cen[0];
#pragma unroll
            for (int k = 1; k < (1 << W); ++k) v = (idx == k) ? cen[k] : v;
            cv[l] = v;
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float4 *q4 = reinterpret_cast<const float4 *>(qr + g * D + 32 * wi);
#pragma unroll
            for (int l4 = 0; l4 < 8; ++l4) {
              const float4 q = q4[l4];
              mse[g] = fmaf(q.x, cv[4 * l4 + 0], mse[g]);
              mse[g] = fmaf(q.y, cv[4 * l4 + 1], mse[g]);
              mse[g] = fmaf(q.z, cv[4 * l4 + 2], mse[g]);
              mse[g] = fmaf(q.w, cv[4 * l4 + 3], mse[g]);
            }
          }
        }
      }
      const uint32_t *sw = reinterpret_cast<const uint32_t *>(job.signs + rec_row(row, sign_bytes, job.rec));
      for (int wi = 0; wi < m / 32; ++wi) {
        const uint32_t bits = sw[wi];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float4 *q4 = reinterpret_cast<const float4 *>(qs + g * m + 32 * wi);
#pragma unroll
          for (int l4 = 0; l4 < 8; ++l4) {
            const float4 q = q4[l4];
            const int l = 4 * l4;
            qjl[g] += ((bits >> word_bit(l + 0)) & 1u) ? q.x : -q.x;
            qjl[g] += ((bits >> word_bit(l + 1)) & 1u) ? q.y : -q.y;
            qjl[g] += ((bits >> word_bit(l + 2)) & 1u) ? q.z : -q.z;
            qjl[g] += ((bits >> word_bit(l + 3)) & 1u) ? q.w : -q.w;
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s_acc[g] = n * mse[g] + kappa * gamma * qjl[g];
        if (job.scores) job.scores[(head0 + g) * job.context + t] = s_acc[g];
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g * kChunk + tid] = valid ? s_acc[g] * lscale : -INFINITY;
    __syncthreads();

    // B. online softmax, one wave per head
    for (int g = wave; g < G; g += kThreads / 64) {
      float v[kChunk / 64];
      float cmax = -INFINITY;
#pragma unroll
      for (int k = 0; k < kChunk / 64; ++k) {
        v[k] = sc[g * kChunk + lane + 64 * k];
        cmax = fmaxf(cmax, v[k]);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
      const float m_old = stat[4 * g + 0];
      const float m_new = fmaxf(m_old, cmax);
      const float f = (m_old == -INFINITY) ? 0.0f : exp2f(m_old - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int k = 0; k < kChunk / 64; ++k) {
        const float p = (v[k] == -INFINITY) ? 0.0f : exp2f(v[k] - m_new);
        sc[g * kChunk + lane + 64 * k] = p;
        psum += p;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off);
      if (lane == 0) {
        stat[4 * g + 0] = m_new;
        stat[4 * g + 1] = stat[4 * g + 1] * f + psum;
        stat[4 * g + 2] = f;
      }
    }
    __syncthreads();

    // C. values: thread owns (head, channel) pairs
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int pi = tid + i * kThreads;
      if (pi < G * D) {
        const int g = pi / D, j = pi % D;
        // 32-token block layout: channel j = 32 grp + 16 hh + n, token 4 ii + r of a block
        const int grp = j >> 5, hh = (j >> 4) & 1, n = j & 15;
        const uint32_t mask = (1u << vb) - 1u;
        float a = acc[i] * stat[4 * g + 2];
        const float *pg = sc + g * kChunk;
        for (int tt = 0; tt < kChunk; ++tt) {
          const int r = tt & 3, ii = (tt >> 2) & 7;
          const int word = (tt >> 5) * (32 * vwords) +
                           (vb == 2 ? (16 * grp + n) * 4 + r : ((16 * grp + n) * 4 + r) * 2 + hh);
          const int shift = vb == 2 ? 8 * hh + 16 * (ii & 1) + 2 * (ii >> 1) : 16 * (ii & 1) + 4 * (ii >> 1);
          const float code = static_cast<float>((vcw[word] >> shift) & mask);
          const float vh = fmaf(code, vsc[tt * kGroups + grp], vmn[tt * kGroups + grp]);
          a = fmaf(pg[tt], vh, a);
        }
        acc[i] = a;
      }
    }
    __syncthreads();
  }

  // partials
  const int64_t pbase = static_cast<int64_t>(job.part_stride);
#pragma unroll
  for (int i = 0; i < kPairs; ++i) {
    const int pi = tid + i * kThreads;
    if (pi < G * D) {
      const int g = pi / D, j = pi % D;
      job.part_acc[((head0 + g) * pbase + split) * D + j] = acc[i];
    }
  }
  if (tid < G) {
    job.part_ml[((head0 + tid) * pbase + split) * 2 + 0] = stat[4 * tid + 0];
    job.part_ml[((head0 + tid) * pbase + split) * 2 + 1] = stat[4 * tid + 1];
  }
}

// Merge the split partials of one query head: M = max_i m_i, weights
// w_i = 2^(m_i - M) (0 for empty splits), out = sum_i w_i acc_i / sum_i w_i l_i.
// The weights go to LDS (1024 splits per pass); 256 / d threads share a channel,
// each summing every (256 / d)-th split.  The thread's first (m, l) pair and its
// first kPre partial outputs are loaded at the start, together: the partials do not
// depend on the weights, and one memory latency then covers the whole merge of
// the usual split counts.  Loads are branch-free (clamped index, value dropped),
// and the sums run in the same order as without the prefetch.
__global__ __launch_bounds__(256) void combine_kernel(DecodeJob job) {
  constexpr int kPre = 16;
  __shared__ float wts[1024];
  __shared__ float red[256];
  const int64_t head = blockIdx.x;
  const int d = job.d, ns = job.part_stride, tid = threadIdx.x;
  const float *ml = job.part_ml + head * ns * 2;
  const float *acc = job.part_acc + head * ns * d;
  const int P = 256 / d;                  // threads per channel
  const int j = tid % d, p = tid / d;
  const int i0 = min(tid, ns - 1);
  const float m0 = ml[2 * i0], l0 = ml[2 * i0 + 1];
  float pre[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) pre[k] = acc[static_cast<int64_t>(min(p + P * k, ns - 1)) * d + j];
  // M over the non-empty splits
  float mx = -INFINITY;
  if (tid < ns && l0 > 0.0f) mx = fmaxf(mx, m0);
  for (int i = tid + 256; i < ns; i += 256)
    if (ml[2 * i + 1] > 0.0f) mx = fmaxf(mx, ml[2 * i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float o = 0.0f, lsum = 0.0f;
  for (int c0 = 0; c0 < ns; c0 += 1024) {
    const int cn = min(1024, ns - c0);
    for (int i = tid; i < cn; i += 256) {
      const bool first = c0 == 0 && i == tid;
      const float l = first ? l0 : ml[2 * (c0 + i) + 1];
      const float m = first ? m0 : ml[2 * (c0 + i)];
      const float w = l > 0.0f ? exp2f(m - mx) : 0.0f;
      wts[i] = w;
      lsum = fmaf(l, w, lsum);
    }
    __syncthreads();
    int i = p;
    if (c0 == 0) {
#pragma unroll
      for (int k = 0; k < kPre; ++k, i += P)
        if (i < cn) o = fmaf(pre[k], wts[i], o);
    }
#pragma unroll 8
    for (; i < cn; i += P) o = fmaf(acc[static_cast<int64_t>(c0 + i) * d + j], wts[i], o);
    __syncthreads();
  }
  // sum of the l weights over the block, partial outputs over the P threads of a channel
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  red[tid] = o;
  __syncthreads();
  __shared__ float lred[4];
  if ((tid & 63) == 0) lred[tid >> 6] = lsum;
  __syncthreads();
  if (p == 0) {
    float t = 0.0f;
    for (int k = 0; k < P; ++k) t += red[k * d + j];
    const float L = lred[0] + lred[1] + lred[2] + lred[3];
    job.out[head * d + j] = L > 0.0f ? t / L : 0.0f;
  }
}

size_t smem_bytes(int d, int w, int g, int m, int vb) {
  return sizeof(float) * ((w > 0 ? g * d : 0) + g * m + g * kChunk + 2 * kChunk * (d / 32) + 4 * g) +
         sizeof(uint32_t) * kChunk * (d * vb / 32);
}

template <int D, int W, int G>
hipError_t launch_dwg(const DecodeJob &job, hipStream_t stream) {
  const size_t smem = smem_bytes(D, W, G, job.m, job.vb);
  if (smem > 64 * 1024) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(job.n_split * job.n_slots));
  decode_kernel<D, W, G><<<grid, kThreads, smem, stream>>>(job);
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_dw(const DecodeJob &job, hipStream_t stream) {
  switch (job.g) {
    case 1: return launch_dwg<D, W, 1>(job, stream);
    case 2: return launch_dwg<D, W, 2>(job, stream);
    case 4: return launch_dwg<D, W, 4>(job, stream);
    case 8: return launch_dwg<D, W, 8>(job, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(const DecodeJob &job, hipStream_t stream) {
  switch (job.w) {
    case 0: return launch_dw<D, 0>(job, stream);
    case 1: return launch_dw<D, 1>(job, stream);
    case 2: return launch_dw<D, 2>(job, stream);
    default: return launch_dw<D, 3>(job, stream);
  }
}

}  // namespace

hipError_t launch_combine(const DecodeJob &job, hipStream_t stream) {
  combine_kernel<<<static_cast<unsigned>(job.n_slots * job.g), 256, 0, stream>>>(job);
  return hipGetLastError();
}

bool decode_supported(int d, int w, int g, int m, int vb) {
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  return smem_bytes(d, w, g, m, vb) <= 64 * 1024;
}

hipError_t launch_decode(const DecodeJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
