// Matrix-core decode, host side and query packing (TurboQuant article §五
// estimator and §六 "the query is rotated and sketched once per query").
//
// decode_pack_kernel turns the prepared query of every head (q_rot = Pi q,
// q_sketch = S q) into the integer A operands of the score products in
// decode_fast.h, once per call instead of once per block:
//   kappa_A  Walsh coefficients of the codebook: c(idx) = c[0] + sum_A kappa_A
//            par_A(idx) over the non-empty subsets A of the index bits;
//   rows     per head: mse hi, mse lo (kappa_A q_rot), qjl hi, qjl lo (2 q_sk),
//            each value rounded to a 15-bit integer v = 128 hi + lo with a
//            per-head scale (max |value| / 16383) and split into int8 parts;
//   consts   per head: the two scales and the constant terms c[0] sum(q_rot)
//            and -sum(q_sk) of the score.
// When every even-size subset has kappa_A == 0 (an odd-symmetric codebook,
// as Lloyd-Max on the symmetric coordinate law gives) only the odd-size planes
// are laid out and the decoder skips the others; it reads that choice from
// qodd.
#include <math.h>

#include "decode_fast.h"

namespace aqkv {
namespace {

using fast::chunks_max;
using fast::heads_rb;

__global__ __launch_bounds__(256) void decode_pack_kernel(DecodeJob job, int ncmax) {
  __shared__ float kappa[8];
  __shared__ int s_odd;
  __shared__ float sig_mse[kMaxQPerKv], sig_qjl[kMaxQPerKv];
  const int D = job.d, W = job.w, m = job.m, G = job.g;
  const int RB = heads_rb(G), HC = D / 64, MC = m / 64;
  const int64_t slot = blockIdx.x, head0 = slot * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    int odd = 1;
    const int L = 1 << W;
    for (int a = 1; a < L; ++a) {
      // alpha_A = 2^-w sum_idx c[idx] prod_{k in A} (2 bit_k(idx) - 1), summed over
      // complementary pairs so odd-symmetric codebooks give exact zeros
      double acc = 0.0;
      for (int i = 0; i < L / 2; ++i) {
        const int j = L - 1 - i;
        double si = 1.0, sj = 1.0;
        for (int k = 0; k < W; ++k)
          if ((a >> k) & 1) {
            si *= ((i >> k) & 1) ? 1.0 : -1.0;
            sj *= ((j >> k) & 1) ? 1.0 : -1.0;
          }
        acc += static_cast<double>(job.centroids[i]) * si + static_cast<double>(job.centroids[j]) * sj;
      }
      const double sgn = (__popc(a) & 1) ? -1.0 : 1.0;   // (-1)^|A|
      const float kap = static_cast<float>(-2.0 * sgn * acc / L);
      kappa[a - 1] = kap;
      if (!(__popc(a) & 1) && kap != 0.0f) odd = 0;
    }
    s_odd = odd;
    job.qodd[slot] = odd;
  }
  __syncthreads();
  const int odd = s_odd;
  int planes[7];
  int np = 0;
  for (int a = 1; a < (1 << W); ++a)
    if (!odd || (__popc(a) & 1)) planes[np++] = a;
  // per head: max |kappa_A q_rot| over the laid-out planes, sum q_rot, max |2 q_sk|, sum q_sk
  for (int g = wave; g < G; g += 4) {
    float mx = 0.0f, sr = 0.0f, mq = 0.0f, sq = 0.0f;
    if (W > 0) {
      float km = 0.0f;
      for (int k = 0; k < np; ++k) km = fmaxf(km, fabsf(kappa[planes[k] - 1]));
      for (int j = lane; j < D; j += 64) {
        const float v = job.q_rot[(head0 + g) * D + j];
        sr += v;
        mx = fmaxf(mx, km * fabsf(v));
      }
    }
    for (int i = lane; i < m; i += 64) {
      const float v = job.q_sketch[(head0 + g) * m + i];
      sq += v;
      mq = fmaxf(mq, fabsf(2.0f * v));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off));
      mq = fmaxf(mq, __shfl_xor(mq, off));
      sr += __shfl_xor(sr, off);
      sq += __shfl_xor(sq, off);
    }
    if (lane == 0) {
      const float sm = mx > 0.0f ? mx / 16383.0f : 1.0f;
      const float sqj = mq > 0.0f ? mq / 16383.0f : 1.0f;
      sig_mse[g] = sm;
      sig_qjl[g] = sqj;
      float *hc = job.qconst + (head0 + g) * 4;
      hc[0] = sm;
      hc[1] = sqj;
      hc[2] = W > 0 ? job.centroids[0] * sr : 0.0f;
      hc[3] = -sq;
    }
  }
  __syncthreads();
  // operand bytes: dword e4 = ((r * ncmax + c) * 64 + lane) * 4 + i0 / 4; byte i of
  // lane (row, q) in chunk c is K-slot 16 q + i; row = 4 (g % 4) + t, g = 4 r + row / 4
  uint32_t *dst = reinterpret_cast<uint32_t *>(job.qpack + slot * static_cast<int64_t>(RB * ncmax * 1024));
  for (int e4 = tid; e4 < RB * ncmax * 256; e4 += 256) {
    const int rc = e4 / 256, rem = e4 % 256;
    const int r = rc / ncmax, c = rc % ncmax;
    const int l = rem / 4, i0 = (rem % 4) * 4;
    const int row = l % 16, q = l / 16;
    const int g = 4 * r + row / 4, t = row % 4;
    uint32_t word = 0;
    if (g < G) {
      const float *src = nullptr;
      float scl = 0.0f;
      if (c < np * HC) {
        if (t < 2) {
          // plane planes[c / HC], coordinates (D/4) q + 16 h .. + 15
          const int h = c % HC;
          src = job.q_rot + (head0 + g) * D + (D / 4) * q + 16 * h + i0;
          scl = kappa[planes[c / HC] - 1] / sig_mse[g];
        }
      } else if (c < np * HC + MC) {
        if (t >= 2) {
          // sketch rows 16 MC q + 16 h .. + 15
          const int h = c - np * HC;
          src = job.q_sketch + (head0 + g) * m + 16 * MC * q + 16 * h + i0;
          scl = 2.0f / sig_qjl[g];
        }
      }
      if (src) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          int v = static_cast<int>(rintf(src[bb] * scl));
          v = max(-16383, min(16383, v));
          const int part = (t & 1) ? (v & 127) : (v >> 7);
          word |= (static_cast<uint32_t>(part) & 0xffu) << (8 * bb);
        }
      }
    }
    dst[e4] = word;
  }
}

// compiled (d, w, m / 64) shapes of decode_fast_kernel, see decode_fast_d*.hip
bool fast_shape(int d, int w, int mc) {
  if (w >= 1 && w <= 3) return mc == d / 64;
  if (w != 0) return false;
  switch (d) {
    case 64: return mc >= 1 && mc <= 4;
    case 128: return mc == 1 || mc == 2 || mc == 3 || mc == 4 || mc == 6 || mc == 8;
    case 256: return mc == 2 || mc == 4 || mc == 6 || mc == 8;
    default: return false;
  }
}

}  // namespace

bool decode_mfma_supported(int d, int w, int g, int m, int vb) {
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  if (vb != 2 && vb != 4) return false;
  if (m % 64 || !fast_shape(d, w, m / 64)) return false;
  return fast::smem_of(d, w, m / 64, g, vb) <= 160 * 1024;
}

int decode_mfma_blocks_per_cu(int d, int w, int g, int m, int vb) {
  const int smem = fast::smem_of(d, w, m / 64, g, vb);
  int by_lds = (160 * 1024) / smem;
  const int by_regs = fast::waves_per_simd(d, g);   // blocks of 4 waves = waves per SIMD
  if (by_lds > by_regs) by_lds = by_regs;
  return by_lds < 1 ? 1 : by_lds;
}

size_t decode_mfma_pack_bytes(int d, int w, int g, int m, int64_t n_slots) {
  return static_cast<size_t>(n_slots) * heads_rb(g) * chunks_max(d, w, m) * 1024;
}

hipError_t launch_decode_mfma(const DecodeJob &job, hipStream_t stream) {
  if (job.n_slots > 0) {
    decode_pack_kernel<<<static_cast<unsigned>(job.n_slots), 256, 0, stream>>>(job, chunks_max(job.d, job.w, job.m));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  switch (job.d) {
    case 64: e = launch_decode_fast_d64(job, stream); break;
    case 128: e = launch_decode_fast_d128(job, stream); break;
    default: e = launch_decode_fast_d256(job, stream); break;
  }
  if (e != hipSuccess) return e;
  return launch_combine(job, stream);
}

}  // namespace aqkv
