// Key quantisation kernel (TurboQuant article §二 three-stage pipeline, §五
// quantize(); A-QJL article, section "QJL", for the pure-QJL mode w == 0).
//
// One block of 256 threads quantises a tile of TK tokens of one slot:
//   1. load the tile into LDS (bf16 or fp32 -> fp32), n = ||x|| per key;
//   2. (w > 0) y = Pi x / n, tiled fp32 product with Pi staged through LDS;
//      idx = number of boundaries below y_j; e = y - c[idx] (rotated residual
//      on the unit sphere); gamma = n ||e|| = ||x - n Pi^T c[idx]||;
//   3. z = P e with P = S Pi^T (w > 0), or z = S x (w == 0): signs of the
//      residual sketch, since S r = n P e; bit = z >= 0, forced to 1 for n == 0;
//   4. write the plane-major code rows, the sign rows and the two norms.
// Thread (kq, jq) of a 16x16 grid owns keys {kq + 16 a} and output rows
// {jq + 16 c} of a 128-row pass; the weight chunk is read from LDS by 16
// consecutive lanes (conflict-free), the key element is an LDS broadcast.
#include "internal.h"

namespace aqkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTK = 32;      // keys per block
constexpr int kKPT = kTK / 16;
constexpr int kKC = 16;      // reduction chunk staged in LDS
constexpr int kRB = 128;     // output rows per pass
constexpr int kRPT = kRB / 16;

// Bit rows are 32-bit words; element j = 4 i + k of a word sits at bit 8 k + i
// (byte k holds the elements j % 4 == k), so a decoder gets 4 consecutive
// elements as 4 operand bytes with one shift and one mask.
__device__ __forceinline__ int word_bit(int j) { return 8 * (j & 3) + (j >> 2); }

// Stage W[r0 .. r0+128)[k0 .. k0+16) transposed into wt[16][128] (rows >= nrows -> 0).
__device__ __forceinline__ void stage_chunk(float (*wt)[kRB], const float *__restrict__ W, int ld, int nrows,
                                            int r0, int k0) {
  const int rr = threadIdx.x >> 1;
  const int half = threadIdx.x & 1;
  const int r = r0 + rr;
  float v[8];
  if (r < nrows) {
    const float4 *p = reinterpret_cast<const float4 *>(W + static_cast<int64_t>(r) * ld + k0 + 8 * half);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) wt[8 * half + i][rr] = v[i];
}

// acc[a][c] += sum_k xs[kq + 16a][k] * W[r0 + jq + 16c][k] over k in [0, D).
template <int D>
__device__ __forceinline__ void tile_product(float (&acc)[kKPT][kRPT], const float (*xs)[D],
                                             float (*wt)[kRB], const float *__restrict__ W, int nrows,
                                             int r0) {
  const int kq = threadIdx.x >> 4, jq = threadIdx.x & 15;
#pragma unroll
  for (int a = 0; a < kKPT; ++a)
#pragma unroll
    for (int c = 0; c < kRPT; ++c) acc[a][c] = 0.0f;
  for (int k0 = 0; k0 < D; k0 += kKC) {
    __syncthreads();
    stage_chunk(wt, W, D, nrows, r0, k0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKC; ++kk) {
      float xv[kKPT];
#pragma unroll
      for (int a = 0; a < kKPT; ++a) xv[a] = xs[kq + 16 * a][k0 + kk];
#pragma unroll
      for (int c = 0; c < kRPT; ++c) {
        const float wv = wt[kk][jq + 16 * c];
#pragma unroll
        for (int a = 0; a < kKPT; ++a) acc[a][c] = fmaf(xv[a], wv, acc[a][c]);
      }
    }
  }
}

template <int D, int W, bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_keys_kernel(KeyJob job) {
  constexpr int kNB = (1 << W) - 1;  // boundaries
  constexpr int kPass1 = (D + kRB - 1) / kRB;
  __shared__ float xs[kTK][D];
  __shared__ float wt[kKC][kRB];
  __shared__ uint8_t idxs[W > 0 ? kTK : 1][W > 0 ? D : 1];
  __shared__ uint32_t sbits[kTK][kMaxSketch / 32];
  __shared__ float nrm[kTK], gam[kTK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kq = tid >> 4, jq = tid & 15;
  const int64_t tiles = (job.n_tokens + kTK - 1) / kTK;
  const int64_t s = blockIdx.x / tiles;
  const int64_t t0 = (blockIdx.x % tiles) * kTK;
  const int nk = static_cast<int>(min<int64_t>(kTK, job.n_tokens - t0));
  const int m = job.m;
  const int64_t b = s / job.heads, h = s % job.heads;
  const int64_t base = b * job.batch_stride + h * job.head_stride;

  // 1. load the tile (8 elements per step)
  for (int e = tid; e < kTK * D / 8; e += kThreads) {
    const int key = e / (D / 8), c8 = (e % (D / 8)) * 8;
    float v[8];
    if (key < nk) {
      const int64_t off = base + (t0 + key) * job.token_stride + c8;
      if (BF16) {
        const uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(job.k) + off);
        const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] = bf16_to_f32(wv[j] & 0xffffu);
          v[2 * j + 1] = bf16_to_f32(wv[j] >> 16);
        }
      } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(job.k) + off);
        const float4 a = p[0], c = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[key][c8 + j] = v[j];
  }
  for (int e = tid; e < kTK * (kMaxSketch / 32); e += kThreads) sbits[e / (kMaxSketch / 32)][e % (kMaxSketch / 32)] = 0u;
  __syncthreads();

  // norms: one wave per key, fixed reduction order
  for (int key = wave; key < kTK; key += kThreads / 64) {
    float acc = 0.0f;
    for (int j = lane; j < D; j += 64) acc = fmaf(xs[key][j], xs[key][j], acc);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) nrm[key] = sqrtf(acc);
  }
  __syncthreads();

  if constexpr (W > 0) {
    // 2. y = Pi x / n, all passes kept in registers until xs may be overwritten
    float y[kPass1][kKPT][kRPT];
    for (int p = 0; p < kPass1; ++p) tile_product<D>(y[p], xs, wt, job.rotation, D, p * kRB);
    float bnd[kNB > 0 ? kNB : 1], cen[kNB + 1];
#pragma unroll
    for (int i = 0; i < kNB; ++i) bnd[i] = job.boundaries[i];
#pragma unroll
    for (int i = 0; i <= kNB; ++i) cen[i] = job.centroids[i];
    __syncthreads();  // every thread is done reading xs
#pragma unroll
    for (int p = 0; p < kPass1; ++p)
#pragma unroll
      for (int a = 0; a < kKPT; ++a) {
        const int key = kq + 16 * a;
        const float n = nrm[key];
#pragma unroll
        for (int c = 0; c < kRPT; ++c) {
          const int j = p * kRB + jq + 16 * c;
          if (j < D) {
            const float yv = n > 0.0f ? y[p][a][c] / n : 0.0f;
            int idx = 0;
            float cv = cen[0];
#pragma unroll
            for (int i = 0; i < kNB; ++i)
              if (yv > bnd[i]) { idx = i + 1; cv = cen[i + 1]; }
            xs[key][j] = yv - cv;                 // rotated residual e
            idxs[key][j] = static_cast<uint8_t>(idx);
          }
        }
      }
    __syncthreads();
    for (int key = wave; key < kTK; key += kThreads / 64) {
      float acc = 0.0f;
      for (int j = lane; j < D; j += 64) acc = fmaf(xs[key][j], xs[key][j], acc);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) gam[key] = nrm[key] * sqrtf(acc);
    }
  }

  // 3. residual sketch signs: z = P e (w > 0) or S x (w == 0), 128 rows per pass
  for (int r0 = 0; r0 < m; r0 += kRB) {
    float z[kKPT][kRPT];
    tile_product<D>(z, xs, wt, job.proj, m, r0);
#pragma unroll
    for (int a = 0; a < kKPT; ++a) {
      const int key = kq + 16 * a;
      const bool zero_key = !(nrm[key] > 0.0f);
#pragma unroll
      for (int c = 0; c < kRPT; ++c) {
        const int i = r0 + jq + 16 * c;
        if (i < m && (z[a][c] >= 0.0f || zero_key)) atomicOr(&sbits[key][i >> 5], 1u << word_bit(i & 31));
      }
    }
  }
  __syncthreads();

  // 4. write rows
  const int64_t row0 = s * job.capacity + job.token_offset + t0;
  if constexpr (W > 0) {
    constexpr int kWordsPerPlane = D / 32;
    for (int e = tid; e < nk * W * kWordsPerPlane; e += kThreads) {
      const int key = e / (W * kWordsPerPlane);
      const int r = e % (W * kWordsPerPlane);
      const int p = r / kWordsPerPlane, wi = r % kWordsPerPlane;
      uint32_t word = 0;
#pragma unroll 8
      for (int l = 0; l < 32; ++l) word |= static_cast<uint32_t>((idxs[key][32 * wi + l] >> p) & 1) << word_bit(l);
      reinterpret_cast<uint32_t *>(job.codes + (row0 + key) * (W * D / 8) + p * (D / 8))[wi] = word;
    }
  }
  const int swords = m / 32;
  for (int e = tid; e < nk * swords; e += kThreads) {
    const int key = e / swords, wi = e % swords;
    reinterpret_cast<uint32_t *>(job.signs + (row0 + key) * (m / 8))[wi] = sbits[key][wi];
  }
  if (tid < nk) {
    job.norm[row0 + tid] = nrm[tid];
    if constexpr (W > 0) job.rnorm[row0 + tid] = gam[tid];
  }
}

template <int D, int W>
hipError_t launch_dw(const KeyJob &job, hipStream_t stream) {
  const int64_t tiles = (job.n_tokens + kTK - 1) / kTK;
  const dim3 grid(static_cast<unsigned>(tiles * job.n_slots));
  if (job.dtype == AQKV_BF16)
    quantize_keys_kernel<D, W, true><<<grid, kThreads, 0, stream>>>(job);
  else
    quantize_keys_kernel<D, W, false><<<grid, kThreads, 0, stream>>>(job);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const KeyJob &job, hipStream_t stream) {
  switch (job.w) {
    case 0: return launch_dw<D, 0>(job, stream);
    case 1: return launch_dw<D, 1>(job, stream);
    case 2: return launch_dw<D, 2>(job, stream);
    default: return launch_dw<D, 3>(job, stream);
  }
}

}  // namespace

hipError_t launch_quantize_keys(const KeyJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
