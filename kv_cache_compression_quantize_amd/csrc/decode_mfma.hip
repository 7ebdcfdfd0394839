// Decode attention on the packed cache with CDNA4 matrix cores
// (TurboQuant article §五 estimator, §六 fused decode with online softmax;
// A-QJL pure-QJL keys).
//
// Scores as integer matrix products on the packed bits.  For a codebook c of
// 2^w levels, c(idx) = c[0] + sum_A kappa_A par_A(idx) over the non-empty
// subsets A of the w index bits, par_A = xor of those bits (a Walsh transform
// of the codebook; for the odd-symmetric Lloyd-Max codebooks only the odd
// subsets are non-zero and only those planes are processed).  Hence
//   <q_rot, c[idx_t]>   = c[0] sum(q_rot) + sum_A kappa_A <q_rot, par_A(t)>
//   <q_sk, 2 bits_t - 1> = 2 <q_sk, bits_t> - sum(q_sk)
// and every score is a fixed combination of dot products between query rows
// and {0,1} bit-planes of the cached keys.  The query side (kappa_A q_rot and
// 2 q_sk per head) is quantised once per block to 15-bit integers split into
// int8 hi/lo parts; v_mfma_i32_16x16x64_i8 contracts 64 coordinates of 16
// tokens for 16 rows = 4 heads x {mse hi, mse lo, qjl hi, qjl lo} with exact
// integer accumulation.  A key bit becomes an int8 {0,1} operand byte
// (4 bits per shift, multiply, mask); no fp key is formed.
//
// Values: out[g] = sum_t p_t (code_t scale_t + min_t).  The f16 operand
// 1 + code/4 (exact: the code sits in mantissa bits 8..9) is built with one
// shift and one mask from the 32-token block word that holds 8 tokens' codes
// of one channel; the token weights a_t = p_t scale_t are split into f16
// hi + lo and v_mfma_f32_16x16x32_f16 accumulates sum_t a_t (1 + code_t/4)
// over 32 tokens; sum_t p_t (min_t - 4 scale_t) is added at the end.
//
// Work: block (slot, split) of 4 waves; each wave walks 32-token tiles of
// the block's range (interleaved across waves) with its own online-softmax
// state.  Tile bytes go global -> LDS with global_load_lds_dwordx4 into a
// double buffer, so the next tile streams in while this one is computed.  The
// waves merge in LDS; the split-combine kernel merges the splits.
#include <math.h>

#include "internal.h"

namespace aqkv {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTT = 32;          // tokens per wave tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;    // keep the running max unless a tile exceeds it by 2^8
constexpr int kMaxG = 8;

// per-block constants of the packed query (LDS)
struct QConst {
  float sig_mse[kMaxG], sig_qjl[kMaxG], c_mse[kMaxG], c_qjl[kMaxG];
  float kappa[8];
  uint32_t plane_mask;
  float c0;
  uint32_t pad[22];
};
static_assert(sizeof(QConst) == 256, "constants block");

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bit-row words hold element j = 4 i + k at bit 8 k + i, so (x >> i) & 0x01010101
// is elements 4i .. 4i+3 as int8 {0,1} bytes.  Half hf of a word (elements
// 16 hf .. 16 hf + 15) -> the 16 operand bytes of one K-chunk.
__device__ __forceinline__ v4i spread_half(uint32_t x, int hf) {
  v4i r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = static_cast<int>((x >> (4 * hf + k)) & 0x01010101u);
  return r;
}

// Wave-wide asynchronous copy of `bytes` (multiple of 16) contiguous global
// bytes to LDS; 16-byte pieces at or past `valid_bytes` are not loaded.
__device__ __forceinline__ void async_copy(const uint8_t *gsrc, uint8_t *ldst, int bytes, int valid_bytes, int lane) {
  for (int off = 0; off < bytes; off += 1024) {
    const int mine = off + 16 * lane;
    if (mine < valid_bytes)
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(gsrc + mine), (lds_u8 *)(ldst + off), 16, 0, 0);
  }
}

// Query rows of the block's G heads as MFMA A operands in LDS:
// qa[((chunk * RB + rb) * 4 + q) * 256 + row * 16 + i] is byte i of lane
// (row, q); row = 4 (g % 4) + t with t = mse hi, mse lo, qjl hi, qjl lo and
// g = 4 rb + row / 4.  Chunks: the active xor planes in order (D/64 each), then
// the m/64 sign chunks.  K-slot i of lane group q in chunk h of a plane is
// coordinate (D/4) q + 16 h + i (sign chunks: (m/4) q + 16 h + i).
template <int D, int W, int G>
__device__ void pack_query(const DecodeJob &job, int64_t head0, uint8_t *qa, QConst *qc) {
  constexpr int RB = (G + 3) / 4;
  constexpr int kPlanes = W > 0 ? (1 << W) - 1 : 0;
  const int m = job.m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    unsigned mask = 0;
    if (W > 0) {
      constexpr int L = 1 << W;
      for (int A = 1; A <= kPlanes; ++A) {
        // alpha_A = 2^-w sum_idx c[idx] prod_{k in A} (2 bit_k(idx) - 1), summed over
        // complementary pairs so odd-symmetric codebooks give exact zeros
        double acc = 0.0;
        for (int i = 0; i < L / 2; ++i) {
          const int j = L - 1 - i;
          double si = 1.0, sj = 1.0;
          for (int k = 0; k < W; ++k)
            if ((A >> k) & 1) {
              si *= ((i >> k) & 1) ? 1.0 : -1.0;
              sj *= ((j >> k) & 1) ? 1.0 : -1.0;
            }
          acc += static_cast<double>(job.centroids[i]) * si + static_cast<double>(job.centroids[j]) * sj;
        }
        const double sgn = (__popc(A) & 1) ? -1.0 : 1.0;   // (-1)^|A|
        const float kap = static_cast<float>(-2.0 * sgn * acc / L);
        qc->kappa[A - 1] = kap;
        if (kap != 0.0f) mask |= 1u << A;
      }
      qc->c0 = job.centroids[0];
    }
    qc->plane_mask = mask;
  }
  __syncthreads();
  const unsigned mask = qc->plane_mask;
  // per head: max |kappa_A q_rot|, sum q_rot, max |2 q_sk|, sum q_sk
  for (int g = wave; g < G; g += kWaves) {
    float mx = 0.0f, sr = 0.0f, mq = 0.0f, sq = 0.0f;
    if constexpr (W > 0) {
      float km = 0.0f;
      for (int A = 1; A <= kPlanes; ++A)
        if ((mask >> A) & 1) km = fmaxf(km, fabsf(qc->kappa[A - 1]));
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
      qc->sig_mse[g] = mx > 0.0f ? mx / 16383.0f : 1.0f;
      qc->sig_qjl[g] = mq > 0.0f ? mq / 16383.0f : 1.0f;
      qc->c_mse[g] = W > 0 ? qc->c0 * sr : 0.0f;
      qc->c_qjl[g] = -sq;
    }
  }
  __syncthreads();
  int active[kPlanes > 0 ? kPlanes : 1];
  int n_active = 0;
#pragma unroll
  for (int A = 1; A <= kPlanes; ++A)
    if ((mask >> A) & 1) active[n_active++] = A;
  const int mse_chunks = n_active * (D / 64);
  const int chunks = mse_chunks + m / 64;
  for (int e4 = tid; e4 < chunks * RB * 256; e4 += kThreads) {   // 4 bytes per step
    const int chunk = e4 / (RB * 256);
    const int rem = e4 % (RB * 256);
    const int rb = rem / 256;
    const int q = (rem % 256) / 64;
    const int row = (rem % 64) / 4;
    const int i0 = (rem % 4) * 4;
    const int g = 4 * rb + row / 4, t = row % 4;
    uint32_t word = 0;
    if (g < G) {
      const bool mse_chunk = chunk < mse_chunks;
      const bool in_part = mse_chunk ? (t < 2) : (t >= 2);
      if (in_part) {
        float scl;
        const float *src;
        if (mse_chunk) {
          int A = 1;
#pragma unroll
          for (int k = 0; k < (kPlanes > 0 ? kPlanes : 1); ++k)
            if (k == chunk / (D / 64)) A = active[k];
          const int h = chunk % (D / 64);
          src = job.q_rot + (head0 + g) * D + (D / 4) * q + 16 * h;
          scl = qc->kappa[A - 1] / qc->sig_mse[g];
        } else {
          const int h = chunk - mse_chunks;
          src = job.q_sketch + (head0 + g) * m + (m / 4) * q + 16 * h;
          scl = 2.0f / qc->sig_qjl[g];
        }
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          int v = static_cast<int>(rintf(src[i0 + bb] * scl));
          v = max(-16383, min(16383, v));
          const int part = (t & 1) ? (v & 127) : (v >> 7);
          word |= (static_cast<uint32_t>(part) & 0xffu) << (8 * bb);
        }
      }
    }
    reinterpret_cast<uint32_t *>(qa)[e4] = word;
  }
}

template <int D, int W, int G, int VB>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeJob job, int n_chunks_max) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int RB = (G + 3) / 4;
  constexpr int kGroups = D / 32;
  constexpr int kPlanes = W > 0 ? (1 << W) - 1 : 0;
  constexpr int CB = W * D / 8;          // key code bytes per token
  constexpr int VBY = D * VB / 8;        // value code bytes per token
  constexpr float kMag = VB == 2 ? 4.0f : 16.0f;
  constexpr int kPairs = (G * kGroups + 3) / 4;   // (head, group) pairs per lane (4 lane groups)
  const int m = job.m;
  const int SB = m / 8;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, q = lane >> 4;
  const int64_t slot = blockIdx.x / job.n_split;
  const int split = static_cast<int>(blockIdx.x % job.n_split);
  const int64_t t_begin = static_cast<int64_t>(split) * job.split_tokens;
  const int64_t t_end = min<int64_t>(job.context, t_begin + job.split_tokens);
  const int64_t head0 = slot * G;

  // ---- LDS carve
  uint8_t *qa = smem;                                                    // [n_chunks][RB][4][16][16]
  QConst *qc = reinterpret_cast<QConst *>(smem + n_chunks_max * RB * 1024);
  const int o_signs = kTT * CB;
  const int o_norm = o_signs + kTT * SB;
  const int o_rnorm = o_norm + kTT * 4;
  const int o_vcodes = o_rnorm + (W > 0 ? kTT * 4 : 0);
  const int o_vscale = o_vcodes + kTT * VBY;
  const int o_vmin = o_vscale + kTT * kGroups * 4;
  const int tile_bytes = o_vmin + kTT * kGroups * 4;
  constexpr int kAvalBytes = kGroups * 4 * 16 * 16;                      // [grp][q][16 rows][8 f16]
  const int wave_bytes = 2 * tile_bytes + G * kTT * 4 + kAvalBytes;
  uint8_t *wbase = smem + n_chunks_max * RB * 1024 + 256 + wave * wave_bytes;
  float *P = reinterpret_cast<float *>(wbase + 2 * tile_bytes);                            // [G][kTT]
  uint8_t *aval = wbase + 2 * tile_bytes + G * kTT * 4;

  // ---- query operands, zero value-weight rows (rows >= 2G stay zero)
  pack_query<D, W, G>(job, head0, qa, qc);
  for (int i = lane; i < kAvalBytes / 16; i += 64) reinterpret_cast<uint4 *>(aval)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const unsigned pmask = qc->plane_mask;
  const float kappa_qjl = 1.2533141373155003f / static_cast<float>(m);   // sqrt(pi/2) / m
  const float lscale = job.softmax_scale * kLog2e;

  // ---- per-wave state
  float m_ref[RB], l_part[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) { m_ref[r] = -INFINITY; l_part[r] = 0.0f; }
  v4f cval[2 * kGroups];
#pragma unroll
  for (int i = 0; i < 2 * kGroups; ++i) cval[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float corr[kPairs];
#pragma unroll
  for (int i = 0; i < kPairs; ++i) corr[i] = 0.0f;

  const int64_t n_tiles = (t_end > t_begin) ? (t_end - t_begin + kTT - 1) / kTT : 0;
  auto issue = [&](int64_t tile, int bsel) {
    const int64_t t0 = t_begin + tile * kTT;
    const int nt = static_cast<int>(min<int64_t>(kTT, t_end - t0));
    const int64_t row0 = slot * job.capacity + t0;
    uint8_t *b = wbase + bsel * tile_bytes;
    if constexpr (W > 0) async_copy(job.codes + row0 * CB, b, kTT * CB, nt * CB, lane);
    async_copy(job.signs + row0 * SB, b + o_signs, kTT * SB, nt * SB, lane);
    async_copy(reinterpret_cast<const uint8_t *>(job.norm + row0), b + o_norm, kTT * 4, nt * 4, lane);
    if constexpr (W > 0)
      async_copy(reinterpret_cast<const uint8_t *>(job.rnorm + row0), b + o_rnorm, kTT * 4, nt * 4, lane);
    // the value codes of a 32-token block interleave all its tokens: copy it whole
    async_copy(job.vcodes + row0 * VBY, b + o_vcodes, kTT * VBY, kTT * VBY, lane);
    async_copy(reinterpret_cast<const uint8_t *>(job.vscale + row0 * kGroups), b + o_vscale, kTT * kGroups * 4,
               nt * kGroups * 4, lane);
    async_copy(reinterpret_cast<const uint8_t *>(job.vmin + row0 * kGroups), b + o_vmin, kTT * kGroups * 4,
               nt * kGroups * 4, lane);
  };

  int bsel = 0;
  int64_t tile = wave;
  if (tile < n_tiles) issue(tile, 0);
  for (; tile < n_tiles; tile += kWaves) {
    __builtin_amdgcn_s_waitcnt(0);       // this tile's bytes have landed in LDS
    compiler_fence();
    if (tile + kWaves < n_tiles) issue(tile + kWaves, bsel ^ 1);
    const uint8_t *tb = wbase + bsel * tile_bytes;
    const int64_t t0 = t_begin + tile * kTT;
    const int nt = static_cast<int>(min<int64_t>(kTT, t_end - t0));

    // ---------------- scores: 2 column tiles of 16 tokens
    float logit[2][RB];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int tok = 16 * ct + n16;
      v4i acc[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[r] = v4i{0, 0, 0, 0};
      int chunk = 0;
      if constexpr (W > 0) {
        // this lane's coordinates (D/4) q .. (D/4) q + D/4 - 1 of each index plane,
        // as the 32-bit words that hold them (D = 64: half of one word)
        constexpr int kWordsPerLane = D >= 128 ? D / 128 : 1;
        uint32_t pl[W > 0 ? W : 1][kWordsPerLane];
#pragma unroll
        for (int k = 0; k < W; ++k)
#pragma unroll
          for (int u = 0; u < kWordsPerLane; ++u) {
            const int word = D >= 128 ? (D / 128) * q + u : q / 2;
            pl[k][u] = *reinterpret_cast<const uint32_t *>(tb + tok * CB + k * (D / 8) + 4 * word);
          }
#pragma unroll
        for (int A = 1; A <= kPlanes; ++A) {
          if ((pmask >> A) & 1u) {
            uint32_t x[kWordsPerLane];
#pragma unroll
            for (int u = 0; u < kWordsPerLane; ++u) {
              x[u] = 0;
#pragma unroll
              for (int k = 0; k < W; ++k)
                if ((A >> k) & 1) x[u] ^= pl[k][u];
            }
#pragma unroll
            for (int h = 0; h < D / 64; ++h) {
              // chunk h = coordinates (D/4) q + 16 h .. + 15
              const int hf = D >= 128 ? (h & 1) : (q & 1);
              const v4i bop = spread_half(x[D >= 128 ? h >> 1 : 0], hf);
#pragma unroll
              for (int r = 0; r < RB; ++r) {
                const v4i aop = *reinterpret_cast<const v4i *>(qa + ((chunk * RB + r) * 4 + q) * 256 + n16 * 16);
                acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, acc[r], 0, 0, 0);
              }
              ++chunk;
            }
          }
        }
      }
      {
        const uint8_t *sp = tb + o_signs + tok * SB;
        for (int h = 0; h < m / 64; ++h) {
          const int c = (m / 4) * q + 16 * h;          // first sketch row of this chunk
          const uint32_t word = *reinterpret_cast<const uint32_t *>(sp + 4 * (c >> 5));
          const v4i bop = spread_half(word, (c >> 4) & 1);
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            const v4i aop = *reinterpret_cast<const v4i *>(qa + ((chunk * RB + r) * 4 + q) * 256 + n16 * 16);
            acc[r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, acc[r], 0, 0, 0);
          }
          ++chunk;
        }
      }
      const float nrm = reinterpret_cast<const float *>(tb + o_norm)[tok];
      const float gam = W > 0 ? reinterpret_cast<const float *>(tb + o_rnorm)[tok] : nrm;
      const bool valid = tok < nt;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int g = 4 * r + q;
        float lg = -INFINITY;
        if (g < G && valid) {
          float s = 0.0f;
          if constexpr (W > 0)
            s = nrm * (qc->sig_mse[g] * static_cast<float>(acc[r][0] * 128 + acc[r][1]) + qc->c_mse[g]);
          const float qjl = qc->sig_qjl[g] * static_cast<float>(acc[r][2] * 128 + acc[r][3]) + qc->c_qjl[g];
          s = fmaf(kappa_qjl * gam, qjl, s);
          lg = s * lscale;
          if (job.scores) job.scores[(head0 + g) * job.context + t0 + tok] = s;
        }
        logit[ct][r] = lg;
      }
    }

    // ---------------- online softmax (lazy rescale); lane group q = head 4r + q
    float fac[RB];
    bool changed = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float tmax = fmaxf(logit[0][r], logit[1][r]);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
      float f = 1.0f;
      if (tmax > m_ref[r] + kLazy) {
        f = (m_ref[r] == -INFINITY) ? 0.0f : exp2f(m_ref[r] - tmax);
        m_ref[r] = tmax;
        changed = true;
      }
      fac[r] = f;
      const int g = 4 * r + q;
      float psum = 0.0f;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float p = (logit[ct][r] == -INFINITY) ? 0.0f : exp2f(logit[ct][r] - m_ref[r]);
        psum += p;
        if (g < G) P[g * kTT + 16 * ct + n16] = p;
      }
      l_part[r] = l_part[r] * f + psum;
    }
    if (__any(changed)) {
      // factor of head g lives in lane 16 * (g % 4), row block g / 4
      float fh[G];
#pragma unroll
      for (int g = 0; g < G; ++g) fh[g] = __shfl(fac[g / 4], 16 * (g % 4));
      // value rows of lane group q: heads 2q, 2q+1 (hi, lo)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float fv = 1.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) fv = (g == 2 * q + e) ? fh[g] : fv;
#pragma unroll
        for (int i = 0; i < 2 * kGroups; ++i) {
          cval[i][2 * e] *= fv;
          cval[i][2 * e + 1] *= fv;
        }
      }
      // correction sums: pair k of lane group q is (head, group) = divmod(q + 4 k, kGroups)
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int pair = q + 4 * k;
        float fv = 1.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) fv = (g == pair / kGroups) ? fh[g] : fv;
        corr[k] *= fv;
      }
    }
    compiler_fence();

    // ---------------- value weights a = p * scale (f16 hi + lo), correction sums
    // K-slot 8 q' + i of the value product is token 4 i + q'; lane (tp, pq)
    // handles tokens t0 = 8 (tp / 4) + tp % 4 and t0 + 4 (slots i, i + 1 of q' = tp % 4).
    {
      const int tp = n16, pq = q;
      const int ta = 8 * (tp >> 2) + (tp & 3), tb4 = ta + 4;
      const int qd = tp & 3, i0 = 2 * (tp >> 2);
      const float *vs = reinterpret_cast<const float *>(tb + o_vscale);
      const float *vm = reinterpret_cast<const float *>(tb + o_vmin);
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int pair = pq + 4 * k;
        if (pair < G * kGroups) {
          const int g = pair / kGroups, grp = pair % kGroups;
          const float pa = P[g * kTT + ta], pb = P[g * kTT + tb4];
          const float sa = vs[ta * kGroups + grp], sb = vs[tb4 * kGroups + grp];
          const float ma = vm[ta * kGroups + grp], mb = vm[tb4 * kGroups + grp];
          float aa = pa > 0.0f ? pa * sa : 0.0f;
          float ab = pb > 0.0f ? pb * sb : 0.0f;
          // pin the fp32 weights so both uses of the f16 high part round the same value
          asm volatile("" : "+v"(aa), "+v"(ab));
          float cacc = corr[k];
          if (pa > 0.0f) cacc = fmaf(pa, ma - kMag * sa, cacc);
          if (pb > 0.0f) cacc = fmaf(pb, mb - kMag * sb, cacc);
          corr[k] = cacc;
          const _Float16 ha = static_cast<_Float16>(aa), hb = static_cast<_Float16>(ab);
          const _Float16 la = static_cast<_Float16>(aa - static_cast<float>(ha));
          const _Float16 lb = static_cast<_Float16>(ab - static_cast<float>(hb));
          uint8_t *dst = aval + ((grp * 4 + qd) * 16 + 2 * g) * 16 + 2 * i0;
          *reinterpret_cast<uint32_t *>(dst) =
              static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ha)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hb)) << 16);
          *reinterpret_cast<uint32_t *>(dst + 16) =
              static_cast<uint32_t>(__builtin_bit_cast(uint16_t, la)) | (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lb)) << 16);
        }
      }
    }
    compiler_fence();

    // ---------------- value products: 32 tokens x 16 channels per MFMA
    {
      const uint8_t *vc = tb + o_vcodes;
#pragma unroll
      for (int grp = 0; grp < kGroups; ++grp) {
        const v8h aop = *reinterpret_cast<const v8h *>(aval + ((grp * 4 + q) * 16 + n16) * 16);
        // block word(s) of column n16: tokens 4 i + q of channels 32 grp + 16 h + n16;
        // operand dword k = K-slots (8q + 2k, 8q + 2k + 1) = i (2k, 2k + 1)
        uint32_t wv[2];
        if constexpr (VB == 2) {
          wv[0] = reinterpret_cast<const uint32_t *>(vc)[(16 * grp + n16) * 4 + q];
        } else {
          const uint2 t2 = reinterpret_cast<const uint2 *>(vc)[(16 * grp + n16) * 4 + q];
          wv[0] = t2.x;
          wv[1] = t2.y;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v4i bw;
          if constexpr (VB == 2) {
            // h = 0: code of i = 2k at bits 2k, of 2k+1 at 16 + 2k; h = 1: 8 bits higher
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t sh = h == 0 ? (wv[0] << (8 - 2 * k)) : (wv[0] >> (2 * k));
              bw[k] = static_cast<int>((sh & 0x03000300u) | 0x3c003c00u);
            }
          } else {
            // code of i = 2k at bits 4k, of 2k+1 at 16 + 4k -> mantissa bits 6..9
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const uint32_t sh = k < 2 ? (wv[h] << (6 - 4 * k)) : (wv[h] >> (4 * k - 6));
              bw[k] = static_cast<int>((sh & 0x03c003c0u) | 0x3c003c00u);
            }
          }
          const v8h bop = __builtin_bit_cast(v8h, bw);
          cval[2 * grp + h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cval[2 * grp + h], 0, 0, 0);
        }
      }
    }
    compiler_fence();
    bsel ^= 1;
  }

  // ---------------- per-wave results -> LDS, merge the 4 waves
  __syncthreads();
  float *mrg = reinterpret_cast<float *>(smem + n_chunks_max * RB * 1024 + 256);   // [wave][G][D]
  float *mrg_ml = mrg + kWaves * G * D;                                             // [wave][G][2]
  float *mrg_corr = mrg_ml + kWaves * G * 2;                                        // [wave][G * kGroups]
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float l = l_part[r];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) l += __shfl_xor(l, off);
    const int g = 4 * r + q;
    if (g < G && n16 == 0) {
      mrg_ml[(wave * G + g) * 2 + 0] = m_ref[r];
      mrg_ml[(wave * G + g) * 2 + 1] = l;
    }
  }
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    float c = corr[k];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) c += __shfl_xor(c, off);
    const int pair = q + 4 * k;
    if (n16 == 0 && pair < G * kGroups) mrg_corr[wave * G * kGroups + pair] = c;
  }
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int g = 2 * q + e;
    if (g < G) {
#pragma unroll
      for (int grp = 0; grp < kGroups; ++grp) {
        const float cg = mrg_corr[wave * G * kGroups + g * kGroups + grp];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ch = 32 * grp + 16 * h + n16;
          const v4f c = cval[2 * grp + h];
          mrg[(wave * G + g) * D + ch] = kMag * (c[2 * e] + c[2 * e + 1]) + cg;
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, j = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv)
      if (mrg_ml[(wv * G + g) * 2 + 1] > 0.0f) M = fmaxf(M, mrg_ml[(wv * G + g) * 2]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float lw = mrg_ml[(wv * G + g) * 2 + 1];
      if (lw > 0.0f) {
        const float f = exp2f(mrg_ml[(wv * G + g) * 2] - M);
        L = fmaf(lw, f, L);
        O = fmaf(mrg[(wv * G + g) * D + j], f, O);
      }
    }
    const int64_t ph = (head0 + g) * job.n_split + split;
    job.part_acc[ph * D + j] = O;
    if (j == 0) {
      job.part_ml[ph * 2 + 0] = M;
      job.part_ml[ph * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- launch

struct MfmaGeo {
  int n_chunks_max;
  size_t smem;
};

MfmaGeo mfma_geo(int d, int w, int m, int g, int vb) {
  MfmaGeo o{};
  const int planes = w > 0 ? (1 << w) - 1 : 0;
  const int rb = (g + 3) / 4;
  o.n_chunks_max = planes * (d / 64) + m / 64;
  const int groups = d / 32;
  const int tile_bytes = kTT * (w * d / 8 + m / 8 + 4 + (w > 0 ? 4 : 0) + d * vb / 8 + 8 * groups);
  const int wave_bytes = 2 * tile_bytes + g * kTT * 4 + groups * 4 * 16 * 16;
  const size_t waves = static_cast<size_t>(kWaves) * wave_bytes;
  const size_t merge = static_cast<size_t>(kWaves) * (g * d + 2 * g + g * groups) * 4;
  o.smem = static_cast<size_t>(o.n_chunks_max) * rb * 1024 + 256 + (waves > merge ? waves : merge);
  return o;
}

template <int D, int W, int G, int VB>
hipError_t launch_dwgv(const DecodeJob &job, hipStream_t stream) {
  const MfmaGeo geo = mfma_geo(D, W, job.m, G, VB);
  auto kern = decode_mfma_kernel<D, W, G, VB>;
  if (geo.smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(geo.smem));
    if (e != hipSuccess) return e;
  }
  kern<<<static_cast<unsigned>(job.n_split * job.n_slots), kThreads, geo.smem, stream>>>(job, geo.n_chunks_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine(job, stream);
}

template <int D, int W, int G>
hipError_t launch_dwg(const DecodeJob &job, hipStream_t stream) {
  return job.vb == 2 ? launch_dwgv<D, W, G, 2>(job, stream) : launch_dwgv<D, W, G, 4>(job, stream);
}

template <int D, int W>
hipError_t launch_dw(const DecodeJob &job, hipStream_t stream) {
  switch (job.g) {
    case 1: return launch_dwg<D, W, 1>(job, stream);
    case 2: return launch_dwg<D, W, 2>(job, stream);
    case 4: return launch_dwg<D, W, 4>(job, stream);
    default: return launch_dwg<D, W, 8>(job, stream);
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

bool decode_mfma_supported(int d, int w, int g, int m, int vb) {
  if (g != 1 && g != 2 && g != 4 && g != 8) return false;
  return mfma_geo(d, w, m, g, vb).smem <= 160 * 1024;
}

int decode_mfma_blocks_per_cu(int d, int w, int g, int m, int vb) {
  const size_t smem = mfma_geo(d, w, m, g, vb).smem;
  int by_lds = static_cast<int>((160 * 1024) / smem);
  const int by_regs = d >= 256 ? 2 : 3;   // register file: waves of 4 per SIMD the kernel fits
  if (by_lds > by_regs) by_lds = by_regs;
  return by_lds < 1 ? 1 : by_lds;
}

hipError_t launch_decode_mfma(const DecodeJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
