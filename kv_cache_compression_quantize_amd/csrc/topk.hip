// Query-aware top-K preselection (QUOKA article §1: pre-aggregation over the KV
// heads, cosine-similarity scoring, dynamic top-K KV selection) on the packed
// cache, and decode attention over the chosen tokens only.
//
//   selection_query_kernel  per KV slot: q_sel = sum of the unit query vectors
//                           of its query heads, rotated and sketched
//   (the estimator of <q_sel, k_t> for every cached token comes from the
//   decoder's score output)
//   topk_select_kernel      per KV slot (1024 threads): cos_t = score_t / ||k_t||
//                           (0 for a zero key) as order-preserving keys, the
//                           `budget` largest by a radix select with digits of
//                           12, 10 and 10 bits, the last two on the candidates of
//                           the first digit's bin (ties to the lower token),
//                           written as increasing token indices
//   sparse_decode_kernel    per (KV slot, chunk of 64 chosen tokens): the chosen
//                           rows are gathered from their block records into LDS
//                           (key planes, signs, norms, value codes, scale and
//                           min), scored for every query head of the slot with
//                           the estimator, and reduced to a split partial
//                           (max, sum, weighted value sum); the split combine
//                           merges the chunks.
#include "internal.h"
#include "query_rows.h"

namespace aqkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSqrtHalfPi = 1.2533141373155003f;   // sqrt(pi / 2)
constexpr int kThreads = 256;
constexpr int kChunkTokens = 64;

__device__ __forceinline__ float block_reduce_sum(float x, float *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// --------------------------------------------------------------- selection query

// Per (KV slot, 64 output rows of the stacked [Pi; S]): the slot's selection
// query q_sel = sum over its query heads of q_h / ||q_h|| is built in LDS, then
// rotated and sketched by the query-preparation GEMV (query_rows.h; every row
// load issued before the query is built).
template <int D>
__global__ __launch_bounds__(kThreads) void selection_query_kernel(const float *__restrict__ q, int g, int m,
                                                                   const float *__restrict__ rotation,
                                                                   const float *__restrict__ sketch,
                                                                   float *__restrict__ q_rot,
                                                                   float *__restrict__ q_sk, int chunks) {
  static_assert(QueryRows<D>::kThreads == kThreads, "one GEMV block per selection block");
  __shared__ float qs[D];
  __shared__ float red[4];
  const int64_t slot = blockIdx.x / chunks;
  const int chunk = static_cast<int>(blockIdx.x % chunks);
  const int tid = threadIdx.x;
  const int d_rot = q_rot ? D : 0;
  const int rows = d_rot + m;
  QueryRows<D> qr;
  qr.load(rotation, sketch, d_rot, rows, chunk);
  float acc = 0.0f;
  for (int h = 0; h < g; ++h) {
    const float x = tid < D ? q[(slot * g + h) * D + tid] : 0.0f;
    const float n = sqrtf(block_reduce_sum(x * x, red));
    acc = fmaf(x, n > 0.0f ? 1.0f / n : 0.0f, acc);
  }
  if (tid < D) qs[tid] = acc;
  __syncthreads();
  qr.apply(qs, d_rot, rows, chunk, q_rot ? q_rot + slot * D : nullptr, q_sk + slot * m);
}

// --------------------------------------------------------------- top-K select

// order-preserving image of a float: larger float -> larger key
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SelectJob {
  float *scores;            // [n_slots][context]; overwritten with the order keys
  const uint8_t *norm;      // key_norm field at its place in record 0; null: the scores are
                            // the ranking values themselves (record selection)
  int sf;                   // half norms (else fp32)
  int64_t rec, capacity, context;
  int budget;               // chosen tokens per slot (<= context)
  int32_t *selected;        // [n_slots][budget]
};

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 4096;            // widest digit: 12 bits
constexpr int64_t kLdsKeys = 32768;       // slots of at most this many tokens keep their keys in LDS

// exclusive scan over the block's threads: a scan within each wave, then the wave totals
__device__ __forceinline__ uint32_t block_scan(uint32_t x, uint32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(inc, off);
    if (lane >= off) inc += v;
  }
  __syncthreads();   // wsum is free again
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) before += w < wave ? wsum[w] : 0u;
  return before + inc - x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// KEYS_LDS: the slot's keys live in dynamic LDS, else in place of its scores.
// Three passes over the keys: (1) compute them and histogram their top 12 bits;
// (2) after the first digit, collect the keys of its bin (the candidates, at
// most kCandMax of them, in the histogram's space) and count per wave the keys
// above it; the last two digits are then found on the candidates alone; (3)
// write the chosen indices in token order.  A bin with more candidates than
// that (many equal keys) takes two more full passes and a counting pass instead.
constexpr int kCandMax = kHistBins - 1024;
template <bool KEYS_LDS>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(SelectJob job) {
  extern __shared__ uint4 lds_keys4[];
  __shared__ uint32_t hist[kHistBins];   // first-digit histogram; then 1024 bins + the candidates
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t wgt[kSelWaves], weq[kSelWaves];
  __shared__ uint32_t pick[2];
  __shared__ uint32_t n_cand;
  const int64_t slot = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = static_cast<int>(job.context);   // chosen indices are int32, so T < 2^31
  const float *sc_row = job.scores + slot * job.context;
  uint32_t *keys = KEYS_LDS ? reinterpret_cast<uint32_t *>(lds_keys4)
                            : reinterpret_cast<uint32_t *>(job.scores + slot * job.context);
  // keys 4 q .. 4 q + 3 (a 16-byte read in LDS; in place of the scores, which need not be
  // 16-byte aligned, four reads)
  auto quad = [&](int q) -> uint4 {
    if (KEYS_LDS) return lds_keys4[q];
    return make_uint4(keys[4 * q], keys[4 * q + 1], keys[4 * q + 2], keys[4 * q + 3]);
  };
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();
  // 1. cos_t = score_t / n_t (0 for a zero key) as order-preserving keys, and the histogram
  //    of their top 12 bits (cosines share their sign and exponent bits, so a wide first
  //    digit spreads them); every load of a batch is issued before the first is used
  constexpr int kBatch = 16;
  const int64_t row0 = slot * job.capacity;
  for (int t0 = 0; t0 < T; t0 += kSelThreads * kBatch) {
    float sc[kBatch], nn[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = t0 + u * kSelThreads + tid;
      sc[u] = t < T ? sc_row[t] : 0.0f;
      nn[u] = t < T && job.norm ? load_side(job.norm + rec_row((row0 + t) & ~int64_t(31), 0, job.rec),
                                            (row0 + t) & 31, job.sf != 0)
                                : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = t0 + u * kSelThreads + tid;
      if (t < T) {
        const uint32_t k = order_key(!job.norm ? sc[u] : nn[u] > 0.0f ? sc[u] / nn[u] : 0.0f);
        keys[t] = k;
        atomicAdd(&hist[k >> 20], 1u);
      }
    }
  }
  __syncthreads();
  // the digit of `bins` histogram bins (from the top) that holds the need-th largest key:
  // thread i holds `per` bins from the top down; the scan gives the count in the bins above
  // them, and the one thread whose bins take that count to `need` writes the digit
  auto find_digit = [&](int bins, uint32_t need) {
    const int per = bins / kSelThreads;
    const int top = bins - 1 - tid * per;
    uint32_t c = 0;
    for (int j = 0; j < per; ++j) c += hist[top - j];
    uint32_t above = block_scan(c, wsum);
    if (above < need && above + c >= need) {
      for (int j = 0; j < per; ++j) {
        const uint32_t h = hist[top - j];
        if (above + h >= need) {
          pick[0] = static_cast<uint32_t>(top - j);
          pick[1] = above;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
  };
  uint32_t need = static_cast<uint32_t>(job.budget);   // still to choose among keys matching prefix
  find_digit(kHistBins, need);
  uint32_t prefix = pick[0] << 20, mask = 0xFFF00000u;
  need -= pick[1];
  const uint32_t nc = hist[pick[0]];
  // wave segments for the collect and write passes: contiguous runs of tokens (a multiple
  // of 256), taken 256 at a time, lane l holding tokens 4 l .. 4 l + 3
  const int seg = ((T + kSelWaves - 1) / kSelWaves + 255) / 256 * 256;
  const int s0 = min(T, wave * seg), s1 = min(T, s0 + seg);
  const uint64_t below = (uint64_t{1} << lane) - 1u;
  auto lane_keys = [&](int b, uint32_t k[4]) -> int {   // valid keys of the lane at b
    const int t = b + 4 * lane;
    if (t + 3 < s1) {
      const uint4 v = quad(t >> 2);
      k[0] = v.x;
      k[1] = v.y;
      k[2] = v.z;
      k[3] = v.w;
      return 4;
    }
    const int nv = max(0, s1 - t);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = j < nv ? keys[t + j] : 0u;
    return nv;
  };
  const int nq = T >> 2;
  if (tid == 0) n_cand = 0;
  __syncthreads();   // nc read by every thread before hist is reused
  for (int i = tid; i < 1024; i += kSelThreads) hist[i] = 0;
  if (nc <= static_cast<uint32_t>(kCandMax)) {
    // 2. the candidates (keys in the first digit's bin) and, per wave, the keys above it
    uint32_t *cand = hist + 1024;
    uint32_t gt = 0;
    for (int b = s0; b < s1; b += 256) {
      uint32_t k[4];
      const int nv = lane_keys(b, k);
      bool c[4];
      uint32_t c_below = 0, c_all = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gt += j < nv && (k[j] & mask) > prefix;
        c[j] = j < nv && (k[j] & mask) == prefix;
        const uint64_t cb = __ballot(c[j]);
        c_below += __popcll(cb & below);
        c_all += __popcll(cb);
      }
      if (c_all > 0) {
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&n_cand, c_all);
        base = __shfl(base, 0);
        uint32_t o = base + c_below;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c[j]) cand[o++] = static_cast<uint32_t>(b + 4 * lane + j);
      }
    }
    gt = wave_sum(gt);
    if (lane == 0) {
      wgt[wave] = gt;
      weq[wave] = 0;
    }
    __syncthreads();
    const int ncand = static_cast<int>(n_cand);
    // the last two digits on the candidates
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      if (pass > 0) {
        for (int i = tid; i < 1024; i += kSelThreads) hist[i] = 0;
        __syncthreads();
      }
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint32_t k = keys[cand[i]];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1u);
      }
      __syncthreads();
      find_digit(1024, need);
      prefix |= pick[0] << shift;
      mask |= 1023u << shift;
      need -= pick[1];
    }
    // per wave: the candidates above the threshold, and those equal to it
    for (int i = tid; i < ncand; i += kSelThreads) {
      const uint32_t t = cand[i];
      const uint32_t k = keys[t];
      const int w = static_cast<int>(t) / seg;
      if (k > prefix) atomicAdd(&wgt[w], 1u);
      else if (k == prefix) atomicAdd(&weq[w], 1u);
    }
    __syncthreads();
  } else {
    // 2'. many keys in one bin: the last two digits over all keys, then the per-wave counts
    __syncthreads();
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = pass == 0 ? 10 : 0;
      if (pass > 0) {
        for (int i = tid; i < 1024; i += kSelThreads) hist[i] = 0;
        __syncthreads();
      }
      auto count = [&](uint32_t k) {
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 1023u], 1u);
      };
#pragma unroll 2
      for (int q = tid; q < nq; q += kSelThreads) {
        const uint4 k = quad(q);
        count(k.x);
        count(k.y);
        count(k.z);
        count(k.w);
      }
      if (4 * nq + tid < T) count(keys[4 * nq + tid]);
      __syncthreads();
      find_digit(1024, need);
      prefix |= pick[0] << shift;
      mask |= 1023u << shift;
      need -= pick[1];
    }
    uint32_t gt = 0, eq = 0;
    for (int b = s0; b < s1; b += 256) {
      uint32_t k[4];
      const int nv = lane_keys(b, k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gt += j < nv && k[j] > prefix;
        eq += j < nv && k[j] == prefix;
      }
    }
    gt = wave_sum(gt);
    eq = wave_sum(eq);
    if (lane == 0) {
      wgt[wave] = gt;
      weq[wave] = eq;
    }
    __syncthreads();
  }
  // 3. keys > prefix are all chosen; of the keys == prefix, the first `need` in token
  //    order.  Each wave ranks its lanes' choices by ballot, so the output comes out in
  //    increasing token order.
  const uint32_t eq = weq[wave];
  uint32_t eq_before = 0, base = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t take = eq_before >= need ? 0u : min(weq[w], need - eq_before);
    base += wgt[w] + take;
    eq_before += weq[w];
  }
  const uint32_t eq_take = eq_before >= need ? 0u : min(eq, need - eq_before);
  int32_t *out = job.selected + slot * job.budget;
  uint32_t pos = base, eq_seen = 0;
  for (int b = s0; b < s1; b += 256) {
    uint32_t k[4];
    const int nv = lane_keys(b, k);
    bool e[4], take[4];
    uint32_t e_below = 0, e_all = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = j < nv && k[j] == prefix;
      const uint64_t eb = __ballot(e[j]);
      e_below += __popcll(eb & below);
      e_all += __popcll(eb);
    }
    uint32_t r = eq_seen + e_below;   // rank among the slot's ties of this lane's next tie
    uint32_t t_below = 0, t_all = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      take[j] = (j < nv && k[j] > prefix) || (e[j] && r < eq_take);
      r += e[j];
      const uint64_t tb = __ballot(take[j]);
      t_below += __popcll(tb & below);
      t_all += __popcll(tb);
    }
    uint32_t p = pos + t_below;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (take[j]) out[p++] = b + 4 * lane + j;
    }
    pos += t_all;
    eq_seen += e_all;
  }
}

// --------------------------------------------------------------- sparse decode

struct SparseJob {
  int d, w, m, vb, g;
  int sf;                          // half side information (else fp32)
  int64_t capacity, rec;
  const uint8_t *codes, *signs, *norm, *rnorm, *vcodes, *vside;   // fields at their place in record 0
  const float *centroids;
  const float *q_rot, *q_sketch;   // [n_slots*g][d], [n_slots*g][m]
  const int32_t *selected;         // [n_slots][budget]
  int budget, n_chunks;
  int64_t context;
  float softmax_scale;
  float *part_acc, *part_ml;       // [n_slots*g][n_chunks][d], [..][2]
};

constexpr int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// centroid of the index whose bits are b0 (bit 0), b1, b2 (W of them); the
// codebook is held in named registers, so the choice is a chain of selects
struct Codebook8 {
  float c0, c1, c2, c3, c4, c5, c6, c7;
};
template <int W>
__device__ __forceinline__ float centroid(const Codebook8 &c, uint32_t b0, uint32_t b1, uint32_t b2) {
  const float l01 = b0 ? c.c1 : c.c0;
  if (W == 1) return l01;
  const float l23 = b0 ? c.c3 : c.c2;
  const float lo = b1 ? l23 : l01;
  if (W == 2) return lo;
  const float l45 = b0 ? c.c5 : c.c4;
  const float l67 = b0 ? c.c7 : c.c6;
  const float hi = b1 ? l67 : l45;
  return b2 ? hi : lo;
}

// LDS bytes of one block
template <int D, int W>
size_t sparse_smem(int m, int g) {
  constexpr int T = kChunkTokens;
  return 4 * static_cast<size_t>(T) * (W * D / 32 + m / 32 + 2) +   // key words, sign words, n and gamma
         static_cast<size_t>(T) * D +                                 // value codes
         4 * static_cast<size_t>(T) * (D / 32) * 2 +                  // value scale and min
         4 * static_cast<size_t>(g) * T +                             // logits, then weights
         4 * static_cast<size_t>(g) * (D + m) +                       // the slot's rotated and sketched queries
         4 * static_cast<size_t>(kThreads);                           // value partial sums
}

template <int D, int W>
__global__ __launch_bounds__(kThreads) void sparse_decode_kernel(SparseJob job) {
  constexpr int T = kChunkTokens;
  constexpr int kGroups = D / 32;
  constexpr int kWords = D / 32;                  // 32-bit words of one bit plane
  constexpr int kw = W * kWords;                  // key-code words per token
  constexpr int kwp = pow2_at_least(kw > 0 ? kw : 1);
  extern __shared__ uint32_t sm[];
  const int M = job.m, G = job.g, VB = job.vb;
  const int sw = M / 32;                          // sign words per token
  const int sws = sw > 1 ? 32 - __clz(sw - 1) : 0;   // ceil(log2(sw))
  uint32_t *kc = sm;                              // [T][kw]
  uint32_t *sg = kc + T * kw;                     // [T][sw]
  float *nr = reinterpret_cast<float *>(sg + T * sw);     // [T][2]: n, gamma
  uint8_t *vc = reinterpret_cast<uint8_t *>(nr + 2 * T);  // [T][D] value codes
  float *vsd = reinterpret_cast<float *>(vc + T * D);     // [T][kGroups][2] scale, min
  float *lg = vsd + T * kGroups * 2;              // [G][T] logits, then weights
  float *qv = lg + G * T;                         // [G][D + M]: q_rot then q_sketch
  float *red = qv + G * (D + M);                  // [kThreads] value partial sums
  __shared__ float stat[2 * kMaxQPerKv];
  __shared__ int64_t rbase[T];                    // byte offset of the chosen row's record
  __shared__ int rtt[T];                          // the row within its record
  const int tid = threadIdx.x;
  const int64_t slot = blockIdx.x / job.n_chunks;
  const int chunk = static_cast<int>(blockIdx.x % job.n_chunks);
  const int c0 = chunk * T;
  const int nt = min(T, job.budget - c0);
  const int32_t *sel_in = job.selected + slot * job.budget + c0;
  // the chosen rows, clamped into the context (the select kernel writes them in
  // range; the clamp keeps every gather inside the slot's records regardless)
  if (tid < nt) {
    const int64_t row = slot * job.capacity + min(max(sel_in[tid], 0), static_cast<int32_t>(job.context - 1));
    rbase[tid] = (row >> 5) * job.rec;
    rtt[tid] = static_cast<int>(row & 31);
  }
  // the slot's queries
  for (int h = 0; h < G; ++h) {
    const int64_t head = slot * G + h;
    if (W > 0)
      for (int j = tid; j < D; j += kThreads) qv[h * (D + M) + j] = job.q_rot[head * D + j];
    for (int j = tid; j < M; j += kThreads) qv[h * (D + M) + D + j] = job.q_sketch[head * M + j];
  }
  Codebook8 cen{};
  if constexpr (W > 0) {
    const float *cg = job.centroids;
    cen.c0 = cg[0];
    cen.c1 = cg[1];
    if constexpr (W > 1) {
      cen.c2 = cg[2];
      cen.c3 = cg[3];
    }
    if constexpr (W > 2) {
      cen.c4 = cg[4];
      cen.c5 = cg[5];
      cen.c6 = cg[6];
      cen.c7 = cg[7];
    }
  }
  __syncthreads();

  // 1. gather the chosen rows: whole words, record offsets from LDS
  if constexpr (W > 0) {
    for (int i = tid; i < nt * kwp; i += kThreads) {
      const int t = i / kwp, wd = i % kwp;
      if (wd < kw)
        kc[t * kw + wd] = reinterpret_cast<const uint32_t *>(job.codes + rbase[t] + rtt[t] * (W * D / 8))[wd];
    }
  }
  for (int i = tid; i < (nt << sws); i += kThreads) {
    const int t = i >> sws, wd = i & ((1 << sws) - 1);
    if (wd < sw) sg[t * sw + wd] = reinterpret_cast<const uint32_t *>(job.signs + rbase[t] + rtt[t] * (M / 8))[wd];
  }
  if (tid < nt) {
    nr[2 * tid] = load_side(job.norm + rbase[tid], rtt[tid], job.sf != 0);
    nr[2 * tid + 1] = W > 0 ? load_side(job.rnorm + rbase[tid], rtt[tid], job.sf != 0) : 0.0f;
  }
  // value codes: item (group, n) of a token gives its channels 32 group + n and 32 group + 16 + n
  for (int i = tid; i < nt * (D / 2); i += kThreads) {
    const int t = i / (D / 2), it = i % (D / 2);
    const int grp = it >> 4, n = it & 15;
    const int tt = rtt[t], r = tt & 3, ii = tt >> 2;
    const uint32_t *blk = reinterpret_cast<const uint32_t *>(job.vcodes + rbase[t]);
    uint32_t c_lo, c_hi;
    if (VB == 2) {
      const uint32_t wv = blk[(16 * grp + n) * 4 + r] >> (16 * (ii & 1) + 2 * (ii >> 1));
      c_lo = wv & 3u;
      c_hi = (wv >> 8) & 3u;
    } else {
      const uint2 wv = *reinterpret_cast<const uint2 *>(blk + ((16 * grp + n) * 4 + r) * 2);
      const int sh = 16 * (ii & 1) + 4 * (ii >> 1);
      c_lo = (wv.x >> sh) & 15u;
      c_hi = (wv.y >> sh) & 15u;
    }
    vc[t * D + 32 * grp + n] = static_cast<uint8_t>(c_lo);
    vc[t * D + 32 * grp + 16 + n] = static_cast<uint8_t>(c_hi);
  }
  for (int i = tid; i < nt * kGroups; i += kThreads) {
    const int t = i / kGroups, grp = i % kGroups;
    const int si = side_index(grp, rtt[t], 0);
    vsd[(t * kGroups + grp) * 2] = load_side(job.vside + rbase[t], si, job.sf != 0);
    vsd[(t * kGroups + grp) * 2 + 1] = load_side(job.vside + rbase[t], si + 1, job.sf != 0);
  }
  __syncthreads();

  // 2. the estimator for every (query head, chosen token): n <q_rot, c[idx]> + sqrt(pi/2)/m gamma <q_sk, 2 b - 1>.
  //    Four neighbouring lanes per (head, token); in a bit word element 4 i + k sits at bit 8 k + i, so
  //    lane k of the four takes byte k of every word: elements 32 word + 4 b + k, b = 0..7.
  const float qjl = kSqrtHalfPi / static_cast<float>(M);
  const float lscale = job.softmax_scale * kLog2e;
  const int quarter = tid & 3;
  for (int i0 = 0; i0 < G * T; i0 += kThreads / 4) {
    const int i = i0 + (tid >> 2);
    const int h = i / T, t = i % T;
    const bool live = i < G * T && t < nt;
    float mse = 0.0f, sk = 0.0f;
    if (live) {
      const float *qr = qv + h * (D + M) + quarter;
      const float *qs = qr + D;
      if constexpr (W > 0) {
        const uint32_t *kt = kc + t * kw;
#pragma unroll 2
        for (int wd = 0; wd < kWords; ++wd) {
          const uint32_t p0 = kt[wd] >> (8 * quarter);
          const uint32_t p1 = W > 1 ? kt[kWords + wd] >> (8 * quarter) : 0u;
          const uint32_t p2 = W > 2 ? kt[2 * kWords + wd] >> (8 * quarter) : 0u;
#pragma unroll
          for (int b = 0; b < 8; ++b)
            mse = fmaf(qr[32 * wd + 4 * b], centroid<W>(cen, (p0 >> b) & 1u, (p1 >> b) & 1u, (p2 >> b) & 1u), mse);
        }
      }
      const uint32_t *st = sg + t * sw;
      for (int wd = 0; wd < sw; ++wd) {
        const uint32_t sb = st[wd] >> (8 * quarter);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const float qq = qs[32 * wd + 4 * b];
          sk += ((sb >> b) & 1u) ? qq : -qq;
        }
      }
    }
    mse += __shfl_xor(mse, 1);
    mse += __shfl_xor(mse, 2);
    sk += __shfl_xor(sk, 1);
    sk += __shfl_xor(sk, 2);
    if (quarter == 0 && i < G * T) {
      const float score = W > 0 ? nr[2 * t] * mse + qjl * nr[2 * t + 1] * sk : qjl * nr[2 * t] * sk;
      lg[i] = live ? score * lscale : -INFINITY;
    }
  }
  __syncthreads();

  // 3. per head: max, weights, sum (one wave a head)
  for (int h = tid >> 6; h < G; h += kThreads / 64) {
    const int lane = tid & 63;
    const float x = lane < nt ? lg[h * T + lane] : -INFINITY;
    float mx = x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float p = lane < nt ? __builtin_amdgcn_exp2f(x - mx) : 0.0f;
    lg[h * T + lane] = p;
    float l = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0) {
      stat[2 * h] = mx;
      stat[2 * h + 1] = l;
    }
  }
  __syncthreads();
  // 4. weighted value sums; when G D < the block, `parts` threads share a channel's tokens
  const int items = G * D;
  const int parts = items >= kThreads ? 1 : kThreads / items;
  for (int i0 = 0; i0 < items * parts; i0 += kThreads) {
    const int i = i0 + tid;
    const int item = i % items, part = i / items;
    float o = 0.0f;
    if (i < items * parts) {
      const int h = item / D, ch = item % D, grp = ch >> 5;
      for (int t = part; t < nt; t += parts) {
        const float v = fmaf(static_cast<float>(vc[t * D + ch]), vsd[(t * kGroups + grp) * 2],
                             vsd[(t * kGroups + grp) * 2 + 1]);
        o = fmaf(lg[h * T + t], v, o);
      }
    }
    if (parts > 1) {
      red[tid] = o;
      __syncthreads();
      if (tid < items) {
        for (int pp = 1; pp < parts; ++pp) o += red[pp * items + tid];
      }
    }
    if (i < items) {
      const int h = item / D, ch = item % D;
      const int64_t ph = (slot * G + h) * job.n_chunks + chunk;
      job.part_acc[ph * D + ch] = o;
      if (ch == 0) {
        job.part_ml[ph * 2] = stat[2 * h];
        job.part_ml[ph * 2 + 1] = stat[2 * h + 1];
      }
    }
  }
}

template <int D, int W>
hipError_t launch_sparse_dw(const SparseJob &job, int64_t n_slots, hipStream_t stream) {
  const size_t smem = sparse_smem<D, W>(job.m, job.g);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(sparse_decode_kernel<D, W>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
  }
  sparse_decode_kernel<D, W><<<static_cast<unsigned>(n_slots * job.n_chunks), kThreads, smem, stream>>>(job);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sparse_d(const SparseJob &job, int64_t n_slots, hipStream_t stream) {
  switch (job.w) {
    case 0: return launch_sparse_dw<D, 0>(job, n_slots, stream);
    case 1: return launch_sparse_dw<D, 1>(job, n_slots, stream);
    case 2: return launch_sparse_dw<D, 2>(job, n_slots, stream);
    default: return launch_sparse_dw<D, 3>(job, n_slots, stream);
  }
}

}  // namespace

int topk_chunks(int budget) { return (budget + kChunkTokens - 1) / kChunkTokens; }

hipError_t launch_selection_query(const float *q, int64_t n_slots, int d, int g, int m, const float *rotation,
                                  const float *sketch, float *q_rot, float *q_sk, hipStream_t stream) {
  const int rows = (q_rot ? d : 0) + m;
  const int chunks = (rows + 63) / 64;   // 64 rows of [Pi; S] per block
  const unsigned grid = static_cast<unsigned>(n_slots * chunks);
  switch (d) {
    case 64:
      selection_query_kernel<64><<<grid, kThreads, 0, stream>>>(q, g, m, rotation, sketch, q_rot, q_sk, chunks);
      break;
    case 128:
      selection_query_kernel<128><<<grid, kThreads, 0, stream>>>(q, g, m, rotation, sketch, q_rot, q_sk, chunks);
      break;
    default:
      selection_query_kernel<256><<<grid, kThreads, 0, stream>>>(q, g, m, rotation, sketch, q_rot, q_sk, chunks);
      break;
  }
  return hipGetLastError();
}

namespace {
hipError_t launch_select(const SelectJob &s, int64_t n_slots, hipStream_t stream) {
  if (s.context <= kLdsKeys) {
    const size_t smem = sizeof(uint4) * static_cast<size_t>((s.context + 3) / 4);
    if (smem > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(topk_select_kernel<true>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
      if (e != hipSuccess) return e;
    }
    topk_select_kernel<true><<<static_cast<unsigned>(n_slots), kSelThreads, smem, stream>>>(s);
  } else {
    topk_select_kernel<false><<<static_cast<unsigned>(n_slots), kSelThreads, 0, stream>>>(s);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_select_records(float *rec_max, int64_t n_slots, int64_t n_records, int budget,
                                 int32_t *selected, hipStream_t stream) {
  SelectJob s{};
  s.scores = rec_max;
  s.norm = nullptr;
  s.context = n_records;
  s.budget = budget;
  s.selected = selected;
  return launch_select(s, n_slots, stream);
}

hipError_t launch_topk(const TopkJob &j, hipStream_t stream) {
  SelectJob s{};
  s.scores = j.scores;
  s.norm = j.norm;
  s.sf = j.sf;
  s.rec = j.rec;
  s.capacity = j.capacity;
  s.context = j.context;
  s.budget = j.budget;
  s.selected = j.selected;
  hipError_t e = launch_select(s, j.n_slots, stream);
  if (e != hipSuccess) return e;
  SparseJob p{};
  p.d = j.d;
  p.w = j.w;
  p.m = j.m;
  p.vb = j.vb;
  p.sf = j.sf;
  p.g = j.g;
  p.capacity = j.capacity;
  p.rec = j.rec;
  p.codes = j.codes;
  p.signs = j.signs;
  p.norm = j.norm;
  p.rnorm = j.rnorm;
  p.vcodes = j.vcodes;
  p.vside = j.vside;
  p.centroids = j.centroids;
  p.q_rot = j.q_rot;
  p.q_sketch = j.q_sketch;
  p.selected = j.selected;
  p.budget = j.budget;
  p.n_chunks = topk_chunks(j.budget);
  p.context = j.context;
  p.softmax_scale = j.softmax_scale;
  p.part_acc = j.part_acc;
  p.part_ml = j.part_ml;
  switch (j.d) {
    case 64: return launch_sparse_d<64>(p, j.n_slots, stream);
    case 128: return launch_sparse_d<128>(p, j.n_slots, stream);
    default: return launch_sparse_d<256>(p, j.n_slots, stream);
  }
}

}  // namespace aqkv
