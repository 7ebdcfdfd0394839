// Key quantisation on CDNA4 matrix cores (TurboQuant article §二 three-stage
// pipeline and §五 quantize(); A-QJL article, section "QJL", for the
// pure-QJL mode w == 0).
//
// Per key x: n = ||x||, y = Pi x / n, idx_j = number of boundaries below y_j,
// e = y - c[idx], gamma = n ||e|| (= ||x - n Pi^T c[idx]|| for orthogonal
// Pi), and the residual sketch S r = n (S Pi^T) e, one sign bit per row
// (w == 0: S x).  The two dense products run on v_mfma_f32_16x16x32_f16 with
// every fp32 operand that is not already an f16 number split into f16 high
// and low parts,
//   a b ~= a_hi b_hi + a_hi b_lo + a_lo b_hi,
// a relative error of about 3 * 2^-22 per product, far inside the 1e-5
// decision window.  The weights are scaled by 2^8 first so the low parts of
// typical entries stay normal f16 numbers.  A bf16 key scaled by a power of
// two is an exact f16 vector, so for bf16 keys the products with the key take
// two passes (W_hi x', W_lo x'), for fp32 keys three (u = x / n split).
//
// Keys are the N side of every product: one MFMA column block is 16 keys, and
// lane (n, g) = (lane % 16, lane / 16) receives rows 4g .. 4g+3 of each 16-row
// output tile for key n.  The rows of the weight operands are permuted so that
// what a lane receives are whole nibbles of the words it writes: in the
// bit-row word layout (element 4 i' + k at bit 8 k + i'),
//   tile t of a full group of 8 tiles: C row (g, i) is element
//       16 (t % 2) + 4 i + (t % 8) / 2 of word 4 (t / 8) + g, i.e. bit 4 (t % 8) + i;
//   tile t of a trailing group of 4 (tt = its place in the group): element
//       16 (tt % 2) + 4 i + 2 (g % 2) + tt / 2 of word 4 G + g / 2, i.e. bit
//       16 (g % 2) + 4 tt + i
// (G full groups).  A lane builds its code words most significant bit first,
// w = 2 w + bit, with no cross-lane traffic (a trailing group merges
// two half words).  The residual e a lane holds for tiles 2k and 2k+1 is, as
// is, its B operand for k-step k of the sketch product, whose weight columns
// follow the same permutation.  No fp key and no reconstruction is formed.
//
// The weights (Pi, and S Pi^T or S) are prepared into the workspace (per
// call, or once per layer through the prepared entry points) as ready-made
// MFMA A operands, [slab][k-step][hi, lo][lane][8 f16],
// one slab per 16-row tile.  When the whole set fits in LDS (d = 128, m = 128:
// 128 KiB) a block of 8 waves loads it once and every wave then walks its own
// 32-key tiles without block synchronisation, prefetching the next tile's
// keys into registers.  Larger sets go through LDS for one key tile per block:
// the rotation in groups of 8 slabs, the sketch in double-buffered chunks
// (global_load_lds_dwordx4).
#include <algorithm>

#include "internal.h"

namespace aqkv {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kUp = 256.0f;   // weights, fp32 split inputs, boundaries and centroids are scaled by 2^8
constexpr float kDown8 = 1.0f / 256.0f;

__host__ __device__ constexpr int chunk_slabs(int d) { return d >= 256 ? 2 : 4; }
__host__ __device__ constexpr int keys_per_wave(int d) { return d >= 256 ? 16 : 32; }

// Output row held by C row r (lane group r / 4, register r % 4) of 16-row tile
// t, when the dimension has `tiles` tiles (a multiple of 4).
__host__ __device__ inline int permuted_row(int t, int r, int tiles) {
  const int full = tiles >> 3;
  const int go = r >> 2, io = r & 3;
  if (t < 8 * full) {
    const int tt = t & 7;
    return 32 * (4 * (t >> 3) + go) + 16 * (tt & 1) + 4 * io + (tt >> 1);
  }
  const int tt = t - 8 * full;
  return 32 * (4 * full + (go >> 1)) + 16 * (tt & 1) + 4 * io + 2 * (go & 1) + (tt >> 1);
}

// (a, b) -> high parts hi2 = (f16(a), f16(b)) and low parts
// lo2 = (f16(a - hi_a), f16(b - hi_b)); a - hi is exact in fp32 and rounded
// once.  a and b are pinned in registers first (an empty asm, no
// instruction), so both parts derive from the same rounded fp32 values: the
// compiler may otherwise fold the product that made a into a mixed-precision
// conversion for one part only.  No instruction is written in asm here: the
// compiler must see every VALU write to keep its wait states against
// in-flight matrix instructions.
// The low parts are fma(hi, minus1, a) with minus1 = -1 from opaque_minus1():
// a mixed-precision fma reads the f16 hi directly (no conversion back to
// fp32); a literal -1 would be folded into a subtraction.
__device__ __forceinline__ float opaque_minus1() {
  float m = -1.0f;
  asm volatile("" : "+s"(m));   // no instruction: the value is only hidden from the optimiser
  return m;
}
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi2, uint32_t &lo2, float minus1) {
  asm volatile("" : "+v"(a), "+v"(b));
  const v2h h = __builtin_convertvector((v2f){a, b}, v2h);
  // a - hi is exact in fp32, so rounding it to f16 in a mixed fma with an f16
  // result is the same as rounding the fp32 difference.  (Compiler-emitted:
  // a matrix instruction may read these operands soon after, and only the
  // compiler's own instructions get the wait states that requires.)
  const v2h l = {static_cast<_Float16>(__builtin_fmaf(static_cast<float>(h[0]), minus1, a)),
                 static_cast<_Float16>(__builtin_fmaf(static_cast<float>(h[1]), minus1, b))};
  hi2 = __builtin_bit_cast(uint32_t, h);
  lo2 = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  asm volatile("" : "+v"(a), "+v"(b));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2h));
}

// w = 2 w + bit
__device__ __forceinline__ uint32_t push_bit(uint32_t w, bool bit) { return w + w + static_cast<uint32_t>(bit); }

// ---------------------------------------------------------------- operands

// Whether every entry of the rotation has one magnitude a (a randomised
// Hadamard rotation: +-1/sqrt(d)); writes a, or 0, to *scale.  One block.
__global__ __launch_bounds__(256) void rotation_scale_kernel(const float *__restrict__ rot, int d,
                                                             float *__restrict__ scale) {
  const float a = d > 0 ? fabsf(rot[0]) : 0.0f;
  bool same = a > 0.0f && a < INFINITY;
  for (int64_t i = threadIdx.x; i < static_cast<int64_t>(d) * d; i += 256) same = same && fabsf(rot[i]) == a;
  same = __syncthreads_and(same);
  if (threadIdx.x == 0) *scale = same ? a : 0.0f;
}

// One thread per (slab, k-step, lane, slot): writes the high and low f16
// parts of one A-operand element (scaled by 2^8).
__global__ __launch_bounds__(256) void key_operands_kernel(const float *__restrict__ rot,
                                                           const float *__restrict__ sketch,
                                                           uint8_t *__restrict__ ops, int d, int w, int m,
                                                           const float *__restrict__ rot_scale) {
  const int ks = d / 32, td = d / 16, tm = m / 16;
  const int slabs = (w > 0 ? td : 0) + tm;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(slabs) * ks * 512) return;
  const int s = static_cast<int>(idx & 7);
  const int lane = static_cast<int>((idx >> 3) & 63);
  const int k = static_cast<int>((idx >> 9) % ks);
  const int slab = static_cast<int>((idx >> 9) / ks);
  const int r = lane & 15, g = lane >> 4;
  float v;
  if (w > 0 && slab < td) {
    // rotation: row = permuted coordinate, column = input coordinate 32k + 8g + s
    const int row = permuted_row(slab, r, td);
    v = rot[static_cast<int64_t>(row) * d + 32 * k + 8 * g + s];
    // one magnitude: the operand is sign(v) (times 2^8 below), exact in f16 with a zero low part
    if (*rot_scale > 0.0f) v = v > 0.0f ? 1.0f : -1.0f;
  } else {
    const int tz = slab - (w > 0 ? td : 0);
    const int row = permuted_row(tz, r, tm);
    const float *srow = sketch + static_cast<int64_t>(row) * d;
    if (w > 0) {
      // (S Pi^T)[row][col], col = the coordinate lane group g holds in slot s of k-step k
      const int col = permuted_row(2 * k + (s >> 2), 4 * g + (s & 3), td);
      const float *prow = rot + static_cast<int64_t>(col) * d;
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) acc = fmaf(srow[j], prow[j], acc);
      v = acc;
    } else {
      v = srow[32 * k + 8 * g + s];
    }
  }
  v *= kUp;
  const _Float16 hi = static_cast<_Float16>(v);
  const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
  uint8_t *base = ops + ((static_cast<int64_t>(slab) * ks + k) * 2) * 1024 + lane * 16 + 2 * s;
  *reinterpret_cast<_Float16 *>(base) = hi;
  *reinterpret_cast<_Float16 *>(base + 1024) = lo;
}

// ---------------------------------------------------------------- keys

__device__ __forceinline__ v8h lds_op(const uint8_t *p) { return *reinterpret_cast<const v8h *>(p); }

template <int D>
struct Geo {
  static constexpr int KS = D / 32;                  // k-steps of a d-long contraction
  static constexpr int TD = D / 16;                  // 16-row tiles of the coordinates
  static constexpr int FD = TD / 8;                  // full 8-tile groups of the coordinates
  static constexpr int WPL = FD + (TD % 8 ? 1 : 0);  // code words per plane a lane builds
  static constexpr int NT = keys_per_wave(D) / 16;   // 16-key column blocks per wave
  static constexpr int KT = NT * 16;                 // keys per wave tile
  static constexpr int SLAB = KS * 2048;             // bytes of one 16-row operand slab
};

// B operand of one k-step: 8 f16 as 4 packed words
struct Op {
  uint32_t w[4];
};
__device__ __forceinline__ v8h as_v8h(const Op &o) { return __builtin_bit_cast(v8h, o); }

template <int D>
using Ops = Op[Geo<D>::NT][Geo<D>::KS];

// Raw key elements of one lane: 8 consecutive elements per k-step
// (bf16: one 16-byte load, fp32: two).
template <int D, bool BF16>
struct RawKeys {
  uint4 v[Geo<D>::NT][Geo<D>::KS][BF16 ? 1 : 2];
};

// Where this lane's keys of a wave tile live: key0 (wave-uniform) + nt*16 + n.
template <int D>
struct TileLoc {
  int64_t src[Geo<D>::NT];    // element offset of the key row in the K view
  int64_t rbase[Geo<D>::NT];  // byte offset of the cache row's record (rec_row's record term)
  int rin[Geo<D>::NT];        // the row's place in its record (0 .. 31)
  bool valid[Geo<D>::NT];
  // byte offset of the row in a field whose rows are rb bytes (= rec_row(row, rb, rec))
  __device__ __forceinline__ int64_t at(int nt, int rb) const { return rbase[nt] + rin[nt] * rb; }
};

template <int D>
__device__ __forceinline__ TileLoc<D> locate(const KeyJob &job, int64_t key0, int n) {
  TileLoc<D> L;
  const int64_t total = job.n_slots * job.n_tokens;
  // the wave-uniform part: slot and token of the tile's first key (a multiply and
  // a shift when the sizes allow it)
  int64_t slot0, b0;
  if (total < (int64_t(1) << 31)) {
    slot0 = div_by(static_cast<uint32_t>(key0), job.tok_m, job.tok_s);
    b0 = div_by(static_cast<uint32_t>(slot0), job.head_m, job.head_s);
  } else {
    slot0 = key0 / job.n_tokens;
    b0 = slot0 / job.heads;
  }
  const int64_t t00 = key0 - slot0 * job.n_tokens;
  const int64_t h0 = slot0 - b0 * job.heads;
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    const int off = nt * 16 + n;
    L.valid[nt] = key0 + off < total;
    int64_t slot, t, b, h;
    if (job.n_tokens >= Geo<D>::KT) {
      // at most one slot boundary inside the tile
      t = t00 + off;
      slot = slot0;
      b = b0;
      h = h0;
      if (t >= job.n_tokens) {
        t -= job.n_tokens;
        ++slot;
        if (++h == job.heads) { h = 0; ++b; }
      }
    } else {
      const int64_t key = L.valid[nt] ? key0 + off : 0;
      slot = key / job.n_tokens;
      t = key - slot * job.n_tokens;
      b = slot / job.heads;
      h = slot - b * job.heads;
    }
    L.src[nt] = b * job.batch_stride + h * job.head_stride + t * job.token_stride;
    const int64_t row = slot * job.capacity + job.token_offset + t;
    L.rbase[nt] = (row >> 5) * job.rec;
    L.rin[nt] = static_cast<int>(row & 31);
  }
  return L;
}

template <int D, bool BF16>
__device__ __forceinline__ void load_keys(const KeyJob &job, const TileLoc<D> &L, int g, RawKeys<D, BF16> &R) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt)
#pragma unroll
    for (int k = 0; k < Geo<D>::KS; ++k) {
      const int64_t off = L.src[nt] + 32 * k + 8 * g;
      if (BF16) {
        R.v[nt][k][0] = L.valid[nt] ? stream_load(reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(job.k) + off))
                                    : make_uint4(0, 0, 0, 0);
      } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(job.k) + off);
        R.v[nt][k][0] = L.valid[nt] ? stream_load(p) : make_uint4(0, 0, 0, 0);
        R.v[nt][k][1] = L.valid[nt] ? stream_load(p + 1) : make_uint4(0, 0, 0, 0);
      }
    }
}

// Keys as B operands.  n = ||x|| (lanes n, n+16, n+32, n+48 hold one key).
// bf16: x' = 2^s x with n 2^s in [128, 256), an exact f16 vector (uh; ul
// stays zero), and yscale = 1 / (n 2^s) turns the rotation product (with
// 2^8 Pi) into y' = 2^8 y.  fp32: u' = 2^8 x / n split into hi/lo and
// yscale = 2^-8.
template <int D, bool BF16>
__device__ __forceinline__ void prepare_keys(const RawKeys<D, BF16> &R, float (&nrm)[Geo<D>::NT],
                                             float (&yscale)[Geo<D>::NT], Ops<D> &uh, Ops<D> &ul) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    float x[Geo<D>::KS][8];
#pragma unroll
    for (int k = 0; k < Geo<D>::KS; ++k) {
      if (BF16) {
        const uint32_t wv[4] = {R.v[nt][k][0].x, R.v[nt][k][0].y, R.v[nt][k][0].z, R.v[nt][k][0].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[k][2 * j] = __uint_as_float(wv[j] << 16);
          x[k][2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
        }
      } else {
        const uint32_t wv[8] = {R.v[nt][k][0].x, R.v[nt][k][0].y, R.v[nt][k][0].z, R.v[nt][k][0].w,
                                R.v[nt][k][1].x, R.v[nt][k][1].y, R.v[nt][k][1].z, R.v[nt][k][1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) x[k][j] = __uint_as_float(wv[j]);
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < Geo<D>::KS; ++k)
#pragma unroll
      for (int s = 0; s < 8; ++s) ss = fmaf(x[k][s], x[k][s], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // (hardware square root and reciprocal below, each within 1 ulp: the norm is stored
    // to fp32 accuracy, and the scale moves every projection by the same factor, far
    // inside the decision windows)
    const float n = __builtin_amdgcn_sqrtf(ss);
    nrm[nt] = n;
    if (BF16) {
      int e = 0;
      (void)frexpf(n, &e);                                       // n = f 2^e, f in [0.5, 1)
      e = max(-100, min(e, 120));
      const float sc = n > 0.0f ? ldexpf(1.0f, 8 - e) : 0.0f;   // n sc in [128, 256)
      yscale[nt] = n > 0.0f ? __builtin_amdgcn_rcpf(n * sc) : 0.0f;
#pragma unroll
      for (int k = 0; k < Geo<D>::KS; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uh[nt][k].w[j] = pack_f16(x[k][2 * j] * sc, x[k][2 * j + 1] * sc);
          ul[nt][k].w[j] = 0u;
        }
    } else {
      const float inv = n > 0.0f ? kUp / n : 0.0f;
      const float minus1 = opaque_minus1();
      yscale[nt] = kDown8;
#pragma unroll
      for (int k = 0; k < Geo<D>::KS; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          split_pair(x[k][2 * j] * inv, x[k][2 * j + 1] * inv, uh[nt][k].w[j], ul[nt][k].w[j], minus1);
    }
  }
}

// The A operands (hi, lo per k-step) of one 16-row slab, fetched from LDS one
// slab ahead of their use so the matrix products do not wait on LDS latency
template <int D>
struct SlabOps {
  v8h a[Geo<D>::KS][2];
};

template <int D>
__device__ __forceinline__ void fetch_slab(SlabOps<D> &A, const uint8_t *slab) {
#pragma unroll
  for (int k = 0; k < Geo<D>::KS; ++k) {
    A.a[k][0] = lds_op(slab + (2 * k) * 1024);
    A.a[k][1] = lds_op(slab + (2 * k + 1) * 1024);
  }
}

// Index stage state across the coordinate tiles of one key tile
template <int D, int W>
struct IndexState {
  static constexpr int NB = (1 << W) - 1;
  static constexpr int NU = W > 0 ? (1 << (W - 1)) - 1 : 0;   // boundaries above the middle one
  float bnd[NB], cen[NB + 1];                // scaled by 2^8
  uint32_t wv[W][Geo<D>::NT];                // words being built, most significant bit first
  float esq[Geo<D>::NT];                     // ||2^8 e||^2 (this lane's part)
  float bts[NU > 0 ? NU : 1][Geo<D>::NT];    // symmetric codebook: upper boundaries / yscale, per key
  float minus1;                              // -1, opaque (split_pair)
};

// An odd-symmetric codebook (c[K-1-i] = -c[i], b[K-2-i] = -b[i], middle
// boundary 0, K = 2^W), as Lloyd-Max gives for the symmetric coordinate law,
// is indexed from the sign and |y| alone: for s = (y > 0) and m = the number
// of upper boundaries below |y|, idx = s ? K/2 + m : K/2 - 1 - m, i.e. the top
// bit is s and the lower bits are those of m, inverted when s = 0; the
// centroid is sign(y) c[K/2 + m].
template <int W>
__device__ __forceinline__ bool codebook_symmetric(const KeyJob &job) {
  if constexpr (W == 0) {
    return false;
  } else {
    constexpr int K = 1 << W;
    bool sym = job.boundaries[K / 2 - 1] == 0.0f;
#pragma unroll
    for (int i = 0; i < K / 2; ++i) sym = sym && job.centroids[K - 1 - i] == -job.centroids[i];
#pragma unroll
    for (int i = 0; i < K / 2 - 1; ++i) sym = sym && job.boundaries[K - 2 - i] == -job.boundaries[i];
    return sym;
  }
}

template <int D, int W>
__device__ __forceinline__ void index_codebook(const KeyJob &job, IndexState<D, W> &S) {
  S.minus1 = opaque_minus1();
#pragma unroll
  for (int i = 0; i < IndexState<D, W>::NB; ++i) S.bnd[i] = job.boundaries[i] * kUp;
#pragma unroll
  for (int i = 0; i <= IndexState<D, W>::NB; ++i) S.cen[i] = job.centroids[i] * kUp;
}

template <int D, int W>
__device__ __forceinline__ void index_begin(IndexState<D, W> &S) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) S.esq[nt] = 0.0f;
}

// Symmetric codebook: |y'| > b' <=> |acc| > b' / yscale (yscale > 0; a zero
// key's infinite threshold leaves m = 0)
template <int D, int W>
__device__ __forceinline__ void index_thresholds(IndexState<D, W> &S, const float (&yscale)[Geo<D>::NT]) {
  constexpr int K = 1 << W;
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    const float inv = __builtin_amdgcn_rcpf(yscale[nt]);   // (1 ulp; rcp(0) = +inf)
#pragma unroll
    for (int j = 0; j < IndexState<D, W>::NU; ++j) S.bts[j][nt] = S.bnd[K / 2 + j] * inv;
  }
}

// The words of a finished group: in the symmetric form the top plane collected
// sign bits (1 = negative) and the lower planes the bits of m; idx's top bit is
// the inverted sign and its lower bits are m's xor the sign.  `valid` masks the
// bits a (half) word holds.
template <int D, int W, bool SYM>
__device__ __forceinline__ void finish_words(IndexState<D, W> &S, uint32_t valid) {
  if constexpr (SYM) {
#pragma unroll
    for (int nt = 0; nt < Geo<D>::NT; ++nt) {
      const uint32_t neg = S.wv[W - 1][nt];
#pragma unroll
      for (int p = 0; p < W - 1; ++p) S.wv[p][nt] ^= neg;
      S.wv[W - 1][nt] = ~neg & valid;
    }
  }
}

// Rotated tile t of the key tile: acc = (2^8 Pi rows of tile t) x (key
// operand); y' = acc * yscale = 2^8 y.  Indices go into the words, e' = y' - c'
// (2^8 e: exact scaling) into the sketch's B operand (slots 4 (t % 2) + i of
// k-step t / 2), e'^2 into esq.  The index is the thermometer count of the
// comparisons; bit p of it is the xor of the comparisons q with
// (q + 1) % 2^p == 0.
// The rotation product of one 16-row tile (matrix cores only); LO = false when
// the rotation's operands are exact (+-1) and their low parts zero
template <int D, bool BF16, bool LO = true>
__device__ __forceinline__ void rot_tile(const SlabOps<D> &A, const Ops<D> &uh, const Ops<D> &ul,
                                         v4f (&acc)[Geo<D>::NT]) {
  constexpr int NT = Geo<D>::NT;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < Geo<D>::KS; ++k) {
    const v8h ah = A.a[k][0];
    const v8h al = A.a[k][1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_v8h(uh[nt][k]), acc[nt], 0, 0, 0);
      if (!BF16) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_v8h(ul[nt][k]), acc[nt], 0, 0, 0);
      if (LO) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, as_v8h(uh[nt][k]), acc[nt], 0, 0, 0);
    }
  }
}

// Indices, residual operand and ||e||^2 of rotated tile t (vector ALU only)
template <int D, int W, bool SYM>
__device__ __forceinline__ void index_vals(int t, const v4f (&acc)[Geo<D>::NT], const float (&yscale)[Geo<D>::NT],
                                           IndexState<D, W> &S, Ops<D> &bh, Ops<D> &bl) {
  constexpr int NT = Geo<D>::NT;
  constexpr int NB = IndexState<D, W>::NB;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float e[4];
    if constexpr (SYM) {
      constexpr int K = 1 << W;
      constexpr int NU = IndexState<D, W>::NU;
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        const float av = acc[nt][i];
        const float aa = fabsf(av);
        bool a[NU > 0 ? NU : 1];
        float cm = S.cen[K / 2];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
          a[j] = aa > S.bts[j][nt];
          cm = a[j] ? S.cen[K / 2 + 1 + j] : cm;
        }
        // top plane: the sign bit of y (inverted when the group's words finish)
        S.wv[W - 1][nt] = __builtin_amdgcn_alignbit(S.wv[W - 1][nt], __float_as_uint(av), 31);
#pragma unroll
        for (int p = 0; p < W - 1; ++p) {
          bool bit = false;
#pragma unroll
          for (int j = 0; j < NU; ++j)
            if (((j + 1) & ((1 << p) - 1)) == 0) bit ^= a[j];
          S.wv[p][nt] = push_bit(S.wv[p][nt], bit);
        }
        // e' = sign(y) (|y'| - c'_m) = y' - sign(y) c'_m (yscale >= 0; rounding is symmetric)
        // (the empty asm keeps the negation on the fma's operand instead of
        // an extra sign flip of av)
        float cs = copysignf(cm, av);
        asm("" : "+v"(cs));
        e[i] = fmaf(av, yscale[nt], -cs);
        S.esq[nt] = fmaf(e[i], e[i], S.esq[nt]);
      }
    } else {
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      const float y = acc[nt][i] * yscale[nt];
      bool c[NB];
      float cv = S.cen[0];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        c[q] = y > S.bnd[q];
        cv = c[q] ? S.cen[q + 1] : cv;
      }
#pragma unroll
      for (int p = 0; p < W; ++p) {
        bool bit = false;
#pragma unroll
        for (int q = 0; q < NB; ++q)
          if (((q + 1) & ((1 << p) - 1)) == 0) bit ^= c[q];
        S.wv[p][nt] = push_bit(S.wv[p][nt], bit);
      }
      e[i] = y - cv;
      S.esq[nt] = fmaf(e[i], e[i], S.esq[nt]);
    }
    }
    split_pair(e[0], e[1], bh[nt][t >> 1].w[2 * (t & 1)], bl[nt][t >> 1].w[2 * (t & 1)], S.minus1);
    split_pair(e[2], e[3], bh[nt][t >> 1].w[2 * (t & 1) + 1], bl[nt][t >> 1].w[2 * (t & 1) + 1], S.minus1);
  }
}

template <int D, int W, bool BF16, bool SYM, bool LO>
__device__ __forceinline__ void index_tile(int t, const SlabOps<D> &A, const Ops<D> &uh, const Ops<D> &ul,
                                           const float (&yscale)[Geo<D>::NT], IndexState<D, W> &S, Ops<D> &bh,
                                           Ops<D> &bl) {
  v4f acc[Geo<D>::NT];
  rot_tile<D, BF16, LO>(A, uh, ul, acc);
  index_vals<D, W, SYM>(t, acc, yscale, S, bh, bl);
}

// Word group wl of the coordinates: its tiles (8, or 4 for a trailing group)
// from the last down, so the bits arrive most significant first.  `group`
// points at this lane's bytes of the group's first slab.
template <int D, int W, bool BF16, bool SYM, bool LO>
__device__ __forceinline__ void index_group(int wl, const uint8_t *group, int g, const Ops<D> &uh, const Ops<D> &ul,
                                            const float (&yscale)[Geo<D>::NT], IndexState<D, W> &S,
                                            uint32_t (&cw)[W][Geo<D>::NT][Geo<D>::WPL], Ops<D> &bh, Ops<D> &bl) {
  constexpr int NT = Geo<D>::NT;
  const int cnt = wl < Geo<D>::FD ? 8 : 4;
#pragma unroll
  for (int p = 0; p < W; ++p)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S.wv[p][nt] = 0u;
  SlabOps<D> A[2];
  fetch_slab<D>(A[(cnt - 1) & 1], group + (cnt - 1) * Geo<D>::SLAB);
#pragma unroll
  for (int j = cnt - 1; j >= 0; --j) {
    if (j > 0) fetch_slab<D>(A[(j - 1) & 1], group + (j - 1) * Geo<D>::SLAB);
    index_tile<D, W, BF16, SYM, LO>(8 * wl + j, A[j & 1], uh, ul, yscale, S, bh, bl);
  }
  finish_words<D, W, SYM>(S, cnt == 8 ? 0xffffffffu : 0xffffu);
#pragma unroll
  for (int p = 0; p < W; ++p)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v = S.wv[p][nt];
      if (cnt == 4) {
        // trailing group: lane groups g and g ^ 1 each hold half of one word
        v <<= 16 * (g & 1);
        v |= __shfl_xor(v, 16);
      }
      asm volatile("" : "+v"(v));   // materialise the word now (see the resident kernel)
      cw[p][nt][wl] = v;
    }
}

template <int D, int W>
__device__ __forceinline__ void index_end(const IndexState<D, W> &S, const float (&nrm)[Geo<D>::NT],
                                          float (&gam)[Geo<D>::NT]) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    float esq = S.esq[nt];
    esq += __shfl_xor(esq, 16);
    esq += __shfl_xor(esq, 32);
    gam[nt] = nrm[nt] * (__builtin_amdgcn_sqrtf(esq) * kDown8);
  }
}

// One 16-row sketch slab tz: z = slab x (e' or the key operand), sign bits
// into sw at 4 (tz % 8) + i (trailing group: 4 (tz % 4) + i, then the half
// words merge); a word is stored as soon as its group is complete.
template <int D, bool THREE>
__device__ __forceinline__ void sketch_slab(const KeyJob &job, const SlabOps<D> &A, int tz, int FM, int g,
                                            const Ops<D> &bh, const Ops<D> &bl, const float (&nrm)[Geo<D>::NT],
                                            const TileLoc<D> &L, uint32_t (&sw)[Geo<D>::NT]) {
  constexpr int NT = Geo<D>::NT;
  v4f z[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) z[nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < Geo<D>::KS; ++k) {
    const v8h ah = A.a[k][0];
    const v8h al = A.a[k][1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      z[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_v8h(bh[nt][k]), z[nt], 0, 0, 0);
      if (THREE) z[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, as_v8h(bl[nt][k]), z[nt], 0, 0, 0);
      z[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, as_v8h(bh[nt][k]), z[nt], 0, 0, 0);
    }
  }
  const bool full = tz < 8 * FM;
  const int sub = full ? (tz & 7) : (tz & 3);
  const int srow_bytes = job.m / 8;
  // sw collects the sign bits of z (bit 4 sub + i from z[i]); a sign bit set
  // means z < 0 (z is never -0: the accumulation starts at +0), so the stored
  // word is its complement, all ones for a zero key
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint32_t nib = 0u;
#pragma unroll
    for (int i = 3; i >= 0; --i) nib = __builtin_amdgcn_alignbit(nib, __float_as_uint(z[nt][i]), 31);
    sw[nt] |= nib << (4 * sub);
  }
  if (full && sub == 7) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t v = nrm[nt] > 0.0f ? ~sw[nt] : 0xffffffffu;
      if (L.valid[nt]) reinterpret_cast<uint32_t *>(job.signs + L.at(nt, srow_bytes))[4 * (tz >> 3) + g] = v;
      sw[nt] = 0u;
    }
  } else if (!full && sub == 3) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint32_t v = (nrm[nt] > 0.0f ? ~sw[nt] : 0xffffffffu) & 0xffffu;
      v <<= 16 * (g & 1);
      v |= __shfl_xor(v, 16);
      if (L.valid[nt] && (g & 1) == 0)
        reinterpret_cast<uint32_t *>(job.signs + L.at(nt, srow_bytes))[4 * FM + (g >> 1)] = v;
      sw[nt] = 0u;
    }
  }
}

template <int D, int W>
__device__ __forceinline__ void store_codes_norms(const KeyJob &job, const TileLoc<D> &L, int g,
                                                  const uint32_t (&cw)[W > 0 ? W : 1][Geo<D>::NT][Geo<D>::WPL],
                                                  const float (&nrm)[Geo<D>::NT], const float (&gam)[Geo<D>::NT]) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    if (!L.valid[nt]) continue;
    if constexpr (W > 0) {
      uint8_t *crow = job.codes + L.at(nt, W * D / 8);
#pragma unroll
      for (int p = 0; p < W; ++p) {
        uint32_t *plane = reinterpret_cast<uint32_t *>(crow + p * (D / 8));
#pragma unroll
        for (int wl = 0; wl < Geo<D>::FD; ++wl) plane[4 * wl + g] = cw[p][nt][wl];
        if constexpr (Geo<D>::TD % 8 != 0)
          if ((g & 1) == 0) plane[4 * Geo<D>::FD + (g >> 1)] = cw[p][nt][Geo<D>::FD];
      }
    }
    if (g == 0) {
      // fp32 or half rows (rec_row's record term is common to both widths)
      const bool sf = job.sf != 0;
      store_side(job.norm + L.rbase[nt], L.rin[nt], sf, nrm[nt]);
      if constexpr (W > 0) store_side(job.rnorm + L.rbase[nt], L.rin[nt], sf, gam[nt]);
    }
  }
}

// Wave-wide copy of `bytes` (a multiple of 1 KiB) of operands into LDS,
// 1 KiB per instruction, waves taking turns.
__device__ __forceinline__ void copy_to_lds(const uint8_t *src, uint8_t *dst, int bytes, int wave, int lane) {
  for (int off = wave * 1024; off < bytes; off += kWaves * 1024)
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src + off + 16 * lane), (lds_u8 *)(dst + off), 16, 0,
                                     0);
}

template <int D>
__device__ __forceinline__ void key_operand_as_sketch_input(const Ops<D> &uh, const Ops<D> &ul, Ops<D> &bh,
                                                            Ops<D> &bl, float (&gam)[Geo<D>::NT]) {
#pragma unroll
  for (int nt = 0; nt < Geo<D>::NT; ++nt) {
    gam[nt] = 0.0f;
#pragma unroll
    for (int k = 0; k < Geo<D>::KS; ++k) {
      bh[nt][k] = uh[nt][k];
      bl[nt][k] = ul[nt][k];
    }
  }
}

// ---- resident operands: the whole operand set sits in LDS; every wave then
// walks its own key tiles (no block synchronisation), the next tile's keys
// loading while the current one is computed.  A tile is rotated and indexed
// first (each rotation tile issued one tile ahead of its index work), then
// sketched slab by slab from the residual operands built by the indexing.
template <int D, int W, bool BF16, int TMS, bool SYM, bool EXACT>
__device__ __forceinline__ void resident_body(const KeyJob &job, int64_t n_tiles, uint8_t *smem) {
  using Gm = Geo<D>;
  constexpr int NT = Gm::NT;
  constexpr int KS = Gm::KS;
  constexpr bool THREE = W > 0 || !BF16;   // the sketch's B operand has a low part
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  constexpr int pi_slabs = W > 0 ? Gm::TD : 0;
  const uint8_t *pi_lds = smem + 16 * lane;
  const uint8_t *sk_lds = smem + pi_slabs * Gm::SLAB + 16 * lane;

  int64_t tile = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  if (tile >= n_tiles) return;
  IndexState<D, W> S;
  if constexpr (W > 0) index_codebook<D, W>(job, S);
  // EXACT: a one-magnitude rotation a * (+-1): operands +-1, y = a * (the product)
  const float rot_a = EXACT ? job.rot_scale[0] : 0.0f;
  constexpr bool lo_pass = !EXACT;
  RawKeys<D, BF16> R;
  // Lk: where the keys in R came from; kept for the tile's stores
  TileLoc<D> Lk = locate<D>(job, tile * Gm::KT, n);
  load_keys<D, BF16>(job, Lk, g, R);
  for (; tile < n_tiles; tile += stride) {
    float nrm[NT], yscale[NT];
    Op uh[NT][KS], ul[NT][KS];
    prepare_keys<D, BF16>(R, nrm, yscale, uh, ul);
    if constexpr (EXACT)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) yscale[nt] *= rot_a;
    uint32_t cw[W > 0 ? W : 1][NT][Gm::WPL];
    float gam[NT];
    Ops<D> bh, bl;   // the sketch's B operand, every k-step
    if constexpr (W > 0) {
      // 1. rotation and indices.  k-steps from the last down: tiles 2k+1, 2k
      // keep the word bits most significant first.  Each tile's rotation is
      // issued one tile ahead of its index work, so the matrix products of the
      // next tile and the vector work of the current one are independent.
      index_begin<D, W>(S);
      if constexpr (SYM) index_thresholds<D, W>(S, yscale);
      // The operands of each rotation tile are fetched from LDS one tile ahead.
      SlabOps<D> A[2];
      v4f acc_hi[NT], acc_lo[NT];
      fetch_slab<D>(A[1], pi_lds + (2 * KS - 1) * Gm::SLAB);
      fetch_slab<D>(A[0], pi_lds + (2 * KS - 2) * Gm::SLAB);
      rot_tile<D, BF16, lo_pass>(A[1], uh, ul, acc_hi);
#pragma unroll
      for (int k = KS - 1; k >= 0; --k) {
        const int t_hi = 2 * k + 1;
        const int wl = t_hi >> 3;
        const bool group_top = wl < Gm::FD ? (t_hi & 7) == 7 : (t_hi & 7) == 3;
        if (group_top) {
#pragma unroll
          for (int p = 0; p < W; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S.wv[p][nt] = 0u;
        }
        rot_tile<D, BF16, lo_pass>(A[0], uh, ul, acc_lo);             // tile t_hi - 1
        if (k > 0) fetch_slab<D>(A[1], pi_lds + (t_hi - 2) * Gm::SLAB);
        index_vals<D, W, SYM>(t_hi, acc_hi, yscale, S, bh, bl);
        if (k > 0) {
          rot_tile<D, BF16, lo_pass>(A[1], uh, ul, acc_hi);           // tile t_hi - 2
          fetch_slab<D>(A[0], pi_lds + (t_hi - 3) * Gm::SLAB);
        }
        index_vals<D, W, SYM>(t_hi - 1, acc_lo, yscale, S, bh, bl);
        if (((t_hi - 1) & 7) == 0) {
          // bottom tile of word group wl: the words are complete
          finish_words<D, W, SYM>(S, wl == Gm::FD ? 0xffffu : 0xffffffffu);
#pragma unroll
          for (int p = 0; p < W; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              uint32_t v = S.wv[p][nt];
              if (wl == Gm::FD) {
                v <<= 16 * (g & 1);
                v |= __shfl_xor(v, 16);
              }
              // materialise the word now (empty asm): left alone, the compiler
              // sinks the bit assembly to the stores and keeps every comparison
              // mask alive until then
              asm volatile("" : "+v"(v));
              cw[p][nt][wl] = v;
            }
        }
      }
      index_end<D, W>(S, nrm, gam);
    } else {
      key_operand_as_sketch_input<D>(uh, ul, bh, bl, gam);
    }
    // 2. the sketch, slab by slab (sign words stored as their groups complete),
    // while the next tile's keys stream in
    const TileLoc<D> Lc = Lk;
    if (tile + stride < n_tiles) {
      Lk = locate<D>(job, (tile + stride) * Gm::KT, n);
      load_keys<D, BF16>(job, Lk, g, R);
    }
    uint32_t sw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sw[nt] = 0u;
    SlabOps<D> As[2];
    fetch_slab<D>(As[0], sk_lds);
#pragma unroll
    for (int tz = 0; tz < TMS; ++tz) {
      if (tz + 1 < TMS) fetch_slab<D>(As[(tz + 1) & 1], sk_lds + (tz + 1) * Gm::SLAB);
      sketch_slab<D, THREE>(job, As[tz & 1], tz, TMS / 8, g, bh, bl, nrm, Lc, sw);
    }
    store_codes_norms<D, W>(job, Lc, g, cw, nrm, gam);
  }
}

template <int D, int W, bool BF16, int TMS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void quantize_keys_resident_kernel(
    KeyJob job, int64_t n_tiles) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int pi_slabs = W > 0 ? Geo<D>::TD : 0;
  copy_to_lds(job.ops, smem, (pi_slabs + TMS) * Geo<D>::SLAB, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // uniform choices, each a body of its own (no branch inside the scheduled loops)
  const bool sym = codebook_symmetric<W>(job);
  const bool exact = W > 0 && job.rot_scale[0] > 0.0f;
  if (sym && exact) resident_body<D, W, BF16, TMS, W != 0, W != 0>(job, n_tiles, smem);
  else if (sym) resident_body<D, W, BF16, TMS, W != 0, false>(job, n_tiles, smem);
  else if (exact) resident_body<D, W, BF16, TMS, false, W != 0>(job, n_tiles, smem);
  else resident_body<D, W, BF16, TMS, false, false>(job, n_tiles, smem);
}

// ---- streamed operands (sets larger than LDS): a block quantises one tile
// of 8 x 32 (d = 256: 8 x 16) keys.  The rotation slabs come through LDS one
// word group (8 slabs, at most 128 KiB) at a time, the sketch slabs in
// double-buffered chunks of 2 or 4 slabs.
template <int D, int W, bool BF16, bool SYM, bool EXACT>
__device__ __forceinline__ void stream_body(const KeyJob &job, uint8_t *smem) {
  using Gm = Geo<D>;
  constexpr int NT = Gm::NT;
  constexpr bool THREE = W > 0 || !BF16;
  constexpr int CH = chunk_slabs(D);
  constexpr int CHUNK = CH * Gm::SLAB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int TM = job.m / 16, FM = TM / 8;
  const int64_t key0 = (static_cast<int64_t>(blockIdx.x) * kWaves + wave) * Gm::KT;
  const TileLoc<D> L = locate<D>(job, key0, n);
  const int pi_slabs = W > 0 ? Gm::TD : 0;
  if (W > 0) copy_to_lds(job.ops, smem, std::min(8, Gm::TD) * Gm::SLAB, wave, lane);
  float nrm[NT], yscale[NT];
  Op uh[NT][Gm::KS], ul[NT][Gm::KS];
  {
    RawKeys<D, BF16> R;
    load_keys<D, BF16>(job, L, g, R);
    prepare_keys<D, BF16>(R, nrm, yscale, uh, ul);
  }
  // EXACT: a one-magnitude rotation a * (+-1): operands +-1, y = a * (the product)
  constexpr bool lo_pass = !EXACT;
  if constexpr (EXACT) {
    const float rot_a = job.rot_scale[0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) yscale[nt] *= rot_a;
  }
  uint32_t cw[W > 0 ? W : 1][NT][Gm::WPL];
  float gam[NT];
  Op bh[NT][Gm::KS], bl[NT][Gm::KS];
  if constexpr (W > 0) {
    IndexState<D, W> S;
    index_codebook<D, W>(job, S);
    index_begin<D, W>(S);
    if constexpr (SYM) index_thresholds<D, W>(S, yscale);
#pragma unroll
    for (int wl = 0; wl < Gm::WPL; ++wl) {
      if (wl > 0) {
        __syncthreads();   // every wave is done with the previous group
        copy_to_lds(job.ops + static_cast<int64_t>(8 * wl) * Gm::SLAB, smem,
                    std::min(8, Gm::TD - 8 * wl) * Gm::SLAB, wave, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      index_group<D, W, BF16, SYM, lo_pass>(wl, smem + 16 * lane, g, uh, ul, yscale, S, cw, bh, bl);
    }
    index_end<D, W>(S, nrm, gam);
    __syncthreads();   // every wave is done with the rotation slabs
  } else {
    key_operand_as_sketch_input<D>(uh, ul, bh, bl, gam);
  }
  const int n_chunks = TM / CH;
  auto stage = [&](int c) {
    copy_to_lds(job.ops + static_cast<int64_t>(pi_slabs + c * CH) * Gm::SLAB, smem + (c & 1) * CHUNK, CHUNK, wave,
                lane);
  };
  stage(0);
  uint32_t sw[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) sw[nt] = 0u;
  for (int c = 0; c < n_chunks; ++c) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c + 1 < n_chunks) stage(c + 1);
    const uint8_t *buf = smem + (c & 1) * CHUNK + 16 * lane;
    SlabOps<D> A[2];
    fetch_slab<D>(A[0], buf);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (j + 1 < CH) fetch_slab<D>(A[(j + 1) & 1], buf + (j + 1) * Gm::SLAB);
      sketch_slab<D, THREE>(job, A[j & 1], c * CH + j, FM, g, bh, bl, nrm, L, sw);
    }
  }
  store_codes_norms<D, W>(job, L, g, cw, nrm, gam);
}

template <int D, int W, bool BF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void quantize_keys_stream_kernel(
    KeyJob job) {
  extern __shared__ __align__(16) uint8_t smem[];
  const bool sym = codebook_symmetric<W>(job);
  const bool exact = W > 0 && job.rot_scale[0] > 0.0f;
  if (sym && exact) stream_body<D, W, BF16, W != 0, W != 0>(job, smem);
  else if (sym) stream_body<D, W, BF16, W != 0, false>(job, smem);
  else if (exact) stream_body<D, W, BF16, false, W != 0>(job, smem);
  else stream_body<D, W, BF16, false, false>(job, smem);
}

constexpr size_t kLdsMax = 160 * 1024;

template <int D, int W>
size_t stream_smem() {
  using Gm = Geo<D>;
  const size_t sketch = static_cast<size_t>(2) * chunk_slabs(D) * Gm::SLAB;
  const size_t rot = W > 0 ? static_cast<size_t>(std::min(8, Gm::TD)) * Gm::SLAB : 0;
  return std::max(sketch, rot);
}

template <int D, int W, bool BF16>
hipError_t launch_dwt(const KeyJob &job_in, hipStream_t stream) {
  using Gm = Geo<D>;
  KeyJob job = job_in;
  div_magic(std::max<int64_t>(job.n_tokens, 1), job.tok_m, job.tok_s);
  div_magic(std::max<int64_t>(job.heads, 1), job.head_m, job.head_s);
  const int64_t total = job.n_slots * job.n_tokens;
  const int64_t n_tiles = (total + Gm::KT - 1) / Gm::KT;
  const size_t ops = key_operand_bytes(D, W, job.m);
  const int tm = job.m / 16;
  // resident: d <= 128, every operand in LDS, at most 16 sketch slabs in registers
  bool resident = false;
  if constexpr (D <= 128) resident = ops <= kLdsMax && tm <= 16;
  if (resident) {
    constexpr int DR = D <= 128 ? D : 128;
    auto kern = tm == 4 ? quantize_keys_resident_kernel<DR, W, BF16, 4>
              : tm == 8 ? quantize_keys_resident_kernel<DR, W, BF16, 8>
              : tm == 12 ? quantize_keys_resident_kernel<DR, W, BF16, 12>
                         : quantize_keys_resident_kernel<DR, W, BF16, 16>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(ops));
    if (e != hipSuccess) return e;
    constexpr int64_t kCUs = 256;   // one resident block per compute unit
    const int64_t blocks = std::min<int64_t>(kCUs, (n_tiles + kWaves - 1) / kWaves);
    kern<<<static_cast<unsigned>(blocks), kThreads, ops, stream>>>(job, n_tiles);
  } else {
    auto kern = quantize_keys_stream_kernel<D, W, BF16>;
    const size_t smem = stream_smem<D, W>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    const int64_t blocks = (n_tiles + kWaves - 1) / kWaves;
    kern<<<static_cast<unsigned>(blocks), kThreads, smem, stream>>>(job);
  }
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_dw(const KeyJob &job, hipStream_t stream) {
  return job.dtype == AQKV_BF16 ? launch_dwt<D, W, true>(job, stream) : launch_dwt<D, W, false>(job, stream);
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

size_t key_operand_bytes(int d, int w, int m) {
  const int slabs = (w > 0 ? d / 16 : 0) + m / 16;
  return static_cast<size_t>(slabs) * (d / 32) * 2048;
}

size_t key_operand_header(int d, int w, int m) { return (key_operand_bytes(d, w, m) + 255) / 256 * 256; }

hipError_t launch_key_operands(const float *rotation, const float *sketch, uint8_t *ops, int d, int w, int m,
                               hipStream_t stream) {
  float *scale = reinterpret_cast<float *>(ops + key_operand_header(d, w, m));
  if (w > 0) {
    rotation_scale_kernel<<<1, 256, 0, stream>>>(rotation, d, scale);
  } else {
    // no rotation: the header stays 0 (a one-thread fill, no memset node in a captured graph)
    rotation_scale_kernel<<<1, 256, 0, stream>>>(sketch, 0, scale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = static_cast<int64_t>(key_operand_bytes(d, w, m) / 4);   // one thread per f16 pair
  key_operands_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(rotation, sketch, ops, d, w,
                                                                                      m, scale);
  e = hipGetLastError();
  if (e != hipSuccess || !qjl_shape(d, w, m)) return e;
  return launch_qjl_operands(sketch, ops + key_operand_header(d, w, m) + 256, m, stream);
}

hipError_t launch_quantize_keys_mfma(const KeyJob &job, hipStream_t stream) {
  if (quantize_keys_qjl_supported(job)) return launch_quantize_keys_qjl(job, stream);
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
