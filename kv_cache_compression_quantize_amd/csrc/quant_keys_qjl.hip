// Pure-QJL key quantisation of bf16 keys at head_dim 128 on CDNA4 matrix
// cores (A-QJL article, section "QJL": one sign bit of each row of S x per
// key, plus ||x||; the sketch size k differs per layer group, section
// "A-QJL：自适应分层压缩策略").
//
// z = S x runs on v_mfma_f32_32x32x16_f16 (twice the work of the 16x16x32
// form per instruction, for the same operand registers) with the sketch rows
// as the A side and 32 keys as the B side.  S, scaled by 2^8, is split into
// f16 high and low parts; a bf16 key scaled by the power of two that brings
// ||x|| into [128, 256) is an exact f16 vector, so two products per k-step
// (S_hi x', S_lo x') give z to a relative error of about 2^-22, far inside the
// 1e-5 decision window.  Only signs are kept, so the positive scale never
// needs undoing.
//
// Weight-stationary layout: a block holds the whole sketch in registers, wave
// (row group r, key team t) two 32-row tiles (64 rows: 2 tiles x 8 k-steps x
// hi/lo, 128 VGPRs), W = k / 64 row groups of 64 keys a tile (k = 320 and 384:
// 2 W waves of one tile each).  The operand rows are permuted so that the 32 C
// rows a lane holds for one key (16 of each tile) are exactly one 32-bit word of
// the key's sign row.  A block walks
// tiles of 64 keys with one barrier per tile.  Keys travel HBM -> LDS by
// buffer_load_dwordx4 ... lds into a four-slot ring, issued three tiles ahead;
// while the matrix instructions of tile i run, the block prepares tile i + 1:
// each key's norm is reduced across the 16 lanes that hold its pieces, and the
// key, scaled by the power of two that brings its norm into [128, 256), is
// converted to f16 and written in operand order into the second of two
// fragment buffers (one 1 KiB fragment per 32 keys and k-step; the 16-byte
// units XOR-swizzled so that both these writes and the operand reads are free
// of bank conflicts).  Each wave's sign words meet in LDS (rows padded to a
// conflict-free stride) and leave as whole 8-byte pieces of each row, one tile
// after the barrier that ends it (kBatch: storing every tile measured faster
// than gathering the rows of 2, 4 or 8 tiles into one burst of stores).
#include <algorithm>

#include "internal.h"

namespace aqkv {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kD = 128;                 // head_dim of this kernel
constexpr int kKS = kD / 16;            // k-steps of a 128-long contraction (16 wide)
constexpr int kTileKeys = 64;           // keys per team and tile
constexpr int kCB = kTileKeys / 32;     // 32-key column blocks per team and tile
constexpr int kRT = 2;                  // 32-row sketch tiles per wave
constexpr int kTileOps = kKS * 2048;    // bytes of one 32-row operand tile (8 k-steps x hi/lo x 1 KiB)
constexpr int kRing = 4;                // raw key tiles in LDS: the one being prepared, three in flight
constexpr int kKeyBuf = kCB * kKS * 1024;   // f16 operand fragments of one team's keys (16 KiB)
constexpr float kUp = 256.0f;           // the sketch is scaled by 2^8 before the split

// Key teams per block (one: the kernel serves sketches of 320 rows and more, W >= 5 row
// groups of 64 rows)
__host__ __device__ constexpr int teams_of(int W) { return 1; }
// Waves per block.  Waves w and w + 4 of a block share a SIMD, so with W waves of two
// 32-row tiles each, W = 5 .. 8, one SIMD always carries four tiles.  For W = 5 and 6 the
// block runs 2 W waves of one tile each instead (wave w takes tile w): every SIMD carries
// at most three tiles on three waves, so more waves hide each other's latencies, and the
// preparation is spread over 128 W threads.  Split this way, a wave's tile is one half of
// a sign word, so its 16 bits go to their half of the word in LDS.
__host__ __device__ constexpr int waves_of(int W) { return W <= 6 ? 2 * W : W; }
__host__ __device__ constexpr bool split_of(int W) { return waves_of(W) != W; }
// Raw loads (1 KiB each) per wave and tile: every wave issues the same number on every
// path through the loop (the loads past a tile's 16 T go to a dummy LDS area, a tile past
// the last reloads a valid key), so the number of vector-memory operations issued after
// any point is fixed and a partial vmcnt wait is exact
__host__ __device__ constexpr int loads_per_wave(int W) {
  return (16 * teams_of(W) + waves_of(W) * teams_of(W) - 1) / (waves_of(W) * teams_of(W));
}
__host__ __device__ constexpr int dummy_bytes(int W) {
  return (loads_per_wave(W) * waves_of(W) * teams_of(W) - 16 * teams_of(W)) * 1024;
}
// Tiles whose sign rows and norms are stored together (one: k = 512 0.96 ms against 0.96,
// 0.99 and 1.00 ms for 2, 4 and 8; k = 384 0.85 against 0.85, 0.86 and 0.87 ms)
constexpr int kBatch = 1;

// Sign-row stride in LDS, in 4-byte words: at least the row, 2 mod 4 so that the 32 keys
// a wave writes (and 2 words each) land in 64 different banks
__host__ __device__ constexpr int sgn_words(int W) { return 2 * W + ((2 - 2 * W) % 4 + 4) % 4; }

// LDS of one block: the raw ring, two fragment buffers, the norms and scales of a batch,
// the tile in the matrix units and the one being prepared, the sign rows of a batch and
// the tile being finished, the dummy load area
__host__ __device__ constexpr int raw_bytes(int T) { return kTileKeys * T * 256; }
__host__ __device__ constexpr int qjl_smem(int W) {
  return kRing * raw_bytes(teams_of(W)) + 2 * kKeyBuf * teams_of(W) + 2 * (kBatch + 2) * kTileKeys * teams_of(W) * 4 +
         (kBatch + 1) * kTileKeys * teams_of(W) * 4 * sgn_words(W) + dummy_bytes(W);
}

// Swizzled position of 16-byte unit u of a fragment buffer: unit u = 64 (8 cb + ks) +
// 32 hh + key holds dims 16 ks + 8 hh .. + 7 of the block's key; its low 4 bits are xored
// with the piece number 2 ks + hh, so the 16 pieces of one key land in 16 banks and a
// wave's 64 consecutive operand reads stay conflict-free
__host__ __device__ constexpr int frag_unit(int u) { return u ^ ((u >> 5) & 15); }

// LDS position (16-byte unit) of piece p of key i in a raw tile: key-major, the pieces
// XOR-swizzled so that the same piece of 16 consecutive keys sits in 16 different banks
__host__ __device__ constexpr int raw_unit(int i, int p) { return 16 * i + (p ^ (i & 15)); }

// Element of a 32-element bit-row word that holds bit b (bit 8 k + i is element 4 i + k)
__host__ __device__ constexpr int word_element(int b) { return 4 * (b & 7) + (b >> 3); }

// The sketch row behind row r of 32-row operand tile t: wave t / 2, its tile t % 2; C row
// r = 8 q + 4 h + i of a 32x32 product sits in lane half h, register 4 q + i, and a lane
// collects bit 16 (t % 2) + 4 q + i of word 2 (t / 2) + h of each key's sign row
__host__ __device__ inline int qjl_row(int t, int r) {
  const int q = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return 32 * (2 * (t >> 1) + h) + word_element(16 * (t & 1) + 4 * q + i);
}

// One thread per (tile, k-step, lane, slot): the high and low f16 parts of one A-operand
// element (scaled by 2^8); lane l, slot s of k-step ks holds row l % 32, column
// 16 ks + 8 (l / 32) + s
__global__ __launch_bounds__(256) void qjl_operands_kernel(const float *__restrict__ sketch,
                                                           uint8_t *__restrict__ ops, int m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(m / 32) * kKS * 512) return;
  const int s = static_cast<int>(idx & 7);
  const int lane = static_cast<int>((idx >> 3) & 63);
  const int ks = static_cast<int>((idx >> 9) % kKS);
  const int t = static_cast<int>((idx >> 9) / kKS);
  const int row = qjl_row(t, lane & 31);
  const float v = sketch[static_cast<int64_t>(row) * kD + 16 * ks + 8 * (lane >> 5) + s] * kUp;
  const _Float16 hi = static_cast<_Float16>(v);
  const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
  uint8_t *base = ops + (static_cast<int64_t>(t) * kKS + ks) * 2048 + lane * 16 + 2 * s;
  *reinterpret_cast<_Float16 *>(base) = hi;
  *reinterpret_cast<_Float16 *>(base + 1024) = lo;
}

// Where key kk (flat over slots x tokens) comes from and goes to
struct KeyAt {
  int64_t src;   // element offset in the K view
  int64_t row;   // cache row (slot * capacity + token_offset + t)
};

// The tile's first key, located once per tile (wave-uniform)
struct TileBase {
  int64_t slot, b, h, t;
};

__device__ __forceinline__ TileBase tile_base(const KeyJob &job, int64_t key0) {
  TileBase B;
  const int64_t total = job.n_slots * job.n_tokens;
  if (total < (int64_t(1) << 31)) {
    B.slot = div_by(static_cast<uint32_t>(key0), job.tok_m, job.tok_s);
    B.b = div_by(static_cast<uint32_t>(B.slot), job.head_m, job.head_s);
  } else {
    B.slot = key0 / job.n_tokens;
    B.b = B.slot / job.heads;
  }
  B.t = key0 - B.slot * job.n_tokens;
  B.h = B.slot - B.b * job.heads;
  return B;
}

// Key i of the tile that starts at key0 (i < 128: at most one slot boundary when a
// slot holds at least 128 tokens; otherwise a division per key)
__device__ __forceinline__ KeyAt key_at(const KeyJob &job, const TileBase &B, int64_t key0, int i) {
  int64_t slot, t, b, h;
  if (job.n_tokens >= 2 * kTileKeys) {
    t = B.t + i;
    slot = B.slot;
    b = B.b;
    h = B.h;
    if (t >= job.n_tokens) {
      t -= job.n_tokens;
      ++slot;
      if (++h == job.heads) {
        h = 0;
        ++b;
      }
    }
  } else {
    const int64_t kk = key0 + i;
    slot = kk / job.n_tokens;
    t = kk - slot * job.n_tokens;
    b = slot / job.heads;
    h = slot - b * job.heads;
  }
  KeyAt a;
  a.src = b * job.batch_stride + h * job.head_stride + t * job.token_stride;
  a.row = slot * job.capacity + job.token_offset + t;
  return a;
}

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The raw bf16 keys of a tile into a ring slot (raw_unit order): wave `wave` issues loads
// wave * IPW .. + IPW - 1, each filling 64 units of 16 B (4 keys; lane l fills unit
// 64 ins + l with the piece raw_unit assigns to it); loads past the tile's 16 T go to the
// dummy area.  A tile inside one slot (the usual case) is read
// through a buffer resource over its key rows, with per-lane offsets (voff, computed
// once: lane pieces of load j) that never change, so no register of a load in flight is
// ever rewritten; keys past the last one fall outside the resource and read as 0.  A
// tile across a slot boundary takes per-lane global addresses instead, kept in fb (the
// caller keeps fb in registers of its own across the loop, so only such tiles rewrite
// them; a key past the last reads the tile's first key, and norms() gives it scale 0).
// A tile past the last one reads key 0 and is never used.
template <int W, int T>
__device__ __forceinline__ void load_tile(const KeyJob &job, int64_t tile, int64_t n_tiles, int64_t total,
                                          uint8_t *slot, uint8_t *dummy, int wave, int lane,
                                          const uint32_t (&voff)[loads_per_wave(W)],
                                          const uint16_t *(&fb)[loads_per_wave(W)]) {
  constexpr int IPW = loads_per_wave(W);
  constexpr int TK = kTileKeys * T;
  const int64_t key0 = tile < n_tiles ? tile * TK : 0;
  const TileBase B = tile_base(job, key0);
  const uint16_t *k = static_cast<const uint16_t *>(job.k);
  const int64_t n_valid = min<int64_t>(TK, total - key0);
  if (B.t + n_valid <= job.n_tokens) {
    const uint16_t *base = k + B.b * job.batch_stride + B.h * job.head_stride + B.t * job.token_stride;
    const uint32_t bytes = static_cast<uint32_t>(((n_valid - 1) * job.token_stride + kD) * 2);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, static_cast<int>(bytes), 0x00020000);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int ins = wave * IPW + j;
      uint8_t *dst = ins < 16 * T ? slot + ins * 1024 : dummy + (ins - 16 * T) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8 *)dst, 16, static_cast<int>(voff[j]), 0, 0, kStreamPolicy);
    }
  } else {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int ins = wave * IPW + j;
      const bool real = ins < 16 * T;
      const int c = (real ? ins : 0) * 64 + lane;
      const int i = c >> 4, part = (c & 15) ^ (i & 15);
      const KeyAt a = key_at(job, B, key0, key0 + i < total ? i : 0);
      uint8_t *dst = real ? slot + ins * 1024 : dummy + (ins - 16 * T) * 1024;
      fb[j] = k + a.src + 8 * part;
      __builtin_amdgcn_global_load_lds(static_cast<const void *>(fb[j]), (lds_u8 *)dst, 16, 0, kStreamPolicy);
    }
  }
}

// Block barrier for LDS hand-offs only: this wave's LDS reads and writes are complete
// (lgkmcnt 0), then s_barrier.  __syncthreads() would add a workgroup release fence,
// which waits for every vector-memory access in flight (vmcnt 0) and so would drain the
// key loads issued ahead; global memory needs no ordering across these barriers.  The
// signal fences keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0); vmcnt, expcnt unchanged
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// sum over the 16 lanes of a DPP row, in every lane of the row
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2h));
}

// Prepares a raw tile (units c = tid + j * threads; the 16 consecutive lanes of a DPP row
// hold the 16 pieces of one key, in raw_unit order): each key's norm and scale (keys
// past the last get 0), and the scaled f16 operand fragments
template <int W, int T>
__device__ __forceinline__ void stage(const uint8_t *raw, uint8_t *kbuf, float *knorm, int64_t key0,
                                      int64_t total) {
  constexpr int NT = 64 * waves_of(W) * T, PIECES = 1024 * T, CPT = (PIECES + NT - 1) / NT;
  // (unrolled, so that every piece's LDS read is in flight at once: k = 512 0.971 ->
  // 0.950 ms, k = 384 0.821 -> 0.808 ms against the rolled loop, no spills)
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = static_cast<int>(threadIdx.x) + j * NT;
    if (CPT * NT > PIECES && c >= PIECES) continue;   // whole rows of 16 lanes skip together
    const int i = c >> 4, part = (c & 15) ^ (i & 15);
    const uint4 rv = *reinterpret_cast<const uint4 *>(raw + c * 16);
    const uint32_t wv[4] = {rv.x, rv.y, rv.z, rv.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(wv[e] << 16);
      x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
    }
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = row_sum16(ss);
    // (the hardware square root, within 1 ulp: the norm is stored to fp32 accuracy and
    // only its exponent picks the scale, which never changes a sign)
    const float n = key0 + i < total ? __builtin_amdgcn_sqrtf(ss) : 0.0f;
    int ex = 0;
    (void)frexpf(n, &ex);                                      // n = f 2^ex, f in [0.5, 1)
    ex = max(-100, min(ex, 120));
    const float sc = n > 0.0f ? ldexpf(1.0f, 8 - ex) : 0.0f;   // n sc in [128, 256)
    uint4 h;
    h.x = pack_f16(x[0] * sc, x[1] * sc);
    h.y = pack_f16(x[2] * sc, x[3] * sc);
    h.z = pack_f16(x[4] * sc, x[5] * sc);
    h.w = pack_f16(x[6] * sc, x[7] * sc);
    // fragment (column block i / 32, k-step part / 2), lane (k half part % 2, key i % 32)
    const int u = ((i >> 5) * kKS + (part >> 1)) * 64 + ((part & 1) << 5) + (i & 31);
    *reinterpret_cast<uint4 *>(kbuf + frag_unit(u) * 16) = h;
    if ((c & 15) == 0) knorm[i] = n;
  }
}

// The sign rows and norms of tiles batch0, batch0 + stride, .. (count of them, from sign
// slots s0, s0 + 1, .. and norm slots n0, n0 + 1, .., modulo the slot counts): per tile one
// 8-byte piece of one key's row per thread and the norms.  Every value and address is
// gathered first, each in registers of its own, so no store's registers are reused before
// the whole batch has been issued.
template <int W, int T>
__device__ __forceinline__ void store_batch(const KeyJob &job, int64_t batch0, int64_t stride, int count, int s0,
                                            int n0, const uint32_t *sgn, const float *knorm, int64_t total) {
  constexpr int NB = kBatch, TK = kTileKeys * T, SW = sgn_words(W), srow = 8 * W;
  const int tid = threadIdx.x;
  const int key = tid / W, u = tid - key * W;   // (threads past 64 W store nothing)
  uint2 sv[NB];
  float nv[NB];
  uint2 *sp[NB];
  uint8_t *np[NB];
  bool ok[NB];
  const bool sf = job.sf != 0;   // half norms (else fp32)
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t key0 = (batch0 + j * stride) * TK;
    ok[j] = j < count && key < TK && key0 + key < total;
    const TileBase B = tile_base(job, key0);
    const KeyAt a = key_at(job, B, key0, ok[j] ? key : 0);
    const int64_t rb = (a.row >> 5) * job.rec, ri = a.row & 31;
    sp[j] = reinterpret_cast<uint2 *>(job.signs + rb + ri * srow + 8 * u);
    np[j] = job.norm + rb + ri * (sf ? 2 : 4);
    const int kk = key < TK ? key : 0;
    sv[j] = *reinterpret_cast<const uint2 *>(sgn + (((s0 + j) % (NB + 1)) * TK + kk) * SW + 2 * u);
    nv[j] = knorm[((n0 + j) % (NB + 2)) * TK + kk];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    if (ok[j]) {
      *sp[j] = sv[j];
      if (u == 0) {
        if (sf) *reinterpret_cast<_Float16 *>(np[j]) = side_half(nv[j]);
        else *reinterpret_cast<float *>(np[j]) = nv[j];
      }
    }
  }
}

template <int W>
__global__ __launch_bounds__(64 * waves_of(W) * teams_of(W)) void quantize_keys_qjl_kernel(KeyJob job,
                                                                                            const uint8_t *ops,
                                                                                            int64_t n_tiles) {
  constexpr int T = teams_of(W), NB = kBatch;
  constexpr int TK = kTileKeys * T;   // keys per tile
  constexpr int SW = sgn_words(W);
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool kSplit = split_of(W);
  const int rg = kSplit ? 0 : wave % W, team = kSplit ? 0 : wave / W;   // row group and key team of this wave
  // (split: this wave's one tile is tile `wave`)
  constexpr bool two = !kSplit;
  const int n = lane & 31, hh = lane >> 5;
  uint8_t *ring = smem;
  uint8_t *kbuf = ring + kRing * raw_bytes(T);                                 // [2][T][kKeyBuf]
  float *knorm = reinterpret_cast<float *>(kbuf + 2 * kKeyBuf * T);           // [NB + 2][TK]
  uint32_t *sgn = reinterpret_cast<uint32_t *>(knorm + (NB + 2) * TK);        // [NB + 1][TK][SW]
  uint8_t *dummy = reinterpret_cast<uint8_t *>(sgn + (NB + 1) * TK * SW);
  const int64_t total = job.n_slots * job.n_tokens;
  const int64_t stride = gridDim.x;
  constexpr int IPW = loads_per_wave(W);

  // this wave's rows of S: operand tiles 2 rg, 2 rg + 1 (split: tile `wave` alone), every
  // k-step, hi and lo
  v8h A[kRT][kKS][2];
#pragma unroll
  for (int r = 0; r < kRT; ++r) {
    const int t = kSplit ? wave : kRT * rg + r;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        A[r][ks][p] =
            *reinterpret_cast<const v8h *>(ops + static_cast<int64_t>(t) * kTileOps + (2 * ks + p) * 1024 + lane * 16);
  }

  // byte offsets of this lane's pieces of its loads inside a tile's key rows (load j of
  // wave w fills units 64 (w IPW + j) + lane: key = unit / 16, piece per raw_unit)
  uint32_t voff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int ins = wave * IPW + j;
    const int c = (ins < 16 * T ? ins : 0) * 64 + lane;
    const int i = c >> 4, part = (c & 15) ^ (i & 15);
    voff[j] = static_cast<uint32_t>((i * job.token_stride + 8 * part) * 2);
  }
  const uint16_t *fb[IPW];   // per-lane addresses of the slot-crossing tiles' loads
#pragma unroll
  for (int j = 0; j < IPW; ++j) fb[j] = static_cast<const uint16_t *>(job.k);

  int64_t tile = blockIdx.x;
  if (tile >= n_tiles) return;
  // prologue: the first tile loaded and prepared, the next two tiles' loads in flight
  static_assert(kRing == 4, "the waits below count three tiles in flight");
  load_tile<W, T>(job, tile, n_tiles, total, ring, dummy, wave, lane, voff, fb);
  load_tile<W, T>(job, tile + stride, n_tiles, total, ring + raw_bytes(T), dummy, wave, lane, voff, fb);
  load_tile<W, T>(job, tile + 2 * stride, n_tiles, total, ring + 2 * raw_bytes(T), dummy, wave, lane, voff, fb);
  wait_vm<2 * IPW>();
  lds_barrier();
  stage<W, T>(ring, kbuf, knorm, tile * TK, total);
  int64_t batch0 = tile;   // the first tile not yet stored
  int it = 0;
  for (; tile < n_tiles; tile += stride, ++it) {
    // the next tile's raw keys have landed (issued two tiles ago); the loads issued since,
    // for the tile after it, may stay in flight (stores issued in between are waited for
    // too: they are older).  The loads of a third tile go out below, after the stores.
    wait_vm<IPW>();
#pragma unroll
    for (int j = 0; j < IPW; ++j) asm volatile("" ::"v"(fb[j]));
    lds_barrier();   // this tile prepared, the next one's raw keys visible, the last ring slot free
    if (it > 0 && it % NB == 0) {
      store_batch<W, T>(job, batch0, stride, NB, it - NB, it - NB, sgn, knorm, total);
      batch0 = tile;
    }
    const int64_t next = tile + stride;
    load_tile<W, T>(job, next + 2 * stride, n_tiles, total, ring + ((it + 3) % kRing) * raw_bytes(T), dummy, wave,
                    lane, voff, fb);
    const uint8_t *kb = kbuf + (it & 1) * kKeyBuf * T;
    const float *kn = knorm + (it % (NB + 2)) * TK;
    uint32_t *sg = sgn + (it % (NB + 1)) * TK * SW;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int key = team * kTileKeys + cb * 32 + n;
      v8h Bk[kKS];
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        Bk[ks] = *reinterpret_cast<const v8h *>(kb + frag_unit(((team * kCB + cb) * kKS + ks) * 64 + lane) * 16);
      v16f acc[kRT];
#pragma unroll
      for (int r = 0; r < kRT; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[r][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int r = 0; r < kRT; ++r)
            if (r == 0 || two) acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[r][ks][p], Bk[ks], acc[r], 0, 0, 0);
      // the next tile's operands are prepared while the matrix instructions run
      if (cb == 0 && next < n_tiles)
        stage<W, T>(ring + ((it + 1) % kRing) * raw_bytes(T), kbuf + ((it + 1) & 1) * kKeyBuf * T,
                    knorm + ((it + 1) % (NB + 2)) * TK, next * TK, total);
      // bit 16 r + e of the word: the sign of z (set = negative); acc starts at +0, so a
      // zero product sum is never -0.  Stored bit 1 = non-negative projection; a zero key
      // stores all ones.
      if (!kSplit) {
        uint32_t h = 0u;
#pragma unroll
        for (int r = kRT - 1; r >= 0; --r)
#pragma unroll
          for (int e = 15; e >= 0; --e) h = __builtin_amdgcn_alignbit(h, __float_as_uint(acc[r][e]), 31);
        sg[key * SW + 2 * rg + hh] = kn[key] > 0.0f ? ~h : 0xffffffffu;
      } else {
        // tile t's 16 bits: half t % 2 of word 2 (t / 2) + hh
        uint16_t *sg16 = reinterpret_cast<uint16_t *>(sg);
#pragma unroll
        for (int r = 0; r < kRT; ++r) {
          if (r == 0 || two) {
            const int t = wave;
            uint32_t h = 0u;
#pragma unroll
            for (int e = 15; e >= 0; --e) h = __builtin_amdgcn_alignbit(h, __float_as_uint(acc[r][e]), 31);
            sg16[(key * SW + 2 * (t >> 1) + hh) * 2 + (t & 1)] =
                static_cast<uint16_t>(kn[key] > 0.0f ? ~h : 0xffffu);
          }
        }
      }
    }
  }
  // the tiles since the last batch (it >= 1 here); then no load may still be writing LDS
  // when the block exits
  lds_barrier();
  const int done = (it - 1) / NB * NB;
  store_batch<W, T>(job, batch0, stride, it - done, done, done, sgn, knorm, total);
  wait_vm<0>();
}

template <int W>
hipError_t launch_w(const KeyJob &job_in, const uint8_t *ops, hipStream_t stream) {
  constexpr int T = teams_of(W);
  KeyJob job = job_in;
  div_magic(std::max<int64_t>(job.n_tokens, 1), job.tok_m, job.tok_s);
  div_magic(std::max<int64_t>(job.heads, 1), job.head_m, job.head_s);
  auto kern = quantize_keys_qjl_kernel<W>;
  static_assert(qjl_smem(W) <= 160 * 1024, "LDS of one block");
  const int smem = qjl_smem(W);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  if (e != hipSuccess) return e;
  const int64_t total = job.n_slots * job.n_tokens;
  const int64_t n_tiles = (total + kTileKeys * T - 1) / (kTileKeys * T);
  constexpr int64_t kCUs = 256;   // one resident block per compute unit
  const int64_t blocks = std::min<int64_t>(n_tiles, kCUs);
  kern<<<static_cast<unsigned>(blocks), 64 * waves_of(W) * T, smem, stream>>>(job, ops, n_tiles);
  return hipGetLastError();
}

}  // namespace

// (sketches below 320 rows take the resident kernel of quant_keys_mfma.hip: fewer than five
// waves of rows leave the compute unit underfilled here)
bool qjl_shape(int d, int w, int m) { return d == kD && w == 0 && m % 64 == 0 && m >= 320 && m <= 512; }

size_t qjl_operand_bytes(int m) { return static_cast<size_t>(m / 32) * kTileOps; }

hipError_t launch_qjl_operands(const float *sketch, uint8_t *ops, int m, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(m / 32) * kKS * 512;   // one thread per element
  qjl_operands_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, stream>>>(sketch, ops, m);
  return hipGetLastError();
}

bool quantize_keys_qjl_supported(const KeyJob &job) {
  return qjl_shape(job.d, job.w, job.m) && job.dtype == AQKV_BF16;
}

hipError_t launch_quantize_keys_qjl(const KeyJob &job, hipStream_t stream) {
  // the operands of this kernel follow the rotation-scale header of the prepared workspace
  const uint8_t *ops = job.ops + key_operand_header(job.d, job.w, job.m) + 256;
  switch (job.m / 64) {
    case 5: return launch_w<5>(job, ops, stream);
    case 6: return launch_w<6>(job, ops, stream);
    case 7: return launch_w<7>(job, ops, stream);
    default: return launch_w<8>(job, ops, stream);
  }
}

}  // namespace aqkv
