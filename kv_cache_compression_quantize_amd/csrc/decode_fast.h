// Decode attention on the packed cache with CDNA4 matrix cores
// (TurboQuant article §五 estimator, §六 fused decode with online softmax;
// A-QJL article, pure-QJL keys).  Template shared by the per-head_dim
// instantiation files decode_fast_d*.hip.
//
// Scores as integer matrix products on the packed bits.  For a codebook c of
// 2^w levels, c(idx) = c[0] + sum_A kappa_A par_A(idx) over the non-empty
// subsets A of the w index bits, par_A = xor of those bits (a Walsh transform
// of the codebook; for an odd-symmetric Lloyd-Max codebook only the subsets of
// odd size have kappa_A != 0).  Hence
//   <q_rot, c[idx_t]>    = c[0] sum(q_rot) + sum_A kappa_A <q_rot, par_A(t)>
//   <q_sk, 2 bits_t - 1> = 2 <q_sk, bits_t> - sum(q_sk)
// and every score is a fixed combination of dot products between query rows
// and {0,1} bit-planes of the cached keys.  Each block first quantises the
// query side of its heads (kappa_A q_rot, 2 q_sk) to 15-bit integers split into
// int8 hi / lo parts, laid out as ready-made matrix-core A operands.
// v_mfma_i32_16x16x64_i8 then contracts 64 coordinates of 16 tokens for 16
// rows = 4 heads x {mse hi, mse lo, qjl hi, qjl lo} with exact integer
// accumulation; a key bit becomes an int8 {0,1} operand byte with one shift
// and one mask per 4 bits (bit rows are byte-transposed for this).  Pure-QJL
// keys have no mse rows, and spend them on a cheaper sign operand: one mask
// per 4 bits, each bit left at its place e in its byte (value 2^e, -128 for
// e = 7), against query values pre-multiplied by 2^(7 - e) (-1 for e = 7) and
// written as three base-128 digits, rows {Q >> 14, (Q >> 7) & 127, Q & 127}.
//
// Values: out[g] = sum_t p_t (code_t scale_t + min_t).  The f16 operand is the
// code itself in the low mantissa bits with a zero exponent, i.e. the exact
// denormal code * 2^-24 (the matrix cores keep f16 denormals), cut from the
// 32-token block word that holds 8 tokens' codes of one channel with one shift
// and one mask per two codes; the token weights a_t = p_t scale_t are split
// into f16 hi + lo rows and v_mfma_f32_16x16x32_f16 accumulates
// sum_t a_t code_t 2^-24 over 32 tokens; the result is scaled by 2^24 and
// sum_t p_t min_t is added at the end.
//
// Work: block (slot, split) of 4 waves; each wave walks 32-token tiles of the
// block's range (interleaved across waves) with its own online-softmax state.
// Every shape parameter is a template constant, so a tile is straight-line
// code.  A tile is one 32-token block record of the cache (all seven fields
// contiguous); it goes HBM -> LDS with buffer_load_dwordx4 ... lds (per-slot
// buffer resource, wave-uniform record offset) into a per-wave ring of two
// tile buffers, so the next tile streams in while one is computed (ring_of
// below: deeper rings cost resident waves).  The waves merge in LDS;
// combine_kernel merges the splits.
#pragma once

#include <math.h>

#include "internal.h"

namespace aqkv {
namespace fast {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTT = 32;          // tokens per wave tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;    // keep the running max unless a tile exceeds it by 2^8
constexpr int kRegAVgprs = 48;   // query operands live in VGPRs up to this many registers, else in LDS

__host__ __device__ constexpr int popc(int x) { return x ? (x & 1) + popc(x >> 1) : 0; }
// bit A set for every non-empty subset A of the w index bits of odd size / of any size
__host__ __device__ constexpr int odd_planes(int w) {
  int m = 0;
  for (int a = 1; a < (1 << w); ++a)
    if (popc(a) & 1) m |= 1 << a;
  return m;
}
__host__ __device__ constexpr int all_planes(int w) {
  int m = 0;
  for (int a = 1; a < (1 << w); ++a) m |= 1 << a;
  return m;
}
__host__ __device__ constexpr int heads_rb(int g) { return (g + 3) / 4; }
// chunks (64 K-slots each) the pack kernel lays out per row block: all planes + signs
__host__ __device__ constexpr int chunks_max(int d, int w, int m) { return ((1 << w) - 1) * (d / 64) + m / 64; }

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// v_mul_legacy_f32: 0 * x = 0 for every x (Inf and NaN included)
__device__ float fmul_legacy(float a, float b) __asm("llvm.amdgcn.fmul.legacy");

// the low / high IEEE half of a 32-bit word, widened to fp32
__device__ __forceinline__ float half_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Bit-row words hold element j = 4 i + k at bit 8 k + i, so (x >> i) & 0x01010101
// is elements 4i .. 4i+3 as int8 {0,1} bytes.  Half hf of a word (elements
// 16 hf .. 16 hf + 15) -> the 16 operand bytes of one K-chunk.
__device__ __forceinline__ v4i spread_half(uint32_t x, int hf) {
  v4i r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = static_cast<int>((x >> (4 * hf + k)) & 0x01010101u);
  return r;
}
// The same bits left in place, one mask per register: byte b of register k is
// bit (4 hf + k) of byte b of x times 2^(4 hf + k) (as int8: -128 for bit 7);
// the A operand carries the inverse weights (pure-QJL sign chunks).
__device__ __forceinline__ v4i mask_half(uint32_t x, int hf) {
  v4i r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = static_cast<int>(x & (0x01010101u << (4 * hf + k)));
  return r;
}

// max over the 16 lanes of a DPP row, result in every lane of the row: the
// same four lane permutations as row_sum16, through the compiler's DPP move
// (so the compiler places the wait states a DPP read of a fresh VALU result
// needs)
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// Buffer resource over the block records of one slot (raw, untyped loads;
// num_records = bytes, reads past them return 0).  Offsets are 32-bit, so a
// slot's records must span fewer than 2^31 bytes (the host checks this).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Wave-wide asynchronous copy of BYTES (multiple of 16) bytes at byte offset
// soff (wave-uniform) of a plane to LDS: lane l moves bytes 16 l .. 16 l + 15
// of every 1 KiB piece (buffer_load_dwordx4 ... lds, non-temporal: each record
// is read once).
template <int BYTES>
__device__ __forceinline__ void copy_region(__amdgpu_buffer_rsrc_t rs, uint32_t soff, uint8_t *l, int lane) {
#pragma unroll
  for (int off = 0; off < BYTES; off += 1024) {
    if (BYTES - off >= 1024 || 16 * lane < BYTES - off)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_u8 *)(l + off), 16, 16 * lane, static_cast<int>(soff + off), 0,
                                               kStreamPolicy);
  }
}
template <int BYTES>
__host__ __device__ constexpr int loads_of() { return (BYTES + 1023) / 1024; }

// s_waitcnt with only the vector-memory counter limited to N (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Per-head constants the pack kernel writes next to the operands.
struct HeadConst {
  float sig_mse, sig_qjl, c_mse, c_qjl;
};

// value-weight pairs per lane: pair k of lane group pq is (head, group) =
// divmod(pq + 4 k, D / 32)
__host__ __device__ constexpr int pairs_of(int g, int d) { return (g * (d / 32) + 3) / 4; }

// Tile staging: every cache plane of 32 tokens, copied whole into a per-wave
// ring of R buffers (tiles t+1 .. t+R-1 stream in while t is computed).
// (sf: side information stored as half, 2 bytes a number instead of 4)
__host__ __device__ constexpr int tile_bytes_of(int d, int w, int mc, int vb, bool sf) {
  const int e = sf ? 2 : 4;
  return kTT * (w * d / 8 + mc * 8 + e + (w > 0 ? e : 0) + d * vb / 8 + 2 * e * (d / 32));   // = record bytes
}
// Two buffers for every shape: measured on the large workloads, three or four
// (two or three tiles in flight, fewer resident waves for the LDS they take)
// decode 3-10 % slower.
__host__ __device__ constexpr int ring_of(int d, int w, int mc, int vb, bool sf) { return 2; }
// LDS bytes per block of decode_fast_kernel<D, W, m / 64, G, VB, SF> (host and device):
// per wave the tile ring and the value-weight operand [groups][4][2G + 1 rows][16 B],
// whose first bytes also hold the softmax weights P [32 tokens][G] until they are
// read; at the end the 4-wave merge
__host__ __device__ constexpr int aval_rows_of(int g) { return 2 * g + 1; }   // + 1 row: writes spread over all banks
__host__ __device__ constexpr int wave_lds_of(int d, int w, int mc, int g, int vb, bool sf) {
  return ring_of(d, w, mc, vb, sf) * tile_bytes_of(d, w, mc, vb, sf) + (d / 32) * 4 * aval_rows_of(g) * 16;
}
__host__ __device__ constexpr int smem_of(int d, int w, int mc, int g, int vb, bool sf) {
  const int waves = kWaves * wave_lds_of(d, w, mc, g, vb, sf);
  const int merge = kWaves * (g * d + 2 * g + g * (d / 32)) * 4;
  const int nc_all = chunks_max(d, w, 64 * mc);
  const int qa = heads_rb(g) * nc_all * 4 <= kRegAVgprs ? 0 : heads_rb(g) * nc_all * 1024;
  return qa + (waves > merge ? waves : merge);
}

template <int D, int W, int MC, int G, int VB, bool SF>
struct Geo {
  static constexpr int RB = heads_rb(G);
  static constexpr int HC = D / 64;                  // K-chunks per code plane
  static constexpr int kGroups = D / 32;
  static constexpr int CB = W * D / 8;               // key code bytes per token
  static constexpr int SB = MC * 8;                  // sign bytes per token (m / 8)
  static constexpr int VBY = D * VB / 8;             // value code bytes per token
  static constexpr int NCmax = chunks_max(D, W, 64 * MC);
  static constexpr int kWpl = D >= 128 ? D / 128 : 1;    // plane words per lane per token
  static constexpr int kSw = (MC + 1) / 2;               // sign words per lane per token
  static constexpr int kPairs = pairs_of(G, D);
  static constexpr int kLG = kGroups >= 4 ? kGroups / 4 : 1;   // value groups one lane reads per tile
  static constexpr int E = SF ? 2 : 4;                  // bytes per side-information number
  static constexpr int o_signs = kTT * CB;
  static constexpr int o_norm = o_signs + kTT * SB;
  static constexpr int o_rnorm = o_norm + kTT * E;
  static constexpr int o_vcodes = o_rnorm + (W > 0 ? kTT * E : 0);
  static constexpr int o_vside = o_vcodes + kTT * VBY;
  static constexpr int tile_bytes = o_vside + kTT * kGroups * 2 * E;
  static_assert(tile_bytes == tile_bytes_of(D, W, MC, VB, SF), "tile geometry");
  static constexpr int kR = ring_of(D, W, MC, VB, SF);   // tile buffers per wave
  static constexpr int wave_lds = wave_lds_of(D, W, MC, G, VB, SF);
  static constexpr int AR = aval_rows_of(G);        // 16-byte rows per (group, lane group) block
  static constexpr int aval_bytes = kGroups * 4 * AR * 16;
  // load instructions per tile (each wave waits on whole tiles)
  static constexpr int loads_per_tile = loads_of<tile_bytes>();
  static constexpr int nc_all = chunks_max(D, W, 64 * MC);
  static constexpr bool reg_a_all = RB * nc_all * 4 <= kRegAVgprs;
  static constexpr int qa_lds_bytes = reg_a_all ? 0 : RB * nc_all * 1024;
  static constexpr int smem = smem_of(D, W, MC, G, VB, SF);
};

// Query side of the slot's G heads, built by the whole block once (the
// TurboQuant article's step that rotates and sketches each query once, here
// also integerised): per head the scales sig = max |value| / 16383 and the constant
// terms c[0] sum(q_rot), -sum(q_sk) go to hc; every A-operand value v = round
// (value / sig) (kappa_A q_rot for the code planes in PL, 2 q_sk for the sign
// chunks) is split into int8 parts hi = v >> 7, lo = v & 127 and written to
// `ops`, lane-major: byte i of lane (row, q) of chunk c in row block r sits at
// ((r * NC + c) * 64 + lane) * 16 + i and is K-slot 16 q + i; row = 4 (g % 4) + t
// with t = mse hi, mse lo, qjl hi, qjl lo (pure QJL: the three digits of the
// bit-place-weighted value, then a zero row) and g = 4 r + row / 4.  K-slot 16 q + i of
// chunk h of a plane is coordinate (D/4) q + 16 h + i; of sign chunk h, sketch row
// 16 MC q + 16 h + i.
template <int D, int W, int MC, int G, int PL>
__device__ __forceinline__ void pack_query(const DecodeJob &job, int64_t head0, const float *kappa, uint8_t *ops,
                                           HeadConst *hc) {
  constexpr int RB = heads_rb(G), HC = D / 64, NP = popc(PL), NC = NP * HC + MC, m = 64 * MC;
  // Every block runs this before its tiles stream (only the first tile's loads are in
  // flight), so the query's global reads are issued together rather than one dependent
  // round per word: each round costs a full memory latency under the other blocks' load.
  constexpr int kWords = RB * NC;                    // words of this thread: word tid of each (r, c)
  constexpr int kGrp = kWords < 8 ? kWords : 8;      // words whose values are loaded together
  constexpr int kHW = (G + kWaves - 1) / kWaves;     // heads a wave reduces
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // word tid of chunk (r, c) holds bytes i0 .. i0 + 3 of operand lane l = tid / 4
  const int l = tid >> 2, i0 = (tid & 3) * 4;
  const int row = l % 16, q = l / 16, t = row % 4;
  // the values behind word j = r NC + c: coordinates of q_rot (plane a of PL, rows
  // t = mse hi / lo) or rows of q_sketch (qjl rows), or none
  auto word_src = [&](int j, int &a) -> const float * {
    const int r = j / NC, c = j % NC, g = 4 * r + row / 4;
    a = 1;
    if (g >= G) return nullptr;
    if (c < NP * HC) {
      if (t >= 2) return nullptr;
      int n = 0;
#pragma unroll
      for (int b = 1; b < (1 << W); ++b)
        if ((PL >> b) & 1) {
          if (n == c / HC) a = b;
          ++n;
        }
      return job.q_rot + (head0 + g) * D + (D / 4) * q + 16 * (c % HC) + i0;
    }
    if (W == 0 ? t >= 3 : t < 2) return nullptr;
    return job.q_sketch + (head0 + g) * m + 16 * MC * q + 16 * (c - NP * HC) + i0;
  };
  float vq[kGrp][4];
  auto load_group = [&](int j0) {
#pragma unroll
    for (int jj = 0; jj < kGrp; ++jj) {
      int a;
      const float *src = j0 + jj < kWords ? word_src(j0 + jj, a) : nullptr;
      // loads without branches (a branch around them makes the compiler wait on each):
      // a word with no source reads the slot's first sketched row and drops it
      const float *rd = src ? src : job.q_sketch + head0 * m;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float x = rd[bb];
        vq[jj][bb] = src ? x : 0.0f;
      }
    }
  };

  // the rows each wave reduces (head g = wave + 4 h), then the first group of words
  float rv[kHW][W > 0 ? D / 64 : 1], sv[kHW][MC];
#pragma unroll
  for (int h = 0; h < kHW; ++h) {
    const int g = wave + kWaves * h;
    if (g < G) {
      if constexpr (W > 0)
#pragma unroll
        for (int k = 0; k < D / 64; ++k) rv[h][k] = job.q_rot[(head0 + g) * D + lane + 64 * k];
#pragma unroll
      for (int k = 0; k < MC; ++k) sv[h][k] = job.q_sketch[(head0 + g) * m + lane + 64 * k];
    }
  }
  load_group(0);

  float km = 0.0f;
#pragma unroll
  for (int a = 1; a < (1 << W); ++a)
    if ((PL >> a) & 1) km = fmaxf(km, fabsf(kappa[a - 1]));
#pragma unroll
  for (int h = 0; h < kHW; ++h) {
    const int g = wave + kWaves * h;
    if (g < G) {
      float mx = 0.0f, sr = 0.0f, mq = 0.0f, sq = 0.0f;
      if constexpr (W > 0)
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          sr += rv[h][k];
          mx = fmaxf(mx, km * fabsf(rv[h][k]));
        }
#pragma unroll
      for (int k = 0; k < MC; ++k) {
        sq += sv[h][k];
        mq = fmaxf(mq, fabsf(2.0f * sv[h][k]));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off));
        mq = fmaxf(mq, __shfl_xor(mq, off));
        sr += __shfl_xor(sr, off);
        sq += __shfl_xor(sq, off);
      }
      if (lane == 0)
        hc[g] = HeadConst{mx > 0.0f ? mx / 16383.0f : 1.0f, mq > 0.0f ? mq / 16383.0f : 1.0f,
                          W > 0 ? job.centroids[0] * sr : 0.0f, -sq};
    }
  }
  __syncthreads();
#pragma unroll
  for (int j0 = 0; j0 < kWords; j0 += kGrp) {
    if (j0 > 0) load_group(j0);
#pragma unroll
    for (int jj = 0; jj < kGrp; ++jj) {
      const int j = j0 + jj;
      if (j >= kWords) break;
      const int c = j % NC, g = 4 * (j / NC) + row / 4;
      int a;
      uint32_t word = 0;
      if (word_src(j, a)) {
        const float scl = c < NP * HC ? kappa[a - 1] / hc[g].sig_mse : 2.0f / hc[g].sig_qjl;
        // pure QJL: the B bytes of this K-slot carry the bit times 2^e (e = 4 hf + i0 / 4, the
        // bit's place in its byte; -128 for e = 7), so the value becomes Q = v 2^(7 - e)
        // (-v for e = 7), < 2^21 in magnitude, in base-128 digits Q >> 14, (Q >> 7) & 127, Q & 127
        const int e = 4 * ((MC * q + (c - NP * HC)) & 1) + i0 / 4;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          int v = static_cast<int>(rintf(vq[jj][bb] * scl));
          v = max(-16383, min(16383, v));
          int part;
          if constexpr (W == 0) {
            const int Q = e == 7 ? -v : v * (1 << (7 - e));
            part = t == 0 ? (Q >> 14) : t == 1 ? ((Q >> 7) & 127) : (Q & 127);
          } else {
            part = (t & 1) ? (v & 127) : (v >> 7);
          }
          word |= (static_cast<uint32_t>(part) & 0xffu) << (8 * bb);
        }
      }
      reinterpret_cast<uint32_t *>(ops)[j * kThreads + tid] = word;
    }
  }
  __syncthreads();
}

template <int D, int W, int MC, int G, int VB, bool SF, int PL>
__device__ __forceinline__ void decode_body(const DecodeJob &job, int64_t slot, int split, uint8_t *smem,
                                            const float *kappa) {
  using Gm = Geo<D, W, MC, G, VB, SF>;
  constexpr int RB = Gm::RB, HC = Gm::HC, kGroups = Gm::kGroups, CB = Gm::CB, SB = Gm::SB, VBY = Gm::VBY;
  constexpr int kWpl = Gm::kWpl, kSw = Gm::kSw, kPairs = Gm::kPairs, kLG = Gm::kLG;
  constexpr int NP = popc(PL);
  constexpr int NC = NP * HC + MC;
  constexpr int NCmax = Gm::NCmax;
  constexpr bool kRegA = RB * NC * 4 <= kRegAVgprs;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform in an SGPR: tile offsets and LDS bases derive from it
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q = lane >> 4;
  const int64_t t_begin = static_cast<int64_t>(split) * job.split_tokens;
  const int64_t t_end = min<int64_t>(job.context, t_begin + job.split_tokens);
  const int64_t head0 = slot * G;

  // ---- LDS: ring slot k of wave w at ring + (k * kWaves + w) * tile_bytes, then
  // the waves' value-weight operands
  uint8_t *qa_lds = smem;
  uint8_t *ring = smem + Gm::qa_lds_bytes;
  constexpr int kRing = Gm::kR;
  uint8_t *aval = ring + kRing * kWaves * Gm::tile_bytes + wave * Gm::aval_bytes;   // [grp][q][AR][16 B]
  float *P = reinterpret_cast<float *>(aval);   // [kTT][G], read out before aval is written
  auto slot_buf = [&](int64_t tile) -> uint8_t * {
    return ring + (static_cast<int>((tile / kWaves) % kRing) * kWaves + wave) * Gm::tile_bytes;
  };

  // ---- the slot's block records: one contiguous record per 32-token tile
  const int64_t n_tiles = (t_end > t_begin) ? (t_end - t_begin + kTT - 1) / kTT : 0;
  const int64_t recs = job.capacity / kTT;
  const __amdgpu_buffer_rsrc_t rs_blocks =
      plane_rsrc(job.blocks + slot * recs * Gm::tile_bytes, static_cast<uint32_t>(recs * Gm::tile_bytes));
  // a scores-only call needs the key fields of a record alone (they come first), so
  // its tiles take fewer loads
  const bool keys_only = job.scores_only != 0;
  // score stores share the vector-memory counter with the tile loads, and a wait
  // for a partial count is only sound with loads alone in flight
  const bool partial_waits = job.scores == nullptr;
  // the record of tile `tile` of the block's range (wave-uniform): the next one, or the
  // listed record (a record list makes the range an index into the slot's list)
  auto rec_of = [&](int64_t tile) -> uint32_t {
    const int64_t i = t_begin / kTT + tile;
    return __builtin_amdgcn_readfirstlane(job.rec_list ? static_cast<uint32_t>(job.rec_list[slot * job.list_stride + i])
                                                       : static_cast<uint32_t>(i));
  };
  auto issue = [&](int64_t tile) {
    const uint32_t rec = rec_of(tile);
    if (keys_only)
      copy_region<Gm::o_vcodes>(rs_blocks, rec * Gm::tile_bytes, slot_buf(tile), lane);
    else
      copy_region<Gm::tile_bytes>(rs_blocks, rec * Gm::tile_bytes, slot_buf(tile), lane);
  };
  // register-resident operands are staged in the last ring slots, which load
  // last, so the first tiles stream in while the query side is built (when the
  // operands need more room they take the whole ring and the tiles wait)
  constexpr bool kStageLast = RB * NC * 1024 <= kWaves * Gm::tile_bytes;
  static_assert(!kRegA || RB * NC * 1024 <= kRing * kWaves * Gm::tile_bytes, "operand staging space");
  uint8_t *ops = !kRegA ? qa_lds : kStageLast ? ring + (kRing - 1) * kWaves * Gm::tile_bytes : ring;
  int64_t tile = wave;
  auto issue_first = [&]() {
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k)
      if (tile + k * kWaves < n_tiles) issue(tile + k * kWaves);
  };
  if constexpr (!kRegA || kStageLast) issue_first();

  // ---- query operands and per-head constants, built by this block
  __shared__ HeadConst s_hc[G];
  pack_query<D, W, MC, G, PL>(job, head0, kappa, ops, s_hc);
  v4i aq[kRegA ? RB : 1][kRegA ? NC : 1];
  if constexpr (kRegA) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int c = 0; c < NC; ++c) aq[r][c] = *reinterpret_cast<const v4i *>(ops + ((r * NC + c) * 64 + lane) * 16);
  }
  auto A = [&](int r, int c) -> v4i {
    if constexpr (kRegA) return aq[r][c];
    else return *reinterpret_cast<const v4i *>(qa_lds + ((r * NC + c) * 64 + lane) * 16);
  };
  HeadConst hc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int g = 4 * r + q;
    hc[r] = g < G ? s_hc[g] : HeadConst{0.0f, 0.0f, 0.0f, 0.0f};
  }
  __syncthreads();   // staging space is free again before tiles land in it
  if constexpr (kRegA && !kStageLast) issue_first();
  const float kappa_qjl = 1.2533141373155003f / static_cast<float>(64 * MC);   // sqrt(pi/2) / m
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

  // weight tokens: K-slot 8 q' + i of the value product is token 4 i + q'; lane
  // (tp, pq) handles tokens ta = 8 (tp / 4) + tp % 4 and ta + 4
  const int ta = 8 * (n16 >> 2) + (n16 & 3), tb4 = ta + 4;

  for (; tile < n_tiles; tile += kWaves) {
    // wait for this tile: the (up to kRing - 2) later tiles already issued may stay in flight
    static_assert(kRing >= 2 && kRing <= 4, "wait ladder");
    {
      const int64_t after = partial_waits ? (n_tiles - 1 - tile) / kWaves : 0;
      if (kRing >= 4 && after >= 2) wait_vm<(kRing >= 4 ? 2 : 0) * Gm::loads_per_tile>();
      else if (kRing >= 3 && after >= 1) wait_vm<(kRing >= 3 ? 1 : 0) * Gm::loads_per_tile>();
      else wait_vm<0>();
    }
    compiler_fence();
    // the tile's first token and its valid tokens (listed records: the record's tokens
    // below the cached length), before the next tile's loads are in flight
    const int64_t t0 = job.rec_list ? static_cast<int64_t>(rec_of(tile)) * kTT : t_begin + tile * kTT;
    const int nt = static_cast<int>(min<int64_t>(kTT, (job.rec_list ? job.list_context : t_end) - t0));
    if (tile + (kRing - 1) * kWaves < n_tiles) issue(tile + (kRing - 1) * kWaves);
    const uint8_t *tb = slot_buf(tile);

    // ---------------- scores: 2 column tiles of 16 tokens, their matrix chains interleaved
    v4i acc[2][RB];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[ct][r] = v4i{0, 0, 0, 0};
    {
      // this lane's words: coordinates (D/4) q .. (D/4) q + D/4 - 1 of each index
      // plane (D = 64: half of one word) and sketch rows 16 MC q .. 16 MC q + 16 MC - 1
      uint32_t pw[2][W > 0 ? W : 1][kWpl], sw[2][kSw];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int tok = 16 * ct + n16;
        if constexpr (W > 0) {
#pragma unroll
          for (int k = 0; k < W; ++k)
#pragma unroll
            for (int u = 0; u < kWpl; ++u) {
              const int word = D >= 128 ? kWpl * q + u : q / 2;
              pw[ct][k][u] = *reinterpret_cast<const uint32_t *>(tb + tok * CB + k * (D / 8) + 4 * word);
            }
        }
#pragma unroll
        for (int u = 0; u < kSw; ++u)
          sw[ct][u] = *reinterpret_cast<const uint32_t *>(tb + Gm::o_signs + tok * SB + 4 * (((MC * q) >> 1) + u));
      }
      int chunk = 0;
      if constexpr (W > 0) {
#pragma unroll
        for (int a = 1; a < (1 << W); ++a) {
          if ((PL >> a) & 1) {
#pragma unroll
            for (int h = 0; h < HC; ++h) {
              // chunk h = coordinates (D/4) q + 16 h .. + 15
              const int hf = D >= 128 ? (h & 1) : (q & 1);
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) {
                uint32_t x = 0;
#pragma unroll
                for (int k = 0; k < W; ++k)
                  if ((a >> k) & 1) x ^= pw[ct][k][D >= 128 ? h >> 1 : 0];
                const v4i bop = spread_half(x, hf);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                  acc[ct][r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A(r, chunk), bop, acc[ct][r], 0, 0, 0);
              }
              ++chunk;
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < MC; ++h) {
        // sketch rows 16 MC q + 16 h .. + 15: word (16 MC q + 16 h) / 32, half ((16 MC q + 16 h) / 16) & 1
        const int c = 16 * MC * q + 16 * h;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          uint32_t word;
          int hf;
          if constexpr (MC % 2 == 0) {
            word = sw[ct][h >> 1];
            hf = h & 1;
          } else {
            // odd MC: the lane's first row may sit in the upper half of a word
            const int wi = (c >> 5) - ((16 * MC * q) >> 5);
            word = sw[ct][0];
#pragma unroll
            for (int u = 1; u < kSw; ++u) word = (wi == u) ? sw[ct][u] : word;
            hf = (c >> 4) & 1;
          }
          // pure QJL: bits in place (three-digit query rows); else one {0,1} byte per bit
          const v4i bop = W == 0 ? mask_half(word, hf) : spread_half(word, hf);
#pragma unroll
          for (int r = 0; r < RB; ++r)
            acc[ct][r] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A(r, chunk), bop, acc[ct][r], 0, 0, 0);
        }
        ++chunk;
      }
    }
    float logit[2][RB], score[2][RB], nrm_ct[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int tok = 16 * ct + n16;
      float nrm, gam;
      if constexpr (SF) {
        nrm = static_cast<float>(reinterpret_cast<const _Float16 *>(tb + Gm::o_norm)[tok]);
        gam = W > 0 ? static_cast<float>(reinterpret_cast<const _Float16 *>(tb + Gm::o_rnorm)[tok]) : nrm;
      } else {
        nrm = reinterpret_cast<const float *>(tb + Gm::o_norm)[tok];
        gam = W > 0 ? reinterpret_cast<const float *>(tb + Gm::o_rnorm)[tok] : nrm;
      }
      const bool valid = tok < nt;
      nrm_ct[ct] = nrm;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int g = 4 * r + q;
        float s = 0.0f;
        if constexpr (W > 0)
          s = nrm * fmaf(hc[r].sig_mse, static_cast<float>(acc[ct][r][0] * 128 + acc[ct][r][1]), hc[r].c_mse);
        // sum of the head's integer query values over the set sign bits: hi * 128 + lo, or
        // for pure QJL the three base-128 digits of 128 x that sum
        const float qs = W == 0 ? fmaf(static_cast<float>(acc[ct][r][0]), 128.0f,
                                       fmaf(static_cast<float>(acc[ct][r][2]), 0.0078125f,
                                            static_cast<float>(acc[ct][r][1])))
                                : static_cast<float>(acc[ct][r][2] * 128 + acc[ct][r][3]);
        const float qjl = fmaf(hc[r].sig_qjl, qs, hc[r].c_qjl);
        s = fmaf(kappa_qjl * gam, qjl, s);
        score[ct][r] = s;
        logit[ct][r] = (valid && g < G) ? s * lscale : -INFINITY;
      }
    }
    if (keys_only) {
      if (job.scores) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            const int g = 4 * r + q, tok = 16 * ct + n16;
            if (g < G && tok < nt) job.scores[(head0 + g) * job.context + t0 + tok] = score[ct][r];
          }
      }
      if (job.rec_max) {
        // the record's largest cosine score / ||k|| of the first head (0 for a zero key)
        float cmax = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const float c = nrm_ct[ct] > 0.0f ? score[ct][0] / nrm_ct[ct] : 0.0f;
          cmax = fmaxf(cmax, 16 * ct + n16 < nt ? c : -INFINITY);
        }
        cmax = row_max16(cmax);
        if (lane == 0) job.rec_max[slot * job.rec_max_stride + t0 / kTT] = cmax;
      }
      continue;
    }

    // ---------------- online softmax (lazy rescale); lane group q = head 4r + q
    float fac[RB];
    bool changed = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float tmax = row_max16(fmaxf(logit[0][r], logit[1][r]));
      float f = 1.0f;
      if (tmax > m_ref[r] + kLazy) {
        f = __builtin_amdgcn_exp2f(m_ref[r] - tmax);       // 0 on the first update (m_ref = -inf)
        m_ref[r] = tmax;
        changed = true;
      }
      fac[r] = f;
      const int g = 4 * r + q;
      float psum = 0.0f;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        // exp2(-inf) = 0 for masked tokens; m_ref is finite for every real head here
        const float p = __builtin_amdgcn_exp2f(logit[ct][r] - m_ref[r]);
        psum += p;
        if (g < G) P[(16 * ct + n16) * G + g] = p;
      }
      l_part[r] = l_part[r] * f + psum;
    }
    if (job.scores) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int g = 4 * r + q, tok = 16 * ct + n16;
          if (g < G && tok < nt) job.scores[(head0 + g) * job.context + t0 + tok] = score[ct][r];
        }
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

    // ---------------- value weights a = p * scale (f16 hi + lo), correction sums p * min
    {
      const int qd = n16 & 3, i0 = 2 * (n16 >> 2);
      // {scale, min} of tokens ta and ta + 4 of group (q + 4u) % kGroups: one
      // contiguous 16-byte (8-byte with half side information) read per lane
      // (group-major val_side field)
      float4 side[kLG];
#pragma unroll
      for (int u = 0; u < kLG; ++u) {
        const int si = ((q + 4 * u) % kGroups) * 16 + n16;
        if constexpr (SF) {
          const uint2 hv = reinterpret_cast<const uint2 *>(tb + Gm::o_vside)[si];
          side[u] = make_float4(half_lo(hv.x), half_hi(hv.x), half_lo(hv.y), half_hi(hv.y));
        } else {
          side[u] = reinterpret_cast<const float4 *>(tb + Gm::o_vside)[si];
        }
      }
      float pa[G], pb[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pa[g] = P[ta * G + g];
        pb[g] = P[tb4 * G + g];
      }
      compiler_fence();   // P shares its bytes with the operand written below
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int pair = q + 4 * k;
        if (pair < G * kGroups) {
          const int g = pair / kGroups, grp = pair % kGroups;
          const float4 sd = side[k % kLG];   // group (q + 4 k) % kGroups
          const float sa = sd.x, ma = sd.y, sb = sd.z, mb = sd.w;
          // legacy multiply: 0 * x = 0 for any x, so masked tokens (p = 0) ignore
          // whatever their cache rows hold
          float aa = fmul_legacy(pa[g], sa);
          float ab = fmul_legacy(pb[g], sb);
          // pin the fp32 weights so both uses of the f16 high part see the same value
          asm volatile("" : "+v"(aa), "+v"(ab));
          corr[k] += fmul_legacy(pa[g], ma) + fmul_legacy(pb[g], mb);
          // hi = the weights rounded toward zero to f16, lo = f16 of the exact fp32 remainders
          const auto hi = __builtin_amdgcn_cvt_pkrtz(aa, ab);
          const auto lo = __builtin_amdgcn_cvt_pkrtz(aa - static_cast<float>(hi[0]), ab - static_cast<float>(hi[1]));
          uint8_t *dst = aval + ((grp * 4 + qd) * Gm::AR + 2 * g) * 16 + 2 * i0;
          *reinterpret_cast<uint32_t *>(dst) = __builtin_bit_cast(uint32_t, hi);
          *reinterpret_cast<uint32_t *>(dst + 16) = __builtin_bit_cast(uint32_t, lo);
        }
      }
    }
    compiler_fence();

    // ---------------- value products: 32 tokens x 16 channels per matrix instruction
    {
      const uint8_t *vc = tb + Gm::o_vcodes;
#pragma unroll
      for (int grp = 0; grp < kGroups; ++grp) {
        // rows >= 2G of the weight operand repeat rows < 2G; their outputs are never read
        const v8h aop = *reinterpret_cast<const v8h *>(aval + ((grp * 4 + q) * Gm::AR + (n16 & (2 * G - 1))) * 16);
        // block word(s) of column n16: tokens 4 i + q of channels 32 grp + 16 h + n16;
        // operand dword k = K-slots (8q + 2k, 8q + 2k + 1) = i (2k, 2k + 1).  The
        // code itself, masked into the low mantissa bits of an f16 with a zero
        // exponent, is the exact denormal code * 2^-24.
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
            // code of i = 2k at bits 8h + 2k, of 2k+1 at 16 + 8h + 2k
#pragma unroll
            for (int k = 0; k < 4; ++k) bw[k] = static_cast<int>((wv[0] >> (8 * h + 2 * k)) & 0x00030003u);
          } else {
            // code of i = 2k at bits 4k, of 2k+1 at 16 + 4k
#pragma unroll
            for (int k = 0; k < 4; ++k) bw[k] = static_cast<int>((wv[h] >> (4 * k)) & 0x000f000fu);
          }
          const v8h bop = __builtin_bit_cast(v8h, bw);
          cval[2 * grp + h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cval[2 * grp + h], 0, 0, 0);
        }
      }
    }
    compiler_fence();
  }

  if (keys_only) return;   // uniform over the block: no partials to merge

  // ---------------- per-wave results -> LDS, merge the 4 waves
  __syncthreads();
  float *mrg = reinterpret_cast<float *>(smem + Gm::qa_lds_bytes);    // [wave][G][D]
  float *mrg_ml = mrg + kWaves * G * D;                               // [wave][G][2]
  float *mrg_corr = mrg_ml + kWaves * G * 2;                          // [wave][G * kGroups]
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const float l = row_sum16(l_part[r]);
    const int g = 4 * r + q;
    if (g < G && n16 == 0) {
      mrg_ml[(wave * G + g) * 2 + 0] = m_ref[r];
      mrg_ml[(wave * G + g) * 2 + 1] = l;
    }
  }
#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const float c = row_sum16(corr[k]);
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
          mrg[(wave * G + g) * D + ch] = 16777216.0f * (c[2 * e] + c[2 * e + 1]) + cg;   // 2^24 undoes the denormal scale
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
    const int64_t ph = (head0 + g) * job.part_stride + split;
    job.part_acc[ph * D + j] = O;
    if (j == 0) {
      job.part_ml[ph * 2 + 0] = M;
      job.part_ml[ph * 2 + 1] = L;
    }
  }

}

// waves per SIMD the register allocation aims for (16 or 8 per CU)
__host__ __device__ constexpr int waves_per_simd(int d, int g) { return (g >= 8 || d >= 256) ? 2 : 4; }

template <int D, int W, int MC, int G, int VB, bool SF>
__global__ __launch_bounds__(kThreads, waves_per_simd(D, G)) void decode_fast_kernel(DecodeJob job) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float s_cen[8], s_kappa[8];
  const int64_t slot = blockIdx.x / job.n_split;
  const int split = static_cast<int>(blockIdx.x % job.n_split);
  const int tid = threadIdx.x;
  constexpr int L = 1 << W;
  if constexpr (W > 0) {
    // kappa_A (thread A) = -2 (-1)^|A| 2^-w sum_idx c[idx] prod_{k in A} (2 bit_k(idx) - 1),
    // summed over complementary index pairs so odd-symmetric codebooks give exact zeros
    if (tid < L) s_cen[tid] = job.centroids[tid];
    __syncthreads();
    if (tid >= 1 && tid < L) {
      double acc = 0.0;
      for (int i = 0; i < L / 2; ++i) {
        const int j = L - 1 - i;
        double si = 1.0, sj = 1.0;
        for (int k = 0; k < W; ++k)
          if ((tid >> k) & 1) {
            si *= ((i >> k) & 1) ? 1.0 : -1.0;
            sj *= ((j >> k) & 1) ? 1.0 : -1.0;
          }
        acc += static_cast<double>(s_cen[i]) * si + static_cast<double>(s_cen[j]) * sj;
      }
      s_kappa[tid - 1] = static_cast<float>(-2.0 * ((__popc(tid) & 1) ? -1.0 : 1.0) * acc / L);
    }
    __syncthreads();
  }
  if constexpr (W >= 2) {
    // only the odd-size planes when every even-size coefficient vanishes (odd-symmetric codebook)
    bool odd = true;
#pragma unroll
    for (int a = 1; a < L; ++a)
      if (!(popc(a) & 1) && s_kappa[a - 1] != 0.0f) odd = false;
    if (odd) decode_body<D, W, MC, G, VB, SF, odd_planes(W)>(job, slot, split, smem, s_kappa);
    else decode_body<D, W, MC, G, VB, SF, all_planes(W)>(job, slot, split, smem, s_kappa);
  } else {
    decode_body<D, W, MC, G, VB, SF, all_planes(W)>(job, slot, split, smem, s_kappa);
  }
}

template <int D, int W, int MC, int G, int VB, bool SF>
hipError_t launch_fast(const DecodeJob &job, hipStream_t stream) {
  using Gm = Geo<D, W, MC, G, VB, SF>;
  auto kern = decode_fast_kernel<D, W, MC, G, VB, SF>;
  if (Gm::smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Gm::smem);
    if (e != hipSuccess) return e;
  }
  kern<<<static_cast<unsigned>(job.n_split * job.n_slots), kThreads, Gm::smem, stream>>>(job);
  return hipGetLastError();
}

template <int D, int W, int MC, int G>
hipError_t launch_fast_g(const DecodeJob &job, hipStream_t stream) {
  if (job.sf) return job.vb == 2 ? launch_fast<D, W, MC, G, 2, true>(job, stream) : launch_fast<D, W, MC, G, 4, true>(job, stream);
  return job.vb == 2 ? launch_fast<D, W, MC, G, 2, false>(job, stream) : launch_fast<D, W, MC, G, 4, false>(job, stream);
}

template <int D, int W, int MC>
hipError_t launch_fast_m(const DecodeJob &job, hipStream_t stream) {
  switch (job.g) {
    case 1: return launch_fast_g<D, W, MC, 1>(job, stream);
    case 2: return launch_fast_g<D, W, MC, 2>(job, stream);
    case 4: return launch_fast_g<D, W, MC, 4>(job, stream);
    default: return launch_fast_g<D, W, MC, 8>(job, stream);
  }
}

}  // namespace fast
}  // namespace aqkv
