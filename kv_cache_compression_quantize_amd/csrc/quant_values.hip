// Value quantisation kernel: per token, per group of 32 contiguous channels,
// min-max quantisation to 2 or 4 bits (TurboQuant article, the value row of the
// component table: grouped min-max at 2 bits per dimension; and §七, the value
// group quantisation and bit packing of its kv_cache.py listing).
//
// code = clamp(rint((v - min) / scale), 0, 2^vb - 1) with scale = (max - min) /
// (2^vb - 1), every step in IEEE fp32 (subtract, correctly rounded divide,
// round-half-even); code 0 when scale == 0.  Scale and min are stored as
// fp32, or rounded to the nearest half for a cache with half side information
// (the codes are decided from the fp32 values either way).
//
// Lane layout.  The code block of a record stores, per (group g, column n,
// token residue r), the codes of channel 32 g + 16 half + n for the tokens
// 8 a + 4 b + r (a = 0..3, b = 0..1) of the record, a = the position inside a
// byte (vb = 2) or half-word (vb = 4), (half, b) = which one (include/aqkv.h).
// So one thread of a record takes the tokens c + 8 a (c = 4 b + r, a = 0..3)
// of one 8-channel chunk: the four codes of each of its channels make one
// finished byte / half-word of the output.  Threads c * (d / 8) + chunk, so the
// 4 threads that share a (token, group) are neighbouring lanes (min / max by
// DPP lane swaps) and each load instruction of a wave reads whole tokens.
//
// Scale.  fl(x / L) for x = max - min in [1e-28, 1e28] is q0 = x * fl(1/L),
// r = fma(-q0, L, x) (exact), fl(x / L) = fma(r, fl(1/L), q0): for L = 3 and
// 15 this equals the IEEE quotient for every fp32 significand (exhaustive
// check in the tests), and the exponent range keeps every step normal; other
// x take the IEEE divide.
//
// Codes.  With rr = rcp(scale) (1 ulp) and c0 = 0.5 - min * rr (one fma),
// fma(v, rr, c0) lies within (5 L + 1 + 2 |c0|) 2^-24 of
// X = fl(fl(v - min) / scale) + 0.5 (L = 2^vb - 1, quotients <= L), well inside
// eps = (|c0| + L + 2) 2^-21.  So t = fma(v, rr, c0 - eps) has X in
// (t, t + 2 eps): when fract(t) < 1 - 2 eps that interval holds no integer,
// floor(t) = floor(X) and X is no tie, so floor(t) is the round-half-even
// code.  A piece (8 values of one token) with a value that fails the test, or
// with a scale outside [1e-30, 1e30], is redone with IEEE subtract, divide and
// rint.
//
// Each record's bytes / half-words are assembled in LDS (rows of 64 words
// padded by 8 so the byte writes of a wave spread over the banks) and leave as
// 16-byte stores; words of a record only partly covered by the call keep the
// bits of the other tokens (read-modify-write), so appends of any length work.
// The pass is a streaming one: HBM bandwidth with a thin VALU margin
// (about 9 vector instructions per value).
#include <algorithm>

#include "internal.h"

namespace aqkv {
namespace {

constexpr int kGroup = 32;
constexpr int kBlockTokens = 32;

// min and max over the 4 consecutive (aligned) lanes that share a group
// (quad permutations read only lanes that exist, so bound_ctrl changes nothing
// and lets the swap fold into the min / max as one DPP instruction)
__device__ __forceinline__ float quad_min(float x) {
  x = fminf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));   // lane ^ 1
  return fminf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));   // lane ^ 2
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));
}

// padded LDS word index of code word wi
__device__ __forceinline__ int lds_word(int wi) { return wi + 8 * (wi >> 6); }

// fl(x / L), L = 2^vb - 1
template <int L>
__device__ __forceinline__ float div_levels(float x) {
  if (!(x >= 1.0e-28f && x <= 1.0e28f)) return x / static_cast<float>(L);   // IEEE divide
  constexpr float z = 1.0f / static_cast<float>(L);
  const float q0 = x * z;
  const float r = __builtin_fmaf(-q0, static_cast<float>(L), x);
  return __builtin_fmaf(r, z, q0);
}

template <int D, int VB, bool BF16>
__global__ __launch_bounds__(256) void quantize_values_kernel(ValueJob job, int blocks_per_slot, int n_rec) {
  constexpr int kLevels = (1 << VB) - 1;
  constexpr int kChunks = D / 8;                  // 8-channel chunks per token
  constexpr int kRpb = 256 / D;                   // records per block (a record's threads are whole waves)
  constexpr int kWords = D * VB;                  // code words per record
  constexpr int kLdsWords = kWords + 8 * (kWords / 64);
  constexpr int kElt = BF16 ? 2 : 4;
  constexpr int kLoads = BF16 ? 1 : 2;            // 16-byte loads per (token, chunk)
  __shared__ uint4 lds_all[kRpb * kLdsWords / 4];
  const int tid = threadIdx.x;
  const int sub = __builtin_amdgcn_readfirstlane(tid / D);   // record within the block
  const int lane = tid % D;
  const int c = lane / kChunks, chunk = lane % kChunks;
  const int rid0 = blockIdx.x * kRpb + sub;
  const bool live = rid0 < n_rec;                  // the last block may hold fewer records (all reach the barrier)
  const int rid = live ? rid0 : 0;
  // slot and record of the slot, batch and head: multiply-shift divisions (rid < 2^31)
  const uint32_t su = div_by(static_cast<uint32_t>(rid), job.bps_m, job.bps_s);
  const int64_t s = su;
  const int64_t ct0 = (job.token_offset / kBlockTokens + (rid - static_cast<int>(su) * blocks_per_slot)) * kBlockTokens;
  // tokens [t_lo, t_hi) of the record are in this call
  const int t_lo = live ? static_cast<int>(max<int64_t>(ct0, job.token_offset) - ct0) : 0;
  const int t_hi = live ? static_cast<int>(min<int64_t>(ct0 + kBlockTokens, job.token_offset + job.n_tokens) - ct0) : 0;
  const uint32_t bu = div_by(su, job.head_m, job.head_s);
  const int64_t b = bu, h = static_cast<int64_t>(su) - static_cast<int64_t>(bu) * job.heads;
  const int64_t stride_bytes = job.token_stride * kElt;
  const char *rbase = static_cast<const char *>(job.v) +
                      (b * job.batch_stride + h * job.head_stride) * kElt + (ct0 - job.token_offset) * stride_bytes;
  const char *lbase = rbase + c * stride_bytes + 8 * chunk * kElt;

  // 1. every load in flight first: tokens c + 8 a, channels 8 chunk .. + 7
  uint4 raw[4][kLoads];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int tt = c + 8 * a;
#pragma unroll
    for (int l = 0; l < kLoads; ++l) raw[a][l] = make_uint4(0, 0, 0, 0);
    if (tt >= t_lo && tt < t_hi) {
      const uint4 *src = reinterpret_cast<const uint4 *>(lbase + 8 * a * stride_bytes);
#pragma unroll
      for (int l = 0; l < kLoads; ++l) raw[a][l] = stream_load(src + l);
    }
  }

  const int g = chunk / 4, q = chunk % 4;         // group, lane within the group
  // val_side element of (g, token c + 8 a, q): side_i + 16 a of the record's field
  uint8_t *side_rec = job.side + rec_row(s * job.capacity + ct0, 0, job.rec);
  const int side_i = side_index(g, c, q);
  uint32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};     // per channel: its 4 codes, VB bits apart
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float v[8];
#pragma unroll
    for (int l = 0; l < kLoads; ++l) {
      const uint32_t wv[4] = {raw[a][l].x, raw[a][l].y, raw[a][l].z, raw[a][l].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (BF16) {
          v[2 * j] = __uint_as_float(wv[j] << 16);
          v[2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
        } else {
          v[4 * l + j] = __uint_as_float(wv[j]);
        }
      }
    }
    float mn = fminf(fminf(fminf(v[0], v[1]), fminf(v[2], v[3])), fminf(fminf(v[4], v[5]), fminf(v[6], v[7])));
    float mx = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
    mn = quad_min(mn);
    mx = quad_max(mx);
    const float scale = div_levels<kLevels>(mx - mn);
    const float rr = __builtin_amdgcn_rcpf(scale);
    const float c0 = fmaf(-mn, rr, 0.5f);
    const float eps = (fabsf(c0) + static_cast<float>(kLevels + 2)) * 4.76837158203125e-7f;
    const float c1 = c0 - eps;                     // t - eps: no integer in (t - eps, t + eps] <=> fract < 1 - 2 eps
    const float th = 1.0f - 2.0f * eps;
    uint32_t codes[8];
    bool near = !(scale >= 1.0e-30f && scale <= 1.0e30f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = fmaf(v[j], rr, c1);
      codes[j] = static_cast<uint32_t>(t);                          // floor: t > 0
      near |= __builtin_amdgcn_fractf(t) >= th;
    }
    if (near) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float cf = scale > 0.0f ? rintf((v[j] - mn) / scale) : 0.0f;
        codes[j] = static_cast<uint32_t>(fminf(fmaxf(cf, 0.0f), static_cast<float>(kLevels)));
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] |= codes[j] << (VB * a);
    const int tt = c + 8 * a;
    if (q < 2 && tt >= t_lo && tt < t_hi) store_side(side_rec, side_i + 16 * a, job.sf != 0, q == 0 ? scale : mn);
  }

  // 2. bytes (vb = 2) / half-words (vb = 4) into the record's LDS words
  uint32_t *lw = reinterpret_cast<uint32_t *>(lds_all) + sub * kLdsWords;
  const int half = q / 2, bb = c / 4, r = c % 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = 8 * (chunk % 2) + j;
    if constexpr (VB == 2) {
      const int wi = g * 64 + n * 4 + r;
      reinterpret_cast<uint8_t *>(lw)[4 * lds_word(wi) + half + 2 * bb] = static_cast<uint8_t>(acc[j]);
    } else {
      const int wi = g * 128 + n * 8 + r * 2 + half;
      reinterpret_cast<uint16_t *>(lw)[2 * lds_word(wi) + bb] = static_cast<uint16_t>(acc[j]);
    }
  }
  __syncthreads();

  // 3. the record's code words, 16 bytes a thread
  if (live && lane < kWords / 4) {
    uint4 w = *reinterpret_cast<const uint4 *>(lw + lds_word(4 * lane));
    uint4 *dst = reinterpret_cast<uint4 *>(job.codes + rec_row(s * job.capacity + ct0, D * VB / 8, job.rec)) + lane;
    if (t_lo != 0 || t_hi != kBlockTokens) {
      // bits of the tokens of this call: word (.., r, ..) holds tokens 4 i + r
      uint32_t cover[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int wi = 4 * lane + k;
        const int rw = VB == 2 ? wi % 4 : (wi / 2) % 4;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tt = 4 * i + rw;
          const int bit = VB == 2 ? 16 * (i & 1) + 2 * (i >> 1) : 16 * (i & 1) + 4 * (i >> 1);
          const uint32_t one = VB == 2 ? (3u << bit) | (3u << (bit + 8)) : 15u << bit;
          if (tt >= t_lo && tt < t_hi) m |= one;
        }
        cover[k] = m;
      }
      const uint4 old = *dst;
      w.x = (old.x & ~cover[0]) | (w.x & cover[0]);
      w.y = (old.y & ~cover[1]) | (w.y & cover[1]);
      w.z = (old.z & ~cover[2]) | (w.z & cover[2]);
      w.w = (old.w & ~cover[3]) | (w.w & cover[3]);
    }
    *dst = w;
  }
}

template <int D>
hipError_t launch_d(const ValueJob &job_in, hipStream_t stream) {
  ValueJob job = job_in;
  const int64_t first = job.token_offset / kBlockTokens;
  const int64_t last = (job.token_offset + job.n_tokens - 1) / kBlockTokens;
  const int64_t per_slot = last - first + 1;
  const int64_t n_rec = per_slot * job.n_slots;
  if (n_rec >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  constexpr int kRpb = 256 / D;
  const dim3 grid(static_cast<unsigned>((n_rec + kRpb - 1) / kRpb));
  const int bps = static_cast<int>(per_slot), nr = static_cast<int>(n_rec);
  div_magic(per_slot, job.bps_m, job.bps_s);
  div_magic(std::max<int64_t>(job.heads, 1), job.head_m, job.head_s);
  const bool bf16 = job.dtype == AQKV_BF16;
  if (job.vb == 2) {
    if (bf16) quantize_values_kernel<D, 2, true><<<grid, 256, 0, stream>>>(job, bps, nr);
    else quantize_values_kernel<D, 2, false><<<grid, 256, 0, stream>>>(job, bps, nr);
  } else {
    if (bf16) quantize_values_kernel<D, 4, true><<<grid, 256, 0, stream>>>(job, bps, nr);
    else quantize_values_kernel<D, 4, false><<<grid, 256, 0, stream>>>(job, bps, nr);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_values(const ValueJob &job, hipStream_t stream) {
  switch (job.d) {
    case 64: return launch_d<64>(job, stream);
    case 128: return launch_d<128>(job, stream);
    default: return launch_d<256>(job, stream);
  }
}

}  // namespace aqkv
