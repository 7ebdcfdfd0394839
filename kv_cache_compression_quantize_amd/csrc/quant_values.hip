// Value quantisation kernel: per token, per group of 32 contiguous channels,
// min-max quantisation to 2 or 4 bits (TurboQuant article, component table
// "Value 分组量化 2 bit/维, min-max", and §七, kv_cache.py "value group
// quantisation and bit packing").
//
// Codes are stored in blocks of 32 tokens (the val_codes field of a cache
// block record) so that a decoder reads, for one channel, the codes of 8
// tokens of the block from one 32-bit word (layout in include/aqkv.h).  One block of 256 threads owns one
// 32-token cache block of one slot:
//   1. one thread per (token, group): 32 elements loaded with 16-byte loads,
//      min / max, scale = (max - min) / (2^vb - 1) and the codes in IEEE fp32
//      (subtract, correctly rounded divide, round-half-even); scale and min go
//      to the record's val_side field, the codes to LDS;
//   2. one thread per output word gathers its 16 (vb = 2) or 8 (vb = 4) codes;
//      words of a block only partly covered by this call keep the bits of the
//      other tokens (read-modify-write), so appends of any length work.
// The pass is a streaming one, bound by HBM bandwidth.
#include "internal.h"

namespace aqkv {
namespace {

constexpr int kGroup = 32;
constexpr int kBlockTokens = 32;

template <int D, int VB, bool BF16>
__global__ __launch_bounds__(256) void quantize_values_kernel(ValueJob job, int64_t blocks_per_slot) {
  constexpr int kGroups = D / kGroup;
  constexpr int kLevels = (1 << VB) - 1;
  __shared__ uint8_t cds[kBlockTokens][D];
  const int tid = threadIdx.x;
  const int64_t s = blockIdx.x / blocks_per_slot;
  const int64_t cblk = job.token_offset / kBlockTokens + blockIdx.x % blocks_per_slot;   // cache block
  const int64_t ct0 = cblk * kBlockTokens;                                              // its first cache token
  const int64_t lo = max<int64_t>(ct0, job.token_offset);
  const int64_t hi = min<int64_t>(ct0 + kBlockTokens, job.token_offset + job.n_tokens);
  const int64_t b = s / job.heads, h = s % job.heads;

  // 1. codes of (token, group)
  for (int item = tid; item < kBlockTokens * kGroups; item += 256) {
    const int tt = item / kGroups, g = item % kGroups;
    const int64_t ct = ct0 + tt;
    if (ct < lo || ct >= hi) continue;
    const int64_t t = ct - job.token_offset;      // input token
    const int64_t src = b * job.batch_stride + h * job.head_stride + t * job.token_stride + g * kGroup;
    float v[kGroup];
    if (BF16) {
      const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(job.v) + src);
#pragma unroll
      for (int i = 0; i < kGroup / 8; ++i) {
        const uint4 qv = p[i];
        const uint32_t wv[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_to_f32(wv[j] & 0xffffu);
          v[8 * i + 2 * j + 1] = bf16_to_f32(wv[j] >> 16);
        }
      }
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(job.v) + src);
#pragma unroll
      for (int i = 0; i < kGroup / 4; ++i) {
        const float4 qv = p[i];
        v[4 * i] = qv.x;
        v[4 * i + 1] = qv.y;
        v[4 * i + 2] = qv.z;
        v[4 * i + 3] = qv.w;
      }
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < kGroup; ++i) {
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
    const float scale = (mx - mn) / static_cast<float>(kLevels);   // IEEE divide
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      uint32_t code = 0;
      if (scale > 0.0f) {
        float c = rintf((v[i] - mn) / scale);                     // IEEE subtract, divide, RNE
        c = fminf(fmaxf(c, 0.0f), static_cast<float>(kLevels));
        code = static_cast<uint32_t>(c);
      }
      cds[tt][g * kGroup + i] = static_cast<uint8_t>(code);
    }
    // scale and min into the record's val_side field (group-major, include/aqkv.h)
    float *side = reinterpret_cast<float *>(job.side + rec_row(s * job.capacity + ct0, 0, job.rec));
    side[side_index(g, tt, 0)] = scale;
    side[side_index(g, tt, 1)] = mn;
  }
  __syncthreads();

  // 2. block words
  constexpr int kWords = kBlockTokens * D * VB / 32;
  // the code block of these 32 tokens: the val_codes field of one record
  uint32_t *dst = reinterpret_cast<uint32_t *>(job.codes + rec_row(s * job.capacity + ct0, D * VB / 8, job.rec));
  const bool full = lo == ct0 && hi == ct0 + kBlockTokens;
  for (int wi = tid; wi < kWords; wi += 256) {
    // word -> (group g, column n, token residue r) and the channel half(s) it holds
    const int g = VB == 2 ? wi / 64 : wi / 128;
    const int n = VB == 2 ? (wi / 4) % 16 : (wi / 8) % 16;
    const int r = VB == 2 ? wi % 4 : (wi / 2) % 4;
    constexpr int kHalves = VB == 2 ? 2 : 1;
    uint32_t word = 0, cover = 0;
#pragma unroll
    for (int e = 0; e < kHalves; ++e) {
      const int half = VB == 2 ? e : wi % 2;
      const int ch = 32 * g + 16 * half + n;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tt = 4 * i + r;
        const int bit = VB == 2 ? 8 * half + 16 * (i & 1) + 2 * (i >> 1) : 16 * (i & 1) + 4 * (i >> 1);
        const int64_t ct = ct0 + tt;
        if (ct >= lo && ct < hi) {
          word |= static_cast<uint32_t>(cds[tt][ch]) << bit;
          cover |= static_cast<uint32_t>(kLevels) << bit;
        }
      }
    }
    if (!full) word = (dst[wi] & ~cover) | word;
    dst[wi] = word;
  }
}

template <int D>
hipError_t launch_d(const ValueJob &job, hipStream_t stream) {
  const int64_t first = job.token_offset / kBlockTokens;
  const int64_t last = (job.token_offset + job.n_tokens - 1) / kBlockTokens;
  const int64_t per_slot = last - first + 1;
  const dim3 grid(static_cast<unsigned>(per_slot * job.n_slots));
  const bool bf16 = job.dtype == AQKV_BF16;
  if (job.vb == 2) {
    if (bf16) quantize_values_kernel<D, 2, true><<<grid, 256, 0, stream>>>(job, per_slot);
    else quantize_values_kernel<D, 2, false><<<grid, 256, 0, stream>>>(job, per_slot);
  } else {
    if (bf16) quantize_values_kernel<D, 4, true><<<grid, 256, 0, stream>>>(job, per_slot);
    else quantize_values_kernel<D, 4, false><<<grid, 256, 0, stream>>>(job, per_slot);
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
