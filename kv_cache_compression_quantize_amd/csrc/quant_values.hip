// Value quantisation kernel: per token, per group of 32 contiguous channels,
// min-max quantisation to 2 or 4 bits with LSB-first packing (TurboQuant
// article, component table "Value 分组量化 2 bit/维, min-max", and §七,
// kv_cache.py "value group quantisation and bit packing").
//
// One thread owns one (slot, token, group): 32 elements are loaded with
// 16-byte loads, reduced to min / max, coded in IEEE fp32 (subtract, correctly
// rounded divide, round-half-even) and written as one 8- or 16-byte word.
// The work is a single streaming pass, bound by HBM bandwidth.
#include "internal.h"

namespace aqkv {
namespace {

constexpr int kGroup = 32;

template <int VB, bool BF16>
__global__ __launch_bounds__(256) void quantize_values_kernel(ValueJob job) {
  const int groups = job.d / kGroup;
  const int64_t total = job.n_slots * job.n_tokens * groups;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int g = static_cast<int>(gid % groups);
  const int64_t rest = gid / groups;
  const int64_t t = rest % job.n_tokens;
  const int64_t s = rest / job.n_tokens;
  const int64_t b = s / job.heads, h = s % job.heads;
  const int64_t src = b * job.batch_stride + h * job.head_stride + t * job.token_stride + g * kGroup;

  float v[kGroup];
  if (BF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(job.v) + src);
#pragma unroll
    for (int i = 0; i < kGroup / 8; ++i) {
      const uint4 q = p[i];
      const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
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
      const float4 q = p[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
  float mn = v[0], mx = v[0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  constexpr int kLevels = (1 << VB) - 1;
  const float scale = (mx - mn) / static_cast<float>(kLevels);   // IEEE divide
  constexpr int kWords = kGroup * VB / 32;
  uint32_t words[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) words[i] = 0;
  if (scale > 0.0f) {
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      float c = rintf((v[i] - mn) / scale);                    // IEEE subtract, divide, RNE
      c = fminf(fmaxf(c, 0.0f), static_cast<float>(kLevels));
      const uint32_t code = static_cast<uint32_t>(c);
      words[(i * VB) / 32] |= code << ((i * VB) % 32);
    }
  }
  const int64_t row = s * job.capacity + job.token_offset + t;
  uint8_t *dst = job.codes + row * (job.d * VB / 8) + g * (kGroup * VB / 8);
  if (VB == 2) {
    *reinterpret_cast<uint2 *>(dst) = make_uint2(words[0], words[1]);
  } else {
    *reinterpret_cast<uint4 *>(dst) = make_uint4(words[0], words[1], words[2 % kWords], words[3 % kWords]);
  }
  job.scale[row * groups + g] = scale;
  job.vmin[row * groups + g] = mn;
}

}  // namespace

hipError_t launch_quantize_values(const ValueJob &job, hipStream_t stream) {
  const int64_t total = job.n_slots * job.n_tokens * (job.d / kGroup);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const bool bf16 = job.dtype == AQKV_BF16;
  if (job.vb == 2) {
    if (bf16) quantize_values_kernel<2, true><<<blocks, threads, 0, stream>>>(job);
    else quantize_values_kernel<2, false><<<blocks, threads, 0, stream>>>(job);
  } else {
    if (bf16) quantize_values_kernel<4, true><<<blocks, threads, 0, stream>>>(job);
    else quantize_values_kernel<4, false><<<blocks, threads, 0, stream>>>(job);
  }
  return hipGetLastError();
}

}  // namespace aqkv
