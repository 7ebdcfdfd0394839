// Internal declarations shared by the host entry points and the kernel
// launchers of libaqkv.so.  Not part of the public ABI (see include/aqkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/aqkv.h"

namespace aqkv {

constexpr int kMaxSketch = 1024;
constexpr int kMaxQPerKv = 16;

// Everything a key-quantise launch needs, already validated.
struct KeyJob {
  const void *k;
  int dtype;             // aqkv_dtype
  int64_t heads;         // view heads (slot = b * heads + h)
  int64_t batch_stride, head_stride, token_stride;  // elements
  int64_t n_slots, n_tokens, token_offset, capacity;
  int d, w, m;
  const uint8_t *ops;     // matrix-core operands of Pi and S Pi^T (or S), see quant_keys_mfma.hip
  const float *centroids, *boundaries;
  uint8_t *codes, *signs;
  float *norm, *rnorm;
};

struct ValueJob {
  const void *v;
  int dtype;
  int64_t heads;
  int64_t batch_stride, head_stride, token_stride;
  int64_t n_slots, n_tokens, token_offset, capacity;
  int d, vb, group;
  uint8_t *codes;
  float *scale, *vmin;
};

struct QueryJob {
  const void *q;
  int dtype;
  int64_t n_q;
  int d, w, m;
  const float *rotation, *sketch;
  float *q_rot, *q_sketch;
};

struct DecodeJob {
  int d, w, m, vb, group;
  int64_t n_slots, capacity, context;
  int g;                 // query heads per kv head
  int n_split;
  int64_t split_tokens;  // tokens per split (multiple of the chunk)
  const float *centroids;
  const uint8_t *codes, *signs;
  const float *norm, *rnorm;
  const uint8_t *vcodes;
  const float *vscale, *vmin;
  const float *q_rot, *q_sketch;
  float softmax_scale;
  float *scores;         // nullable [n_slots*g][context]
  float *out;            // [n_slots*g][d]
  float *part_acc;       // [n_slots*g][n_split][d]
  float *part_ml;        // [n_slots*g][n_split][2]
  // matrix-core decoder only: packed query operands written by decode_pack_kernel
  uint8_t *qpack;        // [n_slots][row blocks][chunks][64 lanes][16 B]
  float *qconst;         // [n_slots*g][4]: integer scales and constant terms per head
  int *qodd;             // [n_slots]: 1 when only the odd-size code planes are laid out
};

// Decode split-K plan shared by the workspace query and the launch.
struct DecodePlan {
  bool mfma;             // matrix-core kernel (else the scalar fallback)
  int n_split;
  int64_t split_tokens;
  size_t acc_bytes, ml_bytes, pack_bytes, const_bytes, odd_bytes, total_bytes;
};
DecodePlan decode_plan(int d, int w, int m, int vb, int64_t n_slots, int g, int64_t context);

// Launchers (return a hipError_t from hipGetLastError after the launch).
// matrix-core key quantisation: operand preparation (workspace) + kernel
size_t key_operand_bytes(int d, int w, int m);
hipError_t launch_key_operands(const float *rotation, const float *sketch, uint8_t *ops, int d, int w, int m,
                               hipStream_t stream);
hipError_t launch_quantize_keys_mfma(const KeyJob &job, hipStream_t stream);
hipError_t launch_quantize_values(const ValueJob &job, hipStream_t stream);
hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream);
hipError_t launch_decode(const DecodeJob &job, hipStream_t stream);
hipError_t launch_combine(const DecodeJob &job, hipStream_t stream);
bool decode_supported(int d, int w, int g, int m, int vb);
// matrix-core decode (query pack + decode + combine), shapes with a compiled kernel
bool decode_mfma_supported(int d, int w, int g, int m, int vb);
int decode_mfma_blocks_per_cu(int d, int w, int g, int m, int vb);
size_t decode_mfma_pack_bytes(int d, int w, int g, int m, int64_t n_slots);
hipError_t launch_decode_mfma(const DecodeJob &job, hipStream_t stream);
// per head_dim kernel launchers (decode_fast_d*.hip)
hipError_t launch_decode_fast_d64(const DecodeJob &job, hipStream_t stream);
hipError_t launch_decode_fast_d128(const DecodeJob &job, hipStream_t stream);
hipError_t launch_decode_fast_d256(const DecodeJob &job, hipStream_t stream);

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

}  // namespace aqkv
