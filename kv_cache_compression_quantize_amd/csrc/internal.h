// Internal declarations shared by the host entry points and the kernel
// launchers of libaqkv.so.  Not part of the public ABI (see include/aqkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/aqkv.h"

namespace aqkv {

constexpr int kMaxSketch = 1024;
constexpr int kMaxQPerKv = 16;
constexpr int kBlockRows = 32;   // token rows per cache block record

// Block-record geometry (include/aqkv.h): fields in record order, bytes per
// row and offsets; rec = bytes of one 32-row record.
enum Field { F_CODES = 0, F_SIGNS, F_NORM, F_RNORM, F_VCODES, F_VSIDE, F_COUNT };
struct BlockLayout {
  int64_t row[F_COUNT];
  int64_t off[F_COUNT];
  int64_t rec;
};
// sf: side information (norms, value scales and minima) stored as half
// instead of fp32.
inline BlockLayout block_layout(int d, int w, int m, int vb, bool sf) {
  const int e = sf ? 2 : 4;   // bytes per side-information number
  BlockLayout L{};
  L.row[F_CODES] = static_cast<int64_t>(w) * d / 8;
  L.row[F_SIGNS] = m / 8;
  L.row[F_NORM] = e;
  L.row[F_RNORM] = w > 0 ? e : 0;
  L.row[F_VCODES] = static_cast<int64_t>(d) * vb / 8;
  L.row[F_VSIDE] = 2 * e * (d / 32);
  int64_t o = 0;
  for (int f = 0; f < F_COUNT; ++f) {
    L.off[f] = o;
    o += kBlockRows * L.row[f];
  }
  L.rec = o;
  return L;
}

// Element index (fp32 or half), within a record's val_side field, of the
// scale (j = 0) or min (j = 1) of value group g of the record's token t
// (0..31): group-major, tokens t and t + 4 of a group side by side
// (include/aqkv.h).
__host__ __device__ inline int side_index(int g, int t, int j) {
  return ((g * 16 + 4 * (t >> 3) + (t & 3)) * 2 + ((t >> 2) & 1)) * 2 + j;
}

// Byte offset, from a field's place in record 0, of cache row `row` (= slot *
// capacity + t, capacity a multiple of 32) of a field with rb bytes per row.
__host__ __device__ inline int64_t rec_row(int64_t row, int64_t rb, int64_t rec) {
  return (row >> 5) * rec + (row & 31) * rb;
}

// Everything a key-quantise launch needs, already validated.
struct KeyJob {
  const void *k;
  int dtype;             // aqkv_dtype
  int64_t heads;         // view heads (slot = b * heads + h)
  int64_t batch_stride, head_stride, token_stride;  // elements
  int64_t n_slots, n_tokens, token_offset, capacity;
  int d, w, m;
  int sf;                 // norms stored as half (else fp32)
  const uint8_t *ops;     // matrix-core operands of Pi and S Pi^T (or S), see quant_keys_mfma.hip
  const float *rot_scale; // a > 0 when every |Pi_ij| == a (then the Pi operands are +-1, exact); else 0
  const float *centroids, *boundaries;
  // cache fields, each at its place in record 0; row r at + rec_row(r, row bytes, rec)
  uint8_t *codes, *signs, *norm, *rnorm;
  int64_t rec;
  // floor(n / n_tokens) and floor(n / heads) for n < 2^31 as (n * m) >> (31 + s)
  // (div_magic; set by the key kernels' launchers)
  uint32_t tok_m, head_m;
  int tok_s, head_s;
};

// Division of 0 <= n < 2^31 by a launch-invariant d >= 1 as one multiply and a shift
// (Granlund and Montgomery, "Division by invariant integers using multiplication", 1994,
// Theorem 4.2 with 31-bit dividends): s = ceil(log2 d), m = ceil(2^(31 + s) / d) < 2^32,
// floor(n / d) = (n m) >> (31 + s)
inline void div_magic(int64_t d, uint32_t &m, int &s) {
  s = 0;
  while ((int64_t(1) << s) < d) ++s;
  m = static_cast<uint32_t>(((uint64_t(1) << (31 + s)) + static_cast<uint64_t>(d) - 1) / static_cast<uint64_t>(d));
}
__device__ __forceinline__ uint32_t div_by(uint32_t n, uint32_t m, int s) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * m) >> (31 + s));
}

struct ValueJob {
  const void *v;
  int dtype;
  int64_t heads;
  int64_t batch_stride, head_stride, token_stride;
  int64_t n_slots, n_tokens, token_offset, capacity;
  int d, vb, group;
  int sf;                 // scale and min stored as half (else fp32)
  // cache fields, each at its place in record 0; row r at + rec_row(r, row bytes, rec)
  uint8_t *codes, *side;
  int64_t rec;
  // floor(n / records per slot) and floor(n / heads) for n < 2^31 as (n * m) >> (31 + s)
  // (div_magic; set by the value kernel's launcher)
  uint32_t bps_m, head_m;
  int bps_s, head_s;
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
  int sf;                // side information stored as half (else fp32)
  int64_t n_slots, capacity, context;
  int g;                 // query heads per kv head
  int n_split;
  int64_t split_tokens;  // tokens per split (multiple of the chunk)
  const float *centroids;
  // cache: the slots' records (blocks) and each field at its place in record 0
  const uint8_t *blocks;
  int64_t rec;
  const uint8_t *codes, *signs, *norm, *rnorm, *vcodes, *vside;
  const float *q_rot, *q_sketch;
  float softmax_scale;
  float *scores;         // nullable [n_slots*g][context]
  float *out;            // [n_slots*g][d]
  float *part_acc;       // [n_slots*g][part_stride][d]
  float *part_ml;        // [n_slots*g][part_stride][2]
  int part_stride;       // partials per head (the decoder's splits; 0 when there is none)
  int scores_only;       // non-zero: only the score output is wanted (the matrix-core decoder then
                         // reads the key fields alone and writes no partials)
  // scores-only calls of the matrix-core decoder (one query head per slot): per record, the
  // largest cosine score / ||k|| of its tokens, at rec_max[slot * rec_max_stride + record]
  float *rec_max;
  int64_t rec_max_stride;
  // matrix-core decoder over listed records only: context is then 32 x the list length,
  // record i of the slot's range is rec_list[slot * list_stride + i], and tokens at or
  // past list_context are masked
  const int32_t *rec_list;
  int64_t list_stride, list_context;
};

// The recent-token window of a decode call, merged in by the combine
constexpr int kMaxWindow = 1024;
struct WindowJob {
  const void *k, *v;     // [batch][heads][n_window][d] views
  int dtype;
  int64_t heads;         // kv heads
  int64_t k_bs, k_hs, k_ts, v_bs, v_hs, v_ts;   // strides in elements
  int n_window;
  const float *q;        // [n_slots*g][d] fp32
  int g;
  float softmax_scale;
};

// Query-aware top-K preselection and decode over the chosen tokens
constexpr int64_t kMaxBudget = int64_t{1} << 20;
// the select kernel indexes a slot's rows with 32-bit integers, a batch of
// rows past the last one included
constexpr int64_t kMaxTopkContext = (int64_t{1} << 31) - (int64_t{1} << 20);
struct TopkJob {
  int d, w, m, vb, g;
  int sf;                          // side information stored as half (else fp32)
  int64_t n_slots, capacity, context, rec;
  const uint8_t *codes, *signs, *norm, *rnorm, *vcodes, *vside;   // fields at their place in record 0
  const float *centroids;
  float *scores;                   // [n_slots][context] estimates for the selection query (overwritten)
  const float *q_rot, *q_sketch;   // per query head
  int budget;                      // chosen tokens per slot (1..context)
  int32_t *selected;               // [n_slots][budget]
  float softmax_scale;
  float *part_acc, *part_ml;       // [n_slots*g][topk_chunks(budget)][d], [..][2]
};

// Decode split-K plan shared by the workspace query and the launch.
struct DecodePlan {
  bool mfma;             // matrix-core kernel (else the scalar fallback)
  int n_split;
  int64_t split_tokens;
  size_t acc_bytes, ml_bytes, total_bytes;
};
DecodePlan decode_plan(int d, int w, int m, int vb, bool sf, int64_t n_slots, int g, int64_t context);

// Launchers (return a hipError_t from hipGetLastError after the launch).
// matrix-core key quantisation: operand preparation (workspace) + kernel
size_t key_operand_bytes(int d, int w, int m);
// the workspace: the operands, then (at key_operand_header(d, w, m)) one float, the rotation's common |Pi_ij| or 0
size_t key_operand_header(int d, int w, int m);
hipError_t launch_key_operands(const float *rotation, const float *sketch, uint8_t *ops, int d, int w, int m,
                               hipStream_t stream);
hipError_t launch_quantize_keys_mfma(const KeyJob &job, hipStream_t stream);
// pure-QJL bf16 keys at d = 128 with the sketch resident in registers (quant_keys_qjl.hip);
// its operands (qjl_operand_bytes(m), from launch_qjl_operands) follow the 256-byte
// rotation-scale header of the prepared workspace for the shapes qjl_shape accepts
bool qjl_shape(int d, int w, int m);
size_t qjl_operand_bytes(int m);
hipError_t launch_qjl_operands(const float *sketch, uint8_t *ops, int m, hipStream_t stream);
bool quantize_keys_qjl_supported(const KeyJob &job);
hipError_t launch_quantize_keys_qjl(const KeyJob &job, hipStream_t stream);
hipError_t launch_quantize_values(const ValueJob &job, hipStream_t stream);
hipError_t launch_prepare_query(const QueryJob &job, hipStream_t stream);
hipError_t launch_decode(const DecodeJob &job, hipStream_t stream);
hipError_t launch_combine(const DecodeJob &job, hipStream_t stream);
int topk_chunks(int budget);
// the slots' selection queries (sum of their heads' unit queries), rotated (q_rot, may be null) and sketched
hipError_t launch_selection_query(const float *q, int64_t n_slots, int d, int g, int m, const float *rotation,
                                  const float *sketch, float *q_rot, float *q_sk, hipStream_t stream);
hipError_t launch_topk(const TopkJob &job, hipStream_t stream);
// the `budget` records with the largest rec_max values of each slot ([n_slots][n_records],
// overwritten with the order keys; ties to the lower record), as increasing record indices
hipError_t launch_select_records(float *rec_max, int64_t n_slots, int64_t n_records, int budget,
                                 int32_t *selected, hipStream_t stream);
// the split combine with a recent-token window merged in (in place of launch_combine)
hipError_t launch_combine_window(const DecodeJob &job, const WindowJob &wj, hipStream_t stream);
bool decode_supported(int d, int w, int g, int m, int vb);
// matrix-core decode kernel (partials only; launch_combine merges them), shapes with a compiled kernel
bool decode_mfma_supported(int d, int w, int g, int m, int vb, bool sf);
int decode_mfma_blocks_per_cu(int d, int w, int g, int m, int vb, bool sf);
hipError_t launch_decode_mfma(const DecodeJob &job, hipStream_t stream);
// per head_dim kernel launchers (decode_fast_d*.hip)
hipError_t launch_decode_fast_d64(const DecodeJob &job, hipStream_t stream);
hipError_t launch_decode_fast_d128(const DecodeJob &job, hipStream_t stream);
hipError_t launch_decode_fast_d256(const DecodeJob &job, hipStream_t stream);

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Cache policy of data a kernel reads once (the K / V views being quantised, the
// cache records a decode streams): non-temporal.  On MI355X a plain 4 GiB read
// stream measured 5.6-6.1 TB/s, the same stream with non-temporal loads 6.2-6.7 TB/s.
constexpr int kStreamPolicy = 2;   // the nt bit of a gfx950 vector-memory instruction's cache policy
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Side information as stored: fp32, or the nearest IEEE half (ties to even;
// finite values beyond the half range saturate to +-65504, so a stored half is
// never infinite unless the fp32 value was).
__device__ __forceinline__ _Float16 side_half(float x) {
  const float a = fabsf(x);
  return static_cast<_Float16>(a > 65504.0f && a < __builtin_inff() ? copysignf(65504.0f, x) : x);
}
// side number i of a field that holds fp32 (sf false) or half (sf true) numbers
__device__ __forceinline__ float load_side(const uint8_t *p, int64_t i, bool sf) {
  return sf ? static_cast<float>(reinterpret_cast<const _Float16 *>(p)[i]) : reinterpret_cast<const float *>(p)[i];
}
__device__ __forceinline__ void store_side(uint8_t *p, int64_t i, bool sf, float x) {
  if (sf) reinterpret_cast<_Float16 *>(p)[i] = side_half(x);
  else reinterpret_cast<float *>(p)[i] = x;
}

}  // namespace aqkv
