// C entry points of libaqkv.so: argument validation on the host, then the
// kernel launchers.  Validation never touches the HIP runtime, so a call that
// fails validation works (and returns its status) on a machine without a GPU.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

using namespace aqkv;

namespace {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

aqkv_status check_config(const aqkv_config *cfg) {
  if (!cfg) return AQKV_ERR_NULL;
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  if (d != 64 && d != 128 && d != 256) return AQKV_ERR_SHAPE;
  if (w < 0 || w > 3) return AQKV_ERR_SHAPE;
  if (m < 64 || m > kMaxSketch || m % 64 != 0) return AQKV_ERR_SHAPE;
  if (cfg->value_bits != 2 && cfg->value_bits != 4) return AQKV_ERR_SHAPE;
  if (cfg->value_group != 32) return AQKV_ERR_SHAPE;
  if (cfg->side_f16 != 0 && cfg->side_f16 != 1) return AQKV_ERR_SHAPE;
  return AQKV_OK;
}

aqkv_status check_view(const aqkv_kv_view *v, int d) {
  if (!v) return AQKV_ERR_NULL;
  if (v->dtype != AQKV_FP32 && v->dtype != AQKV_BF16) return AQKV_ERR_DTYPE;
  if (v->batch < 0 || v->heads < 0 || v->tokens < 0) return AQKV_ERR_SHAPE;
  if (v->tokens > 0 && v->batch * v->heads > 0 && !v->data) return AQKV_ERR_NULL;
  if (v->batch_stride < 0 || v->head_stride < 0 || v->token_stride < d) return AQKV_ERR_SHAPE;
  if (v->batch_stride % 8 || v->head_stride % 8 || v->token_stride % 8) return AQKV_ERR_ALIGN;
  if (v->data && !aligned(v->data, 16)) return AQKV_ERR_ALIGN;
  return AQKV_OK;
}

aqkv_status check_cache_shape(const aqkv_cache *c) {
  if (!c) return AQKV_ERR_NULL;
  if (c->n_slots < 0 || c->capacity < 0) return AQKV_ERR_SHAPE;
  if (c->capacity % kBlockRows) return AQKV_ERR_SHAPE;   // whole 32-token block records
  return AQKV_OK;
}

aqkv_status check_plane(const void *p) {
  if (!p) return AQKV_ERR_NULL;
  if (!aligned(p, 16)) return AQKV_ERR_ALIGN;
  return AQKV_OK;
}

aqkv_status check_blocks(const aqkv_cache *c) {
  if (!c->blocks) return AQKV_ERR_NULL;
  if (!aligned(c->blocks, 16)) return AQKV_ERR_ALIGN;
  return AQKV_OK;
}

BlockLayout layout_of(const aqkv_config *cfg) {
  return block_layout(cfg->head_dim, cfg->mse_bits, cfg->sketch_dim, cfg->value_bits, cfg->side_f16 != 0);
}

aqkv_status hip_status(hipError_t e) { return e == hipSuccess ? AQKV_OK : AQKV_ERR_HIP; }

size_t key_workspace_bytes(int d, int w, int m) {
  // matrix-core operands of Pi and S Pi^T (w > 0) or S (w == 0), f16 hi + lo; then the
  // rotation-scale float (256 bytes); then, for pure-QJL shapes, the sketch in the layout
  // of the register-resident QJL kernel
  return aqkv::key_operand_header(d, w, m) + 256 + (aqkv::qjl_shape(d, w, m) ? aqkv::qjl_operand_bytes(m) : 0);
}

}  // namespace

namespace aqkv {

DecodePlan decode_plan(int d, int w, int m, int vb, bool sf, int64_t n_slots, int g, int64_t context) {
  constexpr int64_t kGrain = 256;      // split granularity (tokens)
  constexpr int64_t kCUs = 256;        // MI355X compute units
  DecodePlan p{};
  p.mfma = decode_mfma_supported(d, w, g, m, vb, sf);
  // one round of resident blocks for the matrix-core kernel (each block pays its
  // query-side prologue once), ~4 per CU otherwise
  const int64_t target = p.mfma ? kCUs * decode_mfma_blocks_per_cu(d, w, g, m, vb, sf) : 4 * kCUs;
  const int64_t grains = (context + kGrain - 1) / kGrain;
  int64_t split = n_slots > 0 ? (target + n_slots - 1) / n_slots : 1;
  if (split > grains) split = grains;
  if (split < 1) split = 1;
  const int64_t per_split = grains > 0 ? (grains + split - 1) / split : 1;
  p.split_tokens = per_split * kGrain;
  p.n_split = static_cast<int>(grains > 0 ? (grains + per_split - 1) / per_split : 1);
  const size_t heads = static_cast<size_t>(n_slots) * g;
  p.acc_bytes = round_up(heads * p.n_split * d * sizeof(float), 256);
  p.ml_bytes = round_up(heads * p.n_split * 2 * sizeof(float), 256);
  p.total_bytes = p.acc_bytes + p.ml_bytes;
  return p;
}

}  // namespace aqkv

extern "C" {

const char *aqkv_status_string(aqkv_status s) {
  switch (s) {
    case AQKV_OK: return "ok";
    case AQKV_ERR_NULL: return "required pointer is NULL";
    case AQKV_ERR_SHAPE: return "unsupported or inconsistent shape";
    case AQKV_ERR_ALIGN: return "misaligned pointer or stride";
    case AQKV_ERR_CAPACITY: return "token range exceeds cache capacity";
    case AQKV_ERR_WORKSPACE: return "workspace missing or too small";
    case AQKV_ERR_DTYPE: return "unknown element type";
    case AQKV_ERR_HIP: return "HIP runtime error";
    case AQKV_ERR_UNSUPPORTED: return "not supported by the library";
    case AQKV_ERR_SCRATCH: return "request needs more than the library's static scratch";
  }
  return "unknown status";
}

aqkv_status aqkv_cache_layout(const aqkv_config *cfg, aqkv_layout *out) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (out) {
    const BlockLayout L = layout_of(cfg);
    aqkv_fields *rb = &out->row_bytes, *of = &out->offset;
    rb->key_codes = L.row[F_CODES];
    rb->key_signs = L.row[F_SIGNS];
    rb->key_norm = L.row[F_NORM];
    rb->key_rnorm = L.row[F_RNORM];
    rb->val_codes = L.row[F_VCODES];
    rb->val_side = L.row[F_VSIDE];
    of->key_codes = L.off[F_CODES];
    of->key_signs = L.off[F_SIGNS];
    of->key_norm = L.off[F_NORM];
    of->key_rnorm = L.off[F_RNORM];
    of->val_codes = L.off[F_VCODES];
    of->val_side = L.off[F_VSIDE];
    out->block_bytes = L.rec;
  }
  return AQKV_OK;
}

size_t aqkv_quantize_keys_workspace_bytes(const aqkv_config *cfg) {
  if (check_config(cfg) != AQKV_OK) return 0;
  return key_workspace_bytes(cfg->head_dim, cfg->mse_bits, cfg->sketch_dim);
}

size_t aqkv_decode_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads,
                                   int32_t n_kv_heads, int64_t context_len) {
  if (check_config(cfg) != AQKV_OK) return 0;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || context_len < 0) return 0;
  const int64_t n_slots = static_cast<int64_t>(batch) * n_kv_heads;
  return decode_plan(cfg->head_dim, cfg->mse_bits, cfg->sketch_dim, cfg->value_bits, cfg->side_f16 != 0, n_slots,
                     n_q_heads / n_kv_heads, context_len)
      .total_bytes;
}

// The layer's matrix-core operands into the workspace (checked arguments)
static aqkv_status key_operands(const aqkv_config *cfg, const aqkv_layer *layer, void *workspace,
                                size_t workspace_bytes, hipStream_t s) {
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  aqkv_status st;
  if (!layer) return AQKV_ERR_NULL;
  if ((st = check_plane(layer->sketch)) != AQKV_OK) return st;
  if (w > 0 && (st = check_plane(layer->rotation)) != AQKV_OK) return st;
  if (!workspace || workspace_bytes < key_workspace_bytes(d, w, m)) return AQKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AQKV_ERR_ALIGN;
  return launch_key_operands(layer->rotation, layer->sketch, static_cast<uint8_t *>(workspace), d, w, m, s) ==
                 hipSuccess
             ? AQKV_OK
             : AQKV_ERR_HIP;
}

aqkv_status aqkv_prepare_key_operands(const aqkv_config *cfg, const aqkv_layer *layer, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  return key_operands(cfg, layer, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

static aqkv_status quantize_keys(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_kv_view *k,
                                 int64_t token_offset, const aqkv_cache *cache, void *workspace,
                                 size_t workspace_bytes, void *stream, bool prepare) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (!layer) return AQKV_ERR_NULL;
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  if ((st = check_view(k, d)) != AQKV_OK) return st;
  if ((st = check_cache_shape(cache)) != AQKV_OK) return st;
  if (k->batch * k->heads != cache->n_slots) return AQKV_ERR_SHAPE;
  if (token_offset < 0) return AQKV_ERR_SHAPE;
  if (token_offset + k->tokens > cache->capacity) return AQKV_ERR_CAPACITY;
  if (prepare) {
    if ((st = check_plane(layer->sketch)) != AQKV_OK) return st;
    if (w > 0 && (st = check_plane(layer->rotation)) != AQKV_OK) return st;
  }
  if (w > 0 && (!layer->centroids || !layer->boundaries)) return AQKV_ERR_NULL;
  if ((st = check_blocks(cache)) != AQKV_OK) return st;
  const size_t need = key_workspace_bytes(d, w, m);
  if (!workspace || workspace_bytes < need) return AQKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AQKV_ERR_ALIGN;
  if (k->tokens == 0 || cache->n_slots == 0) return AQKV_OK;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t *ops = static_cast<uint8_t *>(workspace);
  if (prepare && (st = key_operands(cfg, layer, workspace, workspace_bytes, s)) != AQKV_OK) return st;
  KeyJob job{};
  job.k = k->data;
  job.dtype = k->dtype;
  job.heads = k->heads;
  job.batch_stride = k->batch_stride;
  job.head_stride = k->head_stride;
  job.token_stride = k->token_stride;
  job.n_slots = cache->n_slots;
  job.n_tokens = k->tokens;
  job.token_offset = token_offset;
  job.capacity = cache->capacity;
  job.d = d;
  job.w = w;
  job.m = m;
  job.sf = cfg->side_f16;
  job.ops = ops;
  job.rot_scale = reinterpret_cast<const float *>(ops + key_operand_header(d, w, m));
  job.centroids = layer->centroids;
  job.boundaries = layer->boundaries;
  const BlockLayout L = layout_of(cfg);
  job.codes = cache->blocks + L.off[F_CODES];
  job.signs = cache->blocks + L.off[F_SIGNS];
  job.norm = cache->blocks + L.off[F_NORM];
  job.rnorm = cache->blocks + L.off[F_RNORM];
  job.rec = L.rec;
  return hip_status(launch_quantize_keys_mfma(job, s));
}

aqkv_status aqkv_quantize_keys(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_kv_view *k,
                               int64_t token_offset, const aqkv_cache *cache, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return quantize_keys(cfg, layer, k, token_offset, cache, workspace, workspace_bytes, stream, true);
}

aqkv_status aqkv_quantize_keys_prepared(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_kv_view *k,
                                        int64_t token_offset, const aqkv_cache *cache, const void *workspace,
                                        size_t workspace_bytes, void *stream) {
  return quantize_keys(cfg, layer, k, token_offset, cache, const_cast<void *>(workspace), workspace_bytes, stream,
                       false);
}

aqkv_status aqkv_quantize_values(const aqkv_config *cfg, const aqkv_kv_view *v, int64_t token_offset,
                                 const aqkv_cache *cache, void *stream) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  const int d = cfg->head_dim;
  if ((st = check_view(v, d)) != AQKV_OK) return st;
  if ((st = check_cache_shape(cache)) != AQKV_OK) return st;
  if (v->batch * v->heads != cache->n_slots) return AQKV_ERR_SHAPE;
  if (token_offset < 0) return AQKV_ERR_SHAPE;
  if (token_offset + v->tokens > cache->capacity) return AQKV_ERR_CAPACITY;
  if ((st = check_blocks(cache)) != AQKV_OK) return st;
  if (v->tokens == 0 || cache->n_slots == 0) return AQKV_OK;
  ValueJob job{};
  job.v = v->data;
  job.dtype = v->dtype;
  job.heads = v->heads;
  job.batch_stride = v->batch_stride;
  job.head_stride = v->head_stride;
  job.token_stride = v->token_stride;
  job.n_slots = cache->n_slots;
  job.n_tokens = v->tokens;
  job.token_offset = token_offset;
  job.capacity = cache->capacity;
  job.d = d;
  job.vb = cfg->value_bits;
  job.group = cfg->value_group;
  job.sf = cfg->side_f16;
  const BlockLayout L = layout_of(cfg);
  job.codes = cache->blocks + L.off[F_VCODES];
  job.side = cache->blocks + L.off[F_VSIDE];
  job.rec = L.rec;
  return hip_status(launch_quantize_values(job, static_cast<hipStream_t>(stream)));
}

aqkv_status aqkv_prepare_query(const aqkv_config *cfg, const aqkv_layer *layer, const void *q,
                               aqkv_dtype dtype, int64_t n_q, float *q_rot, float *q_sketch,
                               void *stream) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (!layer) return AQKV_ERR_NULL;
  if (dtype != AQKV_FP32 && dtype != AQKV_BF16) return AQKV_ERR_DTYPE;
  if (n_q < 0) return AQKV_ERR_SHAPE;
  const int w = cfg->mse_bits;
  if (n_q == 0) return AQKV_OK;
  if (!q || !q_sketch || !layer->sketch) return AQKV_ERR_NULL;
  if (w > 0 && (!q_rot || !layer->rotation)) return AQKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(q_sketch, 16) || (q_rot && !aligned(q_rot, 16))) return AQKV_ERR_ALIGN;
  QueryJob job{};
  job.q = q;
  job.dtype = dtype;
  job.n_q = n_q;
  job.d = cfg->head_dim;
  job.w = w;
  job.m = cfg->sketch_dim;
  job.rotation = layer->rotation;
  job.sketch = layer->sketch;
  job.q_rot = w > 0 ? q_rot : nullptr;
  job.q_sketch = q_sketch;
  return hip_status(launch_prepare_query(job, static_cast<hipStream_t>(stream)));
}

// Static device scratch of the allocation-free decode: the split partials live
// here instead of in a caller workspace.  Each device holds its own copy for
// the life of the process; host code reaches it only through the address
// hipGetSymbolAddress reports for the device (the array's name is a host-side
// stand-in, not a device address).
constexpr size_t kStaticScratchBytes = size_t{8} << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];   // per device, set once under scratch_mutex

// This device's copy of the scratch (nullptr on a HIP error); resolved once per
// device, with that device current (it is the caller's current device).
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}
}  // namespace

// The recent-token window of a decode call (all pointers already checked)
struct WindowArgs {
  const float *q;
  const aqkv_kv_view *k, *v;
};

// Matrix-core decoder options of the record top-K: the scoring pass's per-record maximum
// cosine output, or a decode over listed records only (context_len is then 32 x the list
// length and list_context the cached length)
struct DecodeExtra {
  float *rec_max;
  int64_t rec_max_stride;
  const int32_t *rec_list;
  int64_t list_stride, list_context;
};

static aqkv_status decode(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_cache *cache, int32_t batch,
                          int32_t n_q_heads, int32_t n_kv_heads, int64_t context_len, const float *q_rot,
                          const float *q_sketch, float softmax_scale, float *scores, float *out, void *workspace,
                          size_t workspace_bytes, void *stream, const WindowArgs *win, bool scores_only = false,
                          void *(*static_scratch)() = nullptr, const DecodeExtra *extra = nullptr) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (!layer) return AQKV_ERR_NULL;
  if ((st = check_cache_shape(cache)) != AQKV_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || context_len < 0) return AQKV_ERR_SHAPE;
  if (n_q_heads % n_kv_heads) return AQKV_ERR_SHAPE;
  const int g = n_q_heads / n_kv_heads;
  if (g > kMaxQPerKv) return AQKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(batch) * n_kv_heads != cache->n_slots) return AQKV_ERR_SHAPE;
  if (context_len > cache->capacity) return AQKV_ERR_CAPACITY;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return AQKV_ERR_SHAPE;
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  if (!decode_supported(d, w, g, m, cfg->value_bits) &&
      !decode_mfma_supported(d, w, g, m, cfg->value_bits, cfg->side_f16 != 0))
    return AQKV_ERR_UNSUPPORTED;
  if (win) {
    if (!win->k || !win->v) return AQKV_ERR_NULL;
    if ((st = check_view(win->k, d)) != AQKV_OK || (st = check_view(win->v, d)) != AQKV_OK) return st;
    if (win->k->dtype != win->v->dtype) return AQKV_ERR_DTYPE;
    if (win->k->batch != batch || win->v->batch != batch || win->k->heads != n_kv_heads ||
        win->v->heads != n_kv_heads || win->k->tokens != win->v->tokens)
      return AQKV_ERR_SHAPE;
    if (win->k->tokens > kMaxWindow) return AQKV_ERR_UNSUPPORTED;
  }
  if (batch == 0) return AQKV_OK;
  if (!out || !q_sketch) return AQKV_ERR_NULL;
  if (w > 0 && (!q_rot || !layer->centroids)) return AQKV_ERR_NULL;
  if (win && !win->q) return AQKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q_sketch, 16) || (q_rot && !aligned(q_rot, 16)) ||
      (scores && !aligned(scores, 16)) || (win && !aligned(win->q, 16)))
    return AQKV_ERR_ALIGN;
  if (context_len > 0 && (st = check_blocks(cache)) != AQKV_OK) return st;
  const DecodePlan plan = decode_plan(d, w, m, cfg->value_bits, cfg->side_f16 != 0, cache->n_slots, g, context_len);
  if (static_scratch) {
    // the allocation-free call: the partials go to the library's static scratch (looked up
    // only after every host-side check has passed)
    if (plan.total_bytes > kStaticScratchBytes) return AQKV_ERR_SCRATCH;
    workspace = static_scratch();
    workspace_bytes = kStaticScratchBytes;
    if (!workspace) return AQKV_ERR_HIP;
  }
  if (!workspace || workspace_bytes < plan.total_bytes) return AQKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AQKV_ERR_ALIGN;

  DecodeJob job{};
  job.d = d;
  job.w = w;
  job.m = m;
  job.vb = cfg->value_bits;
  job.group = cfg->value_group;
  job.sf = cfg->side_f16;
  job.n_slots = cache->n_slots;
  job.capacity = cache->capacity;
  job.context = context_len;
  job.g = g;
  job.n_split = plan.n_split;
  job.split_tokens = plan.split_tokens;
  job.centroids = layer->centroids;
  const BlockLayout L = layout_of(cfg);
  job.blocks = cache->blocks;
  job.rec = L.rec;
  job.codes = cache->blocks + L.off[F_CODES];
  job.signs = cache->blocks + L.off[F_SIGNS];
  job.norm = cache->blocks + L.off[F_NORM];
  job.rnorm = cache->blocks + L.off[F_RNORM];
  job.vcodes = cache->blocks + L.off[F_VCODES];
  job.vside = cache->blocks + L.off[F_VSIDE];
  job.q_rot = q_rot;
  job.q_sketch = q_sketch;
  job.softmax_scale = softmax_scale;
  job.scores = scores;
  job.out = out;
  job.part_acc = static_cast<float *>(workspace);
  char *ws = static_cast<char *>(workspace);
  job.part_ml = reinterpret_cast<float *>(ws + plan.acc_bytes);
  job.scores_only = scores_only && (scores || (extra && extra->rec_max)) && !win ? 1 : 0;
  if (extra) {
    if (!plan.mfma) return AQKV_ERR_UNSUPPORTED;
    job.rec_max = extra->rec_max;
    job.rec_max_stride = extra->rec_max_stride;
    job.rec_list = extra->rec_list;
    job.list_stride = extra->list_stride;
    job.list_context = extra->list_context;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the matrix-core decoder addresses a slot's records with 32-bit byte offsets
  if (plan.mfma && cache->capacity / kBlockRows * L.rec >= (int64_t(1) << 31)) return AQKV_ERR_UNSUPPORTED;
  // with a window and no history yet, the window is all there is
  const bool history = !win || context_len > 0;
  job.part_stride = history ? plan.n_split : 0;
  if (history) {
    const hipError_t e = plan.mfma ? launch_decode_mfma(job, s) : launch_decode(job, s);
    if (e != hipSuccess) return AQKV_ERR_HIP;
  }
  // scores_only: the caller wants the score output alone, so the partials are not merged
  if (!win) return scores_only ? AQKV_OK : hip_status(launch_combine(job, s));
  {
    WindowJob wj{};
    wj.k = win->k->data;
    wj.v = win->v->data;
    wj.dtype = win->k->dtype;
    wj.heads = n_kv_heads;
    wj.k_bs = win->k->batch_stride;
    wj.k_hs = win->k->head_stride;
    wj.k_ts = win->k->token_stride;
    wj.v_bs = win->v->batch_stride;
    wj.v_hs = win->v->head_stride;
    wj.v_ts = win->v->token_stride;
    wj.n_window = static_cast<int>(win->k->tokens);
    wj.q = win->q;
    wj.g = g;
    wj.softmax_scale = softmax_scale;
    return hip_status(launch_combine_window(job, wj, s));
  }
}

aqkv_status aqkv_decode_attention(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_cache *cache,
                                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t context_len,
                                  const float *q_rot, const float *q_sketch, float softmax_scale,
                                  float *scores, float *out, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  return decode(cfg, layer, cache, batch, n_q_heads, n_kv_heads, context_len, q_rot, q_sketch, softmax_scale,
                scores, out, workspace, workspace_bytes, stream, nullptr);
}

// Workspace of the top-K decode: the selection query, its rotation and sketch,
// the selection scores, the scoring decode's output and split workspace, the
// chosen indices and the chunk partials, each 256-byte aligned.
struct TopkLayout {
  size_t qsel_rot, qsel_sk, scores, dec_out, dec_ws, dec_ws_bytes, sel, acc, ml, total;
};

static TopkLayout topk_layout(const aqkv_config *cfg, int64_t n_slots, int g, int64_t context, int budget) {
  const int d = cfg->head_dim, m = cfg->sketch_dim;
  TopkLayout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += round_up(bytes, 256);
    return here;
  };
  L.qsel_rot = take(sizeof(float) * n_slots * d);
  L.qsel_sk = take(sizeof(float) * n_slots * m);
  L.scores = take(sizeof(float) * n_slots * context);
  L.dec_out = take(sizeof(float) * n_slots * d);
  L.dec_ws_bytes =
      decode_plan(d, cfg->mse_bits, m, cfg->value_bits, cfg->side_f16 != 0, n_slots, 1, context).total_bytes;
  L.dec_ws = take(L.dec_ws_bytes);
  L.sel = take(sizeof(int32_t) * n_slots * budget);
  const int chunks = topk_chunks(budget);
  L.acc = take(sizeof(float) * n_slots * g * chunks * d);
  L.ml = take(sizeof(float) * n_slots * g * chunks * 2);
  L.total = at;
  return L;
}

size_t aqkv_decode_topk_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                        int64_t context_len, int64_t budget) {
  if (check_config(cfg) != AQKV_OK) return 0;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || context_len < 0 || budget < 1)
    return 0;
  const int64_t n_slots = static_cast<int64_t>(batch) * n_kv_heads;
  const int k = static_cast<int>(std::min<int64_t>(std::min<int64_t>(budget, context_len), kMaxBudget));
  return topk_layout(cfg, n_slots, n_q_heads / n_kv_heads, context_len, std::max(k, 1)).total;
}

aqkv_status aqkv_decode_attention_topk(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_cache *cache,
                                       int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t context_len,
                                       const float *q, const float *q_rot, const float *q_sketch, int64_t budget,
                                       float softmax_scale, int32_t *selected, float *out, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (!layer) return AQKV_ERR_NULL;
  if ((st = check_cache_shape(cache)) != AQKV_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || context_len < 0 || budget < 1) return AQKV_ERR_SHAPE;
  if (n_q_heads % n_kv_heads) return AQKV_ERR_SHAPE;
  const int g = n_q_heads / n_kv_heads;
  if (g > kMaxQPerKv) return AQKV_ERR_UNSUPPORTED;
  if (budget > kMaxBudget) return AQKV_ERR_UNSUPPORTED;
  if (context_len > kMaxTopkContext) return AQKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(batch) * n_kv_heads != cache->n_slots) return AQKV_ERR_SHAPE;
  if (context_len > cache->capacity) return AQKV_ERR_CAPACITY;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return AQKV_ERR_SHAPE;
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  if (!decode_supported(d, w, 1, m, cfg->value_bits) &&
      !decode_mfma_supported(d, w, 1, m, cfg->value_bits, cfg->side_f16 != 0))
    return AQKV_ERR_UNSUPPORTED;
  if (batch == 0) return AQKV_OK;
  if (!out || !q || !q_sketch || !layer->sketch) return AQKV_ERR_NULL;
  if (w > 0 && (!q_rot || !layer->centroids || !layer->rotation)) return AQKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(q_sketch, 16) || (q_rot && !aligned(q_rot, 16)) ||
      (selected && !aligned(selected, 4)))
    return AQKV_ERR_ALIGN;
  const int k = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(budget, context_len)));
  const TopkLayout TL = topk_layout(cfg, cache->n_slots, g, context_len, k);
  if (!workspace || workspace_bytes < TL.total) return AQKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AQKV_ERR_ALIGN;
  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (context_len == 0) {   // nothing cached: a combine over no parts writes out = 0
    DecodeJob zj{};
    zj.d = d;
    zj.g = g;
    zj.n_slots = cache->n_slots;
    zj.part_stride = 0;
    zj.part_acc = reinterpret_cast<float *>(ws + TL.acc);
    zj.part_ml = reinterpret_cast<float *>(ws + TL.ml);
    zj.out = out;
    return hip_status(launch_combine(zj, s));
  }
  if ((st = check_blocks(cache)) != AQKV_OK) return st;

  // 1. the selection query of every KV slot, rotated and sketched (one kernel)
  float *qsel_rot = reinterpret_cast<float *>(ws + TL.qsel_rot);
  float *qsel_sk = reinterpret_cast<float *>(ws + TL.qsel_sk);
  if (launch_selection_query(q, cache->n_slots, d, g, m, layer->rotation, layer->sketch, w > 0 ? qsel_rot : nullptr,
                             qsel_sk, s) != hipSuccess)
    return AQKV_ERR_HIP;
  // 2. its estimate for every cached token (the decoder's score output, one query per slot)
  float *scores = reinterpret_cast<float *>(ws + TL.scores);
  st = decode(cfg, layer, cache, batch, n_kv_heads, n_kv_heads, context_len, w > 0 ? qsel_rot : nullptr, qsel_sk,
              softmax_scale, scores, reinterpret_cast<float *>(ws + TL.dec_out), ws + TL.dec_ws, TL.dec_ws_bytes,
              stream, nullptr, true);
  if (st != AQKV_OK) return st;
  // 3. selection and decode over the chosen tokens, then the chunk combine
  const BlockLayout L = layout_of(cfg);
  TopkJob tj{};
  tj.d = d;
  tj.w = w;
  tj.m = m;
  tj.vb = cfg->value_bits;
  tj.sf = cfg->side_f16;
  tj.g = g;
  tj.n_slots = cache->n_slots;
  tj.capacity = cache->capacity;
  tj.context = context_len;
  tj.rec = L.rec;
  tj.codes = cache->blocks + L.off[F_CODES];
  tj.signs = cache->blocks + L.off[F_SIGNS];
  tj.norm = cache->blocks + L.off[F_NORM];
  tj.rnorm = cache->blocks + L.off[F_RNORM];
  tj.vcodes = cache->blocks + L.off[F_VCODES];
  tj.vside = cache->blocks + L.off[F_VSIDE];
  tj.centroids = layer->centroids;
  tj.scores = scores;
  tj.q_rot = q_rot;
  tj.q_sketch = q_sketch;
  tj.budget = k;
  tj.selected = selected ? selected : reinterpret_cast<int32_t *>(ws + TL.sel);
  tj.softmax_scale = softmax_scale;
  tj.part_acc = reinterpret_cast<float *>(ws + TL.acc);
  tj.part_ml = reinterpret_cast<float *>(ws + TL.ml);
  if (launch_topk(tj, s) != hipSuccess) return AQKV_ERR_HIP;
  DecodeJob cj{};
  cj.d = d;
  cj.g = g;
  cj.n_slots = cache->n_slots;
  cj.part_stride = topk_chunks(k);
  cj.part_acc = tj.part_acc;
  cj.part_ml = tj.part_ml;
  cj.out = out;
  return hip_status(launch_combine(cj, s));
}

// Workspace of the record top-K decode: the selection query, its rotation and sketch,
// the per-record maximum cosines, the scoring pass's output and split workspace, the
// chosen records and the split workspace of the decode over them, each 256-byte aligned.
struct BlockTopkLayout {
  size_t qsel_rot, qsel_sk, rec_max, dec_out, dec_ws, dec_ws_bytes, sel, list_ws, list_ws_bytes, total;
};
static BlockTopkLayout block_topk_layout(const aqkv_config *cfg, int64_t n_slots, int g, int64_t context,
                                         int64_t n_rec, int64_t nb) {
  const int d = cfg->head_dim, m = cfg->sketch_dim;
  const bool sf = cfg->side_f16 != 0;
  BlockTopkLayout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += round_up(bytes, 256);
    return here;
  };
  L.qsel_rot = take(sizeof(float) * n_slots * d);
  L.qsel_sk = take(sizeof(float) * n_slots * m);
  L.rec_max = take(sizeof(float) * n_slots * n_rec);
  L.dec_out = take(sizeof(float) * n_slots * d);
  L.dec_ws_bytes = decode_plan(d, cfg->mse_bits, m, cfg->value_bits, sf, n_slots, 1, context).total_bytes;
  L.dec_ws = take(L.dec_ws_bytes);
  L.sel = take(sizeof(int32_t) * n_slots * nb);
  L.list_ws_bytes = decode_plan(d, cfg->mse_bits, m, cfg->value_bits, sf, n_slots, g, nb * kBlockRows).total_bytes;
  L.list_ws = take(L.list_ws_bytes);
  L.total = at;
  return L;
}

// records chosen for a budget of `budget` tokens over n_rec records
static int64_t block_budget(int64_t budget, int64_t n_rec) {
  return std::max<int64_t>(1, std::min<int64_t>((budget + kBlockRows - 1) / kBlockRows, n_rec));
}

size_t aqkv_decode_topk_blocks_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads,
                                               int32_t n_kv_heads, int64_t context_len, int64_t budget) {
  if (check_config(cfg) != AQKV_OK) return 0;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || context_len < 0 || budget < 1)
    return 0;
  const int64_t n_slots = static_cast<int64_t>(batch) * n_kv_heads;
  const int64_t n_rec = (context_len + kBlockRows - 1) / kBlockRows;
  const int64_t nb = block_budget(std::min<int64_t>(budget, kMaxBudget), n_rec);
  return block_topk_layout(cfg, n_slots, n_q_heads / n_kv_heads, context_len, n_rec, nb).total;
}

aqkv_status aqkv_decode_attention_topk_blocks(const aqkv_config *cfg, const aqkv_layer *layer,
                                              const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                              int32_t n_kv_heads, int64_t context_len, const float *q,
                                              const float *q_rot, const float *q_sketch, int64_t budget,
                                              float softmax_scale, int32_t *selected, float *out, void *workspace,
                                              size_t workspace_bytes, void *stream) {
  aqkv_status st = check_config(cfg);
  if (st != AQKV_OK) return st;
  if (!layer) return AQKV_ERR_NULL;
  if ((st = check_cache_shape(cache)) != AQKV_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || context_len < 0 || budget < 1) return AQKV_ERR_SHAPE;
  if (n_q_heads % n_kv_heads) return AQKV_ERR_SHAPE;
  const int g = n_q_heads / n_kv_heads;
  if (g > kMaxQPerKv) return AQKV_ERR_UNSUPPORTED;
  if (budget > kMaxBudget) return AQKV_ERR_UNSUPPORTED;
  if (context_len > kMaxTopkContext) return AQKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(batch) * n_kv_heads != cache->n_slots) return AQKV_ERR_SHAPE;
  if (context_len > cache->capacity) return AQKV_ERR_CAPACITY;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return AQKV_ERR_SHAPE;
  const int d = cfg->head_dim, w = cfg->mse_bits, m = cfg->sketch_dim;
  const bool sf = cfg->side_f16 != 0;
  // both passes run on the matrix-core decoder
  if (!decode_mfma_supported(d, w, 1, m, cfg->value_bits, sf) || !decode_mfma_supported(d, w, g, m, cfg->value_bits, sf))
    return AQKV_ERR_UNSUPPORTED;
  if (batch == 0) return AQKV_OK;
  if (!out || !q || !q_sketch || !layer->sketch) return AQKV_ERR_NULL;
  if (w > 0 && (!q_rot || !layer->centroids || !layer->rotation)) return AQKV_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(q_sketch, 16) || (q_rot && !aligned(q_rot, 16)) ||
      (selected && !aligned(selected, 4)))
    return AQKV_ERR_ALIGN;
  const int64_t n_rec = (context_len + kBlockRows - 1) / kBlockRows;
  const int64_t nb = block_budget(budget, n_rec);
  const BlockTopkLayout TL = block_topk_layout(cfg, cache->n_slots, g, context_len, n_rec, nb);
  if (!workspace || workspace_bytes < TL.total) return AQKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AQKV_ERR_ALIGN;
  char *ws = static_cast<char *>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (context_len == 0) {   // nothing cached: a combine over no parts writes out = 0
    DecodeJob zj{};
    zj.d = d;
    zj.g = g;
    zj.n_slots = cache->n_slots;
    zj.part_stride = 0;
    zj.part_acc = reinterpret_cast<float *>(ws + TL.list_ws);
    zj.part_ml = reinterpret_cast<float *>(ws + TL.list_ws);
    zj.out = out;
    return hip_status(launch_combine(zj, s));
  }
  if ((st = check_blocks(cache)) != AQKV_OK) return st;

  // 1. the selection query of every KV slot, rotated and sketched
  float *qsel_rot = reinterpret_cast<float *>(ws + TL.qsel_rot);
  float *qsel_sk = reinterpret_cast<float *>(ws + TL.qsel_sk);
  if (launch_selection_query(q, cache->n_slots, d, g, m, layer->rotation, layer->sketch, w > 0 ? qsel_rot : nullptr,
                             qsel_sk, s) != hipSuccess)
    return AQKV_ERR_HIP;
  // 2. every record's largest cosine estimate (the decoder's scoring pass, one query per slot)
  float *rec_max = reinterpret_cast<float *>(ws + TL.rec_max);
  DecodeExtra score_pass{rec_max, n_rec, nullptr, 0, 0};
  st = decode(cfg, layer, cache, batch, n_kv_heads, n_kv_heads, context_len, w > 0 ? qsel_rot : nullptr, qsel_sk,
              softmax_scale, nullptr, reinterpret_cast<float *>(ws + TL.dec_out), ws + TL.dec_ws, TL.dec_ws_bytes,
              stream, nullptr, true, nullptr, &score_pass);
  if (st != AQKV_OK) return st;
  // 3. the nb records with the largest maxima, in increasing order
  int32_t *sel = selected ? selected : reinterpret_cast<int32_t *>(ws + TL.sel);
  if (launch_select_records(rec_max, cache->n_slots, n_rec, static_cast<int>(nb), sel, s) != hipSuccess)
    return AQKV_ERR_HIP;
  // 4. decode over the chosen records (and the split combine)
  DecodeExtra list_pass{nullptr, 0, sel, nb, context_len};
  return decode(cfg, layer, cache, batch, n_q_heads, n_kv_heads, nb * kBlockRows, q_rot, q_sketch, softmax_scale,
                nullptr, out, ws + TL.list_ws, TL.list_ws_bytes, stream, nullptr, false, nullptr, &list_pass);
}

size_t aqkv_decode_static_scratch_bytes(void) { return kStaticScratchBytes; }

aqkv_status aqkv_decode_attention_noalloc(const aqkv_config *cfg, const aqkv_layer *layer, const aqkv_cache *cache,
                                          int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t context_len,
                                          const float *q_rot, const float *q_sketch, float softmax_scale,
                                          float *scores, float *out, void *stream) {
  return decode(cfg, layer, cache, batch, n_q_heads, n_kv_heads, context_len, q_rot, q_sketch, softmax_scale,
                scores, out, nullptr, 0, stream, nullptr, false, device_scratch);
}

aqkv_status aqkv_decode_attention_window(const aqkv_config *cfg, const aqkv_layer *layer,
                                         const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t context_len, const float *q,
                                         const float *q_rot, const float *q_sketch, const aqkv_kv_view *k_window,
                                         const aqkv_kv_view *v_window, float softmax_scale, float *scores,
                                         float *out, void *workspace, size_t workspace_bytes, void *stream) {
  const WindowArgs win{q, k_window, v_window};
  return decode(cfg, layer, cache, batch, n_q_heads, n_kv_heads, context_len, q_rot, q_sketch, softmax_scale,
                scores, out, workspace, workspace_bytes, stream, &win);
}

}  // extern "C"
