"""Thin ctypes binding of libaqkv.so (include/aqkv.h).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  torch tensors are used for device memory and the current stream;
host-side numpy arrays for the host-only builders.  A missing library is an
error (``AqkvError``), never a fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("AQKV_LIB", os.path.join(_HERE, "libaqkv.so"))

STATUS = {
    0: "AQKV_OK", -1: "AQKV_ERR_NULL", -2: "AQKV_ERR_SHAPE", -3: "AQKV_ERR_ALIGN",
    -4: "AQKV_ERR_CAPACITY", -5: "AQKV_ERR_WORKSPACE", -6: "AQKV_ERR_DTYPE",
    -7: "AQKV_ERR_HIP", -8: "AQKV_ERR_UNSUPPORTED", -9: "AQKV_ERR_SCRATCH",
}
FP32, BF16 = 0, 1


class AqkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Config(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("mse_bits", C.c_int32), ("sketch_dim", C.c_int32),
                ("value_bits", C.c_int32), ("value_group", C.c_int32), ("side_f16", C.c_int32)]


class LayerParams(C.Structure):
    _fields_ = [("rotation", C.c_void_p), ("sketch", C.c_void_p), ("centroids", C.c_void_p),
                ("boundaries", C.c_void_p)]


class CacheDesc(C.Structure):
    _fields_ = [("blocks", C.c_void_p), ("n_slots", C.c_int64), ("capacity", C.c_int64)]


class KvView(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int), ("batch", C.c_int64), ("heads", C.c_int64),
                ("tokens", C.c_int64), ("batch_stride", C.c_int64), ("head_stride", C.c_int64),
                ("token_stride", C.c_int64)]


FIELDS = ("key_codes", "key_signs", "key_norm", "key_rnorm", "val_codes", "val_side")
FLOAT_FIELDS = ("key_norm", "key_rnorm", "val_side")


def side_index(groups: int) -> np.ndarray:
    """[32 tokens, groups, 2] -> element index (fp32 or half) inside a record's val_side field
    (j = 0 scale, 1 min; include/aqkv.h): ((g * 16 + 4 a + b) * 2 + h) * 2 + j for
    token t = 8 a + 4 h + b."""
    t = np.arange(32)[:, None, None]
    g = np.arange(groups)[None, :, None]
    j = np.arange(2)[None, None, :]
    return ((g * 16 + 4 * (t >> 3) + (t & 3)) * 2 + ((t >> 2) & 1)) * 2 + j


class Fields(C.Structure):
    _fields_ = [(name, C.c_int64) for name in FIELDS]


class LayoutDesc(C.Structure):
    _fields_ = [("row_bytes", Fields), ("offset", Fields), ("block_bytes", C.c_int64)]


_P = C.POINTER
_SIGS = {
    "aqkv_status_string": (C.c_char_p, [C.c_int]),
    "aqkv_cache_layout": (C.c_int, [_P(Config), _P(LayoutDesc)]),
    "aqkv_build_codebook": (C.c_int, [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "aqkv_build_rotation": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p]),
    "aqkv_quantize_keys_workspace_bytes": (C.c_size_t, [_P(Config)]),
    "aqkv_build_hadamard_rotation": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p]),
    "aqkv_decode_workspace_bytes": (C.c_size_t, [_P(Config), C.c_int32, C.c_int32, C.c_int32, C.c_int64]),
    "aqkv_quantize_keys": (C.c_int, [_P(Config), _P(LayerParams), _P(KvView), C.c_int64, _P(CacheDesc),
                                     C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_prepare_key_operands": (C.c_int, [_P(Config), _P(LayerParams), C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_quantize_keys_prepared": (C.c_int, [_P(Config), _P(LayerParams), _P(KvView), C.c_int64, _P(CacheDesc),
                                              C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_decode_topk_workspace_bytes": (C.c_size_t, [_P(Config), C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                                     C.c_int64]),
    "aqkv_decode_attention_topk": (C.c_int, [_P(Config), _P(LayerParams), _P(CacheDesc), C.c_int32, C.c_int32,
                                             C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                             C.c_float, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                             C.c_void_p]),
    "aqkv_quantize_values": (C.c_int, [_P(Config), _P(KvView), C.c_int64, _P(CacheDesc), C.c_void_p]),
    "aqkv_prepare_query": (C.c_int, [_P(Config), _P(LayerParams), C.c_void_p, C.c_int, C.c_int64,
                                     C.c_void_p, C.c_void_p, C.c_void_p]),
    "aqkv_decode_attention": (C.c_int, [_P(Config), _P(LayerParams), _P(CacheDesc), C.c_int32, C.c_int32,
                                        C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_float,
                                        C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_decode_attention_window": (C.c_int, [_P(Config), _P(LayerParams), _P(CacheDesc), C.c_int32, C.c_int32,
                                               C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                               _P(KvView), _P(KvView), C.c_float, C.c_void_p, C.c_void_p,
                                               C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_decode_topk_blocks_workspace_bytes": (C.c_size_t, [_P(Config), C.c_int32, C.c_int32, C.c_int32,
                                                             C.c_int64, C.c_int64]),
    "aqkv_decode_attention_topk_blocks": (C.c_int, [_P(Config), _P(LayerParams), _P(CacheDesc), C.c_int32,
                                                    C.c_int32, C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                                                    C.c_void_p, C.c_int64, C.c_float, C.c_void_p, C.c_void_p,
                                                    C.c_void_p, C.c_size_t, C.c_void_p]),
    "aqkv_read_stream": (C.c_int, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]),
    "aqkv_decode_static_scratch_bytes": (C.c_size_t, []),
    "aqkv_decode_attention_noalloc": (C.c_int, [_P(Config), _P(LayerParams), _P(CacheDesc), C.c_int32, C.c_int32,
                                                C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_float,
                                                C.c_void_p, C.c_void_p, C.c_void_p]),
}

_lib_handle = None


def lib():
    """The loaded libaqkv.so (raises AqkvError-compatible RuntimeError if it is not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libaqkv.so not built at {LIB_PATH}; run "
                               "`python -m kv_cache_compression_quantize_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(st: int, where: str):
    if st != 0:
        raise AqkvError(st, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------- host only

def config(head_dim: int, mse_bits: int, sketch_dim: int, value_bits: int = 2, value_group: int = 32,
           side_f16: bool = False) -> Config:
    return Config(head_dim, mse_bits, sketch_dim, value_bits, value_group, int(bool(side_f16)))


def cache_layout(cfg: Config) -> dict:
    """{"row": bytes per token of each field, "offset": byte offset of each field
    in a 32-token block record, "block_bytes": bytes of one record}."""
    lo = LayoutDesc()
    _check(lib().aqkv_cache_layout(C.byref(cfg), C.byref(lo)), "aqkv_cache_layout")
    return {"row": {n: getattr(lo.row_bytes, n) for n in FIELDS},
            "offset": {n: getattr(lo.offset, n) for n in FIELDS},
            "block_bytes": lo.block_bytes}


def build_codebook(head_dim: int, bits: int):
    """(centroids, boundaries) float32 numpy arrays, computed by the library on the host."""
    c = np.zeros(1 << bits, dtype=np.float32)
    t = np.zeros(max((1 << bits) - 1, 1), dtype=np.float32)
    _check(lib().aqkv_build_codebook(head_dim, bits, c.ctypes.data, t.ctypes.data), "aqkv_build_codebook")
    return c, t[: (1 << bits) - 1]


def build_rotation(gaussian: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(gaussian, dtype=np.float64)
    d = g.shape[0]
    assert g.shape == (d, d)
    out = np.zeros((d, d), dtype=np.float32)
    _check(lib().aqkv_build_rotation(d, g.ctypes.data, out.ctypes.data), "aqkv_build_rotation")
    return out


def build_hadamard_rotation(gaussian: np.ndarray) -> np.ndarray:
    """Randomised Hadamard rotation H diag(sign(gaussian[0])) / sqrt(d), computed by the library."""
    g = np.ascontiguousarray(gaussian, dtype=np.float64)
    d = g.shape[-1]
    out = np.zeros((d, d), dtype=np.float32)
    _check(lib().aqkv_build_hadamard_rotation(d, g.ctypes.data, out.ctypes.data), "aqkv_build_hadamard_rotation")
    return out


def quantize_keys_workspace_bytes(cfg: Config) -> int:
    return int(lib().aqkv_quantize_keys_workspace_bytes(C.byref(cfg)))


def decode_workspace_bytes(cfg: Config, batch: int, n_q_heads: int, n_kv_heads: int, context_len: int) -> int:
    return int(lib().aqkv_decode_workspace_bytes(C.byref(cfg), batch, n_q_heads, n_kv_heads, context_len))


# ------------------------------------------------------------ device objects

@dataclass
class Layer:
    """Device copies of one layer's parameters (fp32 torch tensors)."""
    rotation: object = None
    sketch: object = None
    centroids: object = None
    boundaries: object = None

    def desc(self) -> LayerParams:
        return LayerParams(_ptr(self.rotation), _ptr(self.sketch), _ptr(self.centroids), _ptr(self.boundaries))


@dataclass
class Cache:
    """The cache buffer: n_slots * capacity / 32 block records of block_bytes
    bytes (a uint8 torch tensor [records, block_bytes]); field views and row
    copies for tests and tools."""
    cfg: Config
    n_slots: int
    capacity: int
    blocks: object
    layout: dict

    @staticmethod
    def allocate(cfg: Config, n_slots: int, capacity: int, device="cuda") -> "Cache":
        """Records for n_slots x capacity tokens (capacity rounded up to a multiple of 32)."""
        import torch
        lo = cache_layout(cfg)
        capacity = (capacity + 31) // 32 * 32
        blocks = torch.empty((n_slots * capacity // 32, lo["block_bytes"]), dtype=torch.uint8, device=device)
        return Cache(cfg, n_slots, capacity, blocks, lo)

    def field(self, name: str):
        """Strided view [records, 32, row] of one field (uint8, or float32 / float16 for the
        norms, scales and minima); None when the configuration has no such field."""
        import torch
        rb, off, bb = self.layout["row"][name], self.layout["offset"][name], self.layout["block_bytes"]
        if rb == 0:
            return None
        n_rec = self.blocks.shape[0]
        flat = self.blocks.view(-1)
        # as_strided takes an offset into the whole storage: the buffer may itself be a view
        if name in FLOAT_FIELDS:
            e = 2 if self.cfg.side_f16 else 4
            f = flat.view(dtype=torch.float16 if e == 2 else torch.float32)
            return f.as_strided((n_rec, 32, rb // e), (bb // e, rb // e, 1), f.storage_offset() + off // e)
        return flat.as_strided((n_rec, 32, rb), (bb, rb, 1), flat.storage_offset() + off)

    def rows(self, name: str, row0: int, n: int):
        """Copy of cache rows row0 .. row0 + n - 1 (row = slot * capacity + token) of a field:
        [n, row] (uint8, float32 or float16), [n] for the single-number norms."""
        f = self.field(name)
        if f is None:
            return None
        out = f.flatten(0, 1)[row0:row0 + n].clone()
        return out.reshape(-1) if out.shape[-1] == 1 else out

    def set_rows(self, name: str, row0: int, values):
        """Write values [n, row] (or [n] for single-float fields) into cache rows row0 .. row0 + n - 1."""
        f = self.field(name)
        n = values.shape[0]
        r = row0
        while r < row0 + n:
            rec, i = divmod(r, 32)
            k = min(32 - i, row0 + n - r)
            f[rec, i:i + k] = values[r - row0:r - row0 + k].reshape(k, -1)
            r += k

    def value_side(self, row0: int, n: int):
        """(scale, min) of cache rows row0 .. row0 + n - 1, each [n, groups] in the stored
        type (float32, or float16 for half side information), in token order."""
        import torch
        groups = self.cfg.head_dim // self.cfg.value_group
        f = self.field("val_side").flatten(1)                       # [records, 32 * groups * 2]
        idx = torch.from_numpy(side_index(groups).reshape(-1)).to(f.device)
        tok = f[:, idx].reshape(-1, 32, groups, 2).flatten(0, 1)   # rows in token order
        sel = tok[row0:row0 + n]
        return sel[..., 0].clone(), sel[..., 1].clone()

    def set_value_side(self, row0: int, scale, vmin):
        """Write scale / min [n, groups] into cache rows row0 .. row0 + n - 1."""
        import torch
        groups = self.cfg.head_dim // self.cfg.value_group
        f = self.field("val_side").flatten(1)
        idx = torch.from_numpy(side_index(groups)).to(f.device)
        both = torch.stack([scale, vmin], dim=-1).to(f.dtype)
        for i in range(scale.shape[0]):
            rec, t = divmod(row0 + i, 32)
            f[rec, idx[t].reshape(-1)] = both[i].reshape(-1)

    def desc(self) -> CacheDesc:
        return CacheDesc(_ptr(self.blocks), self.n_slots, self.capacity)


def kv_view(t) -> KvView:
    """View of a [B, H, T, d] tensor (any strides with contiguous channels)."""
    assert t.dim() == 4 and t.stride(3) == 1
    B, H, T, _ = t.shape
    return KvView(_ptr(t), _dtype_code(t), B, H, T, t.stride(0), t.stride(1), t.stride(2))


# ---------------------------------------------------------------- compute

def quantize_keys(cfg: Config, layer: Layer, k, cache: Cache, token_offset: int = 0, workspace=None, stream=None):
    v = kv_view(k)
    ws_bytes = quantize_keys_workspace_bytes(cfg)
    if workspace is None and ws_bytes > 0:
        import torch
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    st = lib().aqkv_quantize_keys(C.byref(cfg), C.byref(layer.desc()), C.byref(v), token_offset,
                                  C.byref(cache.desc()), _ptr(workspace),
                                  workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(st, "aqkv_quantize_keys")


def prepare_key_operands(cfg: Config, layer: Layer, workspace=None, device=None, stream=None):
    """The layer's key-quantisation operands into `workspace` (allocated when None); pass it to
    quantize_keys_prepared."""
    ws_bytes = quantize_keys_workspace_bytes(cfg)
    if workspace is None:
        import torch
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=device or "cuda")
    st = lib().aqkv_prepare_key_operands(C.byref(cfg), C.byref(layer.desc()), _ptr(workspace), workspace.numel(),
                                         _stream(stream))
    _check(st, "aqkv_prepare_key_operands")
    return workspace


def quantize_keys_prepared(cfg: Config, layer: Layer, k, cache: Cache, workspace, token_offset: int = 0,
                           stream=None):
    v = kv_view(k)
    st = lib().aqkv_quantize_keys_prepared(C.byref(cfg), C.byref(layer.desc()), C.byref(v), token_offset,
                                           C.byref(cache.desc()), _ptr(workspace), workspace.numel(),
                                           _stream(stream))
    _check(st, "aqkv_quantize_keys_prepared")


def quantize_values(cfg: Config, v, cache: Cache, token_offset: int = 0, stream=None):
    view = kv_view(v)
    _check(lib().aqkv_quantize_values(C.byref(cfg), C.byref(view), token_offset, C.byref(cache.desc()),
                                      _stream(stream)), "aqkv_quantize_values")


def prepare_query(cfg: Config, layer: Layer, q, q_rot=None, q_sketch=None, stream=None):
    """q [..., d] -> (q_rot [..., d] or None when mse_bits == 0, q_sketch [..., m]) fp32."""
    import torch
    assert q.is_contiguous() and q.shape[-1] == cfg.head_dim
    n_q = q.numel() // cfg.head_dim
    lead = tuple(q.shape[:-1])
    if q_sketch is None:
        q_sketch = torch.empty(lead + (cfg.sketch_dim,), dtype=torch.float32, device=q.device)
    if q_rot is None and cfg.mse_bits > 0:
        q_rot = torch.empty(lead + (cfg.head_dim,), dtype=torch.float32, device=q.device)
    _check(lib().aqkv_prepare_query(C.byref(cfg), C.byref(layer.desc()), _ptr(q), _dtype_code(q), n_q,
                                    _ptr(q_rot), _ptr(q_sketch), _stream(stream)), "aqkv_prepare_query")
    return q_rot, q_sketch


def decode_attention(cfg: Config, layer: Layer, cache: Cache, batch: int, n_q_heads: int, n_kv_heads: int,
                     context_len: int, q_rot, q_sketch, softmax_scale: Optional[float] = None,
                     scores=None, out=None, workspace=None, stream=None):
    import torch
    dev = q_sketch.device
    if softmax_scale is None:
        softmax_scale = 1.0 / float(np.sqrt(cfg.head_dim))
    if out is None:
        out = torch.empty((batch, n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    ws_bytes = decode_workspace_bytes(cfg, batch, n_q_heads, n_kv_heads, context_len)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().aqkv_decode_attention(C.byref(cfg), C.byref(layer.desc()), C.byref(cache.desc()), batch,
                                     n_q_heads, n_kv_heads, context_len, _ptr(q_rot), _ptr(q_sketch),
                                     C.c_float(softmax_scale), _ptr(scores), _ptr(out), _ptr(workspace),
                                     workspace.numel(), _stream(stream))
    _check(st, "aqkv_decode_attention")
    return out


def decode_static_scratch_bytes() -> int:
    return int(lib().aqkv_decode_static_scratch_bytes())


def decode_attention_noalloc(cfg: Config, layer: Layer, cache: Cache, batch: int, n_q_heads: int, n_kv_heads: int,
                             context_len: int, q_rot, q_sketch, out, softmax_scale: Optional[float] = None,
                             scores=None, stream=None):
    """decode_attention with the library's static scratch instead of a workspace; `out` must be given
    (nothing is allocated on this path)."""
    if softmax_scale is None:
        softmax_scale = 1.0 / float(np.sqrt(cfg.head_dim))
    st = lib().aqkv_decode_attention_noalloc(C.byref(cfg), C.byref(layer.desc()), C.byref(cache.desc()), batch,
                                             n_q_heads, n_kv_heads, context_len, _ptr(q_rot), _ptr(q_sketch),
                                             C.c_float(softmax_scale), _ptr(scores), _ptr(out), _stream(stream))
    _check(st, "aqkv_decode_attention_noalloc")
    return out


def decode_attention_window(cfg: Config, layer: Layer, cache: Cache, batch: int, n_q_heads: int, n_kv_heads: int,
                            context_len: int, q, q_rot, q_sketch, k_window, v_window,
                            softmax_scale: Optional[float] = None, scores=None, out=None, workspace=None,
                            stream=None):
    """Decode over cache rows [0, context_len) plus the recent-token window k_window / v_window
    ([batch, n_kv_heads, n_window, d] tensors, any token order); q is the unrotated fp32 query."""
    import torch
    dev = q_sketch.device
    if softmax_scale is None:
        softmax_scale = 1.0 / float(np.sqrt(cfg.head_dim))
    if out is None:
        out = torch.empty((batch, n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    ws_bytes = decode_workspace_bytes(cfg, batch, n_q_heads, n_kv_heads, context_len)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    kv, vv = kv_view(k_window), kv_view(v_window)
    st = lib().aqkv_decode_attention_window(C.byref(cfg), C.byref(layer.desc()), C.byref(cache.desc()), batch,
                                            n_q_heads, n_kv_heads, context_len, _ptr(q), _ptr(q_rot),
                                            _ptr(q_sketch), C.byref(kv), C.byref(vv), C.c_float(softmax_scale),
                                            _ptr(scores), _ptr(out), _ptr(workspace), workspace.numel(),
                                            _stream(stream))
    _check(st, "aqkv_decode_attention_window")
    return out


def decode_topk_workspace_bytes(cfg: Config, batch: int, n_q_heads: int, n_kv_heads: int, context_len: int,
                                budget: int) -> int:
    return int(lib().aqkv_decode_topk_workspace_bytes(C.byref(cfg), batch, n_q_heads, n_kv_heads, context_len,
                                                      budget))


def decode_attention_topk(cfg: Config, layer: Layer, cache: Cache, batch: int, n_q_heads: int, n_kv_heads: int,
                          context_len: int, q, q_rot, q_sketch, budget: int, softmax_scale: Optional[float] = None,
                          selected=None, out=None, workspace=None, stream=None):
    """Decode over the `budget` cached tokens per KV slot with the largest group cosine (q: unrotated fp32)."""
    import torch
    dev = q_sketch.device
    if softmax_scale is None:
        softmax_scale = 1.0 / float(np.sqrt(cfg.head_dim))
    if out is None:
        out = torch.empty((batch, n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    if workspace is None:
        ws_bytes = decode_topk_workspace_bytes(cfg, batch, n_q_heads, n_kv_heads, context_len, budget)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().aqkv_decode_attention_topk(C.byref(cfg), C.byref(layer.desc()), C.byref(cache.desc()), batch,
                                          n_q_heads, n_kv_heads, context_len, _ptr(q), _ptr(q_rot), _ptr(q_sketch),
                                          budget, C.c_float(softmax_scale), _ptr(selected), _ptr(out),
                                          _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "aqkv_decode_attention_topk")
    return out


def decode_topk_blocks_workspace_bytes(cfg: Config, batch: int, n_q_heads: int, n_kv_heads: int,
                                       context_len: int, budget: int) -> int:
    return int(lib().aqkv_decode_topk_blocks_workspace_bytes(C.byref(cfg), batch, n_q_heads, n_kv_heads,
                                                             context_len, budget))


def decode_attention_topk_blocks(cfg: Config, layer: Layer, cache: Cache, batch: int, n_q_heads: int,
                                 n_kv_heads: int, context_len: int, q, q_rot, q_sketch, budget: int,
                                 softmax_scale: Optional[float] = None, selected=None, out=None, workspace=None,
                                 stream=None):
    """Decode over the ceil(budget / 32) block records per KV slot with the largest group cosine of any
    of their rows (q: unrotated fp32)."""
    import torch
    dev = q_sketch.device
    if softmax_scale is None:
        softmax_scale = 1.0 / float(np.sqrt(cfg.head_dim))
    if out is None:
        out = torch.empty((batch, n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    if workspace is None:
        ws_bytes = decode_topk_blocks_workspace_bytes(cfg, batch, n_q_heads, n_kv_heads, context_len, budget)
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    st = lib().aqkv_decode_attention_topk_blocks(C.byref(cfg), C.byref(layer.desc()), C.byref(cache.desc()), batch,
                                                 n_q_heads, n_kv_heads, context_len, _ptr(q), _ptr(q_rot),
                                                 _ptr(q_sketch), budget, C.c_float(softmax_scale), _ptr(selected),
                                                 _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "aqkv_decode_attention_topk_blocks")
    return out


def read_stream(buf, sink, stream=None):
    """One plain read of a device buffer (the HBM read ceiling probe); sink: a 1-element int32 tensor."""
    _check(lib().aqkv_read_stream(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "aqkv_read_stream")
