"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no norms, rotations, quantisers or scores).  Both the GPU
tests and the CPU oracle take their inputs from here, so the two sides see the
same numbers without sharing any code that computes the method.

Workloads follow the shapes of the decode workloads the TurboQuant article
(kwkr.cn, "TurboQuant: near-optimal KV cache quantization", header and §七)
and the A-QJL article (zingnex.cn, "A-QJL", section "实际部署与使用") describe:
head_dim 128/256, long contexts, GQA, bf16 K/V.  The pages' real
workloads (LongBench, qasper, model activations) are not available; seeded
Gaussian tensors with the stated structure stand in for them.

Seeding
-------
* Random Gaussians the method itself draws (the matrix that is orthogonalised
  into the rotation, and the QJL sketch S) come from
  ``numpy.random.PCG64(42 + 7 * layer)``: first the d*d matrix, then the
  m*d sketch, from one stream (TurboQuant article §六, per-layer seed rule).
* K/V elements come from a counter-based generator, so any slice of a large
  cache can be drawn on the host (numpy) or in bulk on the GPU (torch) with
  identical bits: element i = t * d + j of one (workload, layer, batch,
  kv-head, tensor) slot takes u = the top 16 bits of fmix32(key + i * 0x9E3779B9)
  (fmix32: the 32-bit finaliser of MurmurHash3; key: 32 bits from a
  ``SeedSequence`` of the slot's identifiers) and the value
  Phi^-1((u + 1/2) / 2^16) from a 2^16-entry fp32 table of standard normal
  quantiles (|x| <= 4.33), times the recipe's per-channel scale in fp32, then
  rounded to bf16 (RNE) for bf16 workloads.  The same integer code runs on
  numpy and torch arrays; the table and the scales are the same fp32 numbers
  on both sides.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

_TENSOR_IDS = {"k": 1, "v": 2, "q": 3, "outlier": 4, "kscale": 5, "vscale": 6}


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload: cache shape, codec and value recipe."""

    name: str
    wid: int                 # numeric id mixed into every seed
    batch: int
    n_q_heads: int
    n_kv_heads: int
    context: int
    head_dim: int
    mse_bits: int            # Lloyd-Max bits per rotated coordinate (0 = pure QJL)
    sketch_dims: Tuple[int, ...]   # per layer; length == layers
    value_bits: int = 2
    value_group: int = 32
    layers: int = 1
    dtype: str = "bf16"      # K/V element type handed to the kernels
    recipe: str = "normal"   # normal | outliers | chscale | layer_sigma
    scores: bool = False     # also return the per-token score estimates
    notes: str = ""

    def sketch_dim(self, layer: int) -> int:
        return self.sketch_dims[layer]

    @property
    def n_slots(self) -> int:
        return self.batch * self.n_kv_heads


def _aqjl_dims(layers: int = 32) -> Tuple[int, ...]:
    # A-QJL article, "实际部署与使用": boundaries 8,16,24 and k = 512,384,256,192
    ks = (512, 384, 256, 192)
    bounds = (8, 16, 24)
    out = []
    for layer in range(layers):
        g = sum(layer >= b for b in bounds)
        out.append(ks[g])
    return tuple(out)


WORKLOADS = {
    "single_head_d128_t1k": Workload(
        "single_head_d128_t1k", 1, batch=1, n_q_heads=1, n_kv_heads=1, context=1024,
        head_dim=128, mse_bits=2, sketch_dims=(128,), dtype="fp32", recipe="normal",
        scores=True, notes="fp32 K/V/q ~N(0,1); 2-bit Lloyd-Max + 1-bit QJL keys"),
    "llama2_7b_layer_mha32_t32k": Workload(
        "llama2_7b_layer_mha32_t32k", 2, batch=1, n_q_heads=32, n_kv_heads=32,
        context=32768, head_dim=128, mse_bits=2, sketch_dims=(128,), recipe="outliers",
        notes="bf16 K/V ~N(0,1), 4 outlier channels per head scaled x10"),
    "llama3_8b_layer_gqa32x8_b8_t128k": Workload(
        "llama3_8b_layer_gqa32x8_b8_t128k", 3, batch=8, n_q_heads=32, n_kv_heads=8,
        context=131072, head_dim=128, mse_bits=2, sketch_dims=(128,), recipe="chscale",
        notes="bf16 K/V ~N(0,1) x per-(kv head, channel) LogNormal(0,0.5) scale"),
    "d256_gqa32x16_b4_t64k": Workload(
        "d256_gqa32x16_b4_t64k", 4, batch=4, n_q_heads=32, n_kv_heads=16, context=65536,
        head_dim=256, mse_bits=3, sketch_dims=(256,), recipe="normal",
        notes="bf16 K/V ~N(0,1); 3-bit Lloyd-Max + 1-bit QJL keys"),
    "aqjl_32layer_gqa32x8_b16_t32k": Workload(
        "aqjl_32layer_gqa32x8_b16_t32k", 5, batch=16, n_q_heads=32, n_kv_heads=8,
        context=32768, head_dim=128, mse_bits=0, sketch_dims=_aqjl_dims(32), layers=32,
        recipe="layer_sigma",
        notes="pure 1-bit QJL keys, k per layer group; keys ~N(0, sigma_l^2)"),
}


# --------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even from fp32, plain bit handling)
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# random matrices drawn by the method (per layer)
# --------------------------------------------------------------------------

def layer_seed(layer: int) -> int:
    """TurboQuant article §六: each layer's matrices come from seed 42 + 7*layer."""
    return 42 + 7 * layer


def layer_gaussians(layer: int, head_dim: int, sketch_dim: int) -> Tuple[np.ndarray, np.ndarray]:
    """(G, S): G is d x d N(0,1) (to be orthogonalised into the rotation),
    S is m x d N(0,1) (the QJL sketch), float64, one PCG64 stream per layer."""
    rng = np.random.Generator(np.random.PCG64(layer_seed(layer)))
    g = rng.standard_normal((head_dim, head_dim))
    s = rng.standard_normal((sketch_dim, head_dim))
    return g, s


# --------------------------------------------------------------------------
# K / V / q tensors
# --------------------------------------------------------------------------

def _rng(w: Workload, layer: int, b: int, h: int, tensor: str, block: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([w.wid, layer, b, h, _TENSOR_IDS[tensor], block])
    return np.random.Generator(np.random.PCG64(ss))


def slot_key(w: Workload, layer: int, b: int, h: int, tensor: str) -> int:
    """32-bit key of one K/V slot for the counter-based generator."""
    ss = np.random.SeedSequence([w.wid, layer, b, h, _TENSOR_IDS[tensor]])
    return int(ss.generate_state(1, np.uint32)[0])


_M32 = 0xFFFFFFFF
_WEYL = 0x9E3779B9


def _mul32(h, c: int):
    """(h * c) mod 2^32 for int64 arrays h < 2^32 (numpy or torch): the constant is
    split in 16-bit halves so no product leaves int64."""
    return (h * (c & 0xFFFF) + (((h * (c >> 16)) & 0xFFFF) << 16)) & _M32


def _fmix32(h):
    """MurmurHash3's 32-bit finaliser on int64 arrays holding 32-bit values."""
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    return h ^ (h >> 16)


def counter_u16(key, index):
    """Top 16 bits of fmix32(key + index * 0x9E3779B9 mod 2^32); key and index are
    int64 arrays (or ints) of the same backend, index < 2^32."""
    return _fmix32((key + index * _WEYL) & _M32) >> 16


_QTABLE = None


def normal_table() -> np.ndarray:
    """fp32 standard normal quantiles Phi^-1((u + 1/2) / 2^16), u = 0 .. 2^16 - 1."""
    global _QTABLE
    if _QTABLE is None:
        from scipy.special import ndtri
        _QTABLE = ndtri((np.arange(1 << 16, dtype=np.float64) + 0.5) / (1 << 16)).astype(np.float32)
    return _QTABLE


def _channel_scale(w: Workload, layer: int, h: int, tensor: str) -> Optional[np.ndarray]:
    d = w.head_dim
    if w.recipe == "outliers":
        rng = _rng(w, layer, 0, h, "outlier")
        ch = rng.choice(d, size=4, replace=False)
        sc = np.ones(d, dtype=np.float32)
        sc[ch] = 10.0
        return sc
    if w.recipe == "chscale":
        rng = _rng(w, layer, 0, h, "kscale" if tensor == "k" else "vscale")
        return rng.lognormal(0.0, 0.5, size=d).astype(np.float32)
    if w.recipe == "layer_sigma" and tensor == "k":
        sigma = 2.0 - 1.5 * layer / max(w.layers - 1, 1)
        return np.full(d, sigma, dtype=np.float32)
    return None


def kv_slot(w: Workload, layer: int, b: int, h: int, tensor: str,
            t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """Tokens [t0, t1) of one (batch, kv-head) slot of K or V as float32 [T, d].

    For bf16 workloads the values are already rounded to bf16 (so they are
    exactly what the device sees); use ``to_bf16_bits`` to get the bits."""
    assert tensor in ("k", "v")
    t1 = w.context if t1 is None else t1
    d = w.head_dim
    assert w.context * d <= (1 << 32)
    idx = np.arange(t0 * d, t1 * d, dtype=np.int64)
    u = counter_u16(np.int64(slot_key(w, layer, b, h, tensor)), idx)
    out = normal_table()[u].reshape(t1 - t0, d)
    sc = _channel_scale(w, layer, h, tensor)
    if sc is not None:
        out = out * sc
    if w.dtype == "bf16":
        out = bf16_bits_to_f32(to_bf16_bits(out))
    return out


def kv_device(w: Workload, layer: int, tensor: str, device="cuda", slots_per_pass: int = 16):
    """The whole K or V tensor [B, Hkv, T, d] of a workload layer drawn on the GPU
    (bf16 or fp32 torch tensor): the same numbers as kv_slot gives slot by slot."""
    import torch
    d, T = w.head_dim, w.context
    assert T * d <= (1 << 32)
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.empty((w.batch, w.n_kv_heads, T, d), dtype=tdtype, device=device)
    table = torch.from_numpy(normal_table()).to(device)
    idx = torch.arange(T * d, dtype=torch.int64, device=device)
    flat = out.view(w.n_slots, T, d)
    for s0 in range(0, w.n_slots, slots_per_pass):
        s1 = min(w.n_slots, s0 + slots_per_pass)
        keys, scales = [], []
        for s in range(s0, s1):
            b, h = divmod(s, w.n_kv_heads)
            keys.append(slot_key(w, layer, b, h, tensor))
            scales.append(_channel_scale(w, layer, h, tensor))
        key_t = torch.tensor(keys, dtype=torch.int64, device=device)[:, None]
        x = table[counter_u16(key_t, idx[None, :])].view(s1 - s0, T, d)
        if scales[0] is not None:   # a recipe scales every slot of a tensor or none
            x = x * torch.from_numpy(np.stack(scales)).to(device)[:, None, :]
        flat[s0:s1] = x.to(tdtype)
        del x
    return out


def queries(w: Workload, layer: int) -> np.ndarray:
    """Decode queries [B, Hq, d] float32 ~N(0,1)."""
    rng = _rng(w, layer, 0, 0, "q")
    return rng.standard_normal((w.batch, w.n_q_heads, w.head_dim), dtype=np.float32)


def kv_tensor(w: Workload, layer: int, tensor: str, batches=None, heads=None,
              t0: int = 0, t1: Optional[int] = None) -> np.ndarray:
    """[len(batches), len(heads), T, d] float32 built slot by slot."""
    batches = range(w.batch) if batches is None else batches
    heads = range(w.n_kv_heads) if heads is None else heads
    t1 = w.context if t1 is None else t1
    out = np.empty((len(batches), len(heads), t1 - t0, w.head_dim), dtype=np.float32)
    for i, b in enumerate(batches):
        for j, h in enumerate(heads):
            out[i, j] = kv_slot(w, layer, b, h, tensor, t0, t1)
    return out


def small_workload(base: Workload, **over) -> Workload:
    """A reduced copy of a workload (same recipe and codec) for parity tests
    the oracle finishes in seconds."""
    fields = dict(base.__dict__)
    fields.update(over)
    if "layers" in over and "sketch_dims" not in over:
        fields["sketch_dims"] = base.sketch_dims[: over["layers"]]
    return Workload(**fields)
