"""Shared helpers for the GPU parity tests (HIP path through the C ABI vs the oracle).

Inputs come from kv_cache_compression_quantize_amd.inputs; the layer
parameters (rotation, sketch, codebook) handed to BOTH sides are built by the
oracle from those seeded Gaussians, so every comparison is on identical inputs.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

from kv_cache_compression_quantize_amd import aqkv, inputs
from oracle import attention as oatt
from oracle import codebook as ocb
from oracle import keys as okeys
from oracle import layout as olay
from oracle import rotation as orot
from oracle import values as ovals

SCORE_RTOL = 1e-3      # |s - s_ref| <= 1e-3 * max(|s_ref|, RMS_t s_ref)
OUT_ATOL = 2e-3        # attention output, absolute
WINDOW = 1e-5          # decision-boundary window for codes and signs


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


@dataclass
class HostLayer:
    d: int
    w: int
    m: int
    rotation: np.ndarray   # fp32 [d, d]
    sketch: np.ndarray     # fp32 [m, d]
    centroids: np.ndarray  # fp32
    boundaries: np.ndarray # fp32


def host_layer(d: int, w: int, m: int, layer: int = 0, rotation: str = "qr") -> HostLayer:
    g, s = inputs.layer_gaussians(layer, d, m)
    pi = orot.rotation_fp32(g) if rotation == "qr" else orot.randomized_hadamard_fp32(g)
    if w > 0:
        c, t = ocb.codebook_fp32(d, w)
    else:
        c, t = np.zeros(1, np.float32), np.zeros(1, np.float32)
    return HostLayer(d, w, m, pi, s.astype(np.float32), c, t)


def device_layer(hl: HostLayer) -> aqkv.Layer:
    torch, dev = torch_dev()
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    return aqkv.Layer(rotation=f(hl.rotation), sketch=f(hl.sketch), centroids=f(hl.centroids),
                      boundaries=f(hl.boundaries))


def to_device_kv(x: np.ndarray, dtype: str):
    """[B, H, T, d] float32 -> device tensor (bf16 exact when dtype == 'bf16')."""
    torch, dev = torch_dev()
    if dtype == "bf16":
        bits = inputs.to_bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def cfg_of(hl: HostLayer, vb: int = 2, side_f16: bool = False):
    return aqkv.config(hl.d, hl.w, hl.m, vb, 32, side_f16)


def read_planes(cache: aqkv.Cache, slot: int, t0: int, t1: int) -> dict:
    """Host copies of rows [t0, t1) of one slot, field by field."""
    r0, r1 = slot * cache.capacity + t0, slot * cache.capacity + t1
    g = lambda name: None if cache.field(name) is None else cache.rows(name, r0, r1 - r0).cpu().numpy()
    # value codes live in 32-token blocks: whole blocks covering [t0, t1) (only when t0 % 32 == 0)
    b1 = slot * cache.capacity + (t1 + 31) // 32 * 32
    vcodes = cache.rows("val_codes", r0, b1 - r0).cpu().numpy() if t0 % 32 == 0 else None
    vscale, vmin = cache.value_side(r0, r1 - r0)
    return dict(codes=g("key_codes"), signs=g("key_signs"), norm=g("key_norm"), rnorm=g("key_rnorm"),
                vcodes=vcodes, vscale=vscale.cpu().numpy(), vmin=vmin.cpu().numpy())


def oracle_rows(hl: HostLayer, k: np.ndarray, v: np.ndarray, vb: int = 2, side_f16: bool = False):
    """Oracle quantisation of one slot: (QuantizedKeys, packed key rows, value tuple, packed
    value codes); norms, scales and minima as the cache stores them (fp32, or halves)."""
    qk = okeys.quantize_keys(k, hl.rotation, hl.sketch, hl.centroids, hl.boundaries, hl.w)
    kr = qk.packed(hl.w, side_f16)
    vc, vs, vm = ovals.quantize_values(v, vb)
    vt = (vc, olay.stored_side(vs, side_f16), olay.stored_side(vm, side_f16))
    return qk, kr, vt, olay.pack_value_codes(vc, vb)


def half_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of the IEEE half grid at |x| (finite halves)."""
    a = np.abs(np.asarray(x, dtype=np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))      # subnormals share the smallest normal's spacing
    return 2.0 ** (e - 10)


@dataclass
class KeyParity:
    n: int
    idx_mismatch_outside: int
    idx_in_window: int
    idx_mismatch_in_window: int
    sign_mismatch_outside: int
    sign_in_window: int
    cascaded_keys: int


def compare_keys(hl: HostLayer, k: np.ndarray, qk, gpu: dict) -> KeyParity:
    """Bit-level comparison of one slot's key rows.  Codes: exact outside the
    boundary window.  Signs: exact outside the window on keys whose indices all
    match; keys with a flipped index (inside the window) are checked against
    the oracle's signs recomputed from the GPU's indices."""
    n = k.shape[0]
    d, w, m = hl.d, hl.w, hl.m
    res = KeyParity(n, 0, 0, 0, 0, 0, 0)
    bits_gpu = olay.unpack_bits(gpu["signs"], m)
    swin = okeys.sign_window(qk.z, qk.rnorm, WINDOW)
    res.sign_in_window = int(swin.sum())
    if w > 0:
        idx_gpu = olay.unpack_code_planes(gpu["codes"], d, w)
        win = okeys.index_window(qk.y, hl.boundaries, WINDOW)
        diff = idx_gpu != qk.idx
        res.idx_in_window = int(win.sum())
        res.idx_mismatch_in_window = int((diff & win).sum())
        res.idx_mismatch_outside = int((diff & ~win).sum())
        clean = ~diff.any(axis=1)
        res.cascaded_keys = int((~clean).sum())
        sd = (bits_gpu != qk.bits) & ~swin
        res.sign_mismatch_outside = int(sd[clean].sum())
        if (~clean).any():
            # recompute the oracle's residual sketch from the GPU's indices
            kk = k[~clean].astype(np.float64)
            nrm = np.linalg.norm(kk, axis=1)
            xt = nrm[:, None] * (hl.centroids.astype(np.float64)[idx_gpu[~clean]] @ hl.rotation.astype(np.float64))
            r = kk - xt
            z = r @ hl.sketch.astype(np.float64).T
            g2 = np.linalg.norm(r, axis=1)
            ref = z >= 0
            win2 = np.abs(z) < WINDOW * g2[:, None]
            res.sign_mismatch_outside += int(((bits_gpu[~clean] != ref) & ~win2).sum())
    else:
        res.sign_mismatch_outside = int(((bits_gpu != qk.bits) & ~swin).sum())
    return res


def score_err(s_gpu: np.ndarray, s_ref: np.ndarray) -> float:
    """max over entries of |s - s_ref| / max(|s_ref|, RMS over tokens of s_ref) (per query head)."""
    rms = np.sqrt(np.mean(s_ref ** 2, axis=-1, keepdims=True))
    den = np.maximum(np.abs(s_ref), rms)
    return float(np.max(np.abs(s_gpu - s_ref) / den))
