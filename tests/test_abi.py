"""The C ABI on the CPU: library loads, exports what the header declares,
validates arguments (status codes, no launch), and its host-only parameter
builders agree with the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv, inputs
from oracle import codebook as ocb
from oracle import rotation as orot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "aqkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aqkv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = aqkv.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = aqkv.lib()
    for code in aqkv.STATUS:
        assert lib.aqkv_status_string(code)
    assert lib.aqkv_status_string(0) == b"ok"


def test_cache_layout_and_bad_configs():
    lo = aqkv.cache_layout(aqkv.config(128, 2, 128))
    rb = lo["row"]
    assert rb == dict(key_codes=32, key_signs=16, key_norm=4, key_rnorm=4, val_codes=32, val_side=32)
    assert sum(rb.values()) == 120 and lo["block_bytes"] == 32 * 120
    # a record holds the six fields one after the other, 32 rows each
    off = 0
    for name in aqkv.FIELDS:
        assert lo["offset"][name] == off
        off += 32 * rb[name]
    assert off == lo["block_bytes"]
    lo = aqkv.cache_layout(aqkv.config(256, 3, 256))
    assert sum(lo["row"].values()) == 96 + 32 + 8 + 64 + 64 == 264
    lo = aqkv.cache_layout(aqkv.config(128, 0, 192))
    rb = lo["row"]
    assert rb["key_codes"] == 0 and rb["key_rnorm"] == 0 and rb["key_signs"] == 24
    assert lo["block_bytes"] % 16 == 0
    for bad in [(96, 2, 128), (128, 4, 128), (128, 2, 100), (128, 2, 2048), (128, -1, 128)]:
        with pytest.raises(aqkv.AqkvError) as e:
            aqkv.cache_layout(aqkv.config(*bad))
        assert e.value.status == -2
    with pytest.raises(aqkv.AqkvError):
        aqkv.cache_layout(aqkv.config(128, 2, 128, value_bits=3))
    assert aqkv.lib().aqkv_cache_layout(None, None) == -1
    bad = aqkv.config(128, 2, 128)
    bad.side_f16 = 2
    with pytest.raises(aqkv.AqkvError) as e:
        aqkv.cache_layout(bad)
    assert e.value.status == -2


def test_half_side_information_layout():
    # d = 256, 3-bit keys (w = 2, m = d), 2-bit values: 196 bytes a token, 1024 / 196 = 5.22x bf16 K + V
    lo = aqkv.cache_layout(aqkv.config(256, 2, 256, side_f16=True))
    rb = lo["row"]
    assert rb == dict(key_codes=64, key_signs=32, key_norm=2, key_rnorm=2, val_codes=64, val_side=32)
    assert sum(rb.values()) == 196 and round(1024 / 196, 2) == 5.22
    assert sum(aqkv.cache_layout(aqkv.config(256, 2, 256))["row"].values()) == 232
    for d, w, m, vb in [(64, 0, 64, 2), (128, 0, 192, 4), (256, 3, 1024, 2), (128, 1, 128, 4)]:
        full = aqkv.cache_layout(aqkv.config(d, w, m, vb))
        half = aqkv.cache_layout(aqkv.config(d, w, m, vb, side_f16=True))
        off = 0
        for name in aqkv.FIELDS:
            assert half["offset"][name] == off
            off += 32 * half["row"][name]
            wide = name in aqkv.FLOAT_FIELDS
            assert half["row"][name] == (full["row"][name] // 2 if wide else full["row"][name])
        assert off == half["block_bytes"] and off % 16 == 0


def test_workspace_sizes():
    cfg = aqkv.config(128, 2, 128)
    # ready-made matrix-core operands: one 16-row slab per tile of Pi (w > 0) and
    # of the sketch, (d / 32) k-steps x (hi, lo) x 1 KiB each
    for d, w, m in [(128, 2, 128), (128, 0, 256), (256, 3, 256), (64, 1, 64), (128, 0, 192), (128, 0, 384),
                    (128, 0, 512)]:
        slabs = (d // 16 if w > 0 else 0) + m // 16
        # the operands, then a 256-byte header (the rotation's common magnitude), then for pure-QJL
        # shapes at d = 128 with 320 <= m <= 512 the sketch again in the register-resident kernel's
        # layout (m / 32 tiles x 8 k-steps x hi/lo x 1 KiB)
        qjl = m * 512 if (d == 128 and w == 0 and 320 <= m <= 512) else 0
        assert aqkv.quantize_keys_workspace_bytes(aqkv.config(d, w, m)) == slabs * (d // 32) * 2048 + 256 + qjl
    ws = aqkv.decode_workspace_bytes(cfg, 8, 32, 8, 131072)
    assert ws > 0 and ws % 256 == 0
    assert aqkv.decode_workspace_bytes(cfg, 1, 32, 5, 100) == 0   # Hq % Hkv != 0


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _cache(n_slots=2, cap=64, misalign=0, blocks=FAKE):
    return aqkv.CacheDesc(None if blocks is None else blocks + misalign, n_slots, cap)


def _view(tokens=8, dtype=aqkv.BF16, data=FAKE, stride=128):
    return aqkv.KvView(data, dtype, 1, 2, tokens, 2 * 64 * stride, 64 * stride, stride)


def test_quantize_keys_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    ws = 1 << 20

    def call(cfg=cfg, layer=layer, view=None, off=0, cache=None, wsp=FAKE, wsb=ws):
        view = view or _view()
        cache = cache or _cache()
        return lib.aqkv_quantize_keys(C.byref(cfg) if cfg else None, C.byref(layer) if layer else None,
                                      C.byref(view), off, C.byref(cache), wsp, wsb, None)

    assert call(cfg=None) == -1
    assert call(layer=None) == -1
    assert call(cfg=aqkv.config(100, 2, 128)) == -2
    assert call(view=_view(dtype=7)) == -6
    assert call(view=_view(data=FAKE + 4)) == -3
    assert call(view=_view(stride=132)) == -3
    assert call(view=_view(stride=100)) == -2
    assert call(cache=_cache(n_slots=3)) == -2
    assert call(off=60) == -4
    assert call(off=-1) == -2
    assert call(cache=_cache(misalign=8)) == -3
    assert call(cache=_cache(blocks=None)) == -1
    assert call(cache=_cache(cap=48)) == -2          # capacity must be whole 32-token records
    assert call(wsb=16) == -5
    assert call(wsp=None) == -5
    assert call(layer=aqkv.LayerParams(FAKE, None, FAKE, FAKE)) == -1
    # zero tokens: valid and nothing to launch
    assert call(view=_view(tokens=0)) == 0


def test_prepared_key_entry_points_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    ws = aqkv.quantize_keys_workspace_bytes(cfg)
    assert lib.aqkv_prepare_key_operands(None, C.byref(layer), FAKE, ws, None) == -1
    assert lib.aqkv_prepare_key_operands(C.byref(cfg), None, FAKE, ws, None) == -1
    assert lib.aqkv_prepare_key_operands(C.byref(cfg), C.byref(layer), FAKE, ws - 1, None) == -5
    assert lib.aqkv_prepare_key_operands(C.byref(cfg), C.byref(layer), FAKE + 16, ws, None) == -3
    assert lib.aqkv_prepare_key_operands(C.byref(cfg), C.byref(aqkv.LayerParams(FAKE, None, FAKE, FAKE)),
                                         FAKE, ws, None) == -1

    def call(view=None, cache=None, wsb=ws, layer=layer):
        return lib.aqkv_quantize_keys_prepared(C.byref(cfg), C.byref(layer), C.byref(view or _view()), 0,
                                               C.byref(cache or _cache()), FAKE, wsb, None)

    assert call(wsb=16) == -5
    assert call(cache=_cache(n_slots=3)) == -2
    assert call(layer=aqkv.LayerParams(FAKE, FAKE, None, FAKE)) == -1   # the codebook is still read
    # rotation and sketch are not read: NULL passes validation (zero tokens: nothing to launch)
    assert call(view=_view(tokens=0), layer=aqkv.LayerParams(None, None, FAKE, FAKE)) == 0


def test_quantize_values_and_query_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    v = _view()
    assert lib.aqkv_quantize_values(C.byref(cfg), C.byref(v), 57, C.byref(_cache()), None) == -4
    assert lib.aqkv_quantize_values(C.byref(cfg), C.byref(v), 0, C.byref(_cache(misalign=4)), None) == -3
    assert lib.aqkv_quantize_values(C.byref(cfg), C.byref(_view(tokens=0)), 0, C.byref(_cache()), None) == 0
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    assert lib.aqkv_prepare_query(C.byref(cfg), C.byref(layer), FAKE, 5, 4, FAKE, FAKE, None) == -6
    assert lib.aqkv_prepare_query(C.byref(cfg), C.byref(layer), FAKE + 2, 0, 4, FAKE, FAKE, None) == -3
    assert lib.aqkv_prepare_query(C.byref(cfg), C.byref(layer), FAKE, 0, 4, None, FAKE, None) == -1
    assert lib.aqkv_prepare_query(C.byref(cfg), C.byref(layer), FAKE, 0, 0, FAKE, FAKE, None) == 0


def test_decode_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    need = aqkv.decode_workspace_bytes(cfg, 1, 4, 2, 64)

    def call(b=1, hq=4, hkv=2, T=64, scale=0.1, ws=need, cache=None, out=FAKE):
        cache = cache or _cache()
        return lib.aqkv_decode_attention(C.byref(cfg), C.byref(layer), C.byref(cache), b, hq, hkv, T,
                                         FAKE, FAKE, C.c_float(scale), None, out, FAKE, ws, None)

    assert call(hq=5) == -2
    assert call(b=2) == -2               # n_slots mismatch
    assert call(T=65) == -4
    assert call(scale=0.0) == -2
    assert call(scale=float("nan")) == -2
    assert call(ws=need - 1) == -5
    assert call(out=None) == -1
    assert call(hq=64, hkv=2) == -8      # 32 query heads per kv head: not built
    assert call(b=0, cache=_cache(n_slots=0)) == 0


def test_decode_window_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    need = aqkv.decode_workspace_bytes(cfg, 1, 4, 2, 64)

    def win(tokens=8, dtype=aqkv.BF16, heads=2, batch=1):
        return aqkv.KvView(FAKE, dtype, batch, heads, tokens, heads * 1024 * 128, 1024 * 128, 128)

    def call(kw=None, vw=None, q=FAKE, T=64):
        kw = kw or win()
        vw = vw or win()
        return lib.aqkv_decode_attention_window(C.byref(cfg), C.byref(layer), C.byref(_cache()), 1, 4, 2, T, q,
                                                FAKE, FAKE, C.byref(kw), C.byref(vw), C.c_float(0.1), None, FAKE,
                                                FAKE, need, None)

    assert lib.aqkv_decode_attention_window(C.byref(cfg), C.byref(layer), C.byref(_cache()), 1, 4, 2, 64, FAKE,
                                            FAKE, FAKE, None, C.byref(win()), C.c_float(0.1), None, FAKE, FAKE,
                                            need, None) == -1
    assert call(q=None) == -1
    assert call(q=FAKE + 4) == -3
    assert call(vw=win(dtype=aqkv.FP32)) == -6
    assert call(vw=win(tokens=9)) == -2
    assert call(kw=win(heads=3), vw=win(heads=3)) == -2
    assert call(kw=win(tokens=1025), vw=win(tokens=1025)) == -8
    assert call(kw=win(dtype=7), vw=win(dtype=7)) == -6


@pytest.mark.parametrize("d,bits", [(128, 1), (128, 2), (128, 3), (256, 2), (256, 3), (64, 2), (3, 2)])
def test_library_codebook_equals_oracle(d, bits):
    c, t = aqkv.build_codebook(d, bits)
    oc, ot = ocb.codebook_fp32(d, bits)
    np.testing.assert_array_equal(c, oc)
    np.testing.assert_array_equal(t, ot)


@pytest.mark.parametrize("d,layer", [(128, 0), (128, 5), (256, 0), (64, 1)])
def test_library_rotation_matches_oracle(d, layer):
    g, _ = inputs.layer_gaussians(layer, d, d)
    pi = aqkv.build_rotation(g)
    ref = orot.rotation_from_gaussian(g)
    assert np.max(np.abs(pi.astype(np.float64) - ref)) < 2e-7
    assert np.max(np.abs(pi.astype(np.float64).T @ pi.astype(np.float64) - np.eye(d))) < 1e-6


def test_value_side_index_is_a_permutation():
    # the scale / min of every (token, group) of a record has its own float of the field,
    # and tokens t, t + 4 of a group share one 16-byte quad
    for groups in (2, 4, 8):
        idx = aqkv.side_index(groups)
        assert sorted(idx.reshape(-1).tolist()) == list(range(32 * groups * 2))
        for t in range(32):
            if (t >> 2) & 1 == 0:
                np.testing.assert_array_equal(idx[t + 4] // 4, idx[t] // 4)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_library_hadamard_rotation_equals_oracle(d):
    g, _ = inputs.layer_gaussians(2, d, d)
    np.testing.assert_array_equal(aqkv.build_hadamard_rotation(g), orot.randomized_hadamard_fp32(g))
    with pytest.raises(aqkv.AqkvError) as e:
        aqkv.build_hadamard_rotation(np.zeros((96, 96)))
    assert e.value.status == -2


def test_decode_topk_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    need = aqkv.decode_topk_workspace_bytes(cfg, 1, 4, 2, 64, 16)
    assert need > 0 and need % 256 == 0
    assert aqkv.decode_topk_workspace_bytes(cfg, 1, 4, 2, 64, 0) == 0

    def call(budget=16, q=FAKE, hq=4, ws=need):
        return lib.aqkv_decode_attention_topk(C.byref(cfg), C.byref(layer), C.byref(_cache()), 1, hq, 2, 64, q,
                                              FAKE, FAKE, budget, C.c_float(0.1), None, FAKE, FAKE, ws, None)

    assert call(budget=0) == -2
    assert call(budget=(1 << 20) + 1) == -8
    assert call(q=None) == -1
    assert call(q=FAKE + 4) == -3
    assert call(hq=5) == -2
    assert call(ws=need - 1) == -5
    # row indices of the select are 32-bit: longer contexts are refused before any launch
    big = (1 << 31) - (1 << 20) + 32
    cache = _cache(cap=big)
    assert lib.aqkv_decode_attention_topk(C.byref(cfg), C.byref(layer), C.byref(cache), 1, 4, 2, big, FAKE, FAKE,
                                          FAKE, 16, C.c_float(0.1), None, FAKE, FAKE, need, None) == -8


def test_decode_topk_blocks_validation_codes():
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    need = aqkv.decode_topk_blocks_workspace_bytes(cfg, 1, 4, 2, 64, 16)
    assert need > 0 and need % 256 == 0
    assert aqkv.decode_topk_blocks_workspace_bytes(cfg, 1, 4, 2, 64, 0) == 0
    # more budget never needs less workspace; a budget past the context needs what the whole context does
    assert aqkv.decode_topk_blocks_workspace_bytes(cfg, 1, 4, 2, 64, 64) >= need
    assert aqkv.decode_topk_blocks_workspace_bytes(cfg, 1, 4, 2, 64, 10 ** 5) == \
        aqkv.decode_topk_blocks_workspace_bytes(cfg, 1, 4, 2, 64, 64)

    def call(budget=16, q=FAKE, hq=4, ws=need, c=cfg):
        return lib.aqkv_decode_attention_topk_blocks(C.byref(c), C.byref(layer), C.byref(_cache()), 1, hq, 2, 64,
                                                     q, FAKE, FAKE, budget, C.c_float(0.1), None, FAKE, FAKE, ws,
                                                     None)

    assert call(budget=0) == -2
    assert call(budget=(1 << 20) + 1) == -8
    assert call(q=None) == -1
    assert call(q=FAKE + 4) == -3
    assert call(hq=5) == -2
    assert call(ws=need - 1) == -5
    # shapes without a matrix-core decoder (sketch rows != d with mse bits) are not covered
    assert call(c=aqkv.config(128, 2, 256)) == -8


def test_noalloc_decode_validation_codes():
    # the allocation-free decode checks its sizes against the static scratch before any HIP call
    lib = aqkv.lib()
    cfg = aqkv.config(128, 2, 128)
    layer = aqkv.LayerParams(FAKE, FAKE, FAKE, FAKE)
    assert lib.aqkv_decode_static_scratch_bytes() == 8 << 20
    big = aqkv.CacheDesc(FAKE, 4096 * 8, 4096)
    assert lib.aqkv_decode_attention_noalloc(C.byref(cfg), C.byref(layer), C.byref(big), 4096, 64, 8, 4096, FAKE,
                                             FAKE, C.c_float(0.1), None, FAKE, None) == -9
    assert lib.aqkv_status_string(-9) == b"request needs more than the library's static scratch"

    def call(b=1, hq=4, hkv=2, T=64, scale=0.1, out=FAKE):
        return lib.aqkv_decode_attention_noalloc(C.byref(cfg), C.byref(layer), C.byref(_cache()), b, hq, hkv, T,
                                                 FAKE, FAKE, C.c_float(scale), None, out, None)

    assert call(hq=5) == -2
    assert call(b=2) == -2
    assert call(T=65) == -4
    assert call(scale=0.0) == -2
    assert call(out=None) == -1
    assert call(b=0, hkv=2) == -2                       # zero batch against a two-slot cache


@pytest.mark.parametrize("side_f16", [False, True])
def test_cache_field_views_over_a_buffer_view(side_f16):
    # a cache whose records are a slice of a larger buffer (guard records around it): every
    # field view reads the slice's bytes, not the larger buffer's
    import torch
    cfg = aqkv.config(128, 2, 128, side_f16=side_f16)
    lo = aqkv.cache_layout(cfg)
    big = (torch.arange(10 * lo["block_bytes"]) % 251).to(torch.uint8).reshape(10, -1)
    inner = aqkv.Cache(cfg, 2, 64, big[3:7], lo)
    copy = aqkv.Cache(cfg, 2, 64, big[3:7].clone(), lo)
    for name in aqkv.FIELDS:
        a, b = inner.field(name), copy.field(name)
        assert a.dtype == b.dtype and torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
    s1, m1 = inner.value_side(5, 40)
    s2, m2 = copy.value_side(5, 40)
    assert torch.equal(s1.view(torch.uint8), s2.view(torch.uint8)) and torch.equal(m1.view(torch.uint8), m2.view(torch.uint8))
