"""GPU parity of the half side-information option (key norm, residual norm,
value scale and min stored as IEEE halves), through the C ABI, against the
oracle's reading (oracle.layout.stored_side: the fp32 number rounded to the
nearest half, saturating at +-65504; every code decided from the unrounded
numbers).

Bars: codes and sign bits as with fp32 side information (bit-exact outside
the 1e-5 window); value scale and min halves bit-exact (both sides round the
same bit-exact fp32 numbers); key norms within one half ulp of the oracle's
(the two sides' fp32 norms differ by a few fp32 ulps, so a norm next to a
half rounding midpoint may round the other way) and equal on all but a
handful; decode scores within 1e-3 relative and outputs within 2e-3 absolute,
on planes the oracle quantised (the same bars as for fp32 side information)
and end to end."""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv, inputs
from oracle import attention as oatt
from oracle import layout as olay
from oracle import values as ovals

from gpu_helpers import (OUT_ATOL, SCORE_RTOL, cfg_of, compare_keys, device_layer, half_ulp, host_layer,
                         oracle_rows, read_planes, say, to_device_kv, torch_dev)
from test_gpu_parity import run_decode_parity
from test_gpu_topk import run_topk

pytestmark = pytest.mark.gpu


def _as_dtype(x, dtype):
    return inputs.bf16_bits_to_f32(inputs.to_bf16_bits(x)) if dtype == "bf16" else x


def _norms_match(gpu, ref, min_equal):
    """gpu and ref halves: every pair within one half ulp, at least min_equal of them equal."""
    g, r = gpu.astype(np.float64), ref.astype(np.float64)
    assert np.all(np.abs(g - r) <= half_ulp(ref)), np.max(np.abs(g - r) / half_ulp(ref))
    eq = float(np.mean(g == r)) if g.size else 1.0
    assert eq >= min_equal, eq
    return eq


# d, w, m, key dtype: both key quantisers (the pure-QJL register-resident one at m = 512)
KEY_CASES = [(128, 2, 128, "bf16"), (256, 2, 256, "bf16"), (128, 0, 512, "bf16"), (128, 0, 192, "bf16"),
             (64, 1, 64, "fp32"), (128, 0, 384, "fp32")]


@pytest.mark.parametrize("d,w,m,dtype", KEY_CASES)
def test_quantize_keys_half_norms(d, w, m, dtype):
    torch, dev = torch_dev()
    say("quantize_keys half side", d, w, m, dtype)
    B, H, T = 2, 2, 700
    rng = np.random.default_rng(d + m + 3 * w)
    k = _as_dtype((rng.standard_normal((B, H, T, d)) * 1.5).astype(np.float32), dtype)
    k[0, 0, 5] = 0.0                     # zero key
    k[1, 1, 7] *= 2.0 ** 17              # norm past the half range: saturates to 65504
    k[0, 1, 9] *= 2.0 ** -20             # norm in the half subnormal range
    hl = host_layer(d, w, m, layer=1)
    cfg = cfg_of(hl, 2, True)
    cache = aqkv.Cache.allocate(cfg, B * H, T + 40)
    aqkv.quantize_keys(cfg, device_layer(hl), to_device_kv(k, dtype), cache, token_offset=40)
    torch.cuda.synchronize()
    eqs = []
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 40, 40 + T)
        assert gpu["norm"].dtype == np.float16
        qk, kr, _, _ = oracle_rows(hl, k[b, h], np.zeros((T, d), np.float32), side_f16=True)
        par = compare_keys(hl, k[b, h], qk, gpu)
        assert par.idx_mismatch_outside == 0, par
        assert par.sign_mismatch_outside == 0, par
        eqs.append(_norms_match(gpu["norm"], kr[2], 0.99))
        if w > 0:
            clean = (olay.unpack_code_planes(gpu["codes"], d, w) == qk.idx).all(axis=1)
            _norms_match(gpu["rnorm"][clean], kr[3][clean], 0.95)
        if s == 0:
            assert gpu["norm"][5] == 0.0 and np.all(gpu["signs"][5] == 0xFF)
        if s == 3:
            assert gpu["norm"][7] == 65504.0
        if s == 1:
            assert 0.0 < gpu["norm"][9] < 2.0 ** -14       # a subnormal half
    say(f"norm halves equal to the oracle's: {min(eqs):.4f} (worst slot)")


@pytest.mark.parametrize("d,vb,dtype", [(128, 2, "bf16"), (256, 2, "bf16"), (64, 4, "fp32"), (128, 4, "bf16")])
def test_quantize_values_half_side_bit_exact(d, vb, dtype):
    torch, dev = torch_dev()
    say("quantize_values half side", d, vb, dtype)
    B, H, T = 2, 3, 555
    v = _as_dtype((np.random.default_rng(9 + d + vb).standard_normal((B, H, T, d)) * 3.0).astype(np.float32),
                  dtype)
    v[0, 0, 3, :32] = 1.25                                   # constant group: scale 0
    v[0, 2, 4, :32] = np.arange(32) * 1e-7                   # scale a half subnormal
    v[1, 1, 8, 32:64] = np.linspace(-1e6, 1e6, 32)           # scale and min past the half range
    v[1, 2, 10, :32] = np.linspace(-70000.0, -60000.0, 32)   # min saturates, scale stays normal
    v = _as_dtype(v, dtype)
    hl = host_layer(d, 2, d)
    cfg = cfg_of(hl, vb, True)
    cache = aqkv.Cache.allocate(cfg, B * H, T)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache)
    torch.cuda.synchronize()
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 0, T)
        assert gpu["vscale"].dtype == np.float16
        vc, vs, vm = ovals.quantize_values(v[b, h], vb)
        np.testing.assert_array_equal(olay.unpack_value_codes(gpu["vcodes"], T, d, vb), vc)
        np.testing.assert_array_equal(gpu["vscale"].view(np.uint16), olay.stored_side(vs, True).view(np.uint16))
        np.testing.assert_array_equal(gpu["vmin"].view(np.uint16), olay.stored_side(vm, True).view(np.uint16))
    gpu = read_planes(cache, 4, 0, T)
    assert gpu["vmin"][8, 1] == -65504.0 and gpu["vscale"][8, 1] == 65504.0


DECODE_CASES = [
    # d, w, m, G, vb, T: the 5.22x configuration (d = 256, 3-bit keys, 2-bit values) first
    (256, 2, 256, 2, 2, 700), (256, 2, 256, 8, 2, 300), (128, 2, 128, 4, 2, 1000), (128, 2, 128, 8, 4, 4097),
    (128, 0, 384, 4, 4, 333), (128, 0, 512, 4, 2, 300), (64, 1, 64, 4, 4, 255), (64, 0, 64, 1, 2, 100),
    (128, 3, 128, 2, 2, 33),
    # the scalar decoder (no matrix-core kernel for these shapes)
    (128, 2, 256, 4, 2, 700), (64, 2, 128, 2, 4, 300),
]


@pytest.mark.parametrize("d,w,m,G,vb,T", DECODE_CASES)
def test_decode_half_side_on_oracle_planes(d, w, m, G, vb, T):
    run_decode_parity(d, w, m, G, vb, T, side_f16=True)


@pytest.mark.parametrize("d,w,m,G,T,budget,vb", [(256, 2, 256, 2, 300, 129, 2), (128, 0, 384, 4, 700, 90, 2),
                                                 (128, 2, 128, 2, 900, 300, 4)])
def test_topk_half_side(d, w, m, G, T, budget, vb):
    run_topk(d, w, m, G, T, budget, vb, side_f16=True)


@pytest.mark.parametrize("d,w,m,G,dtype", [(256, 2, 256, 2, "bf16"), (128, 2, 128, 4, "bf16"),
                                           (128, 0, 512, 4, "bf16"), (128, 0, 256, 4, "bf16")])
def test_end_to_end_half_side(d, w, m, G, dtype):
    torch, dev = torch_dev()
    say("end to end half side", d, w, m, G, dtype)
    B, Hkv, T = 2, 2, 1200
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=4)
    cfg = cfg_of(hl, 2, True)
    layer = device_layer(hl)
    rng = np.random.default_rng(21)
    k = _as_dtype(rng.standard_normal((B, Hkv, T, d)).astype(np.float32), dtype)
    v = _as_dtype(rng.standard_normal((B, Hkv, T, d)).astype(np.float32), dtype)
    q = _as_dtype(rng.standard_normal((B, Hq, d)).astype(np.float32), dtype)
    cache = aqkv.Cache.allocate(cfg, B * Hkv, T)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, dtype), cache)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache)
    qd = to_device_kv(q.reshape(1, B, Hq, d), dtype).reshape(B, Hq, d).contiguous()
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    scores = torch.empty((B, Hq, T), device=dev)
    out = aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, scores=scores)
    torch.cuda.synchronize()
    out, scores = out.cpu().numpy(), scores.cpu().numpy()
    for s in range(B * Hkv):
        b, h = divmod(s, Hkv)
        gpu = read_planes(cache, s, 0, T)
        qk, kr, vt, _ = oracle_rows(hl, k[b, h], v[b, h], side_f16=True)
        qh = q[b, h * G:(h + 1) * G]
        rows = (qk.idx, qk.bits, kr[2].astype(np.float64), kr[3].astype(np.float64))
        s_ref, o_ref = oatt.decode_slot(qh, rows, vt, hl.rotation, hl.sketch, hl.centroids, w)
        assert np.max(np.abs(out[b, h * G:(h + 1) * G] - o_ref)) <= OUT_ATOL
        clean = np.ones(T, bool)
        if w > 0:
            clean &= (olay.unpack_code_planes(gpu["codes"], d, w) == qk.idx).all(axis=1)
        clean &= (olay.unpack_bits(gpu["signs"], m) == qk.bits).all(axis=1)
        sg = scores[b, h * G:(h + 1) * G]
        rms = np.sqrt(np.mean(s_ref ** 2, axis=-1, keepdims=True))
        rel = np.abs(sg - s_ref) / np.maximum(np.abs(s_ref), rms)
        assert np.max(rel[:, clean]) <= SCORE_RTOL
