"""GPU parity: every HIP entry point, called through the C ABI, against the
oracle on the same seeded inputs, at sizes the oracle finishes in seconds that
still span several tiles and a ragged tail.

Bars: packed codes and sign bits bit-exact outside the 1e-5 decision-boundary
window (mismatch rate inside the window reported); value codes, scales and
minima bit-exact (both sides decide them in IEEE fp32); key norms within 2e-6
relative (an fp32 sum of 128-256 squares); residual norms within 5e-5
relative: the kernel takes gamma = n ||y - c[idx]|| in the rotated frame, and
y carries the split-product error of the rotation (about 2^-22 per rotated
coordinate, so ~3e-6 in ||y - c||, which is typically 0.1-0.3: up to ~1.5e-5
relative), plus the fp32 rotation's departure from orthogonality (~1e-7);
scores within 1e-3 relative; attention outputs within 2e-3 absolute.
"""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv, inputs
from oracle import attention as oatt
from oracle import layout as olay
from oracle import values as ovals

from gpu_helpers import (OUT_ATOL, SCORE_RTOL, cfg_of, compare_keys, device_layer, host_layer,
                         oracle_rows, read_planes, say, score_err, to_device_kv, torch_dev)

pytestmark = pytest.mark.gpu


def _kv(B, H, T, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, T, d)) * scale).astype(np.float32)


def _as_dtype(x, dtype):
    return inputs.bf16_bits_to_f32(inputs.to_bf16_bits(x)) if dtype == "bf16" else x


KEY_CASES = [
    (128, 2, 128, "bf16"), (128, 2, 128, "fp32"), (256, 3, 256, "bf16"), (128, 0, 192, "bf16"),
    (128, 0, 512, "bf16"), (64, 1, 64, "fp32"), (128, 1, 128, "bf16"), (128, 3, 128, "bf16"),
    (128, 2, 256, "bf16"), (256, 0, 384, "fp32"),
    # every A-QJL layer group's sketch size at d = 128 (k = 512, 384, 256, 192)
    (128, 0, 384, "bf16"), (128, 0, 256, "bf16"), (128, 0, 384, "fp32"),
    # the largest sketch the library takes (1024 rows)
    (128, 0, 1024, "bf16"), (256, 2, 1024, "fp32"),
]


@pytest.mark.parametrize("d,w,m,dtype", KEY_CASES)
def test_quantize_keys_parity(d, w, m, dtype):
    _key_parity(d, w, m, dtype, 2, 2, 1000)


# the pure-QJL kernel at every wave count (k = 320 .. 512 in steps of 64) over 40000 keys:
# 625 tiles of 64 keys on at most 256 blocks, so every block runs its loop two or three
# times (ring reuse, the next tile prepared while the current one is in the matrix
# units, sign rows stored in batches) and slot boundaries fall inside tiles
@pytest.mark.parametrize("m", [320, 384, 448, 512])
def test_quantize_keys_qjl_many_tiles(m):
    _key_parity(128, 0, m, "bf16", 2, 4, 5000)


def _key_parity(d, w, m, dtype, B, H, T):
    torch, dev = torch_dev()
    say("quantize_keys", d, w, m, dtype, B, H, T)
    k = _as_dtype(_kv(B, H, T, d, seed=d + w + m), dtype)
    k[0, 0, 5] = 0.0                     # a zero key
    k[1, 1, 7] *= 1024.0                 # a large one (power of two: stays exactly representable)
    hl = host_layer(d, w, m, layer=1)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, B * H, T + 24)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, dtype), cache, token_offset=24)
    torch.cuda.synchronize()
    tot_win = tot_mis_win = 0
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 24, 24 + T)
        qk, kr, _, _ = oracle_rows(hl, k[b, h], np.zeros((T, d), np.float32))
        par = compare_keys(hl, k[b, h], qk, gpu)
        assert par.idx_mismatch_outside == 0, par
        assert par.sign_mismatch_outside == 0, par
        tot_win += par.idx_in_window
        tot_mis_win += par.idx_mismatch_in_window
        np.testing.assert_allclose(gpu["norm"], qk.norm, rtol=2e-6, atol=0)
        if w > 0:
            clean = (olay.unpack_code_planes(gpu["codes"], d, w) == qk.idx).all(axis=1)
            np.testing.assert_allclose(gpu["rnorm"][clean], qk.rnorm[clean], rtol=5e-5, atol=1e-30)
        if s == 0:
            assert gpu["norm"][5] == 0.0 and np.all(gpu["signs"][5] == 0xFF)
            if w > 0:
                assert gpu["rnorm"][5] == 0.0
    say(f"index window: {tot_win} coords, {tot_mis_win} differ inside it")


@pytest.mark.parametrize("d,w,m,dtype", [(128, 2, 128, "bf16"), (256, 3, 256, "bf16"), (64, 1, 64, "fp32"),
                                         (128, 3, 256, "fp32")])
def test_hadamard_rotation_keys_and_decode(d, w, m, dtype):
    # a randomised Hadamard rotation through the same kernels (its +-1 operands take one
    # matrix pass): key rows against the oracle, then decode over them end to end
    torch, dev = torch_dev()
    say("hadamard rotation", d, w, m, dtype)
    B, H, T, G = 2, 2, 700, 2
    k = _kv(B, H, T, d, seed=31 + d + w)
    k[0, 1, 3, :4] *= 10.0                   # an outlier key
    k = _as_dtype(k, dtype)
    v = _as_dtype(_kv(B, H, T, d, seed=32 + d), dtype)
    hl = host_layer(d, w, m, layer=5, rotation="hadamard")
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, B * H, T)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, dtype), cache)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache)
    torch.cuda.synchronize()
    refs = []
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 0, T)
        qk, kr, vt, _ = oracle_rows(hl, k[b, h], v[b, h])
        par = compare_keys(hl, k[b, h], qk, gpu)
        assert par.idx_mismatch_outside == 0, par
        assert par.sign_mismatch_outside == 0, par
        np.testing.assert_allclose(gpu["norm"], qk.norm, rtol=2e-6, atol=0)
        idx = olay.unpack_code_planes(gpu["codes"], d, w)
        bits = olay.unpack_bits(gpu["signs"], m)
        refs.append(((idx, bits, gpu["norm"].astype(np.float64), gpu["rnorm"].astype(np.float64)), vt))
    q = np.random.default_rng(33).standard_normal((B, H * G, d)).astype(np.float32)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, torch.from_numpy(q).to(dev))
    out = aqkv.decode_attention(cfg, layer, cache, B, H * G, H, T, q_rot, q_sk).cpu().numpy()
    worst = 0.0
    for s in range(B * H):
        b, h = divmod(s, H)
        _, o_ref = oatt.decode_slot(q[b, h * G:(h + 1) * G], refs[s][0], refs[s][1], hl.rotation, hl.sketch,
                                    hl.centroids, w)
        worst = max(worst, float(np.max(np.abs(out[b, h * G:(h + 1) * G] - o_ref))))
    say(f"out err {worst:.2e}")
    assert worst <= OUT_ATOL


@pytest.mark.parametrize("d,w,m,nt", [(128, 2, 128, 1), (128, 2, 128, 7), (256, 3, 256, 5), (128, 0, 512, 3),
                                      (128, 0, 384, 2)])
def test_quantize_keys_small_append_many_slots(d, w, m, nt):
    """Decode-time appends: a few tokens for each of many slots, so one key
    tile spans several slots (and heads of several batches)."""
    torch, dev = torch_dev()
    say("small append", d, w, m, nt)
    B, H, off = 3, 5, 40
    k = _as_dtype(_kv(B, H, nt, d, seed=100 + nt), "bf16")
    hl = host_layer(d, w, m, layer=2)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, B * H, 64)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, "bf16"), cache, token_offset=off)
    torch.cuda.synchronize()
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, off, off + nt)
        qk, _, _, _ = oracle_rows(hl, k[b, h], np.zeros((nt, d), np.float32))
        par = compare_keys(hl, k[b, h], qk, gpu)
        assert par.idx_mismatch_outside == 0 and par.sign_mismatch_outside == 0, par
        np.testing.assert_allclose(gpu["norm"], qk.norm, rtol=2e-6, atol=0)


@pytest.mark.parametrize("d,vb,dtype", [(128, 2, "bf16"), (128, 2, "fp32"), (256, 2, "bf16"), (64, 4, "fp32"),
                                        (128, 4, "bf16"), (256, 4, "bf16"), (64, 2, "bf16")])
def test_quantize_values_bit_exact(d, vb, dtype):
    torch, dev = torch_dev()
    say("quantize_values", d, vb, dtype)
    B, H, T = 2, 3, 777
    v = _as_dtype(_kv(B, H, T, d, seed=7 + d + vb, scale=3.0), dtype)
    v[0, 0, 3, :32] = 1.25                # constant group
    v[1, 2, 9, 32:64] = -0.0
    # groups spanning exactly 2^vb - 1 in steps of 1/2: scale 1 and every other
    # quotient an exact tie (round half to even)
    levels = (1 << vb) - 1
    ties = (np.arange(32) % (2 * levels + 1)) * 0.5
    v[0, 1, 5, :32] = ties
    v[1, 0, 6, d - 32:] = ties - 1.0
    v[1, 1, 30, :32] = ties[::-1] * 0.25 + 3.0     # the same ties at scale 1/4, away from zero
    hl = host_layer(d, 2, d)
    cfg = cfg_of(hl, vb)
    cache = aqkv.Cache.allocate(cfg, B * H, T)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache)
    torch.cuda.synchronize()
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 0, T)
        vc, vs, vm = ovals.quantize_values(v[b, h], vb)
        np.testing.assert_array_equal(olay.unpack_value_codes(gpu["vcodes"], T, d, vb), vc)
        np.testing.assert_array_equal(gpu["vscale"].view(np.uint32), vs.view(np.uint32))
        np.testing.assert_array_equal(gpu["vmin"].view(np.uint32), vm.view(np.uint32))


# the value kernel over many records (8k-32k records, thousands of blocks, every
# records-per-block shape: d = 64, 128, 256; partly covered records at both ends)
@pytest.mark.parametrize("d,vb,dtype,B,H,T,off", [(128, 2, "bf16", 2, 4, 32768, 0), (64, 4, "fp32", 4, 4, 32000, 5),
                                                  (256, 2, "bf16", 2, 2, 32768, 13)])
def test_quantize_values_many_records(d, vb, dtype, B, H, T, off):
    torch, dev = torch_dev()
    say("quantize_values many records", d, vb, dtype, B, H, T, off)
    v = _as_dtype(_kv(B, H, T, d, seed=11 + d + vb, scale=2.0), dtype)
    hl = host_layer(d, 2, d)
    cfg = cfg_of(hl, vb)
    cache = aqkv.Cache.allocate(cfg, B * H, off + T + 7)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache, off)
    torch.cuda.synchronize()
    for s in range(B * H):
        b, h = divmod(s, H)
        gpu = read_planes(cache, s, 0, off + T)    # (codes come in whole 32-token blocks)
        vc, vs, vm = ovals.quantize_values(v[b, h], vb)
        np.testing.assert_array_equal(olay.unpack_value_codes(gpu["vcodes"], off + T, d, vb)[off:], vc)
        np.testing.assert_array_equal(gpu["vscale"][off:].view(np.uint32), vs.view(np.uint32))
        np.testing.assert_array_equal(gpu["vmin"][off:].view(np.uint32), vm.view(np.uint32))


@pytest.mark.parametrize("d,w,m", [(128, 2, 128), (256, 3, 256), (128, 0, 192)])
def test_prepared_key_operands_match_one_call(d, w, m):
    # one operand pass, then appends of 1, 2, 37 and the rest of the tokens: the same
    # cache bytes as one self-contained call
    torch, dev = torch_dev()
    say("prepared key operands", d, w, m)
    B, H, T = 2, 2, 300
    k = _as_dtype(_kv(B, H, T, d, seed=11 + d + w), "bf16")
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    kd = to_device_kv(k, "bf16")
    one = aqkv.Cache.allocate(cfg, B * H, T)
    one.blocks.zero_()
    aqkv.quantize_keys(cfg, layer, kd, one)
    parts = aqkv.Cache.allocate(cfg, B * H, T)
    parts.blocks.zero_()
    ws = aqkv.prepare_key_operands(cfg, layer, device=dev)
    for a, e in ((0, 1), (1, 3), (3, 40), (40, T)):
        aqkv.quantize_keys_prepared(cfg, layer, kd[:, :, a:e], parts, ws, token_offset=a)
    torch.cuda.synchronize()
    assert torch.equal(one.blocks, parts.blocks)


def test_chunked_append_matches_one_call():
    torch, dev = torch_dev()
    say("chunked append")
    d, w, m = 128, 2, 128
    B, H, T = 1, 2, 700
    k = _as_dtype(_kv(B, H, T, d, seed=3), "bf16")
    v = _as_dtype(_kv(B, H, T, d, seed=4), "bf16")
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    kd, vd = to_device_kv(k, "bf16"), to_device_kv(v, "bf16")
    def zeroed(cache):
        # rows past T (capacity is rounded up to 32) must compare equal too
        cache.blocks.zero_()
        return cache

    one = zeroed(aqkv.Cache.allocate(cfg, B * H, T))
    aqkv.quantize_keys(cfg, layer, kd, one)
    aqkv.quantize_values(cfg, vd, one)
    parts = zeroed(aqkv.Cache.allocate(cfg, B * H, T))
    for a, e in ((0, 300), (300, 301), (301, 333), (333, T)):
        aqkv.quantize_keys(cfg, layer, kd[:, :, a:e], parts, token_offset=a)
        aqkv.quantize_values(cfg, vd[:, :, a:e], parts, token_offset=a)
    torch.cuda.synchronize()
    for name in aqkv.FIELDS:
        a, b = one.field(name), parts.field(name)
        assert (a is None and b is None) or torch.equal(a, b), name
    assert torch.equal(one.blocks, parts.blocks)


@pytest.mark.parametrize("d,w,m,qdtype", [(128, 2, 128, "fp32"), (128, 0, 512, "bf16"), (256, 3, 256, "fp32"),
                                           (64, 1, 64, "bf16"), (256, 0, 1024, "fp32"), (128, 0, 384, "fp32")])
def test_prepare_query_parity(d, w, m, qdtype):
    torch, dev = torch_dev()
    say("prepare_query", d, w, m, qdtype)
    hl = host_layer(d, w, m, layer=2)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    q = _as_dtype(np.random.default_rng(5).standard_normal((3, 5, d)).astype(np.float32), qdtype)
    qd = to_device_kv(q.reshape(1, 3, 5, d), qdtype).reshape(3, 5, d).contiguous()
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    torch.cuda.synchronize()
    r_rot, r_sk = oatt.prepare_query(q.reshape(-1, d), hl.rotation, hl.sketch, w)
    qn = np.linalg.norm(q.reshape(-1, d), axis=1, keepdims=True)
    assert np.max(np.abs(q_sk.cpu().numpy().reshape(-1, m) - r_sk) / qn) < 2e-5
    if w > 0:
        assert np.max(np.abs(q_rot.cpu().numpy().reshape(-1, d) - r_rot) / qn) < 2e-6
    else:
        assert q_rot is None


def _upload_oracle_cache(hl, cfg, ks, vs, vb, capacity):
    """Oracle-quantised planes for slots ks[s] / vs[s] copied into a device cache."""
    torch, dev = torch_dev()
    n_slots = len(ks)
    cache = aqkv.Cache.allocate(cfg, n_slots, capacity)
    cache.blocks.zero_()
    refs = []
    for s in range(n_slots):
        qk, kr, vt, vpacked = oracle_rows(hl, ks[s], vs[s], vb, bool(cfg.side_f16))
        T = ks[s].shape[0]
        r0 = s * cache.capacity          # allocate() rounds the capacity up to 32
        codes, signs, norm, rnorm = kr
        if hl.w > 0:
            cache.set_rows("key_codes", r0, torch.from_numpy(codes).to(dev))
            cache.set_rows("key_rnorm", r0, torch.from_numpy(rnorm).to(dev))
        cache.set_rows("key_signs", r0, torch.from_numpy(signs).to(dev))
        cache.set_rows("key_norm", r0, torch.from_numpy(norm).to(dev))
        cache.set_rows("val_codes", r0, torch.from_numpy(vpacked).to(dev))
        cache.set_value_side(r0, torch.from_numpy(vt[1]).to(dev), torch.from_numpy(vt[2]).to(dev))
        # the oracle consumes exactly what was stored (fp32 or half norms, scales and minima)
        refs.append(((qk.idx, qk.bits, norm.astype(np.float64), rnorm.astype(np.float64)), vt))
    return cache, refs


DECODE_CASES = [
    # d, w, m, G, vb, T
    (128, 2, 128, 4, 2, 1000), (128, 2, 128, 1, 2, 256), (128, 2, 128, 2, 2, 1), (128, 2, 128, 8, 2, 4097),
    (256, 3, 256, 2, 2, 700), (128, 0, 192, 4, 2, 513), (128, 0, 512, 4, 2, 300), (64, 1, 64, 4, 4, 255),
    (128, 2, 128, 4, 4, 999),
    # the A-QJL layer groups at d = 128, GQA 4 (k = 384 and 256 with 2- and 4-bit values)
    (128, 0, 384, 4, 2, 700), (128, 0, 384, 4, 4, 333), (128, 0, 256, 4, 2, 4100), (128, 0, 256, 4, 4, 97),
    (128, 0, 512, 4, 4, 1025), (128, 0, 192, 4, 4, 64),
    # shapes without a matrix-core kernel (sketch rows != 64 x d/64 with mse bits): the scalar decoder
    (128, 2, 256, 4, 2, 700), (64, 2, 128, 2, 4, 300), (128, 1, 192, 8, 2, 257),
    # the largest sketch (1024 rows)
    (128, 0, 1024, 2, 2, 300), (256, 2, 1024, 1, 2, 200),
]


@pytest.mark.parametrize("d,w,m,G,vb,T", DECODE_CASES)
def test_decode_parity_on_oracle_planes(d, w, m, G, vb, T):
    run_decode_parity(d, w, m, G, vb, T)


def run_decode_parity(d, w, m, G, vb, T, side_f16=False):
    torch, dev = torch_dev()
    say("decode", d, w, m, G, vb, T, "half side" if side_f16 else "")
    B, Hkv = 2, 2
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=3)
    cfg = cfg_of(hl, vb, side_f16)
    layer = device_layer(hl)
    rng = np.random.default_rng(d * 7 + T)
    ks = [rng.standard_normal((T, d)).astype(np.float32) for _ in range(B * Hkv)]
    vs = [(rng.standard_normal((T, d)) * 2).astype(np.float32) for _ in range(B * Hkv)]
    cache, refs = _upload_oracle_cache(hl, cfg, ks, vs, vb, capacity=T + 5)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    q_rot, q_sk = oatt.prepare_query(q.reshape(-1, d), hl.rotation, hl.sketch, w)
    qr_d = torch.from_numpy(q_rot.astype(np.float32)).to(dev) if w > 0 else None
    qs_d = torch.from_numpy(q_sk.astype(np.float32)).to(dev)
    scores = torch.full((B, Hq, T), float("nan"), device=dev)
    out = aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, qr_d, qs_d, scores=scores)
    torch.cuda.synchronize()
    out, scores = out.cpu().numpy(), scores.cpu().numpy()
    worst_s = worst_o = 0.0
    for s in range(B * Hkv):
        b, hkv = divmod(s, Hkv)
        qh = q[b, hkv * G:(hkv + 1) * G]
        s_ref, o_ref = oatt.decode_slot(qh, refs[s][0], refs[s][1], hl.rotation, hl.sketch, hl.centroids, w)
        worst_s = max(worst_s, score_err(scores[b, hkv * G:(hkv + 1) * G], s_ref))
        worst_o = max(worst_o, float(np.max(np.abs(out[b, hkv * G:(hkv + 1) * G] - o_ref))))
    say(f"score err {worst_s:.2e}, out err {worst_o:.2e}")
    assert worst_s <= SCORE_RTOL
    assert worst_o <= OUT_ATOL


def test_decode_empty_context_and_degenerate_softmax():
    torch, dev = torch_dev()
    say("decode edge cases")
    d, w, m, G = 128, 2, 128, 2
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    rng = np.random.default_rng(0)
    T = 300
    ks = [rng.standard_normal((T, d)).astype(np.float32)]
    vs = [rng.standard_normal((T, d)).astype(np.float32)]
    cache, refs = _upload_oracle_cache(hl, cfg, ks, vs, 2, capacity=T)
    q = np.zeros((1, G, d), np.float32)          # all scores equal -> mean of the values
    qr = torch.zeros((1, G, d), device=dev)
    qs = torch.zeros((1, G, m), device=dev)
    out = aqkv.decode_attention(cfg, layer, cache, 1, G, 1, T, qr, qs).cpu().numpy()
    v_hat = ovals.dequantize_values(*refs[0][1])
    np.testing.assert_allclose(out[0], np.broadcast_to(v_hat.mean(0), (G, d)), atol=OUT_ATOL)
    out0 = aqkv.decode_attention(cfg, layer, cache, 1, G, 1, 0, qr, qs).cpu().numpy()
    assert np.all(out0 == 0.0)
    out1 = aqkv.decode_attention(cfg, layer, cache, 1, G, 1, 1, qr, qs).cpu().numpy()
    np.testing.assert_allclose(out1[0], np.broadcast_to(v_hat[0], (G, d)), atol=1e-5)


@pytest.mark.parametrize("d,w,m,G,dtype", [(128, 2, 128, 4, "bf16"), (128, 2, 128, 1, "fp32"),
                                           (256, 3, 256, 2, "bf16"), (128, 0, 256, 4, "bf16"),
                                           (128, 0, 384, 4, "bf16"), (128, 0, 512, 4, "bf16")])
def test_end_to_end(d, w, m, G, dtype):
    torch, dev = torch_dev()
    say("end to end", d, w, m, G, dtype)
    B, Hkv, T = 2, 2, 1500
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=4)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    k = _as_dtype(_kv(B, Hkv, T, d, seed=11), dtype)
    v = _as_dtype(_kv(B, Hkv, T, d, seed=12), dtype)
    q = _as_dtype(np.random.default_rng(13).standard_normal((B, Hq, d)).astype(np.float32), dtype)
    cache = aqkv.Cache.allocate(cfg, B * Hkv, T)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, dtype), cache)
    aqkv.quantize_values(cfg, to_device_kv(v, dtype), cache)
    qd = to_device_kv(q.reshape(1, B, Hq, d), dtype).reshape(B, Hq, d).contiguous()
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    scores = torch.empty((B, Hq, T), device=dev)
    out = aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, scores=scores)
    out2 = aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)       # deterministic
    out, scores = out.cpu().numpy(), scores.cpu().numpy()
    for s in range(B * Hkv):
        b, h = divmod(s, Hkv)
        gpu = read_planes(cache, s, 0, T)
        qk, kr, vt, _ = oracle_rows(hl, k[b, h], v[b, h])
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
        say(f"slot {s}: {int((~clean).sum())} keys differ from the oracle inside the boundary window")


def test_empty_calls_succeed_and_write_nothing():
    """Zero tokens to quantise and zero queries are valid calls that leave the
    cache as it was (a decode over zero cached rows is covered above)."""
    torch, dev = torch_dev()
    say("empty calls")
    d, w, m = 128, 2, 128
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, 4, 64)
    cache.blocks.fill_(0xAB)
    before = cache.blocks.clone()
    empty = torch.empty((2, 2, 0, d), dtype=torch.bfloat16, device=dev)
    aqkv.quantize_keys(cfg, layer, empty, cache, token_offset=5)
    aqkv.quantize_values(cfg, empty, cache, 5)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, torch.empty((0, d), device=dev))
    assert q_rot.shape == (0, d) and q_sk.shape == (0, m)
    torch.cuda.synchronize()
    assert torch.equal(cache.blocks, before)
