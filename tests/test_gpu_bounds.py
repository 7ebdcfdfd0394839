"""Bounds and determinism checks of every entry point on the GPU.

* Guard bands: every buffer a call writes sits inside a larger allocation
  whose bytes before and after it hold a known pattern (cache records before
  and after the cache; bytes past out, scores, selected, q_rot, q_sketch and
  the workspace); after the call the pattern must be intact.
* Inside the cache a quantise call writes only rows [token_offset,
  token_offset + n) of every slot, and only its own fields (keys: codes,
  signs, norms; values: codes and side information); every other token of
  every field keeps its bytes, including the tokens that share a 32-token
  record (and a packed value-code word) with the written ones.  Decode calls
  leave the cache untouched.
* Run twice: every call, repeated on the same inputs into fresh buffers with
  the same initial bytes, gives bit-identical results (no order-dependent
  reduction, no race between blocks).
"""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv
from oracle import layout as olay

from gpu_helpers import cfg_of, device_layer, host_layer, say, to_device_kv, torch_dev

pytestmark = pytest.mark.gpu

PAT = 0xA5           # guard byte
GUARD = 4096         # guard bytes on each side (keeps 256-byte alignment)
GREC = 3             # guard records on each side of a cache

KEY_FIELDS = ("key_codes", "key_signs", "key_norm", "key_rnorm")
VALUE_FIELDS = ("val_codes", "val_side")


def _guarded(nbytes):
    """(whole buffer, the middle view of nbytes) with the guard pattern everywhere."""
    torch, dev = torch_dev()
    buf = torch.full((2 * GUARD + nbytes,), PAT, dtype=torch.uint8, device=dev)
    return buf, buf[GUARD:GUARD + nbytes]


def _guards_intact(buf, nbytes, what):
    b = buf.cpu().numpy()
    assert np.all(b[:GUARD] == PAT), f"{what}: bytes before the buffer changed"
    assert np.all(b[GUARD + nbytes:] == PAT), f"{what}: bytes past the buffer changed"


def _f32(shape):
    n = int(np.prod(shape))
    buf, view = _guarded(4 * n)
    return buf, view.view(__import__("torch").float32).reshape(shape)


def _guarded_cache(cfg, n_slots, capacity, seed):
    """A cache whose records sit between GREC guard records on each side, every byte random."""
    torch, dev = torch_dev()
    lo = aqkv.cache_layout(cfg)
    n_rec = n_slots * capacity // 32
    g = torch.Generator(device="cpu").manual_seed(seed)
    big = torch.randint(0, 256, (n_rec + 2 * GREC, lo["block_bytes"]), dtype=torch.uint8, generator=g).to(dev)
    cache = aqkv.Cache(cfg, n_slots, capacity, big[GREC:GREC + n_rec], lo)
    return big, cache


def _cache_over(cfg, n_slots, capacity, big):
    lo = aqkv.cache_layout(cfg)
    return aqkv.Cache(cfg, n_slots, capacity, big[GREC:GREC + n_slots * capacity // 32], lo)


def _token_rows(cache, name, slot):
    """Per-token bytes of one slot's field, [capacity, row bytes] (value codes unpacked to one
    code per channel, value side information to [capacity, groups, 2])."""
    cap = cache.capacity
    r0 = slot * cap
    if name == "val_codes":
        rows = cache.rows("val_codes", r0, cap).cpu().numpy()
        return olay.unpack_value_codes(rows, cap, cache.cfg.head_dim, cache.cfg.value_bits)
    if name == "val_side":
        sc, mn = cache.value_side(r0, cap)
        both = np.stack([sc.cpu().numpy(), mn.cpu().numpy()], axis=-1)
        return both.view(np.uint16 if both.dtype == np.float16 else np.uint32)
    f = cache.field(name)
    if f is None:
        return None
    rows = f.flatten(0, 1)[r0:r0 + cap].contiguous().view(__import__("torch").uint8)
    return rows.cpu().numpy().reshape(cap, -1)


def _check_cache_writes(cfg, n_slots, cap, before, after, written, off, n):
    """Guard records intact; fields not in `written` unchanged everywhere; fields in `written`
    unchanged outside token rows [off, off + n) of every slot."""
    b, a = before.cpu().numpy(), after.cpu().numpy()
    assert np.array_equal(b[:GREC], a[:GREC]), "guard records before the cache changed"
    assert np.array_equal(b[-GREC:], a[-GREC:]), "guard records after the cache changed"
    cb, ca = _cache_over(cfg, n_slots, cap, before), _cache_over(cfg, n_slots, cap, after)
    outside = np.ones(cap, bool)
    outside[off:off + n] = False
    changed_inside = 0
    for name in aqkv.FIELDS:
        for s in range(n_slots):
            rb, ra = _token_rows(cb, name, s), _token_rows(ca, name, s)
            if rb is None:
                continue
            if name not in written:
                assert np.array_equal(rb, ra), f"{name} of slot {s} written by a call that does not own it"
                continue
            same = (rb == ra).reshape(cap, -1).all(axis=1)
            bad = np.flatnonzero(outside & ~same)
            assert bad.size == 0, f"{name} of slot {s}: tokens {bad[:8]} outside [{off}, {off + n}) changed"
            changed_inside += int((~same[off:off + n]).sum())
    return changed_inside


KEY_CASES = [
    # d, w, m, dtype, token_offset, tokens, half side information
    (128, 2, 128, "bf16", 37, 70, False), (128, 0, 512, "bf16", 45, 200, False),
    (128, 0, 384, "bf16", 3, 129, False), (256, 3, 256, "fp32", 0, 33, False),
    (128, 0, 192, "bf16", 96, 64, False), (64, 1, 64, "fp32", 5, 1, False),
    (256, 2, 256, "bf16", 13, 100, True), (128, 0, 512, "bf16", 31, 66, True),
]


@pytest.mark.parametrize("d,w,m,dtype,off,n,sf", KEY_CASES)
def test_quantize_keys_writes_only_its_rows(d, w, m, dtype, off, n, sf):
    torch, dev = torch_dev()
    say("bounds quantize_keys", d, w, m, dtype, off, n, sf)
    B, H = 1, 3
    cap = (off + n + 40 + 31) // 32 * 32
    hl = host_layer(d, w, m, layer=5)
    cfg = cfg_of(hl, 2, sf)
    layer = device_layer(hl)
    k = (np.random.default_rng(d + off).standard_normal((B, H, n, d)) * 2).astype(np.float32)
    kd = to_device_kv(k, dtype)
    ws_bytes = aqkv.quantize_keys_workspace_bytes(cfg)
    results = []
    for rep in range(2):
        big, cache = _guarded_cache(cfg, B * H, cap, seed=1234)
        before = big.clone()
        wbuf, ws = _guarded(ws_bytes)
        aqkv.quantize_keys(cfg, layer, kd, cache, token_offset=off, workspace=ws)
        torch.cuda.synchronize()
        _guards_intact(wbuf, ws_bytes, "key workspace")
        changed = _check_cache_writes(cfg, B * H, cap, before, big, KEY_FIELDS, off, n)
        assert changed > 0
        results.append(big.cpu().numpy())
    assert np.array_equal(results[0], results[1]), "two runs differ"


VALUE_CASES = [
    # d, vb, dtype, token_offset, tokens, half side information
    (128, 2, "bf16", 37, 70, False), (128, 4, "bf16", 31, 2, False), (64, 4, "fp32", 0, 100, False),
    (256, 2, "bf16", 64, 64, False), (128, 2, "bf16", 3, 40, True), (256, 4, "fp32", 17, 1, True),
]


@pytest.mark.parametrize("d,vb,dtype,off,n,sf", VALUE_CASES)
def test_quantize_values_writes_only_its_rows(d, vb, dtype, off, n, sf):
    torch, dev = torch_dev()
    say("bounds quantize_values", d, vb, dtype, off, n, sf)
    B, H = 2, 2
    cap = (off + n + 40 + 31) // 32 * 32
    hl = host_layer(d, 2, d)
    cfg = cfg_of(hl, vb, sf)
    v = (np.random.default_rng(d + vb + off).standard_normal((B, H, n, d)) * 3).astype(np.float32)
    vd = to_device_kv(v, dtype)
    results = []
    for rep in range(2):
        big, cache = _guarded_cache(cfg, B * H, cap, seed=99)
        before = big.clone()
        aqkv.quantize_values(cfg, vd, cache, token_offset=off)
        torch.cuda.synchronize()
        changed = _check_cache_writes(cfg, B * H, cap, before, big, VALUE_FIELDS, off, n)
        assert changed > 0
        results.append(big.cpu().numpy())
    assert np.array_equal(results[0], results[1]), "two runs differ"


def _filled_cache(hl, cfg, B, Hkv, T, seed):
    """A guarded cache with T tokens of keys and values quantised by the library."""
    torch, dev = torch_dev()
    cap = (T + 31) // 32 * 32
    big, cache = _guarded_cache(cfg, B * Hkv, cap, seed=seed)
    rng = np.random.default_rng(seed)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, hl.d)).astype(np.float32)).to(dev)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, hl.d)).astype(np.float32)).to(dev)
    layer = device_layer(hl)
    aqkv.quantize_keys(cfg, layer, k, cache)
    aqkv.quantize_values(cfg, v, cache)
    return big, cache, layer


DECODE_CASES = [
    # d, w, m, G, T, half side information: matrix-core decoder, scalar decoder, pure QJL
    (128, 2, 128, 4, 1000, False), (128, 2, 256, 2, 300, False), (128, 0, 384, 4, 777, False),
    (256, 2, 256, 2, 100, True), (64, 1, 64, 8, 33, False),
]


@pytest.mark.parametrize("d,w,m,G,T,sf", DECODE_CASES)
def test_decode_calls_stay_in_their_buffers(d, w, m, G, T, sf):
    torch, dev = torch_dev()
    say("bounds decode", d, w, m, G, T, sf)
    B, Hkv = 2, 2
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=7)
    cfg = cfg_of(hl, 2, sf)
    big, cache, layer = _filled_cache(hl, cfg, B, Hkv, T, seed=d + T)
    torch.cuda.synchronize()
    cache_before = big.clone()
    q = torch.from_numpy(np.random.default_rng(3).standard_normal((B, Hq, d)).astype(np.float32)).to(dev)

    # prepare_query: q_rot and q_sketch with guards
    runs = []
    for rep in range(2):
        rbuf, q_rot = _f32((B, Hq, d)) if w > 0 else (None, None)
        sbuf, q_sk = _f32((B, Hq, m))
        aqkv.prepare_query(cfg, layer, q, q_rot=q_rot, q_sketch=q_sk)
        torch.cuda.synchronize()
        if w > 0:
            _guards_intact(rbuf, 4 * B * Hq * d, "q_rot")
        _guards_intact(sbuf, 4 * B * Hq * m, "q_sketch")
        runs.append((None if q_rot is None else q_rot.clone(), q_sk.clone()))
    assert torch.equal(runs[0][1], runs[1][1]) and (w == 0 or torch.equal(runs[0][0], runs[1][0]))
    q_rot, q_sk = runs[0]

    # decode: out, scores and workspace with guards
    ws_bytes = aqkv.decode_workspace_bytes(cfg, B, Hq, Hkv, T)
    outs = []
    for rep in range(2):
        obuf, out = _f32((B, Hq, d))
        scbuf, scores = _f32((B, Hq, T))
        wbuf, ws = _guarded(ws_bytes)
        aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, scores=scores, out=out, workspace=ws)
        torch.cuda.synchronize()
        _guards_intact(obuf, 4 * B * Hq * d, "decode out")
        _guards_intact(scbuf, 4 * B * Hq * T, "decode scores")
        _guards_intact(wbuf, ws_bytes, "decode workspace")
        assert torch.isfinite(out).all() and torch.isfinite(scores).all()
        outs.append((out.clone(), scores.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), "two decode runs differ"

    # the allocation-free variant: same bits as the workspace call, guards intact
    obuf, out = _f32((B, Hq, d))
    scbuf, scores = _f32((B, Hq, T))
    aqkv.decode_attention_noalloc(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, out, scores=scores)
    torch.cuda.synchronize()
    _guards_intact(obuf, 4 * B * Hq * d, "noalloc out")
    _guards_intact(scbuf, 4 * B * Hq * T, "noalloc scores")
    assert torch.equal(out, outs[0][0]) and torch.equal(scores, outs[0][1])

    # recent-token window
    nw = 37
    kw = torch.from_numpy(np.random.default_rng(4).standard_normal((B, Hkv, nw, d)).astype(np.float32)).to(dev)
    vw = torch.from_numpy(np.random.default_rng(5).standard_normal((B, Hkv, nw, d)).astype(np.float32)).to(dev)
    wins = []
    for rep in range(2):
        obuf, out = _f32((B, Hq, d))
        wbuf, ws = _guarded(ws_bytes)
        aqkv.decode_attention_window(cfg, layer, cache, B, Hq, Hkv, T, q, q_rot, q_sk, kw, vw, out=out, workspace=ws)
        torch.cuda.synchronize()
        _guards_intact(obuf, 4 * B * Hq * d, "window out")
        _guards_intact(wbuf, ws_bytes, "window workspace")
        wins.append(out.clone())
    assert torch.equal(wins[0], wins[1]), "two window runs differ"

    # top-K: selected, out and workspace with guards
    budget = max(1, T // 8)
    tk_bytes = aqkv.decode_topk_workspace_bytes(cfg, B, Hq, Hkv, T, budget)
    tks = []
    for rep in range(2):
        obuf, out = _f32((B, Hq, d))
        selbuf, selv = _guarded(4 * B * Hkv * budget)
        sel = selv.view(torch.int32).reshape(B * Hkv, budget)
        wbuf, ws = _guarded(tk_bytes)
        aqkv.decode_attention_topk(cfg, layer, cache, B, Hq, Hkv, T, q, q_rot, q_sk, budget, selected=sel, out=out,
                                   workspace=ws)
        torch.cuda.synchronize()
        _guards_intact(obuf, 4 * B * Hq * d, "top-k out")
        _guards_intact(selbuf, 4 * B * Hkv * budget, "top-k selected")
        _guards_intact(wbuf, tk_bytes, "top-k workspace")
        s = sel.cpu().numpy()
        assert np.all((s >= 0) & (s < T)) and np.all(np.diff(s, axis=1) > 0)
        tks.append((out.clone(), sel.clone()))
    assert torch.equal(tks[0][0], tks[1][0]) and torch.equal(tks[0][1], tks[1][1]), "two top-k runs differ"

    # no decode call writes the cache
    assert torch.equal(big, cache_before), "a decode call wrote the cache"
