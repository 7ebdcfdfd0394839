"""GPU parity of query-aware top-K preselection and decode over the chosen
tokens, through the C ABI, against the oracle on the same seeded inputs (the
cache planes quantised by the oracle and uploaded).

Bars: the chosen sets agree except for tokens whose oracle cosine lies within
2e-3 x RMS of the selection threshold (estimates agree to ~1e-4 relative, so
near-ties may swap); outputs, computed by the oracle over the GPU's chosen
set, within 2e-3 absolute."""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv
from oracle import attention as oatt

from gpu_helpers import OUT_ATOL, cfg_of, device_layer, host_layer, say, torch_dev
from test_gpu_parity import _upload_oracle_cache

pytestmark = pytest.mark.gpu

CASES = [
    # d, w, m, G, T, budget, value bits
    (128, 2, 128, 4, 1000, 100, 2), (128, 2, 128, 1, 700, 64, 2), (128, 2, 128, 8, 2050, 1, 2),
    (256, 3, 256, 2, 300, 129, 2), (128, 0, 192, 4, 513, 200, 2), (64, 1, 64, 2, 400, 65, 2),
    (128, 2, 128, 4, 300, 1000, 2), (128, 2, 128, 2, 900, 300, 4), (256, 3, 256, 1, 260, 70, 4),
    # the A-QJL layer groups' sketch sizes (k = 384, 512) at GQA 4
    (128, 0, 384, 4, 700, 90, 2), (128, 0, 512, 4, 400, 50, 4),
    # contexts past the select kernel's LDS capacity (32768 keys): keys in place of the scores
    (128, 2, 128, 1, 32769, 3000, 2), (128, 2, 128, 2, 40000, 500, 2),
]


@pytest.mark.parametrize("d,w,m,G,T,budget,vb", CASES)
def test_topk_selection_and_decode(d, w, m, G, T, budget, vb):
    run_topk(d, w, m, G, T, budget, vb)


def run_topk(d, w, m, G, T, budget, vb, side_f16=False):
    torch, dev = torch_dev()
    say("top-k", d, w, m, G, T, budget, vb, "half side" if side_f16 else "")
    B, Hkv = 2, 2
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=6)
    cfg = cfg_of(hl, vb, side_f16)
    layer = device_layer(hl)
    rng = np.random.default_rng(d + T + budget)
    ks = [rng.standard_normal((T, d)).astype(np.float32) for _ in range(B * Hkv)]
    vs = [(rng.standard_normal((T, d)) * 2).astype(np.float32) for _ in range(B * Hkv)]
    cache, refs = _upload_oracle_cache(hl, cfg, ks, vs, vb, capacity=T + 3)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    qd = torch.from_numpy(q).to(dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    K = min(budget, T)
    sel = torch.full((B * Hkv, K), -1, dtype=torch.int32, device=dev)
    out = aqkv.decode_attention_topk(cfg, layer, cache, B, Hq, Hkv, T, qd, q_rot, q_sk, budget, selected=sel)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    worst = 0.0
    swapped = 0
    for s in range(B * Hkv):
        b, h = divmod(s, Hkv)
        qh = q[b, h * G:(h + 1) * G]
        gs = sel[s]
        assert np.all(np.diff(gs) > 0) and gs[0] >= 0 and gs[-1] < T
        osel, cos = oatt.select_top_k(qh, refs[s][0], hl.rotation, hl.sketch, hl.centroids, w, budget)
        thr = np.sort(cos)[::-1][K - 1]
        tol = 2e-3 * np.sqrt(np.mean(cos ** 2))
        diff = np.setxor1d(gs, osel)
        assert np.all(np.abs(cos[diff] - thr) <= tol), (diff, cos[diff], thr)
        swapped += diff.size // 2
        # the output over the GPU's chosen rows
        sub_k = tuple(np.asarray(a)[gs] for a in refs[s][0])
        sub_v = tuple(np.asarray(a)[gs] for a in refs[s][1])
        _, o_ref = oatt.decode_slot(qh, sub_k, sub_v, hl.rotation, hl.sketch, hl.centroids, w)
        worst = max(worst, float(np.max(np.abs(out[b, h * G:(h + 1) * G] - o_ref))))
    say(f"out err {worst:.2e}, near-tie swaps {swapped}")
    assert worst <= OUT_ATOL
    if K == T:
        assert swapped == 0


def test_topk_empty_context():
    torch, dev = torch_dev()
    d, w, m, G = 128, 2, 128, 2
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, 1, 64)
    q = torch.randn((1, G, d), device=dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, q)
    out = aqkv.decode_attention_topk(cfg, layer, cache, 1, G, 1, 0, q, q_rot, q_sk, 16)
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_topk_many_equal_keys():
    """Every cached key the same: all cosines tie, so the chosen rows are the first
    `budget` tokens (ties go to the lower token).  More keys share the top-digit bin
    than the select kernel collects as candidates, so this takes its full-pass route."""
    torch, dev = torch_dev()
    d, w, m, G, T, budget = 128, 2, 128, 2, 5000, 300
    B, Hkv = 1, 2
    hl = host_layer(d, w, m, layer=2)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    rng = np.random.default_rng(17)
    ks = [np.tile(rng.standard_normal((1, d)).astype(np.float32), (T, 1)) for _ in range(B * Hkv)]
    vs = [rng.standard_normal((T, d)).astype(np.float32) for _ in range(B * Hkv)]
    cache, refs = _upload_oracle_cache(hl, cfg, ks, vs, 2, capacity=T)
    q = rng.standard_normal((B, Hkv * G, d)).astype(np.float32)
    qd = torch.from_numpy(q).to(dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    sel = torch.full((B * Hkv, budget), -1, dtype=torch.int32, device=dev)
    out = aqkv.decode_attention_topk(cfg, layer, cache, B, Hkv * G, Hkv, T, qd, q_rot, q_sk, budget, selected=sel)
    torch.cuda.synchronize()
    sel, out = sel.cpu().numpy(), out.cpu().numpy()
    for s in range(B * Hkv):
        np.testing.assert_array_equal(sel[s], np.arange(budget))
        qh = q[0, s * G:(s + 1) * G]
        osel, _ = oatt.select_top_k(qh, refs[s][0], hl.rotation, hl.sketch, hl.centroids, w, budget)
        np.testing.assert_array_equal(np.sort(osel), np.arange(budget))
        sub_k = tuple(np.asarray(a)[sel[s]] for a in refs[s][0])
        sub_v = tuple(np.asarray(a)[sel[s]] for a in refs[s][1])
        _, o_ref = oatt.decode_slot(qh, sub_k, sub_v, hl.rotation, hl.sketch, hl.centroids, w)
        assert np.max(np.abs(out[0, s * G:(s + 1) * G] - o_ref)) <= OUT_ATOL


# ------------------------------------------------------ block-record selection

BLOCK_CASES = [
    # d, w, m, G, T, budget, value bits, half side information
    (128, 2, 128, 4, 1000, 128, 2, False), (128, 0, 512, 4, 4096, 512, 2, False),
    (128, 0, 384, 4, 700, 90, 2, False), (256, 3, 256, 2, 300, 129, 2, False),
    (128, 2, 128, 8, 2050, 1, 2, False), (128, 2, 128, 2, 900, 10 ** 5, 2, False),
    (64, 1, 64, 2, 400, 65, 4, False), (256, 2, 256, 2, 300, 129, 2, True),
]


@pytest.mark.parametrize("d,w,m,G,T,budget,vb,sf", BLOCK_CASES)
def test_topk_blocks_selection_and_decode(d, w, m, G, T, budget, vb, sf):
    torch, dev = torch_dev()
    say("top-k blocks", d, w, m, G, T, budget, vb, "half side" if sf else "")
    B, Hkv = 2, 2
    Hq = Hkv * G
    hl = host_layer(d, w, m, layer=6)
    cfg = cfg_of(hl, vb, sf)
    layer = device_layer(hl)
    rng = np.random.default_rng(d + T + budget + 1)
    ks = [rng.standard_normal((T, d)).astype(np.float32) for _ in range(B * Hkv)]
    vs = [(rng.standard_normal((T, d)) * 2).astype(np.float32) for _ in range(B * Hkv)]
    cache, refs = _upload_oracle_cache(hl, cfg, ks, vs, vb, capacity=T + 3)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    qd = torch.from_numpy(q).to(dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, qd)
    n_blk = (T + 31) // 32
    nb = max(1, min((budget + 31) // 32, n_blk))
    sel = torch.full((B * Hkv, nb), -1, dtype=torch.int32, device=dev)
    out = aqkv.decode_attention_topk_blocks(cfg, layer, cache, B, Hq, Hkv, T, qd, q_rot, q_sk, budget, selected=sel)
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    worst, swapped = 0.0, 0
    for s in range(B * Hkv):
        b, h = divmod(s, Hkv)
        qh = q[b, h * G:(h + 1) * G]
        gs = sel[s]
        assert np.all(np.diff(gs) > 0) and gs[0] >= 0 and gs[-1] < n_blk
        oblk, rank = oatt.select_top_k_blocks(qh, refs[s][0], hl.rotation, hl.sketch, hl.centroids, w, budget)
        thr = np.sort(rank)[::-1][nb - 1]
        tol = 2e-3 * np.sqrt(np.mean(rank ** 2))
        diff = np.setxor1d(gs, oblk)
        assert np.all(np.abs(rank[diff] - thr) <= tol), (diff, rank[diff], thr)
        swapped += diff.size // 2
        # the output over every row of the GPU's chosen blocks
        rows = np.array([t for blk in gs for t in range(32 * blk, min(32 * blk + 32, T))])
        sub_k = tuple(np.asarray(a)[rows] for a in refs[s][0])
        sub_v = tuple(np.asarray(a)[rows] for a in refs[s][1])
        _, o_ref = oatt.decode_slot(qh, sub_k, sub_v, hl.rotation, hl.sketch, hl.centroids, w)
        worst = max(worst, float(np.max(np.abs(out[b, h * G:(h + 1) * G] - o_ref))))
    say(f"out err {worst:.2e}, near-tie swaps {swapped}")
    assert worst <= OUT_ATOL
    if nb == n_blk:
        assert swapped == 0


def test_topk_blocks_empty_context():
    torch, dev = torch_dev()
    d, w, m, G = 128, 2, 128, 2
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    cache = aqkv.Cache.allocate(cfg, 1, 64)
    q = torch.randn((1, G, d), device=dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, q)
    out = aqkv.decode_attention_topk_blocks(cfg, layer, cache, 1, G, 1, 0, q, q_rot, q_sk, 16)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
