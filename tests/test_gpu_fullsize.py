"""GPU parity at the full sizes of the pages' decode workloads, in the launch
configuration bench.py times: its Path object (layer operands prepared once,
the value quantiser on a second stream beside the key kernel, split-K decode
and combine) runs one step, then outputs the oracle can compute one by one
are sampled and checked.

Samples per workload: in three KV slots (the first, the last, one drawn) the
rows of three 32-token records (the first, the last, one drawn) -- key codes
and sign bits bit-exact outside the 1e-5 decision window, norms to fp32
rounding, value codes, scales and minima bit-exact; for two query heads the
attention output over the whole context (and the step's score output where
the workload asks for it) against the oracle's decode of the slot's stored
planes, within 2e-3 absolute (scores 1e-3 relative)."""
import zlib

import numpy as np
import pytest

import bench
from kv_cache_compression_quantize_amd import inputs
from oracle import attention as oatt
from oracle import layout as olay

from gpu_helpers import (OUT_ATOL, SCORE_RTOL, compare_keys, host_layer, oracle_rows, read_planes, say,
                         score_err, torch_dev)

pytestmark = pytest.mark.gpu

CASES = [
    ("single_head_d128_t1k", 0),
    ("llama2_7b_layer_mha32_t32k", 0),
    ("llama3_8b_layer_gqa32x8_b8_t128k", 0),
    ("d256_gqa32x16_b4_t64k", 0),
    # one layer of every A-QJL group: sketch k = 512, 384, 256, 192
    ("aqjl_32layer_gqa32x8_b16_t32k", 0),
    ("aqjl_32layer_gqa32x8_b16_t32k", 8),
    ("aqjl_32layer_gqa32x8_b16_t32k", 16),
    ("aqjl_32layer_gqa32x8_b16_t32k", 31),
]


def _slot_input(w, layer, b, h, tensor):
    """The slot's tensor exactly as the step received it (bf16-rounded for bf16 workloads)."""
    x = inputs.kv_slot(w, layer, b, h, tensor)
    return inputs.bf16_bits_to_f32(inputs.to_bf16_bits(x)) if w.dtype == "bf16" else x


@pytest.mark.parametrize("name,layer", CASES)
def test_full_size_step_against_oracle_samples(name, layer):
    torch, dev = torch_dev()
    w = inputs.WORKLOADS[name]
    d, m, T = w.head_dim, w.sketch_dim(layer), w.context
    G = w.n_q_heads // w.n_kv_heads
    say("full size", name, "layer", layer, "slots", w.n_slots, "context", T)
    path = bench.Path(w, layer, "qr")
    path.step()
    torch.cuda.synchronize()
    hl = host_layer(d, w.mse_bits, m, layer=layer)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + layer)
    n_slots = w.n_slots
    slots = sorted({0, n_slots - 1, int(rng.integers(n_slots))})
    n_rec = T // 32
    recs = sorted({0, n_rec - 1, int(rng.integers(n_rec))})
    win = mis_win = 0
    for s in slots:
        b, h = divmod(s, w.n_kv_heads)
        xk = _slot_input(w, layer, b, h, "k")
        xv = _slot_input(w, layer, b, h, "v")
        for r in recs:
            t0, t1 = 32 * r, 32 * r + 32
            gpu = read_planes(path.cache, s, t0, t1)
            qk, kr, vt, _ = oracle_rows(hl, xk[t0:t1], xv[t0:t1], w.value_bits)
            par = compare_keys(hl, xk[t0:t1], qk, gpu)
            assert par.idx_mismatch_outside == 0, (s, r, par)
            assert par.sign_mismatch_outside == 0, (s, r, par)
            win += par.idx_in_window
            mis_win += par.idx_mismatch_in_window
            np.testing.assert_allclose(gpu["norm"], qk.norm, rtol=2e-6, atol=0)
            vc, vs, vm = vt
            np.testing.assert_array_equal(olay.unpack_value_codes(gpu["vcodes"], 32, d, w.value_bits), vc)
            np.testing.assert_array_equal(gpu["vscale"].view(np.uint32), vs.view(np.uint32))
            np.testing.assert_array_equal(gpu["vmin"].view(np.uint32), vm.view(np.uint32))
    say(f"rows: {len(slots)} slots x {len(recs)} records; index window {win} coords, {mis_win} differ inside")

    # attention of two query heads over the whole context, from the slot's stored planes
    q = path.x["q"].float().cpu().numpy()
    out = path.out.cpu().numpy()
    scores = path.scores.cpu().numpy() if path.scores is not None else None
    heads = sorted({(0, 0), (w.batch - 1, w.n_q_heads - 1)})
    for b, hq in heads:
        s = b * w.n_kv_heads + hq // G
        gpu = read_planes(path.cache, s, 0, T)
        idx = olay.unpack_code_planes(gpu["codes"], d, w.mse_bits) if w.mse_bits > 0 else None
        # pure QJL keys (no mse bits) store only the norm, which is then also gamma
        gamma = gpu["rnorm"] if w.mse_bits > 0 else gpu["norm"]
        rows = (idx, olay.unpack_bits(gpu["signs"], m), gpu["norm"].astype(np.float64), gamma.astype(np.float64))
        vals = (olay.unpack_value_codes(gpu["vcodes"], T, d, w.value_bits), gpu["vscale"], gpu["vmin"])
        s_ref, o_ref = oatt.decode_slot(q[b, hq][None], rows, vals, hl.rotation, hl.sketch, hl.centroids,
                                        w.mse_bits)
        err = float(np.max(np.abs(out[b, hq] - o_ref[0])))
        say(f"head ({b}, {hq}) of slot {s}: out err {err:.2e}")
        assert err <= OUT_ATOL
        if scores is not None:
            assert score_err(scores[b, hq][None], s_ref) <= SCORE_RTOL
