"""The allocation-free decode entry point (aqkv_decode_attention_noalloc),
called through the C ABI: its split partials live in the library's static
device scratch, and its outputs equal those of aqkv_decode_attention with a
caller workspace, bit for bit (the same kernels run), on two calls in a row,
the second smaller than the first, then on another codec."""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv

from gpu_helpers import cfg_of, device_layer, host_layer, say, to_device_kv, torch_dev

pytestmark = pytest.mark.gpu


def _cache_and_query(d, w, m, B, Hkv, G, T, seed):
    torch, dev = torch_dev()
    hl = host_layer(d, w, m, layer=7)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    cache = aqkv.Cache.allocate(cfg, B * Hkv, T)
    aqkv.quantize_keys(cfg, layer, to_device_kv(k, "fp32"), cache)
    aqkv.quantize_values(cfg, to_device_kv(v, "fp32"), cache)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(dev)
    q_rot, q_sk = aqkv.prepare_query(cfg, layer, q)
    return cfg, layer, cache, q_rot, q_sk


@pytest.mark.parametrize("calls", [[(128, 2, 128, 2, 4, 4, 5000), (128, 2, 128, 1, 2, 2, 700),
                                    (128, 0, 384, 2, 2, 4, 1500)]])
def test_noalloc_decode_equals_workspace_decode(calls):
    torch, dev = torch_dev()
    assert aqkv.decode_static_scratch_bytes() == 8 << 20
    for d, w, m, B, Hkv, G, T in calls:
        say("noalloc decode", d, w, m, B, Hkv, G, T)
        cfg, layer, cache, q_rot, q_sk = _cache_and_query(d, w, m, B, Hkv, G, T, seed=T + m)
        Hq = Hkv * G
        assert aqkv.decode_workspace_bytes(cfg, B, Hq, Hkv, T) <= aqkv.decode_static_scratch_bytes()
        ref_scores = torch.empty((B, Hq, T), device=dev)
        ref = aqkv.decode_attention(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, scores=ref_scores)
        out = torch.full((B, Hq, d), float("nan"), device=dev)
        scores = torch.full((B, Hq, T), float("nan"), device=dev)
        aqkv.decode_attention_noalloc(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, out, scores=scores)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(scores, ref_scores)
        # a second call right after, into fresh outputs: the same bits again
        out2 = torch.empty_like(out)
        aqkv.decode_attention_noalloc(cfg, layer, cache, B, Hq, Hkv, T, q_rot, q_sk, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_refuses_more_than_the_scratch():
    torch, dev = torch_dev()
    cfg = aqkv.config(128, 2, 128)
    B, Hq, Hkv, T = 4096, 64, 8, 4096     # partials of 32768 slots x 8 heads: far past 8 MiB
    assert aqkv.decode_workspace_bytes(cfg, B, Hq, Hkv, T) > aqkv.decode_static_scratch_bytes()
    cache = aqkv.CacheDesc(0x10000, B * Hkv, T)
    layer = aqkv.LayerParams(0x10000, 0x10000, 0x10000, 0x10000)
    st = aqkv.lib().aqkv_decode_attention_noalloc(cfg, layer, cache, B, Hq, Hkv, T, 0x10000, 0x10000, 0.1, None,
                                                  0x10000, None)
    assert st == -9
