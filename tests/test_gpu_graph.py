"""The whole hot path (key and value quantisation, query preparation, decode)
captured once in a HIP graph and replayed: every replay, with eager work and
synchronisations between replays, gives the eager results byte for byte."""
import numpy as np
import pytest

from kv_cache_compression_quantize_amd import aqkv, inputs

from gpu_helpers import cfg_of, device_layer, host_layer, say, to_device_kv, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("forked", [False, True])
def test_step_graph_replays_match_eager(forked):
    torch, dev = torch_dev()
    say("graph replay of the step, values and query on a second stream" if forked else "graph replay of the step")
    d, w, m = 128, 2, 128
    B, Hkv, G, T = 2, 2, 4, 1000
    rng = np.random.default_rng(21)
    f32 = lambda *s: rng.standard_normal(s).astype(np.float32)
    bf = lambda x: inputs.bf16_bits_to_f32(inputs.to_bf16_bits(x))
    hl = host_layer(d, w, m)
    cfg = cfg_of(hl)
    layer = device_layer(hl)
    kd, vd = to_device_kv(bf(f32(B, Hkv, T, d)), "bf16"), to_device_kv(bf(f32(B, Hkv, T, d)), "bf16")
    q = torch.from_numpy(f32(B, Hkv * G, d)).to(dev)
    kws = aqkv.prepare_key_operands(cfg, layer, device=dev)
    dws = torch.empty(max(aqkv.decode_workspace_bytes(cfg, B, Hkv * G, Hkv, T), 256), dtype=torch.uint8, device=dev)

    def buffers():
        cache = aqkv.Cache.allocate(cfg, B * Hkv, T)
        cache.blocks.zero_()
        return dict(cache=cache, q_rot=torch.zeros((B, Hkv * G, d), device=dev),
                    q_sk=torch.zeros((B, Hkv * G, m), device=dev), out=torch.zeros((B, Hkv * G, d), device=dev),
                    scores=torch.zeros((B, Hkv * G, T), device=dev))

    side = torch.cuda.Stream(device=dev)

    def step(b):
        cur = torch.cuda.current_stream()
        if forked:
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                aqkv.quantize_values(cfg, vd, b["cache"])
                aqkv.prepare_query(cfg, layer, q, b["q_rot"], b["q_sk"])
        aqkv.quantize_keys_prepared(cfg, layer, kd, b["cache"], kws)
        if forked:
            cur.wait_stream(side)
        else:
            aqkv.quantize_values(cfg, vd, b["cache"])
            aqkv.prepare_query(cfg, layer, q, b["q_rot"], b["q_sk"])
        aqkv.decode_attention(cfg, layer, b["cache"], B, Hkv * G, Hkv, T, b["q_rot"], b["q_sk"], None,
                              b["scores"], b["out"], dws)

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()

    gb = buffers()
    step(gb)                      # first launches outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(gb)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (gb["out"], gb["scores"], gb["q_rot"], gb["q_sk"]):
            t.fill_(float(rep + 7))
        gb["cache"].blocks.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gb["cache"].blocks, ref["cache"].blocks), rep
        for name in ("q_rot", "q_sk", "scores", "out"):
            assert torch.equal(gb[name], ref[name]), (rep, name)
