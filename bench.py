"""Benchmark of the compressed-KV hot path on one MI355X.

One step = the whole path over one batch of synthetic input, inputs already
resident in HBM: quantise every key (norm, rotation, Lloyd-Max index, residual
QJL signs, norms) and every value (min-max 2-bit groups) of the workload's
cache, prepare the queries (rotation + sketch), and decode attention for every
query head on the packed bits (split-K + combine).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  `value` is keys scored per second over the whole step
(B * Hq * T per step / step time).  The `roofline` object covers the kernel
that takes the most time in the step, measured with HIP events on the stream
the kernels are launched on; `decode` and `quantize` carry the per-stage
figures; `cpu_baseline` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attn: keys scored/s + HBM GB/s (%peak); quantize tokens/s"
DEFAULT_WORKLOAD = "llama2_7b_layer_mha32_t32k"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "i8": 5000.0, "fp32": 157.3}
WINDOW_TOKENS = 128   # recent-token window of the detail timing

KERNEL_SOURCES = {
    "decode": ["decode_fast.h", "decode_launch.hip", "decode_fast_d64.hip", "decode_fast_d128.hip",
               "decode_fast_d256.hip", "decode.hip"],
    "quantize_keys": ["quant_keys_mfma.hip"],
    "quantize_values": ["quant_values.hip"],
    "prepare_query": ["query.hip"],
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of a call's kernel sources with their comments removed (a comment
    edit does not change what the counters measured)."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "kv_cache_compression_quantize_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(text.encode())
    return h.hexdigest()[:16]


def build_layer(w, layer: int, rotation: str = "qr"):
    """Layer parameters built by the library itself (host builders), then copied to HBM."""
    import torch

    from kv_cache_compression_quantize_amd import aqkv, inputs
    d, m = w.head_dim, w.sketch_dim(layer)
    g, s = inputs.layer_gaussians(layer, d, m)
    dev = torch.device("cuda:0")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    if w.mse_bits > 0:
        pi = aqkv.build_rotation(g) if rotation == "qr" else aqkv.build_hadamard_rotation(g)
        c, t = aqkv.build_codebook(d, w.mse_bits)
        return aqkv.Layer(rotation=f(pi), sketch=f(s), centroids=f(c), boundaries=f(t))
    return aqkv.Layer(sketch=f(s))


def make_inputs(w, layer: int):
    import torch

    from kv_cache_compression_quantize_amd import inputs
    dev = torch.device("cuda:0")
    shape = (w.batch, w.n_kv_heads, w.context, w.head_dim)
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {}
    for name in ("k", "v"):
        t = torch.empty(shape, dtype=tdtype, device=dev)
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                x = inputs.kv_slot(w, layer, b, h, name)
                if w.dtype == "bf16":
                    t[b, h] = torch.from_numpy(inputs.to_bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)
                else:
                    t[b, h] = torch.from_numpy(x).to(dev)
        out[name] = t
    out["q"] = torch.from_numpy(inputs.queries(w, layer)).to(dev)
    return out


class Path:
    """All buffers for one layer of the workload and the four calls of one step."""

    def __init__(self, w, layer: int, rotation: str = "qr"):
        import torch

        from kv_cache_compression_quantize_amd import aqkv
        self.aqkv = aqkv
        self.w = w
        self.cfg = aqkv.config(w.head_dim, w.mse_bits, w.sketch_dim(layer), w.value_bits, w.value_group)
        self.layer = build_layer(w, layer, rotation)
        self.x = make_inputs(w, layer)
        dev = torch.device("cuda:0")
        self.cache = aqkv.Cache.allocate(self.cfg, w.n_slots, w.context)
        # the layer's key operands (Pi and S Pi^T as matrix-core operands) are built once per layer,
        # as a serving loop would; every step quantises against them
        self.kws = aqkv.prepare_key_operands(self.cfg, self.layer, device=dev)
        self.dws = torch.empty(aqkv.decode_workspace_bytes(self.cfg, w.batch, w.n_q_heads, w.n_kv_heads, w.context),
                               dtype=torch.uint8, device=dev)
        self.q_rot = (torch.empty((w.batch, w.n_q_heads, w.head_dim), device=dev) if w.mse_bits > 0 else None)
        self.q_sk = torch.empty((w.batch, w.n_q_heads, self.cfg.sketch_dim), device=dev)
        self.out = torch.empty((w.batch, w.n_q_heads, w.head_dim), device=dev)
        self.scores = (torch.empty((w.batch, w.n_q_heads, w.context), device=dev) if w.scores else None)
        # a full-precision recent-token window beside the compressed history (detail timing only)
        g = torch.Generator(device=dev)
        g.manual_seed(5)
        self.n_window = WINDOW_TOKENS
        self.win_k = torch.randn((w.batch, w.n_kv_heads, self.n_window, w.head_dim), generator=g,
                                 device=dev).to(torch.bfloat16)
        self.win_v = torch.randn((w.batch, w.n_kv_heads, self.n_window, w.head_dim), generator=g,
                                 device=dev).to(torch.bfloat16)
        self.q_f32 = self.x["q"].float().contiguous()
        # query-aware top-K preselection with QUOKA's budget rule min(4096, max(1024, T / 8)) (detail timing)
        self.budget = min(4096, max(1024, w.context // 8))
        self.tws = torch.empty(max(aqkv.decode_topk_workspace_bytes(self.cfg, w.batch, w.n_q_heads, w.n_kv_heads,
                                                                    w.context, self.budget), 256),
                               dtype=torch.uint8, device=dev)

    def quantize_keys(self):
        self.aqkv.quantize_keys_prepared(self.cfg, self.layer, self.x["k"], self.cache, self.kws)

    def prepare_key_operands(self):
        self.aqkv.prepare_key_operands(self.cfg, self.layer, self.kws)

    def quantize_values(self):
        self.aqkv.quantize_values(self.cfg, self.x["v"], self.cache, 0)

    def prepare_query(self):
        self.aqkv.prepare_query(self.cfg, self.layer, self.x["q"], self.q_rot, self.q_sk)

    def decode(self):
        w = self.w
        self.aqkv.decode_attention(self.cfg, self.layer, self.cache, w.batch, w.n_q_heads, w.n_kv_heads,
                                   w.context, self.q_rot, self.q_sk, None, self.scores, self.out, self.dws)

    def decode_window(self):
        w = self.w
        self.aqkv.decode_attention_window(self.cfg, self.layer, self.cache, w.batch, w.n_q_heads, w.n_kv_heads,
                                          w.context, self.q_f32, self.q_rot, self.q_sk, self.win_k, self.win_v,
                                          None, None, self.out, self.dws)

    def decode_topk(self):
        w = self.w
        self.aqkv.decode_attention_topk(self.cfg, self.layer, self.cache, w.batch, w.n_q_heads, w.n_kv_heads,
                                        w.context, self.q_f32, self.q_rot, self.q_sk, self.budget, None, None,
                                        self.out, self.tws)

    def step(self, ev=None):
        # one stream: values, keys, the query, then decode (split-K + combine).  A second stream
        # for the value quantiser beside the key kernel measured about 5 % faster per step, but
        # timing events between the calls take that overlap away again, and a profiler runs the
        # two streams one after the other: on one stream the key kernel's duration inside the
        # step, its duration under the profiler and its duration alone agree.  ev: an optional
        # pair of timing events recorded around the key quantiser.
        self.quantize_values()
        if ev:
            ev[0].record()
        self.quantize_keys()
        if ev:
            ev[1].record()
        self.prepare_query()
        self.decode()


def unit_costs(w, layer: int) -> dict:
    """Algorithmic bytes / flops per unit of each kernel (stated in the design notes)."""
    d, wb, m, vb = w.head_dim, w.mse_bits, w.sketch_dim(layer), w.value_bits
    in_bytes = 2 if w.dtype == "bf16" else 4
    key_row = wb * d // 8 + m // 8 + 4 + (4 if wb > 0 else 0)
    val_row = d * vb // 8 + 2 * 4 * (d // w.value_group)
    return {
        # decode: the compressed planes of one token of one kv head
        "decode_bytes_per_token_head": key_row + val_row,
        # key quantise: read the key, write its row; flops of Pi x, Pi^T c and S r
        "qkeys_bytes_per_key": d * in_bytes + key_row,
        "qkeys_flops_per_key": (4 * d * d + 2 * m * d) if wb > 0 else 2 * m * d,
        "qvals_bytes_per_value": d * in_bytes + val_row,
    }


def time_calls(path, reps: int) -> dict:
    """Average duration of each call launched on its own, HIP events on the launch
    stream.  A spin kernel (~0.4 ms) runs before each call's first event, so the GPU
    is still busy while the host issues the call and its closing event: the interval
    holds the call's own work, not the host's launch latency."""
    import torch
    stream = torch.cuda.current_stream()
    names = ["quantize_keys", "quantize_values", "prepare_query", "decode", "prepare_key_operands", "decode_window",
             "decode_topk"]
    ev = {n: [] for n in names}
    for _ in range(reps):
        for n in names:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(1_000_000)
            a.record(stream)
            getattr(path, n)()
            b.record(stream)
            ev[n].append((a, b))
    torch.cuda.synchronize()
    return {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}


def time_decode_cold(path, reps: int) -> float:
    """Decode duration with the last-level cache (256 MB Infinity Cache) cleared
    of the cache's bytes before every launch by reading a 1 GiB buffer: a read
    leaves only clean lines behind, so the timed kernel pays no write-backs of
    the flush itself.  HIP events around the decode only."""
    import torch
    stream = torch.cuda.current_stream()
    flush = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.empty((), dtype=torch.float32, device="cuda:0")
    ts = []
    for _ in range(reps):
        torch.sum(flush, dim=0, out=sink)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        path.decode()
        b.record(stream)
        ts.append((a, b))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ts]))


def counters_path(workload: str, layer: int) -> str:
    """The committed HBM counter summary of one workload and layer."""
    return os.path.join(ROOT, "profiles", f"hbm_counters_{workload}_layer{layer}.json")


def traffic_from_profiles(kernel: str, workload: str, layer: int):
    """HBM bytes per launch from the committed counter summary of this workload and
    layer, if it was taken on the current kernel source; else None."""
    p = counters_path(workload, layer)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


def cpu_baseline(w, layer: int, budget_s: float = 20.0) -> dict:
    """The oracle, as it stands, on whole slots of the same workload (one slot
    = one (batch, kv head) at full context with its query heads): quantise keys
    and values, then decode.  Reports keys scored per second."""
    from threadpoolctl import threadpool_info

    from kv_cache_compression_quantize_amd import inputs
    from oracle import attention as oatt
    from oracle import codebook as ocb
    from oracle import keys as okeys
    from oracle import rotation as orot
    from oracle import values as ovals
    d, m = w.head_dim, w.sketch_dim(layer)
    g, s = inputs.layer_gaussians(layer, d, m)
    pi = orot.rotation_fp32(g) if w.mse_bits > 0 else None
    s32 = s.astype(np.float32)
    c, t = ocb.codebook_fp32(d, w.mse_bits) if w.mse_bits > 0 else (np.zeros(1, np.float32), np.zeros(0, np.float32))
    q = inputs.queries(w, layer)
    G = w.n_q_heads // w.n_kv_heads
    slots, keys_scored, busy = 0, 0, 0.0
    while busy < budget_s and slots < w.n_slots:
        b, h = divmod(slots, w.n_kv_heads)
        k = inputs.kv_slot(w, layer, b, h, "k")
        v = inputs.kv_slot(w, layer, b, h, "v")
        t0 = time.perf_counter()
        qk = okeys.quantize_keys(k, pi, s32, c, t, w.mse_bits)
        vr = ovals.quantize_values(v, w.value_bits, w.value_group)
        rows = (qk.idx, qk.bits, qk.norm, qk.rnorm)
        oatt.decode_slot(q[b, h * G:(h + 1) * G], rows, vr, pi, s32, c, w.mse_bits, group=w.value_group)
        busy += time.perf_counter() - t0
        slots += 1
        keys_scored += G * w.context
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"value": keys_scored / busy, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{slots} of {w.n_slots} (batch, kv-head) slots at full context {w.context} with their "
                      f"{G} query heads: oracle key+value quantisation and decode, {busy:.1f} s of CPU work; "
                      f"numpy BLAS threads = {threads}, elementwise numpy single-threaded"}


# kernels of each call, as rocprofv3 names them (substring match)
KERNEL_NAMES = {
    "decode": ["decode_fast_kernel", "combine_kernel", "decode_kernel"],
    "quantize_keys": ["quantize_keys_resident_kernel", "quantize_keys_stream_kernel"],
    "quantize_values": ["quantize_values_kernel"],
}


def write_counters(fetch_csv: str, write_csv: str, out: str, workload: str, layer: int) -> dict:
    """The HBM counter summary (counters_path) from two rocprofv3 --pmc passes (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch) over `bench.py --calibrate-copy`: each
    counter is scaled by what it reads for the plain 1 GiB device copy (1 GiB
    fetched and 1 GiB written), and each call's HBM bytes per launch are the sum
    over its kernels of the mean per dispatch."""
    import collections
    import csv

    def means(path, counter):
        acc = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return acc

    fetch, write = means(fetch_csv, "FETCH_SIZE"), means(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    # the 1 GiB copy: FETCH_SIZE reads about half its bytes on this part, so the cut is a
    # quarter (the input set-up copies are a few MB)
    copy_f = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs if v > 0.25 * gib_kib]
    copy_w = [v for k, vs in write.items() if "copyBuffer" in k for v in vs if v > 0.25 * gib_kib]
    if not copy_f or not copy_w:
        raise SystemExit("no 1 GiB copy dispatch in the counter files (run bench.py with --calibrate-copy)")
    f_fetch = gib_kib / float(np.mean(copy_f))
    f_write = gib_kib / float(np.mean(copy_w))
    rec = {"workload": workload, "layer": layer,
           "calibration": {"copy_bytes": 1 << 30, "fetch_kib_read": float(np.mean(copy_f)),
                           "write_kib_read": float(np.mean(copy_w)), "fetch_factor": f_fetch,
                           "write_factor": f_write},
           "kernels": {}}
    for call, subs in KERNEL_NAMES.items():
        kb_f = sum(float(np.mean(v)) for k, v in fetch.items() if any(x in k for x in subs))
        kb_w = sum(float(np.mean(v)) for k, v in write.items() if any(x in k for x in subs))
        if kb_f == 0 and kb_w == 0:
            continue
        rec["kernels"][call] = {"source_hash": source_hash(call),
                                "fetch_bytes_per_launch": kb_f * 1024 * f_fetch,
                                "write_bytes_per_launch": kb_w * 1024 * f_write,
                                "hbm_bytes_per_launch": kb_f * 1024 * f_fetch + kb_w * 1024 * f_write}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true", help="skip per-call timing (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--rotation", choices=["qr", "hadamard"], default="qr",
                    help="the keys' rotation: Haar (QR of a Gaussian) or randomised Hadamard")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step captured once as a HIP graph instead of launching each call from Python "
                         "(measured no faster for these kernel sizes)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: write the workload's profiles/hbm_counters_*.json from two rocprofv3 "
                         "counter_collection.csv "
                         "files (FETCH_SIZE, WRITE_SIZE) of a --calibrate-copy run")
    args = ap.parse_args()
    if args.write_counters:
        print(json.dumps(write_counters(*args.write_counters, counters_path(args.workload, args.layer),
                                        args.workload, args.layer), indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU only (no multi-GPU form); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from kv_cache_compression_quantize_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    layer = args.layer
    log(f"workload {w.name}: setting up inputs")
    path = Path(w, layer, args.rotation)
    torch.cuda.synchronize()
    log("warmup")
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()
    run = path.step
    if args.graph:
        # the four calls captured once as a HIP graph: every replay launches the same kernels
        # on the same buffers, without the per-call host overhead between them
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            path.step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(max(args.warmup, 1)):
            run()
        torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # HIP events around the key quantiser (the step's largest call on the default workload) in
    # every timed step, on its launch stream (eager launches only: a replayed graph has no place
    # for them); created beforehand, read after the clock stops.
    in_step = None
    if not args.graph:
        in_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        if in_step is None:
            run()
        else:
            run(in_step[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = None
    if in_step is not None:
        step_ms = {"quantize_keys": float(np.mean([a.elapsed_time(b) for a, b in in_step]))}
    ms_per_step = elapsed / max(args.steps, 1) * 1e3
    G = w.n_q_heads // w.n_kv_heads
    keys_per_step = w.batch * w.n_q_heads * w.context
    value = keys_per_step / (ms_per_step / 1e3)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    rec = {"metric": METRIC, "value": value, "unit": "keys/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                      "context": w.context, "head_dim": w.head_dim, "mse_bits": w.mse_bits,
                      "sketch_dim": w.sketch_dim(layer), "value_bits": w.value_bits,
                      "value_group": w.value_group, "kv_dtype": w.dtype, "recipe": w.recipe,
                      "launch": "hip_graph" if args.graph else "eager", "rotation": args.rotation}}
    if step_ms is not None:
        rec["in_step_ms"] = step_ms
    if not args.no_detail:
        log("per-call timing")
        per = time_calls(path, reps=max(5, min(args.steps, 50)))
        # the largest call by its own duration; the roofline then takes that call's duration
        # inside the timed steps where it was measured there (the key quantiser), else its own
        live = dict(per)
        if step_ms is not None:
            live.update(step_ms)
        cold = time_decode_cold(path, reps=5)
        uc = unit_costs(w, layer)
        th = w.n_slots * w.context
        dec_bytes = uc["decode_bytes_per_token_head"] * th
        qk_bytes = uc["qkeys_bytes_per_key"] * th
        qk_flops = uc["qkeys_flops_per_key"] * th
        qv_bytes = uc["qvals_bytes_per_value"] * th
        rec["decode"] = {
            "ms": per["decode"], "ms_cold_llc": cold,
            "keys_scored_per_s": keys_per_step / (per["decode"] / 1e3),
            "kv_token_heads_per_s": th / (per["decode"] / 1e3),
            "GBps": dec_bytes / (per["decode"] / 1e3) / 1e9,
            "GBps_cold_llc": dec_bytes / (cold / 1e3) / 1e9,
            "pct_peak_hbm": 100 * dec_bytes / (per["decode"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "bytes_per_launch": dec_bytes}
        rec["quantize"] = {
            "keys_ms": per["quantize_keys"], "values_ms": per["quantize_values"],
            "tokens_per_s": w.batch * w.context / ((per["quantize_keys"] + per["quantize_values"]) / 1e3),
            "token_heads_per_s": th / ((per["quantize_keys"] + per["quantize_values"]) / 1e3),
            "keys_TFLOPs": qk_flops / (per["quantize_keys"] / 1e3) / 1e12,
            "keys_GBps": qk_bytes / (per["quantize_keys"] / 1e3) / 1e9,
            "values_GBps": qv_bytes / (per["quantize_values"] / 1e3) / 1e9}
        rec["decode_window"] = {"window_tokens": path.n_window, "ms": per["decode_window"],
                                "extra_ms_over_decode": per["decode_window"] - per["decode"]}
        rec["decode_topk"] = {"budget": path.budget, "ms": per["decode_topk"]}
        rec["prepare_query_ms"] = per["prepare_query"]
        rec["prepare_key_operands_ms_once_per_layer"] = per["prepare_key_operands"]
        dominant = max(["decode", "quantize_keys", "quantize_values"], key=lambda n: per[n])
        if dominant == "decode":
            ach = dec_bytes / (live["decode"] / 1e3) / 1e9
            rec["roofline"] = {"kernel": "decode_attention (decode + combine)", "bound": "hbm", "achieved": ach,
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                               "traffic": traffic_from_profiles("decode", w.name, layer)}
        elif dominant == "quantize_keys":
            ach = qk_flops / (live["quantize_keys"] / 1e3) / 1e12
            # the contraction runs on f16 matrix cores (split hi/lo operands): priced
            # against the dense f16 peak with the algorithmic flop count
            rec["roofline"] = {"kernel": "quantize_keys", "bound": "mfma", "achieved": ach,
                               "peak": MFMA_PEAK_TFLOPS["fp16"], "unit": "TFLOP/s",
                               "frac": ach / MFMA_PEAK_TFLOPS["fp16"],
                               "traffic": traffic_from_profiles("quantize_keys", w.name, layer)}
        else:
            ach = qv_bytes / (live["quantize_values"] / 1e3) / 1e9
            rec["roofline"] = {"kernel": "quantize_values", "bound": "hbm", "achieved": ach,
                               "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS,
                               "traffic": traffic_from_profiles("quantize_values", w.name, layer)}
        rec["roofline"]["launch_ms"] = live[dominant]
        rec["roofline"]["timing"] = ("HIP events around the call in every timed step"
                                     if step_ms is not None and dominant in step_ms
                                     else "HIP events around isolated calls")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(w, layer)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
