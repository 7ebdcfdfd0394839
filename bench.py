"""Benchmark of the compressed-KV hot path on one MI355X.

One step = the whole path over one batch of synthetic input, inputs already
resident in HBM, for every layer of the workload: quantise every key (norm,
rotation, Lloyd-Max index, residual QJL signs, norms; pure QJL signs of S x
for the A-QJL stack) and every value (min-max groups) of the layer's cache,
prepare the queries (rotation + sketch), and decode attention for every query
head on the packed bits (split-K + combine).  The default workload is the
largest one: the 32-layer A-QJL stack (16 x 8 KV heads x 32768 tokens per
layer, sketch size k = 512 / 384 / 256 / 192 per 8-layer group).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layer L] [--no-cpu-baseline]

Prints ONE JSON line.  `value` is keys scored per second over the whole step
(B * Hq * T * layers per step / step time).  The `roofline` object covers the
call that takes the most time in the step (summed over the layers), measured
with HIP events around it on its launch stream in every timed step; `decode`
and `quantize` carry the per-stage figures, `read_stream` the plain HBM read
ceiling measured in the same run, `cpu_baseline` the CPU oracle on a bounded
sample.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode attn: keys scored/s + HBM GB/s (%peak); quantize tokens/s"
DEFAULT_WORKLOAD = "aqjl_32layer_gqa32x8_b16_t32k"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "i8": 5000.0, "fp32": 157.3}
WINDOW_TOKENS = 128   # recent-token window of the detail timing
CALLS = ("quantize_values", "quantize_keys", "prepare_query", "decode")
# the arithmetic the path computes in (the pages' fp32 reference arithmetic, reached through
# split operands on the matrix cores)
ARITHMETIC = ("keys: f16 hi/lo split products on matrix cores, fp32 accumulate (fp32-accurate); "
              "decode scores: int8 matrix products of the packed bits with a 15-bit fixed-point query "
              "(int8 hi/lo), int32 accumulate; values: f16 matrix products (p*scale split hi/lo, codes exact), "
              "fp32 accumulate; softmax, norms, value codec in fp32")

KERNEL_SOURCES = {
    "decode": ["decode_fast.h", "decode_launch.hip", "decode_fast_d64.hip", "decode_fast_d128.hip",
               "decode_fast_d256.hip", "decode.hip"],
    "quantize_keys": ["quant_keys_mfma.hip", "quant_keys_qjl.hip"],
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
    """K and V of one layer drawn on the GPU by the counter-based generator (the
    host can regenerate any slot of them), queries from the host."""
    import torch

    from kv_cache_compression_quantize_amd import inputs
    dev = torch.device("cuda:0")
    return {"k": inputs.kv_device(w, layer, "k", device=dev), "v": inputs.kv_device(w, layer, "v", device=dev),
            "q": torch.from_numpy(inputs.queries(w, layer)).to(dev)}


class Path:
    """All buffers for one layer of the workload and the four calls of one step
    (aux: also the buffers of the window and top-K detail calls)."""

    def __init__(self, w, layer: int, rotation: str = "qr", aux: bool = True, side_f16: bool = False,
                 topk_budget=None):
        import torch

        from kv_cache_compression_quantize_amd import aqkv
        self.aqkv = aqkv
        self.w = w
        self.layer_index = layer
        self.cfg = aqkv.config(w.head_dim, w.mse_bits, w.sketch_dim(layer), w.value_bits, w.value_group, side_f16)
        self.layer = build_layer(w, layer, rotation)
        self.x = make_inputs(w, layer)
        dev = torch.device("cuda:0")
        self.cache = aqkv.Cache.allocate(self.cfg, w.n_slots, w.context)
        # the layer's key operands (Pi and S Pi^T, or S, as matrix-core operands) are built once
        # per layer, as a serving loop would; every step quantises against them
        self.kws = aqkv.prepare_key_operands(self.cfg, self.layer, device=dev)
        self.dws = torch.empty(max(aqkv.decode_workspace_bytes(self.cfg, w.batch, w.n_q_heads, w.n_kv_heads,
                                                               w.context), 256), dtype=torch.uint8, device=dev)
        self.q_rot = (torch.empty((w.batch, w.n_q_heads, w.head_dim), device=dev) if w.mse_bits > 0 else None)
        self.q_sk = torch.empty((w.batch, w.n_q_heads, self.cfg.sketch_dim), device=dev)
        self.out = torch.empty((w.batch, w.n_q_heads, w.head_dim), device=dev)
        self.scores = (torch.empty((w.batch, w.n_q_heads, w.context), device=dev) if w.scores else None)
        self.aux = aux
        if aux:
            # a full-precision recent-token window beside the compressed history (detail timing only)
            g = torch.Generator(device=dev)
            g.manual_seed(5)
            self.n_window = WINDOW_TOKENS
            self.win_k = torch.randn((w.batch, w.n_kv_heads, self.n_window, w.head_dim), generator=g,
                                     device=dev).to(torch.bfloat16)
            self.win_v = torch.randn((w.batch, w.n_kv_heads, self.n_window, w.head_dim), generator=g,
                                     device=dev).to(torch.bfloat16)
            self.q_f32 = self.x["q"].float().contiguous()
            # query-aware top-K preselection with QUOKA's budget rule min(4096, max(1024, T / 8))
            self.budget = topk_budget or min(4096, max(1024, w.context // 8))
            self.tws = torch.empty(max(aqkv.decode_topk_workspace_bytes(self.cfg, w.batch, w.n_q_heads,
                                                                        w.n_kv_heads, w.context, self.budget), 256),
                                   dtype=torch.uint8, device=dev)
            self.bws = torch.empty(max(aqkv.decode_topk_blocks_workspace_bytes(
                self.cfg, w.batch, w.n_q_heads, w.n_kv_heads, w.context, self.budget), 256),
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

    def decode_topk_blocks(self):
        w = self.w
        self.aqkv.decode_attention_topk_blocks(self.cfg, self.layer, self.cache, w.batch, w.n_q_heads,
                                               w.n_kv_heads, w.context, self.q_f32, self.q_rot, self.q_sk,
                                               self.budget, None, None, self.out, self.bws)

    def step(self, ev=None):
        # one stream: values, keys, the query, then decode (split-K + combine).  A second stream
        # for the value quantiser beside the key kernel measured about 5 % faster per step, but
        # timing events between the calls take that overlap away again, and a profiler runs the
        # two streams one after the other: on one stream each call's duration inside the step,
        # under the profiler and alone agree.  ev: optional {call: (start, end)} timing events
        # recorded around the calls.
        for name in CALLS:
            if ev:
                ev[name][0].record()
            getattr(self, name)()
            if ev:
                ev[name][1].record()


class Stack:
    """The paths of the workload's layers; one step runs every layer in order."""

    def __init__(self, w, layers, rotation: str = "qr", aux_layers=(), side_f16: bool = False, topk_budget=None):
        self.w = w
        self.paths = []
        for layer in layers:
            self.paths.append(Path(w, layer, rotation, aux=layer in aux_layers, side_f16=side_f16,
                                   topk_budget=topk_budget))

    def step(self, evs=None):
        for i, p in enumerate(self.paths):
            p.step(evs[i] if evs else None)


def unit_costs(w, layer: int, side_f16: bool = False) -> dict:
    """Algorithmic bytes / flops per unit of each kernel (stated in the design notes); side_f16:
    norms, scales and minima stored as halves."""
    d, wb, m, vb = w.head_dim, w.mse_bits, w.sketch_dim(layer), w.value_bits
    in_bytes = 2 if w.dtype == "bf16" else 4
    e = 2 if side_f16 else 4
    key_row = wb * d // 8 + m // 8 + e + (e if wb > 0 else 0)
    val_row = d * vb // 8 + 2 * e * (d // w.value_group)
    return {
        # decode: the compressed planes of one token of one kv head
        "decode_bytes_per_token_head": key_row + val_row,
        # key quantise: read the key, write its row; flops of Pi x, Pi^T c and S r
        "qkeys_bytes_per_key": d * in_bytes + key_row,
        "qkeys_flops_per_key": (4 * d * d + 2 * m * d) if wb > 0 else 2 * m * d,
        "qvals_bytes_per_value": d * in_bytes + val_row,
    }


def compression_ratio(w, layers, side_f16: bool = False) -> float:
    """bf16 K + V bytes over compressed bytes, summed over the layers."""
    uc = [unit_costs(w, layer, side_f16)["decode_bytes_per_token_head"] for layer in layers]
    return 4 * w.head_dim * len(layers) / float(sum(uc))


def representative_layers(w) -> list:
    """One layer per distinct codec setting of the workload (A-QJL: the first layer of each group)."""
    seen, out = set(), []
    for layer in range(w.layers):
        if w.sketch_dim(layer) not in seen:
            seen.add(w.sketch_dim(layer))
            out.append(layer)
    return out


def time_calls(path, reps: int, names=None) -> dict:
    """Average duration of each call launched on its own, HIP events on the launch
    stream.  A spin kernel (~0.4 ms) runs before each call's first event, so the GPU
    is still busy while the host issues the call and its closing event: the interval
    holds the call's own work, not the host's launch latency."""
    import torch
    stream = torch.cuda.current_stream()
    names = names or ["quantize_keys", "quantize_values", "prepare_query", "decode", "prepare_key_operands",
                      "decode_window", "decode_topk", "decode_topk_blocks"]
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


def read_stream_ceiling(reps: int = 10, gib: int = 4) -> dict:
    """The plain HBM read rate of the library's read-stream helper over a buffer far
    larger than the last-level cache (best and median of reps, HIP events)."""
    import torch

    from kv_cache_compression_quantize_amd import aqkv
    stream = torch.cuda.current_stream()
    buf = torch.ones(gib * (1 << 30) // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    aqkv.read_stream(buf, sink)
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        aqkv.read_stream(buf, sink)
        b.record(stream)
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ts])
    nbytes = buf.numel() * 4
    del buf
    return {"bytes": nbytes, "GBps_best": nbytes / (ms.min() / 1e3) / 1e9,
            "GBps_median": nbytes / (np.median(ms) / 1e3) / 1e9}


def counters_path(workload: str, layer) -> str:
    """The committed HBM counter summary of one workload and layer ("all": the whole stack)."""
    tag = "all_layers" if layer == "all" else f"layer{layer}"
    return os.path.join(ROOT, "profiles", f"hbm_counters_{workload}_{tag}.json")


def traffic_from_profiles(kernel: str, workload: str, layer):
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


def _oracle_slot(w, layer, b, h, params):
    """Oracle key + value quantisation and decode of one slot (its query heads); seconds."""
    from kv_cache_compression_quantize_amd import inputs
    from oracle import attention as oatt
    from oracle import keys as okeys
    from oracle import values as ovals
    pi, s32, c, t, q = params
    G = w.n_q_heads // w.n_kv_heads
    k = inputs.kv_slot(w, layer, b, h, "k")
    v = inputs.kv_slot(w, layer, b, h, "v")
    t0 = time.perf_counter()
    qk = okeys.quantize_keys(k, pi, s32, c, t, w.mse_bits)
    vr = ovals.quantize_values(v, w.value_bits, w.value_group)
    rows = (qk.idx, qk.bits, qk.norm, qk.rnorm)
    oatt.decode_slot(q[b, h * G:(h + 1) * G], rows, vr, pi, s32, c, w.mse_bits, group=w.value_group)
    return time.perf_counter() - t0


def cpu_baseline(w, layers, budget_s: float = 16.0) -> dict:
    """The oracle, as it stands, on whole slots of the same workload (one slot =
    one (batch, kv head) at full context with its query heads): quantise keys
    and values, then decode; one codec setting per representative layer.  Run
    with numpy's BLAS on every host core this process may use, then on one
    thread; keys scored per second at the full core count, and the full
    configuration's time extrapolated from the per-slot times."""
    from threadpoolctl import threadpool_limits

    from kv_cache_compression_quantize_amd import inputs
    from oracle import codebook as ocb
    from oracle import rotation as orot
    cores = len(os.sched_getaffinity(0))
    G = w.n_q_heads // w.n_kv_heads
    reps = representative_layers(w) if w.layers > 1 else list(layers)
    params = {}
    for layer in reps:
        d, m = w.head_dim, w.sketch_dim(layer)
        g, s = inputs.layer_gaussians(layer, d, m)
        pi = orot.rotation_fp32(g) if w.mse_bits > 0 else None
        c, t = (ocb.codebook_fp32(d, w.mse_bits) if w.mse_bits > 0
                else (np.zeros(1, np.float32), np.zeros(0, np.float32)))
        params[layer] = (pi, s.astype(np.float32), c, t, inputs.queries(w, layer))
    per_slot = {}
    slots_done, busy = 0, 0.0
    with threadpool_limits(cores):
        for layer in reps:
            ts = []
            while sum(ts) < budget_s / len(reps) and len(ts) < w.n_slots:
                b, h = divmod(len(ts), w.n_kv_heads)
                ts.append(_oracle_slot(w, layer, b, h, params[layer]))
            per_slot[layer] = float(np.mean(ts))
            slots_done += len(ts)
            busy += sum(ts)
    one = {}
    with threadpool_limits(1):
        for layer in reps:
            one[layer] = _oracle_slot(w, layer, 0, 0, params[layer])
    # every layer of the workload takes its group's per-slot time
    group_of = {layer: max(r for r in reps if w.sketch_dim(r) == w.sketch_dim(layer)) for layer in layers}
    full_s = sum(per_slot[group_of[layer]] for layer in layers) * w.n_slots
    full_1 = sum(one[group_of[layer]] for layer in layers) * w.n_slots
    keys_full = w.batch * w.n_q_heads * w.context * len(layers)
    return {"value": keys_full / full_s, "unit": "keys/s", "cores": cores, "kind": "oracle",
            "sample": f"{slots_done} (batch, kv-head) slots of layers {reps} at full context {w.context} with their "
                      f"{G} query heads: oracle key+value quantisation and decode, {busy:.1f} s of CPU work with "
                      f"numpy BLAS on {cores} threads (elementwise numpy single-threaded); value = keys scored "
                      f"over the whole configuration / its time extrapolated from the per-slot times",
            "value_1_thread": keys_full / full_1,
            "extrapolated_full_config_s": full_s,
            "extrapolated_full_config_s_1_thread": full_1,
            "per_slot_s": {str(k): v for k, v in per_slot.items()},
            "per_slot_s_1_thread": {str(k): v for k, v in one.items()}}


CALIBRATION_COPIES = 3   # plain 1 GiB device copies after the timed steps (--calibrate-copy)

# kernels of each call, as rocprofv3 names them (substring match): (the alternatives one of
# which every launch of the call runs, the companions it runs beside it)
KERNEL_NAMES = {
    "decode": (["decode_fast_kernel", "::decode_kernel"], ["combine_kernel"]),
    "quantize_keys": (["quantize_keys_resident_kernel", "quantize_keys_stream_kernel", "quantize_keys_qjl_kernel"],
                      []),
    "quantize_values": (["quantize_values_kernel"], []),
}


def write_counters(fetch_csv: str, write_csv: str, out: str, workload: str, layer) -> dict:
    """The HBM counter summary (counters_path) from two rocprofv3 --pmc passes (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch) over `bench.py --calibrate-copy`: each
    counter is scaled by what it reads for the plain 1 GiB device copy (1 GiB
    fetched and 1 GiB written), and each call's HBM bytes per launch are the bytes
    of all its kernels' dispatches over the number of its launches (the dispatches
    of its main kernel, whichever variant and template arguments a launch runs: for
    a whole stack, the mean over its layers)."""
    import csv

    def means(path, counter):
        acc = collections.defaultdict(list)
        copies = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
                    if "copyBuffer" in r["Kernel_Name"]:
                        copies.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        return acc, copies

    (fetch, copies_f), (write, copies_w) = means(fetch_csv, "FETCH_SIZE"), means(write_csv, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    # the 1 GiB copies of --calibrate-copy are the run's last CALIBRATION_COPIES copy dispatches
    # (the input set-up copies come before the timed steps and can be as large)
    copy_f = [v for _, v in sorted(copies_f)[-CALIBRATION_COPIES:] if v > 0.25 * gib_kib]
    copy_w = [v for _, v in sorted(copies_w)[-CALIBRATION_COPIES:] if v > 0.25 * gib_kib]
    if len(copy_f) < CALIBRATION_COPIES or len(copy_w) < CALIBRATION_COPIES:
        raise SystemExit("no 1 GiB copy dispatch in the counter files (run bench.py with --calibrate-copy)")
    f_fetch = gib_kib / float(np.mean(copy_f))
    f_write = gib_kib / float(np.mean(copy_w))
    rec = {"workload": workload, "layer": layer,
           "calibration": {"copy_bytes": 1 << 30, "fetch_kib_read": float(np.mean(copy_f)),
                           "write_kib_read": float(np.mean(copy_w)), "fetch_factor": f_fetch,
                           "write_factor": f_write},
           "kernels": {}}

    def per_launch(table, main, extra):
        launches = sum(len(vs) for k, vs in table.items() if any(x in k for x in main))
        total = sum(sum(vs) for k, vs in table.items() if any(x in k for x in main + extra))
        return total / launches if launches else 0.0

    for call, (main, extra) in KERNEL_NAMES.items():
        kb_f = per_launch(fetch, main, extra)
        kb_w = per_launch(write, main, extra)
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
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200 for one layer, 50 for a layer stack)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layer", type=int, default=None,
                    help="run one layer of a multi-layer workload (default: every layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true", help="skip the untimed detail legs (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--rotation", choices=["qr", "hadamard"], default="qr",
                    help="the keys' rotation: Haar (QR of a Gaussian) or randomised Hadamard")
    ap.add_argument("--topk-budget", type=int, default=None,
                    help="tokens the top-K detail legs keep per KV head (default: QUOKA's min(4096, max(1024, T/8)))")
    ap.add_argument("--side-f16", action="store_true",
                    help="store norms, value scales and minima as IEEE halves (the cache's half side-information option)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step captured once as a HIP graph instead of launching each call from Python")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: write the workload's profiles/hbm_counters_*.json from two rocprofv3 "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a --calibrate-copy run")
    args = ap.parse_args()
    from kv_cache_compression_quantize_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    layers = list(range(w.layers)) if args.layer is None else [args.layer]
    layer_tag = "all" if len(layers) > 1 else layers[0]
    if args.write_counters:
        print(json.dumps(write_counters(*args.write_counters, counters_path(args.workload, layer_tag),
                                        args.workload, layer_tag), indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU only (no multi-GPU form); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    steps = args.steps if args.steps is not None else (200 if len(layers) == 1 else 50)

    import torch
    reps = [layer for layer in representative_layers(w) if layer in layers] or layers[:1]
    log(f"workload {w.name}: setting up inputs for {len(layers)} layer(s)")
    t_setup = time.perf_counter()
    stack = Stack(w, layers, args.rotation, aux_layers=() if args.no_detail else reps, side_f16=args.side_f16,
                  topk_budget=args.topk_budget)
    torch.cuda.synchronize()
    log(f"set-up {time.perf_counter() - t_setup:.1f} s; warmup")
    for _ in range(args.warmup):
        stack.step()
    torch.cuda.synchronize()
    run = stack.step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            stack.step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(max(args.warmup, 1)):
            run()
        torch.cuda.synchronize()
    log(f"timing {steps} steps")
    # HIP events around every call of every layer in every timed step, on the launch stream
    # (eager launches only: a replayed graph has no place for them); created beforehand, read
    # after the clock stops
    evs = None
    if not args.graph:
        mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        evs = [[{n: mk() for n in CALLS} for _ in layers] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if evs is None:
            run()
        else:
            run(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / max(steps, 1) * 1e3
    keys_per_step = w.batch * w.n_q_heads * w.context * len(layers)
    value = keys_per_step / (ms_per_step / 1e3)
    # in-step means per (layer, call)
    in_step = None
    if evs is not None:
        in_step = [{n: float(np.mean([evs[i][j][n][0].elapsed_time(evs[i][j][n][1]) for i in range(steps)]))
                    for n in CALLS} for j in range(len(layers))]

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(CALIBRATION_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()

    th = w.n_slots * w.context                       # token-heads per layer
    ucs = [unit_costs(w, layer, args.side_f16) for layer in layers]
    dec_bytes = [u["decode_bytes_per_token_head"] * th for u in ucs]
    qk_flops = [u["qkeys_flops_per_key"] * th for u in ucs]
    qk_bytes = [u["qkeys_bytes_per_key"] * th for u in ucs]
    qv_bytes = [u["qvals_bytes_per_value"] * th for u in ucs]
    rec = {"metric": METRIC, "value": value, "unit": "keys/s", "n_gpus": 1, "steps": steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16x2+i8x2 mfma, fp32 accumulate", "data": "synthetic",
           "config": {"workload": w.name, "layers": len(layers) if len(layers) > 1 else f"layer {layers[0]}",
                      "batch": w.batch, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "context": w.context,
                      "head_dim": w.head_dim, "mse_bits": w.mse_bits,
                      "sketch_dim": sorted(set(w.sketch_dim(layer) for layer in layers)),
                      "value_bits": w.value_bits, "value_group": w.value_group, "kv_dtype": w.dtype,
                      "recipe": w.recipe, "launch": "hip_graph" if args.graph else "eager",
                      "rotation": args.rotation if w.mse_bits > 0 else None,
                      "compressed_bytes_per_step": int(sum(dec_bytes)),
                      "side_info": "f16" if args.side_f16 else "fp32",
                      "compression_ratio_vs_bf16": compression_ratio(w, layers, args.side_f16),
                      "arithmetic": ARITHMETIC}}
    if in_step is not None:
        tot = {n: sum(s[n] for s in in_step) for n in CALLS}
        rec["in_step_ms"] = tot
        rec["decode"] = {"all_layers_ms": tot["decode"], "bytes": int(sum(dec_bytes)),
                         "GBps": sum(dec_bytes) / (tot["decode"] / 1e3) / 1e9,
                         "pct_peak_hbm": 100 * sum(dec_bytes) / (tot["decode"] / 1e3) / 1e9 / HBM_PEAK_GBPS,
                         "keys_scored_per_s": keys_per_step / (tot["decode"] / 1e3),
                         "timing": "HIP events around each layer's decode call (decode + combine) in every "
                                   "timed step"}
        rec["quantize"] = {
            "keys_ms": tot["quantize_keys"], "values_ms": tot["quantize_values"],
            "tokens_per_s": w.batch * w.context * len(layers)
            / ((tot["quantize_keys"] + tot["quantize_values"]) / 1e3),
            "token_heads_per_s": th * len(layers) / ((tot["quantize_keys"] + tot["quantize_values"]) / 1e3),
            "keys_TFLOPs": sum(qk_flops) / (tot["quantize_keys"] / 1e3) / 1e12,
            "keys_GBps": sum(qk_bytes) / (tot["quantize_keys"] / 1e3) / 1e9,
            "values_GBps": sum(qv_bytes) / (tot["quantize_values"] / 1e3) / 1e9}
        # the roofline of the call with the largest share of the step, over every layer:
        # algorithmic work of all its launches / the sum of their in-step durations
        dominant = max(["decode", "quantize_keys", "quantize_values"], key=lambda n: tot[n])
        n_launch = len(layers)
        if dominant == "quantize_keys":
            ach = sum(qk_flops) / (tot[dominant] / 1e3) / 1e12
            rec["roofline"] = {"kernel": "quantize_keys", "bound": "mfma", "achieved": ach,
                               "peak": MFMA_PEAK_TFLOPS["fp16"], "unit": "TFLOP/s",
                               "frac": ach / MFMA_PEAK_TFLOPS["fp16"]}
            alg_bytes = sum(qk_bytes) / n_launch
        else:
            by = dec_bytes if dominant == "decode" else qv_bytes
            ach = sum(by) / (tot[dominant] / 1e3) / 1e9
            rec["roofline"] = {"kernel": dominant, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS,
                               "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS}
            alg_bytes = sum(by) / n_launch
        # the committed counters were taken with fp32 side information
        rec["roofline"]["traffic"] = None if args.side_f16 else traffic_from_profiles(dominant, w.name, layer_tag)
        rec["roofline"]["algorithmic_bytes_per_launch"] = alg_bytes
        rec["roofline"]["launch_ms"] = tot[dominant] / n_launch
        rec["roofline"]["launches_per_step"] = n_launch
        rec["roofline"]["timing"] = "HIP events around the call in every timed step, mean over its launches"
        if len(layers) > 1:
            groups = collections.OrderedDict()
            for j, layer in enumerate(layers):
                groups.setdefault(w.sketch_dim(layer), []).append(j)
            rec["per_group"] = {}
            for k, js in groups.items():
                kt = sum(in_step[j]["quantize_keys"] for j in js)
                dt = sum(in_step[j]["decode"] for j in js)
                rec["per_group"][f"k{k}"] = {
                    "layers": [layers[j] for j in js],
                    "quantize_keys_ms_per_layer": kt / len(js),
                    "quantize_keys_TFLOPs": sum(qk_flops[j] for j in js) / (kt / 1e3) / 1e12,
                    "quantize_values_ms_per_layer": sum(in_step[j]["quantize_values"] for j in js) / len(js),
                    "decode_ms_per_layer": dt / len(js),
                    "decode_GBps": sum(dec_bytes[j] for j in js) / (dt / 1e3) / 1e9,
                    "decode_bytes_per_token_head": ucs[js[0]]["decode_bytes_per_token_head"]}
    if not args.no_detail:
        log("per-call timing on " + ", ".join(f"layer {r}" for r in reps))
        rec["read_stream"] = read_stream_ceiling()
        rec["detail"] = {}
        for layer in reps:
            path = stack.paths[layers.index(layer)]
            per = time_calls(path, reps=max(5, min(steps, 20)))
            cold = time_decode_cold(path, reps=5)
            uc = unit_costs(w, layer, args.side_f16)
            db = uc["decode_bytes_per_token_head"] * th
            rec["detail"][f"layer{layer}"] = {
                "sketch_dim": w.sketch_dim(layer),
                "decode_ms": per["decode"], "decode_ms_cold_llc": cold,
                "decode_GBps": db / (per["decode"] / 1e3) / 1e9,
                "decode_GBps_cold_llc": db / (cold / 1e3) / 1e9,
                "decode_pct_of_read_stream": 100 * db / (min(cold, per["decode"]) / 1e3) / 1e9
                / rec["read_stream"]["GBps_best"],
                "quantize_keys_ms": per["quantize_keys"], "quantize_values_ms": per["quantize_values"],
                "prepare_query_ms": per["prepare_query"],
                "prepare_key_operands_ms_once_per_layer": per["prepare_key_operands"],
                "decode_window_ms": per["decode_window"], "window_tokens": path.n_window,
                "decode_topk_ms": per["decode_topk"], "topk_budget": path.budget,
                "decode_topk_blocks_ms": per["decode_topk_blocks"],
                "topk_blocks_records": -(-path.budget // 32)}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(w, layers)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
