"""bench.py host logic on the CPU: the one-GPU guard, the HBM counter summary
(calibration by a plain copy, per workload and layer, tied to the kernel
sources) and the algorithmic bytes per unit."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from kv_cache_compression_quantize_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_is_calibrated_by_the_copy(tmp_path):
    gib_kib = 1 << 20
    # the copy reads half of its bytes through FETCH_SIZE (factor 2) and all through WRITE_SIZE;
    # two decode launches (each a decode kernel and a combine); four key launches of a layer
    # stack, two on each of two alternative kernels
    # an input set-up copy as large as half the calibration copy comes first and must not count
    copies_f = [("__amd_rocclr_copyBuffer", gib_kib / 2)] * bench.CALIBRATION_COPIES
    copies_w = [("__amd_rocclr_copyBuffer", gib_kib)] * bench.CALIBRATION_COPIES
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", gib_kib / 3), ("__amd_rocclr_copyBuffer", 10.0),
        ("void aqkv::fast::decode_fast_kernel<128, 2, 2, 1, 2>(aqkv::DecodeJob)", 1000.0),
        ("void aqkv::fast::decode_fast_kernel<128, 2, 2, 1, 2>(aqkv::DecodeJob)", 1200.0),
        ("aqkv::(anonymous namespace)::combine_kernel(aqkv::DecodeJob)", 10.0),
        ("aqkv::(anonymous namespace)::combine_kernel(aqkv::DecodeJob)", 30.0),
        ("void aqkv::(anonymous namespace)::quantize_keys_qjl_kernel<8>(aqkv::KeyJob, unsigned char const*, long)",
         500.0),
        ("void aqkv::(anonymous namespace)::quantize_keys_qjl_kernel<8>(aqkv::KeyJob, unsigned char const*, long)",
         500.0),
        ("void aqkv::(anonymous namespace)::quantize_keys_resident_kernel<128, 0, true, 12>(aqkv::KeyJob, long)",
         300.0),
        ("void aqkv::(anonymous namespace)::quantize_keys_resident_kernel<128, 0, true, 12>(aqkv::KeyJob, long)",
         300.0)] + copies_f)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", gib_kib / 1.5),
        ("void aqkv::fast::decode_fast_kernel<128, 2, 2, 1, 2>(aqkv::DecodeJob)", 4.0),
        ("void aqkv::fast::decode_fast_kernel<128, 2, 2, 1, 2>(aqkv::DecodeJob)", 4.0),
        ("aqkv::(anonymous namespace)::combine_kernel(aqkv::DecodeJob)", 2.0),
        ("aqkv::(anonymous namespace)::combine_kernel(aqkv::DecodeJob)", 2.0)] + copies_w)
    out = tmp_path / "c.json"
    rec = bench.write_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out), "wl", 3)
    assert rec["workload"] == "wl" and rec["layer"] == 3
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    dec = rec["kernels"]["decode"]
    # all of the call's bytes over its launches (its main kernel's dispatches), scaled, in bytes
    assert dec["fetch_bytes_per_launch"] == pytest.approx((1000.0 + 1200.0 + 10.0 + 30.0) / 2 * 1024 * 2.0)
    assert dec["write_bytes_per_launch"] == pytest.approx((4.0 + 2.0) * 1024)
    assert dec["source_hash"] == bench.source_hash("decode")
    # alternative kernels of one call are averaged, never added
    keys = rec["kernels"]["quantize_keys"]
    assert keys["fetch_bytes_per_launch"] == pytest.approx((500.0 + 300.0) / 2 * 1024 * 2.0)
    assert "quantize_values" not in rec["kernels"]      # no dispatch of it in the files
    assert json.loads(out.read_text()) == rec


def test_counter_summary_without_a_copy_is_refused(tmp_path):
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("x", 1.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [("x", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "c.json"), "wl", 0)


def test_traffic_only_from_the_same_workload_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda k: "h_" + k)
    os.makedirs(tmp_path / "profiles")
    rec = {"workload": "wl", "layer": 0, "kernels": {
        "decode": {"source_hash": "h_decode", "hbm_bytes_per_launch": 123.0},
        "quantize_values": {"source_hash": "stale", "hbm_bytes_per_launch": 456.0}}}
    (tmp_path / "profiles" / "hbm_counters_wl_layer0.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("decode", "wl", 0) == 123.0
    assert bench.traffic_from_profiles("quantize_values", "wl", 0) is None     # sources changed since
    assert bench.traffic_from_profiles("decode", "wl", 1) is None              # another layer
    assert bench.traffic_from_profiles("decode", "other", 0) is None           # another workload


def test_algorithmic_bytes_per_unit():
    w = inputs.WORKLOADS["llama2_7b_layer_mha32_t32k"]
    uc = bench.unit_costs(w, 0)
    # 2-bit codes (32 B) + 128 sign bits (16 B) + n and gamma (8 B); 2-bit values (32 B) + fp32 scale/min per 32 (32 B)
    assert uc["decode_bytes_per_token_head"] == 32 + 16 + 8 + 32 + 32
    assert uc["qkeys_bytes_per_key"] == 2 * 128 + 56
    assert uc["qvals_bytes_per_value"] == 2 * 128 + 64
    assert uc["qkeys_flops_per_key"] == 4 * 128 * 128 + 2 * 128 * 128
    a = inputs.WORKLOADS["aqjl_32layer_gqa32x8_b16_t32k"]
    # pure QJL keys: k sign bits and the norm only; no rotation flops
    assert bench.unit_costs(a, 0)["decode_bytes_per_token_head"] == 512 // 8 + 4 + 64
    assert bench.unit_costs(a, 0)["qkeys_flops_per_key"] == 2 * 512 * 128
