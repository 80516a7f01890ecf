"""Host logic of bench.py (CPU): the one-GPU guard and the HBM-traffic arithmetic that turns
rocprofv3 FETCH_SIZE / WRITE_SIZE counters into bytes per launch."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _counters(path, rows):
    """A counter_collection.csv with one row per (kernel name, KiB per dispatch)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, kib) in enumerate(rows):
            w.writerow([i + 1, name, "X", kib])
    return str(path)


def test_traffic_is_scaled_by_the_plain_copy(tmp_path, monkeypatch):
    """A 1 GiB copy whose FETCH_SIZE reads half its bytes and whose WRITE_SIZE reads them all
    gives scales 2 and 1; the kernel's mean counter per dispatch is scaled by them."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kern = "void rkv::(anonymous namespace)::chunk_attn_kernel<128, 4, 2, true>(rkv::ChunkAttnArgs)"
    other = "void at::native::vectorized_elementwise_kernel<4>(int)"
    args = SimpleNamespace(
        copy_fetch=_counters(tmp_path / "cf.csv", [("__amd_rocclr_copyBuffer", 524288.0)]),
        copy_write=_counters(tmp_path / "cw.csv", [("__amd_rocclr_copyBuffer", 1048576.0)]),
        fetch=_counters(tmp_path / "kf.csv", [(kern, 131000.0), (other, 9e9), (kern, 131144.0)]),
        write=_counters(tmp_path / "kw.csv", [(kern, 8256.0), (kern, 8256.0)]))
    bench.traffic_summary(args)
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["dispatches"] == 2
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["hbm_fetch_bytes_per_launch"] == 131072 * 1024 * 2       # mean of the two dispatches
    assert t["hbm_write_bytes_per_launch"] == 8256 * 1024
    assert t["algorithmic_bytes_per_launch"] == 2 * 131072 * 4 * 128 * 2
    assert t["traffic_over_algorithmic"] == round((268435456 + 8454144) / 268435456, 4)
    assert t["kernel_sha"] == bench.kernel_hash()


def test_traffic_is_dropped_once_the_kernel_source_changes(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({"kernel_sha": bench.kernel_hash(), "hbm_bytes_per_launch": 123}))
    assert bench.traffic_entry(268435456) == 123
    f.write_text(json.dumps({"kernel_sha": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_entry(268435456) is None


def test_step_parity_compares_outputs_and_the_accept():
    import numpy as np
    g = np.random.default_rng(5)
    ref = {l: (g.standard_normal((16, 16, 128)), g.standard_normal((16, 16))) for l in (3, 0, 1, 2)}
    ref["accept"] = (2, np.array([7, 9, 4], np.int32), np.zeros(17, np.int32))
    committed = np.array([7, 9, 4] + [-1] * 14, np.int32)
    same = {l: (ref[l][0].astype(np.float32), ref[l][1].astype(np.float32)) for l in (0, 1, 2, 3)}
    same["accept"] = (2, committed)
    p = bench.step_parity(same, ref)
    assert p["layers"] == [0, 1, 2, 3] and p["within_tolerance"] and p["accept_exact"]
    assert p["max_abs_out"] < 1e-6 and p["max_abs_lse"] < 1e-6
    off = dict(same)
    off[3] = (same[3][0] + 0.02, same[3][1])
    off["accept"] = (2, np.array([7, 9, 5] + [-1] * 14, np.int32))
    p = bench.step_parity(off, ref)
    assert not p["within_tolerance"] and not p["accept_exact"]
    assert abs(p["max_abs_out"] - 0.02) < 1e-5


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("// head\nint f() { return 1; } /* tail */\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", [str(src)])
    h0 = bench.kernel_hash()
    src.write_text("// another comment\nint f()  {\n  return 1;   // why\n}\n")
    assert bench.kernel_hash() == h0
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_hash() != h0
