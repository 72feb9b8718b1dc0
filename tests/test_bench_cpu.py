"""Host-side arithmetic of bench.py: algorithmic bytes and flops, kept-tile and token-edge
counts, the HBM-counter scaling, and the one-GPU guard.  No GPU is touched."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_work_matches_the_tensor_sizes():
    wl = synth.WORKLOADS[4]                       # 8 x 8192 B, 12 heads, d 64, bf16
    x = 8 * 12 * 8192 * 64 * 2                    # one [B, H, T, d] bf16 tensor
    r = 8 * 12 * 8192 * 4                         # one fp32 [B, H, T] vector
    assert x == 100_663_296 and r == 3_145_728
    tile = 64 * 64 * 64
    assert bench.kernel_work("fwd", wl, 10) == (4 * x + r, 4 * tile * 10)
    assert bench.kernel_work("bwd_dkdv", wl, 10) == (6 * x + 2 * r, 8 * tile * 10)
    dq_bytes, dq_flops = bench.kernel_work("bwd_dq", wl, 10)
    assert dq_bytes == 6 * x + 2 * r and dq_flops == 6 * tile * 10 + 2 * 8 * 12 * 8192 * 64
    # forward + both backward stages count 4 + 6 + 8 = 18 b^2 d per tile of matrix work,
    # of which the algorithmic 14 (4 forward, 10 backward) enter the headline figure
    assert bench.kernel_work("fwd", wl, 1)[1] + bench.kernel_work("bwd_dkdv", wl, 1)[1] + \
        bench.kernel_work("bwd_dq", wl, 1)[1] - 2 * 8 * 12 * 8192 * 64 == 18 * tile


def test_kept_tiles_and_token_edges_by_brute_force():
    rng = np.random.default_rng(3)
    n, b, n_heads = 7, 4, (2, 1, 3)
    flags = rng.integers(0, 2, (2, n)).astype(bool)
    masks = oracle.block_masks(flags, 1)                          # [2, 3, n, n]
    n_edges = np.array([[int(masks[s, k].sum()) for k in range(3)] for s in range(2)])
    assert bench.kept_tiles(n_edges, n_heads) == sum(
        n_heads[k] * int(masks[s, k].sum()) for s in range(2) for k in range(3))
    tok = 0
    for s in range(2):
        for k in range(3):
            tm = oracle.token_mask(masks[s, k], b)
            tok += n_heads[k] * int(tm.sum())
    assert bench.token_edges(n_edges, n_heads, n, b) == tok


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_pmc_means_average_per_kernel(tmp_path):
    p = tmp_path / "c.csv"
    _counter_csv(p, [
        {"Kernel_Name": "void gsa::attn_fwd_kernel<bf16>(...)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100},
        {"Kernel_Name": "void gsa::attn_fwd_kernel<bf16>(...)", "Counter_Name": "FETCH_SIZE", "Counter_Value": 300},
        {"Kernel_Name": "void gsa::attn_fwd_kernel<bf16>(...)", "Counter_Name": "WRITE_SIZE", "Counter_Value": 7},
        {"Kernel_Name": "neg_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 512},
        {"Kernel_Name": "something_else", "Counter_Name": "FETCH_SIZE", "Counter_Value": 9},
    ])
    m = bench._pmc_means(str(p), "FETCH_SIZE")
    assert m["fwd"] == (200.0, 2) and m["copy"] == (512.0, 1) and len(m) == 2


def test_gpus_above_one_exit_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["fwd", "bwd_dq", "bwd_dkdv"])
def test_traffic_records(name):
    # a committed record is used only while it matches the kernel's sources and build
    # flags; its bytes are at least the compulsory ones
    wl = synth.WORKLOADS[4]
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{wl.name}.json")
    rec = json.load(open(path))
    assert abs(rec["bytes_per_launch"] - rec["fetch_bytes"] - rec["write_bytes"]) <= 1   # each rounded
    compulsory = bench.kernel_work(name, wl, 0)[0]
    assert compulsory <= rec["bytes_per_launch"] < 2 * compulsory
    current = rec["source_hash"] == bench.kernel_source_hash(name)
    assert bench.load_traffic(name, wl) == (float(rec["bytes_per_launch"]) if current else None)


def test_cpu_baseline_reports_parity_against_the_device_outputs():
    # device outputs equal to the oracle's give zero error; a perturbed O exceeds the fp32
    # tolerance and is reported as such
    import torch
    wl = synth.WORKLOADS[1]                        # 1 x 256 B, b 16, 4 heads, d 32, fp32, fwd
    x = synth.gen_bytes(wl)
    t = synth.gen_tensors(wl, ("q", "k", "v"))
    c = oracle.compressed_lengths(x[:1], wl.block)
    flags, _ = oracle.literal_flags(c, wl.block)
    bm = oracle.block_masks(flags, wl.window)
    f64 = lambda z: z.double().numpy()
    o, lse = oracle.attn_fwd(f64(t["q"][:1]), f64(t["k"][:1]), f64(t["v"][:1]), bm, wl.n_heads, wl.block)
    dev = {"o": torch.from_numpy(o).float(), "lse": torch.from_numpy(lse).float()}   # [s][h]
    rec = bench.cpu_baseline(wl, x, t, dev, budget_s=60.0)
    assert rec["cores"] == wl.heads and rec["value"] > 0
    par = rec["parity"]
    assert par["heads"] == wl.heads and par["within_tol"]
    assert par["tensors"]["o"]["max_abs_err"] < 1e-6 and par["tensors"]["o"]["max_abs_ref"] > 0.1
    dev["o"] = dev["o"] + 1e-3
    par = bench.cpu_baseline(wl, x, t, dev, budget_s=60.0)["parity"]
    assert not par["within_tol"] and abs(par["tensors"]["o"]["max_abs_err"] - 1e-3) < 1e-6


def test_trace_summary_takes_the_last_dispatches(tmp_path):
    # two dispatches of one kernel (1 us, then 2 us) and one of another: the "last 1"
    # column holds the second dispatch only
    p = tmp_path / "kernel_trace.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerow({"Kernel_Name": "void gsa::attn_fwd_kernel<bf16>(int)", "Start_Timestamp": 100,
                    "End_Timestamp": 1100})
        w.writerow({"Kernel_Name": "void gsa::attn_fwd_kernel<bf16>(int)", "Start_Timestamp": 2000,
                    "End_Timestamp": 4000})
        w.writerow({"Kernel_Name": "mask_kernel(int)", "Start_Timestamp": 10, "End_Timestamp": 510})
    out = bench.trace_summary(str(p), 1)
    row = [l for l in out.splitlines() if "attn_fwd_kernel" in l][0]
    assert [c.strip() for c in row.split("|")[2:7]] == ["2", "1.5", "2.0", "2.0", "2.0"]


def test_demangle_kernel_names():
    assert bench._demangle("_ZN3gsa12_GLOBAL__N_115attn_fwd_kernelIDF16bLi64ELi64EEEvPKT_S4_S4_PS2_PfNS_9WorkListsEf") \
        == "gsa::attn_fwd_kernel<bf16, 64, 64>"
    assert bench._demangle("_ZN3gsa12_GLOBAL__N_115bwd_dkdv_kernelIfLi16ELi32EEEvPKT_S4_S4_S4_PKfS6_PS2_S7_NS_9WorkLi"
                           "stsEff") == "gsa::bwd_dkdv_kernel<float, 16, 32>"
    assert bench._demangle("gsa::mask_kernel(int)") == "gsa::mask_kernel(int)"
