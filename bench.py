#!/usr/bin/env python3
"""Benchmark of the gzip-guided block-sparse attention hot path on one MI355X.

One step = one pass of the device path over one batch: build the mask (flags, CSR/CSC
lists, work order) from the per-block gzip sizes resident in HBM, forward, and the two
backward stages (dQ, which also forms D, then dK/dV).  The host gzip stage
(gsa_prepare) and the PCIe hand-over of its sizes are timed separately
(``host_prepare_ms``, ``c_upload_ms``, ``ms_per_step_with_upload``).

The workload is 8 samples x 8192 bytes, block 64, window 2, 12 heads (6 local /
3 literal / 3 hybrid), head_dim 64, bf16, forward + backward, on seeded synthetic
text-like bytes (the pages' PG-19 runs at 8K bytes are the shape it stands in for).

Prints ONE JSON line.  ``value`` is effective TFLOP/s on kept blocks: algorithmic
FLOPs (4 b^2 d per kept tile forward, 10 b^2 d backward, diagonal tiles counted whole)
divided by the step time.  ``roofline`` rates the kernel that takes the most time per
step against its binding MI355X roof, from HIP events around each kernel on its stream;
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same workload and
compares the timed step's outputs on that sample with it (``cpu_baseline.parity``);
``env`` names the GPU, HIP, torch and zlib versions and the seeds.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s on kept blocks + fwd/bwd ms per batch at 8K bytes, % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
KERNELS = ("mask", "fwd", "bwd_dq", "bwd_dkdv")   # in step order
KERNEL_SOURCES = {"fwd": "gsa_attn_fwd.hip", "bwd_prep": "gsa_attn_bwd.hip", "bwd_dkdv": "gsa_attn_bwd.hip",
                  "bwd_dq": "gsa_attn_bwd.hip", "mask": "gsa_mask.hip"}


def kernel_source_hash(name: str) -> str:
    """Hash of what a kernel is built from: its file, the shared headers and the build
    script (its compiler flags)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "content_adaptive_block_amd")
    for f in (os.path.join("csrc", KERNEL_SOURCES[name]), os.path.join("csrc", "gsa_attn_common.hpp"),
              os.path.join("csrc", "gsa_device.hpp"), "_build.py"):
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kept_tiles(n_edges: np.ndarray, n_heads) -> int:
    """Sum over samples and classes of heads-in-class x kept block pairs."""
    return int(sum(int(n_heads[k]) * int(n_edges[s, k]) for s in range(n_edges.shape[0]) for k in range(3)))


def token_edges(n_edges: np.ndarray, n_heads, n: int, b: int) -> int:
    """Kept (query, key) token pairs: full b x b off-diagonal tiles plus causal diagonals."""
    tot = 0
    for s in range(n_edges.shape[0]):
        for k in range(3):
            e = int(n_edges[s, k])
            tot += int(n_heads[k]) * (b * b * (e - n) + n * b * (b + 1) // 2)
    return tot


def kernel_work(name, wl, tiles):
    """(algorithmic bytes, algorithmic flops) of one launch of kernel ``name``."""
    b, d = wl.block, wl.head_dim
    elem = 4 if wl.dtype == "f32" else 2
    x = wl.batch * wl.heads * wl.seq_len * d * elem          # one [B, H, T, d] tensor
    r = wl.batch * wl.heads * wl.seq_len * 4                 # one fp32 [B, H, T] vector
    tile = b * b * d
    if name == "fwd":              # read Q K V, write O and LSE
        return 4 * x + r, 4 * tile * tiles
    if name == "bwd_prep":         # read O dO, write D
        return 2 * x + r, 2 * wl.batch * wl.heads * wl.seq_len * d
    if name == "bwd_dkdv":         # read Q K V dO LSE D, write dK dV; S, dP, dV, dK
        return 6 * x + 2 * r, 8 * tile * tiles
    if name == "bwd_dq":           # read Q K V O dO LSE, write dQ D; S, dP, dQ, D
        return 6 * x + 2 * r, 6 * tile * tiles + 2 * wl.batch * wl.heads * wl.seq_len * d
    n = wl.n_blocks
    return wl.batch * n * 4 * 2 + 3 * wl.batch * (2 * (n + 1) + n * (n + 1)) * 4, 0   # mask


def load_traffic(name: str, wl) -> float | None:
    """Measured HBM bytes per launch from a committed rocprofv3 PMC summary, if that summary
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(name):
        return None
    return float(rec["bytes_per_launch"])


PMC_KERNELS = {"attn_fwd_kernel": "fwd", "bwd_dq_kernel": "bwd_dq", "bwd_dkdv_kernel": "bwd_dkdv",
               "bwd_pre_kernel": "bwd_prep"}


def _pmc_means(path: str, counter: str) -> dict:
    """Mean counter value (KiB) per dispatch for each kernel of a rocprofv3 counter_collection.csv."""
    import csv
    vals: dict = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = next((v for k, v in PMC_KERNELS.items() if k in name), None)
            if key is None and "neg_kernel" in name:
                key = "copy"
            if key is not None:
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v)), len(v)) for k, v in vals.items()}


def record_traffic(args, fetch_csv: str, write_csv: str):
    """Per-launch HBM bytes of each attention kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the calibration copy of
    --copy-mib MiB, written to profiles/traffic_<kernel>_<workload>.json."""
    import synth
    wl = synth.WORKLOADS[args.config]
    if args.copy_mib <= 0:
        raise SystemExit("--traffic-from needs the --copy-mib of the profiled run")
    fetch, write = _pmc_means(fetch_csv, "FETCH_SIZE"), _pmc_means(write_csv, "WRITE_SIZE")
    copy_bytes = float(args.copy_mib << 20)
    scale_f = copy_bytes / (fetch["copy"][0] * 1024.0)
    scale_w = copy_bytes / (write["copy"][0] * 1024.0)
    rows = []
    for name in sorted(set(fetch) & set(write) - {"copy"}):
        fb, wb = fetch[name][0] * 1024.0 * scale_f, write[name][0] * 1024.0 * scale_w
        rec = {"kernel": name, "workload": wl.name, "bytes_per_launch": round(fb + wb),
               "fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": fetch[name][1],
               "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4),
               "copy_mib": args.copy_mib, "source_hash": kernel_source_hash(name)}
        with open(os.path.join(ROOT, "profiles", f"traffic_{name}_{wl.name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        rows.append(rec)
    print(f"| kernel | dispatches | FETCH bytes | WRITE bytes | HBM bytes / launch |")
    print(f"|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['kernel']} | {r['dispatches']} | {r['fetch_bytes']:,} | {r['write_bytes']:,} | "
              f"{r['bytes_per_launch']:,} |")
    print(f"\nscale: FETCH x {scale_f:.4f}, WRITE x {scale_w:.4f} (copy of {args.copy_mib} MiB)")


def cpu_baseline(wl, x_bytes, tensors, device_out, budget_s: float):
    """The fp64 oracle on whole heads of sample 0 until ``budget_s`` seconds are spent.

    ``device_out`` holds the timed step's outputs for sample 0 (O, LSE and, for backward
    workloads, dQ, dK, dV); each head the oracle finishes is compared with them, and the
    largest absolute error per tensor is reported beside the largest reference value."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    c = oracle.compressed_lengths(x_bytes[:1], wl.block)
    flags, _ = oracle.literal_flags(c, wl.block)
    bm = oracle.block_masks(flags, wl.window)
    t_mask = time.perf_counter() - t0
    classes = oracle.head_classes(wl.n_heads)
    f64 = lambda z: z.float().numpy().astype(np.float64)
    done, flops, t_attn = 0, 0.0, 0.0
    tile = wl.block * wl.block * wl.head_dim
    names = ("o", "lse", "dq", "dk", "dv") if wl.backward else ("o", "lse")
    err = {nm: 0.0 for nm in names}
    ref_max = {nm: 0.0 for nm in names}
    for h in range(wl.heads):
        q, k, v = (f64(tensors[nm][0:1, h:h + 1]) for nm in ("q", "k", "v"))
        nh = [0, 0, 0]
        nh[classes[h]] = 1
        sub = np.zeros((1, 3) + bm.shape[2:], dtype=bool)
        sub[0, classes[h]] = bm[0, classes[h]]
        t1 = time.perf_counter()
        refs = list(oracle.attn_fwd(q, k, v, sub, tuple(nh), wl.block))
        if wl.backward:
            do = f64(tensors["do"][0:1, h:h + 1])
            refs += list(oracle.attn_bwd(q, k, v, do, sub, tuple(nh), wl.block))
        t_attn += time.perf_counter() - t1
        if device_out is not None:
            for nm, ref in zip(names, refs):
                got = device_out[nm][h].double().numpy()
                err[nm] = max(err[nm], float(np.max(np.abs(got - ref[0, 0]))))
                ref_max[nm] = max(ref_max[nm], float(np.max(np.abs(ref))))
        flops += (14 if wl.backward else 4) * tile * int(bm[0, classes[h]].sum())
        done += 1
        if t_attn + t_mask >= budget_s:
            break
    secs = t_attn + t_mask
    rec = {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"sample 0 of {wl.batch}, {done} of {wl.heads} heads, full {wl.seq_len}-byte context; "
                     f"zlib+mask {t_mask:.2f} s, attention fwd{'+bwd' if wl.backward else ''} {t_attn:.2f} s",
           "seconds": secs}
    if device_out is not None:
        # the tolerances of the parity tests: absolute, on values of order one
        tol = {nm: (1e-5 if wl.dtype == "f32" else (1e-3 if nm == "lse" else 2e-2)) for nm in names}
        rec["parity"] = {"heads": done, "tensors": {nm: {"max_abs_err": err[nm], "max_abs_ref": ref_max[nm],
                                                          "tol": tol[nm]} for nm in names},
                         "within_tol": all(err[nm] <= tol[nm] for nm in names)}
    return rec


class DevicePath:
    """Device buffers of one workload and its step: build the mask from c (resident in
    HBM, uploaded once), forward, and (for backward workloads) dQ then dK/dV, all on the
    current stream.  ``step(upload=True)`` first copies c from pinned host memory, as a
    pipeline that feeds new batches does."""

    def __init__(self, torch, gsa, wl, c, t, dev, blocks=None):
        self.torch, self.gsa, self.wl, self.t = torch, gsa, wl, t
        self.blocks = blocks   # a given block mask (uint8 [B, 3, N, N]) instead of the gzip one
        self.c_host = torch.from_numpy(c).pin_memory()
        self.c_dev = torch.empty_like(self.c_host, device=dev)
        self.mask = gsa.GsaMask.empty(wl.batch, wl.n_blocks, wl.window, wl.n_heads, dev)
        self.o = torch.empty_like(t["q"])
        self.lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device=dev)
        self.grads = tuple(torch.empty_like(t["q"]) for _ in range(3)) if wl.backward else None
        self.ws = torch.empty_like(self.lse)
        self.stream = torch.cuda.current_stream(dev)
        self.kernels = KERNELS if wl.backward else KERNELS[:2]
        self.c_dev.copy_(self.c_host)
        if blocks is not None:   # a fixed pattern: its lists are built once, not per batch
            gsa.gsa_build_mask_from_blocks(blocks, wl.n_heads, out=self.mask)
        torch.cuda.synchronize()

    def events(self):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.kernels) + 1)]

    def step(self, ev=None, upload=False):
        gsa, wl, t = self.gsa, self.wl, self.t
        if ev is not None:
            ev[0].record(self.stream)
        if self.blocks is None:
            if upload:
                self.c_dev.copy_(self.c_host, non_blocking=True)
            gsa.gsa_build_mask(self.c_dev, wl.window, wl.n_heads, out=self.mask)
        if ev is not None:
            ev[1].record(self.stream)
        gsa.gsa_attn_fwd(t["q"], t["k"], t["v"], self.mask, wl.block, out=self.o, lse=self.lse)
        if ev is not None:
            ev[2].record(self.stream)
        if wl.backward:
            for i, stage in enumerate(("dq", "dkdv")):
                gsa.gsa_attn_bwd(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], self.mask, wl.block,
                                 workspace=self.ws, out=self.grads, stage=stage)
                if ev is not None:
                    ev[3 + i].record(self.stream)

    def settle(self, ms: float, max_steps: int = 2000) -> float:
        """Untimed steps until `ms` of device time has passed (returns the time spent)."""
        torch = self.torch
        if ms <= 0:
            return 0.0
        spent = 0.0
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        done = 0
        while spent < ms and done < max_steps:
            start.record(self.stream)
            for _ in range(10):
                self.step()
            end.record(self.stream)
            end.synchronize()
            spent += start.elapsed_time(end)
            done += 10
        return spent

    def time(self, steps: int, warmup: int, settle_ms: float = 0.0):
        """(ms per step over `steps` back-to-back steps, mean ms per kernel).

        First `settle_ms` of device time in untimed steps, then `warmup` untimed steps.
        The step time comes from `steps` steps with nothing recorded between their kernels;
        the per-kernel times come from a second run of `steps` steps with an event after
        every kernel, on the same stream."""
        torch = self.torch
        self.settle(settle_ms)
        for _ in range(warmup):
            self.step()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(self.stream)
        for _ in range(steps):
            self.step()
        end.record(self.stream)
        torch.cuda.synchronize()
        evs = [self.events() for _ in range(steps)]
        for k in range(steps):
            self.step(evs[k])
        torch.cuda.synchronize()
        per = {nm: [ev[i].elapsed_time(ev[i + 1]) for ev in evs] for i, nm in enumerate(self.kernels)}
        return start.elapsed_time(end) / steps, {nm: float(np.mean(v)) for nm, v in per.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="untimed device time before the warm-up steps: the first ~25 ms of sustained "
                         "load run up to 20%% slower while the clocks settle (0: none)")
    ap.add_argument("--config", type=int, default=4, help="workload id (1-5); 4 is the headline")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (0: skip)")
    ap.add_argument("--dense", action="store_true",
                    help="time the dense causal variant of the workload (window N - 1, every head local)")
    ap.add_argument("--dense-steps", type=int, default=5,
                    help="also time this many steps of the dense causal variant for comparison (0: skip)")
    ap.add_argument("--bigbird-steps", type=int, default=10,
                    help="steps of a BigBird-style fixed mask at the same shape, for comparison (0: skip)")
    ap.add_argument("--layer-steps", type=int, default=5,
                    help="fwd+bwd steps of the ByteLM attention layer (projections + kernels) (0: skip)")
    ap.add_argument("--pipeline-steps", type=int, default=20,
                    help="batches for the serial vs pipelined host-stage comparison (0: skip)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps timed one by one after a 512 MiB cache flush (0: skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain elementwise copy of this many MiB 3 times (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE, of a run with --copy-mib) into per-launch HBM bytes under profiles/")
    args = ap.parse_args()
    if args.traffic_from:
        record_traffic(args, *args.traffic_from)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(samples shard across GPUs with no communication; run --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import content_adaptive_block_amd as gsa
    import synth

    wl = synth.WORKLOADS[args.config]
    if args.dense:
        wl = synth.dense_causal(wl)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_mib > 0:   # reads and writes copy_mib MiB per launch, 16-byte vector accesses
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    x = synth.gen_bytes(wl)
    names = ("q", "k", "v", "do") if wl.backward else ("q", "k", "v")
    host_t = synth.gen_tensors(wl, names)
    t = {nm: v.to(dev) for nm, v in host_t.items()}

    # host stage, timed on its own (all cores, then one thread)
    c = gsa.gsa_prepare(x, wl.block)
    reps = 20
    t0 = time.perf_counter()
    for _ in range(reps):
        gsa.gsa_prepare(x, wl.block)
    prep_ms = (time.perf_counter() - t0) / reps * 1e3
    t0 = time.perf_counter()
    for _ in range(3):
        gsa.gsa_prepare(x, wl.block, n_threads=1)
    prep1_ms = (time.perf_counter() - t0) / 3 * 1e3

    path = DevicePath(torch, gsa, wl, c, t, dev)
    ms_step, kern_ms = path.time(args.steps, args.warmup, args.settle_ms)
    mask = path.mask
    # The timed steps' outputs for sample 0, for the oracle comparison in cpu_baseline.
    device_out = None
    if args.cpu_budget > 0:
        outs = (path.o, path.lse) + (path.grads if wl.backward else ())
        device_out = {nm: x_[0].float().cpu() for nm, x_ in zip(("o", "lse", "dq", "dk", "dv"), outs)}
    # The hand-over of c from pinned host memory (4 bytes per block over PCIe), timed on
    # its own: the step starts from c resident in HBM.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(path.stream)
    for _ in range(50):
        path.c_dev.copy_(path.c_host, non_blocking=True)
    e1.record(path.stream)
    torch.cuda.synchronize()
    upload_ms = e0.elapsed_time(e1) / 50

    # Cold-cache steps: a 512 MiB write (more than the 256 MB MALL) before each step,
    # outside the events that time it.
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
        cold_ms = []
        for _ in range(args.cold_steps):
            flush.fill_(1.0)
            ev = path.events()
            path.step(ev)
            torch.cuda.synchronize()
            cold_ms.append([ev[i].elapsed_time(ev[i + 1]) for i in range(len(ev) - 1)])
        del flush
        cold_arr = np.array(cold_ms)
        cold = {"steps": args.cold_steps, "ms_per_step": round(float(np.median(cold_arr.sum(axis=1))), 4),
                "kernels_ms": {nm: round(float(np.median(cold_arr[:, i])), 4)
                               for i, nm in enumerate(path.kernels)}}

    # Host-stage pipeline: the gzip sizes of batch k + 1 are computed by the persistent
    # pool while the device runs batch k, against the serial order (sizes, then device).
    pipeline = None
    if args.pipeline_steps > 0:
        xs = [x, np.ascontiguousarray(np.roll(x, wl.block, axis=1))]   # two batches, masks differ
        bufs = [torch.empty(c.shape, dtype=torch.int32).pin_memory() for _ in xs]
        threads = max(1, (os.cpu_count() or 2) - 1)
        saved = path.c_host
        k_steps = args.pipeline_steps
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(k_steps):
            bufs[k % 2].numpy()[...] = gsa.gsa_prepare(xs[k % 2], wl.block, n_threads=threads)
            path.c_host = bufs[k % 2]
            path.step(upload=True)
            torch.cuda.synchronize()
        serial = (time.perf_counter() - t0) / k_steps * 1e3
        with gsa.PrepPool(threads) as pool:
            pool.submit(xs[0], wl.block, bufs[0])
            pool.wait()
            prev = None
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(k_steps):
                path.c_host = bufs[k % 2]
                path.step(upload=True)
                done = torch.cuda.Event()
                done.record(path.stream)
                if prev is not None:
                    prev.synchronize()   # batch k - 1 (the other buffer's copy) has finished
                if k + 1 < k_steps:
                    pool.submit(xs[(k + 1) % 2], wl.block, bufs[(k + 1) % 2])
                    pool.wait()
                prev = done
            torch.cuda.synchronize()
            pipelined = (time.perf_counter() - t0) / k_steps * 1e3
        path.c_host = saved
        pipeline = {"batches": k_steps, "host_threads": threads, "serial_ms_per_batch": round(serial, 4),
                    "pipelined_ms_per_batch": round(pipelined, 4), "device_ms_per_step": round(ms_step, 4)}

    # ByteLM attention layer at this shape: Q/K/V and output projections (D = H d) around
    # the same kernels, forward and backward.
    layer = None
    if args.layer_steps > 0 and wl.backward and wl.dtype == "bf16":
        from content_adaptive_block_amd.layer import GsaAttentionLayer
        dm = wl.heads * wl.head_dim
        torch.manual_seed(0)
        lyr = GsaAttentionLayer(dm, wl.heads, wl.head_dim, wl.block, wl.n_heads, device=dev)
        xin = (torch.randn(wl.batch, wl.seq_len, dm, device=dev) * 0.5).to(torch.bfloat16).requires_grad_(True)
        gy = torch.randn(wl.batch, wl.seq_len, dm, device=dev).to(torch.bfloat16)

        def layer_step():
            lyr(xin, path.mask).backward(gy)

        for _ in range(2):
            layer_step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(path.stream)
        for _ in range(args.layer_steps):
            layer_step()
        e1.record(path.stream)
        torch.cuda.synchronize()
        l_ms = e0.elapsed_time(e1) / args.layer_steps
        attn_ms = kern_ms["fwd"] + kern_ms.get("bwd_dq", 0.0) + kern_ms.get("bwd_dkdv", 0.0)
        layer = {"d_model": dm, "ms_fwd_bwd": round(l_ms, 4), "attention_ms": round(attn_ms, 4),
                 "attention_share": round(attn_ms / l_ms, 3)}
        del lyr, xin, gy

    # BigBird-style fixed mask (window w, one global block, one random block per row; the
    # pages give no BigBird parameters) at this shape through the same kernels.
    bigbird = None
    if args.bigbird_steps > 0:
        import dataclasses
        n_global, n_random = 1, 1
        picks = synth.bigbird_picks(wl, n_random)
        blocks = gsa.gsa_bigbird_blocks(torch.from_numpy(picks).to(dev), wl.window, n_global)
        bwl = dataclasses.replace(wl, name=wl.name + "-bigbird", n_heads=(wl.heads, 0, 0))
        bpath = DevicePath(torch, gsa, bwl, c, t, dev, blocks=blocks)
        b_ms, b_kern = bpath.time(args.bigbird_steps, 2)
        b_edges = bpath.mask.n_edges.cpu().numpy().reshape(wl.batch, 3)
        b_tiles = kept_tiles(b_edges, bwl.n_heads)
        b_flops = (4 + (10 if wl.backward else 0)) * wl.block * wl.block * wl.head_dim * b_tiles
        b_attn = sum(v for nm, v in b_kern.items() if nm != "mask")
        g_attn = sum(v for nm, v in kern_ms.items() if nm != "mask")
        bigbird = {"window": wl.window, "n_global": n_global, "n_random": n_random, "kept_tiles": b_tiles,
                   "gzip_kept_tiles": kept_tiles(path.mask.n_edges.cpu().numpy().reshape(wl.batch, 3), wl.n_heads),
                   "mask": "fixed: lists built once, outside the timed steps",
                   "ms_per_step": round(b_ms, 4), "kernels_ms": {nm: round(v, 4) for nm, v in b_kern.items()},
                   "attention_ms": round(b_attn, 4), "gzip_attention_ms": round(g_attn, 4),
                   "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 3)}
        del bpath, blocks

    # The same shape as dense causal attention (window >= N - 1, every head local) through
    # the same kernels: the wall-clock the sparsity saves.
    dense = None
    if args.dense_steps > 0 and wl.window < wl.n_blocks - 1:
        dwl = synth.dense_causal(wl)
        dpath = DevicePath(torch, gsa, dwl, c, t, dev)
        d_ms, d_kern = dpath.time(args.dense_steps, 2)
        dense = {"workload": dwl.name, "ms_per_step": round(d_ms, 4),
                 "kernels_ms": {nm: round(v, 4) for nm, v in d_kern.items()},
                 "sparse_speedup": round(d_ms / ms_step, 2)}
        del dpath

    n_edges = mask.n_edges.cpu().numpy().reshape(wl.batch, 3)
    n_lit = mask.n_literal.cpu().numpy()[:wl.batch]
    tiles = kept_tiles(n_edges, wl.n_heads)
    tok = token_edges(n_edges, wl.n_heads, wl.n_blocks, wl.block)
    tile = wl.block * wl.block * wl.head_dim
    fl_fwd, fl_bwd = 4 * tile * tiles, (10 * tile * tiles if wl.backward else 0)
    flops = fl_fwd + fl_bwd
    value = flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    fwd_ms = kern_ms["fwd"]
    bwd_ms = sum(kern_ms.get(nm, 0.0) for nm in ("bwd_dq", "bwd_dkdv"))

    kernels = {}
    for nm, ms in kern_ms.items():
        nbytes, nflops = kernel_work(nm, wl, tiles)
        kernels[nm] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "TFLOP/s": round(nflops / (ms * 1e-3) / 1e12, 2), "bytes": nbytes, "flops": nflops}
    dom = max((nm for nm in kern_ms if nm != "mask"), key=lambda nm: kern_ms[nm])
    nbytes, nflops = kernel_work(dom, wl, tiles)
    t_hbm, t_mfma = nbytes / (PEAK_HBM_GBS * 1e9), nflops / (peak * 1e12)
    sec = kern_ms[dom] * 1e-3
    traffic = load_traffic(dom, wl)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(nflops / sec / 1e12, 2), "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = nflops

    rec = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.batch} x {wl.seq_len} bytes, block {wl.block}, window {wl.window}, "
                               f"{wl.heads} heads {'/'.join(map(str, wl.n_heads))}, head_dim {wl.head_dim}, "
                               f"{wl.dtype}, {'fwd+bwd' if wl.backward else 'fwd'}",
                   "global_batch": wl.batch, "seq_len": wl.seq_len, "parallelism": "single GPU"},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "mask_ms": round(kern_ms["mask"], 4),
        "c_upload_ms": round(upload_ms, 4), "ms_per_step_with_upload": round(ms_step + upload_ms, 4),
        "pct_mfma_peak": round(100 * value / peak, 2),
        "token_exact_tflops": round((4 + (10 if wl.backward else 0)) * wl.head_dim * tok / (ms_step * 1e-3) / 1e12, 3),
        "kept_tiles": tiles, "literal_blocks": n_lit.tolist(),
        "host_prepare_ms": {"all_cores": round(prep_ms, 3), "one_thread": round(prep1_ms, 3)},
        "kernels": kernels, "roofline": roof, "cold": cold, "dense_causal": dense,
        "host_pipeline": pipeline, "layer": layer, "bigbird": bigbird,
        "n_edges": n_edges.tolist(),
        "env": {"gpu": torch.cuda.get_device_name(dev), "hip": torch.version.hip, "torch": torch.__version__,
                "zlib": gsa.zlib_version(), "host_cpus": os.cpu_count(),
                "seeds": f"numpy default_rng([{wl.seed_id}, stream]); streams: bytes 0, q 1, k 2, v 3, do 4"},
    }
    if args.cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, x, host_t, device_out, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
