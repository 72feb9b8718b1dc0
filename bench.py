#!/usr/bin/env python3
"""Benchmark of the gzip-guided block-sparse attention hot path on one MI355X.

One step = one pass of the device path over one batch: build the mask (flags, CSR/CSC
lists, work order) from the per-block gzip sizes resident in HBM, forward, and the two
backward stages (dQ, which also forms D, then dK/dV).  The host gzip stage
(gsa_prepare) and the PCIe hand-over of its sizes are timed separately
(``host_prepare_ms``, ``c_upload_ms``, ``ms_per_step_with_upload``).

The headline workload is 8 samples x 8192 bytes, block 64, window 2, 12 heads (6 local /
3 literal / 3 hybrid), head_dim 64, bf16, forward + backward, on seeded synthetic
text-like bytes (the pages' PG-19 runs at 8K bytes are the shape it stands in for).

Timing: the primary figures are cold-cache steps.  Before each step a 512 MiB buffer
(larger than the 256 MB Infinity Cache) is read, outside the events that time the step,
so that no line of the workload's tensors is cached when it starts.  The flush reads
rather than writes: a written buffer leaves the Infinity Cache full of dirty lines, and
the step's first kernel then pays for writing them back to HBM (``cold_write_fill``
reports the step time under that protocol).  HIP events on the launch stream mark each
timed step's start and end; the per-kernel times come from as many more cold steps with
an event after every kernel (each such event holds the next kernel back by about 5 us).
The device first runs ``--settle-ms`` of such steps untimed (its clocks settle under
sustained load), then ``--warmup`` steps, then ``--steps`` timed steps; the step time is
their median.  ``warm`` gives the same for back-to-back steps with nothing in
between (secondary).

Prints ONE JSON line.  ``value`` is effective TFLOP/s on kept blocks: algorithmic
FLOPs (4 b^2 d per kept tile forward, 10 b^2 d backward, diagonal tiles counted whole)
divided by the cold step time.  ``roofline`` rates the kernel that takes the most time per
cold step against its binding MI355X roof; ``cpu_baseline`` times the fp64 CPU oracle on
a bounded sample of the same workload, one (sample, head) per worker process with one
BLAS thread each, and compares the timed step's outputs on that sample with it
(``cpu_baseline.parity``); ``configs`` holds the same step and roofline figures for the
other workloads (tiny fp32, 8 x 4 KiB, 8 x 8 KiB forward, 2 x 64 KiB forward+backward);
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


def _demangle(name: str) -> str:
    """Readable form of a mangled kernel name: its nested name and template arguments
    (bf16 / float types and integer values), e.g. gsa::attn_fwd_kernel<bf16, 64, 64>."""
    import re
    if not name.startswith("_ZN"):
        return name
    pos, parts = 3, []
    while pos < len(name) and name[pos].isdigit():
        m = re.match(r"\d+", name[pos:])
        n = int(m.group())
        pos += len(m.group())
        ident = name[pos:pos + n]
        pos += n
        if not ident.startswith("_GLOBAL__N"):
            parts.append(ident)
    args = []
    if pos < len(name) and name[pos] == "I":
        body = name[pos + 1:name.find("EE", pos) + 1]
        args = ["bf16" if t == "DF16b" else ("float" if t == "f" else t[2:-1])
                for t in re.findall(r"DF16b|Li\d+E|f", body)]
    return "::".join(parts) + (f"<{', '.join(args)}>" if args else "")


def trace_summary(csv_path: str, last: int) -> str:
    """Markdown table of per-kernel durations from a rocprofv3 kernel_trace.csv: count and
    mean over every dispatch, and mean, min and max over each kernel's last ``last``
    dispatches (the timed steps of a run whose timed steps come last)."""
    import csv
    durs: dict = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            name = _demangle(r["Kernel_Name"]).replace("(anonymous namespace)::", "").replace("void ", "")
            short = name.split("(")[0].strip()
            durs.setdefault(short, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    lines = ["| kernel | calls | avg us (all) | avg us (last %d) | min us (last) | max us (last) |" % last,
             "|---|---|---|---|---|---|"]
    rows = []
    for nm, v in durs.items():
        v.sort()
        d = np.array([(e - b) / 1e3 for b, e in v])
        tail = d[-last:] if last > 0 else d
        rows.append((float(d.sum()), f"| {nm} | {len(d)} | {d.mean():.1f} | {tail.mean():.1f} | {tail.min():.1f} | "
                                     f"{tail.max():.1f} |"))
    for _, line in sorted(rows, reverse=True):
        lines.append(line)
    return "\n".join(lines)


def _oracle_head(task):
    """One (sample, head) of the oracle, in a worker process with one BLAS thread:
    forward (and backward) of that head over its class's block mask.  Returns the
    outputs and the seconds it took."""
    from threadpoolctl import threadpool_limits

    import oracle
    block, cls, bm, backward, q, k, v, do = task
    nh = [0, 0, 0]
    nh[cls] = 1
    sub = np.zeros((1, 3) + bm.shape, dtype=bool)
    sub[0, cls] = bm
    with threadpool_limits(1):
        t0 = time.perf_counter()
        refs = list(oracle.attn_fwd(q[None, None], k[None, None], v[None, None], sub, tuple(nh), block))
        if backward:
            refs += list(oracle.attn_bwd(q[None, None], k[None, None], v[None, None], do[None, None], sub,
                                         tuple(nh), block))
        secs = time.perf_counter() - t0
    return [r[0, 0] for r in refs], secs


def _noop(_):
    return os.getpid()


def host_cores() -> int:
    """CPUs this process may run on, capped at 16 (a GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, x_bytes, tensors, device_out, budget_s: float, workers: int | None = None):
    """The fp64 oracle on whole (sample, head) pairs, one pair per worker process at a time
    (one BLAS thread each), samples and heads in order: a first wave of one pair per
    worker, then as many more pairs as the time of that wave says will fit in
    ``budget_s`` seconds (up to the whole batch).

    The oracle's gzip and mask stage for the samples taken is timed on its own.  ``value``
    is the algorithmic FLOPs of the pairs done over the wall-clock of the attention stage.
    ``device_out`` holds the timed step's outputs (O, LSE and, for backward workloads,
    dQ, dK, dV) indexed [s][h] (any float dtype, on the host); each pair is compared with
    them and the largest absolute error per tensor is reported beside the largest
    reference value."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import oracle
    workers = host_cores() if workers is None else workers
    pairs = [(s, h) for s in range(wl.batch) for h in range(wl.heads)]
    t0 = time.perf_counter()
    c = oracle.compressed_lengths(x_bytes, wl.block)
    flags, _ = oracle.literal_flags(c, wl.block)
    bm = oracle.block_masks(flags, wl.window)
    t_mask = time.perf_counter() - t0
    classes = oracle.head_classes(wl.n_heads)
    f64 = lambda z: z.float().numpy().astype(np.float64)
    names = ("o", "lse", "dq", "dk", "dv") if wl.backward else ("o", "lse")

    def task(s, h):
        hv = [f64(tensors[nm][s, h]) for nm in ("q", "k", "v")]
        do = f64(tensors["do"][s, h]) if wl.backward else None
        return (wl.block, classes[h], bm[s, classes[h]], wl.backward, *hv, do)

    ctx = mp.get_context("spawn")
    first = pairs[:workers]
    with ProcessPoolExecutor(min(workers, len(pairs)), mp_context=ctx) as ex:
        list(ex.map(_noop, range(len(first))))           # start-up outside the timed region
        t1 = time.perf_counter()
        results = list(ex.map(_oracle_head, [task(s, h) for s, h in first]))
        t_wave = time.perf_counter() - t1
        waves = int(max(0.0, budget_s - t_wave - t_mask) // max(t_wave, 1e-3))
        more = pairs[len(first):len(first) + waves * len(first)]
        t_more = 0.0
        if more:
            t1 = time.perf_counter()
            results += list(ex.map(_oracle_head, [task(s, h) for s, h in more]))
            t_more = time.perf_counter() - t1
    done = first + more
    t_attn = t_wave + t_more
    samples = sorted({s for s, _ in done})
    tile = wl.block * wl.block * wl.head_dim
    flops = sum((14 if wl.backward else 4) * tile * int(bm[s, classes[h]].sum()) for s, h in done)
    err = {nm: 0.0 for nm in names}
    ref_max = {nm: 0.0 for nm in names}
    if device_out is not None:
        for (s, h), (refs, _) in zip(done, results):
            for nm, ref in zip(names, refs):
                got = device_out[nm][s][h].double().numpy()
                err[nm] = max(err[nm], float(np.max(np.abs(got - ref))))
                ref_max[nm] = max(ref_max[nm], float(np.max(np.abs(ref))))
    per_pair = [r[1] for r in results]
    rec = {"value": flops / t_attn / 1e12, "unit": "TFLOP/s", "cores": min(workers, len(pairs)), "kind": "oracle",
           "sample": f"{len(done)} of {len(pairs)} (sample, head) pairs (samples {samples[0]}-{samples[-1]}), full "
                     f"{wl.seq_len}-byte context, {min(workers, len(pairs))} worker processes with one BLAS thread "
                     f"each; zlib+mask {t_mask:.2f} s, attention fwd{'+bwd' if wl.backward else ''} {t_attn:.2f} s "
                     f"wall (per pair {min(per_pair):.2f}-{max(per_pair):.2f} s)",
           "seconds": t_mask + t_attn, "attention_seconds": t_attn, "mask_seconds": t_mask,
           "pairs": len(done), "budget_s": budget_s}
    if device_out is not None:
        # the tolerances of the parity tests: absolute, on values of order one
        tol = {nm: (1e-5 if wl.dtype == "f32" else (1e-3 if nm == "lse" else 2e-2)) for nm in names}
        rec["parity"] = {"heads": len(done), "tensors": {nm: {"max_abs_err": err[nm], "max_abs_ref": ref_max[nm],
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
        self.attention(self.mask, ev)

    def attention(self, mask, ev=None):
        """Forward, then (backward workloads) dQ and dK/dV through ``mask``."""
        gsa, wl, t = self.gsa, self.wl, self.t
        gsa.gsa_attn_fwd(t["q"], t["k"], t["v"], mask, wl.block, out=self.o, lse=self.lse)
        if ev is not None:
            ev[2].record(self.stream)
        if wl.backward:
            for i, stage in enumerate(("dq", "dkdv")):
                gsa.gsa_attn_bwd(t["q"], t["k"], t["v"], self.o, self.lse, t["do"], mask, wl.block,
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

    def time_cold(self, steps: int, warmup: int, settle_ms: float, flush):
        """Cold-cache steps: ``flush`` (a callable that reads, or writes, more than the
        Infinity Cache holds) runs before every step, outside the events around it.  ``settle_ms`` of device
        time in such steps and ``warmup`` more run untimed first.  Returns (median ms per
        step, mean ms per step, mean ms per kernel, per-step ms list)."""
        torch = self.torch
        spent, done = 0.0, 0
        while spent < settle_ms and done < 4000:
            ev = self.events()
            flush()
            self.step(ev)
            ev[-1].synchronize()
            spent += ev[0].elapsed_time(ev[-1])
            done += 1
        for _ in range(warmup):
            flush()
            self.step()
        torch.cuda.synchronize()
        # Step times: events only at each step's start and end.  An event recorded between
        # two kernels holds the next one back by about 5 us of queue time, which is no part
        # of the step's work.
        marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for k in range(steps):
            flush()
            marks[k][0].record(self.stream)
            self.step()
            marks[k][1].record(self.stream)
        torch.cuda.synchronize()
        step_ms = [a.elapsed_time(b) for a, b in marks]
        # Per-kernel times: as many more cold steps, with an event after every kernel.
        evs = [self.events() for _ in range(steps)]
        for k in range(steps):
            flush()
            self.step(evs[k])
        torch.cuda.synchronize()
        per = {nm: [ev[i].elapsed_time(ev[i + 1]) for ev in evs] for i, nm in enumerate(self.kernels)}
        return (float(np.median(step_ms)), float(np.mean(step_ms)), {nm: float(np.mean(v)) for nm, v in per.items()},
                step_ms)

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


def roofline(wl, kern_ms: dict, tiles: int) -> dict:
    """Roofline record of the kernel that takes the most time per step (mask kernels
    aside): its algorithmic bytes or flops per launch over its mean launch time, against
    the MI355X roof that binds it (HBM when its bytes take longer at peak than its flops)."""
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    dom = max((nm for nm in kern_ms if nm != "mask"), key=lambda nm: kern_ms[nm])
    nbytes, nflops = kernel_work(dom, wl, tiles)
    t_hbm, t_mfma = nbytes / (PEAK_HBM_GBS * 1e9), nflops / (peak * 1e12)
    sec = kern_ms[dom] * 1e-3
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(nflops / sec / 1e12, 2), "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = load_traffic(dom, wl)
    roof["kernel"] = dom
    roof["kernel_ms"] = round(kern_ms[dom], 4)
    roof["algorithmic_bytes"] = nbytes
    roof["algorithmic_flops"] = nflops
    return roof


def kernel_table(wl, kern_ms: dict, tiles: int) -> dict:
    out = {}
    for nm, ms in kern_ms.items():
        nbytes, nflops = kernel_work(nm, wl, tiles)
        out[nm] = {"ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "TFLOP/s": round(nflops / (ms * 1e-3) / 1e12, 2), "bytes": nbytes, "flops": nflops}
    return out


def workload_name(wl) -> str:
    return (f"{wl.batch} x {wl.seq_len} bytes, block {wl.block}, window {wl.window}, "
            f"{wl.heads} heads {'/'.join(map(str, wl.n_heads))}, head_dim {wl.head_dim}, "
            f"{wl.dtype}, {'fwd+bwd' if wl.backward else 'fwd'}")


def measure(torch, gsa, wl, dev, c, t, flush, steps: int, warmup: int, settle_ms: float, warm_steps: int = 0,
            fill=None, fill_steps: int = 0):
    """Cold steps (primary) and ``warm_steps`` back-to-back steps of one workload:
    (DevicePath, record).  The record holds the step times, per-kernel times, effective
    TFLOP/s and the dominant kernel's roofline, all from the cold steps.  With ``fill``
    (a callable that writes more than the Infinity Cache holds), ``fill_steps`` more cold
    steps run after it instead of ``flush`` (``cold_write_fill``)."""
    path = DevicePath(torch, gsa, wl, c, t, dev)
    med, mean, kern, step_ms = path.time_cold(steps, warmup, settle_ms, flush)
    n_edges = path.mask.n_edges.cpu().numpy().reshape(wl.batch, 3)
    tiles = kept_tiles(n_edges, wl.n_heads)
    tok = token_edges(n_edges, wl.n_heads, wl.n_blocks, wl.block)
    fl = (4 + (10 if wl.backward else 0)) * wl.block * wl.block * wl.head_dim
    peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
    value = fl * tiles / (med * 1e-3) / 1e12
    rec = {"workload": workload_name(wl), "dtype": wl.dtype, "steps": steps, "ms_per_step": round(med, 4),
           "ms_per_step_mean": round(mean, 4), "ms_per_step_min": round(min(step_ms), 4),
           "tflops": round(value, 3), "pct_mfma_peak": round(100 * value / peak, 2),
           "token_exact_tflops": round((fl // (wl.block * wl.block)) * tok / (med * 1e-3) / 1e12, 3),
           "kept_tiles": tiles, "literal_blocks": path.mask.n_literal.cpu().numpy()[:wl.batch].tolist(),
           "kernels": kernel_table(wl, kern, tiles), "roofline": roofline(wl, kern, tiles)}
    if warm_steps > 0:
        # back-to-back steps draw more power than cold ones: settle again before timing them
        w_ms, w_kern = path.time(warm_steps, warmup, settle_ms)
        rec["warm"] = {"ms_per_step": round(w_ms, 4), "tflops": round(fl * tiles / (w_ms * 1e-3) / 1e12, 3),
                       "kernels_ms": {nm: round(v, 4) for nm, v in w_kern.items()}}
    if fill is not None and fill_steps > 0:
        f_med, _, f_kern, _ = path.time_cold(fill_steps, warmup, settle_ms / 2, fill)
        rec["cold_write_fill"] = {"ms_per_step": round(f_med, 4),
                                  "tflops": round(fl * tiles / (f_med * 1e-3) / 1e12, 3),
                                  "kernels_ms": {nm: round(v, 4) for nm, v in f_kern.items()}}
    return path, rec


def sdpa_dense(torch, t, flush, steps: int):
    """Dense causal attention through torch's scaled_dot_product_attention with only its
    flash or memory-efficient backend allowed (whichever runs and is faster), forward and
    backward on the workload's Q, K, V, dO, each step after the cache flush.  None when
    neither backend is available."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    best = None
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            q, k, v = (t[nm].detach().clone().requires_grad_(True) for nm in ("q", "k", "v"))
            with sdpa_kernel([be]):
                for _ in range(2):
                    F.scaled_dot_product_attention(q, k, v, is_causal=True).backward(t["do"])
                torch.cuda.synchronize()
                fw, bw = [], []
                for _ in range(steps):
                    q.grad = k.grad = v.grad = None
                    flush()
                    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                    e[0].record()
                    o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
                    e[1].record()
                    o.backward(t["do"])
                    e[2].record()
                    torch.cuda.synchronize()
                    fw.append(e[0].elapsed_time(e[1]))
                    bw.append(e[1].elapsed_time(e[2]))
            rec = {"backend": name, "fwd_ms": round(float(np.median(fw)), 4), "bwd_ms": round(float(np.median(bw)), 4)}
            rec["ms_per_step"] = round(rec["fwd_ms"] + rec["bwd_ms"], 4)
            if best is None or rec["ms_per_step"] < best["ms_per_step"]:
                best = rec
            del q, k, v
        except RuntimeError:
            continue
    return best


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed cold steps (median reported)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="untimed device time (in cold steps) before the warm-up steps: the first ~25 ms "
                         "of sustained load run up to 20%% slower while the clocks settle (0: none)")
    ap.add_argument("--config", type=int, default=4, help="workload id (1-5); 4 is the headline")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (0: skip)")
    ap.add_argument("--dense", action="store_true",
                    help="time the dense causal variant of the workload (window N - 1, every head local)")
    ap.add_argument("--dense-steps", type=int, default=5,
                    help="also time this many steps of the dense causal variant for comparison (0: skip)")
    ap.add_argument("--bigbird-steps", type=int, default=10,
                    help="steps of a BigBird-style fixed mask at the same shape, for comparison (0: skip)")
    ap.add_argument("--sdpa-steps", type=int, default=5,
                    help="cold fwd+bwd steps of torch SDPA (flash / memory-efficient backends) as dense causal "
                         "attention at the same shape, for comparison (0: skip)")
    ap.add_argument("--layer-steps", type=int, default=5,
                    help="fwd+bwd steps of the ByteLM attention layer (projections + kernels) (0: skip)")
    ap.add_argument("--pipeline-steps", type=int, default=20,
                    help="batches for the serial vs pipelined host-stage comparison (0: skip)")
    ap.add_argument("--other-configs", default="1,2,3,5",
                    help="comma-separated workload ids also timed (cold protocol, --other-steps steps)")
    ap.add_argument("--other-steps", type=int, default=20)
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain elementwise copy of this many MiB 3 times (HBM counter calibration)")
    ap.add_argument("--fill-steps", type=int, default=20,
                    help="cold steps after a 512 MiB write instead of the read flush (cold_write_fill; 0: none)")
    ap.add_argument("--warm-steps", type=int, default=-1,
                    help="back-to-back (warm) steps timed after the cold ones (-1: as many as --steps; 0: none)")
    ap.add_argument("--trace-from", metavar="KERNEL_TRACE_CSV",
                    help="no GPU: per-kernel durations of a rocprofv3 kernel_trace.csv, over every dispatch "
                         "and over each kernel's last --steps dispatches")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE, of a run with --copy-mib) into per-launch HBM bytes under profiles/")
    args = ap.parse_args()
    if args.trace_from:
        print(trace_summary(args.trace_from, args.steps))
        return
    if args.traffic_from:
        record_traffic(args, *args.traffic_from)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
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

    # Cache flush: a 512 MiB buffer, written once here, then read before every cold step
    # (a sum into a preallocated scalar): the caches end up holding its clean lines only.
    flush_buf = torch.ones(512 << 18, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, dtype=torch.float32, out=flush_sink)

    def fill():   # the write-fill protocol, for cold_write_fill
        flush_buf.fill_(1.0)

    warm_steps = args.steps if args.warm_steps < 0 else args.warm_steps
    path, head = measure(torch, gsa, wl, dev, c, t, flush, args.steps, args.warmup, args.settle_ms, warm_steps,
                         fill=fill, fill_steps=args.fill_steps)
    ms_step = head["ms_per_step"]
    kern_ms = {nm: v["ms"] for nm, v in head["kernels"].items()}
    mask = path.mask
    # The timed steps' outputs (host copies), for the oracle comparison in cpu_baseline.
    device_out = None
    if args.cpu_budget > 0:
        outs = (path.o, path.lse) + (path.grads if wl.backward else ())
        device_out = {nm: x_.cpu() for nm, x_ in zip(("o", "lse", "dq", "dk", "dv"), outs)}
    # The hand-over of c from pinned host memory (4 bytes per block over PCIe), timed on
    # its own: the step starts from c resident in HBM.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(path.stream)
    for _ in range(50):
        path.c_dev.copy_(path.c_host, non_blocking=True)
    e1.record(path.stream)
    torch.cuda.synchronize()
    upload_ms = e0.elapsed_time(e1) / 50

    # Host-stage pipeline: the gzip sizes of batch k + 1 are computed by the persistent
    # pool while the device runs batch k (MaskPipeline), against the serial order (sizes,
    # upload, mask, attention, wait).
    pipeline = None
    if args.pipeline_steps > 0:
        from content_adaptive_block_amd.pipeline import MaskPipeline
        xs = [x, np.ascontiguousarray(np.roll(x, wl.block, axis=1))]   # two batches, masks differ
        batches = [xs[k % 2] for k in range(args.pipeline_steps)]
        threads = max(1, (os.cpu_count() or 2) - 1)
        k_steps = len(batches)
        c_pin = torch.empty(c.shape, dtype=torch.int32).pin_memory()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for xb in batches:
            c_pin.numpy()[...] = gsa.gsa_prepare(xb, wl.block, n_threads=threads)
            path.c_dev.copy_(c_pin, non_blocking=True)
            gsa.gsa_build_mask(path.c_dev, wl.window, wl.n_heads, out=path.mask)
            path.attention(path.mask)
            torch.cuda.synchronize()
        serial = (time.perf_counter() - t0) / k_steps * 1e3
        with MaskPipeline(wl.batch, wl.seq_len, wl.block, wl.window, wl.n_heads, dev, threads) as pipe:
            pipe.run(batches[:2], lambda k, m: path.attention(m))
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pipe.run(batches, lambda k, m: path.attention(m))
            torch.cuda.synchronize()
            pipelined = (time.perf_counter() - t0) / k_steps * 1e3
        path.c_dev.copy_(path.c_host)
        torch.cuda.synchronize()
        pipeline = {"batches": k_steps, "host_threads": threads, "serial_ms_per_batch": round(serial, 4),
                    "pipelined_ms_per_batch": round(pipelined, 4),
                    "device_ms_per_step_warm": head["warm"]["ms_per_step"] if head.get("warm") else None}

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
        wk = head["warm"]["kernels_ms"] if head.get("warm") else kern_ms   # back-to-back, like the layer
        attn_ms = wk["fwd"] + wk.get("bwd_dq", 0.0) + wk.get("bwd_dkdv", 0.0)
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
        b_ms, _, b_kern, _ = bpath.time_cold(args.bigbird_steps, 2, 0.0, flush)
        b_edges = bpath.mask.n_edges.cpu().numpy().reshape(wl.batch, 3)
        b_tiles = kept_tiles(b_edges, bwl.n_heads)
        b_flops = (4 + (10 if wl.backward else 0)) * wl.block * wl.block * wl.head_dim * b_tiles
        b_attn = sum(v for nm, v in b_kern.items() if nm != "mask")
        g_attn = sum(v for nm, v in kern_ms.items() if nm != "mask")
        bigbird = {"window": wl.window, "n_global": n_global, "n_random": n_random, "kept_tiles": b_tiles,
                   "gzip_kept_tiles": kept_tiles(path.mask.n_edges.cpu().numpy().reshape(wl.batch, 3), wl.n_heads),
                   "mask": "fixed: lists built once, outside the timed (cold) steps",
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
        d_ms, _, d_kern, _ = dpath.time_cold(args.dense_steps, 1, 0.0, flush)
        dense = {"workload": dwl.name, "ms_per_step": round(d_ms, 4),
                 "kernels_ms": {nm: round(v, 4) for nm, v in d_kern.items()},
                 "sparse_speedup": round(d_ms / ms_step, 2)}
        del dpath

    # The vendor library's dense causal attention at the same shape (torch SDPA restricted
    # to its flash and memory-efficient backends, never the math path), forward and
    # backward, cold steps like ours: context for the dense figure above.
    sdpa = None
    if args.sdpa_steps > 0 and wl.dtype == "bf16" and wl.backward:
        sdpa = sdpa_dense(torch, t, flush, args.sdpa_steps)
        if sdpa is not None:
            sdpa["this_library_dense_ms"] = dense["ms_per_step"] if dense else None
            sdpa["gzip_sparse_speedup"] = round(sdpa["ms_per_step"] / ms_step, 2)

    n_edges = mask.n_edges.cpu().numpy().reshape(wl.batch, 3)
    rec = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": head["workload"], "global_batch": wl.batch, "seq_len": wl.seq_len,
                   "parallelism": "single GPU"},
        "timing": "cold: 512 MiB read before every step, outside its events; median of the timed steps",
        "cold_write_fill": head.get("cold_write_fill"),
        "ms_per_step_mean": head["ms_per_step_mean"], "ms_per_step_min": head["ms_per_step_min"],
        "fwd_ms": round(kern_ms["fwd"], 4), "bwd_ms": round(sum(kern_ms.get(nm, 0.0) for nm in ("bwd_dq", "bwd_dkdv")), 4),
        "mask_ms": round(kern_ms["mask"], 4),
        "c_upload_ms": round(upload_ms, 4), "ms_per_step_with_upload": round(ms_step + upload_ms, 4),
        "pct_mfma_peak": head["pct_mfma_peak"], "token_exact_tflops": head["token_exact_tflops"],
        "kept_tiles": head["kept_tiles"], "literal_blocks": head["literal_blocks"],
        "host_prepare_ms": {"all_cores": round(prep_ms, 3), "one_thread": round(prep1_ms, 3)},
        "kernels": head["kernels"], "roofline": head["roofline"], "warm": head.get("warm"), "dense_causal": dense,
        "host_pipeline": pipeline, "layer": layer, "bigbird": bigbird, "torch_sdpa_dense": sdpa,
        "n_edges": n_edges.tolist(),
        "env": {"gpu": torch.cuda.get_device_name(dev), "hip": torch.version.hip, "torch": torch.__version__,
                "zlib": gsa.zlib_version(), "host_cpus": os.cpu_count(),
                "seeds": f"numpy default_rng([{wl.seed_id}, stream]); streams: bytes 0, q 1, k 2, v 3, do 4"},
    }
    if args.cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(wl, x, host_t, device_out, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    del path, t, device_out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # The other workloads: the same cold protocol with fewer steps, no oracle.
    others = {}
    for cid in [int(z) for z in args.other_configs.split(",") if z.strip()]:
        if cid == args.config or cid not in synth.WORKLOADS:
            continue
        owl = synth.WORKLOADS[cid]
        onames = ("q", "k", "v", "do") if owl.backward else ("q", "k", "v")
        ox = synth.gen_bytes(owl)
        ot = {nm: v.to(dev) for nm, v in synth.gen_tensors(owl, onames).items()}
        oc = gsa.gsa_prepare(ox, owl.block)
        opath, orec = measure(torch, gsa, owl, dev, oc, ot, flush, args.other_steps, 3, args.settle_ms / 2,
                              args.other_steps)
        others[str(cid)] = orec
        del opath, ot
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    rec["configs"] = others
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
