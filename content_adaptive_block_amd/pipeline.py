"""Host-stage pipeline: the gzip sizes of batch k + 1 are computed on the persistent host
pool while the device runs batch k.

The gzip stage comes first on the path ("Gzip-guided Sparse Attention", daiwk.github.io
reproduction note, flowchart under 背景与主要改动: bytes -> fixed blocks -> gzip level 1
per block -> ratios), and it runs on the host.  Per batch k:

  1. its sizes are already in pinned host buffer k % 2 (computed during batch k - 1);
  2. they are copied to the device asynchronously, on the current stream;
  3. the mask kernels run on that stream, then the caller's device work for batch k;
  4. the host waits until batch k - 1 has finished on the device (so buffer (k + 1) % 2
     is no longer being read), then computes batch k + 1's sizes into it with the pool
     while the device still runs batch k.

Every device step of a batch is ordered on one stream, so the single device copy of the
sizes and the single mask are reused without further synchronisation.
"""
from __future__ import annotations

import numpy as np
import torch

from . import GsaMask, PrepPool, gsa_build_mask

__all__ = ["MaskPipeline"]


class MaskPipeline:
    """Pipelined bytes -> sizes -> mask for batches of ``batch`` x ``seq_len`` bytes.

    ``run(batches, work)`` calls ``work(k, mask)`` once per batch, after batch k's mask
    has been enqueued on the current stream; ``work`` enqueues its own device work on
    that stream and must not keep the mask beyond it (the next batch reuses the buffers).
    """

    def __init__(self, batch: int, seq_len: int, block: int, window: int, n_heads, device=None,
                 threads: int = 0):
        if block <= 0 or seq_len % block:
            raise ValueError("seq_len must be a positive multiple of block")
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.batch, self.seq_len, self.block, self.window = batch, seq_len, block, window
        self.n_heads = tuple(int(h) for h in n_heads)
        n = seq_len // block
        self.pool = PrepPool(threads)
        self.c_host = [torch.empty((batch, n), dtype=torch.int32).pin_memory() for _ in range(2)]
        self.c_dev = torch.empty((batch, n), dtype=torch.int32, device=self.device)
        self.mask = GsaMask.empty(batch, n, window, self.n_heads, self.device)

    def run(self, batches, work) -> None:
        batches = [np.ascontiguousarray(np.asarray(x, dtype=np.uint8)) for x in batches]
        for x in batches:
            if x.shape != (self.batch, self.seq_len):
                raise ValueError(f"batch of shape {x.shape}, expected {(self.batch, self.seq_len)}")
        if not batches:
            return
        stream = torch.cuda.current_stream(self.device)
        self.pool.submit(batches[0], self.block, self.c_host[0])
        self.pool.wait()
        prev = None
        for k in range(len(batches)):
            self.c_dev.copy_(self.c_host[k % 2], non_blocking=True)
            gsa_build_mask(self.c_dev, self.window, self.n_heads, out=self.mask)
            work(k, self.mask)
            done = torch.cuda.Event()
            done.record(stream)
            if k + 1 < len(batches):
                if prev is not None:
                    prev.synchronize()   # batch k - 1, whose sizes were in buffer (k + 1) % 2, is done
                self.pool.submit(batches[k + 1], self.block, self.c_host[(k + 1) % 2])
                self.pool.wait()
            prev = done

    def close(self) -> None:
        self.pool.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
