"""GPU check of the host-stage pipeline (MaskPipeline): per-batch gzip sizes from the
persistent host pool into alternating pinned buffers, non-blocking upload into one
device buffer, and the mask kernels into one reused mask, with batch k + 1's sizes
computed while the device runs batch k.  Every batch's sizes, flags, lists and work
descriptors, as the device held them right after that batch's mask build, must equal
the oracle's for that batch's bytes, bit for bit: a buffer reused too early would
show up as another batch's sizes or lists."""
import dataclasses

import numpy as np
import pytest
import torch

import content_adaptive_block_amd as gsa
from content_adaptive_block_amd.pipeline import MaskPipeline
import oracle
import synth
from gpu_cases import check_mask, log

pytestmark = pytest.mark.gpu


def _batches(wl, count):
    """``count`` different byte batches of the workload's shape (fresh seeded streams,
    every third with constant runs so that its literal sets differ more)."""
    out = []
    for k in range(count):
        x = synth.gen_bytes(dataclasses.replace(wl, seed_id=100 + k))
        if k % 3 == 2:
            x[:, (k % 7) * wl.block:(k % 7 + 20) * wl.block] = ord("e")
        out.append(x)
    return out


@pytest.mark.parametrize("cid", [4, 5])
def test_pipeline_masks_bit_exact_per_batch(cid):
    wl = synth.WORKLOADS[cid]
    count = 8 if cid == 4 else 6
    log(f"  pipeline cfg{cid}: {count} batches of {wl.batch} x {wl.seq_len} bytes")
    batches = _batches(wl, count)
    snaps = []
    t = synth.gen_tensors(wl, ("q", "k", "v"))
    q, k, v = (t[nm].cuda() for nm in ("q", "k", "v"))

    with MaskPipeline(wl.batch, wl.seq_len, wl.block, wl.window, wl.n_heads, threads=4) as pipe:
        def work(kk, m):
            # the device state right after this batch's mask build (copies on the stream),
            # then some attention work so that batches overlap the host stage
            snaps.append(({f: getattr(m, f).clone() for f in gsa.MASK_FIELDS}, pipe.c_dev.clone()))
            gsa.gsa_attn_fwd(q, k, v, m, wl.block)

        pipe.run(batches, work)
        torch.cuda.synchronize()
    assert len(snaps) == count
    for kk, (bufs, c_dev) in enumerate(snaps):
        c_ref = oracle.compressed_lengths(batches[kk], wl.block)
        assert np.array_equal(c_dev.cpu().numpy(), c_ref), kk
        m = gsa.GsaMask(wl.batch, wl.n_blocks, wl.window, wl.n_heads, **bufs, built=True)
        check_mask(m, c_ref, wl.block, wl.window, wl.n_heads)
        log(f"    batch {kk}: L = {m.n_literal.cpu().numpy()[:wl.batch].tolist()} bit-exact")
    # consecutive batches really differ, so a stale buffer could not pass
    assert len({s[1].cpu().numpy().tobytes() for s in snaps}) == count
