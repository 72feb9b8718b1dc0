"""GPU parity of the mask kernel: flags, L, CSR, CSC, edge counts and work order must be
bit-exact against the oracle's set logic, on every config's bytes and on synthetic size
patterns (ragged N around the wave and workgroup sizes, empty literal sets, windows of
0 and beyond N, the maximum N)."""
import numpy as np
import pytest
import torch

import content_adaptive_block_amd as gsa
import oracle
import synth
from gpu_cases import check_mask, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_mask_on_config_bytes(cid):
    wl = synth.WORKLOADS[cid]
    log(f"  mask cfg{cid}: B={wl.batch} N={wl.n_blocks} w={wl.window} heads={wl.n_heads}")
    x = synth.gen_bytes(wl)
    c = gsa.gsa_prepare(x, wl.block)
    assert np.array_equal(c, oracle.compressed_lengths(x, wl.block))
    m = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), wl.window, wl.n_heads)
    torch.cuda.synchronize()
    check_mask(m, c, wl.block, wl.window, wl.n_heads)


def _c_patterns(n, rng):
    big = n > 200          # the oracle's set logic is O(N^2) Python work per (sample, class)
    yield "random", rng.integers(20, 90, (1 if big else 3, n))
    yield "all-equal", np.full((1 if big else 2, n), 37)
    alt = np.tile(np.array([30, 80]), (n + 1) // 2)[None, :n]
    yield "alternating", alt
    if big:
        return
    one = np.full((1, n), 30)
    one[0, n // 2] = 80
    yield "one-literal", one
    yield "mixed-batch", np.stack([np.full(n, 5), rng.integers(1, 200, n), np.arange(n) + 1])


@pytest.mark.parametrize("n", [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 500, 1023, 1024])
def test_mask_size_patterns(n):
    rng = np.random.default_rng(n)
    windows = (0, 1, 2, 4, n + 5) if n <= 200 else (0, 4)
    for window in windows:
        for name, c in _c_patterns(n, rng):
            c = np.ascontiguousarray(c.astype(np.int32))
            heads = (2, 1, 1) if n < 600 else (1, 1, 1)
            log(f"  mask N={n} w={window} {name} B={c.shape[0]}")
            m = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), window, heads)
            torch.cuda.synchronize()
            check_mask(m, c, 64, window, heads)


@pytest.mark.parametrize("batch", [127, 128, 129, 200])
def test_mask_batch_sizes(batch):
    # the work order is built in one launch while a list's histogram fits in LDS (up to
    # 128 samples) and in two above that; both must give the same descriptors
    rng = np.random.default_rng(batch)
    c = rng.integers(20, 90, (batch, 9)).astype(np.int32)
    c[::7] = 40                                   # some samples without literal blocks
    log(f"  mask B={batch} N=9")
    m = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), 1, (2, 1, 1))
    torch.cuda.synchronize()
    check_mask(m, c, 64, 1, (2, 1, 1))


@pytest.mark.parametrize("heads", [(4, 0, 0), (0, 3, 0), (0, 0, 2), (0, 0, 0), (3, 1, 5)])
def test_mask_head_splits(heads):
    rng = np.random.default_rng(9)
    c = rng.integers(20, 90, (4, 33)).astype(np.int32)
    log(f"  mask heads={heads}")
    m = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), 2, heads)
    torch.cuda.synchronize()
    check_mask(m, c, 64, 2, heads)


def test_mask_deterministic_and_reusable():
    rng = np.random.default_rng(4)
    c = rng.integers(20, 150, (2, 512)).astype(np.int32)
    a = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), 4, (8, 4, 4))
    b = gsa.gsa_build_mask(torch.from_numpy(c).cuda(), 4, (8, 4, 4))
    # rebuild into the same buffers from different sizes, then back
    c2 = rng.integers(20, 150, (2, 512)).astype(np.int32)
    gsa.gsa_build_mask(torch.from_numpy(c2).cuda(), 4, (8, 4, 4), out=b)
    gsa.gsa_build_mask(torch.from_numpy(c).cuda(), 4, (8, 4, 4), out=b)
    torch.cuda.synchronize()
    for f in gsa.MASK_FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        if f in ("col_idx", "row_idx", "sched"):
            continue            # entries past each segment's total, and the scratch, are unspecified
        assert torch.equal(x, y), f
    check_mask(b, c, 64, 4, (8, 4, 4))
