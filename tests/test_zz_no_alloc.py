"""gsa_build_mask_noalloc (the mask call that allocates nothing) against gsa_build_mask.

Two calls in a row on one GPU, the second with a smaller input, each compared bit for
bit with gsa_build_mask on the same sizes (every buffer but sched, which the
no-allocation call does not use); the second call must not see anything the first left
in the shared scratch.  Oversized batches are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import content_adaptive_block_amd as gsa
import synth
from gpu_cases import log

pytestmark = pytest.mark.gpu

COMPARED = [f for f in gsa.MASK_FIELDS if f != "sched"]


def _both(wl, batch, n_blocks, window, n_heads):
    x = synth.gen_bytes(wl, batch=batch, seq_len=n_blocks * wl.block)
    c = torch.from_numpy(gsa.gsa_prepare(x, wl.block)).cuda()
    ref = gsa.gsa_build_mask(c, window, n_heads)
    out = gsa.GsaMask.empty(batch, n_blocks, window, n_heads, "cuda")
    for f in gsa.MASK_FIELDS:
        getattr(out, f).fill_(-1 if getattr(out, f).dtype != torch.uint8 else 255)
    torch.cuda.synchronize()
    return c, ref, out


def test_noalloc_matches_build_mask_twice_second_smaller():
    cases = [(synth.WORKLOADS[5], 2, 512, 4, (8, 4, 4)), (synth.WORKLOADS[4], 3, 40, 2, (2, 1, 3))]
    for wl, batch, n, window, n_heads in cases:
        log(f"  noalloc B={batch} N={n} w={window} heads={n_heads}")
        c, ref, out = _both(wl, batch, n, window, n_heads)
        gsa.gsa_build_mask_noalloc(c, window, n_heads, out)
        torch.cuda.synchronize()
        assert out.built
        for f in COMPARED:
            a, b = getattr(out, f), getattr(ref, f)
            if f in ("col_idx", "row_idx"):   # entries past each segment's total are unspecified
                cap = n * (n + 1) // 2
                tot = ref.n_edges.view(batch, 3).cpu().numpy()
                a2, b2 = a.view(batch, 3, cap).cpu().numpy(), b.view(batch, 3, cap).cpu().numpy()
                for s in range(batch):
                    for k in range(3):
                        assert np.array_equal(a2[s, k, :tot[s, k]], b2[s, k, :tot[s, k]]), (f, s, k)
            else:
                assert torch.equal(a, b), f


def test_noalloc_attention_runs_on_its_mask():
    wl = synth.WORKLOADS[4]
    batch, n, n_heads = 2, 16, (2, 1, 1)
    c, ref, out = _both(wl, batch, n, 2, n_heads)
    gsa.gsa_build_mask_noalloc(c, 2, n_heads, out)
    t = synth.gen_tensors(wl, ("q", "k", "v"), batch=batch, heads=4, seq_len=n * 64)
    q, k, v = (t[nm].cuda() for nm in ("q", "k", "v"))
    o1, l1 = gsa.gsa_attn_fwd(q, k, v, ref, 64)
    o2, l2 = gsa.gsa_attn_fwd(q, k, v, out, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_rejects_oversized_batches():
    # 2 * 3 * B * (N + 32) int32 words above GSA_NOALLOC_SCHED_BYTES (2 MiB): B = 100, N = 1024
    lib = gsa.load_library()
    m = gsa._Mask()
    m.batch, m.n_blocks, m.window = 100, 1024, 2
    m.n_heads[:] = [1, 1, 1]
    for f in gsa.MASK_FIELDS:
        setattr(m, f, 0x10000 if f != "sched" else None)
    assert lib.gsa_build_mask_noalloc(0x10000, m, None) == gsa.GSA_ERR_UNSUPPORTED
    assert b"scratch" in lib.gsa_last_error()
    # the largest batch that fits at N = 1024 is accepted by the checks: B = 82 (not run)
    assert 2 * 3 * 82 * (1024 + 32) * 4 <= 2 << 20 < 2 * 3 * 83 * (1024 + 32) * 4
