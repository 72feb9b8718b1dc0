"""GPU checks of the block-mask list builder and the BigBird-style comparison mask.

* gsa_build_mask_from_blocks: lists, edge counts and work descriptors equal the
  oracle's lists of (lower triangle of the given mask, plus the diagonal), bit for bit;
  flags and L are zero.  Masks carry noise above the diagonal and missing diagonal
  entries on purpose (both must be ignored / restored).
* gsa_bigbird_blocks equals the oracle's BigBird-style mask for the same random picks.
* Attention through a BigBird-style mask matches the oracle (same tolerances as the
  gzip mask)."""
import numpy as np
import pytest
import torch

import content_adaptive_block_amd as gsa
import oracle
import synth
from gpu_cases import BF16_TOL, F32_TOL, assert_close, check_lists, f64, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,n,n_heads,density,seed", [
    (1, 1, (1, 0, 0), 0.5, 0), (2, 16, (2, 1, 1), 0.3, 1), (3, 37, (1, 2, 0), 0.1, 2),
    (2, 128, (6, 3, 3), 0.05, 3), (1, 300, (0, 0, 2), 0.02, 4), (1, 1024, (1, 1, 1), 0.003, 5)])
def test_lists_from_given_blocks(batch, n, n_heads, density, seed):
    log(f"  blocks B={batch} N={n} heads={n_heads} density={density}")
    rng = np.random.default_rng(seed)
    raw = rng.random((batch, 3, n, n)) < density          # noise on both sides of the diagonal
    raw[..., np.arange(n), np.arange(n)] &= rng.random((batch, 3, n)) < 0.5   # some diagonals missing
    expect = np.tril(raw) | np.eye(n, dtype=bool)
    m = gsa.gsa_build_mask_from_blocks(torch.from_numpy(raw.astype(np.uint8)).cuda(), n_heads)
    torch.cuda.synchronize()
    assert not m.flags.cpu().numpy().any() and not m.n_literal.cpu().numpy()[:batch].any()
    check_lists(m, expect, n_heads)


@pytest.mark.parametrize("batch,n,w,g,r", [(2, 16, 1, 1, 2), (1, 128, 2, 1, 1), (2, 512, 4, 2, 3), (1, 3, 0, 0, 1)])
def test_bigbird_blocks_match_oracle(batch, n, w, g, r):
    picks = synth.bigbird_picks(synth.WORKLOADS[3], r, batch=batch, n_blocks=n)
    got = gsa.gsa_bigbird_blocks(torch.from_numpy(picks).cuda(), w, g).cpu().numpy().astype(bool)
    assert np.array_equal(got, oracle.bigbird_masks(picks, w, g))


@pytest.mark.parametrize("inst,batch,n,heads,w,g,r", [
    (("bf16", 64, 64), 2, 12, 3, 2, 1, 2), (("f32", 16, 32), 1, 20, 2, 1, 2, 1),
    (("bf16", 128, 128), 1, 8, 2, 1, 1, 1)])
def test_attention_through_bigbird_mask(inst, batch, n, heads, w, g, r):
    dtype, block, hd = inst
    wl = {("f32", 16, 32): synth.WORKLOADS[1], ("bf16", 64, 64): synth.WORKLOADS[3],
          ("bf16", 128, 128): synth.WORKLOADS[5]}[inst]
    log(f"  bigbird attention {dtype} b={block} B={batch} N={n} H={heads} w={w} g={g} r={r}")
    picks = synth.bigbird_picks(wl, r, batch=batch, n_blocks=n)
    t = synth.gen_tensors(wl, ("q", "k", "v", "do"), batch=batch, heads=heads, seq_len=n * block, head_dim=hd)
    n_heads = (heads, 0, 0)
    blocks = gsa.gsa_bigbird_blocks(torch.from_numpy(picks).cuda(), w, g)
    m = gsa.gsa_build_mask_from_blocks(blocks, n_heads)
    q, k, v, do = (t[nm].cuda() for nm in ("q", "k", "v", "do"))
    o, lse = gsa.gsa_attn_fwd(q, k, v, m, block)
    dq, dk, dv = gsa.gsa_attn_bwd(q, k, v, o, lse, do, m, block)
    torch.cuda.synchronize()
    masks = oracle.bigbird_masks(picks, w, g)
    check_lists(m, masks, n_heads)
    ref_o, ref_lse = oracle.attn_fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), masks, n_heads, block)
    ref_g = oracle.attn_bwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), f64(t["do"]), masks, n_heads, block)
    tol, ltol = (F32_TOL, F32_TOL) if dtype == "f32" else (BF16_TOL, 1e-3)
    assert_close("O", f64(o), ref_o, tol)
    assert_close("LSE", f64(lse), ref_lse, ltol)
    for nm, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref_g):
        assert_close(nm, f64(got), ref, tol)
