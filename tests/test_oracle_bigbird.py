"""Pins of the oracle's BigBird-style block mask (a comparison baseline; the pages give
no parameters, so window, global blocks and random picks are inputs).

Pinned by reductions to masks pinned elsewhere and by properties:
* no globals and no picks -> exactly the gzip oracle's local-class mask of the same window;
* as many globals as blocks -> the full causal triangle;
* window >= N - 1 -> the full causal triangle;
* every row holds its window, the global columns, its own picks and nothing above the
  diagonal, and no more than (w + 1) + g + r blocks (or i + 1)."""
import numpy as np
import pytest

import oracle
import synth


def _local(n, w):
    return oracle.block_masks(np.zeros((1, n), dtype=bool), w)[0, oracle.LOCAL]


@pytest.mark.parametrize("n,w", [(1, 0), (5, 1), (12, 2), (40, 4), (9, 20)])
def test_no_globals_no_picks_is_local(n, w):
    picks = np.zeros((n, 0), dtype=np.int32)
    assert np.array_equal(oracle.bigbird_block_mask(n, w, 0, picks), _local(n, w))


@pytest.mark.parametrize("n", [1, 7, 30])
def test_all_global_or_wide_window_is_causal(n):
    rng = np.random.default_rng(n)
    picks = (rng.random((n, 2)) * np.arange(1, n + 1)[:, None]).astype(np.int32)
    tri = np.tril(np.ones((n, n), dtype=bool))
    assert np.array_equal(oracle.bigbird_block_mask(n, 0, n, picks), tri)
    assert np.array_equal(oracle.bigbird_block_mask(n, n - 1, 0, picks), tri)


@pytest.mark.parametrize("seed", range(5))
def test_rows_hold_window_globals_and_picks(seed):
    rng = np.random.default_rng(100 + seed)
    n, w, g, r = int(rng.integers(2, 60)), int(rng.integers(0, 4)), int(rng.integers(0, 3)), int(rng.integers(0, 4))
    picks = (rng.random((n, r)) * np.arange(1, n + 1)[:, None]).astype(np.int32)
    m = oracle.bigbird_block_mask(n, w, g, picks)
    assert not np.triu(m, 1).any()
    assert np.diag(m).all()
    for i in range(n):
        for j in range(max(0, i - w), i + 1):
            assert m[i, j]
        for j in range(min(g, i + 1)):
            assert m[i, j]
        for j in picks[i]:
            assert m[i, j]
        if i < g:
            assert m[i, :i + 1].all()
        assert m[i].sum() <= min(i + 1, (w + 1) + g + r) or i < g


def test_bigbird_masks_classes_and_synth_picks():
    wl = synth.WORKLOADS[3]
    picks = synth.bigbird_picks(wl, 2, batch=3, n_blocks=16)
    assert picks.shape == (3, 16, 2) and picks.dtype == np.int32
    assert (picks >= 0).all() and (picks <= np.arange(16)[None, :, None]).all()
    m = oracle.bigbird_masks(picks, 1, 1)
    assert m.shape == (3, 3, 16, 16)
    for s in range(3):
        assert np.array_equal(m[s, 0], oracle.bigbird_block_mask(16, 1, 1, picks[s]))
        assert np.array_equal(m[s, 1], np.eye(16, dtype=bool)) and np.array_equal(m[s, 2], np.eye(16, dtype=bool))
