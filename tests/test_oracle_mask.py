"""Pins of the oracle's literal flags and block masks.

Flags: worked examples from the ratio formula ("Gzip-guided Sparse Attention",
核心公式 first display) plus invariances that hold for r_i > mean(r).
Masks: worked examples from the mask formula (核心公式 second display), closed-form
edge counts derived independently of set logic, and the O(L^2 + N w) bound
(核心公式 third display).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ flags
@pytest.mark.parametrize("case", _load("flags_worked.json")["cases"])
def test_flags_worked_examples(case):
    c = np.array(case["c"])
    flags, n_lit = oracle.literal_flags(c, case["block"])
    assert flags.astype(int).tolist() == case["flags"], case["why"]
    assert n_lit.tolist() == [sum(r) for r in case["flags"]]


def test_flags_invariances():
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        b = int(rng.choice([16, 64, 128]))
        c = rng.integers(20, b + 24, (1, n))
        f, n_lit = oracle.literal_flags(c, b)
        # constant shift and positive scaling of all lengths keep the flags
        assert np.array_equal(oracle.literal_flags(c + 17, b)[0], f)
        assert np.array_equal(oracle.literal_flags(c * 3, b)[0], f)
        # the block size only rescales every ratio
        assert np.array_equal(oracle.literal_flags(c, 2 * b)[0], f)
        # permutation equivariance
        p = rng.permutation(n)
        assert np.array_equal(oracle.literal_flags(c[:, p], b)[0], f[:, p])
        # at least one block is at or below the mean; L = 0 iff all lengths are equal
        assert n_lit[0] <= n - 1
        assert (n_lit[0] == 0) == bool(np.all(c == c[0, 0]))


def test_repeated_bytes_give_no_literals():
    # A sample made of one repeated byte has identical blocks, so every ratio equals the mean.
    data = np.full((2, 64 * 16), ord("q"), dtype=np.uint8)
    data[1] = np.resize(np.frombuffer(b"abcdefgh", np.uint8), 64 * 16)  # period 8 divides b
    c = oracle.compressed_lengths(data, 64)
    _, n_lit = oracle.literal_flags(c, 64)
    assert n_lit.tolist() == [0, 0]


# ------------------------------------------------------------------ masks
@pytest.mark.parametrize("case", _load("mask_worked.json")["cases"])
def test_mask_worked_examples(case):
    for cls, name in enumerate(oracle.CLASS_NAMES):
        m = oracle.block_mask(case["flags"], case["window"], cls)
        rows = [[j for j in range(m.shape[1]) if m[i, j]] for i in range(m.shape[0])]
        assert rows == case[name], name
        assert int(m.sum()) == case["edges"][cls]


def _closed_forms(flags, w):
    """Edge counts derived from the row structure, not from set logic."""
    n = len(flags)
    lit = [i for i in range(n) if flags[i]]
    n_lit = len(lit)
    e_local = n * (w + 1) - w * (w + 1) // 2 if n > w else n * (n + 1) // 2
    e_lit = n_lit * (n_lit + 1) // 2 + (n - n_lit)
    p_w = sum(1 for i in lit for j in lit if 0 <= i - j <= w)
    e_hyb = e_local + n_lit * (n_lit + 1) // 2 - p_w
    return e_local, e_lit, e_hyb


def test_edge_counts_closed_form_and_bound():
    rng = np.random.default_rng(11)
    for _ in range(400):
        n = int(rng.integers(1, 48))
        w = int(rng.integers(0, 7))
        flags = rng.random(n) < rng.random()
        m = oracle.block_masks(flags[None, :], w)[0]
        e = [int(m[c].sum()) for c in range(3)]
        assert tuple(e) == _closed_forms(flags, w), (n, w, flags)
        n_lit = int(flags.sum())
        assert e[2] <= n_lit * (n_lit + 1) // 2 + n * (w + 1)      # O(L^2 + N w)


def test_mask_special_cases():
    rng = np.random.default_rng(5)
    for n in (1, 2, 7, 16):
        tri = np.tril(np.ones((n, n), bool))
        flags = rng.random(n) < 0.4
        # window covering the whole sequence: local heads are plain causal attention
        assert np.array_equal(oracle.block_mask(flags, n - 1, oracle.LOCAL), tri)
        assert np.array_equal(oracle.block_mask(flags, n + 3, oracle.HYBRID), tri)
        # no literal blocks: literal heads see only their own block, hybrid equals local
        none = np.zeros(n, bool)
        assert np.array_equal(oracle.block_mask(none, 2, oracle.LITERAL), np.eye(n, dtype=bool))
        assert np.array_equal(oracle.block_mask(none, 2, oracle.HYBRID),
                              oracle.block_mask(none, 2, oracle.LOCAL))
        # every block literal: literal heads are causal
        assert np.array_equal(oracle.block_mask(np.ones(n, bool), 0, oracle.LITERAL), tri)
        # window 0: local heads are block diagonal
        assert np.array_equal(oracle.block_mask(flags, 0, oracle.LOCAL), np.eye(n, dtype=bool))


def test_mask_invariants():
    rng = np.random.default_rng(8)
    for _ in range(100):
        n = int(rng.integers(2, 40))
        w = int(rng.integers(0, 5))
        flags = rng.random(n) < 0.3
        m = oracle.block_masks(flags[None], w)[0]
        for cls in range(3):
            assert np.all(np.diag(m[cls]))                 # self connection
            assert not np.any(np.triu(m[cls], 1))          # causal
        # no fixed global blocks: a non-literal block beyond the window sees nothing far back
        for i in range(n):
            if not flags[i]:
                far = [j for j in range(n) if m[2, i, j] and i - j > w]
                assert far == []
                assert [j for j in range(n) if m[1, i, j]] == [i]
        # literal edges only join literal blocks
        for i in range(n):
            for j in range(i):
                if m[1, i, j]:
                    assert flags[i] and flags[j]
        assert np.array_equal(m[2], m[0] | m[1])


def test_csr_csc():
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(1, 30))
        m = rng.random((n, n)) < 0.3
        rp, ci = oracle.to_csr(m)
        cp, ri = oracle.to_csc(m)
        assert rp[-1] == m.sum() == cp[-1]
        for i in range(n):
            seg = ci[rp[i]:rp[i + 1]]
            assert np.all(np.diff(seg) > 0)
            assert set(seg.tolist()) == set(np.nonzero(m[i])[0].tolist())
        for j in range(n):
            seg = ri[cp[j]:cp[j + 1]]
            assert np.all(np.diff(seg) > 0)
            assert set(seg.tolist()) == set(np.nonzero(m[:, j])[0].tolist())


def test_head_classes():
    assert oracle.default_head_counts(4) == (2, 1, 1)
    assert oracle.default_head_counts(12) == (6, 3, 3)
    assert oracle.default_head_counts(16) == (8, 4, 4)
    assert oracle.default_head_counts(6) == (3, 1, 2)
    assert oracle.head_classes((2, 1, 1)) == [0, 0, 1, 2]


def test_token_mask():
    bm = oracle.block_mask([0, 1, 0, 1], 0, oracle.LITERAL)
    a = oracle.token_mask(bm, 2)
    # token (t=7, block 3) sees block 1 fully and itself causally, nothing else
    assert np.nonzero(a[7])[0].tolist() == [2, 3, 6, 7]
    assert np.nonzero(a[6])[0].tolist() == [2, 3, 6]
    assert np.nonzero(a[4])[0].tolist() == [4]
    assert np.nonzero(a[0])[0].tolist() == [0]
