"""Pins of the oracle's attention forward and backward.

The forward is the masked softmax attention the pages describe (dense scores, then
the adaptive causal mask: "Gzip-guided Sparse Attention", 核心公式 second display and
复现边界).  It is pinned to torch's scaled_dot_product_attention (an independent
library routine) in the special cases where the gzip mask reduces to a standard
mask, and with an explicit boolean mask in general; the backward is pinned to torch
autograd of that routine and to central finite differences of the oracle's own
forward.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _masks_for(flags, w):
    return oracle.block_masks(np.asarray(flags, bool), w)


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64)
    out = F.scaled_dot_product_attention(t(q), t(k), t(v),
                                         attn_mask=None if mask is None else torch.from_numpy(mask),
                                         is_causal=causal, scale=scale)
    return out.numpy()


def test_full_window_is_causal_attention():
    b, n, d = 8, 6, 16
    q, k, v = (_rand((1, 2, n * b, d), s) for s in (1, 2, 3))
    bm = _masks_for([[0, 1, 0, 0, 1, 0]], n - 1)
    o, lse = oracle.attn_fwd(q, k, v, bm, (2, 0, 0), b)
    ref = _sdpa(q, k, v, causal=True)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_single_block_is_causal_attention_for_every_class():
    b, d = 16, 8
    q, k, v = (_rand((2, 3, b, d), s) for s in (4, 5, 6))
    bm = _masks_for([[1], [0]], 2)
    o, _ = oracle.attn_fwd(q, k, v, bm, (1, 1, 1), b)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=0, atol=1e-12)


def test_no_literals_literal_heads_are_block_diagonal():
    b, n, d = 4, 5, 8
    q, k, v = (_rand((1, 1, n * b, d), s) for s in (7, 8, 9))
    bm = _masks_for([[0] * n], 1)
    o, _ = oracle.attn_fwd(q, k, v, bm, (0, 1, 0), b)
    for i in range(n):
        sl = slice(i * b, (i + 1) * b)
        ref = _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], causal=True)
        np.testing.assert_allclose(o[:, :, sl], ref, rtol=0, atol=1e-12)


def test_general_mask_matches_sdpa_with_explicit_mask_and_logsumexp():
    b, n, d = 4, 9, 8
    flags = [[0, 1, 0, 1, 1, 0, 0, 1, 0]]
    w = 1
    q, k, v = (_rand((1, 3, n * b, d), s) for s in (10, 11, 12))
    bm = _masks_for(flags, w)
    sc = 0.37
    o, lse = oracle.attn_fwd(q, k, v, bm, (1, 1, 1), b, scale=sc)
    for h in range(3):
        a = oracle.token_mask(bm[0, h], b)
        ref = _sdpa(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], mask=a, scale=sc)
        np.testing.assert_allclose(o[:, h:h + 1], ref, rtol=0, atol=1e-12)
        s = torch.from_numpy(sc * q[0, h] @ k[0, h].T).masked_fill(~torch.from_numpy(a), -np.inf)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_first_row_is_v0_and_rows_are_convex_combinations():
    b, n, d = 8, 4, 16
    q, k, v = (_rand((2, 3, n * b, d), s) for s in (13, 14, 15))
    bm = _masks_for([[1, 0, 1, 1], [0, 0, 0, 1]], 1)
    o, _ = oracle.attn_fwd(q, k, v, bm, (1, 1, 1), b)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    # every output lies within the per-column range of the visible values
    assert np.all(o <= v.max(axis=2, keepdims=True) + 1e-12)
    assert np.all(o >= v.min(axis=2, keepdims=True) - 1e-12)


def test_locality_outside_kept_blocks():
    b, n, d = 4, 8, 8
    flags = [[0, 1, 0, 0, 1, 0, 1, 0]]
    bm = _masks_for(flags, 1)
    q, k, v = (_rand((1, 3, n * b, d), s) for s in (16, 17, 18))
    o, _ = oracle.attn_fwd(q, k, v, bm, (1, 1, 1), b)
    for h in range(3):
        for i in range(n):
            k2, v2 = k.copy(), v.copy()
            for j in range(n):
                if not bm[0, h, i, j]:
                    k2[0, h, j * b:(j + 1) * b] += 5.0
                    v2[0, h, j * b:(j + 1) * b] -= 3.0
            o2, _ = oracle.attn_fwd(q, k2, v2, bm, (1, 1, 1), b)
            assert np.array_equal(o2[0, h, i * b:(i + 1) * b], o[0, h, i * b:(i + 1) * b])


def test_row_and_block_helpers_agree_with_full():
    b, n, d = 4, 6, 8
    bm = _masks_for([[1, 0, 1, 1, 0, 1]], 1)
    q, k, v, do = (_rand((1, 3, n * b, d), s) for s in (19, 20, 21, 22))
    o, lse = oracle.attn_fwd(q, k, v, bm, (1, 1, 1), b)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, bm, (1, 1, 1), b)
    for h in range(3):
        rows = [0, 5, 13, 23]
        orow, lrow = oracle.attn_fwd_rows(q[0, h], k[0, h], v[0, h], bm[0, h], b, rows)
        np.testing.assert_allclose(orow, o[0, h, rows], atol=1e-13)
        np.testing.assert_allclose(lrow, lse[0, h, rows], atol=1e-13)
        for i in range(n):
            g = oracle.attn_bwd_qblock(q[0, h], k[0, h], v[0, h], do[0, h], bm[0, h], b, i)
            np.testing.assert_allclose(g, dq[0, h, i * b:(i + 1) * b], atol=1e-13)
            gk, gv = oracle.attn_bwd_kblock(q[0, h], k[0, h], v[0, h], do[0, h], bm[0, h], b, i)
            np.testing.assert_allclose(gk, dk[0, h, i * b:(i + 1) * b], atol=1e-13)
            np.testing.assert_allclose(gv, dv[0, h, i * b:(i + 1) * b], atol=1e-13)


def test_backward_matches_torch_autograd():
    b, n, d = 4, 7, 8
    flags = [[0, 1, 1, 0, 0, 1, 0], [1, 0, 0, 0, 1, 0, 0]]
    bm = _masks_for(flags, 1)
    nh = (1, 1, 1)
    q, k, v, do = (_rand((2, 3, n * b, d), s) for s in (23, 24, 25, 26))
    sc = 0.41
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, bm, nh, b, scale=sc)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    classes = oracle.head_classes(nh)
    mask = np.stack([np.stack([oracle.token_mask(bm[s, classes[h]], b) for h in range(3)])
                     for s in range(2)])
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=sc)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_backward_finite_differences():
    b, n, d = 4, 5, 6
    bm = _masks_for([[0, 1, 0, 1, 1]], 1)
    nh = (1, 1, 1)
    q, k, v, do = (_rand((1, 3, n * b, d), s) for s in (27, 28, 29, 30))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, bm, nh, b)

    def loss(q_, k_, v_):
        o, _ = oracle.attn_fwd(q_, k_, v_, bm, nh, b)
        return float((o * do).sum())

    rng = np.random.default_rng(31)
    eps = 1e-6
    for which, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(12):
            idx = (0, int(rng.integers(3)), int(rng.integers(n * b)), int(rng.integers(d)))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[which][idx] += eps
            up = loss(args["q"], args["k"], args["v"])
            args[which][idx] -= 2 * eps
            dn = loss(args["q"], args["k"], args["v"])
            assert abs((up - dn) / (2 * eps) - grad[idx]) < 1e-7, (which, idx)


def test_backward_invariants():
    b, n, d = 8, 6, 8
    bm = _masks_for([[0, 1, 1, 0, 1, 0]], 2)
    q, k, v, do = (_rand((1, 3, n * b, d), s) for s in (32, 33, 34, 35))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, bm, (1, 1, 1), b)
    # softmax rows sum to one, so each row of dS sums to zero and so does sum_u dK_u
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # dO = 0 gives zero gradients
    z = oracle.attn_bwd(q, k, v, np.zeros_like(do), bm, (1, 1, 1), b)
    assert all(np.all(g == 0) for g in z)
    # dO = 1 gives dV_u = sum over rows of P[t, u] (column sums of P), which sum to T
    _, _, dv1 = oracle.attn_bwd(q, k, v, np.ones_like(do), bm, (1, 1, 1), b)
    np.testing.assert_allclose(dv1[..., 0].sum(axis=2), n * b, atol=1e-10)
    assert np.allclose(dv1[..., 0:1], dv1)


def test_kept_keys_is_the_union_of_visible_positions():
    # brute force: position u belongs to row i's kept keys iff some query of block i may
    # see it, i.e. its block is kept by row i and lies at or before i
    b, n = 3, 7
    bm = _masks_for([[1, 0, 1, 0, 0, 1, 1]], 1)[0, 2]
    for i in range(n):
        want = [u for u in range(n * b) if u // b <= i and bm[i, u // b]]
        assert oracle.kept_keys(bm, b, i).tolist() == want


def test_kblock_matches_torch_autograd_on_long_columns():
    # every block literal and w = 0 in the literal class: column j is kept by every
    # query block i >= j, so column 0 has n entries
    b, n, d = 4, 12, 8
    bm = _masks_for([[1] * n], 0)
    q, k, v, do = (_rand((1, 1, n * b, d), s) for s in (36, 37, 38, 39))
    sc = 0.29
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    a = oracle.token_mask(bm[0, 1], b)
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(a), scale=sc)
    out.backward(torch.from_numpy(do))
    for j in (0, 1, n // 2, n - 1):
        gk, gv = oracle.attn_bwd_kblock(q[0, 0], k[0, 0], v[0, 0], do[0, 0], bm[0, 1], b, j, scale=sc)
        sl = slice(j * b, (j + 1) * b)
        np.testing.assert_allclose(gk, tk.grad.numpy()[0, 0, sl], atol=1e-12)
        np.testing.assert_allclose(gv, tv.grad.numpy()[0, 0, sl], atol=1e-12)
