"""CPU oracle for gzip-guided block-sparse causal attention (fp64, plain and slow).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run this
module: only the tests, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, tables or helpers with the HIP library;
both sides receive the same seeded inputs from the ``synth`` package and nothing else.

Sources (web pages, cited by title and section):

* [note] "Gzip-guided Sparse Attention：用压缩率选择长程内容", the daiwk.github.io
  auto-research reproduction of arXiv 2607.21752.  Sections used: 背景与主要改动
  (head split, no fixed global tokens, every block keeps a local window), the
  flowchart under it (bytes -> fixed blocks -> gzip level 1 per block -> ratios ->
  above-mean literal blocks -> literal/local edges -> causal adaptive mask),
  核心公式 (first display: ratio r_i and literal flag; second display: the mask
  M = M^lit U M^local U I intersected with the causal mask; third display: the
  O(L^2 + N w) edge bound) and 复现边界 (the reproduction computes the dense score
  matrix and then masks).
* [abstract] "Parameter-free Adaptive Sparse Attention via Compression-Based Content
  Selection" (newx.sg summary), Abstract: per-block gzip ratios, no extra parameters,
  no architectural change to the Transformer.

Readings where the pages leave a step open (each one is the plainest reading the
rest supports):

* gzip container: one whole gzip member per block (RFC 1952 header + deflate body +
  CRC32/ISIZE trailer) from zlib at level 1, windowBits 15, memLevel 8, default
  strategy.  The literal flag depends only on differences of lengths, so any
  constant container overhead cancels.
* The mean r-bar is over the blocks of one sample, never over the batch.
* Literal test is strict (a block exactly at the mean is not literal), evaluated in
  exact rational arithmetic.
* Window: block distance |i - j| <= w, then causality j <= i.  Inside the diagonal
  block causality is token level (key position <= query position); off-diagonal kept
  blocks are fully visible.
* Head classes in order local | literal | hybrid.  Local = M^local U I, literal =
  M^lit U I (a non-literal query block then sees only itself), hybrid = all three.
* Softmax scale 1/sqrt(d) unless given; no dropout, bias or global tokens.
* Attention is the dense masked softmax.  Rows are evaluated one query block at a
  time over the causal prefix of keys [0, (i+1) b): every key beyond the prefix is
  masked by causality and would add an exact zero, and each row's softmax is
  independent of the others, so this is the same arithmetic as the full T x T form.

Pins: every public function here is checked in tests/test_oracle_*.py against the
gzip format (RFC 1952), worked examples derived by hand from the formulas, closed
forms of the edge counts, brute-force properties, special cases that reduce to
torch's scaled_dot_product_attention, and central finite differences.
"""

from __future__ import annotations

import zlib
from fractions import Fraction

import numpy as np

LOCAL, LITERAL, HYBRID = 0, 1, 2
CLASS_NAMES = ("local", "literal", "hybrid")

# gzip as the [note] flowchart names it ("level 1 per block"): zlib deflate level 1,
# windowBits 15 with +16 selecting the gzip wrapper, memLevel 8, default strategy.
GZIP_LEVEL = 1
GZIP_WBITS = 16 + 15
GZIP_MEMLEVEL = 8


def zlib_runtime_version() -> str:
    """Version string of the libz that Python's zlib module is linked against."""
    return zlib.ZLIB_RUNTIME_VERSION


def gzip_member(block: bytes) -> bytes:
    """The gzip member (RFC 1952) of one block, compressed at level 1.  [note] flowchart."""
    co = zlib.compressobj(GZIP_LEVEL, zlib.DEFLATED, GZIP_WBITS, GZIP_MEMLEVEL,
                          zlib.Z_DEFAULT_STRATEGY)
    return co.compress(block) + co.flush(zlib.Z_FINISH)


def gzip_length(block: bytes) -> int:
    """|gzip(x)|: length in bytes of the level-1 gzip member.  [note] 核心公式, first display."""
    return len(gzip_member(block))


def compressed_lengths(data, block: int) -> np.ndarray:
    """c[s, i] = |gzip(x_s[i b:(i+1) b])| for every sample s and block i.

    [note] 核心公式 first display; blocks are 0-based half-open byte ranges.
    ``data`` is uint8 [B, T] with T a multiple of ``block``.
    """
    data = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    if data.ndim != 2:
        raise ValueError("data must be [batch, seq_len]")
    batch, seq_len = data.shape
    if block <= 0 or seq_len % block:
        raise ValueError("seq_len must be a positive multiple of block")
    n = seq_len // block
    out = np.zeros((batch, n), dtype=np.int64)
    for s in range(batch):
        for i in range(n):
            out[s, i] = gzip_length(data[s, i * block:(i + 1) * block].tobytes())
    return out


def literal_flags(c, block: int):
    """Literal flags l_i = 1[r_i > r_bar], r_i = c_i / b, r_bar = mean of r over the sample.

    [note] 核心公式 first display; "above the sample mean" in 背景与主要改动.
    Exact rationals, strict comparison.  Returns (flags bool [B, N], L int64 [B]).
    """
    c = np.asarray(c)
    batch, n = c.shape
    flags = np.zeros((batch, n), dtype=bool)
    for s in range(batch):
        r = [Fraction(int(ci), block) for ci in c[s]]
        r_bar = sum(r, Fraction(0)) / n
        for i in range(n):
            flags[s, i] = r[i] > r_bar
    return flags, flags.sum(axis=1).astype(np.int64)


def block_mask(flags_row, window: int, cls: int) -> np.ndarray:
    """N x N boolean block mask of one sample for one head class, by set logic.

    [note] 核心公式 second display: M = M^lit U M^local U I with
    M^lit_ij = 1[l_i = l_j = 1], M^local_ij = 1[|i - j| <= w], I the identity,
    intersected with the causal mask; head classes from 背景与主要改动.
    """
    flags_row = [bool(x) for x in flags_row]
    n = len(flags_row)
    lit_blocks = {i for i in range(n) if flags_row[i]}
    m_lit = {(i, j) for i in lit_blocks for j in lit_blocks}
    m_local = {(i, j) for i in range(n) for j in range(n) if abs(i - j) <= window}
    ident = {(i, i) for i in range(n)}
    causal = {(i, j) for i in range(n) for j in range(i + 1)}
    if cls == LOCAL:
        m = m_local | ident
    elif cls == LITERAL:
        m = m_lit | ident
    elif cls == HYBRID:
        m = m_lit | m_local | ident
    else:
        raise ValueError("class must be LOCAL, LITERAL or HYBRID")
    m &= causal
    out = np.zeros((n, n), dtype=bool)
    for i, j in m:
        out[i, j] = True
    return out


def block_masks(flags, window: int) -> np.ndarray:
    """All masks: bool [B, 3, N, N], class order local | literal | hybrid."""
    flags = np.asarray(flags, dtype=bool)
    batch, n = flags.shape
    out = np.zeros((batch, 3, n, n), dtype=bool)
    for s in range(batch):
        for cls in (LOCAL, LITERAL, HYBRID):
            out[s, cls] = block_mask(flags[s], window, cls)
    return out


def default_head_counts(heads: int):
    """Heads per class: half local, a quarter literal, the rest hybrid.  [note] 背景与主要改动."""
    n_local = heads // 2
    n_literal = heads // 4
    return (n_local, n_literal, heads - n_local - n_literal)


def bigbird_block_mask(n: int, window: int, n_global: int, picks) -> np.ndarray:
    """BigBird-style causal block mask (the baseline the pages compare against in
    [note] 论文离线与线上效果; its parameters are not on the pages, so they are inputs).

    Query block i keeps key block j <= i when j is in the window (i - j <= window), j is
    a global block (j < n_global), i is a global block (i < n_global: it sees every
    earlier block), or j is one of row i's random picks ``picks[i]``.  Set logic.
    """
    out = np.zeros((n, n), dtype=bool)
    for i in range(n):
        keep = set(range(max(0, i - window), i + 1))
        keep |= set(range(min(n_global, i + 1)))
        if i < n_global:
            keep |= set(range(i + 1))
        keep |= {int(j) for j in picks[i] if 0 <= int(j) <= i}
        for j in keep:
            out[i, j] = True
    return out


def bigbird_masks(picks, window: int, n_global: int) -> np.ndarray:
    """bool [B, 3, N, N]: class 0 the BigBird-style mask of each sample's picks [N, r],
    classes 1 and 2 the diagonal only (every head of a BigBird run is class 0)."""
    picks = np.asarray(picks)
    batch, n = picks.shape[0], picks.shape[1]
    out = np.zeros((batch, 3, n, n), dtype=bool)
    for s in range(batch):
        out[s, 0] = bigbird_block_mask(n, window, n_global, picks[s])
        out[s, 1] = out[s, 2] = np.eye(n, dtype=bool)
    return out


def head_classes(n_heads) -> list:
    """Class of every head, contiguous in the order local | literal | hybrid."""
    return [LOCAL] * n_heads[0] + [LITERAL] * n_heads[1] + [HYBRID] * n_heads[2]


def to_csr(mask: np.ndarray):
    """Row lists of an N x N boolean mask, ascending column: (row_ptr [N+1], col_idx [E])."""
    n = mask.shape[0]
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    cols = []
    for i in range(n):
        js = [j for j in range(n) if mask[i, j]]
        cols.extend(js)
        row_ptr[i + 1] = row_ptr[i] + len(js)
    return row_ptr, np.array(cols, dtype=np.int64)


def to_csc(mask: np.ndarray):
    """Column lists, ascending row: (col_ptr [N+1], row_idx [E])."""
    return to_csr(np.ascontiguousarray(mask.T))


def token_mask(bmask: np.ndarray, block: int, rows=None, keys=None) -> np.ndarray:
    """A[t, u] = M[t // b, u // b] and u <= t.

    Causality at token level as in [note] 核心公式 ("intersected with the causal mask").
    ``rows`` selects query positions and ``keys`` key positions (default all of [0, T)).
    """
    n = bmask.shape[0]
    seq_len = n * block
    t = np.arange(seq_len) if rows is None else np.asarray(rows)
    u = np.arange(seq_len) if keys is None else np.asarray(keys)
    return bmask[t[:, None] // block, u[None, :] // block] & (u[None, :] <= t[:, None])


def _scale(head_dim: int, scale):
    return 1.0 / np.sqrt(head_dim) if not scale else float(scale)


def kept_keys(bmask: np.ndarray, block: int, i: int) -> np.ndarray:
    """Token positions of the key blocks that query block i keeps (row i of ``bmask``,
    causal part), ascending."""
    js = np.nonzero(bmask[i, :i + 1])[0]
    return (js[:, None] * block + np.arange(block)[None, :]).ravel()


def _rows_forward(q, k, v, bmask, block, scale, rows, keys=None):
    """Dense masked softmax attention for the query positions ``rows`` of one head.

    Scores over the key positions ``keys`` (default: the causal prefix
    [0, max(rows)+1)), masked entries set to -inf, max-subtracted softmax, O = P V,
    LSE = log sum exp of the masked scores.  Any key outside ``keys`` must be masked
    for every row; it would carry weight exactly zero, so leaving it out changes nothing.
    """
    rows = np.asarray(rows)
    if keys is None:
        keys = np.arange(int(rows.max()) + 1)
    a = token_mask(bmask, block, rows, keys)
    s = scale * (q[rows] @ k[keys].T)
    s = np.where(a, s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    p = p / l[:, None]
    o = p @ v[keys]
    lse = m + np.log(l)
    return o, lse, p, a


def attn_fwd(q, k, v, bmasks, n_heads, block: int, scale=None):
    """Forward of the masked attention for every (sample, head).

    q, k, v: float arrays [B, H, T, d] (upcast to fp64); bmasks: bool [B, 3, N, N].
    Returns O fp64 [B, H, T, d] and LSE fp64 [B, H, T] (natural log).
    [note] 核心公式 second display for the mask; 复现边界 for dense-then-mask.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    batch, heads, seq_len, d = q.shape
    sc = _scale(d, scale)
    classes = head_classes(n_heads)
    o = np.zeros_like(q)
    lse = np.zeros((batch, heads, seq_len))
    n = seq_len // block
    for s in range(batch):
        for h in range(heads):
            bm = bmasks[s, classes[h]]
            for i in range(n):
                rows = np.arange(i * block, (i + 1) * block)
                oo, ll, _, _ = _rows_forward(q[s, h], k[s, h], v[s, h], bm, block, sc, rows)
                o[s, h, rows] = oo
                lse[s, h, rows] = ll
    return o, lse


def attn_fwd_rows(q, k, v, bmask, block: int, rows, scale=None):
    """Forward for selected query rows of ONE head (q, k, v: [T, d]); for sampled checks."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    o, lse, _, _ = _rows_forward(q, k, v, bmask, block, _scale(q.shape[1], scale), rows)
    return o, lse


def _qblock_backward(q, k, v, do, bmask, block, sc, i):
    """Backward pieces of query block i of one head (standard softmax calculus).

    Returns (dq_rows, dk_prefix, dv_prefix, prefix): dV = P^T dO, dP = dO V^T,
    D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
    """
    rows = np.arange(i * block, (i + 1) * block)
    o, _, p, _ = _rows_forward(q, k, v, bmask, block, sc, rows)
    prefix = (i + 1) * block
    dov = do[rows]
    dv = p.T @ dov
    dp = dov @ v[:prefix].T
    dd = (dov * o).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = sc * (ds @ k[:prefix])
    dk = sc * (ds.T @ q[rows])
    return dq, dk, dv, prefix


def attn_bwd(q, k, v, do, bmasks, n_heads, block: int, scale=None):
    """Gradients dQ, dK, dV (fp64 [B, H, T, d]) of sum(O * dO) w.r.t. q, k, v."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    batch, heads, seq_len, d = q.shape
    sc = _scale(d, scale)
    classes = head_classes(n_heads)
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    n = seq_len // block
    for s in range(batch):
        for h in range(heads):
            bm = bmasks[s, classes[h]]
            for i in range(n):
                g_q, g_k, g_v, prefix = _qblock_backward(q[s, h], k[s, h], v[s, h], do[s, h],
                                                        bm, block, sc, i)
                dq[s, h, i * block:(i + 1) * block] = g_q
                dk[s, h, :prefix] += g_k
                dv[s, h, :prefix] += g_v
    return dq, dk, dv


def attn_bwd_qblock(q, k, v, do, bmask, block: int, i: int, scale=None):
    """dQ rows of query block i of ONE head ([T, d] inputs); for sampled checks."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    g_q, _, _, _ = _qblock_backward(q, k, v, do, bmask, block, _scale(q.shape[1], scale), i)
    return g_q


def attn_bwd_kblock(q, k, v, do, bmask, block: int, j: int, scale=None):
    """dK, dV rows of key block j of ONE head, summed over every query block that keeps j.

    Query blocks that do not keep block j contribute exact zeros to it, so only the
    column list of j is visited.  Each such query block i takes its softmax over the keys
    of the blocks its row keeps (every other key is masked: weight exactly zero under
    [note] 核心公式 second display), and only block j's columns of the backward are
    formed: with P_i the kept softmax of i's rows, O_i = P_i V, D_i = rowsum(dO_i * O_i)
    and P_ij the columns of P_i that belong to block j,
      dV_j += P_ij^T dO_i,   dS_ij = P_ij * (dO_i V_j^T - D_i),   dK_j += scale dS_ij^T Q_i.
    For sampled checks at full size.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    sc = _scale(q.shape[1], scale)
    n = bmask.shape[0]
    cols = np.arange(j * block, (j + 1) * block)
    dk = np.zeros((block, q.shape[1]))
    dv = np.zeros((block, q.shape[1]))
    for i in range(j, n):
        if not bmask[i, j]:
            continue
        rows = np.arange(i * block, (i + 1) * block)
        keys = kept_keys(bmask, block, i)
        o, _, p, _ = _rows_forward(q, k, v, bmask, block, sc, rows, keys)
        dov = do[rows]
        dd = (dov * o).sum(axis=1)
        p_j = p[:, np.searchsorted(keys, cols)]
        dv += p_j.T @ dov
        ds = p_j * (dov @ v[cols].T - dd[:, None])
        dk += sc * (ds.T @ q[rows])
    return dk, dv
