"""Shared helpers of the GPU parity tests: expected mask arrays from the oracle, and
running the HIP path through the binding.  No arithmetic of the method lives here:
every expected value comes from ``oracle``."""
import numpy as np
import torch

import content_adaptive_block_amd as gsa
import oracle

BF16_TOL = 2e-2
F32_TOL = 1e-5


def log(msg):
    print(msg, flush=True)


def expected_mask(c: np.ndarray, block: int, window: int):
    """Oracle flags, L, per-(s, class) CSR/CSC lists and edge counts."""
    flags, n_lit = oracle.literal_flags(c, block)
    masks = oracle.block_masks(flags, window)
    b, n = c.shape
    csr = [[oracle.to_csr(masks[s, k]) for k in range(3)] for s in range(b)]
    csc = [[oracle.to_csc(masks[s, k]) for k in range(3)] for s in range(b)]
    return flags, n_lit, masks, csr, csc


def expected_work(masks, n_heads, by_columns: bool):
    """Every (s, h, i) as (s*H + h)*N + i, sorted by the octave of its list length,
    floor(log2 len) + 1, largest first, ties by ascending index."""
    classes = oracle.head_classes(n_heads)
    b, _, n, _ = masks.shape
    lengths = []
    for s in range(b):
        for h in range(len(classes)):
            m = masks[s, classes[h]]
            lengths.append(m.sum(axis=0) if by_columns else m.sum(axis=1))
    lengths = np.concatenate(lengths) if lengths else np.zeros(0, np.int64)
    key = np.array([int(x).bit_length() for x in lengths], dtype=np.int64)
    return np.argsort(-key, kind="stable").astype(np.int64)


def check_lists(m: gsa.GsaMask, masks: np.ndarray, n_heads):
    """Bit-exact comparison of the lists, edge counts and work descriptors of ``m`` with
    the oracle's lists of the block masks ``masks`` bool [B, 3, N, N]."""
    b, _, n, _ = masks.shape
    cap = n * (n + 1) // 2
    row_ptr = m.row_ptr.cpu().numpy().reshape(b, 3, n + 1)
    col_ptr = m.col_ptr.cpu().numpy().reshape(b, 3, n + 1)
    col_idx = m.col_idx.cpu().numpy().reshape(b, 3, cap)
    row_idx = m.row_idx.cpu().numpy().reshape(b, 3, cap)
    n_edges = m.n_edges.cpu().numpy().reshape(b, 3)
    for s in range(b):
        for k in range(3):
            rp, ci = oracle.to_csr(masks[s, k])
            cp, ri = oracle.to_csc(masks[s, k])
            assert np.array_equal(row_ptr[s, k], rp), (s, k)
            assert np.array_equal(col_idx[s, k, :rp[-1]], ci), (s, k)
            assert np.array_equal(col_ptr[s, k], cp), (s, k)
            assert np.array_equal(row_idx[s, k, :cp[-1]], ri), (s, k)
            assert n_edges[s, k] == masks[s, k].sum()
    if sum(n_heads):
        heads = sum(n_heads)
        classes = oracle.head_classes(n_heads)
        for name, by_cols, ptr, idx in (("work_row", False, row_ptr, col_idx), ("work_col", True, col_ptr, row_idx)):
            desc = getattr(m, name).cpu().numpy().reshape(-1, 4)
            order = expected_work(masks, n_heads, by_cols)
            assert np.array_equal(desc[:, 0], order), name
            s_, h_, i_ = order // (heads * n), (order // n) % heads, order % n
            k_ = np.asarray(classes)[h_]
            assert np.array_equal(desc[:, 1], ptr[s_, k_, i_]), name
            assert np.array_equal(desc[:, 2], ptr[s_, k_, i_ + 1]), name
            assert np.array_equal(desc[:, 3], idx[s_, k_, desc[:, 1]]), name


def check_mask(m: gsa.GsaMask, c: np.ndarray, block: int, window: int, n_heads):
    """Bit-exact comparison of every mask buffer with the oracle."""
    flags, n_lit, masks, _, _ = expected_mask(c, block, window)
    b, n = c.shape
    assert np.array_equal(m.flags.cpu().numpy().reshape(b, n), flags.astype(np.uint8))
    assert np.array_equal(m.n_literal.cpu().numpy()[:b], n_lit)
    check_lists(m, masks, n_heads)
    return masks


def run_path(x_bytes, block, window, n_heads, tensors, backward, device="cuda"):
    """bytes -> c (host) -> mask (GPU) -> O, LSE (and dQ, dK, dV) through the C ABI."""
    c = gsa.gsa_prepare(x_bytes, block)
    m = gsa.gsa_build_mask(torch.from_numpy(c).to(device), window, n_heads)
    q, k, v = (tensors[nm].to(device) for nm in ("q", "k", "v"))
    o, lse = gsa.gsa_attn_fwd(q, k, v, m, block)
    out = {"c": c, "mask": m, "o": o, "lse": lse}
    if backward:
        do = tensors["do"].to(device)
        out["dq"], out["dk"], out["dv"] = gsa.gsa_attn_bwd(q, k, v, o, lse, do, m, block)
    torch.cuda.synchronize()
    return out


def oracle_map(fn, jobs, workers: int = 8):
    """[fn(*job) for job in jobs], run on a thread pool with one BLAS thread per worker:
    the oracle's NumPy work releases the GIL, so independent blocks run side by side."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    if len(jobs) <= 1:
        return [fn(*job) for job in jobs]
    with threadpool_limits(1), ThreadPoolExecutor(min(workers, len(jobs))) as ex:
        return list(ex.map(lambda job: fn(*job), jobs))


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def assert_close(name, got, ref, tol):
    err = max_err(got, ref)
    log(f"    {name}: max|err| = {err:.3e}  max|ref| = {float(np.max(np.abs(ref))) if np.size(ref) else 0:.3e}"
        f"  tol = {tol:.1e}  margin = {tol - err:.3e}")
    assert np.all(np.isfinite(got)), name
    assert err <= tol, f"{name}: {err} > {tol}"
