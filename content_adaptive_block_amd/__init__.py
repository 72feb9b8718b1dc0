"""gzip-guided block-sparse causal attention for AMD MI355X (gfx950).

Thin ctypes binding over libgsa.so (see include/gsa.h).  The names mirror the C ABI:
``gsa_prepare`` (host gzip stage), ``gsa_build_mask`` (HIP mask kernel),
``gsa_attn_fwd`` / ``gsa_attn_bwd`` (HIP attention kernels).  torch supplies device
memory and the current stream; every step of the computation runs in the library.
If the library has not been built this module raises on first use: there is no
fallback implementation.

Method: "Gzip-guided Sparse Attention：用压缩率选择长程内容" (daiwk.github.io reproduction
of arXiv 2607.21752), sections 背景与主要改动 and 核心公式.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # loaded first: libgsa binds to the HIP runtime torch has already mapped

__all__ = [
    "GsaError", "GsaMask", "PrepPool", "lib_path", "load_library", "gsa_prepare", "gsa_mask_bytes",
    "gsa_mask_sizes",
    "gsa_build_mask", "gsa_build_mask_noalloc", "gsa_build_mask_from_blocks", "gsa_bigbird_blocks",
    "gsa_attn_fwd", "gsa_attn_bwd", "attention", "zlib_version", "default_head_counts",
    "GSA_OK", "GSA_ERR_ARG", "GSA_ERR_SHAPE", "GSA_ERR_ZLIB", "GSA_ERR_HIP", "GSA_ERR_UNSUPPORTED",
]

GSA_OK, GSA_ERR_ARG, GSA_ERR_SHAPE, GSA_ERR_ZLIB, GSA_ERR_HIP, GSA_ERR_UNSUPPORTED = range(6)
GSA_F32, GSA_BF16 = 0, 1
GSA_MAX_BLOCKS = 1024
MASK_FIELDS = ("flags", "n_literal", "row_ptr", "col_idx", "col_ptr", "row_idx", "n_edges",
               "work_row", "work_col", "sched")
_MASK_DTYPES = (torch.uint8, torch.int32, torch.int32, torch.int32, torch.int32, torch.int32,
                torch.int64, torch.int32, torch.int32, torch.int32)

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_PKG_DIR, "libgsa.so")


class GsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


class _Mask(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("n_blocks", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_heads", ctypes.c_int32 * 3)] + [(f, ctypes.c_void_p) for f in MASK_FIELDS]


class _FwdArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int64),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("scale", ctypes.c_float)]


class _BwdArgs(ctypes.Structure):
    _fields_ = [("f", _FwdArgs), ("dout", ctypes.c_void_p), ("dq", ctypes.c_void_p),
                ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p), ("workspace", ctypes.c_void_p)]


_LIB = None


def load_library():
    """Loads libgsa.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    i32, i64, vp, cp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_char_p
    lib.gsa_status_str.argtypes, lib.gsa_status_str.restype = [i32], cp
    lib.gsa_last_error.argtypes, lib.gsa_last_error.restype = [], cp
    lib.gsa_zlib_version.argtypes, lib.gsa_zlib_version.restype = [], cp
    lib.gsa_abi_version.argtypes, lib.gsa_abi_version.restype = [], i32
    lib.gsa_prepare.argtypes = [vp, i64, i64, i32, i32, vp]
    lib.gsa_prepare.restype = i32
    lib.gsa_prep_pool_create.argtypes = [i32, ctypes.POINTER(vp)]
    lib.gsa_prep_pool_submit.argtypes = [vp, vp, i64, i64, i32, vp]
    lib.gsa_prep_pool_wait.argtypes = [vp]
    lib.gsa_prep_pool_destroy.argtypes = [vp]
    for nm in ("gsa_prep_pool_create", "gsa_prep_pool_submit", "gsa_prep_pool_wait", "gsa_prep_pool_destroy"):
        getattr(lib, nm).restype = i32
    for nm in ("gsa_mask_bytes", "gsa_mask_sizes"):
        getattr(lib, nm).argtypes = [i64, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_size_t)]
        getattr(lib, nm).restype = i32
    lib.gsa_default_head_counts.argtypes = [i32, ctypes.POINTER(i32)]
    lib.gsa_default_head_counts.restype = i32
    lib.gsa_build_mask.argtypes = [vp, ctypes.POINTER(_Mask), vp]
    lib.gsa_build_mask.restype = i32
    lib.gsa_build_mask_noalloc.argtypes = [vp, ctypes.POINTER(_Mask), vp]
    lib.gsa_build_mask_noalloc.restype = i32
    lib.gsa_build_mask_from_blocks.argtypes = [vp, ctypes.POINTER(_Mask), vp]
    lib.gsa_build_mask_from_blocks.restype = i32
    lib.gsa_bigbird_blocks.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp]
    lib.gsa_bigbird_blocks.restype = i32
    lib.gsa_attn_fwd.argtypes = [ctypes.POINTER(_FwdArgs), ctypes.POINTER(_Mask), vp]
    lib.gsa_attn_fwd.restype = i32
    for nm in ("gsa_attn_bwd", "gsa_attn_bwd_prep", "gsa_attn_bwd_dkdv", "gsa_attn_bwd_dq"):
        fn = getattr(lib, nm)
        fn.argtypes = [ctypes.POINTER(_BwdArgs), ctypes.POINTER(_Mask), vp]
        fn.restype = i32
    _LIB = lib
    return lib


def _status_name(st: int) -> str:
    try:
        return load_library().gsa_status_str(st).decode()
    except Exception:  # pragma: no cover - only while reporting a load failure
        return str(st)


def _check(st: int, where: str):
    if st != GSA_OK:
        raise GsaError(st, where, load_library().gsa_last_error().decode())


def zlib_version() -> str:
    return load_library().gsa_zlib_version().decode()


def default_head_counts(heads: int):
    """The library's default split of ``heads`` into (local, literal, hybrid) counts
    (gsa_default_head_counts)."""
    out = (ctypes.c_int32 * 3)()
    _check(load_library().gsa_default_head_counts(heads, out), "gsa_default_head_counts")
    return tuple(int(x) for x in out)


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------------------- (1)
def gsa_prepare(data, block: int, n_threads: int = 0) -> np.ndarray:
    """Per-block gzip level-1 sizes c [B, N] int32 of host bytes ``data`` uint8 [B, T]."""
    if isinstance(data, torch.Tensor):
        if data.device.type != "cpu":
            raise ValueError("gsa_prepare takes host bytes")
        data = data.numpy()
    arr = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
    if arr.ndim != 2:
        raise ValueError("data must be [batch, seq_len]")
    batch, seq_len = arr.shape
    n = seq_len // block if block > 0 else 0
    out = np.zeros((batch, n), dtype=np.int32)
    st = load_library().gsa_prepare(arr.ctypes.data, batch, seq_len, block, n_threads, out.ctypes.data)
    _check(st, "gsa_prepare")
    return out


class PrepPool:
    """Persistent host pool for the gzip stage (gsa_prep_pool_*): ``submit`` starts a
    batch and returns at once, ``wait`` blocks until its sizes are in ``out``."""

    def __init__(self, n_threads: int = 0):
        handle = ctypes.c_void_p()
        _check(load_library().gsa_prep_pool_create(n_threads, ctypes.byref(handle)), "gsa_prep_pool_create")
        self._h = handle
        self._keep = None   # the running batch's buffers stay referenced until it is done

    def submit(self, data: np.ndarray, block: int, out) -> None:
        """Start sizes of host bytes ``data`` uint8 [B, T] into ``out`` int32 [B, T/block]
        (a numpy array or a CPU tensor, e.g. pinned for a later device copy)."""
        arr = np.ascontiguousarray(np.asarray(data, dtype=np.uint8))
        if arr.ndim != 2:
            raise ValueError("data must be [batch, seq_len]")
        batch, seq_len = arr.shape
        n = seq_len // block if block > 0 else 0
        if isinstance(out, torch.Tensor):
            if out.device.type != "cpu" or out.dtype != torch.int32 or not out.is_contiguous():
                raise ValueError("out must be a contiguous int32 host tensor")
            ptr, size = out.data_ptr(), out.numel()
        else:
            if out.dtype != np.int32 or not out.flags.c_contiguous:
                raise ValueError("out must be a contiguous int32 array")
            ptr, size = out.ctypes.data, out.size
        if size != batch * n:
            raise ValueError(f"out has {size} entries, expected {batch * n}")
        _check(load_library().gsa_prep_pool_submit(self._h, arr.ctypes.data, batch, seq_len, block, ptr),
               "gsa_prep_pool_submit")
        self._keep = (arr, out)

    def wait(self) -> None:
        try:
            _check(load_library().gsa_prep_pool_wait(self._h), "gsa_prep_pool_wait")
        finally:
            self._keep = None

    def close(self) -> None:
        if self._h is not None and self._h.value:
            load_library().gsa_prep_pool_destroy(self._h)
        self._h = None
        self._keep = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


# ---------------------------------------------------------------------------------- (2)
def gsa_mask_bytes(batch: int, n_blocks: int, n_heads) -> list:
    """Byte sizes of the mask buffers, in ``MASK_FIELDS`` order."""
    nh = (ctypes.c_int32 * 3)(*n_heads)
    sizes = (ctypes.c_size_t * len(MASK_FIELDS))()
    _check(load_library().gsa_mask_bytes(batch, n_blocks, nh, sizes), "gsa_mask_bytes")
    return list(sizes)


gsa_mask_sizes = gsa_mask_bytes


@dataclass
class GsaMask:
    """Device-resident mask of one batch (buffers as in include/gsa.h).  ``built`` is set
    once a mask call has been enqueued into the buffers; the attention calls refuse a mask
    whose buffers were never filled."""
    batch: int
    n_blocks: int
    window: int
    n_heads: tuple
    flags: torch.Tensor
    n_literal: torch.Tensor
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    col_ptr: torch.Tensor
    row_idx: torch.Tensor
    n_edges: torch.Tensor
    work_row: torch.Tensor
    work_col: torch.Tensor
    sched: torch.Tensor
    built: bool = False

    @property
    def cap(self) -> int:
        return self.n_blocks * (self.n_blocks + 1) // 2

    def struct(self) -> _Mask:
        """The C struct over these buffers (for mask and attention calls)."""
        m = _Mask()
        m.batch, m.n_blocks, m.window = self.batch, self.n_blocks, self.window
        m.n_heads[:] = list(self.n_heads)
        for f in MASK_FIELDS:
            setattr(m, f, getattr(self, f).data_ptr())
        return m

    @staticmethod
    def empty(batch: int, n_blocks: int, window: int, n_heads, device) -> "GsaMask":
        sizes = gsa_mask_sizes(batch, n_blocks, n_heads)
        bufs = {}
        for f, dt, nbytes in zip(MASK_FIELDS, _MASK_DTYPES, sizes):
            itemsize = torch.empty(0, dtype=dt).element_size()
            bufs[f] = torch.empty(max(nbytes // itemsize, 1), dtype=dt, device=device)
        return GsaMask(batch, n_blocks, window, tuple(int(h) for h in n_heads), **bufs)


def gsa_build_mask(c, window: int, n_heads, device=None, out: GsaMask | None = None) -> GsaMask:
    """Literal flags, CSR/CSC block lists and work order from sizes ``c`` [B, N].

    ``c`` may be a host array (uploaded on the current stream) or a device int32 tensor.
    """
    if not isinstance(c, torch.Tensor):
        c = torch.from_numpy(np.ascontiguousarray(np.asarray(c, dtype=np.int32)))
    if device is None:
        device = c.device if c.is_cuda else torch.device("cuda", torch.cuda.current_device())
    c = c.to(device=device, dtype=torch.int32, non_blocking=True).contiguous()
    if c.dim() != 2:
        raise ValueError("c must be [batch, n_blocks]")
    batch, n = c.shape
    m = out if out is not None else GsaMask.empty(batch, n, window, n_heads, device)
    if (m.batch, m.n_blocks) != (batch, n) or m.n_heads != tuple(int(h) for h in n_heads):
        raise ValueError("preallocated mask has another shape or head split")
    m.window = window
    ms = m.struct()
    _check(load_library().gsa_build_mask(c.data_ptr(), ctypes.byref(ms), _stream_ptr(device)),
           "gsa_build_mask")
    m.built = True
    return m


def gsa_build_mask_noalloc(c: torch.Tensor, window: int, n_heads, out: GsaMask) -> GsaMask:
    """gsa_build_mask for callers that cannot allocate device memory: ``c`` must already
    be a contiguous device int32 tensor [B, N] and ``out`` a mask of that shape; its
    ``sched`` buffer is not used (the library's own scratch array serves instead).
    Nothing is allocated here or in the library."""
    if not (isinstance(c, torch.Tensor) and c.is_cuda and c.dtype == torch.int32 and c.dim() == 2
            and c.is_contiguous()):
        raise ValueError("c must be a contiguous device int32 tensor [batch, n_blocks]")
    if not isinstance(out, GsaMask):
        raise ValueError("out must be a preallocated GsaMask")
    batch, n = c.shape
    if (out.batch, out.n_blocks) != (batch, n) or out.n_heads != tuple(int(h) for h in n_heads):
        raise ValueError("preallocated mask has another shape or head split")
    out.window = window
    ms = out.struct()
    _check(load_library().gsa_build_mask_noalloc(c.data_ptr(), ctypes.byref(ms), _stream_ptr(c.device)),
           "gsa_build_mask_noalloc")
    out.built = True
    return out


def gsa_build_mask_from_blocks(blocks: torch.Tensor, n_heads, out: GsaMask | None = None) -> GsaMask:
    """Block lists and work order of a given block mask ``blocks`` (device uint8
    [B, 3, N, N]; entries above the diagonal ignored, the diagonal always kept)."""
    if not (isinstance(blocks, torch.Tensor) and blocks.is_cuda and blocks.dtype == torch.uint8
            and blocks.dim() == 4 and blocks.shape[1] == 3 and blocks.shape[2] == blocks.shape[3]):
        raise ValueError("blocks must be a device uint8 tensor [B, 3, N, N]")
    blocks = blocks.contiguous()
    batch, n = blocks.shape[0], blocks.shape[2]
    m = out if out is not None else GsaMask.empty(batch, n, 0, n_heads, blocks.device)
    if (m.batch, m.n_blocks) != (batch, n) or m.n_heads != tuple(int(h) for h in n_heads):
        raise ValueError("preallocated mask has another shape or head split")
    m.window = 0
    ms = m.struct()
    _check(load_library().gsa_build_mask_from_blocks(blocks.data_ptr(), ctypes.byref(ms), _stream_ptr(blocks.device)),
           "gsa_build_mask_from_blocks")
    m.built = True
    return m


def gsa_bigbird_blocks(random: torch.Tensor, window: int, n_global: int, out: torch.Tensor | None = None):
    """BigBird-style causal block mask (class 0; classes 1, 2 diagonal only) as device
    uint8 [B, 3, N, N], from the random picks ``random`` device int32 [B, N, r] (each
    entry of row i in 0..i)."""
    if not (isinstance(random, torch.Tensor) and random.is_cuda and random.dtype == torch.int32
            and random.dim() == 3):
        raise ValueError("random must be a device int32 tensor [B, N, r]")
    random = random.contiguous()
    batch, n, r = random.shape
    if out is None:
        out = torch.empty((batch, 3, n, n), dtype=torch.uint8, device=random.device)
    _check(load_library().gsa_bigbird_blocks(batch, n, window, n_global, r, random.data_ptr(), out.data_ptr(),
                                             _stream_ptr(random.device)), "gsa_bigbird_blocks")
    return out


# ---------------------------------------------------------------------------------- (3), (4)
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GSA_BF16
    if t.dtype == torch.float32:
        return GSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _check_tensors(*ts):
    ref = ts[0]
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device:
            raise ValueError("tensors must live on the same GPU")
        if t.dtype != ref.dtype or t.shape != ref.shape:
            raise ValueError("q, k, v (and o, dout) must share dtype and shape [B, H, T, d]")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, T, d]")


def _check_out(t, ref, name):
    """An output the caller passes in must be a contiguous tensor like ``ref``."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.device == ref.device and t.dtype == ref.dtype
            and t.shape == ref.shape and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {ref.dtype} tensor {tuple(ref.shape)} on {ref.device}")


def _check_rows(t, ref, name):
    """A per-row fp32 vector [B, H, T] for the tensors shaped like ``ref``."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.device == ref.device and t.dtype == torch.float32
            and t.shape == ref.shape[:3] and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 tensor {tuple(ref.shape[:3])} on {ref.device}")


def _check_built(mask: GsaMask):
    if not (isinstance(mask, GsaMask) and mask.built):
        raise ValueError("the mask was never built: call gsa_build_mask or gsa_build_mask_from_blocks first")


def _fwd_struct(q, k, v, o, lse, block, scale) -> _FwdArgs:
    a = _FwdArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    a.dtype = _dtype_code(q)
    a.batch, a.heads, a.seq_len, a.head_dim = q.shape
    a.block, a.scale = block, float(scale)
    return a


def gsa_attn_fwd(q, k, v, mask: GsaMask, block: int, scale: float = 0.0, with_lse: bool = True,
                 out=None, lse=None):
    """O [B, H, T, d] (and LSE fp32 [B, H, T]) of the gzip-masked causal attention."""
    _check_built(mask)
    _check_tensors(q, k, v)
    o = torch.empty_like(q) if out is None else out
    _check_out(o, q, "out")
    if with_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if with_lse:
        _check_rows(lse, q, "lse")
    a = _fwd_struct(q, k, v, o, lse if with_lse else None, block, scale)
    ms = mask.struct()
    _check(load_library().gsa_attn_fwd(ctypes.byref(a), ctypes.byref(ms), _stream_ptr(q.device)),
           "gsa_attn_fwd")
    return (o, lse) if with_lse else o


def _bwd_struct(q, k, v, o, lse, dout, dq, dk, dv, workspace, block, scale) -> _BwdArgs:
    b = _BwdArgs()
    b.f = _fwd_struct(q, k, v, o, lse, block, scale)
    b.dout, b.dq, b.dk, b.dv, b.workspace = _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace)
    return b


BWD_STAGES = {"all": "gsa_attn_bwd", "prep": "gsa_attn_bwd_prep", "dkdv": "gsa_attn_bwd_dkdv",
              "dq": "gsa_attn_bwd_dq"}


def gsa_attn_bwd(q, k, v, o, lse, dout, mask: GsaMask, block: int, scale: float = 0.0,
                 workspace=None, out=None, stage: str = "all"):
    """dQ, dK, dV of sum(O * dout).  ``stage`` runs one backward stage only: "dq" (also
    writes D into ``workspace``), then "dkdv" (reads it); "prep" writes D alone, for
    running "dkdv" without "dq".  Stages share ``workspace`` and ``out``."""
    _check_built(mask)
    _check_tensors(q, k, v, o, dout)
    if lse is not None or stage != "prep":   # the D-only stage reads no LSE
        _check_rows(lse, q, "lse")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if out is None else out
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_out(t, q, name)
    if workspace is None:
        workspace = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _check_rows(workspace, q, "workspace")
    b = _bwd_struct(q, k, v, o, lse, dout, dq, dk, dv, workspace, block, scale)
    ms = mask.struct()
    fn = getattr(load_library(), BWD_STAGES[stage])
    _check(fn(ctypes.byref(b), ctypes.byref(ms), _stream_ptr(q.device)), BWD_STAGES[stage])
    return dq, dk, dv


class _GsaAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, mask, block, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = gsa_attn_fwd(q, k, v, mask, block, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.mask, ctx.block, ctx.scale = mask, block, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = gsa_attn_bwd(q, k, v, o, lse, do.contiguous(), ctx.mask, ctx.block, ctx.scale)
        return dq, dk, dv, None, None, None


def attention(q, k, v, mask: GsaMask, block: int, scale: float = 0.0):
    """Differentiable gzip-masked attention (forward and backward through libgsa)."""
    return _GsaAttention.apply(q, k, v, mask, block, scale)
