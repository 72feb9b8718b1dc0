"""C ABI checks that need no GPU: the library loads and exports every declared symbol,
the host gzip stage equals the oracle byte for byte, and argument validation rejects
bad calls before any HIP call is made."""
import ctypes
import os
import re

import numpy as np
import pytest

import content_adaptive_block_amd as gsa
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return gsa.load_library()


def test_exports_every_declared_symbol(lib):
    text = open(os.path.join(ROOT, "include", "gsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(gsa_[a-z_]+)\s*\(", text))
    assert {"gsa_prepare", "gsa_build_mask", "gsa_attn_fwd", "gsa_attn_bwd", "gsa_mask_bytes", "gsa_mask_sizes",
            "gsa_default_head_counts"} <= names
    for nm in sorted(names):
        assert hasattr(lib, nm), nm
    assert lib.gsa_abi_version() == 1


def test_zlib_version_matches_oracle():
    assert gsa.zlib_version() == oracle.zlib_runtime_version()


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
@pytest.mark.parametrize("threads", [1, 0, 3])
def test_prepare_matches_oracle_on_every_config(cid, threads):
    wl = synth.WORKLOADS[cid]
    x = synth.gen_bytes(wl)
    c = gsa.gsa_prepare(x, wl.block, n_threads=threads)
    ref = oracle.compressed_lengths(x, wl.block)
    assert c.dtype == np.int32 and c.shape == ref.shape
    assert np.array_equal(c, ref)


def test_prepare_odd_blocks_and_edge_bytes():
    rng = np.random.default_rng(0)
    for b in (1, 2, 7, 16, 100, 4096):
        x = rng.integers(0, 256, (3, b * 5), dtype=np.uint8)
        x[1] = 0
        x[2, : b * 2] = 255
        assert np.array_equal(gsa.gsa_prepare(x, b), oracle.compressed_lengths(x, b))


def test_prepare_errors(lib):
    x = np.zeros((2, 100), np.uint8)
    with pytest.raises(gsa.GsaError) as e:
        gsa.gsa_prepare(x, 64)
    assert e.value.status == gsa.GSA_ERR_SHAPE
    with pytest.raises(gsa.GsaError) as e:
        gsa.gsa_prepare(x, 0)
    assert e.value.status == gsa.GSA_ERR_ARG
    out = np.zeros(4, np.int32)
    assert lib.gsa_prepare(None, 1, 64, 16, 1, out.ctypes.data) == gsa.GSA_ERR_ARG
    assert b"NULL" in lib.gsa_last_error()
    assert lib.gsa_prepare(x.ctypes.data, -1, 64, 16, 1, out.ctypes.data) == gsa.GSA_ERR_ARG
    # empty work is a no-op
    assert lib.gsa_prepare(None, 0, 64, 16, 1, None) == gsa.GSA_OK
    assert gsa.gsa_prepare(np.zeros((0, 64), np.uint8), 16).shape == (0, 4)


def test_mask_bytes(lib):
    sizes = gsa.gsa_mask_bytes(2, 5, (2, 1, 1))
    cap = 15
    assert sizes == [10, 8, 2 * 3 * 6 * 4, 2 * 3 * cap * 4, 2 * 3 * 6 * 4, 2 * 3 * cap * 4, 2 * 3 * 8,
                     2 * 4 * 5 * 16, 2 * 4 * 5 * 16, 2 * 3 * 2 * (5 + 32) * 4]
    assert gsa.gsa_mask_sizes(3, 128, (6, 3, 3)) == gsa.gsa_mask_bytes(3, 128, (6, 3, 3))
    with pytest.raises(gsa.GsaError):
        gsa.gsa_mask_bytes(-1, 5, (1, 1, 1))
    with pytest.raises(gsa.GsaError):
        gsa.gsa_mask_bytes(1, 5, (1, -1, 1))
    # straight through the C ABI: ten sizes, NULL arguments rejected
    nh = (ctypes.c_int32 * 3)(6, 3, 3)
    out = (ctypes.c_size_t * 10)()
    assert lib.gsa_mask_bytes(8, 128, nh, out) == gsa.GSA_OK
    assert list(out)[7] == 8 * 12 * 128 * 16
    assert lib.gsa_mask_bytes(8, 128, None, out) == gsa.GSA_ERR_ARG
    assert lib.gsa_mask_bytes(8, 128, nh, None) == gsa.GSA_ERR_ARG


def test_default_head_counts(lib):
    # [note] 背景与主要改动: half local, a quarter literal, the rest hybrid; the library's
    # split agrees with the oracle's on every head count
    for h in range(0, 40):
        assert gsa.default_head_counts(h) == oracle.default_head_counts(h)
    assert gsa.default_head_counts(12) == (6, 3, 3)
    with pytest.raises(gsa.GsaError):
        gsa.default_head_counts(-1)
    assert lib.gsa_default_head_counts(4, None) == gsa.GSA_ERR_ARG


FAKE = 0x10000   # a non-NULL, aligned address: validation must fail before it is used


def _mask(batch=2, n=4, window=1, heads=(2, 1, 1), null=(), misalign=()):
    m = gsa._Mask()
    m.batch, m.n_blocks, m.window = batch, n, window
    m.n_heads[:] = list(heads)
    for f in gsa.MASK_FIELDS:
        setattr(m, f, None if f in null else FAKE + (4 if f in misalign else 0))
    return m


def _fwd(dtype=gsa.GSA_BF16, batch=2, heads=4, seq_len=256, head_dim=64, block=64, scale=0.0, null=(),
         misalign=()):
    a = gsa._FwdArgs()
    for f in ("q", "k", "v", "o", "lse"):
        setattr(a, f, None if f in null else FAKE + (2 if f in misalign else 0))
    a.dtype, a.batch, a.heads, a.seq_len, a.head_dim, a.block, a.scale = (dtype, batch, heads, seq_len,
                                                                         head_dim, block, scale)
    return a


def _call_fwd(lib, a, m):
    return lib.gsa_attn_fwd(ctypes.byref(a), ctypes.byref(m), None)


def test_build_mask_validation(lib):
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(window=-1)), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(n=0)), None) == gsa.GSA_ERR_UNSUPPORTED
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(n=1025)), None) == gsa.GSA_ERR_UNSUPPORTED
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(heads=(1, -1, 1))), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(null=("col_idx",))), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(null=("flags",))), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(null=("sched",))), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(misalign=("sched",))), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(None, ctypes.byref(_mask()), None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(FAKE, None, None) == gsa.GSA_ERR_ARG
    assert lib.gsa_build_mask(None, ctypes.byref(_mask(batch=0)), None) == gsa.GSA_OK
    assert lib.gsa_build_mask(FAKE, ctypes.byref(_mask(window=-1)), None) == gsa.GSA_ERR_ARG
    assert b"window" in lib.gsa_last_error()


def test_attn_fwd_validation(lib):
    m = _mask(batch=2, n=4)
    assert _call_fwd(lib, _fwd(seq_len=250), m) == gsa.GSA_ERR_SHAPE           # T % b != 0
    assert _call_fwd(lib, _fwd(heads=5), m) == gsa.GSA_ERR_ARG                 # heads != 2+1+1
    assert _call_fwd(lib, _fwd(seq_len=320), m) == gsa.GSA_ERR_SHAPE           # N = 5 != 4
    assert _call_fwd(lib, _fwd(batch=3), m) == gsa.GSA_ERR_SHAPE               # batch mismatch
    assert _call_fwd(lib, _fwd(head_dim=96), m) == gsa.GSA_ERR_UNSUPPORTED
    assert _call_fwd(lib, _fwd(dtype=gsa.GSA_F32), m) == gsa.GSA_ERR_UNSUPPORTED
    assert _call_fwd(lib, _fwd(dtype=7), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(null=("v",)), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(misalign=("q",)), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(misalign=("lse",)), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(scale=-1.0), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(block=0), m) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(), _mask(null=("work_row",))) == gsa.GSA_ERR_ARG
    assert _call_fwd(lib, _fwd(), _mask(misalign=("work_row",))) == gsa.GSA_ERR_ARG
    assert lib.gsa_attn_fwd(None, ctypes.byref(m), None) == gsa.GSA_ERR_ARG
    # empty work is a no-op
    assert _call_fwd(lib, _fwd(batch=0, null=("q", "k", "v", "o", "lse")), _mask(batch=0)) == gsa.GSA_OK
    assert _call_fwd(lib, _fwd(seq_len=0, null=("q", "k", "v", "o", "lse")), m) == gsa.GSA_OK
    assert _call_fwd(lib, _fwd(heads=5), m) == gsa.GSA_ERR_ARG
    assert "heads" in lib.gsa_last_error().decode()


def test_attn_bwd_validation(lib):
    m = _mask(batch=2, n=4)
    b = gsa._BwdArgs()
    b.f = _fwd()
    b.dout = b.dq = b.dk = b.dv = b.workspace = FAKE
    b.dk = None
    assert lib.gsa_attn_bwd(ctypes.byref(b), ctypes.byref(m), None) == gsa.GSA_ERR_ARG
    b.dk = FAKE
    b.f = _fwd(null=("lse",))
    assert lib.gsa_attn_bwd(ctypes.byref(b), ctypes.byref(m), None) == gsa.GSA_ERR_ARG
    b.f = _fwd()
    b.workspace = FAKE + 4
    assert lib.gsa_attn_bwd(ctypes.byref(b), ctypes.byref(m), None) == gsa.GSA_ERR_ARG
    b.workspace = FAKE
    b.f = _fwd(seq_len=100)
    assert lib.gsa_attn_bwd(ctypes.byref(b), ctypes.byref(m), None) == gsa.GSA_ERR_SHAPE
    assert lib.gsa_attn_bwd(None, ctypes.byref(m), None) == gsa.GSA_ERR_ARG


def test_status_strings(lib):
    assert lib.gsa_status_str(gsa.GSA_ERR_SHAPE) == b"GSA_ERR_SHAPE"
    assert lib.gsa_status_str(99) == b"GSA_ERR_UNKNOWN"


# ------------------------------------------------------------------ host-stage pool
def test_prep_pool_matches_prepare_and_oracle():
    """Every config through one pool (block sizes change between batches), twice, with
    results equal to gsa_prepare and to the oracle's independent zlib path."""
    with gsa.PrepPool(3) as pool:
        for rep in range(2):
            for cid in (1, 2, 5, 3):
                wl = synth.WORKLOADS[cid]
                x = synth.gen_bytes(wl, batch=min(wl.batch, 2))
                out = np.full((x.shape[0], x.shape[1] // wl.block), -1, dtype=np.int32)
                pool.submit(x, wl.block, out)
                pool.wait()
                assert np.array_equal(out, gsa.gsa_prepare(x, wl.block)), (rep, cid)
                if rep == 0:
                    assert np.array_equal(out, oracle.compressed_lengths(x, wl.block)), cid


def test_prep_pool_overlapping_submits():
    """A submit waits for the previous batch; each output buffer gets its own batch."""
    wl = synth.WORKLOADS[2]
    xs = [synth.gen_bytes(wl, batch=3), np.roll(synth.gen_bytes(wl, batch=3), 17)]
    outs = [np.zeros((3, wl.n_blocks), np.int32) for _ in xs]
    with gsa.PrepPool(0) as pool:
        for x, o in zip(xs, outs):
            pool.submit(x, wl.block, o)   # the second submit waits for the first batch
        pool.wait()
    for x, o in zip(xs, outs):
        assert np.array_equal(o, gsa.gsa_prepare(x, wl.block))


def test_prep_pool_errors(lib):
    h = ctypes.c_void_p()
    assert lib.gsa_prep_pool_create(2, ctypes.byref(h)) == gsa.GSA_OK and h.value
    buf = np.zeros((2, 64), np.uint8)
    out = np.zeros((2, 4), np.int32)
    sub = lib.gsa_prep_pool_submit
    assert sub(h, buf.ctypes.data, -1, 64, 16, out.ctypes.data) == gsa.GSA_ERR_ARG
    assert sub(h, buf.ctypes.data, 2, 64, 0, out.ctypes.data) == gsa.GSA_ERR_ARG
    assert sub(h, buf.ctypes.data, 2, 60, 16, out.ctypes.data) == gsa.GSA_ERR_SHAPE
    assert sub(h, None, 2, 64, 16, out.ctypes.data) == gsa.GSA_ERR_ARG
    assert sub(h, buf.ctypes.data, 0, 64, 16, None) == gsa.GSA_OK          # empty batch
    assert sub(h, buf.ctypes.data, 2, 64, 16, out.ctypes.data) == gsa.GSA_OK
    assert lib.gsa_prep_pool_wait(h) == gsa.GSA_OK
    assert (out > 0).all()
    assert lib.gsa_prep_pool_wait(h) == gsa.GSA_OK                          # nothing pending
    assert lib.gsa_prep_pool_submit(None, buf.ctypes.data, 2, 64, 16, out.ctypes.data) == gsa.GSA_ERR_ARG
    assert lib.gsa_prep_pool_wait(None) == gsa.GSA_ERR_ARG
    assert lib.gsa_prep_pool_destroy(h) == gsa.GSA_OK
    assert lib.gsa_prep_pool_destroy(None) == gsa.GSA_OK
    assert lib.gsa_prep_pool_create(1, None) == gsa.GSA_ERR_ARG
    with gsa.PrepPool(1) as pool:
        with pytest.raises(ValueError):
            pool.submit(buf, 16, np.zeros((2, 3), np.int32))
