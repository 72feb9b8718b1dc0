"""The seeded generators: deterministic, the right shapes, and literal counts in the
configured ranges (L per 8 KiB sample in [11, 40]; long-context samples near 23 and 200)."""
import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_bytes_deterministic_and_shaped(cid):
    wl = synth.WORKLOADS[cid]
    a = synth.gen_bytes(wl)
    b = synth.gen_bytes(wl)
    assert a.dtype == np.uint8 and a.shape == (wl.batch, wl.seq_len)
    assert np.array_equal(a, b)
    assert wl.seq_len % wl.block == 0


def test_markov_bytes_are_printable():
    x = synth.gen_bytes(synth.WORKLOADS[2])
    assert set(np.unique(x).tolist()) <= set(synth.ALPHABET.tolist())


def test_config4_shares_config3_inputs():
    assert np.array_equal(synth.gen_bytes(synth.WORKLOADS[3]), synth.gen_bytes(synth.WORKLOADS[4]))
    t3 = synth.gen_tensors(synth.WORKLOADS[3], ("q",), batch=1, heads=1, seq_len=64)
    t4 = synth.gen_tensors(synth.WORKLOADS[4], ("q",), batch=1, heads=1, seq_len=64)
    assert torch.equal(t3["q"], t4["q"])


def test_tensors_dtype_and_scale():
    t = synth.gen_tensors(synth.WORKLOADS[2], ("q", "do"), batch=2, heads=3, seq_len=512)
    assert t["q"].dtype == torch.bfloat16 and t["q"].shape == (2, 3, 512, 64)
    assert abs(t["q"].float().std().item() - 1 / 8) < 0.01
    assert abs(t["do"].float().std().item() - 1.0) < 0.05
    t1 = synth.gen_tensors(synth.WORKLOADS[1])
    assert t1["q"].dtype == torch.float32 and t1["q"].shape == (1, 4, 256, 32)


def test_realized_literal_counts():
    for cid in (3, 4):
        wl = synth.WORKLOADS[cid]
        _, n_lit = oracle.literal_flags(oracle.compressed_lengths(synth.gen_bytes(wl), wl.block), wl.block)
        assert n_lit.min() >= 11 and n_lit.max() <= 40, n_lit
    wl = synth.WORKLOADS[5]
    _, n_lit = oracle.literal_flags(oracle.compressed_lengths(synth.gen_bytes(wl), wl.block), wl.block)
    assert abs(n_lit[0] - 23) <= 10 and abs(n_lit[1] - 200) <= 30, n_lit
