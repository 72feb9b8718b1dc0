"""Seeded synthetic workloads for gzip-guided sparse attention.

This module only draws random numbers: it holds none of the method's arithmetic
(no compression, no flags, no masks, no attention).  Both the HIP library's tests
and the CPU oracle consume what it returns, so it is the one thing they share.

The pages train on PG-19 at 8K bytes and on WikiText-2 raw bytes at 256 bytes
("Gzip-guided Sparse Attention：用压缩率选择长程内容", 论文离线与线上效果 and 本地复现).
Neither corpus is available, so text-like byte streams of the same shapes stand in:
printable ASCII from an order-2 Markov chain whose per-segment temperature switches
between near-deterministic (highly compressible) and flat (incompressible) regimes,
and, for the tiny and long-context cases, spliced runs of uniform random bytes.

Seeds: ``numpy.random.default_rng([seed_id, stream])`` with streams
0 = bytes, 1 = Q, 2 = K, 3 = V, 4 = dO, 5 = Markov transition table.
Floating-point tensors are float32 normal draws times a per-config scale; bf16
tensors are those draws rounded to nearest-even by torch.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

STREAM_BYTES, STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_TABLE, STREAM_PICKS = range(7)

# 96 symbols: the 95 printable ASCII characters 0x20..0x7E plus '\n'.
ALPHABET = np.array([0x0A] + list(range(0x20, 0x7F)), dtype=np.uint8)


@dataclass(frozen=True)
class Workload:
    """One benchmark shape.  ``seed_id`` selects the random streams (configs 3 and 4 share)."""
    cfg_id: int
    name: str
    batch: int
    seq_len: int
    block: int
    window: int
    heads: int
    n_heads: tuple
    head_dim: int
    dtype: str            # "f32" or "bf16"
    backward: bool
    qkv_std: float
    seed_id: int
    byte_gen: str
    byte_params: dict = field(default_factory=dict)

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block


# Markov segment mixes: probabilities of temperatures (0.2, 1.0, 3.0) per segment.
_MIX_4K = {"p_temp": (0.8, 0.1, 0.1), "seg_len": (64, 256)}
_MIX_8K = {"p_temp": (0.8, 0.1, 0.1), "seg_len": (64, 256)}

WORKLOADS = {
    1: Workload(1, "tiny-f32-256B", 1, 256, 16, 1, 4, (2, 1, 1), 32, "f32", False, 1.0, 1,
                "alternating", {"seg_len": (16, 64), "phrase_len": (4, 8)}),
    2: Workload(2, "b8-4KiB-bf16-fwd", 8, 4096, 64, 2, 12, (6, 3, 3), 64, "bf16", False,
                1.0 / 8.0, 2, "markov", _MIX_4K),
    3: Workload(3, "b8-8KiB-bf16-fwd", 8, 8192, 64, 2, 12, (6, 3, 3), 64, "bf16", False,
                1.0 / 8.0, 3, "markov", _MIX_8K),
    4: Workload(4, "b8-8KiB-bf16-fwdbwd", 8, 8192, 64, 2, 12, (6, 3, 3), 64, "bf16", True,
                1.0 / 8.0, 3, "markov", _MIX_8K),
    5: Workload(5, "b2-64KiB-bf16-fwdbwd", 2, 65536, 128, 4, 16, (8, 4, 4), 128, "bf16", True,
                1.0 / math.sqrt(128.0), 5, "long",
                {"seg_len": (64, 512), "p_random": (0.045, 0.40)}),
}


def rng_for(seed_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed_id, stream])


# ---------------------------------------------------------------- byte streams
def alternating_bytes(rng: np.random.Generator, seq_len: int, seg_len=(16, 64),
                      phrase_len=(4, 8)) -> np.ndarray:
    """Alternating segments, starting with uniform random bytes 0..255, then a run that
    tiles a fresh lowercase phrase; segment lengths uniform in ``seg_len``; the last
    segment is cut at ``seq_len``."""
    out = np.empty(seq_len, dtype=np.uint8)
    pos, random_seg = 0, True
    while pos < seq_len:
        n = int(rng.integers(seg_len[0], seg_len[1] + 1))
        n = min(n, seq_len - pos)
        if random_seg:
            out[pos:pos + n] = rng.integers(0, 256, n, dtype=np.uint8)
        else:
            plen = int(rng.integers(phrase_len[0], phrase_len[1] + 1))
            phrase = rng.integers(ord("a"), ord("z") + 1, plen, dtype=np.uint8)
            out[pos:pos + n] = np.resize(phrase, n)
        pos += n
        random_seg = not random_seg
    return out


class MarkovText:
    """Order-2 Markov chain over the 96-symbol alphabet.

    Logits are N(0,1) plus a bonus of 8 on one preferred successor per context, the
    preferred successor drawn from a 6-symbol sub-alphabet; the next symbol is drawn
    with probability proportional to exp((logit - max) / tau).  At tau = 0.2 the chain
    follows short cycles (compressible); at tau = 3 it is close to uniform.
    """

    TEMPS = (0.2, 1.0, 3.0)

    def __init__(self, rng: np.random.Generator, bonus: float = 8.0, sub_alphabet: int = 6):
        k = len(ALPHABET)
        logits = rng.standard_normal((k * k, k))
        sub = rng.choice(k, size=sub_alphabet, replace=False)
        pref = sub[rng.integers(0, sub_alphabet, k * k)]
        logits[np.arange(k * k), pref] += bonus
        self.cdf = np.empty((len(self.TEMPS), k * k, k))
        for ti, tau in enumerate(self.TEMPS):
            z = np.exp((logits - logits.max(axis=1, keepdims=True)) / tau)
            c = np.cumsum(z, axis=1)
            self.cdf[ti] = c / c[:, -1:]
        self.k = k

    def sample(self, rng: np.random.Generator, temps_per_pos: np.ndarray) -> np.ndarray:
        """Draw one symbol index per position; ``temps_per_pos`` holds temperature indices."""
        n = len(temps_per_pos)
        sym = np.empty(n, dtype=np.int64)
        a, b = rng.integers(0, self.k, 2)
        u = rng.random(n)
        for t in range(n):
            row = self.cdf[temps_per_pos[t], a * self.k + b]
            nxt = int(np.searchsorted(row, u[t], side="right"))
            nxt = min(nxt, self.k - 1)
            sym[t] = nxt
            a, b = b, nxt
        return sym


def _segment_labels(rng, seq_len, seg_len, probs) -> np.ndarray:
    """Per-position labels drawn per segment: segment lengths uniform in ``seg_len``,
    label of each segment drawn from ``probs``."""
    labels = np.empty(seq_len, dtype=np.int64)
    pos = 0
    while pos < seq_len:
        n = min(int(rng.integers(seg_len[0], seg_len[1] + 1)), seq_len - pos)
        labels[pos:pos + n] = rng.choice(len(probs), p=probs)
        pos += n
    return labels


def markov_bytes(rng, table: MarkovText, seq_len, p_temp, seg_len) -> np.ndarray:
    temps = _segment_labels(rng, seq_len, seg_len, np.asarray(p_temp, dtype=float))
    return ALPHABET[table.sample(rng, temps)]


def long_bytes(rng, table: MarkovText, seq_len, p_random, seg_len) -> np.ndarray:
    """Low-temperature Markov text with segments replaced by uniform random bytes with
    probability ``p_random``."""
    kinds = _segment_labels(rng, seq_len, seg_len, np.array([1.0 - p_random, p_random]))
    text = ALPHABET[table.sample(rng, np.zeros(seq_len, dtype=np.int64))]
    noise = rng.integers(0, 256, seq_len, dtype=np.uint8)
    return np.where(kinds == 1, noise, text).astype(np.uint8)


def gen_bytes(wl: Workload, batch: int | None = None, seq_len: int | None = None) -> np.ndarray:
    """uint8 [batch, seq_len] byte streams of workload ``wl`` (defaults: its own shape)."""
    batch = wl.batch if batch is None else batch
    seq_len = wl.seq_len if seq_len is None else seq_len
    rng = rng_for(wl.seed_id, STREAM_BYTES)
    out = np.empty((batch, seq_len), dtype=np.uint8)
    p = wl.byte_params
    if wl.byte_gen == "alternating":
        for s in range(batch):
            out[s] = alternating_bytes(rng, seq_len, p["seg_len"], p["phrase_len"])
        return out
    table = MarkovText(rng_for(wl.seed_id, STREAM_TABLE))
    for s in range(batch):
        if wl.byte_gen == "markov":
            out[s] = markov_bytes(rng, table, seq_len, p["p_temp"], p["seg_len"])
        elif wl.byte_gen == "long":
            pr = p["p_random"][s % len(p["p_random"])]
            out[s] = long_bytes(rng, table, seq_len, pr, p["seg_len"])
        else:
            raise ValueError(wl.byte_gen)
    return out


# ---------------------------------------------------------------- tensors
def gen_normal(seed_id: int, stream: int, shape, std: float) -> np.ndarray:
    """float32 N(0, std^2) draws of ``shape``."""
    x = rng_for(seed_id, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def gen_tensors(wl: Workload, names=("q", "k", "v"), batch=None, heads=None, seq_len=None,
                head_dim=None):
    """torch CPU tensors [B, H, T, d] in the workload's dtype (fp32, or bf16 rounded RNE).

    dO is N(0, 1) for every workload; Q, K, V use ``wl.qkv_std``.
    """
    import torch

    shape = (wl.batch if batch is None else batch, wl.heads if heads is None else heads,
             wl.seq_len if seq_len is None else seq_len,
             wl.head_dim if head_dim is None else head_dim)
    streams = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V, "do": STREAM_DO}
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    out = {}
    for nm in names:
        std = 1.0 if nm == "do" else wl.qkv_std
        x = torch.from_numpy(gen_normal(wl.seed_id, streams[nm], shape, std))
        out[nm] = x if dt == torch.float32 else x.to(dt)
    return out


def dense_causal(wl: Workload) -> Workload:
    """The same shape as ``wl`` with every head local and a window covering the whole
    sequence: the mask is then the full causal triangle (dense causal attention)."""
    return replace(wl, name=wl.name + "-dense", window=wl.n_blocks - 1, n_heads=(wl.heads, 0, 0))


def bigbird_picks(wl: Workload, n_random: int, batch: int | None = None, n_blocks: int | None = None) -> np.ndarray:
    """int32 [B, N, r]: the random key blocks of a BigBird-style mask, row i's picks
    uniform on 0..i (seeded stream 6 of the workload)."""
    batch = wl.batch if batch is None else batch
    n = wl.n_blocks if n_blocks is None else n_blocks
    rng = rng_for(wl.seed_id, STREAM_PICKS)
    hi = np.arange(1, n + 1)[None, :, None]
    return (rng.random((batch, n, n_random)) * hi).astype(np.int32)
