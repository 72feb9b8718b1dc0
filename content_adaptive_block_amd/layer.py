"""ByteLM attention layer around the gzip-masked attention kernels.

A byte-level language model keeps the standard Transformer and changes only which keys
each query may see ("Gzip-guided Sparse Attention", daiwk.github.io reproduction note,
背景与主要改动; the byte-level model of 论文离线与线上效果).  This module supplies that
attention block: a fused Q/K/V projection (D -> 3 H d), the block-sparse causal
attention through libgsa (forward and backward in the HIP kernels), and the output
projection (H d -> D).  The mask depends only on the batch's bytes, so it is built once
per batch (host gzip sizes, then the mask kernels) and shared by every layer.

The projections are plain PyTorch linears (hipBLASLt GEMMs); the attention step has no
PyTorch fallback.
"""
from __future__ import annotations

import numpy as np
import torch

from . import GsaMask, attention, default_head_counts, gsa_build_mask, gsa_prepare

__all__ = ["batch_mask", "GsaAttentionLayer", "ByteLM"]


def batch_mask(data, block: int, window: int, n_heads, device) -> GsaMask:
    """The gzip-guided mask of one batch of host bytes uint8 [B, T]."""
    c = gsa_prepare(np.asarray(data, dtype=np.uint8), block)
    return gsa_build_mask(torch.from_numpy(c).to(device), window, n_heads)


class GsaAttentionLayer(torch.nn.Module):
    """x [B, T, D] -> gzip-masked multi-head causal attention -> [B, T, D].

    ``heads`` heads of ``head_dim`` features, classes local | literal | hybrid in the
    counts ``n_heads`` (default: half, a quarter, the rest)."""

    def __init__(self, d_model: int, heads: int, head_dim: int, block: int, n_heads=None, bias: bool = False,
                 device=None, dtype=torch.bfloat16):
        super().__init__()
        self.heads, self.head_dim, self.block = heads, head_dim, block
        self.n_heads = tuple(n_heads) if n_heads is not None else default_head_counts(heads)
        if sum(self.n_heads) != heads:
            raise ValueError("n_heads must sum to heads")
        kw = {"device": device, "dtype": dtype}
        self.qkv = torch.nn.Linear(d_model, 3 * heads * head_dim, bias=bias, **kw)
        self.proj = torch.nn.Linear(heads * head_dim, d_model, bias=bias, **kw)

    def forward(self, x: torch.Tensor, mask: GsaMask) -> torch.Tensor:
        b, t, _ = x.shape
        h, d = self.heads, self.head_dim
        qkv = self.qkv(x).view(b, t, 3, h, d).permute(2, 0, 3, 1, 4)   # [3, B, H, T, d]
        q, k, v = (z.contiguous() for z in qkv)
        o = attention(q, k, v, mask, self.block)                         # [B, H, T, d]
        return self.proj(o.permute(0, 2, 1, 3).reshape(b, t, h * d))


class ByteLM(torch.nn.Module):
    """A small byte-level language model: byte embedding, pre-norm blocks of gzip-masked
    attention and a GELU MLP, and a 256-way output head."""

    def __init__(self, d_model: int, heads: int, head_dim: int, layers: int, block: int, window: int,
                 n_heads=None, device=None, dtype=torch.bfloat16):
        super().__init__()
        kw = {"device": device, "dtype": dtype}
        self.block, self.window = block, window
        self.embed = torch.nn.Embedding(256, d_model, **kw)
        self.blocks = torch.nn.ModuleList()
        for _ in range(layers):
            self.blocks.append(torch.nn.ModuleDict({
                "ln1": torch.nn.LayerNorm(d_model, **kw),
                "attn": GsaAttentionLayer(d_model, heads, head_dim, block, n_heads, device=device, dtype=dtype),
                "ln2": torch.nn.LayerNorm(d_model, **kw),
                "mlp": torch.nn.Sequential(torch.nn.Linear(d_model, 4 * d_model, **kw), torch.nn.GELU(),
                                           torch.nn.Linear(4 * d_model, d_model, **kw)),
            }))
        self.ln = torch.nn.LayerNorm(d_model, **kw)
        self.head = torch.nn.Linear(d_model, 256, **kw)
        self.n_heads = self.blocks[0]["attn"].n_heads if layers else (heads, 0, 0)

    def forward(self, tokens: torch.Tensor, mask: GsaMask) -> torch.Tensor:
        """Logits [B, T, 256] for byte tokens [B, T] (int64, on the model's device)."""
        x = self.embed(tokens)
        for blk in self.blocks:
            x = x + blk["attn"](blk["ln1"](x), mask)
            x = x + blk["mlp"](blk["ln2"](x))
        return self.head(self.ln(x))

    def loss(self, data: np.ndarray) -> torch.Tensor:
        """Next-byte cross entropy of host bytes uint8 [B, T] (the mask comes from the same
        bytes; the last position has no target)."""
        device = self.head.weight.device
        mask = batch_mask(data, self.block, self.window, self.n_heads, device)
        tokens = torch.from_numpy(np.asarray(data, dtype=np.int64)).to(device)
        logits = self(tokens, mask)
        return torch.nn.functional.cross_entropy(logits[:, :-1].float().reshape(-1, 256),
                                                 tokens[:, 1:].reshape(-1))
