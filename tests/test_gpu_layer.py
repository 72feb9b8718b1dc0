"""GPU checks of the ByteLM attention layer (projections around the HIP attention).

Parity: the layer in bf16 against the same layer in fp64 on the CPU with the oracle's
token mask (dense masked softmax), for the output and the gradients of the input and
of both projection weights.  Tolerance 3e-2 x max(1, max|ref|) per tensor: the bf16
path rounds x, the weights, Q/K/V and the attention output (each about 2^-9 relative),
on top of the attention kernels' own 2e-2 budget.

Training smoke test: a two-layer ByteLM on seeded synthetic text bytes; 40 Adam steps
must lower the next-byte loss by at least 15%."""
import numpy as np
import pytest
import torch

import content_adaptive_block_amd as gsa
import oracle
import synth
from content_adaptive_block_amd.layer import ByteLM, GsaAttentionLayer, batch_mask
from gpu_cases import log

pytestmark = pytest.mark.gpu


def _reference_layer(x, w_qkv, w_proj, masks, n_heads, block, heads, head_dim):
    """fp64 CPU: the same projections, dense masked softmax attention with the oracle's
    token mask per head class."""
    b, t, _ = x.shape
    qkv = (x @ w_qkv.T).view(b, t, 3, heads, head_dim).permute(2, 0, 3, 1, 4)
    q, k, v = qkv[0], qkv[1], qkv[2]
    classes = oracle.head_classes(n_heads)
    outs = []
    for s in range(b):
        per_head = []
        for h in range(heads):
            allowed = torch.from_numpy(oracle.token_mask(masks[s, classes[h]], block))
            sc = (q[s, h] @ k[s, h].T) / np.sqrt(head_dim)
            sc = sc.masked_fill(~allowed, float("-inf"))
            per_head.append(torch.softmax(sc, dim=-1) @ v[s, h])
        outs.append(torch.stack(per_head))
    o = torch.stack(outs)                                   # [B, H, T, d]
    return o.permute(0, 2, 1, 3).reshape(b, t, heads * head_dim) @ w_proj.T


@pytest.mark.parametrize("heads,n_heads,window", [(4, (2, 1, 1), 2), (3, (0, 1, 2), 1)])
def test_layer_matches_fp64_reference(heads, n_heads, window):
    torch.manual_seed(0)
    wl = synth.WORKLOADS[3]
    b, t, block, d, dm = 2, 512, 64, 64, 192
    x_bytes = synth.gen_bytes(wl, batch=b, seq_len=t)
    layer = GsaAttentionLayer(dm, heads, d, block, n_heads, device="cuda")
    x = (torch.randn(b, t, dm) * 0.5).to(torch.bfloat16)
    xg = x.cuda().requires_grad_(True)
    mask = batch_mask(x_bytes, block, window, n_heads, "cuda")
    y = layer(xg, mask)
    gy = torch.randn_like(y)
    y.backward(gy)
    torch.cuda.synchronize()

    c = oracle.compressed_lengths(x_bytes, block)
    flags, _ = oracle.literal_flags(c, block)
    masks = oracle.block_masks(flags, window)
    x64 = x.double().requires_grad_(True)
    wq = layer.qkv.weight.detach().cpu().double().requires_grad_(True)
    wp = layer.proj.weight.detach().cpu().double().requires_grad_(True)
    ref = _reference_layer(x64, wq, wp, masks, n_heads, block, heads, d)
    ref.backward(gy.cpu().double())
    for name, got, want in (("y", y, ref), ("dx", xg.grad, x64.grad), ("dW_qkv", layer.qkv.weight.grad, wq.grad),
                            ("dW_proj", layer.proj.weight.grad, wp.grad)):
        got = got.detach().float().cpu().double()
        want = want.detach()
        err = float((got - want).abs().max())
        bound = 3e-2 * max(1.0, float(want.abs().max()))
        log(f"    {name}: max|err| = {err:.3e}  max|ref| = {float(want.abs().max()):.3e}  tol = {bound:.2e}")
        assert err <= bound, name


def test_bytelm_training_lowers_loss():
    torch.manual_seed(1)
    wl = synth.WORKLOADS[3]
    model = ByteLM(d_model=128, heads=4, head_dim=32 * 2, layers=2, block=64, window=2, device="cuda")
    opt = torch.optim.Adam(model.parameters(), lr=3e-3)
    data = synth.gen_bytes(wl, batch=4, seq_len=1024)
    losses = []
    for step in range(40):
        opt.zero_grad()
        loss = model.loss(data)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    log(f"    loss {losses[0]:.3f} -> {losses[-1]:.3f}")
    assert np.isfinite(losses).all()
    assert losses[-1] < 0.85 * losses[0]
