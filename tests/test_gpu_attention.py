"""Decode attention on the GPU against the fp64 oracle.

Bound, per output (h, d): |o - o_ref| <= 1e-5 * sum_j p[h][j] |v[j][d]|, with p
the exact softmax weights.  The scores are fp32 sums of D exact bf16 products
(relative error about D * 2^-24 of sum |q k|, times scale: near 1e-6 for unit
inputs), the exponentials are base 2 in fp32 and the weighted sums fp32 over a
split of keys and then over the splits; each contributes relative errors of
order 1e-6 of sum p |v|, a few times inside the bound."""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
BF16 = synth.BF16


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def abs_weighted(q, k, v, scale):
    """sum_j p[h][j] |v[j][d]| in fp64 (the scale of the bound)."""
    qf = oracle.act_to_f64(np.asarray(q).ravel(), BF16).reshape(np.asarray(q).shape)
    kf = oracle.act_to_f64(np.asarray(k).ravel(), BF16).reshape(np.asarray(k).shape)
    vf = oracle.act_to_f64(np.asarray(v).ravel(), BF16).reshape(np.asarray(v).shape)
    s = scale * (qf @ kf.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ np.abs(vf)


def check(o, q, k, v, scale):
    ref = oracle.decode_attention(q, k, v, scale)
    a = abs_weighted(q, k, v, scale)
    err = np.abs(o.cpu().numpy().astype(np.float64) - ref)
    ratio = np.where(a > 0, err / np.where(a > 0, a, 1.0), np.where(err > 0, np.inf, 0.0))
    assert ratio.max() <= 1e-5, ratio.max()


@pytest.mark.parametrize("H,D,L", [(8, 512, 1), (8, 512, 3), (8, 512, 512), (1, 256, 1000), (5, 512, 4099),
                                   (8, 256, 70000)])
def test_attention_vs_oracle(w4, H, D, L):
    print(f"attention H={H} D={D} L={L}", flush=True)
    rng = np.random.default_rng(H * 1000 + L)
    q = synth.act_bits(rng.standard_normal((H, D)), BF16)
    k = synth.act_bits(rng.standard_normal((L, D)), BF16)
    v = synth.act_bits(rng.standard_normal((L, D)), BF16)
    scale = 1.0 / np.sqrt(D)
    o = w4.w4_decode_attention(dev(q), dev(k), dev(v), scale)
    torch.cuda.synchronize()
    check(o, q, k, v, scale)


def test_attention_full_context_and_strided_ring(w4):
    """The page's full cache: 131072 positions of one head of width 512, 8 query
    heads; and a 512-slot ring stored inside wider rows (row stride 1024), whose
    result must not depend on the order of the slots."""
    rng = np.random.default_rng(5)
    H, D = 8, 512
    q = synth.act_bits(rng.standard_normal((H, D)), BF16)
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    L = 131072
    k = (torch.randn((L, D), generator=g, device="cuda")).to(torch.bfloat16)
    v = (torch.randn((L, D), generator=g, device="cuda")).to(torch.bfloat16)
    o = w4.w4_decode_attention(dev(q), k, v, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    kb = k.view(torch.int16).cpu().numpy().view(np.uint16)
    vb = v.view(torch.int16).cpu().numpy().view(np.uint16)
    check(o, q, kb, vb, 1.0 / np.sqrt(D))
    ring_k = torch.zeros((512, 1024), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros((512, 1024), dtype=torch.bfloat16, device="cuda")
    ring_k[:, :D] = k[:512]
    ring_v[:, :D] = v[:512]
    o1 = w4.w4_decode_attention(dev(q), ring_k[:, :D], ring_v[:, :D], 0.05)
    perm = torch.randperm(512, device="cuda")
    o2 = w4.w4_decode_attention(dev(q), ring_k[perm][:, :D].contiguous(), ring_v[perm][:, :D].contiguous(), 0.05)
    torch.cuda.synchronize()
    check(o1, q, kb[:512], vb[:512], 0.05)
    assert torch.allclose(o1, o2, rtol=0, atol=1e-5)


def test_attention_argument_errors(w4):
    q = torch.zeros((9, 512), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w4.W4Error):
        w4.w4_decode_attention(q, k, k, 1.0)          # 9 heads
    with pytest.raises(w4.W4Error):
        w4.w4_decode_attention(q[:8, :384].contiguous(), k[:, :384], k[:, :384], 1.0)   # D = 384


@pytest.mark.parametrize("L", [4099, 20000])
def test_attention_one_hot_rows_expose_every_key(w4, L):
    """All scores equal (q = 0: uniform weights 1/L) and every value row one-hot
    at its own column (7j mod D): output d counts the keys whose row hits d, so a
    key dropped or counted twice at a split boundary moves that output by 1/L,
    far beyond the bound (1e-5 of the count over L)."""
    H, D = 2, 512
    q = np.zeros((H, D), dtype=np.uint16)
    rng = np.random.default_rng(L)
    k = synth.act_bits(rng.standard_normal((L, D)), BF16)
    vals = np.zeros((L, D))
    vals[np.arange(L), (7 * np.arange(L)) % D] = 1.0
    v = synth.act_bits(vals, BF16)
    o = w4.w4_decode_attention(dev(q), dev(k), dev(v), 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    counts = np.bincount((7 * np.arange(L)) % D, minlength=D) / L
    got = o.cpu().numpy().astype(np.float64)
    for h in range(H):
        assert np.all(np.abs(got[h] - counts) <= 1e-5 * counts + 1e-12), np.abs(got[h] - counts).max()
    check(o, q, k, v, 1.0 / np.sqrt(D))
