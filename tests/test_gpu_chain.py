"""The decode-step chain (one persistent launch) on the GPU.

Parity is teacher-forced: for each matrix, its input is recomputed from the
chain's own previous output with w4_rms_renorm (bitwise the chain's internal
input), and the matrix's output is checked against the oracle on that input.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_act, host_bits, within_bound

pytestmark = pytest.mark.gpu
F16 = synth.F16


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def make_mats(shapes, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    mats = []
    for N, K in shapes:
        c, s = synth.w4_matrix_torch(g, N, K, "cuda")
        mats.append((c[0], s[0].view(torch.bfloat16)))
    return mats


def check_teacher_forced(w4, mats, x0, ys, rows=None, full_upto=None):
    x = x0
    for i, ((c, s), y) in enumerate(zip(mats, ys)):
        N, K = c.shape[0], c.shape[1] * 8
        if i > 0:
            x = w4.w4_rms_renorm(ys[i - 1], K, out_dtype=torch.float16)
        torch.cuda.synchronize()
        cn = c.cpu().numpy().view(np.uint32)
        sn = s.view(torch.int16).cpu().numpy().view(np.uint16)
        xn = host_bits(x)
        yn = y.cpu().numpy()
        if full_upto is None or i < full_upto:
            yo, ao = oracle.gemv(cn, sn, N, K, xn, F16, threads=True)
            ok, worst = within_bound(yn[:N], yo, ao)
        else:
            ok = True
            for n0, n1 in rows(N):
                yo, ao = oracle.gemv(cn, sn, N, K, xn, F16, rows=(n0, n1))
                ok_r, worst = within_bound(yn[n0:n1], yo, ao)
                ok = ok and ok_r
        assert ok, (i, N, K, worst)


def test_chain_ragged_shapes(w4):
    shapes = [(100, 64), (200, 96), (33, 192), (4096, 32), (257, 2048), (1536, 256)]
    mats = make_mats(shapes, 1)
    ys = [torch.full((N,), float("nan"), device="cuda") for N, _ in shapes]
    rng = np.random.default_rng(1)
    x0 = dev_act(synth.activations(rng, 64, F16), F16)
    desc = w4.w4_chain_desc(mats, ys)
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(desc, x0, sync)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    # a call that ends without error leaves every exchange cell cleared
    assert int(torch.count_nonzero(sync)) == 0
    check_teacher_forced(w4, mats, x0, ys)
    # a second call reuses the sync buffer and reproduces every output bitwise
    first = [y.clone() for y in ys]
    w4.w4_gemv_chain(desc, x0, sync)
    torch.cuda.synchronize()
    for a, b in zip(first, ys):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_chain_decode_sweep_35_layers(w4):
    """Decode-step weight sweep: 35 layers of Wqkv 2560x1536, Wo 1536x2048,
    Wgate/up 16384x1536, Wdown 1536x8192 (distinct seeded weights), fp16 input
    ~ N(0,1), outputs renormalised between matrices."""
    shapes = [(2560, 1536), (1536, 2048), (16384, 1536), (1536, 8192)] * 35
    mats = make_mats(shapes, 0)
    ys = [torch.empty(N, device="cuda") for N, _ in shapes]
    x0 = dev_act(synth.activations(np.random.default_rng(0), 1536, F16), F16)
    desc = w4.w4_chain_desc(mats, ys)
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(desc, x0, sync)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    assert int(torch.count_nonzero(sync)) == 0

    def rows(N):
        return [(0, 64), (N // 2, N // 2 + 64), (N - 64, N)]
    check_teacher_forced(w4, mats, x0, ys, rows=rows, full_upto=4)


def test_chain_longer_than_descriptor_cache(w4):
    """300 small matrices: descriptors past the first 256 are brought into the
    kernel's table while the chain runs."""
    shapes = [(96, 64), (64, 96), (160, 64)] * 100
    mats = make_mats(shapes, 4)
    ys = [torch.full((N,), float("nan"), device="cuda") for N, _ in shapes]
    x0 = dev_act(synth.activations(np.random.default_rng(4), 64, F16), F16)
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(w4.w4_chain_desc(mats, ys), x0, sync)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    check_teacher_forced(w4, mats, x0, ys)


def test_chain_invalid_descriptor_sets_error_word(w4):
    shapes = [(64, 64), (64, 128)]          # K of matrix 1 exceeds N of matrix 0
    mats = make_mats(shapes, 2)
    ys = [torch.full((N,), float("nan"), device="cuda") for N, _ in shapes]
    x0 = torch.zeros(64, dtype=torch.float16, device="cuda")
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(w4.w4_chain_desc(mats, ys), x0, sync)
    torch.cuda.synchronize()
    assert sync[2].item() == 2 and sync[0].item() == 0
    assert torch.all(torch.isnan(ys[0]))


def test_chain_barrier_timeout_is_reported_and_recovers(w4, w4_settings):
    shapes = [(512, 64), (512, 512), (512, 512)]
    mats = make_mats(shapes, 3)
    ys = [torch.zeros(N, device="cuda") for N, _ in shapes]
    x0 = dev_act(synth.activations(np.random.default_rng(3), 64, F16), F16)
    desc = w4.w4_chain_desc(mats, ys)
    sync = w4.w4_chain_sync(len(shapes))
    w4_settings("W4_CHAIN_SPIN_LIMIT", "0")   # host-forced: every barrier wait gives up
    w4.w4_gemv_chain(desc, x0, sync)
    torch.cuda.synchronize()
    assert sync[2].item() == 1                        # reported, no hang
    assert sync[0].item() == 0
    w4_settings("W4_CHAIN_SPIN_LIMIT")
    sync.zero_()
    w4.w4_gemv_chain(desc, x0, sync)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    check_teacher_forced(w4, mats, x0, ys)
