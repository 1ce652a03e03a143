"""The decode-step chain (one persistent launch) on the GPU.

Parity is teacher-forced: for each matrix i > 0, its input is the exact value
x = u / r, with u the leading K entries of the chain's own output of matrix
i - 1 and r their RMS (both in fp64 on the host), and the matrix's output is
checked against the oracle's product on that x, within the bound
|y - y_exact| <= 1e-3 * sum_k |w x| per output.
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


def chain_input(x0, ys, i, K):
    """The exact input of matrix i: x0 (fp16 values) for the first, else the
    previous output's leading K entries over their RMS, in fp64."""
    if i == 0:
        return oracle.act_to_f64(host_bits(x0), F16)
    u = ys[i - 1][:K].cpu().numpy().astype(np.float64)
    r = np.sqrt(np.mean(u * u))
    return u / r if r > 0 else np.zeros(K)


def check_teacher_forced(w4, mats, x0, ys, rows=None, full_upto=None):
    torch.cuda.synchronize()
    for i, ((c, s), y) in enumerate(zip(mats, ys)):
        N, K = c.shape[0], c.shape[1] * 8
        cn = c.cpu().numpy().view(np.uint32)
        sn = s.view(torch.int16).cpu().numpy().view(np.uint16)
        x = chain_input(x0, ys, i, K)
        yn = y.cpu().numpy()
        if full_upto is None or i < full_upto:
            yo, ao = oracle.gemv_x64(cn, sn, N, K, x)
            ok, worst = within_bound(yn[:N], yo, ao)
        else:
            ok = True
            for n0, n1 in rows(N):
                yo, ao = oracle.gemv_x64(cn, sn, N, K, x, rows=(n0, n1))
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


def test_chain_on_a_stream_of_its_own_matches_the_default_stream(w4):
    """The cooperative chain launched on a non-default stream (as the sweep
    benchmark runs it), with other streams in use, gives the bits of the same
    chain on the default stream and leaves every exchange cell cleared."""
    shapes = [(2560, 1536), (1536, 2048), (16384, 1536), (1536, 8192)] * 3
    mats = make_mats(shapes, 5)
    x0 = dev_act(synth.activations(np.random.default_rng(5), 1536, F16), F16)
    ref = [torch.empty(N, device="cuda") for N, _ in shapes]
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(w4.w4_chain_desc(mats, ref), x0, sync)
    torch.cuda.synchronize()
    busy = torch.zeros(1 << 16, device="cuda")
    others = [torch.cuda.Stream() for _ in range(4)]
    for s_ in others:
        with torch.cuda.stream(s_):
            busy.add_(1.0)
    own = torch.cuda.Stream()
    ys = [torch.full((N,), float("nan"), device="cuda") for N, _ in shapes]
    desc = w4.w4_chain_desc(mats, ys)
    torch.cuda.synchronize()
    with torch.cuda.stream(own):
        w4.w4_gemv_chain(desc, x0, sync)
        w4.w4_gemv_chain(desc, x0, sync, stream=own)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    assert int(torch.count_nonzero(sync)) == 0
    for a, b in zip(ref, ys):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


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


def test_chain_wide_range_and_zero_vectors(w4):
    """Steps spanning 2^-60 .. 2^70 between matrices (outputs far outside fp16's
    range; each input group gets its own power of two), a group of huge values
    next to tiny ones, and a matrix whose codes are all 8 (a zero output, so
    the next input is the zero vector and gives zeros)."""
    rng = np.random.default_rng(12)
    shapes = [(512, 64), (640, 512), (256, 640), (256, 256), (384, 256)]
    scales = [2.0 ** 70, 2.0 ** -60, 1.0, 1.0, 2.0 ** 20]   # squares of 2^72 overflow fp32
    mats = []
    for (N, K), sc in zip(shapes, scales):
        codes, steps = synth.w4_matrix(rng, N, K)
        sv = oracle.act_to_f64(steps.ravel(), synth.BF16).reshape(steps.shape) * sc
        steps = synth.act_bits(sv, synth.BF16)
        mats.append((codes, steps))
    # rows 0..31 of matrix 1 get steps 2^40 larger: one input group of matrix
    # 2 is huge next to the others
    c1, s1 = mats[1]
    s1 = s1.copy()
    s1[:32] = synth.act_bits(oracle.act_to_f64(s1[:32].ravel(), synth.BF16).reshape(32, -1) * 2.0 ** 40,
                             synth.BF16)
    mats[1] = (c1, s1)
    mats[3] = (np.full_like(mats[3][0], 0x88888888), mats[3][1])   # all codes 8
    dm = [(torch.from_numpy(c.view(np.int32)).cuda(),
           torch.from_numpy(s.view(np.int16)).cuda().view(torch.bfloat16)) for c, s in mats]
    ys = [torch.full((N,), float("nan"), device="cuda") for N, _ in shapes]
    x0 = dev_act(synth.activations(rng, 64, F16), F16)
    sync = w4.w4_chain_sync(len(shapes))
    w4.w4_gemv_chain(w4.w4_chain_desc(dm, ys), x0, sync)
    torch.cuda.synchronize()
    assert sync[0].item() == 0 and sync[2].item() == 0
    assert torch.all(ys[3] == 0) and torch.all(ys[4] == 0)
    check_teacher_forced(w4, dm, x0, ys)
