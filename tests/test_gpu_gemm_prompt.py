"""Prompt-chunk W4A16 product (matrix cores, M up to 4096) against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_act, dev_codes, dev_steps, within_bound

pytestmark = pytest.mark.gpu
F16, BF16 = synth.F16, synth.BF16


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def run_prompt(w4, codes, steps, X, dt, M, K, ldx=None, ldy=None):
    N = codes.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    dX = dev_act(X.reshape(M, ldx), dt)
    Y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4_gemm_prompt(dev_codes(codes), dev_steps(steps), dX, Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()[:, :N]


def check(Y, codes, steps, K, X, dt, M):
    Yo, Ao = oracle.gemm(codes, steps, codes.shape[0], K, X, dt, M, ldx=X.shape[1])
    ok, worst = within_bound(Y, Yo, Ao)
    assert ok, worst


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("N,K,M", [(1, 32, 1), (193, 96, 17), (200, 1536, 256), (1000, 704, 100),
                                   (64, 8192, 33), (385, 2816, 129), (577, 1536, 64),
                                   (31, 16384, 3), (250, 3104, 300)])
def test_prompt_shapes_vs_oracle(w4, N, K, M, dt):
    """Ragged on every axis: N past a 192-row block, K/32 not a multiple of 4,
    M past a 16-, 32-, 64- or 128-row block."""
    print(f"prompt N={N} K={K} M={M} dt={dt}", flush=True)
    rng = np.random.default_rng(N * 7 + K + M + dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), dt)
    Y = run_prompt(w4, codes, steps, X, dt, M, K)
    check(Y, codes, steps, K, X, dt, M)


def test_prompt_strided_rows(w4):
    rng = np.random.default_rng(5)
    N, K, M, ldx, ldy = 300, 1536, 40, 1600, 310
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, ldx), BF16)
    dX = dev_act(X, BF16)
    Y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4_gemm_prompt(dev_codes(codes), dev_steps(steps), dX, Y)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    check(Yh[:, :N], codes, steps, K, X, BF16, M)
    assert np.all(np.isnan(Yh[:, N:]))  # columns past N untouched


def test_prompt_chunk_full_size_sampled(w4):
    """[256, 1536] x [1536, 24576], bf16 rows, seed 0: the whole product on the
    GPU, checked on blocks of weight rows (the first, a middle one, the ragged
    end) for all 256 activation rows; two calls give the same bits."""
    rng = np.random.default_rng(0)
    N, K, M = 24576, 1536, 256
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), BF16)
    dc, ds, dX = dev_codes(codes), dev_steps(steps), dev_act(X, BF16)
    Y = w4.w4_gemm_prompt(dc, ds, dX)
    Y2 = w4.w4_gemm_prompt(dc, ds, dX)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int32), Y2.view(torch.int32))
    Yh = Y.cpu().numpy()
    for n0, n1 in [(0, 192), (12000, 12384), (N - 200, N)]:
        Yo, Ao = oracle.gemm(codes[n0:n1], steps[n0:n1], n1 - n0, K, X, BF16, M)
        ok, worst = within_bound(Yh[:, n0:n1], Yo, Ao)
        assert ok, (n0, worst)


def test_prompt_rows_with_wide_steps_take_the_exact_path(w4):
    """Weight rows whose steps span more than 2^25, or hold a bf16 subnormal,
    cannot be scaled into fp16 by one power of two; their tiles apply each
    group's step to the fp32 sums instead -- still within the bound."""
    rng = np.random.default_rng(9)
    N, K, M = 400, 1536, 48
    codes, steps = synth.w4_matrix(rng, N, K)
    steps = steps.copy()
    steps[3, 5] = oracle.f64_to_bf16(1e-12)      # 2^-40 against steps near 2^-6
    steps[250, 0] = oracle.f64_to_bf16(3e4)
    steps[251, 7] = 0x0003                       # a bf16 subnormal step
    steps[100, :] = 0                            # an all-zero row
    X = synth.activations(rng, (M, K), F16)
    Y = run_prompt(w4, codes, steps, X, F16, M, K)
    check(Y, codes, steps, K, X, F16, M)
    assert np.all(Y[:, 100] == 0.0)


@pytest.mark.parametrize("span", [20, 21, 22])
def test_prompt_step_span_at_the_scaling_limit(w4, span):
    """A weight row whose nonzero steps span 2^span: up to 2^21 it is scaled
    into fp16 with its steps inside the operand, beyond that its tile applies
    the steps to fp32 sums.  Both sides of the limit stay within the bound."""
    rng = np.random.default_rng(40 + span)
    N, K, M = 100, 1024, 40
    codes, steps = synth.w4_matrix(rng, N, K)
    steps = steps.copy()
    steps[17, :] = oracle.f64_to_bf16(1.0)
    steps[17, 3] = oracle.f64_to_bf16(2.0 ** -span)
    X = synth.activations(rng, (M, K), BF16)
    Y = run_prompt(w4, codes, steps, X, BF16, M, K)
    check(Y, codes, steps, K, X, BF16, M)


def test_prompt_largest_chunk(w4):
    """M = 4096 activation rows (the largest chunk), a narrow matrix."""
    rng = np.random.default_rng(77)
    N, K, M = 70, 64, 4096
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), BF16)
    Y = run_prompt(w4, codes, steps, X, BF16, M, K)
    check(Y, codes, steps, K, X, BF16, M)


def test_prompt_bf16_rows_beyond_fp16_range(w4):
    """A bf16 activation row spanning more than 2^31 cannot be staged as fp16
    with one power of two; its block of rows is computed with plain fp32
    products -- still within the bound, and the other blocks are unaffected."""
    rng = np.random.default_rng(13)
    N, K, M = 300, 704, 200
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), BF16).copy()
    X[7, 3] = oracle.f64_to_bf16(1e20)
    X[7, 9] = oracle.f64_to_bf16(1e-20)
    X[150, :] = 0
    Y = run_prompt(w4, codes, steps, X, BF16, M, K)
    check(Y, codes, steps, K, X, BF16, M)
    assert np.all(Y[150] == 0.0)


def test_prompt_integer_operands_are_exact(w4):
    """Integer activations and power-of-two steps: every partial sum is an
    integer below 2^24, so the result must equal the oracle exactly."""
    rng = np.random.default_rng(21)
    N, K, M = 200, 512, 40
    codes = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    steps = np.full((N, K // 32), oracle.f64_to_bf16(0.5), dtype=np.uint16)
    steps[::3] = oracle.f64_to_bf16(4.0)
    X = np.array([[oracle.f64_to_f16(float(v)) for v in row]
                  for row in rng.integers(-6, 7, size=(M, K))], dtype=np.uint16)
    Y = run_prompt(w4, codes, steps, X, F16, M, K)
    Yo, _ = oracle.gemm(codes, steps, N, K, X, F16, M)
    assert np.array_equal(Y.astype(np.float64), Yo)


def test_prompt_argument_errors(w4):
    rng = np.random.default_rng(1)
    codes, steps = synth.w4_matrix(rng, 64, 64)
    X = torch.zeros((4097, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4Error):
        w4.w4_gemm_prompt(dev_codes(codes), dev_steps(steps), X)
