"""Small-M W4A16 product on the GPU (MFMA path) against the CPU oracle."""

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


def run_gemm(w4, codes, steps, X, dt, M, K, ldx=None, ldy=None):
    N = codes.shape[0]
    ldx = K if ldx is None else ldx
    ldy = N if ldy is None else ldy
    dX = dev_act(X.reshape(M, ldx), dt)
    Y = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4_gemm_smallM(dev_codes(codes), dev_steps(steps), dX, Y)
    torch.cuda.synchronize()
    return Y.cpu().numpy()[:, :N]


def oracle_rows(codes, steps, N, K, X, dt, M):
    Y, A = [], []
    for m in range(M):
        y, a = oracle.gemv(codes, steps, N, K, X[m, :K], dt, threads=True)
        Y.append(y)
        A.append(a)
    return np.array(Y), np.array(A)


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("N,K,M", [(33, 64, 1), (97, 704, 2), (257, 1536, 4), (1000, 2048, 8),
                                   (129, 8192, 16), (1536, 2816, 3), (65, 96, 16),
                                   (4097, 1536, 16), (17, 4096, 5), (31, 8192, 7),
                                   (300, 3104, 9), (65, 3072, 16), (31, 16384, 2)])
def test_gemm_shapes_vs_oracle(w4, N, K, M, dt):
    print(f"gemm N={N} K={K} M={M} dt={dt}", flush=True)
    rng = np.random.default_rng(N + K + M + dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), dt)
    Y = run_gemm(w4, codes, steps, X, dt, M, K)
    Yo, Ao = oracle_rows(codes, steps, N, K, X, dt, M)
    ok, worst = within_bound(Y, Yo, Ao)
    assert ok, worst


@pytest.mark.parametrize("M", [2, 4, 8, 16])
def test_gemm_decode_sweep_shapes(w4, M):
    """Small-batch GEMM on the four decode-sweep shapes, bf16 rows, seed 0."""
    rng = np.random.default_rng(0)
    for N, K in [(2560, 1536), (1536, 2048), (16384, 1536), (1536, 8192)]:
        codes, steps = synth.w4_matrix(rng, N, K)
        X = synth.activations(rng, (M, K), BF16)
        Y = run_gemm(w4, codes, steps, X, BF16, M, K)
        Y2 = run_gemm(w4, codes, steps, X, BF16, M, K)
        assert Y.tobytes() == Y2.tobytes()
        Yo, Ao = oracle_rows(codes, steps, N, K, X, BF16, M)
        ok, worst = within_bound(Y, Yo, Ao)
        assert ok, (N, K, M, worst)


def test_gemm_split_k_is_deterministic_and_survives_other_calls(w4, w4_settings):
    """A product split into K-slices and summed by the last slice to arrive:
    bitwise the same on every call, also when expert products (which share the
    library's device buffer) run in between.  (Four rows on the matrix cores.)"""
    w4_settings("W4_SMALLM_ROWS_MAX", "0")
    rng = np.random.default_rng(11)
    N, K, M = 1536, 8192, 4
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), BF16)
    first = run_gemm(w4, codes, steps, X, BF16, M, K)
    Yo, Ao = oracle_rows(codes, steps, N, K, X, BF16, M)
    assert within_bound(first, Yo, Ao)[0]
    # an expert product with route weights in between (it uses the same buffer)
    E, Ne, Ke, topk = 4, 64, 256, 2
    ec, es = synth.w4_matrix(rng, E * Ne, Ke)
    ids = torch.tensor([[0, 3]], dtype=torch.int32, device="cuda")
    route = torch.tensor([[0.25, 0.75]], dtype=torch.float32, device="cuda")
    xe = dev_act(synth.activations(rng, (1, Ke), BF16), BF16)
    Ye = torch.empty((1, Ne), device="cuda")
    w4.w4_moe_gemv_ids(dev_codes(ec), dev_steps(es), Ne * Ke // 8, Ne * Ke // 32, Ne, Ke, xe, ids,
                       n_experts=E, route_w=route, Y=Ye)
    for _ in range(3):
        again = run_gemm(w4, codes, steps, X, BF16, M, K)
        assert again.tobytes() == first.tobytes()


def test_gemm_leading_dimensions(w4):
    rng = np.random.default_rng(1)
    N, K, M, ldx, ldy = 300, 1536, 6, 1600, 333
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, ldx), F16)
    Y = run_gemm(w4, codes, steps, X, F16, M, K, ldx=ldx, ldy=ldy)
    Yo, Ao = oracle_rows(codes, steps, N, K, X, F16, M)
    assert within_bound(Y, Yo, Ao)[0]


@pytest.mark.parametrize("M,dt", [(8, BF16), (16, F16), (6, BF16)])
def test_gemm_rows_not_16_byte_aligned(w4, M, dt):
    """Activation rows that are not 16-byte aligned (an odd row stride, and a
    view that starts one element in) are staged by 16-bit loads instead of
    direct-to-LDS copies: the same staged values, so the same bits as the
    aligned rows, and within the bound of the oracle."""
    print(f"smallM unaligned rows M={M} dt={dt}", flush=True)
    rng = np.random.default_rng(30 + M + dt)
    N, K = 700, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), dt)
    dc, ds = dev_codes(codes), dev_steps(steps)
    ref = w4.w4_gemm_smallM(dc, ds, dev_act(X, dt))
    ld = K + 3                                   # odd row stride (not a multiple of 8)
    big = np.zeros((M, ld + 1), dtype=np.uint16)
    big[:, 1:K + 1] = X                          # rows start one element in
    dbig = dev_act(big, dt)
    Xv = dbig[:, 1:K + 1]
    assert Xv.stride(0) == ld + 1 and (Xv.data_ptr() % 16) != 0
    got = w4.w4_gemm_smallM(dc, ds, Xv)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))
    Yo, Ao = oracle_rows(codes, steps, N, K, X, dt, M)
    assert within_bound(got.cpu().numpy(), Yo, Ao)[0]


def test_gemm_one_hot_rows_are_bit_exact(w4):
    rng = np.random.default_rng(2)
    N, K, M = 64, 2048, 16
    codes, steps = synth.w4_matrix(rng, N, K)
    X = np.zeros((M, K), dtype=np.uint16)
    for m in range(M):
        X[m, (m * 131) % K] = [0x3C00, 0x0001, 0xB555, 0x03FF][m % 4]
    Y = run_gemm(w4, codes, steps, X, F16, M, K)
    Yo, _ = oracle_rows(codes, steps, N, K, X, F16, M)
    assert np.array_equal(Y.astype(np.float64), Yo)


def test_gemm_rows_of_very_different_scale(w4):
    rng = np.random.default_rng(3)
    N, K, M = 200, 1536, 4
    codes, steps = synth.w4_matrix(rng, N, K)
    v = rng.normal(0, 1, (M, K)) * np.array([[1e-6], [1.0], [1e4], [3e-2]])
    X = synth.act_bits(v, BF16)
    Y = run_gemm(w4, codes, steps, X, BF16, M, K)
    Yo, Ao = oracle_rows(codes, steps, N, K, X, BF16, M)
    assert within_bound(Y, Yo, Ao)[0]


def test_gemm_wide_range_row_takes_exact_path(w4):
    rng = np.random.default_rng(4)
    N, K, M = 100, 2048, 3
    codes, steps = synth.w4_matrix(rng, N, K)
    v = rng.normal(0, 1, (M, K))
    v[1, ::5] *= 2.0**14
    v[1, 1::7] *= 2.0**-20
    X = synth.act_bits(v, F16)
    Y = run_gemm(w4, codes, steps, X, F16, M, K)
    Yo, Ao = oracle_rows(codes, steps, N, K, X, F16, M)
    assert within_bound(Y, Yo, Ao)[0]


def test_gemm_integer_inputs_are_bit_exact(w4):
    rng = np.random.default_rng(5)
    N, K, M = 130, 1536, 8
    codes, _ = synth.w4_matrix(rng, N, K)
    steps = (0x3F80 - 0x80 * rng.integers(0, 5, size=(N, K // 32))).astype(np.uint16)
    X = rng.choice(np.array([0xBC00, 0x0000, 0x3C00], dtype=np.uint16), size=(M, K))
    Y = run_gemm(w4, codes, steps, X, F16, M, K)
    Yo, _ = oracle_rows(codes, steps, N, K, X, F16, M)
    assert np.array_equal(Y.astype(np.float64), Yo)


def test_gemm_rejects_k_beyond_limit(w4):
    K = w4.W4_MAX_K_SMALLM + 32
    codes = torch.zeros((4, K // 8), dtype=torch.int32, device="cuda")
    steps = torch.zeros((4, K // 32), dtype=torch.bfloat16, device="cuda")
    X = torch.zeros((2, K), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4Error) as e:
        w4.w4_gemm_smallM(codes, steps, X)
    assert e.value.status == w4.W4_ERR_UNSUPPORTED


@pytest.mark.parametrize("M", [2, 3, 4])
def test_gemm_few_rows_match_batch1_bitwise(w4, M):
    """Up to four rows run as batch-1 products side by side: every row has the
    bits of w4_gemv on that row alone."""
    rng = np.random.default_rng(40 + M)
    N, K = 5000, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, K), BF16)
    Y = run_gemm(w4, codes, steps, X, BF16, M, K)
    for m in range(M):
        y = torch.empty(N, device="cuda")
        w4.w4_gemv(dev_codes(codes), dev_steps(steps), dev_act(X[m], BF16), y)
        torch.cuda.synchronize()
        assert y.cpu().numpy().tobytes() == Y[m].tobytes(), m


def test_gemm_few_rows_on_the_matrix_cores(w4, w4_settings):
    """Two to four rows forced onto the MFMA engine (the path from 5 rows)."""
    w4_settings("W4_SMALLM_ROWS_MAX", "0")
    rng = np.random.default_rng(30)
    for N, K, M in [(2560, 1536, 2), (1536, 2048, 4), (97, 704, 3), (1536, 8192, 4)]:
        codes, steps = synth.w4_matrix(rng, N, K)
        X = synth.activations(rng, (M, K), BF16)
        Y = run_gemm(w4, codes, steps, X, BF16, M, K)
        Yo, Ao = oracle_rows(codes, steps, N, K, X, BF16, M)
        assert within_bound(Y, Yo, Ao)[0], (N, K, M)
