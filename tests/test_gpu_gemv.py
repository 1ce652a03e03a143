"""GEMV parity on the GPU: libw4 (through the C ABI) against the CPU oracle."""

import os

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


def run_gemv(w4, codes, steps, x, dt):
    y = torch.full((codes.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4_gemv(dev_codes(codes), dev_steps(steps), dev_act(x, dt), y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("N,K", [(1, 32), (7, 64), (33, 96), (65, 704), (97, 1536), (257, 2048),
                                 (1000, 2816), (129, 8192), (31, 16384), (513, 4096),
                                 (4097, 1536), (20000, 704)])
def test_gemv_shapes_vs_oracle(w4, N, K, dt):
    print(f"gemv N={N} K={K} dt={dt}", flush=True)
    rng = np.random.default_rng(N * 7 + K + dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    x = synth.activations(rng, K, dt)
    y = run_gemv(w4, codes, steps, x, dt)
    yo, ao = oracle.gemv(codes, steps, N, K, x, dt, threads=True)
    ok, worst = within_bound(y, yo, ao)
    assert ok, f"worst |err|/sum|wx| = {worst}"


# The streaming (LDS ring) variant, forced through the tile override
# "L,NG,R,waves,blocks,ring depth" on shapes that span several tiles per wave,
# a ragged last tile, waves without any tile, and every ring depth.
RING_CASES = [(1000, 1536, "16,3,1,8,3,4"), (257, 2048, "16,4,1,8,2,3"),
              (129, 8192, "64,4,1,8,5,2"), (1000, 2816, "32,3,1,8,4,5"), (700, 1536, "16,3,1,4,3,6"),
              (33, 1536, "16,3,1,8,64,5"), (4097, 4096, "32,4,1,4,7,5"),
              (20001, 1536, "16,3,1,8,256,5")]


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("N,K,tile", RING_CASES)
def test_gemv_streaming_variant_vs_oracle(w4, w4_settings, N, K, tile, dt):
    print(f"gemv ring N={N} K={K} tile={tile} dt={dt}", flush=True)
    w4_settings("W4_GEMV_TILE", tile)
    rng = np.random.default_rng(N * 11 + K + dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    x = synth.activations(rng, K, dt)
    y = run_gemv(w4, codes, steps, x, dt)
    yo, ao = oracle.gemv(codes, steps, N, K, x, dt, threads=True)
    ok, worst = within_bound(y, yo, ao)
    assert ok, f"worst |err|/sum|wx| = {worst}"


def test_gemv_streaming_variant_exact_cases(w4, w4_settings):
    """Integer inputs (bit-exact), a one-hot subnormal x (bit-exact) and a
    vector too wide for fp16 staging (the exact fp32 path) through the ring."""
    w4_settings("W4_GEMV_TILE", "16,4,1,8,2,4")
    rng = np.random.default_rng(14)
    N, K = 300, 2048
    codes, _ = synth.w4_matrix(rng, N, K)
    steps = (0x3F80 - 0x80 * rng.integers(0, 5, size=(N, K // 32))).astype(np.uint16)
    x = rng.choice(np.array([0xBC00, 0x0000, 0x3C00], dtype=np.uint16), size=K)
    y = run_gemv(w4, codes, steps, x, F16)
    yo, _ = oracle.gemv(codes, steps, N, K, x, F16)
    assert np.array_equal(y.astype(np.float64), yo)
    x = np.zeros(K, dtype=np.uint16)
    x[1999] = 0x0001
    y = run_gemv(w4, codes, steps, x, F16)
    yo, _ = oracle.gemv(codes, steps, N, K, x, F16)
    assert np.array_equal(y.astype(np.float64), yo)
    w4_settings("W4_GEMV_TILE", "16,3,1,8,2,5")
    N, K = 129, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    v = rng.normal(0, 1, K)
    v[::7] *= 2.0**12
    v[3::11] *= 2.0**-20
    for dt in (F16, BF16):
        x = synth.act_bits(v, dt)
        y = run_gemv(w4, codes, steps, x, dt)
        yo, ao = oracle.gemv(codes, steps, N, K, x, dt)
        assert within_bound(y, yo, ao)[0], dt


def test_gemv_config_single_2048x1536_f16(w4):
    """Single W4A16 GEMV: 2048 x 1536, fp16 x, seed 0 -- every output."""
    rng = np.random.default_rng(0)
    codes, steps = synth.w4_matrix(rng, 2048, 1536)
    x = synth.activations(rng, 1536, F16)
    y = run_gemv(w4, codes, steps, x, F16)
    yo, ao = oracle.gemv(codes, steps, 2048, 1536, x, F16, threads=True)
    ok, worst = within_bound(y, yo, ao)
    assert ok, worst
    print(f"worst |err|/sum|wx| = {worst:.3e}")


def test_gemv_vocab_head_262144x1536_bf16_sampled(w4):
    """Vocabulary-head GEMV 262144 x 1536, bf16 x, in the benchmark's launch
    configuration; the oracle checks sampled row ranges."""
    rng = np.random.default_rng(0)
    V, K = 262144, 1536
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, BF16)
    y = run_gemv(w4, codes, steps, x, BF16)
    y2 = run_gemv(w4, codes, steps, x, BF16)
    assert y.tobytes() == y2.tobytes()           # deterministic
    for n0, n1 in [(0, 1024), (131000, 131500), (V - 1024, V)]:
        yo, ao = oracle.gemv(codes, steps, V, K, x, BF16, rows=(n0, n1))
        ok, worst = within_bound(y[n0:n1], yo, ao)
        assert ok, (n0, worst)
    for n in np.random.default_rng(1).integers(0, V, 64):
        yo, ao = oracle.gemv(codes, steps, V, K, x, BF16, rows=(n, n + 1))
        assert within_bound(y[n:n + 1], yo, ao)[0]


@pytest.mark.parametrize("dt", [F16, BF16])
@pytest.mark.parametrize("N,K", [(97, 1536), (1000, 2816), (20000, 704)])
def test_gemv_x_not_16_byte_aligned(w4, N, K, dt):
    """An activation vector that starts one element past a 16-byte boundary is
    copied to LDS by 16-bit loads instead of direct-to-LDS copies: the same
    staged values, so the bits of the aligned vector."""
    print(f"gemv unaligned x N={N} K={K} dt={dt}", flush=True)
    rng = np.random.default_rng(N + K + 5 * dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    x = synth.activations(rng, K, dt)
    dc, ds = dev_codes(codes), dev_steps(steps)
    ref = w4.w4_gemv(dc, ds, dev_act(x, dt))
    big = np.zeros(K + 8, dtype=np.uint16)
    big[1:K + 1] = x
    xv = dev_act(big, dt)[1:K + 1]
    assert xv.data_ptr() % 16 != 0
    got = w4.w4_gemv(dc, ds, xv)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


@pytest.mark.parametrize("dt", [F16, BF16])
def test_gemv_one_hot_is_bit_exact(w4, dt):
    rng = np.random.default_rng(3)
    N, K = 77, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    vals = [0x3C00, 0x0001, 0x03FF, 0xB555] if dt == F16 else [0x3F80, 0x2F80, 0xBEAB, 0x4B00]
    for k, xb in zip([0, 37, 1000, 1535], vals):
        x = np.zeros(K, dtype=np.uint16)
        x[k] = xb
        y = run_gemv(w4, codes, steps, x, dt)
        yo, _ = oracle.gemv(codes, steps, N, K, x, dt)
        assert np.array_equal(y.astype(np.float64), yo), (k, hex(xb))


def test_gemv_integer_inputs_are_bit_exact(w4):
    rng = np.random.default_rng(4)
    N, K = 300, 2048
    codes, _ = synth.w4_matrix(rng, N, K)
    steps = (0x3F80 - 0x80 * rng.integers(0, 5, size=(N, K // 32))).astype(np.uint16)  # 2^-4..1
    x = rng.choice(np.array([0xBC00, 0x0000, 0x3C00], dtype=np.uint16), size=K)      # -1, 0, 1
    y = run_gemv(w4, codes, steps, x, F16)
    yo, _ = oracle.gemv(codes, steps, N, K, x, F16)
    assert np.array_equal(y.astype(np.float64), yo)


def test_gemv_zero_weight_rows_are_exactly_zero(w4):
    rng = np.random.default_rng(5)
    N, K = 64, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    codes[::3] = 0x88888888
    x = synth.activations(rng, K, BF16)
    y = run_gemv(w4, codes, steps, x, BF16)
    assert np.all(y[::3] == 0.0)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_gemv_wide_range_activations(w4, dt):
    """A vector spanning more than 2^28 cannot be staged exactly in fp16 and
    takes the fp32 path; results must still meet the bound."""
    rng = np.random.default_rng(6)
    N, K = 129, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    v = rng.normal(0, 1, K)
    v[::7] *= 2.0**12
    v[3::11] *= 2.0**-20
    x = synth.act_bits(v, dt)
    y = run_gemv(w4, codes, steps, x, dt)
    yo, ao = oracle.gemv(codes, steps, N, K, x, dt)
    ok, worst = within_bound(y, yo, ao)
    assert ok, worst


def test_gemv_subnormal_f16_activations(w4):
    rng = np.random.default_rng(7)
    N, K = 100, 1536
    codes, steps = synth.w4_matrix(rng, N, K)
    x = rng.integers(1, 0x0400, size=K).astype(np.uint16)  # all fp16 subnormals
    x[::2] |= 0x8000
    y = run_gemv(w4, codes, steps, x, F16)
    yo, ao = oracle.gemv(codes, steps, N, K, x, F16)
    assert within_bound(y, yo, ao)[0]


def test_gemv_k_zero_writes_zeros(w4):
    y = torch.full((5,), float("nan"), device="cuda")
    codes = torch.zeros((5, 0), dtype=torch.int32, device="cuda")
    steps = torch.zeros((5, 0), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(0, dtype=torch.float16, device="cuda")
    w4.w4_gemv(codes, steps, x, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_gemv_failed_launch_leaves_poisoned_output(w4, w4_settings):
    rng = np.random.default_rng(8)
    codes, steps = synth.w4_matrix(rng, 16, 64)
    x = synth.activations(rng, 64, F16)
    y = torch.full((16,), float("nan"), device="cuda")
    w4_settings("W4_FORCE_LAUNCH_ERROR", "1")
    with pytest.raises(w4.W4Error) as e:
        w4.w4_gemv(dev_codes(codes), dev_steps(steps), dev_act(x, F16), y)
    assert e.value.status == w4.W4_ERR_HIP
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(y))


def test_rms_renorm_within_one_ulp(w4):
    rng = np.random.default_rng(9)
    for K, dt in [(1536, F16), (2048, F16), (8192, BF16), (704, BF16), (12288, F16), (4, BF16)]:
        v = (rng.normal(0, 5, size=K + 100)).astype(np.float32)
        out = w4.w4_rms_renorm(torch.from_numpy(v).cuda(), K,
                               out_dtype=torch.float16 if dt == F16 else torch.bfloat16)
        assert out.shape == (K,)
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
        ref = oracle.rms_renorm(v, K, dt).astype(np.int64)
        # same sign; neighbouring bit patterns are neighbouring values
        assert np.all(np.abs(got - ref) <= 1), (K, dt)
