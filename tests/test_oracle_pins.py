"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: the IEEE/bf16 format
definitions as implemented by NumPy and PyTorch, a NumPy brute force that unpacks
through a byte view, closed forms, hand-derived fixtures under ``tests/golden``,
and invariants stated on the pages.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F16, BF16 = synth.F16, synth.BF16


# --- format decoders and rounding -------------------------------------------

def test_f16_decode_exhaustive_matches_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.act_to_f64(bits, F16)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_bf16_decode_exhaustive_matches_bit_reinterpretation():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.act_to_f64(bits, BF16)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def _rounding_probe_values(rng):
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 7e4, 2.0**-24, 2.0**-25,
         3 * 2.0**-26, 2.0**-14, 2.0**-14 - 2.0**-25, 1e-30, 3e38, 3.4e38, 1e39]
    # ties of both formats: midpoints between neighbours
    v += [1 + 2.0**-11, 1 + 3 * 2.0**-11, 1 + 2.0**-8, 1 + 3 * 2.0**-8, 2049.0, 2051.0]
    v += list(rng.normal(0, 1, 3000)) + list(rng.normal(0, 1, 3000) * 1e-6)
    v += list(np.exp(rng.uniform(-100, 100, 3000)))
    return np.array(v, dtype=np.float64)


def test_f64_to_f16_rne_matches_numpy():
    vals = _rounding_probe_values(np.random.default_rng(1))
    vals = np.concatenate([vals, -vals])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_f64_to_bf16_rne_matches_torch_on_f32_values():
    # torch rounds float32 -> bfloat16 to nearest-even; feed values exact in fp32
    vals = _rounding_probe_values(np.random.default_rng(2)).astype(np.float32)
    vals = np.concatenate([vals, -vals, np.array([np.float32(1 + 2.0**-8)])])
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# --- the packed format ------------------------------------------------------

def test_unpack_every_code_at_every_nibble_position():
    # Build words from a byte array (low nibble of byte b = column 2b), which is
    # a different construction from the oracle's shift-and-mask.
    rng = np.random.default_rng(3)
    for pos in range(8):
        for v in range(16):
            cols = rng.integers(0, 16, size=8).astype(np.uint8)
            cols[pos] = v
            by = (cols[0::2] | (cols[1::2] << 4)).astype(np.uint8)
            word = by.view("<u4")
            assert oracle.code(word.reshape(1, 1), 8, 0, pos) == v


def test_unpack_matches_byte_view_on_random_rows():
    rng = np.random.default_rng(4)
    codes, steps = synth.w4_matrix(rng, 5, 96)
    ref = brute.unpack_codes(codes, 96)
    for n in range(5):
        for k in range(96):
            assert oracle.code(codes, 96, n, k) == ref[n, k]


def test_dequant_matches_brute_force_and_grid_invariants():
    rng = np.random.default_rng(5)
    N, K = 7, 704
    codes, steps = synth.w4_matrix(rng, N, K)
    W = oracle.dequant(codes, steps, N, K)
    assert np.array_equal(W, brute.dense(codes, steps, K))
    s = brute.bf16_bits_to_f64(steps)
    c = brute.unpack_codes(codes, K).astype(np.int64)
    # value 0 exactly where the code is 8; range [-8, 7] * step
    assert np.array_equal(W == 0.0, c == 8)
    ratio = W / np.repeat(s, 32, axis=1)
    assert ratio.min() >= -8 and ratio.max() <= 7
    assert np.array_equal(ratio, np.round(ratio))
    # every group of 32 holds at most 16 distinct values (Step 2 of the dev.to page)
    for n in range(N):
        for g in range(K // 32):
            assert np.unique(W[n, g * 32:(g + 1) * 32]).size <= 16


def test_generator_invariants():
    rng = np.random.default_rng(6)
    codes, steps = synth.w4_matrix(rng, 64, 1536)
    s = brute.bf16_bits_to_f64(steps)
    assert codes.dtype == np.uint32 and codes.shape == (64, 192)
    assert steps.shape == (64, 48)
    assert np.all(s > 0) and np.all(np.isfinite(s)) and s.min() >= 1e-4 * 0.99
    c = brute.unpack_codes(codes, 1536)
    counts = np.bincount(c.reshape(-1), minlength=16)
    assert counts.size == 16 and counts.min() > 0.8 * counts.mean()


def test_magic_float_conversions_are_exact():
    # Step 3 of the dev.to page: OR the code into the bits of 2^23 and subtract
    # 2^23 + 8.  The fp16 analogue (bits of 1024, subtract 1032) is what the
    # GPU kernels use; both must give c - 8 exactly for all 16 codes.
    for c in range(16):
        f32 = np.array([0x4B000000 | c], dtype=np.uint32).view(np.float32)[0]
        assert float(f32 - np.float32(2.0**23 + 8)) == c - 8
        f16 = np.array([0x6400 | c], dtype=np.uint16).view(np.float16)[0]
        assert float(f16 - np.float16(1032)) == c - 8
        f16hi = np.array([0x6400 | (c << 4)], dtype=np.uint16).view(np.float16)[0]
        assert float(np.float16(f16hi * np.float16(1 / 16)) - np.float16(72)) == c - 8
        # The form the GPU kernels use: a nibble in the low mantissa bits with a
        # zero exponent field is the subnormal c * 2^-24 (16c * 2^-24 four bits
        # higher), and one fp16 subtraction of 8 * 2^-24 (128 * 2^-24) gives
        # (c - 8) * 2^-24 (16 (c - 8) * 2^-24) exactly, as a subnormal.
        lo = np.array([c], dtype=np.uint16).view(np.float16)[0]
        hi = np.array([c << 4], dtype=np.uint16).view(np.float16)[0]
        assert float(lo) == c * 2.0**-24 and float(hi) == 16 * c * 2.0**-24
        d_lo = np.float16(lo - np.array([8], dtype=np.uint16).view(np.float16)[0])
        d_hi = np.float16(hi - np.array([128], dtype=np.uint16).view(np.float16)[0])
        assert float(d_lo) == (c - 8) * 2.0**-24
        assert float(d_hi) == 16 * (c - 8) * 2.0**-24
        # and the product with any fp16 x is exact in fp32 (at most 4 + 11 bits)
        for xb in (0x0001, 0x03FF, 0x3C00, 0x7BFF, 0xB555):
            x = np.array([xb], dtype=np.uint16).view(np.float16)[0]
            prod = np.float32(d_lo) * np.float32(x)
            assert float(prod) == (c - 8) * 2.0**-24 * float(x)


# --- matrix-vector product --------------------------------------------------

@pytest.mark.parametrize("N", [1, 7, 33, 65, 97])
@pytest.mark.parametrize("K", [32, 64, 96, 704])
@pytest.mark.parametrize("dt", [F16, BF16])
def test_gemv_matches_brute_force(N, K, dt):
    rng = np.random.default_rng(N * 1000 + K + dt)
    codes, steps = synth.w4_matrix(rng, N, K)
    x = synth.activations(rng, K, dt)
    y, a = oracle.gemv(codes, steps, N, K, x, dt)
    yb, ab = brute.gemv(codes, steps, K, x, dt)
    assert np.allclose(a, ab, rtol=1e-13, atol=0)
    assert np.all(np.abs(y - yb) <= 1e-13 * ab)


@pytest.mark.parametrize("N,K", [(1, 32), (33, 96), (65, 704)])
def test_gemv_on_exact_input_matches_brute_force(N, K):
    """The product on an fp64 input vector (the decode chain's u / r): against
    the dense dequantised matrix times that vector, and a sampled row range."""
    rng = np.random.default_rng(N * 7 + K)
    codes, steps = synth.w4_matrix(rng, N, K)
    x = rng.standard_normal(K) * 3.7
    y, a = oracle.gemv_x64(codes, steps, N, K, x)
    W = brute.dense(codes, steps, K)
    assert np.all(np.abs(y - W @ x) <= 1e-13 * (np.abs(W) @ np.abs(x)))
    assert np.allclose(a, np.abs(W) @ np.abs(x), rtol=1e-13, atol=0)
    y2, a2 = oracle.gemv_x64(codes, steps, N, K, x, rows=(N // 2, N))
    assert np.array_equal(y2, y[N // 2:]) and np.array_equal(a2, a[N // 2:])


def test_gemv_closed_forms():
    K, N = 256, 3
    ones = np.full(K, 0x3C00, dtype=np.uint16)           # fp16 1.0
    step1 = np.full((N, K // 32), 0x3F80, dtype=np.uint16)  # bf16 1.0
    for word, val in [(0xFFFFFFFF, 7), (0x00000000, -8), (0x88888888, 0)]:
        codes = np.full((N, K // 8), word, dtype=np.uint32)
        y, a = oracle.gemv(codes, step1, N, K, ones, F16)
        assert np.all(y == val * K)
        assert np.all(a == abs(val) * K)
    # nibble-alternating word 0x7F7F7F7F: columns alternate 15, 7 -> +7, -1
    codes = np.full((N, K // 8), 0x7F7F7F7F, dtype=np.uint32)
    x = np.zeros(K, dtype=np.uint16)
    x[0::2] = 0x3C00   # +1 on even columns (code 15 -> +7)
    x[1::2] = 0xC000   # -2 on odd columns (code 7 -> -1)
    y, _ = oracle.gemv(codes, step1, N, K, x, F16)
    assert np.all(y == (7 * 1 + (-1) * (-2)) * K / 2)


def test_gemv_one_hot_is_a_single_weight():
    rng = np.random.default_rng(7)
    N, K = 9, 96
    codes, steps = synth.w4_matrix(rng, N, K)
    W = brute.dense(codes, steps, K)
    for k, xb in [(0, 0x3C00), (37, 0x0001), (95, 0xB555)]:   # 1.0, smallest subnormal, -0.333
        x = np.zeros(K, dtype=np.uint16)
        x[k] = xb
        y, _ = oracle.gemv(codes, steps, N, K, x, F16)
        xv = np.array([xb], dtype=np.uint16).view(np.float16).astype(np.float64)[0]
        assert np.array_equal(y, W[:, k] * xv)


def test_gemv_group_step_index():
    # Only group g has a nonzero step: y must equal that group's partial sum.
    rng = np.random.default_rng(8)
    N, K = 4, 128
    codes, _ = synth.w4_matrix(rng, N, K)
    x = synth.activations(rng, K, BF16)
    c = brute.unpack_codes(codes, K).astype(np.float64) - 8
    xv = brute.bf16_bits_to_f64(x)
    for g in range(K // 32):
        steps = np.zeros((N, K // 32), dtype=np.uint16)
        steps[:, g] = 0x4000  # 2.0
        y, _ = oracle.gemv(codes, steps, N, K, x, BF16)
        ref = 2.0 * (c[:, g * 32:(g + 1) * 32] @ xv[g * 32:(g + 1) * 32])
        assert np.allclose(y, ref, rtol=1e-14, atol=1e-14)


def test_gemm_rows_and_leading_dimension():
    rng = np.random.default_rng(9)
    N, K, M, ldx = 33, 96, 3, 128
    codes, steps = synth.w4_matrix(rng, N, K)
    X = synth.activations(rng, (M, ldx), BF16)
    Y, A = oracle.gemm(codes, steps, N, K, X, BF16, M, ldx)
    W = brute.dense(codes, steps, K)
    Xf = brute.bf16_bits_to_f64(X[:, :K])
    assert np.all(np.abs(Y - Xf @ W.T) <= 1e-13 * A)
    assert np.allclose(A, np.abs(Xf) @ np.abs(W).T, rtol=1e-13)


# --- gather -----------------------------------------------------------------

def test_gather_golden_ties():
    rows = []
    with open(os.path.join(GOLDEN, "gather_ties.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, s, e = line.split()
                rows.append((int(c), int(s, 16), int(e, 16)))
    K = 32
    for c, s, e in rows:
        codes = np.full((1, K // 8), 0x11111111 * c, dtype=np.uint32)
        steps = np.full((1, 1), s, dtype=np.uint16)
        out, bad = oracle.gather(codes, steps, 1, K, np.array([0], dtype=np.int32))
        assert bad == 0
        assert np.all(out == e), (c, hex(s), hex(out[0, 0]), hex(e))


def test_gather_matches_torch_rounding_of_exact_products():
    rng = np.random.default_rng(10)
    V, K = 50, 704
    codes, steps = synth.w4_matrix(rng, V, K)
    ids = np.array([0, 49, 7, 7, 23], dtype=np.int32)
    out, bad = oracle.gather(codes, steps, V, K, ids)
    assert bad == 0
    W = brute.dense(codes, steps, K)[ids].astype(np.float32)   # exact in fp32
    ref = torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)
    # every (code, step) pair over a range of bf16 steps, including ties
    sb = np.arange(0x3800, 0x4000, 7, dtype=np.uint16)
    for c in range(16):
        codes1 = np.full((sb.size, 4), 0x11111111 * c, dtype=np.uint32)
        steps1 = sb.reshape(-1, 1)
        o, _ = oracle.gather(codes1, steps1, sb.size, 32, np.arange(sb.size, dtype=np.int32))
        p = ((c - 8) * brute.bf16_bits_to_f64(sb)).astype(np.float32)
        r = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(o[:, 0], r)


def test_gather_reports_bad_ids():
    rng = np.random.default_rng(11)
    codes, steps = synth.w4_matrix(rng, 4, 32)
    _, bad = oracle.gather(codes, steps, 4, 32, np.array([0, 4, -1, 3], dtype=np.int32))
    assert bad == 2


# --- expert-indexed product --------------------------------------------------

def _experts(rng, E, N, K):
    codes, steps = synth.w4_matrix(rng, E * N, K)
    return codes.reshape(E, N, K // 8), steps.reshape(E, N, K // 32)


def test_moe_direct_matches_per_expert_brute_force():
    rng = np.random.default_rng(12)
    E, N, K, T, topk = 6, 9, 64, 2, 3
    codes, steps = _experts(rng, E, N, K)
    ids = np.array([[4, 0, 2], [1, 4, 5]], dtype=np.int32)
    X = synth.activations(rng, (T, K), BF16)
    Y, A = oracle.moe(codes, steps, N * K // 8, N * K // 32, N, K, X, BF16, 0, ids, topk,
                      n_experts=E)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            yb, ab = brute.gemv(codes[e], steps[e], K, X[t], BF16)
            assert np.all(np.abs(Y[t * topk + j] - yb) <= 1e-13 * ab)


def test_moe_per_pair_inputs_match_brute_force():
    rng = np.random.default_rng(18)
    E, N, K, T, topk, ldx = 5, 7, 96, 2, 3, 128
    codes, steps = _experts(rng, E, N, K)
    ids = np.array([[3, 1, 0], [0, 2, 4]], dtype=np.int32)
    X = synth.activations(rng, (T * topk, ldx), F16)
    Y, A = oracle.moe(codes, steps, N * K // 8, N * K // 32, N, K, X, F16, 1, ids, topk,
                      n_experts=E, ldx=ldx)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            yb, ab = brute.gemv(codes[e], steps[e], K, X[t * topk + j, :K], F16)
            assert np.all(np.abs(Y[t * topk + j] - yb) <= 1e-13 * ab)


def test_moe_pool_addressing_is_bitwise_identical_to_direct():
    # anyesh.me page, "Streaming without touching a single GPU kernel": reading a
    # pool through slot ids must give exactly the bytes of the full tensor.
    rng = np.random.default_rng(13)
    E, N, K, T, topk, S = 24, 11, 96, 4, 4, 16
    codes, steps = _experts(rng, E, N, K)
    ids, route = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    pool_c = np.zeros((S, N, K // 8), dtype=np.uint32)
    pool_s = np.zeros((S, N, K // 32), dtype=np.uint16)
    pool_c[slot_of[used]] = codes[used]
    pool_s[slot_of[used]] = steps[used]
    X = synth.activations(rng, (T * topk, K), BF16)
    scale = rng.uniform(0.5, 1.5, size=(E, N)).astype(np.float32)
    sc, ss = N * K // 8, N * K // 32
    for rw in (None, route):
        kw = dict(n_experts=E, row_scale=scale, route_w=rw)
        Yd, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 1, ids, topk, **kw)
        Yp, _ = oracle.moe(pool_c, pool_s, sc, ss, N, K, X, BF16, 1, ids, topk,
                           slot_of=slot_of, n_slots=S, **kw)
        assert Yd.tobytes() == Yp.tobytes()


def test_moe_side_input_needs_real_ids():
    # Feeding slot ids to a per-expert side input (the "quietly stupider" mistake)
    # must change the result.
    rng = np.random.default_rng(14)
    E, N, K, T, topk, S = 16, 8, 64, 1, 4, 8
    codes, steps = _experts(rng, E, N, K)
    ids, _ = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    X = synth.activations(rng, (T, K), BF16)
    scale = rng.uniform(0.5, 1.5, size=(E, N)).astype(np.float32)
    sc, ss = N * K // 8, N * K // 32
    Y, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 0, ids, topk, n_experts=E,
                      row_scale=scale)
    # wrong: the scale row of the slot instead of the expert
    wrong = np.empty_like(scale)
    wrong[used] = scale[slot_of[used]]
    Yw, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 0, ids, topk, n_experts=E,
                       row_scale=wrong)
    assert not np.array_equal(Y, Yw)
    # and the right result is the unscaled product times the real id's scale row
    Y0, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 0, ids, topk, n_experts=E)
    assert np.allclose(Y, Y0 * scale[ids.reshape(-1)], rtol=1e-15, atol=0)


def test_moe_combine_closed_forms():
    rng = np.random.default_rng(15)
    E, N, K, T, topk = 8, 5, 64, 2, 4
    codes, steps = _experts(rng, E, N, K)
    ids, _ = synth.expert_choice(rng, T, E, topk)
    X = synth.activations(rng, (T * topk, K), BF16)
    sc, ss = N * K // 8, N * K // 32
    per, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 1, ids, topk, n_experts=E)
    for j in range(topk):   # a one-hot route picks one choice exactly
        r = np.zeros((T, topk), dtype=np.float32)
        r[:, j] = 1.0
        Y, _ = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 1, ids, topk, n_experts=E,
                          route_w=r)
        for t in range(T):
            assert np.array_equal(Y[t], per[t * topk + j])
    r = rng.uniform(0, 1, size=(T, topk)).astype(np.float32)
    Y, A = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 1, ids, topk, n_experts=E,
                      route_w=r)
    ref = np.einsum("tj,tjn->tn", r.astype(np.float64), per.reshape(T, topk, N))
    assert np.all(np.abs(Y - ref) <= 1e-14 * A)


def test_moe_rejects_out_of_range_ids():
    rng = np.random.default_rng(16)
    codes, steps = _experts(rng, 4, 2, 32)
    X = synth.activations(rng, (1, 32), BF16)
    with pytest.raises(ValueError):
        oracle.moe(codes, steps, 8, 2, 2, 32, X, BF16, 0, np.array([[4]], np.int32), 1,
                   n_experts=4)
    with pytest.raises(ValueError):
        oracle.moe(codes, steps, 8, 2, 2, 32, X, BF16, 0, np.array([[1]], np.int32), 1,
                   n_experts=4, slot_of=np.array([0, -1, 2, 3], np.int32), n_slots=4)


# --- renormalisation between layers ------------------------------------------

@pytest.mark.parametrize("dt", [F16, BF16])
def test_rms_renorm_matches_library_rounding(dt):
    rng = np.random.default_rng(17 + dt)
    v = (rng.normal(0, 3, size=2560)).astype(np.float32)
    K = 1536
    out = oracle.rms_renorm(v, K, dt)
    u = v[:K].astype(np.float64)
    q = u / np.sqrt(np.mean(u * u))
    if dt == F16:
        ref = q.astype(np.float16).view(np.uint16)
        back = ref.view(np.float16).astype(np.float64)
    else:
        # fp64 -> bf16 through fp32 can double-round; check the oracle against the
        # exact nearest value instead: |out - q| is at most half an ulp of bf16
        back = brute.bf16_bits_to_f64(out)
        ulp = 2.0 ** (np.floor(np.log2(np.abs(q))) - 7)
        assert np.all(np.abs(back - q) <= 0.5 * ulp)
        ref = out
    assert np.array_equal(out, ref)
    assert abs(np.mean(back ** 2) - 1.0) < 1e-2


def test_rms_renorm_zero_vector_gives_zeros():
    out = oracle.rms_renorm(np.zeros(64, np.float32), 64, F16)
    assert np.all(out == 0)


# --- the metric arithmetic the pages print -----------------------------------

def test_gbps_formula_reproduces_the_pages_figures():
    from bench import gbps
    g = json.load(open(os.path.join(GOLDEN, "metric_p1_step3.json")))
    nbytes = g["bytes_per_token_MiB"] * 2**20
    # v5 forward: 1222.8 MiB in 9.12 ms is 140.6 GB/s
    assert round(gbps(nbytes, g["v5"]["ms_per_token"] * 1e-3), 1) == g["v5"]["GBps_effective"]
    # both rows backward: the time implied by the printed GB/s rounds to the
    # printed ms at the precision the page prints it (9.3 and 9.12)
    for v in ("v4", "v5"):
        ms_txt = repr(g[v]["ms_per_token"])
        decimals = len(ms_txt.split(".")[1])
        implied_ms = nbytes / (g[v]["GBps_effective"] * 1e9) * 1e3
        assert round(implied_ms, decimals) == g[v]["ms_per_token"]
    # decimal megabytes would not reproduce the page's figure
    assert round(gbps(g["bytes_per_token_MiB"] * 1e6, 9.12e-3), 1) != g["v5"]["GBps_effective"]
    frac = g["v5"]["GBps_effective"] / g["plain_sum_read_GBps"]
    assert round(100 * frac) == g["v5_fraction_of_plain_read_percent"]


# --- grid packing of a 16-bit table ----------------------------------------------

def _pack_words(c):
    """codes [N, K] in 0..15 -> packed uint32 words [N, K/8] (nibble j = column 8w+j)."""
    N, K = c.shape
    codes = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        codes |= (c[:, j::8].astype(np.uint32) << np.uint32(4 * j))
    return codes


def _grid_table(rng, N, K):
    """Codes and 5-bit-significand positive bf16 steps (so every (c - 8) * step
    is exact in bf16), with each group holding code 0 or 15 at a random place
    (and, for the second kind, no code 0) and codes 7 and 8 next to each other
    (so the group's levels share no common factor: its own grid is the
    coarsest one); the table is the oracle's exact dequantisation rounded
    (exactly) to bf16."""
    G = K // 32
    c = rng.integers(0, 16, size=(N, K), dtype=np.int64)
    use15 = rng.random((N, G)) < 0.5
    for n in range(N):
        for g in range(G):
            grp = c[n, 32 * g:32 * g + 32]
            if use15[n, g]:
                grp[grp == 0] = 1
                p = rng.permutation(32)[:3]
                grp[p] = (15, 7, 8)
            else:
                p = rng.permutation(32)[:3]
                grp[p] = (0, 7, 8)
    codes = _pack_words(c)
    exp = rng.integers(100, 140, size=(N, G), dtype=np.uint16)
    mant = (rng.integers(0, 16, size=(N, G), dtype=np.uint16) << 3)
    steps = ((exp << 7) | mant).astype(np.uint16)         # positive, low 3 mantissa bits zero
    W = oracle.dequant(codes, steps, N, K)
    table = np.array([oracle.f64_to_bf16(v) for v in W.ravel()], dtype=np.uint16).reshape(N, K)
    assert np.array_equal(oracle.act_to_f64(table.ravel(), BF16).reshape(N, K), W)  # exact grid
    return codes, steps, table


def _sparse_grid_table(rng, N, K):
    """Exact grid groups that use a random subset of levels -- often without
    code 0 or 15, sometimes only even levels or only a few -- plus a few
    all-positive and all-negative groups.  Returns the table bits."""
    G = K // 32
    c = np.zeros((N, K), dtype=np.int64)
    for n in range(N):
        for g in range(G):
            kind = rng.integers(0, 5)
            if kind == 0:
                levels = rng.choice(np.arange(-5, 6), size=rng.integers(2, 6), replace=False)
            elif kind == 1:
                levels = 2 * rng.choice(np.arange(-4, 4), size=rng.integers(2, 5), replace=False)
            elif kind == 2:
                levels = np.array([0, 2, 5]) * rng.choice([-1, 1])
            elif kind == 3:
                levels = rng.choice(np.arange(1, 8), size=rng.integers(1, 4), replace=False)
            else:
                levels = -rng.choice(np.arange(1, 9), size=rng.integers(1, 4), replace=False)
            c[n, 32 * g:32 * g + 32] = rng.choice(levels, size=32) + 8
    codes = _pack_words(c)
    exp = rng.integers(100, 140, size=(N, G), dtype=np.uint16)
    steps = ((exp << 7) | (rng.integers(0, 16, size=(N, G), dtype=np.uint16) << 3)).astype(np.uint16)
    W = oracle.dequant(codes, steps, N, K)
    table = np.array([oracle.f64_to_bf16(v) for v in W.ravel()], dtype=np.uint16).reshape(N, K)
    assert np.array_equal(oracle.act_to_f64(table.ravel(), BF16).reshape(N, K), W)
    return table


def _coarsest_grid_step(vals):
    """The largest s = a bf16 value > 0 with every value m * s, m an integer in
    [-8, 7], by exact rational arithmetic over every candidate the group's
    extremes allow (None if there is none)."""
    from fractions import Fraction
    fv = [Fraction(float(v)) for v in vals]
    neg = [-v for v in fv if v < 0]
    pos = [v for v in fv if v > 0]
    cands = set()
    if neg:
        cands |= {max(neg) / j for j in range(1, 9)}
    if pos:
        cands |= {max(pos) / i for i in range(1, 8)}
    best = None
    for s in cands:
        if float(s) == 0.0 or Fraction(oracle.bf16_to_f64(oracle.f64_to_bf16(float(s)))) != s:
            continue
        ms = [v / s for v in fv]
        if all(m.denominator == 1 and -8 <= m <= 7 for m in ms):
            best = s if best is None or s > best else best
    return best


def test_grid_packing_round_trips_exact_grids():
    """A table whose groups are exact grid values using code 0 or 15, with two
    neighbouring levels, packs back into exactly the codes and steps it came
    from."""
    rng = np.random.default_rng(31)
    N, K = 9, 96
    codes, steps, table = _grid_table(rng, N, K)
    c2, s2 = oracle.grid_to_codes(table, N, K)
    assert np.array_equal(s2, steps)
    assert np.array_equal(c2, codes)


def test_grid_packing_recovers_grids_without_extreme_codes():
    """Groups whose levels stop short of code 0 or 15 (or use every other level,
    or lie on one side of zero) come back value for value, on the coarsest
    grid that holds them: the step is the largest one an exact rational search
    over the group's candidates finds."""
    rng = np.random.default_rng(33)
    N, K = 12, 256
    table = _sparse_grid_table(rng, N, K)
    codes, steps = oracle.grid_to_codes(table, N, K)
    v = oracle.act_to_f64(table.ravel(), BF16).reshape(N, K)
    W = oracle.dequant(codes, steps, N, K)
    assert np.array_equal(W, v)                                   # every value back exactly
    sf = oracle.act_to_f64(steps.ravel(), BF16).reshape(N, K // 32)
    for n in range(N):
        for g in range(K // 32):
            best = _coarsest_grid_step(v[n, 32 * g:32 * g + 32])
            assert best is not None and float(best) == sf[n, g], (n, g)


def test_grid_packing_golden_ties():
    """Half-step values on an exact division (tests/golden/grid_ties.txt, each
    case derived with exact rationals) take the even code, also where the
    fp32 product with the step's reciprocal lands on the other side."""
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "grid_ties.txt")):
        if line.startswith("#") or not line.strip():
            continue
        vb, sb, _, code = line.split()
        rows.append((int(vb, 16), int(sb, 16), int(code)))
    assert len(rows) >= 10
    # one group per case: -8 steps (the negative extreme sets the step; no
    # coarser grid holds the half-step value), the value, zeros elsewhere
    t = np.zeros((len(rows), 32), dtype=np.uint16)
    for i, (vb, sb, _) in enumerate(rows):
        t[i, 0] = oracle.f64_to_bf16(-8.0 * oracle.bf16_to_f64(sb))
        t[i, 5] = vb
    codes, steps = oracle.grid_to_codes(t, len(rows), 32)
    for i, (vb, sb, code) in enumerate(rows):
        assert int(steps[i, 0]) == sb
        assert oracle.code(codes, 32, i, 5) == code, (hex(vb), hex(sb))
        assert oracle.code(codes, 32, i, 0) == 0


def test_grid_packing_closed_forms():
    # all zeros: step 0 and code 8 everywhere
    c, s = oracle.grid_to_codes(np.zeros((1, 32), dtype=np.uint16), 1, 32)
    assert s[0, 0] == 0 and np.all(c == 0x88888888)
    # +a and -a alone: the coarsest grid is a itself, levels -1 and +1
    a = 7 * 0.125
    t = np.zeros((1, 32), dtype=np.uint16)
    t[0, 3] = oracle.f64_to_bf16(a)
    t[0, 9] = oracle.f64_to_bf16(-a)
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == a
    assert oracle.code(c, 32, 0, 3) == 9 and oracle.code(c, 32, 0, 9) == 7
    # 0.875 and -1.0: only the grid of 0.125 holds both (levels 7 and -8)
    t[0, 9] = oracle.f64_to_bf16(-1.0)
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == 0.125 and oracle.code(c, 32, 0, 9) == 0
    assert oracle.code(c, 32, 0, 3) == 15   # 0.875 / 0.125 = 7
    # values off every grid: the extreme rule (a larger negative extreme is
    # 8 steps below zero, otherwise the positive extreme is 7 steps above)
    t = np.zeros((1, 32), dtype=np.uint16)
    t[0, 0] = oracle.f64_to_bf16(-1.0)
    t[0, 1] = oracle.f64_to_bf16(0.3)
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == 0.125
    assert oracle.code(c, 32, 0, 1) == 10                   # 0.3 / 0.125 = 2.4
    t[0, 0] = oracle.f64_to_bf16(-0.3)
    t[0, 1] = oracle.f64_to_bf16(1.0)
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == oracle.bf16_to_f64(oracle.f64_to_bf16(1.0 / 7.0))
    assert oracle.code(c, 32, 0, 1) == 15
    # equal extremes off every grid: the positive one is 7 steps up, so both
    # extremes stay inside the range (codes 15 and 1)
    t[0, 0] = oracle.f64_to_bf16(-1.0)
    t[0, 2] = oracle.f64_to_bf16(0.3)
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == oracle.bf16_to_f64(oracle.f64_to_bf16(1.0 / 7.0))
    assert oracle.code(c, 32, 0, 1) == 15 and oracle.code(c, 32, 0, 0) == 1
    # a grid of bf16 subnormals: step 2^-133 * 3, levels -8..7 exact
    sub = 3 * 2.0 ** -133
    t = np.array([[oracle.f64_to_bf16(((k % 16) - 8) * sub) for k in range(32)]], dtype=np.uint16)
    assert all(oracle.bf16_to_f64(int(b)) == ((k % 16) - 8) * sub for k, b in enumerate(t[0]))
    c, s = oracle.grid_to_codes(t, 1, 32)
    assert oracle.bf16_to_f64(int(s[0, 0])) == sub
    assert all(oracle.code(c, 32, 0, k) == k % 16 for k in range(32))


def test_grid_packing_error_bound_on_arbitrary_tables():
    """On values that are not on a grid, each packed value is within half a
    step of the input when it lies inside the grid's range, and within about
    one step when it is the clamped positive extreme of a group whose negative
    extreme sets the step."""
    rng = np.random.default_rng(32)
    N, K = 16, 256
    table = synth.act_bits(rng.standard_normal((N, K)) * 0.05, BF16)
    codes, steps = oracle.grid_to_codes(table, N, K)
    v = oracle.act_to_f64(table.ravel(), BF16).reshape(N, K)
    W = oracle.dequant(codes, steps, N, K)
    sf = np.repeat(oracle.act_to_f64(steps.ravel(), BF16).reshape(N, K // 32), 32, axis=1)
    err = np.abs(W - v)
    inside = (v / sf >= -8.5) & (v / sf <= 7.5)
    assert np.all(err[inside] <= 0.5 * sf[inside])
    assert np.all(err <= 1.05 * sf)


# --- decode attention ---------------------------------------------------------

def _bits(rng, shape, scale=1.0):
    return synth.act_bits(rng.standard_normal(shape) * scale, BF16)


def test_attention_closed_forms():
    rng = np.random.default_rng(71)
    q, k, v = _bits(rng, (8, 64)), _bits(rng, (1, 64)), _bits(rng, (1, 64))
    vv = oracle.act_to_f64(v.ravel(), BF16).reshape(1, 64)
    # one cached position: every head returns its value row exactly
    assert np.array_equal(oracle.decode_attention(q, k, v, 0.125), np.repeat(vv, 8, axis=0))
    # equal keys, or a zero scale: uniform weights, the mean of the values
    k5 = np.repeat(_bits(rng, (1, 64)), 5, axis=0)
    v5 = _bits(rng, (5, 64))
    mean = oracle.act_to_f64(v5.ravel(), BF16).reshape(5, 64).mean(axis=0)
    assert np.allclose(oracle.decode_attention(q, k5, v5, 0.3), mean[None, :], rtol=0, atol=1e-15)
    assert np.allclose(oracle.decode_attention(q, _bits(rng, (5, 64)), v5, 0.0), mean[None, :], rtol=0, atol=1e-15)


def test_attention_dominant_key_and_order():
    rng = np.random.default_rng(72)
    H, D, L = 8, 64, 40
    q = _bits(rng, (H, D))
    k, v = _bits(rng, (L, D)), _bits(rng, (L, D))
    # a key aligned with every head's query, scaled up, takes all the weight
    qq = oracle.act_to_f64(q.ravel(), BF16).reshape(H, D)
    k2 = k.copy()
    k2[7] = synth.act_bits(qq.sum(axis=0) * 64.0, BF16)
    o = oracle.decode_attention(q, k2, v, 1.0)
    v7 = oracle.act_to_f64(v[7], BF16)
    assert np.abs(o - v7[None, :]).max() < 1e-12
    # the order of the cached positions does not matter (a ring's slots)
    perm = rng.permutation(L)
    assert np.allclose(oracle.decode_attention(q, k[perm], v[perm], 0.2),
                       oracle.decode_attention(q, k, v, 0.2), rtol=0, atol=1e-14)
