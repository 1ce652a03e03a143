"""Grid packing of a 16-bit table on the GPU: codes and steps bit-exact against
the CPU oracle, whose codes come from the exact quotient v / step."""

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.test_oracle_pins import _grid_table, _sparse_grid_table

pytestmark = pytest.mark.gpu
BF16 = synth.BF16


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def run_pack(w4, table_bits):
    t = torch.from_numpy(np.ascontiguousarray(table_bits).view(np.int16)).cuda().view(torch.bfloat16)
    codes, steps = w4.w4_grid_to_codes(t)
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32), steps.view(torch.int16).cpu().numpy().view(np.uint16)


def test_grid_packing_recovers_exact_grids(w4):
    rng = np.random.default_rng(61)
    N, K = 33, 160
    codes, steps, table = _grid_table(rng, N, K)
    c2, s2 = run_pack(w4, table)
    assert np.array_equal(s2, steps)
    assert np.array_equal(c2, codes)


def test_grid_packing_sparse_levels_match_oracle(w4):
    """Groups whose levels stop short of code 0 or 15, use every other level or
    one side of zero: the coarsest grid, bit for bit as the oracle."""
    rng = np.random.default_rng(62)
    N, K = 41, 512
    table = _sparse_grid_table(rng, N, K)
    c2, s2 = run_pack(w4, table)
    c1, s1 = oracle.grid_to_codes(table, N, K)
    assert np.array_equal(s2, s1)
    assert np.array_equal(c2, c1)


def test_grid_packing_golden_ties(w4):
    """Half-step values decided by ties to even on the exact quotient, where the
    fp32 product with the reciprocal falls on the other side
    (tests/golden/grid_ties.txt)."""
    rows = []
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "grid_ties.txt")):
        if line.startswith("#") or not line.strip():
            continue
        vb, sb, _, code = line.split()
        rows.append((int(vb, 16), int(sb, 16), int(code)))
    t = np.zeros((len(rows), 64), dtype=np.uint16)
    for i, (vb, sb, _) in enumerate(rows):
        for g in range(2):   # the case at two places of the group
            t[i, 32 * g] = oracle.f64_to_bf16(-8.0 * oracle.bf16_to_f64(sb))
            t[i, 32 * g + 5 + 22 * g] = vb
    codes, steps = run_pack(w4, t)
    for i, (vb, sb, code) in enumerate(rows):
        assert int(steps[i, 0]) == sb and int(steps[i, 1]) == sb
        assert oracle.code(codes, 64, i, 5) == code, (hex(vb), hex(sb))
        assert oracle.code(codes, 64, i, 59) == code, (hex(vb), hex(sb))


@pytest.mark.parametrize("N,K,scale", [(1, 32, 0.05), (257, 1536, 0.05), (70, 8960, 1.0),
                                       (5, 64, 1e-30), (9, 96, 3e30), (6, 64, 1e-38)])
def test_grid_packing_matches_oracle(w4, N, K, scale):
    print(f"grid N={N} K={K} scale={scale}", flush=True)
    rng = np.random.default_rng(N + K)
    table = synth.act_bits(rng.standard_normal((N, K)) * scale, BF16)
    table[0, :32] = 0                                   # an all-zero group
    if K >= 64:
        table[0, 32:64] = table[0, 32:64] & 0x7FFF      # a group with no negative value
    c2, s2 = run_pack(w4, table)
    c1, s1 = oracle.grid_to_codes(table, N, K)
    assert np.array_equal(s2, s1)
    assert np.array_equal(c2, c1)


def test_grid_packing_subnormal_grids(w4):
    """Exact grids of bf16 subnormal steps, and tiny off-grid groups whose
    step rounds into the subnormal range."""
    rng = np.random.default_rng(63)
    N, K = 8, 128
    t = np.zeros((N, K), dtype=np.uint16)
    for n in range(N):
        for g in range(K // 32):
            sub = int(rng.integers(1, 16)) * 2.0 ** -133
            levels = rng.integers(-8, 8, size=32)
            if g == 3:   # off every grid
                t[n, 32 * g:32 * g + 32] = synth.act_bits(rng.standard_normal(32) * 2.0 ** -125, BF16)
            else:
                t[n, 32 * g:32 * g + 32] = [oracle.f64_to_bf16(float(m) * sub) for m in levels]
    c2, s2 = run_pack(w4, t)
    c1, s1 = oracle.grid_to_codes(t, N, K)
    assert np.array_equal(s2, s1)
    assert np.array_equal(c2, c1)


def test_grid_packing_full_vocabulary_table_sampled(w4):
    """262144 x 1536 bf16 table (805 MB, generated on the device), sampled rows
    bit-exact against the oracle."""
    V, K = 262144, 1536
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    t = (torch.randn((V, K), generator=g, device="cuda") * 0.03).to(torch.bfloat16)
    codes, steps = w4.w4_grid_to_codes(t)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 4095, 131072, V - 1], device="cuda")
    sub = t.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)
    c1, s1 = oracle.grid_to_codes(sub, len(rows), K)
    assert np.array_equal(codes.index_select(0, rows).cpu().numpy().view(np.uint32), c1)
    assert np.array_equal(steps.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16), s1)
