"""The expert product's no-allocation entry point (scratch in a fixed array of
the library's device image): bit for bit the output of w4_moe_gemv_ids on the
same inputs, on two calls in a row with the second one smaller, on both of the
product's paths; a call that needs more scratch than the array holds is
refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_codes, dev_steps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def _bits(t):
    return t.contiguous().view(torch.int32).cpu()


def _experts(rng, E, N, K):
    codes, steps = synth.w4_matrix(rng, E * N, K)
    return dev_codes(codes), dev_steps(steps)


def _case(w4, rng, dc, ds, E, N, K, T, topk, x_dtype, x_per_pair, route):
    ids_np, rw_np = synth.expert_choice(rng, T, E, topk)
    ids = torch.from_numpy(ids_np).cuda()
    rw = torch.from_numpy(rw_np).cuda() if route else None
    rows = T * topk if x_per_pair else T
    X = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32) * 3.0).cuda()
    if x_dtype is not torch.float32:
        X = X.to(x_dtype)
    out_rows = T if route else T * topk
    args = (dc, ds, N * K // 8, N * K // 32, N, K, X, ids)
    kw = dict(x_per_pair=x_per_pair, n_experts=E, route_w=rw)
    ref = w4.w4_moe_gemv_ids(*args, **kw)
    Y = torch.full((out_rows, N), float("nan"), device="cuda")
    w4.w4_moe_gemv_ids_noalloc(*args, Y=Y, **kw)
    torch.cuda.synchronize()
    return Y, ref


@pytest.mark.parametrize("path", ["pairs", "engine"])
def test_noalloc_matches_the_workspace_entry_point(w4, path):
    print(f"noalloc expert product, {path} path", flush=True)
    rng = np.random.default_rng(401 if path == "pairs" else 402)
    E, topk = 16, 8
    if path == "pairs":
        # combined route-weighted sum of per-choice rows staged in the scratch
        N, K = 1408, 2816
        dc, ds = _experts(rng, E, N, K)
        sizes = [(4, torch.bfloat16, False), (1, torch.bfloat16, False)]
    else:
        # fp32 rows renormalised into the scratch, then the matrix engine (with
        # K-slices summed through the scratch) and the combined sum
        N, K = 2816, 704
        dc, ds = _experts(rng, E, N, K)
        sizes = [(8, torch.float32, True), (5, torch.float32, True)]
    for T, xdt, xpp in sizes:
        xk = w4.W4_F32_RMS if xdt is torch.float32 else w4.W4_BF16
        need = w4.w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, xk, xpp, True)
        assert 0 < need <= w4.W4_NOALLOC_SCRATCH_BYTES
        Y, ref = _case(w4, rng, dc, ds, E, N, K, T, topk, xdt, xpp, route=True)
        assert torch.equal(_bits(Y), _bits(ref)), (path, T)
    # and a per-choice (uncombined) call after them
    Y, ref = _case(w4, rng, dc, ds, E, N, K, 2, topk, torch.bfloat16, False, route=False)
    assert torch.equal(_bits(Y), _bits(ref))


def test_noalloc_refuses_shapes_beyond_its_scratch(w4):
    rng = np.random.default_rng(403)
    E, N, K, T, topk = 4, 2816, 704, 128, 8
    need = w4.w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, w4.W4_BF16, True, True)
    assert need > w4.W4_NOALLOC_SCRATCH_BYTES
    dc, ds = _experts(rng, E, N, K)
    ids = torch.from_numpy(np.tile(np.arange(topk, dtype=np.int32) % E, (T, 1))).cuda()
    rw = torch.full((T, topk), 0.125, device="cuda")
    X = torch.zeros((T * topk, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((T, N), float("nan"), device="cuda")
    with pytest.raises(w4.W4Error) as e:
        w4.w4_moe_gemv_ids_noalloc(dc, ds, N * K // 8, N * K // 32, N, K, X, ids, x_per_pair=True,
                                   n_experts=E, route_w=rw, Y=Y)
    assert e.value.status == w4.W4_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(Y))
