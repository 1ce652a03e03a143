"""Caller-owned workspaces: calls on two streams, each with its own workspace,
running at the same time, give bitwise the results of the same calls made one
after another; and a workspace is left reusable (its counters back at zero)."""

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


def _two_streams(calls):
    """Runs calls[0] on stream A and calls[1] on stream B, interleaved, and
    returns after both finished."""
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(sa):
            calls[0](sa)
        with torch.cuda.stream(sb):
            calls[1](sb)
    torch.cuda.synchronize()


def test_small_m_split_k_on_two_streams(w4):
    rng = np.random.default_rng(301)
    N, K, M = 1536, 8192, 16
    need = w4.w4_gemm_smallM_workspace_bytes(N, K, M)
    assert need > 0, "this shape is meant to split K through the workspace"
    mats = [synth.w4_matrix(rng, N, K) for _ in range(2)]
    dm = [(dev_codes(c), dev_steps(s)) for c, s in mats]
    X = [torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda().to(torch.bfloat16)
         for _ in range(2)]
    ref = [w4.w4_gemm_smallM(*dm[i], X[i]) for i in range(2)]
    torch.cuda.synchronize()
    ws = [w4.new_workspace(need) for _ in range(2)]
    Y = [torch.full((M, N), float("nan"), device="cuda") for _ in range(2)]
    _two_streams([lambda s, i=i: w4.w4_gemm_smallM(*dm[i], X[i], Y[i], stream=s, workspace=ws[i])
                  for i in range(2)])
    for i in range(2):
        assert torch.equal(_bits(Y[i]), _bits(ref[i]))
        assert int(ws[i][:16384].count_nonzero()) == 0   # counters back at zero


def test_combined_experts_and_attention_on_two_streams(w4):
    rng = np.random.default_rng(302)
    E, N, K, T, topk = 16, 704, 1408, 4, 8
    codes, steps = synth.w4_matrix(rng, E * N, K)
    dc, ds = dev_codes(codes), dev_steps(steps)
    ids = [torch.from_numpy(synth.expert_choice(rng, T, E, topk)[0]).cuda() for _ in range(2)]
    route = [torch.from_numpy(synth.expert_choice(rng, T, E, topk)[1]).cuda() for _ in range(2)]
    X = [torch.from_numpy(rng.standard_normal((T, K)).astype(np.float32)).cuda().to(torch.bfloat16)
         for _ in range(2)]

    def moe(i, Y=None, s=None, ws=None):
        return w4.w4_moe_gemv_ids(dc, ds, N * K // 8, N * K // 32, N, K, X[i], ids[i], n_experts=E,
                                  route_w=route[i], Y=Y, stream=s, workspace=ws)
    need = w4.w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, w4.W4_BF16, False, True)
    assert need > 0
    ref = [moe(i) for i in range(2)]
    H, D, L = 8, 512, 3000
    q = [torch.randn((H, D), device="cuda").to(torch.bfloat16) for _ in range(2)]
    kv = [torch.randn((L, D), device="cuda").to(torch.bfloat16) for _ in range(2)]
    aref = [w4.w4_decode_attention(q[i], kv[i], kv[1 - i], 0.05) for i in range(2)]
    torch.cuda.synchronize()
    wsm = [w4.new_workspace(need) for _ in range(2)]
    wsa = [w4.new_workspace(w4.w4_decode_attention_workspace_bytes(H, D, L)) for _ in range(2)]
    Y = [torch.full((T, N), float("nan"), device="cuda") for _ in range(2)]
    O = [torch.full((H, D), float("nan"), device="cuda") for _ in range(2)]

    def both(i, s):
        moe(i, Y[i], s, wsm[i])
        w4.w4_decode_attention(q[i], kv[i], kv[1 - i], 0.05, O[i], stream=s, workspace=wsa[i])
    _two_streams([lambda s, i=i: both(i, s) for i in range(2)])
    for i in range(2):
        assert torch.equal(_bits(Y[i]), _bits(ref[i]))
        assert torch.equal(_bits(O[i]), _bits(aref[i]))


def test_prompt_chunk_on_two_streams(w4):
    rng = np.random.default_rng(303)
    N, K, M = 3072, 1536, 256
    mats = [synth.w4_matrix(rng, N, K) for _ in range(2)]
    dm = [(dev_codes(c), dev_steps(s)) for c, s in mats]
    X = [torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda().to(torch.float16)
         for _ in range(2)]
    ref = [w4.w4_gemm_prompt(*dm[i], X[i]) for i in range(2)]
    torch.cuda.synchronize()
    need = w4.w4_gemm_prompt_workspace_bytes(N, K, M)
    ws = [w4.new_workspace(need) for _ in range(2)]
    Y = [torch.full((M, N), float("nan"), device="cuda") for _ in range(2)]
    _two_streams([lambda s, i=i: w4.w4_gemm_prompt(*dm[i], X[i], Y[i], stream=s, workspace=ws[i])
                  for i in range(2)])
    for i in range(2):
        assert torch.equal(_bits(Y[i]), _bits(ref[i]))


def test_missing_or_short_workspace_is_refused(w4):
    rng = np.random.default_rng(304)
    N, K, M = 1536, 8192, 16
    codes, steps = synth.w4_matrix(rng, N, K)
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    Y = torch.full((M, N), float("nan"), device="cuda")
    need = w4.w4_gemm_smallM_workspace_bytes(N, K, M)
    short = w4.new_workspace(need - 256)
    with pytest.raises(w4.W4Error) as e:
        w4.w4_gemm_smallM(dev_codes(codes), dev_steps(steps), X, Y, workspace=short)
    assert e.value.status == w4.W4_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(Y))


def test_one_workspace_shared_by_every_entry_point(w4):
    """One workspace, sized for the largest need, serves the prompt chunk, the
    attention and then a split-K small-M product on one stream: the counters
    at its start stay zero whatever the other calls staged after them."""
    rng = np.random.default_rng(305)
    N, K, M = 1536, 8192, 16
    codes, steps = synth.w4_matrix(rng, N, K)
    dc, ds = dev_codes(codes), dev_steps(steps)
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).cuda().to(torch.bfloat16)
    ref = w4.w4_gemm_smallM(dc, ds, X, workspace=w4.new_workspace(w4.w4_gemm_smallM_workspace_bytes(N, K, M)))
    Xp = torch.from_numpy(rng.standard_normal((64, K)).astype(np.float32)).cuda().to(torch.bfloat16)
    q = torch.randn((8, 512), device="cuda").to(torch.bfloat16)
    kv = torch.randn((4096, 512), device="cuda").to(torch.bfloat16)
    need = max(w4.w4_gemm_smallM_workspace_bytes(N, K, M), w4.w4_gemm_prompt_workspace_bytes(N, K, 64),
               w4.w4_decode_attention_workspace_bytes(8, 512, 4096))
    ws = w4.new_workspace(need)
    w4.w4_gemm_prompt(dc, ds, Xp, workspace=ws)
    w4.w4_decode_attention(q, kv, kv, 0.05, workspace=ws)
    Y = w4.w4_gemm_smallM(dc, ds, X, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(Y), _bits(ref))
