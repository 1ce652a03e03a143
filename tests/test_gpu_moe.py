"""Expert-indexed W4A16 product on the GPU: parity with the oracle, bitwise
identity of slot-pool and direct addressing, and the error path."""

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


def experts(rng, E, N, K):
    codes, steps = synth.w4_matrix(rng, E * N, K)
    return codes.reshape(E, N, K // 8), steps.reshape(E, N, K // 32)


def run(w4, codes, steps, N, K, X, dt, ids, x_per_pair, slot_of=None, n_slots=0, scale=None,
        route=None, n_experts=None, err=None):
    T, topk = ids.shape
    rows = T * topk if route is None else T
    Y = torch.full((rows, N), float("nan"), dtype=torch.float32, device="cuda")
    w4.w4_moe_gemv_ids(dev_codes(codes.reshape(-1, K // 8)), dev_steps(steps.reshape(-1, K // 32)),
                       N * K // 8, N * K // 32, N, K, dev_act(X, dt),
                       torch.from_numpy(ids.astype(np.int32)).cuda(), x_per_pair=x_per_pair,
                       slot_of=None if slot_of is None else torch.from_numpy(slot_of).cuda(),
                       n_experts=n_experts if n_experts is not None else codes.shape[0],
                       n_slots=n_slots,
                       row_scale=None if scale is None else torch.from_numpy(scale).cuda(),
                       route_w=None if route is None else torch.from_numpy(route).cuda(),
                       Y=Y, dev_err=err)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def pool_of(codes, steps, slot_of, used, S):
    pc = np.zeros((S,) + codes.shape[1:], dtype=codes.dtype)
    ps = np.zeros((S,) + steps.shape[1:], dtype=steps.dtype)
    pc[slot_of[used]] = codes[used]
    ps[slot_of[used]] = steps[used]
    return pc, ps


@pytest.mark.parametrize("T,topk,xpp,dt", [(1, 8, 0, BF16), (4, 8, 0, BF16), (4, 8, 1, F16),
                                           (3, 3, 1, BF16), (1, 1, 0, F16), (5, 4, 0, F16)])
def test_moe_small_vs_oracle_and_pool_identity(w4, T, topk, xpp, dt):
    print(f"moe T={T} topk={topk} xpp={xpp} dt={dt}", flush=True)
    rng = np.random.default_rng(T * 100 + topk * 10 + xpp + dt)
    E, N, K, S = 24, 33, 96, 24
    codes, steps = experts(rng, E, N, K)
    ids, route = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    pc, ps = pool_of(codes, steps, slot_of, used, S)
    X = synth.activations(rng, (T * topk if xpp else T, K), dt)
    scale = rng.uniform(0.5, 1.5, size=(E, N)).astype(np.float32)
    sc, ss = N * K // 8, N * K // 32
    for rw in (None, route):
        Yd = run(w4, codes, steps, N, K, X, dt, ids, xpp, scale=scale, route=rw)
        Yp = run(w4, pc, ps, N, K, X, dt, ids, xpp, slot_of=slot_of, n_slots=S, scale=scale,
                 route=rw, n_experts=E)
        assert Yd.tobytes() == Yp.tobytes()     # same bytes, different addressing
        Yo, Ao = oracle.moe(codes, steps, sc, ss, N, K, X, dt, xpp, ids, topk, n_experts=E,
                            row_scale=scale, route_w=rw)
        ok, worst = within_bound(Yd, Yo, Ao)
        assert ok, worst


def test_moe_few_tokens_on_the_matrix_engine(w4, w4_settings):
    """Four tokens forced onto the matrix engine (the path of larger batches):
    the same parity and pool identity as the default matrix-vector path."""
    w4_settings("W4_MOE_PAIRS_MAX_T", "0")
    test_moe_small_vs_oracle_and_pool_identity(w4, 4, 8, 1, F16)
    test_moe_small_vs_oracle_and_pool_identity(w4, 1, 8, 0, BF16)


@pytest.mark.parametrize("dt", [F16, BF16])
def test_moe_long_rows_summed_over_k_slices(w4, dt):
    """K = 3200 (100 groups) on the matrix engine (five tokens) is split into
    two K-slices whose partial rows are added in order by the finishing pass;
    also with a bad id (NaN rows)."""
    print(f"moe k-slices dt={dt}", flush=True)
    rng = np.random.default_rng(40 + dt)
    E, N, K, S, T, topk = 12, 70, 3200, 12, 5, 4
    codes, steps = experts(rng, E, N, K)
    ids, route = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    pc, ps = pool_of(codes, steps, slot_of, used, S)
    X = synth.activations(rng, (T, K), dt)
    scale = rng.uniform(0.5, 1.5, size=(E, N)).astype(np.float32)
    for rw in (None, route):
        Yd = run(w4, codes, steps, N, K, X, dt, ids, 0, scale=scale, route=rw)
        Yp = run(w4, pc, ps, N, K, X, dt, ids, 0, slot_of=slot_of, n_slots=S, scale=scale,
                 route=rw, n_experts=E)
        assert Yd.tobytes() == Yp.tobytes()
        Yo, Ao = oracle.moe(codes, steps, N * K // 8, N * K // 32, N, K, X, dt, 0, ids, topk,
                            n_experts=E, row_scale=scale, route_w=rw)
        ok, worst = within_bound(Yd, Yo, Ao)
        assert ok, worst
    bad = ids.copy()
    bad[1, 2] = E + 3
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = run(w4, codes, steps, N, K, X, dt, bad, 0, scale=scale, err=err)
    assert err.item() == 1
    assert np.all(np.isnan(Y[1 * topk + 2]))
    assert not np.any(np.isnan(np.delete(Y, 1 * topk + 2, axis=0)))


def test_moe_side_input_follows_real_ids_under_pool_addressing(w4):
    """Only the weight read goes through slot_of: a per-expert side input read
    at the slot id instead of the real id would change the result."""
    rng = np.random.default_rng(41)
    E, N, K, S, T, topk = 16, 48, 256, 16, 2, 4
    codes, steps = experts(rng, E, N, K)
    ids, _ = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    pc, ps = pool_of(codes, steps, slot_of, used, S)
    X = synth.activations(rng, (T, K), BF16)
    scale = rng.uniform(0.5, 1.5, size=(E, N)).astype(np.float32)
    Yp = run(w4, pc, ps, N, K, X, BF16, ids, 0, slot_of=slot_of, n_slots=S, scale=scale,
             n_experts=E)
    sc, ss = N * K // 8, N * K // 32
    Yo, Ao = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 0, ids, topk, n_experts=E,
                        row_scale=scale)
    assert within_bound(Yp, Yo, Ao)[0]
    # the wrong reading: side input indexed by slot id
    wrong = np.zeros_like(scale)
    for e in used:
        wrong[e] = scale[slot_of[e]]
    assert np.any(slot_of[used] != used)
    Yw, Aw = oracle.moe(codes, steps, sc, ss, N, K, X, BF16, 0, ids, topk, n_experts=E,
                        row_scale=wrong)
    assert not within_bound(Yp, Yw, Aw)[0]


def test_moe_bad_id_and_missing_slot_give_nan_and_flag(w4):
    rng = np.random.default_rng(5)
    E, N, K = 8, 20, 64
    codes, steps = experts(rng, E, N, K)
    X = synth.activations(rng, (2, K), BF16)
    ids = np.array([[0, 9], [3, 2]], dtype=np.int32)          # 9 is out of range
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = run(w4, codes, steps, N, K, X, BF16, ids, 0, err=err)
    assert err.item() == 1
    assert np.all(np.isnan(Y[1])) and not np.any(np.isnan(Y[[0, 2, 3]]))
    slot_of = np.array([0, 1, -1, 3, 4, 5, 6, 7], dtype=np.int32)   # expert 2 not resident
    err.zero_()
    ids2 = np.array([[0, 1], [3, 2]], dtype=np.int32)
    Y = run(w4, codes, steps, N, K, X, BF16, ids2, 0, slot_of=slot_of, n_slots=8, err=err)
    assert err.item() == 1
    assert np.all(np.isnan(Y[3])) and not np.any(np.isnan(Y[[0, 1, 2]]))


def test_moe_single_token_bad_id_and_missing_slot(w4):
    """One token runs as side-by-side matrix-vector products: a bad id or a
    missing slot still gives NaN rows (and the route-weighted row) and the flag."""
    rng = np.random.default_rng(8)
    E, N, K = 8, 300, 512
    codes, steps = experts(rng, E, N, K)
    X = synth.activations(rng, (1, K), BF16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = np.array([[0, 9, 2]], dtype=np.int32)                # 9 is out of range
    Y = run(w4, codes, steps, N, K, X, BF16, ids, 0, err=err)
    assert err.item() == 1
    assert np.all(np.isnan(Y[1])) and not np.any(np.isnan(Y[[0, 2]]))
    err.zero_()
    route = np.array([[0.5, 0.25, 0.25]], dtype=np.float32)
    Y = run(w4, codes, steps, N, K, X, BF16, ids, 0, route=route, err=err)
    assert err.item() == 1 and np.all(np.isnan(Y))
    slot_of = np.array([0, 1, -1, 3, 4, 5, 6, 7], dtype=np.int32)   # expert 2 not resident
    err.zero_()
    ids2 = np.array([[0, 1, 2]], dtype=np.int32)
    Y = run(w4, codes, steps, N, K, X, BF16, ids2, 0, slot_of=slot_of, n_slots=8, err=err)
    assert err.item() == 1
    assert np.all(np.isnan(Y[2])) and not np.any(np.isnan(Y[[0, 1]]))


@pytest.mark.parametrize("T,xpp,K", [(1, 0, 704), (1, 1, 704), (3, 1, 704), (5, 0, 704), (5, 1, 704),
                                     (1, 0, 2816), (2, 1, 2816), (1, 0, 8192)])
def test_moe_fp32_rows_renormalised_on_load(w4, T, xpp, K):
    """fp32 activation rows renormalised as part of the product give the bits
    of w4_rms_renorm (fp16) followed by the product, with and without route
    weights, on both paths (up to four tokens fused; from five the rows are
    renormalised into the library's buffer first)."""
    rng = np.random.default_rng(60 + T * 2 + xpp + K)
    E, N, topk, ld = 16, 200, 4, K + 64
    codes, steps = experts(rng, E, N, K)
    ids, route = synth.expert_choice(rng, T, E, topk)
    rows = T * topk if xpp else T
    X32 = torch.from_numpy((rng.normal(0, 3, size=(rows, ld))).astype(np.float32)).cuda()
    Xh = w4.w4_rms_renorm(X32, K, out_dtype=torch.float16)
    dc, ds = dev_codes(codes.reshape(-1, K // 8)), dev_steps(steps.reshape(-1, K // 32))
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    for rw in (None, torch.from_numpy(route).cuda()):
        out = []
        for X in (X32, Xh):
            Y = torch.full((T * topk if rw is None else T, N), float("nan"), device="cuda")
            w4.w4_moe_gemv_ids(dc, ds, N * K // 8, N * K // 32, N, K, X, dids, x_per_pair=bool(xpp),
                               n_experts=E, route_w=rw, Y=Y)
            out.append(Y)
        torch.cuda.synchronize()
        assert torch.equal(out[0].view(torch.int32), out[1].view(torch.int32)), (T, xpp, rw is None)
    # and the product itself against the oracle on the renormalised rows
    Xo = Xh.view(torch.int16).cpu().numpy().view(np.uint16)
    Yo, Ao = oracle.moe(codes, steps, N * K // 8, N * K // 32, N, K, Xo, F16, xpp, ids, topk, n_experts=E)
    Y = torch.empty((T * topk, N), device="cuda")
    w4.w4_moe_gemv_ids(dc, ds, N * K // 8, N * K // 32, N, K, X32, dids, x_per_pair=bool(xpp),
                       n_experts=E, Y=Y)
    torch.cuda.synchronize()
    ok, worst = within_bound(Y.cpu().numpy(), Yo, Ao)
    assert ok, worst


@pytest.mark.parametrize("T,K", [(1, 2816), (4, 704), (6, 704)])
def test_moe_rows_not_16_byte_aligned(w4, T, K):
    """Activation rows at an odd row stride (fp32 rows renormalised on load,
    and bf16 rows) are read without vector loads or direct-to-LDS copies: the
    bits of the same rows at an aligned stride, on both paths."""
    print(f"moe unaligned rows T={T} K={K}", flush=True)
    rng = np.random.default_rng(90 + T + K)
    E, N, topk = 12, 160, 4
    codes, steps = experts(rng, E, N, K)
    ids, route = synth.expert_choice(rng, T, E, topk)
    dc, ds = dev_codes(codes.reshape(-1, K // 8)), dev_steps(steps.reshape(-1, K // 32))
    dids = torch.from_numpy(ids.astype(np.int32)).cuda()
    X32 = torch.from_numpy(rng.normal(0, 2, size=(T, K)).astype(np.float32)).cuda()
    Xb = dev_act(synth.activations(rng, (T, K), BF16), BF16)
    for X in (X32, Xb):
        big = torch.zeros((T, K + 3), dtype=X.dtype, device="cuda")
        big[:, 1:K + 1] = X
        Xv = big[:, 1:K + 1]
        ref = w4.w4_moe_gemv_ids(dc, ds, N * K // 8, N * K // 32, N, K, X.contiguous(), dids, n_experts=E,
                                 route_w=torch.from_numpy(route).cuda())
        got = w4.w4_moe_gemv_ids(dc, ds, N * K // 8, N * K // 32, N, K, Xv, dids, n_experts=E,
                                 route_w=torch.from_numpy(route).cuda())
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), (T, K, X.dtype)


def test_moe_many_pairs_share_an_expert(w4):
    # 20 tokens all choose expert 3 first: more pairs than one MFMA tile of rows
    rng = np.random.default_rng(6)
    E, N, K, T, topk = 6, 40, 128, 20, 2
    codes, steps = experts(rng, E, N, K)
    ids = np.stack([np.array([3, rng.integers(0, 3)]) for _ in range(T)]).astype(np.int32)
    X = synth.activations(rng, (T, K), F16)
    Y = run(w4, codes, steps, N, K, X, F16, ids, 0)
    Yo, Ao = oracle.moe(codes, steps, N * K // 8, N * K // 32, N, K, X, F16, 0, ids, topk,
                        n_experts=E)
    assert within_bound(Y, Yo, Ao)[0]


@pytest.mark.parametrize("T", [1, 4])
def test_moe_expert_layer_full_size(w4, T):
    """One layer of the expert configuration: 128 experts, gate/up 1408x2816 and
    down 2816x704 (group 32, bf16 steps), top-8 of 128 per token; direct and
    32-slot pool addressing; the oracle checks every output of the chosen
    experts."""
    print(f"moe full layer T={T}", flush=True)
    E, topk, S = 128, 8, 32
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    gu_c, gu_s = synth.w4_matrix_torch(g, 1408, 2816, "cuda", count=E)
    dn_c, dn_s = synth.w4_matrix_torch(g, 2816, 704, "cuda", count=E)
    rng = np.random.default_rng(T)
    ids, route = synth.expert_choice(rng, T, E, topk)
    slot_of, used = synth.slot_map(rng, ids, E, S)
    X = synth.activations(rng, (T, 2816), BF16)
    dids = torch.from_numpy(ids).cuda()
    dslot = torch.from_numpy(slot_of).cuda()
    sel = torch.from_numpy(used).cuda().long()
    dsl = torch.from_numpy(slot_of[used]).cuda().long()
    results = {}
    for name, (c, s, N, K) in {"gu": (gu_c, gu_s, 1408, 2816), "down": (dn_c, dn_s, 2816, 704)}.items():
        pool_c = torch.zeros((S,) + tuple(c.shape[1:]), dtype=c.dtype, device="cuda")
        pool_s = torch.zeros((S,) + tuple(s.shape[1:]), dtype=s.dtype, device="cuda")
        pool_c[dsl] = c[sel]
        pool_s[dsl] = s[sel]
        if name == "gu":
            Xin, xpp = dev_act(X, BF16), False
        else:
            # per-pair inputs: the renormalised leading 704 of each gate/up row
            Xin = w4.w4_rms_renorm(results["gu"][0], 704, out_dtype=torch.bfloat16)
            xpp = True
        outs = []
        for rw in (None, torch.from_numpy(route).cuda()):
            if name == "gu" and rw is not None:
                continue
            yd = w4.w4_moe_gemv_ids(c.view(-1, K // 8), s.view(-1, K // 32).view(torch.bfloat16),
                                    N * K // 8, N * K // 32, N, K, Xin, dids, x_per_pair=xpp,
                                    n_experts=E, route_w=rw)
            yp = w4.w4_moe_gemv_ids(pool_c.view(-1, K // 8), pool_s.view(-1, K // 32).view(torch.bfloat16),
                                    N * K // 8, N * K // 32, N, K, Xin, dids, x_per_pair=xpp,
                                    slot_of=dslot, n_experts=E, n_slots=S, route_w=rw)
            torch.cuda.synchronize()
            assert torch.equal(yd.view(torch.int32), yp.view(torch.int32)), (name, rw is None)
            outs.append(yd)
        results[name] = outs
        # oracle on the experts actually used
        cc = c[sel].cpu().numpy().view(np.uint32)
        ssn = s[sel].cpu().numpy().view(np.uint16)
        remap = {int(e): i for i, e in enumerate(used)}
        lids = np.vectorize(lambda e: remap[int(e)])(ids).astype(np.int32)
        Xh = Xin.view(torch.int16).cpu().numpy().view(np.uint16)
        Yo, Ao = oracle.moe(cc, ssn, N * K // 8, N * K // 32, N, K, Xh, BF16, int(xpp), lids, topk,
                            n_experts=len(used))
        ok, worst = within_bound(outs[0].cpu().numpy(), Yo, Ao)
        assert ok, (name, worst)
        if name == "down":
            Yc, Ac = oracle.moe(cc, ssn, N * K // 8, N * K // 32, N, K, Xh, BF16, 1, lids, topk,
                                n_experts=len(used), route_w=route)
            ok, worst = within_bound(outs[1].cpu().numpy(), Yc, Ac)
            assert ok, ("combine", worst)


def test_rms_renorm_rows(w4):
    rng = np.random.default_rng(7)
    v = rng.normal(0, 2, size=(5, 1408)).astype(np.float32)
    out = w4.w4_rms_renorm(torch.from_numpy(v).cuda(), 704, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
    for r in range(5):
        ref = oracle.rms_renorm(v[r], 704, BF16).astype(np.int64)
        assert np.all(np.abs(got[r] - ref) <= 1)
    # odd output row stride: rows 1, 3 start 2 bytes off an 8-byte boundary
    o = torch.zeros((5, 705), dtype=torch.float16, device="cuda")
    w4.w4_rms_renorm(torch.from_numpy(v).cuda(), 704, out=o[:, :704])
    torch.cuda.synchronize()
    got2 = o.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
    for r in range(5):
        ref = oracle.rms_renorm(v[r], 704, F16).astype(np.int64)
        assert np.all(np.abs(got2[r, :704] - ref) <= 1) and got2[r, 704] == 0
