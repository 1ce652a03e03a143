"""Expert streaming through slot pools on the GPU: several decode steps of
three expert layers with streaming on (per-layer LFU pools of 16 slots filled
by asynchronous copies from a pinned host store on a second stream, a dense
product on the compute stream overlapping them, one join per layer) give every
output bit for bit as streaming off (the full expert tensors addressed
directly) -- the page's identity bar (the anyesh.me page, "Streaming without
touching a single GPU kernel": same kernels, same bytes, different
addressing)."""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def _bits(t):
    return t.contiguous().view(torch.int32).cpu()


def test_streaming_on_matches_off_bitwise_over_steps(w4):
    L, E, S, T, topk, steps = 3, 48, 16, 2, 4, 8
    NG, KG = 256, 512        # gate/up [2 x 128, 512]
    ND, KD = 512, 128        # down [512, 128] on the gate half
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    full, pools, host, slot_dev = [], [], [], []
    for _ in range(L):
        gc, gs = synth.w4_matrix_torch(g, NG, KG, "cuda", count=E)
        dc, ds = synth.w4_matrix_torch(g, ND, KD, "cuda", count=E)
        parts = [gc.reshape(E, -1), gs.reshape(E, -1), dc.reshape(E, -1), ds.reshape(E, -1)]
        full.append(parts)
        host.append([p.view(torch.uint8).cpu().pin_memory() for p in parts])
        pools.append([torch.zeros((S, p.shape[1]), dtype=p.dtype, device="cuda") for p in parts])
        slot_dev.append(torch.full((E,), -1, dtype=torch.int32, device="cuda"))
    part_bytes = [p[0].numel() * p.element_size() for p in full[0]]
    dense = [synth.w4_matrix_torch(g, ND, ND, "cuda") for _ in range(L)]
    pool = w4.w4_pool_create(L, E, S, part_bytes)
    copy_stream = torch.cuda.Stream()
    rng = np.random.default_rng(5)
    prev = [None] * L

    def layer_views(parts):
        gc, gs, dc, ds = parts
        return (gc.reshape(-1, KG // 8), gs.reshape(-1, KG // 32).view(torch.bfloat16),
                dc.reshape(-1, KD // 8), ds.reshape(-1, KD // 32).view(torch.bfloat16))

    def run_layer(li, x, ids_dev, route, parts, slot_of):
        gc, gs, dc, ds = layer_views(parts)
        kw = {} if slot_of is None else dict(slot_of=slot_of, n_slots=S)
        G = w4.w4_moe_gemv_ids(gc, gs, NG * KG // 8, NG * KG // 32, NG, KG, x, ids_dev, n_experts=E, **kw)
        D = w4.w4_moe_gemv_ids(dc, ds, ND * KD // 8, ND * KD // 32, ND, KD, G, ids_dev, x_per_pair=True,
                               n_experts=E, route_w=route, **kw)
        return G, D

    try:
        for step in range(steps):
            x_on = x_off = torch.from_numpy(rng.standard_normal((T, KG)).astype(np.float32)).cuda()
            outs_on, outs_off = [], []
            for li in range(L):
                # routing with reuse between steps, so that some choices hit
                ids = np.empty((T, topk), dtype=np.int32)
                for t in range(T):
                    keep = prev[li][t][:2] if prev[li] is not None and rng.random() < 0.7 else []
                    rest = [e for e in rng.permutation(E) if e not in keep][:topk - len(keep)]
                    ids[t] = list(keep) + rest
                prev[li] = ids
                route = torch.from_numpy(synth.expert_choice(rng, T, E, topk)[1]).cuda()
                ids_dev = torch.from_numpy(ids).cuda()
                # streaming on: copies on the side stream, dense work meanwhile, one join
                w4.w4_pool_prepare(pool, li, ids, host[li], pools[li], slot_dev[li], copy_stream)
                dn_on = w4.w4_gemm_smallM(dense[li][0][0], dense[li][1][0].view(torch.bfloat16),
                                          torch.zeros((T, ND), dtype=torch.bfloat16, device="cuda") +
                                          x_on[:, :ND].to(torch.bfloat16))
                w4.w4_pool_join(pool, li)
                G, D = run_layer(li, x_on, ids_dev, route, pools[li], slot_dev[li])
                w4.w4_pool_release(pool, li)
                outs_on += [G, D, dn_on]
                # streaming off: the full tensors, direct addressing
                dn_off = w4.w4_gemm_smallM(dense[li][0][0], dense[li][1][0].view(torch.bfloat16),
                                           torch.zeros((T, ND), dtype=torch.bfloat16, device="cuda") +
                                           x_off[:, :ND].to(torch.bfloat16))
                G2, D2 = run_layer(li, x_off, ids_dev, route, full[li], None)
                outs_off += [G2, D2, dn_off]
                x_on, x_off = D, D2
            torch.cuda.synchronize()
            for a, b in zip(outs_on, outs_off):
                assert torch.equal(_bits(a), _bits(b)), step
        hits, misses, nbytes = w4.w4_pool_stats(pool)
        assert hits > 0 and misses > 0
        assert nbytes == misses * sum(part_bytes)
    finally:
        torch.cuda.synchronize()
        w4.w4_pool_destroy(pool)
