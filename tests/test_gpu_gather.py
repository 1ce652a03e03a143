"""4-bit row gather on the GPU: bit-exact against the oracle."""

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_act, dev_codes, dev_steps, host_bits, within_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w4():
    import bit_weight_only_02_amd as m
    return m


def test_gather_vocab_table_64_ids_bit_exact(w4):
    rng = np.random.default_rng(0)
    V, K = 262144, 1536
    codes, steps = synth.w4_matrix(rng, V, K)
    ids = synth.token_ids(np.random.default_rng(1), 64, V)
    out = w4.w4_embed_gather(dev_codes(codes), dev_steps(steps), torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    ref, bad = oracle.gather(codes, steps, V, K, ids)
    assert bad == 0
    assert np.array_equal(host_bits(out), ref)


def test_gather_per_layer_table_width_8960(w4):
    """The per-layer 4-bit table at its own width: 262144 rows x 8960 columns
    (1.32 GB packed, generated on the device), 64 ids, bit-exact against the
    oracle on the gathered rows."""
    V, K = 262144, 8960
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    dc, ds = synth.w4_matrix_torch(g, V, K, "cuda")
    dc, ds = dc.view(V, K // 8), ds.view(V, K // 32).view(torch.bfloat16)
    ids = synth.token_ids(np.random.default_rng(4), 64, V)
    ids[:2] = [0, V - 1]
    dids = torch.from_numpy(ids).cuda()
    out = w4.w4_embed_gather(dc, ds, dids)
    torch.cuda.synchronize()
    sub_c = dc.index_select(0, dids.long()).cpu().numpy().view(np.uint32)
    sub_s = ds.view(torch.int16).index_select(0, dids.long()).cpu().numpy().view(np.uint16)
    ref, bad = oracle.gather(sub_c, sub_s, 64, K, np.arange(64, dtype=np.int32))
    assert bad == 0
    assert np.array_equal(host_bits(out), ref)


def test_gather_golden_ties(w4):
    rows = []
    path = os.path.join(os.path.dirname(__file__), "golden", "gather_ties.txt")
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            c, s, e = line.split()
            rows.append((int(c), int(s, 16), int(e, 16)))
    K = 32
    codes = np.stack([np.full(K // 8, 0x11111111 * c, dtype=np.uint32) for c, _, _ in rows])
    steps = np.array([[s] for _, s, _ in rows], dtype=np.uint16)
    ids = np.arange(len(rows), dtype=np.int32)
    out = host_bits(w4.w4_embed_gather(dev_codes(codes), dev_steps(steps),
                                       torch.from_numpy(ids).cuda()))
    for i, (_, _, e) in enumerate(rows):
        assert np.all(out[i] == e)


def test_gather_every_code_step_pair(w4):
    sb = np.arange(0x0080, 0x7F80, 3, dtype=np.uint16)     # normal positive bf16 steps
    K = 128
    V = sb.size
    rng = np.random.default_rng(2)
    codes, _ = synth.w4_matrix(rng, V, K)
    steps = np.repeat(sb.reshape(-1, 1), K // 32, axis=1)
    ids = np.arange(V, dtype=np.int32)
    out = host_bits(w4.w4_embed_gather(dev_codes(codes), dev_steps(steps),
                                       torch.from_numpy(ids).cuda()))
    ref, _ = oracle.gather(codes, steps, V, K, ids)
    assert np.array_equal(out, ref)


def test_gather_bad_ids_give_nan_rows_and_error_flag(w4):
    rng = np.random.default_rng(3)
    V, K = 10, 64
    codes, steps = synth.w4_matrix(rng, V, K)
    ids = np.array([0, 10, -1, 9], dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = w4.w4_embed_gather(dev_codes(codes), dev_steps(steps), torch.from_numpy(ids).cuda(),
                             dev_err=err)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert err.item() == 1
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    ref, bad = oracle.gather(codes, steps, V, K, ids[[0, 3]])
    assert np.array_equal(host_bits(out)[[0, 3]], ref)


# ---- the product and the gather of one table in a single launch ----------------

def run_fused(w4, dc, ds, x, ids, n_out=None):
    V, K = dc.shape[0], dc.shape[1] * 8
    y = torch.full((V,), float("nan"), dtype=torch.float32, device="cuda")
    n = ids.numel()
    out = torch.full((n, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    w4.w4_gemv_gather(dc, ds, x, ids, y, out, err)
    torch.cuda.synchronize()
    return y, out, int(err.item())


@pytest.mark.parametrize("dt", [synth.F16, synth.BF16])
@pytest.mark.parametrize("V,K,n", [(1, 32, 1), (33, 96, 5), (4097, 1536, 64), (1000, 2816, 7),
                                   (513, 8960, 3), (20000, 704, 1), (129, 16384, 2)])
def test_gemv_gather_vs_oracle(w4, V, K, n, dt):
    """Both outputs of the single launch against the oracle: every output of
    the product within the bound, every gathered row bit-exact (rows 0 and
    V - 1 included; 8960 and 16384 columns take several slices per row)."""
    print(f"gemv_gather V={V} K={K} n={n} dt={dt}", flush=True)
    rng = np.random.default_rng(V * 13 + K + n + dt)
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, dt)
    ids = synth.token_ids(rng, n, V)
    ids[0] = V - 1
    if n > 1:
        ids[1] = 0
    y, out, err = run_fused(w4, dev_codes(codes), dev_steps(steps), dev_act(x, dt), torch.from_numpy(ids).cuda())
    assert err == 0
    yo, ao = oracle.gemv(codes, steps, V, K, x, dt, threads=True)
    ok, worst = within_bound(y.cpu().numpy(), yo, ao)
    assert ok, f"worst |err|/sum|wx| = {worst}"
    ref, bad = oracle.gather(codes, steps, V, K, ids)
    assert bad == 0
    assert np.array_equal(host_bits(out), ref)


def test_gemv_gather_vocab_head_equals_separate_launches(w4):
    """The decode step's shape, 262144 x 1536 with bf16 x and 64 ids: the
    single launch gives bitwise the outputs of w4_gemv and w4_embed_gather,
    and its gathered rows equal the oracle's."""
    rng = np.random.default_rng(0)
    V, K = 262144, 1536
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, synth.BF16)
    ids = synth.token_ids(np.random.default_rng(1), 64, V)
    dc, ds, dx, dids = dev_codes(codes), dev_steps(steps), dev_act(x, synth.BF16), torch.from_numpy(ids).cuda()
    y, out, err = run_fused(w4, dc, ds, dx, dids)
    assert err == 0
    y_sep = w4.w4_gemv(dc, ds, dx)
    out_sep = w4.w4_embed_gather(dc, ds, dids)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_sep.view(torch.int32))
    assert torch.equal(out.view(torch.int16), out_sep.view(torch.int16))
    ref, bad = oracle.gather(codes, steps, V, K, ids)
    assert bad == 0 and np.array_equal(host_bits(out), ref)
    yo, ao = oracle.gemv(codes, steps, V, K, x, synth.BF16, rows=(V - 4096, V))
    ok, worst = within_bound(y[V - 4096:].cpu().numpy(), yo, ao)
    assert ok, f"worst |err|/sum|wx| = {worst}"


def test_gemv_gather_bad_id_and_no_ids(w4):
    """An id out of range: its row is NaN and the error word is set, the
    other rows and the product are unaffected; n = 0 runs the product alone."""
    rng = np.random.default_rng(21)
    V, K = 3000, 1536
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, synth.F16)
    dc, ds, dx = dev_codes(codes), dev_steps(steps), dev_act(x, synth.F16)
    ids = np.array([5, V, 7, -1], dtype=np.int32)
    y, out, err = run_fused(w4, dc, ds, dx, torch.from_numpy(ids).cuda())
    assert err == 1
    bits = host_bits(out)
    ref, _ = oracle.gather(codes, steps, V, K, np.array([5, 0, 7, 0], dtype=np.int32))
    assert np.array_equal(bits[0], ref[0]) and np.array_equal(bits[2], ref[2])
    assert np.all(bits[1] == 0x7FC0) and np.all(bits[3] == 0x7FC0)
    y_sep = w4.w4_gemv(dc, ds, dx)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y_sep.view(torch.int32))
    y0, out0, err0 = run_fused(w4, dc, ds, dx, torch.empty(0, dtype=torch.int32, device="cuda"))
    assert err0 == 0 and out0.numel() == 0
    assert torch.equal(y0.view(torch.int32), y_sep.view(torch.int32))
