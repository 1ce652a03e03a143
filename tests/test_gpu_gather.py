"""4-bit row gather on the GPU: bit-exact against the oracle."""

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import dev_codes, dev_steps, host_bits

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
