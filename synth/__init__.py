"""Seeded synthetic inputs for the W4A16 decode path.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws random numbers and lays them out in the packed storage format; it holds no
part of the arithmetic being tested (no unpacking, no dequantisation, no dot
products).  Both the CPU oracle and the GPU library are fed from here.

Storage format (the compressed-tensors W4A16 layout described on the dev.to page
"Gemma 4 on a 4 GB GPU in Plain PyTorch", section "Step 1 - Load Google's QAT
Weights Without Unpacking Them": 4-bit codes in groups of 32 along the input
dimension, one 16-bit step per group stored in bf16):

* ``codes``: ``uint32[N][K/8]``.  A weight matrix is ``[N_out][K_in]``.  Nibble j
  (bits 4j..4j+3) of word w in a row holds the code of column 8w+j.  Because
  every nibble of a uniformly random uint32 is an independent uniform draw from
  0..15, codes are generated as whole random words.
* ``steps``: ``bf16[N][K/32]`` carried as raw ``uint16`` bit patterns.
* activations: fp16 or bf16, carried as raw ``uint16`` bit patterns.

Recipe (every draw from ``numpy.random.default_rng(seed)`` in a fixed order):
codes uniform in 0..15; steps = bf16_RNE(|N(0, 0.02)| + 1e-4); activations
N(0, 1) rounded to nearest-even into the stated dtype.
"""

from __future__ import annotations

import numpy as np
import torch

F16 = 0
BF16 = 1
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}


def _bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even, torch's conversion) and
    return the bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _f16_bits_from_f64(a: np.ndarray) -> np.ndarray:
    """Round to IEEE binary16 (numpy's correctly rounded conversion)."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16).copy()


def act_bits(values: np.ndarray, dtype: int) -> np.ndarray:
    """Round arbitrary float values into the activation dtype (RNE); uint16 bits."""
    if dtype == F16:
        return _f16_bits_from_f64(values)
    if dtype == BF16:
        return _bf16_bits_from_f32(np.asarray(values, dtype=np.float32))
    raise ValueError(f"unknown activation dtype {dtype}")


def w4_matrix(rng: np.random.Generator, n: int, k: int, step_sigma: float = 0.02,
              step_floor: float = 1e-4):
    """One packed W4 matrix [n][k]: (codes uint32[n][k/8], steps uint16[n][k/32])."""
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = rng.integers(0, 2**32, size=(n, k // 8), dtype=np.uint32)
    s = np.abs(rng.normal(0.0, step_sigma, size=(n, k // 32))) + step_floor
    steps = _bf16_bits_from_f32(s.astype(np.float32))
    return codes, steps


def activations(rng: np.random.Generator, shape, dtype: int) -> np.ndarray:
    """N(0,1) activations rounded into fp16/bf16; uint16 bit patterns."""
    return act_bits(rng.normal(0.0, 1.0, size=shape), dtype)


def token_ids(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def expert_choice(rng: np.random.Generator, tokens: int, n_experts: int, topk: int):
    """Per token, ``topk`` expert ids drawn uniformly without replacement, kept in
    draw order; router weights are the softmax (fp64, stored fp32) of ``topk``
    N(0,1) logits."""
    ids = np.stack([rng.choice(n_experts, size=topk, replace=False) for _ in range(tokens)])
    logits = rng.normal(0.0, 1.0, size=(tokens, topk))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    route = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.astype(np.int32), route


def slot_map(rng: np.random.Generator, ids: np.ndarray, n_experts: int, n_slots: int):
    """A seeded injective map from the experts a layer uses into ``n_slots`` pool
    slots; ``-1`` for experts with no slot.  Returns (slot_of int32[n_experts],
    used expert ids in ascending order)."""
    used = np.unique(ids.reshape(-1))
    if used.size > n_slots:
        raise ValueError("more distinct experts than pool slots")
    slots = rng.permutation(n_slots)[: used.size]
    slot_of = np.full(n_experts, -1, dtype=np.int32)
    slot_of[used] = slots.astype(np.int32)
    return slot_of, used


# --- device-side generation for the big expert tables -----------------------

def w4_matrix_torch(gen: torch.Generator, n: int, k: int, device, count: int = 1,
                    step_sigma: float = 0.02, step_floor: float = 1e-4):
    """``count`` packed W4 matrices [n][k] drawn with a seeded torch generator on
    ``device`` (used where host generation of many GB would be slow).  Returns
    (codes int32[count][n][k/8] viewed as uint32 words, steps int16[count][n][k/32]
    as bf16 bits)."""
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    codes = torch.randint(-(2**31), 2**31, (count, n, k // 8), generator=gen,
                          device=device, dtype=torch.int32)
    s = torch.randn((count, n, k // 32), generator=gen, device=device,
                    dtype=torch.float32).mul_(step_sigma).abs_().add_(step_floor)
    steps = s.to(torch.bfloat16).view(torch.int16)
    return codes, steps
