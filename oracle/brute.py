"""NumPy brute force for pinning the C oracle -- TEST INFRASTRUCTURE ONLY.

This is the per-layer unpack-then-multiply path that the dev.to page "Gemma 4 on
a 4 GB GPU in Plain PyTorch" (section "Step 1 - Load Google's QAT Weights
Without Unpacking Them") ran before its packed kernel: materialise the whole
dequantised matrix, then one dense matmul.  It is written independently of the
C oracle: codes are taken from a little-endian *byte* view of the packed words
(low nibble of byte b is column 2b, high nibble column 2b+1), steps are widened
by bit reinterpretation, and the product is a library matmul in fp64.
"""

from __future__ import annotations

import numpy as np


def unpack_codes(codes: np.ndarray, K: int) -> np.ndarray:
    """uint32[N][K/8] -> uint8[N][K] codes via the byte view."""
    c = np.ascontiguousarray(codes, dtype="<u4")
    N = c.shape[0]
    by = c.view(np.uint8).reshape(N, K // 2)
    out = np.empty((N, K), dtype=np.uint8)
    out[:, 0::2] = by & 0x0F
    out[:, 1::2] = by >> 4
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def act_bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    return f16_bits_to_f64(bits) if dtype == 0 else bf16_bits_to_f64(bits)


def dense(codes: np.ndarray, steps: np.ndarray, K: int) -> np.ndarray:
    """Dense fp64 dequantised matrix [N][K]."""
    c = unpack_codes(codes, K).astype(np.float64) - 8.0
    s = bf16_bits_to_f64(steps)               # [N][K/32]
    return c * np.repeat(s, 32, axis=1)


def gemv(codes, steps, K, x_bits, xdtype):
    W = dense(codes, steps, K)
    x = act_bits_to_f64(x_bits, xdtype)
    return W @ x, np.abs(W) @ np.abs(x)
