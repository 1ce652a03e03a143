"""CPU oracle for the W4A16 decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  It shares no code with the GPU library
(``bit_weight_only_02_amd``) and the library never calls it.

Two independent implementations live here:

* ``w4_oracle.c`` -- plain scalar C, fp64 accumulation, ascending index order
  (the definition written out; see the header of that file for the passages it
  follows).  Wrapped below with ctypes.
* ``brute.py`` -- NumPy brute force: dequantise the whole (tiny) matrix to a
  dense fp64 array through a byte view of the packed words, then a library
  matmul.  Used only to pin the C oracle.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_w4.so")

F16 = 0
BF16 = 1


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (IEEE semantics: no fast-math, no FMA
    contraction).  Returns the path of the shared library."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
            "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        # W4O_LIB lets the mutation test load a deliberately broken copy
        L = ctypes.CDLL(os.environ.get("W4O_LIB") or build())
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.w4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.w4o_f16_to_f64.restype = ctypes.c_double
        L.w4o_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.w4o_bf16_to_f64.restype = ctypes.c_double
        L.w4o_f64_to_f16_rne.argtypes = [ctypes.c_double]
        L.w4o_f64_to_f16_rne.restype = ctypes.c_uint16
        L.w4o_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        L.w4o_f64_to_bf16_rne.restype = ctypes.c_uint16
        L.w4o_code.argtypes = [P, i64, i64, i64]
        L.w4o_code.restype = i32
        L.w4o_dequant.argtypes = [P, P, i64, i64, P]
        L.w4o_dequant.restype = None
        L.w4o_gemv_rows.argtypes = [P, P, i64, i64, P, i32, i64, i64, P, P]
        L.w4o_gemv_rows.restype = None
        L.w4o_gemv.argtypes = [P, P, i64, i64, P, i32, P, P]
        L.w4o_gemv.restype = None
        L.w4o_gemv_omp.argtypes = [P, P, i64, i64, P, i32, P, P]
        L.w4o_gemv_omp.restype = None
        L.w4o_gemv_x64_rows.argtypes = [P, P, i64, P, i64, i64, P, P]
        L.w4o_gemv_x64_rows.restype = None
        L.w4o_gemm.argtypes = [P, P, i64, i64, P, i32, i64, i64, P, P]
        L.w4o_gemm.restype = None
        L.w4o_gather.argtypes = [P, P, i64, i64, P, i64, P]
        L.w4o_gather.restype = i32
        L.w4o_moe.argtypes = [P, P, i64, i64, i64, i64, P, i32, i32, i64, P, i64, i64,
                              P, i64, i64, P, P, P, P]
        L.w4o_moe.restype = i32
        L.w4o_rms_renorm.argtypes = [P, i64, i32, P]
        L.w4o_rms_renorm.restype = None
        L.w4o_grid_to_codes.argtypes = [P, i64, i64, P, P]
        L.w4o_grid_to_codes.restype = None
        L.w4o_num_threads.argtypes = []
        L.w4o_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- scalar conversions -------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return lib().w4o_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return lib().w4o_bf16_to_f64(int(bits))


def f64_to_f16(v: float) -> int:
    return lib().w4o_f64_to_f16_rne(float(v))


def f64_to_bf16(v: float) -> int:
    return lib().w4o_f64_to_bf16_rne(float(v))


def code(codes: np.ndarray, K: int, n: int, k: int) -> int:
    codes = _c(codes, np.uint32)
    return lib().w4o_code(_p(codes), K, n, k)


# --- array entry points -------------------------------------------------------

def dequant(codes, steps, N, K):
    codes, steps = _c(codes, np.uint32), _c(steps, np.uint16)
    W = np.empty((N, K), dtype=np.float64)
    lib().w4o_dequant(_p(codes), _p(steps), N, K, _p(W))
    return W


def gemv(codes, steps, N, K, x, xdtype, rows=None, threads=False):
    """y, a (fp64) of the packed GEMV; ``rows`` = (n0, n1) samples a row range."""
    codes, steps, x = _c(codes, np.uint32), _c(steps, np.uint16), _c(x, np.uint16)
    if rows is None:
        y = np.empty(N, dtype=np.float64)
        a = np.empty(N, dtype=np.float64)
        fn = lib().w4o_gemv_omp if threads else lib().w4o_gemv
        fn(_p(codes), _p(steps), N, K, _p(x), xdtype, _p(y), _p(a))
        return y, a
    n0, n1 = rows
    y = np.empty(n1 - n0, dtype=np.float64)
    a = np.empty(n1 - n0, dtype=np.float64)
    lib().w4o_gemv_rows(_p(codes), _p(steps), N, K, _p(x), xdtype, n0, n1, _p(y), _p(a))
    return y, a


def gemv_x64(codes, steps, N, K, x, rows=None):
    """y, a (fp64) of the packed GEMV on an fp64 input vector x (exact values);
    ``rows`` = (n0, n1) samples a row range."""
    codes, steps = _c(codes, np.uint32), _c(steps, np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float64)
    n0, n1 = (0, N) if rows is None else rows
    y = np.empty(n1 - n0, dtype=np.float64)
    a = np.empty(n1 - n0, dtype=np.float64)
    lib().w4o_gemv_x64_rows(_p(codes), _p(steps), K, _p(x), n0, n1, _p(y), _p(a))
    return y, a


def gemm(codes, steps, N, K, X, xdtype, M, ldx=None):
    codes, steps, X = _c(codes, np.uint32), _c(steps, np.uint16), _c(X, np.uint16)
    ldx = K if ldx is None else ldx
    Y = np.empty((M, N), dtype=np.float64)
    A = np.empty((M, N), dtype=np.float64)
    lib().w4o_gemm(_p(codes), _p(steps), N, K, _p(X), xdtype, M, ldx, _p(Y), _p(A))
    return Y, A


def gather(codes, steps, V, K, ids):
    codes, steps, ids = _c(codes, np.uint32), _c(steps, np.uint16), _c(ids, np.int32)
    out = np.zeros((ids.size, K), dtype=np.uint16)
    bad = lib().w4o_gather(_p(codes), _p(steps), V, K, _p(ids), ids.size, _p(out))
    return out, bad


def moe(codes_base, steps_base, stride_codes, stride_steps, N, K, X, xdtype, x_per_pair,
        ids, topk, slot_of=None, n_experts=None, n_slots=0, row_scale=None, route_w=None,
        ldx=None):
    """Expert-indexed product (see ``w4o_moe`` in the C source).  ``ids`` is
    int32[T][topk] of real expert ids; addresses are base + a*stride with
    a = id (``slot_of`` None) or a = slot_of[id]."""
    codes_base, steps_base = _c(codes_base, np.uint32), _c(steps_base, np.uint16)
    X, ids = _c(X, np.uint16), _c(ids, np.int32)
    T = ids.shape[0]
    ldx = K if ldx is None else ldx
    if slot_of is not None:
        slot_of = _c(slot_of, np.int32)
    if row_scale is not None:
        row_scale = _c(row_scale, np.float32)
    if route_w is not None:
        route_w = _c(route_w, np.float32)
        Y = np.empty((T, N), dtype=np.float64)
        A = np.empty((T, N), dtype=np.float64)
    else:
        Y = np.empty((T * topk, N), dtype=np.float64)
        A = np.empty((T * topk, N), dtype=np.float64)
    rc = lib().w4o_moe(_p(codes_base), _p(steps_base), stride_codes, stride_steps, N, K,
                       _p(X), xdtype, int(x_per_pair), ldx, _p(ids), T, topk,
                       _p(slot_of), n_experts, n_slots, _p(row_scale), _p(route_w),
                       _p(Y), _p(A))
    if rc != 0:
        raise ValueError("expert id or slot out of range")
    return Y, A


def rms_renorm(v, K, out_dtype):
    v = _c(v, np.float32)
    out = np.empty(K, dtype=np.uint16)
    lib().w4o_rms_renorm(_p(v), K, out_dtype, _p(out))
    return out


def grid_to_codes(table, N, K):
    """Codes uint32[N][K/8] and bf16 steps uint16[N][K/32] of a bf16 table
    (bits) whose groups lie on a 4-bit grid (see w4o_grid_to_codes)."""
    table = _c(table, np.uint16)
    codes = np.empty((N, K // 8), dtype=np.uint32)
    steps = np.empty((N, K // 32), dtype=np.uint16)
    lib().w4o_grid_to_codes(_p(table), N, K, _p(codes), _p(steps))
    return codes, steps


def decode_attention(q_bits, k_bits, v_bits, scale):
    """One query token's attention in fp64 [P1-S5]: heads of q (bf16 bits
    [H, D]) over the cached keys and values (bf16 bits [L, D]):
    o[h] = sum_j softmax_j(scale * q[h] . k[j]) v[j]."""
    q = act_to_f64(np.asarray(q_bits).ravel(), 1).reshape(np.shape(q_bits))
    k = act_to_f64(np.asarray(k_bits).ravel(), 1).reshape(np.shape(k_bits))
    v = act_to_f64(np.asarray(v_bits).ravel(), 1).reshape(np.shape(v_bits))
    s = (q @ k.T) * float(scale)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def num_threads() -> int:
    return lib().w4o_num_threads()


def act_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Vector form of the activation decode (calls the scalar C decoder)."""
    f = lib().w4o_f16_to_f64 if dtype == F16 else lib().w4o_bf16_to_f64
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([f(int(v)) for v in b], dtype=np.float64).reshape(np.shape(bits))
