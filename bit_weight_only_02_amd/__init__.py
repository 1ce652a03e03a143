"""Python binding of libw4, the MI355X W4A16 decode library.

Argument marshalling only: every function here takes torch device tensors,
passes their device pointers and the current HIP stream to the C entry point of
the same name in ``libw4.so`` (declared in ``include/w4.h``), and raises on a
non-zero status.  Nothing is computed in Python and there is no fallback: if
``libw4.so`` is missing or fails to load, the import fails.

Tensor conventions:
  codes  int32 (or uint32) tensor [N, K/8]: packed words (nibble j of word w is
         column 8w+j);
  steps  bfloat16 tensor (or int16/uint16 holding bf16 bits) [N, K/32];
  activations float16 or bfloat16 tensors (their dtype selects W4_F16/W4_BF16);
  outputs float32 (products) or bfloat16 (row gather).

Workspaces: w4_gemm_smallM, w4_gemm_prompt, w4_decode_attention and
w4_moe_gemv_ids take a caller-owned device workspace (``workspace=``, a
zero-initialised byte tensor of at least the matching ``*_workspace_bytes``
size).  When none is given, a zeroed one is taken from a cache kept per
(device, stream), grown when a call needs more; calls issued on different
streams therefore never share one.
"""

from __future__ import annotations

import ctypes
import os

import torch  # must load before libw4 so that both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4.so")

W4_OK = 0
W4_ERR_INVALID_ARG = -1
W4_ERR_ALIGNMENT = -2
W4_ERR_DTYPE = -3
W4_ERR_UNSUPPORTED = -4
W4_ERR_NODEV = -5
W4_ERR_HIP = -6
W4_F16 = 0
W4_BF16 = 1
W4_F32_RMS = 2  # w4_moe_gemv_ids: fp32 rows renormalised on load
W4_MAX_K = 16384
W4_MAX_K_SMALLM = 16384
W4_MAX_K_CHAIN = 8192
W4_MAX_M = 16
W4_MAX_TOPK = 32
W4_MAX_M_PROMPT = 4096

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with bit_weight_only_02_amd/build.py "
                      "(or __graft_entry__.build()) first")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

lib = ctypes.CDLL(LIB_PATH)

_SIGNATURES = {
    "w4_gemv": [_P, _P, _I32, _I32, _P, _I32, _P, _P],
    "w4_gemm_smallM": [_P, _P, _I32, _I32, _P, _I32, _I32, _I64, _P, _I64, _P, _I64, _P],
    "w4_gemm_prompt": [_P, _P, _I32, _I32, _P, _I32, _I32, _I64, _P, _I64, _P, _I64, _P],
    "w4_grid_to_codes": [_P, _I32, _I32, _P, _P, _P],
    "w4_decode_attention": [_P, _I32, _I32, _P, _I64, _P, _I64, _I32, ctypes.c_float, _P, _P, _I64,
                            _P],
    "w4_moe_gemv_ids": [_P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _I64, _P, _I32, _I32,
                        _P, _I32, _I32, _P, _P, _P, _P, _P, _I64, _P],
    "w4_moe_gemv_ids_noalloc": [_P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _I64, _P, _I32, _I32,
                                _P, _I32, _I32, _P, _P, _P, _P, _P],
    "w4_embed_gather": [_P, _P, _I32, _I32, _P, _I32, _P, _P, _P],
    "w4_gemv_gather": [_P, _P, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _P, _P],
    "w4_rms_renorm": [_P, _I64, _I32, _I32, _P, _I64, _I32, _P],
    "w4_gemv_chain": [_P, _I32, _P, _P, _I64, _P],
    "w4_probe_stream": [_P, _I64, _P, _P],
}
for _name, _args in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
_WS_SIGNATURES = {
    "w4_gemm_smallM_workspace_bytes": [_I32, _I32, _I32],
    "w4_gemm_prompt_workspace_bytes": [_I32, _I32, _I32],
    "w4_decode_attention_workspace_bytes": [_I32, _I32, _I32],
    "w4_moe_gemv_ids_workspace_bytes": [_I32, _I32, _I32, _I32, _I32, _I32, _I32],
}
for _name, _args in _WS_SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int64
_POOL_SIGNATURES = {
    "w4_pool_create": [_I32, _I32, _I32, _I32, _P, _P],
    "w4_pool_plan": [_P, _I32, _P, _I32, _P, _P, _P],
    "w4_pool_prepare": [_P, _I32, _P, _I32, _P, _P, _P, _P],
    "w4_pool_join": [_P, _I32, _P],
    "w4_pool_release": [_P, _I32, _P],
    "w4_pool_stats": [_P, _P, _P, _P],
}
for _name, _args in _POOL_SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
lib.w4_pool_destroy.argtypes = [_P]
lib.w4_pool_destroy.restype = None
lib.w4_reload_settings.argtypes = []
lib.w4_reload_settings.restype = None
lib.w4_strerror.argtypes = [ctypes.c_int]
lib.w4_strerror.restype = ctypes.c_char_p
lib.w4_last_error_detail.argtypes = []
lib.w4_last_error_detail.restype = ctypes.c_char_p


class W4Error(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        detail = lib.w4_last_error_detail().decode()
        super().__init__(f"{fn}: {lib.w4_strerror(status).decode()} ({status}) {detail}")


def _check(status: int, fn: str) -> None:
    if status != W4_OK:
        raise W4Error(status, fn)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws_size(n: int, fn: str) -> int:
    if n < 0:
        raise W4Error(int(n), fn)
    return int(n)


_WS_CACHE: dict = {}


def _workspace(nbytes: int, device, stream, given):
    """(pointer, bytes) of the workspace for one call: the caller's tensor, or
    a zeroed one cached per (device, stream) and grown on demand."""
    if nbytes == 0:
        return None, 0
    if given is not None:
        return given.data_ptr(), given.numel() * given.element_size()
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (torch.device(device).index, s.cuda_stream)
    buf = _WS_CACHE.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WS_CACHE[key] = buf
    return buf.data_ptr(), buf.numel()


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace of nbytes (torch's allocations are 256-byte aligned)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def w4_reload_settings() -> None:
    """Re-read the library's W4_* settings variables (tests)."""
    lib.w4_reload_settings()


reload_settings = w4_reload_settings


def w4_gemm_smallM_workspace_bytes(N: int, K: int, M: int) -> int:
    return _ws_size(lib.w4_gemm_smallM_workspace_bytes(N, K, M), "w4_gemm_smallM_workspace_bytes")


def w4_gemm_prompt_workspace_bytes(N: int, K: int, M: int) -> int:
    return _ws_size(lib.w4_gemm_prompt_workspace_bytes(N, K, M), "w4_gemm_prompt_workspace_bytes")


def w4_decode_attention_workspace_bytes(H: int, D: int, L: int) -> int:
    return _ws_size(lib.w4_decode_attention_workspace_bytes(H, D, L), "w4_decode_attention_workspace_bytes")


def w4_moe_gemv_ids_workspace_bytes(N: int, K: int, T: int, topk: int, xdt: int, x_per_pair: bool,
                                    combined: bool) -> int:
    return _ws_size(lib.w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, xdt, int(x_per_pair), int(combined)),
                    "w4_moe_gemv_ids_workspace_bytes")


def _act_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return W4_F16
    if t.dtype == torch.bfloat16:
        return W4_BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _matrix(codes: torch.Tensor, steps: torch.Tensor):
    if codes.dim() != 2 or steps.dim() != 2:
        raise ValueError("codes and steps must be 2-D [N, K/8] and [N, K/32]")
    if codes.element_size() != 4 or steps.element_size() != 2:
        raise TypeError("codes must hold 32-bit words and steps 16-bit bf16 bits")
    if not (codes.is_contiguous() and steps.is_contiguous()):
        raise ValueError("codes and steps must be contiguous")
    N, K = codes.shape[0], codes.shape[1] * 8
    if tuple(steps.shape) != (N, K // 32):
        raise ValueError(f"steps shape {tuple(steps.shape)} does not match codes [N={N}, K={K}]")
    return N, K


def w4_gemv(codes, steps, x, y=None, stream=None):
    """y[n] = sum_k (code(n,k) - 8) * step(n,k/32) * x[k]; returns y (fp32 [N])."""
    N, K = _matrix(codes, steps)
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be contiguous with K elements")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=codes.device)
    _check(lib.w4_gemv(_ptr(codes), _ptr(steps), N, K, _ptr(x), _act_dtype(x), _ptr(y),
                       _stream(stream)), "w4_gemv")
    return y


def w4_gemm_smallM(codes, steps, X, Y=None, stream=None, workspace=None):
    """Y[m, n] for the M rows of X ([M, ldx] with row stride >= K); Y fp32 [M, N]."""
    N, K = _matrix(codes, steps)
    if X.dim() != 2 or X.stride(1) != 1 or X.shape[1] < K:
        raise ValueError("X must be [M, >=K] with unit column stride")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    if Y.dim() != 2 or Y.stride(1) != 1 or Y.shape[0] != M or Y.shape[1] < N:
        raise ValueError("Y must be [M, >=N] with unit column stride")
    ws, wsb = _workspace(max(int(lib.w4_gemm_smallM_workspace_bytes(N, K, M)), 0), codes.device, stream,
                         workspace)
    _check(lib.w4_gemm_smallM(_ptr(codes), _ptr(steps), N, K, _ptr(X), _act_dtype(X), M,
                              X.stride(0), _ptr(Y), Y.stride(0), ws, wsb, _stream(stream)),
           "w4_gemm_smallM")
    return Y


def w4_gemm_prompt(codes, steps, X, Y=None, stream=None, workspace=None):
    """Prompt-chunk product: Y[m, n] for the M rows of X ([M, ldx], ldx >= K,
    M up to W4_MAX_M_PROMPT) on the matrix cores; Y fp32 [M, N]."""
    N, K = _matrix(codes, steps)
    if X.dim() != 2 or X.stride(1) != 1 or X.shape[1] < K:
        raise ValueError("X must be [M, >=K] with unit column stride")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    if Y.dim() != 2 or Y.stride(1) != 1 or Y.shape[0] != M or Y.shape[1] < N:
        raise ValueError("Y must be [M, >=N] with unit column stride")
    ws, wsb = _workspace(max(int(lib.w4_gemm_prompt_workspace_bytes(N, K, M)), 0), codes.device, stream,
                         workspace)
    _check(lib.w4_gemm_prompt(_ptr(codes), _ptr(steps), N, K, _ptr(X), _act_dtype(X), M,
                              X.stride(0), _ptr(Y), Y.stride(0), ws, wsb, _stream(stream)),
           "w4_gemm_prompt")
    return Y


def w4_grid_to_codes(table, codes=None, steps=None, stream=None):
    """Packs a bf16 table [N, K] whose groups of 32 lie on a 4-bit grid into
    codes (int32 [N, K/8], uint32 words) and bf16 steps [N, K/32]."""
    if table.dim() != 2 or not table.is_contiguous() or table.dtype != torch.bfloat16:
        raise ValueError("table must be a contiguous bf16 [N, K] tensor")
    N, K = table.shape
    if codes is None:
        codes = torch.empty((N, K // 8), dtype=torch.int32, device=table.device)
    if steps is None:
        steps = torch.empty((N, K // 32), dtype=torch.bfloat16, device=table.device)
    _check(lib.w4_grid_to_codes(_ptr(table), N, K, _ptr(codes), _ptr(steps), _stream(stream)),
           "w4_grid_to_codes")
    return codes, steps


def w4_decode_attention(q, k, v, scale, o=None, stream=None, workspace=None):
    """One query token's attention: q bf16 [H, D] (H <= 8 heads sharing one
    key/value head), k, v bf16 [L, >=D] rows; returns o fp32 [H, D]."""
    if q.dim() != 2 or not q.is_contiguous() or k.dim() != 2 or v.dim() != 2 or k.shape[0] != v.shape[0]:
        raise ValueError("q [H, D] contiguous; k, v [L, >=D] with the same L")
    if k.stride(1) != 1 or v.stride(1) != 1:
        raise ValueError("k, v need unit column stride")
    H, D = q.shape
    if o is None:
        o = torch.empty((H, D), dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(max(int(lib.w4_decode_attention_workspace_bytes(H, D, k.shape[0])), 0), q.device,
                         stream, workspace)
    _check(lib.w4_decode_attention(_ptr(q), H, D, _ptr(k), k.stride(0), _ptr(v), v.stride(0), k.shape[0],
                                   float(scale), _ptr(o), ws, wsb, _stream(stream)), "w4_decode_attention")
    return o


def w4_moe_gemv_ids(codes_base, steps_base, expert_stride_codes, expert_stride_steps, N, K,
                    X, ids, x_per_pair=False, slot_of=None, n_experts=None, n_slots=0,
                    row_scale=None, route_w=None, Y=None, dev_err=None, stream=None, workspace=None):
    """Expert-indexed product (see w4.h).  ``ids`` int32 [T, topk] of real ids;
    strides in uint32 words / uint16 elements; ``slot_of`` int32 [n_experts]
    selects pool addressing.  A float32 ``X`` is renormalised on load (each
    row's leading K entries divided by their RMS and rounded to fp16, as
    w4_rms_renorm does)."""
    T, topk = ids.shape
    if n_experts is None:
        raise ValueError("n_experts is required")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    rows = T * topk if route_w is None else T
    if Y is None:
        Y = torch.empty((rows, N), dtype=torch.float32, device=X.device)
    xdt = W4_F32_RMS if X.dtype == torch.float32 else _act_dtype(X)
    need = lib.w4_moe_gemv_ids_workspace_bytes(N, K, T, topk, xdt, 1 if x_per_pair else 0,
                                               0 if route_w is None else 1)
    ws, wsb = _workspace(max(int(need), 0), X.device, stream, workspace)
    _check(lib.w4_moe_gemv_ids(_ptr(codes_base), _ptr(steps_base), expert_stride_codes,
                               expert_stride_steps, N, K, _ptr(X), xdt,
                               1 if x_per_pair else 0, X.stride(0), _ptr(ids), T, topk,
                               _ptr(slot_of), n_experts, n_slots, _ptr(row_scale),
                               _ptr(route_w), _ptr(Y), _ptr(dev_err), ws, wsb, _stream(stream)),
           "w4_moe_gemv_ids")
    return Y


def w4_moe_gemv_ids_noalloc(codes_base, steps_base, expert_stride_codes, expert_stride_steps, N, K,
                            X, ids, x_per_pair=False, slot_of=None, n_experts=None, n_slots=0,
                            row_scale=None, route_w=None, Y=None, dev_err=None, stream=None):
    """w4_moe_gemv_ids whose scratch is the library's fixed per-GPU array
    (nothing is allocated; overlapping calls on one GPU race)."""
    T, topk = ids.shape
    if n_experts is None:
        raise ValueError("n_experts is required")
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    if Y is None:
        raise ValueError("Y is required (this entry point is for callers that allocate nothing)")
    xdt = W4_F32_RMS if X.dtype == torch.float32 else _act_dtype(X)
    _check(lib.w4_moe_gemv_ids_noalloc(_ptr(codes_base), _ptr(steps_base), expert_stride_codes,
                                       expert_stride_steps, N, K, _ptr(X), xdt,
                                       1 if x_per_pair else 0, X.stride(0), _ptr(ids), T, topk,
                                       _ptr(slot_of), n_experts, n_slots, _ptr(row_scale),
                                       _ptr(route_w), _ptr(Y), _ptr(dev_err), _stream(stream)),
           "w4_moe_gemv_ids_noalloc")
    return Y


W4_NOALLOC_SCRATCH_BYTES = 8 << 20


def _i32_host(a):
    import numpy as np
    return np.ascontiguousarray(a, dtype=np.int32)


def w4_pool_create(n_layers, n_experts, n_slots, part_bytes):
    """Host-side manager of per-layer expert slot pools (see w4.h); returns an
    opaque handle.  part_bytes: the bytes of each part of one expert."""
    import numpy as np
    pb = np.ascontiguousarray(part_bytes, dtype=np.int64)
    h = ctypes.c_void_p()
    _check(lib.w4_pool_create(n_layers, n_experts, n_slots, pb.size, pb.ctypes.data, ctypes.byref(h)),
           "w4_pool_create")
    return h


def w4_pool_destroy(pool):
    lib.w4_pool_destroy(pool)


def w4_pool_plan(pool, layer, ids, n_experts):
    """The LFU decision alone: returns (slot_of int32[n_experts], [(expert, slot)
    of each miss])."""
    import numpy as np
    ids = _i32_host(ids).ravel()
    slot_of = np.empty(n_experts, dtype=np.int32)
    me = np.empty(max(ids.size, 1), dtype=np.int32)
    ms = np.empty(max(ids.size, 1), dtype=np.int32)
    n = lib.w4_pool_plan(pool, layer, ids.ctypes.data, ids.size, slot_of.ctypes.data, me.ctypes.data,
                         ms.ctypes.data)
    if n < 0:
        raise W4Error(n, "w4_pool_plan")
    return slot_of, list(zip(me[:n].tolist(), ms[:n].tolist()))


def w4_pool_prepare(pool, layer, ids, host_parts, dev_parts, dev_slot_of, copy_stream):
    """LFU decision, then the misses' copies and the slot map's upload on
    copy_stream.  host_parts: pinned host tensors (expert-major), dev_parts:
    the layer's device pool tensors (slot-major), dev_slot_of: int32 device
    tensor [n_experts]."""
    ids = _i32_host(ids).ravel()
    hp = (ctypes.c_void_p * len(host_parts))(*[t.data_ptr() for t in host_parts])
    dp = (ctypes.c_void_p * len(dev_parts))(*[t.data_ptr() for t in dev_parts])
    _check(lib.w4_pool_prepare(pool, layer, ids.ctypes.data, ids.size, hp, dp, dev_slot_of.data_ptr(),
                               copy_stream.cuda_stream), "w4_pool_prepare")


def w4_pool_join(pool, layer, stream=None):
    _check(lib.w4_pool_join(pool, layer, _stream(stream)), "w4_pool_join")


def w4_pool_release(pool, layer, stream=None):
    _check(lib.w4_pool_release(pool, layer, _stream(stream)), "w4_pool_release")


def w4_pool_stats(pool):
    """(hits, misses, bytes copied) since creation."""
    h, m, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.w4_pool_stats(pool, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)), "w4_pool_stats")
    return h.value, m.value, b.value


def w4_embed_gather(codes, steps, ids, out=None, dev_err=None, stream=None):
    """bf16 rows (code - 8) * step of the table rows ``ids``; returns [n, K] bf16."""
    V, K = _matrix(codes, steps)
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib.w4_embed_gather(_ptr(codes), _ptr(steps), V, K, _ptr(ids), n, _ptr(out),
                               _ptr(dev_err), _stream(stream)), "w4_embed_gather")
    return out


def w4_gemv_gather(codes, steps, x, ids, y=None, out=None, dev_err=None, stream=None):
    """w4_gemv and w4_embed_gather of the same table in one launch; returns
    (y fp32 [V], out bf16 [n, K])."""
    V, K = _matrix(codes, steps)
    if x.numel() != K or not x.is_contiguous():
        raise ValueError("x must be contiguous with K elements")
    n = ids.numel()
    if y is None:
        y = torch.empty(V, dtype=torch.float32, device=codes.device)
    if out is None:
        out = torch.empty((n, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib.w4_gemv_gather(_ptr(codes), _ptr(steps), V, K, _ptr(x), _act_dtype(x), _ptr(y), _ptr(ids), n,
                              _ptr(out), _ptr(dev_err), _stream(stream)), "w4_gemv_gather")
    return y, out


def w4_rms_renorm(v, K, out=None, out_dtype=torch.float16, stream=None):
    """Leading K entries of each fp32 row of ``v`` ([K'] or [rows, K'] with unit
    column stride) divided by their RMS, rounded to out_dtype; returns [K] or
    [rows, K]."""
    rows = 1 if v.dim() == 1 else v.shape[0]
    ldv = v.shape[-1] if v.dim() == 1 else v.stride(0)
    if out is None:
        shape = (K,) if v.dim() == 1 else (rows, K)
        out = torch.empty(shape, dtype=out_dtype, device=v.device)
    ldo = K if out.dim() == 1 else out.stride(0)
    _check(lib.w4_rms_renorm(_ptr(v), ldv, K, rows, _ptr(out), ldo, _act_dtype(out),
                             _stream(stream)), "w4_rms_renorm")
    return out


def w4_chain_desc(mats, ys):
    """Device descriptor array for w4_gemv_chain: ``mats`` is a list of
    (codes, steps) and ``ys`` the fp32 outputs.  Returns an int64 tensor of
    records {codes, steps, y, N | K << 32} (the layout of w4_chain_mat)."""
    rec = []
    for (c, s), y in zip(mats, ys):
        N, K = _matrix(c, s)
        if y.numel() < N or y.dtype != torch.float32:
            raise ValueError("each y must be fp32 with at least N elements")
        rec.append([c.data_ptr(), s.data_ptr(), y.data_ptr(), (N & 0xFFFFFFFF) | (K << 32)])
    return torch.tensor(rec, dtype=torch.int64).cuda()


def w4_chain_sync_bytes(n_mats: int) -> int:
    """Bytes of the sync buffer of a chain of n_mats matrices
    (W4_CHAIN_SYNC_BYTES(n_mats) of w4.h)."""
    return 256 + n_mats * 32768


def w4_chain_sync(n_mats: int, device="cuda"):
    """A zeroed sync buffer for a w4_gemv_chain of n_mats matrices."""
    return torch.zeros(w4_chain_sync_bytes(n_mats) // 4, dtype=torch.int32, device=device)


def w4_gemv_chain(desc, x0, sync, stream=None):
    """Run the chain described by ``desc`` (from w4_chain_desc) on fp16 ``x0``."""
    if x0.dtype != torch.float16:
        raise TypeError("x0 must be float16")
    _check(lib.w4_gemv_chain(_ptr(desc), desc.shape[0], _ptr(x0), _ptr(sync),
                             sync.numel() * sync.element_size(), _stream(stream)),
           "w4_gemv_chain")


def w4_probe_stream(buf, out, stream=None):
    """Streaming read of ``buf`` (bytes multiple of 16); word sum added into out."""
    _check(lib.w4_probe_stream(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out),
                               _stream(stream)), "w4_probe_stream")
    return out
