"""ctypes front end of the C oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Every function works on host NumPy arrays; the
pool arrays are updated in place exactly as one decode launch would update
the device pool.  What the loop computes, and which page passage each step
follows, is written out in kda_oracle.h.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

POOL_F32 = 0
POOL_F16 = 1
POOL_BF16 = 2

_lib = None


def lib() -> ctypes.CDLL:
    """Load oracle/libkda_oracle.so, compiling it first if it is missing.
    KDA_ORACLE_LIB names another build of the same source to load instead
    (the tests' sanitizer run)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KDA_ORACLE_LIB") or _build.LIB
    if path == _build.LIB and not os.path.exists(path):
        _build.build()
    L = ctypes.CDLL(path)
    c_f = ctypes.POINTER(ctypes.c_float)
    c_d = ctypes.POINTER(ctypes.c_double)
    c_i = ctypes.POINTER(ctypes.c_int32)
    c_u16 = ctypes.POINTER(ctypes.c_uint16)
    L.kdao_f32_to_f16_rne.argtypes = [ctypes.c_float]
    L.kdao_f32_to_f16_rne.restype = ctypes.c_uint16
    L.kdao_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.kdao_f16_to_f32.restype = ctypes.c_float
    L.kdao_f32_to_f16_rne_array.argtypes = [c_f, c_u16, ctypes.c_int64]
    L.kdao_f32_to_f16_rne_array.restype = None
    L.kdao_f16_to_f32_array.argtypes = [c_u16, c_f, ctypes.c_int64]
    L.kdao_f16_to_f32_array.restype = None
    L.kdao_f32_to_bf16_rne_array.argtypes = [c_f, c_u16, ctypes.c_int64]
    L.kdao_f32_to_bf16_rne_array.restype = None
    i32 = ctypes.c_int32
    L.kdao_step_f32.argtypes = [ctypes.c_void_p, ctypes.c_int, i32, i32, i32, i32,
                                c_i, c_i, i32, i32, c_f, c_f, c_f, c_f, c_f,
                                ctypes.c_float, c_f]
    L.kdao_step_f32.restype = ctypes.c_int
    L.kdao_step_f64.argtypes = [c_d, i32, i32, i32, i32, c_i, c_i, i32, i32,
                                c_f, c_f, c_f, c_f, c_f, ctypes.c_double, c_d]
    L.kdao_step_f64.restype = ctypes.c_int
    L.kdao_prefill_f32.argtypes = [ctypes.c_void_p, ctypes.c_int, i32, i32, i32, i32, c_i, c_i, c_i,
                                   i32, c_f, c_f, c_f, c_f, c_f, ctypes.c_float, c_f]
    L.kdao_prefill_f32.restype = ctypes.c_int
    L.kdao_prefill_f64.argtypes = [c_d, i32, i32, i32, i32, c_i, c_i, c_i, i32,
                                   c_f, c_f, c_f, c_f, c_f, ctypes.c_double, c_d]
    L.kdao_prefill_f64.restype = ctypes.c_int
    L.kdao_conv_f32.argtypes = [c_u16, i32, i32, c_i, c_i, i32, i32, c_f, c_f, c_f]
    L.kdao_conv_f32.restype = ctypes.c_int
    L.kdao_set_mutation.argtypes = [ctypes.c_int]
    L.kdao_set_mutation.restype = None
    _lib = L
    return L


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def f32_to_f16_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> binary16 bits (uint16), round to nearest even."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().kdao_f32_to_f16_rne_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    """binary16 bits (uint16) -> binary32, exact."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().kdao_f16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bits (uint16), round to nearest even."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().kdao_f32_to_bf16_rne_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def _init_ptr(init_slot_ids, n_req):
    """(array kept alive, pointer) for an optional per-request initial slot table."""
    if init_slot_ids is None:
        return None, None
    arr = np.ascontiguousarray(init_slot_ids, dtype=np.int32).reshape(-1)
    if arr.size != n_req:
        raise ValueError("init_slot_ids needs one entry per request")
    return arr, _ptr(arr, ctypes.c_int32)


def _check_inputs(pool, slot_ids, q, k, v, g, b, n_rows):
    n_slots, H, K, V = pool.shape
    slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32).reshape(-1)
    R = slot_ids.size
    if R % n_rows:
        raise ValueError("slot_ids length %d is not a multiple of n_rows %d" % (R, n_rows))
    q, k, v, g, b = (_f32(x) for x in (q, k, v, g, b))
    if q.shape != (R, H, K) or k.shape != (R, H, K) or g.shape != (R, H, K):
        raise ValueError("q, k, g must be [R, H, K]")
    if v.shape != (R, H, V):
        raise ValueError("v must be [R, H, V]")
    if b.shape != (R, H):
        raise ValueError("b must be [R, H]")
    return (n_slots, H, K, V), slot_ids, q, k, v, g, b


def step_f32(pool: np.ndarray, slot_ids, q, k, v, g, b, n_rows: int = 1,
             scale: float | None = None, init_slot_ids=None, bf16: bool = False) -> np.ndarray:
    """One decode launch in fp32 on a host pool (float32 or uint16 fp16 bits,
    shape [n_slots, H, K, V]), updated in place.  Returns out [R, H, V].
    init_slot_ids: optional [n_req] slots holding each request's initial
    state (default: each request's row-0 slot).  bf16=True reads a uint16
    pool as bfloat16 bits (error studies only)."""
    if not pool.flags["C_CONTIGUOUS"]:
        raise ValueError("pool must be C-contiguous")
    if pool.dtype == np.float32:
        kind = POOL_F32
    elif pool.dtype == np.uint16:
        kind = POOL_BF16 if bf16 else POOL_F16
    else:
        raise TypeError("oracle pool must be float32 or uint16 (fp16 bits)")
    (n_slots, H, K, V), slot_ids, q, k, v, g, b = _check_inputs(pool, slot_ids, q, k, v, g, b, n_rows)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    R = slot_ids.size
    out = np.zeros((R, H, V), dtype=np.float32)
    keep, init_p = _init_ptr(init_slot_ids, R // n_rows)
    rc = lib().kdao_step_f32(pool.ctypes.data, kind, n_slots, H, K, V,
                             _ptr(slot_ids, ctypes.c_int32), init_p, R // n_rows, n_rows,
                             _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                             _ptr(v, ctypes.c_float), _ptr(g, ctypes.c_float),
                             _ptr(b, ctypes.c_float), float(scale),
                             _ptr(out, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return out


def step_f64(pool: np.ndarray, slot_ids, q, k, v, g, b, n_rows: int = 1,
             scale: float | None = None, init_slot_ids=None) -> np.ndarray:
    """The same launch in fp64 on a float64 host pool, updated in place."""
    if pool.dtype != np.float64 or not pool.flags["C_CONTIGUOUS"]:
        raise TypeError("fp64 oracle pool must be a C-contiguous float64 array")
    (n_slots, H, K, V), slot_ids, q, k, v, g, b = _check_inputs(pool, slot_ids, q, k, v, g, b, n_rows)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    R = slot_ids.size
    out = np.zeros((R, H, V), dtype=np.float64)
    keep, init_p = _init_ptr(init_slot_ids, R // n_rows)
    rc = lib().kdao_step_f64(_ptr(pool, ctypes.c_double), n_slots, H, K, V,
                             _ptr(slot_ids, ctypes.c_int32), init_p, R // n_rows, n_rows,
                             _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float),
                             _ptr(v, ctypes.c_float), _ptr(g, ctypes.c_float),
                             _ptr(b, ctypes.c_float), float(scale),
                             _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return out


def _prefill_args(pool, init_slot_ids, dst_slot_ids, cu_seqlens, q, k, v, g, b):
    n_slots, H, K, V = pool.shape
    init = np.ascontiguousarray(init_slot_ids, dtype=np.int32).reshape(-1)
    n_seq = init.size
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32).reshape(-1)
    if cu.size != n_seq + 1:
        raise ValueError("cu_seqlens needs n_seq + 1 entries")
    dst = None if dst_slot_ids is None else np.ascontiguousarray(dst_slot_ids, dtype=np.int32).reshape(-1)
    if dst is not None and dst.size != n_seq:
        raise ValueError("dst_slot_ids needs one entry per sequence")
    T = int(cu[-1]) if n_seq else 0
    q, k, v, g, b = (_f32(x) for x in (q, k, v, g, b))
    if q.shape[0] < T or k.shape[0] < T or v.shape[0] < T or g.shape[0] < T or b.shape[0] < T:
        raise ValueError("q, k, v, g, b hold fewer tokens than cu_seqlens addresses")
    if q.shape[1:] != (H, K) or k.shape[1:] != (H, K) or g.shape[1:] != (H, K) \
            or v.shape[1:] != (H, V) or b.shape[1:] != (H,):
        raise ValueError("q, k, g [T, H, K]; v [T, H, V]; b [T, H]")
    return (n_slots, H, K, V), init, dst, cu, n_seq, q, k, v, g, b


def prefill_f32(pool: np.ndarray, init_slot_ids, cu_seqlens, q, k, v, g, b, dst_slot_ids=None,
                scale: float | None = None, bf16: bool = False) -> np.ndarray:
    """Prefill in fp32 on a host pool (float32, or uint16 fp16 / bf16 bits),
    updated in place with each sequence's final state.  Returns out [T, H, V]
    (rows past cu_seqlens[-1], if any, stay zero)."""
    if not pool.flags["C_CONTIGUOUS"]:
        raise ValueError("pool must be C-contiguous")
    kind = POOL_F32 if pool.dtype == np.float32 else (POOL_BF16 if bf16 else POOL_F16)
    if pool.dtype not in (np.float32, np.uint16):
        raise TypeError("oracle pool must be float32 or uint16")
    (n_slots, H, K, V), init, dst, cu, n_seq, q, k, v, g, b = _prefill_args(
        pool, init_slot_ids, dst_slot_ids, cu_seqlens, q, k, v, g, b)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    out = np.zeros((q.shape[0], H, V), dtype=np.float32)
    rc = lib().kdao_prefill_f32(pool.ctypes.data, kind, n_slots, H, K, V, _ptr(init, ctypes.c_int32),
                                None if dst is None else _ptr(dst, ctypes.c_int32),
                                _ptr(cu, ctypes.c_int32), n_seq, _ptr(q, ctypes.c_float),
                                _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                                _ptr(g, ctypes.c_float), _ptr(b, ctypes.c_float), float(scale),
                                _ptr(out, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return out


def prefill_f64(pool: np.ndarray, init_slot_ids, cu_seqlens, q, k, v, g, b, dst_slot_ids=None,
                scale: float | None = None) -> np.ndarray:
    """The same prefill in fp64 on a float64 host pool, updated in place."""
    if pool.dtype != np.float64 or not pool.flags["C_CONTIGUOUS"]:
        raise TypeError("fp64 oracle pool must be a C-contiguous float64 array")
    (n_slots, H, K, V), init, dst, cu, n_seq, q, k, v, g, b = _prefill_args(
        pool, init_slot_ids, dst_slot_ids, cu_seqlens, q, k, v, g, b)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    out = np.zeros((q.shape[0], H, V), dtype=np.float64)
    rc = lib().kdao_prefill_f64(_ptr(pool, ctypes.c_double), n_slots, H, K, V,
                                _ptr(init, ctypes.c_int32),
                                None if dst is None else _ptr(dst, ctypes.c_int32),
                                _ptr(cu, ctypes.c_int32), n_seq, _ptr(q, ctypes.c_float),
                                _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                                _ptr(g, ctypes.c_float), _ptr(b, ctypes.c_float), float(scale),
                                _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return out


def conv_f32(conv_pool: np.ndarray, slot_ids, x, w, n_rows: int = 1,
             init_slot_ids=None) -> np.ndarray:
    """Short causal convolution + SiLU over a host conv pool [n_slots, 3, C]
    of bfloat16 bits (uint16), updated in place with each row's history
    snapshot.  x: [R, C] fp32, w: [C, 4] fp32.  Returns y [R, C] fp32."""
    if conv_pool.dtype != np.uint16 or conv_pool.ndim != 3 or conv_pool.shape[1] != 3 \
            or not conv_pool.flags["C_CONTIGUOUS"]:
        raise TypeError("conv pool must be a C-contiguous uint16 [n_slots, 3, C] array")
    n_slots, _, C = conv_pool.shape
    slot_ids = np.ascontiguousarray(slot_ids, dtype=np.int32).reshape(-1)
    R = slot_ids.size
    x = _f32(x).reshape(R, C)
    w = _f32(w).reshape(C, 4)
    y = np.zeros((R, C), dtype=np.float32)
    keep, init_p = _init_ptr(init_slot_ids, R // n_rows)
    rc = lib().kdao_conv_f32(_ptr(conv_pool, ctypes.c_uint16), n_slots, C,
                             _ptr(slot_ids, ctypes.c_int32), init_p, R // n_rows, n_rows,
                             _ptr(x, ctypes.c_float), _ptr(w, ctypes.c_float), _ptr(y, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return y


def log_decay_from_gate(x) -> np.ndarray:
    """The log-decay g = -softplus(x) = -log(1 + e^x) of a raw gate x, taken
    in fp64 in the overflow-free form -(max(x, 0) + log1p(e^-|x|)) and
    rounded to fp32: the decay input of the step (a = e^g) when the fused
    front end is given the raw gate (ROCm/ATOM PR #2894, the two-node trial:
    the gate is computed inside the fused front end).  Test infrastructure,
    like the rest of this module."""
    x = np.asarray(x, dtype=np.float64)
    return (-(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))).astype(np.float32)


def set_mutation(which: int) -> None:
    """Plant one mistake in the oracle (tests of the pins only); 0 clears."""
    lib().kdao_set_mutation(int(which))
