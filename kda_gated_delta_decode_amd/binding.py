"""Python binding of the KDA decode C ABI (include/kda_decode.h).

Argument marshalling only: every entry point here turns torch tensors (for
device buffers), NumPy arrays (for host tables) and Python numbers into the
C call of the same name, and raises KdaError on a non-zero status.  All
arithmetic of the decode update runs in the library's gfx950 kernels; there
is no fallback path.  If libkda_decode.so has not been built, the first call
raises ImportError.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda_decode.so")

# kda_dtype
KDA_F32 = 0
KDA_F16 = 1
KDA_BF16 = 2
_UNKNOWN_DTYPE = 99  # what a dtype the ABI does not name is passed as

# kda_status
KDA_OK = 0
KDA_ERR_NULL = 1
KDA_ERR_DTYPE_REFUSED = 2
KDA_ERR_DTYPE_MISMATCH = 3
KDA_ERR_SHAPE = 4
KDA_ERR_ROWS = 5
KDA_ERR_SLOT = 6
KDA_ERR_ALIGN = 7
KDA_ERR_ARG = 8
KDA_ERR_LAUNCH = 9

KDA_HEAD_K = 128
KDA_HEAD_V = 128
KDA_MAX_ROWS = 8
KDA_ROWS_DEFAULT = 0
KDA_ROWS_K_SPLIT = 1
KDA_ROWS_WAVE_K = 2
KDA_ROWS_MATRIX = 3
KDA_NOALLOC_MAX_PAIRS = 4096  # pair counters of kda_decode_step_conv_noalloc
KDA_PROBE_COPY = 0
KDA_PROBE_READ = 1
KDA_PROBE_WRITE = 2


class kda_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("n_slots", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int)]


class kda_conv_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("n_slots", ctypes.c_int32), ("H", ctypes.c_int32)]


class kda_launch_opts(ctypes.Structure):
    _fields_ = [("waves_per_tile", ctypes.c_int32), ("bv", ctypes.c_int32),
                ("block_rows", ctypes.c_int32), ("rows_layout", ctypes.c_int32),
                ("g_raw", ctypes.c_int32)]


class kda_prefill_opts(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32)]


class kda_launch_desc(ctypes.Structure):
    _fields_ = [("bv", ctypes.c_int32), ("waves_per_tile", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("tiles", ctypes.c_int32),
                ("blocks", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("kernel", ctypes.c_char_p), ("rows_layout", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = int(code)
        super().__init__("%s: %s (code %d)" % (where, kda_strerror(code), code))


# The C symbols and their signatures, as include/kda_decode.h declares them.
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
SIGNATURES = {
    "kda_decode_step": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _P, _P, _P, _P, _P,
                                       _I32, _I32, ctypes.c_int, ctypes.c_float, _P]),
    "kda_decode_step_ex": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _P, _P, _P, _P, _P,
                                          _P, _I32, _I32, ctypes.c_int, ctypes.c_float,
                                          ctypes.POINTER(kda_launch_opts), _P]),
    "kda_decode_step_conv": (ctypes.c_int, [ctypes.POINTER(kda_pool), ctypes.POINTER(kda_conv_pool),
                                            _P, _P, _P, _P, _P, _P, _P, _I32, _I32, ctypes.c_int,
                                            ctypes.c_float, ctypes.POINTER(kda_launch_opts), _P]),
    "kda_decode_step_conv_ws": (ctypes.c_int, [ctypes.POINTER(kda_pool), ctypes.POINTER(kda_conv_pool),
                                               _P, _P, _P, _P, _P, _P, _P, _I32, _I32, ctypes.c_int,
                                               ctypes.c_float, _P, _I32, ctypes.POINTER(kda_launch_opts),
                                               _P]),
    "kda_decode_step_conv_noalloc": (ctypes.c_int, [ctypes.POINTER(kda_pool), ctypes.POINTER(kda_conv_pool),
                                                    _P, _P, _P, _P, _P, _P, _P, _I32, _I32, ctypes.c_int,
                                                    ctypes.c_float, ctypes.POINTER(kda_launch_opts), _P]),
    "kda_validate": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _I32, _I32, ctypes.c_int]),
    "kda_state_copy": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _I32, ctypes.c_int, _P]),
    "kda_prefill": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _I32, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                   ctypes.POINTER(kda_prefill_opts), _P]),
    "kda_prefill_validate": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _P, _I32,
                                            ctypes.c_int64, ctypes.c_int]),
    "kda_state_at": (ctypes.c_int64, [ctypes.POINTER(kda_pool), _P, _I32, _I32, _I32]),
    "kda_pool_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, ctypes.c_int]),
    "kda_tile_bv": (_I32, [ctypes.c_int]),
    "kda_describe_launch": (ctypes.c_int, [_I32, _I32, _I32, ctypes.c_int,
                                           ctypes.POINTER(kda_launch_opts),
                                           ctypes.POINTER(kda_launch_desc)]),
    "kda_tile_of_block": (_I32, [_I32, _I32]),
    "kda_copy_probe": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "kda_bw_probe": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _I32, _I32, _I32, _P]),
    "kda_tile_probe": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _I32, ctypes.c_int, _P]),
    "kda_rows_probe": (ctypes.c_int, [ctypes.POINTER(kda_pool), _P, _P, _I32, _I32, _I32, _I32, ctypes.c_int,
                                      _P]),
    "kda_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_abi_version": (ctypes.c_int, []),
}

_lib = None


def library() -> ctypes.CDLL:
    """The loaded libkda_decode.so (ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkda_decode.so is not built at %s; build it with "
                          "`python -m kda_gated_delta_decode_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def dtype_code(torch_dtype) -> int:
    import torch
    if torch_dtype == torch.float32:
        return KDA_F32
    if torch_dtype == torch.float16:
        return KDA_F16
    if torch_dtype == torch.bfloat16:
        return KDA_BF16
    return _UNKNOWN_DTYPE


def _dtype_arg(d) -> int:
    if isinstance(d, (int, np.integer)):
        return int(d)
    if isinstance(d, str):
        return {"f32": KDA_F32, "fp32": KDA_F32, "float32": KDA_F32, "f16": KDA_F16,
                "fp16": KDA_F16, "float16": KDA_F16, "bf16": KDA_BF16,
                "bfloat16": KDA_BF16}.get(d, _UNKNOWN_DTYPE)
    return dtype_code(d)


def _on_gpu(t, name):
    """The library takes device addresses only: a host tensor's pointer
    would reach a kernel as a wild address, so it is refused here."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise TypeError("%s must be a GPU tensor, got one on %s" % (name, t.device))


def make_pool(pool, dtype=None) -> kda_pool:
    """kda_pool describing a device tensor [n_slots, H, K, V] (contiguous).
    `dtype` overrides the element type the struct declares (default: the
    tensor's own)."""
    _on_gpu(pool, "pool")
    if not pool.is_contiguous():
        raise ValueError("pool must be contiguous [n_slots, H, K, V]")
    if pool.dim() != 4:
        raise ValueError("pool must be 4-D [n_slots, H, K, V]")
    n_slots, H, K, V = pool.shape
    code = dtype_code(pool.dtype) if dtype is None else _dtype_arg(dtype)
    return kda_pool(ctypes.c_void_p(pool.data_ptr()), n_slots, H, K, V, code)


def _dev(t, name, dtype=None, device=None):
    """The device address of tensor t (None passes through as NULL).  t must
    be a contiguous GPU tensor, of `dtype` if given and on the same device
    as `device` (the pool) if given."""
    if t is None:
        return None
    _on_gpu(t, name)
    if device is not None and t.device != device:
        raise TypeError("%s is on %s, the pool on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _need_numel(t, name, n):
    """The library cannot see tensor sizes: refuse a tensor that holds fewer
    (or more) elements than the launch will address."""
    if t is not None and t.numel() != n:
        raise ValueError("%s holds %d elements, the launch addresses %d" % (name, t.numel(), n))


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(code: int, where: str) -> None:
    if code != KDA_OK:
        raise KdaError(code, where)


# ---------------------------------------------------------------------------
# the entry points
# ---------------------------------------------------------------------------

def kda_decode_step(pool, slot_ids, q, k, v, g, b, out, n_rows_per_slot: int = 1,
                    state_dtype=None, scale: float | None = None, stream=None,
                    waves_per_tile: int = 0, bv: int = 0, pool_dtype=None,
                    init_slot_ids=None, block_rows: bool = False, rows_layout: int = 0) -> None:
    """One decode launch (see kda_decode_step in include/kda_decode.h).

    pool: device tensor [n_slots, H, 128, 128], float32 or float16, updated
    in place.  slot_ids: device int32 [R]; q, k, g: device float32 [R, H, 128];
    v, out: [R, H, 128]; b: [R, H].  state_dtype defaults to the pool's
    dtype; pool_dtype overrides what the pool struct declares (tests of the
    refusals).  init_slot_ids (device int32 [n_req]) reads each request's
    initial state from that slot; block_rows takes chained rows as one block
    instead of one after the other; rows_layout picks the chained-row layout
    (KDA_ROWS_K_SPLIT, KDA_ROWS_WAVE_K or KDA_ROWS_MATRIX); any of these, or a non-zero
    waves_per_tile or bv, selects kda_decode_step_ex."""
    import torch
    P = make_pool(pool, pool_dtype)
    dv = pool.device
    sd = P.dtype if state_dtype is None else _dtype_arg(state_dtype)
    R = slot_ids.numel()
    if R % n_rows_per_slot != 0:
        raise ValueError("slot_ids holds %d rows, not a multiple of %d" % (R, n_rows_per_slot))
    n_req = R // n_rows_per_slot
    if scale is None:
        scale = 1.0 / math.sqrt(pool.shape[2])
    H = pool.shape[1]
    for t, name, n in ((q, "q", R * H * pool.shape[2]), (k, "k", R * H * pool.shape[2]),
                       (g, "g", R * H * pool.shape[2]), (v, "v", R * H * pool.shape[3]),
                       (out, "out", R * H * pool.shape[3]), (b, "b", R * H)):
        _need_numel(t, name, n)
    f32 = torch.float32
    rows = (_dev(q, "q", f32, dv), _dev(k, "k", f32, dv), _dev(v, "v", f32, dv),
            _dev(g, "g", f32, dv), _dev(b, "b", f32, dv), _dev(out, "out", f32, dv),
            n_req, n_rows_per_slot, sd, float(scale))
    ids = _dev(slot_ids, "slot_ids", torch.int32, dv)
    if waves_per_tile or bv or block_rows or rows_layout or init_slot_ids is not None:
        if init_slot_ids is not None and init_slot_ids.numel() != n_req:
            raise ValueError("init_slot_ids needs one entry per request")
        opts = kda_launch_opts(int(waves_per_tile), int(bv), int(bool(block_rows)), int(rows_layout))
        rc = library().kda_decode_step_ex(ctypes.byref(P), ids,
                                          _dev(init_slot_ids, "init_slot_ids", torch.int32, dv), *rows,
                                          ctypes.byref(opts), _stream_ptr(stream))
        _check(rc, "kda_decode_step_ex")
    else:
        rc = library().kda_decode_step(ctypes.byref(P), ids, *rows, _stream_ptr(stream))
        _check(rc, "kda_decode_step")


def make_conv_pool(conv) -> kda_conv_pool:
    """kda_conv_pool describing a device tensor [n_slots, 3, 3, H, 128] of
    bfloat16 (the history of q | k | v)."""
    import torch
    if conv.dtype != torch.bfloat16 or not conv.is_contiguous() or conv.dim() != 5 \
            or tuple(conv.shape[1:3]) != (3, 3) or conv.shape[4] != KDA_HEAD_K:
        raise ValueError("conv pool must be a contiguous bfloat16 [n_slots, 3, 3, H, 128] tensor")
    return kda_conv_pool(ctypes.c_void_p(conv.data_ptr()), conv.shape[0], conv.shape[3])


def conv_pair_counts(n_req: int, H: int, device):
    """Zeroed pair counters for kda_decode_step_conv(pair_counts=...): one
    int32 per (request, head) of the largest launch they serve.  Launches
    leave them even, so one buffer serves any number of launches in a row,
    but not launches that may overlap (another stream, a concurrent graph)."""
    import torch
    return torch.zeros(int(n_req) * int(H), dtype=torch.int32, device=device)


def kda_decode_step_conv(pool, conv, slot_ids, x, conv_w, g, b, out, n_rows_per_slot: int = 1,
                         state_dtype=None, scale: float | None = None, stream=None,
                         init_slot_ids=None, waves_per_tile: int = 0, bv: int = 0,
                         block_rows: bool = False, rows_layout: int = 0, pair_counts=None,
                         g_raw: bool = False) -> None:
    """Decode step with the short causal convolution fused in front (see
    kda_decode_step_conv in include/kda_decode.h).  conv: bfloat16 history
    [n_slots, 3, 3, H, 128]; x: fp32 raw q|k|v [R, 3, H, 128]; conv_w: fp32
    taps [3, H, 128, 4]; pair_counts: None, or device int32 counters from
    conv_pair_counts (kda_decode_step_conv_ws: chained rows then take
    64-column halves); g_raw: g holds the raw gate x, the log-decay being
    -softplus(x); the other arguments as kda_decode_step."""
    _conv_step(pool, conv, slot_ids, x, conv_w, g, b, out, n_rows_per_slot, state_dtype, scale, stream,
               init_slot_ids, waves_per_tile, bv, block_rows, rows_layout, pair_counts, False, g_raw)


def kda_decode_step_conv_noalloc(pool, conv, slot_ids, x, conv_w, g, b, out, n_rows_per_slot: int = 1,
                                 state_dtype=None, scale: float | None = None, stream=None,
                                 init_slot_ids=None, waves_per_tile: int = 0, bv: int = 0,
                                 block_rows: bool = False, rows_layout: int = 0, g_raw: bool = False) -> None:
    """kda_decode_step_conv with the library's own pair counters (see
    kda_decode_step_conv_noalloc in include/kda_decode.h): allocates nothing;
    at most KDA_NOALLOC_MAX_PAIRS requests x heads; calls that overlap on one
    GPU race."""
    _conv_step(pool, conv, slot_ids, x, conv_w, g, b, out, n_rows_per_slot, state_dtype, scale, stream,
               init_slot_ids, waves_per_tile, bv, block_rows, rows_layout, None, True, g_raw)


def _conv_step(pool, conv, slot_ids, x, conv_w, g, b, out, n_rows_per_slot, state_dtype, scale, stream,
               init_slot_ids, waves_per_tile, bv, block_rows, rows_layout, pair_counts, noalloc, g_raw):
    import torch
    P = make_pool(pool)
    Cv = make_conv_pool(conv)
    dv = pool.device
    sd = P.dtype if state_dtype is None else _dtype_arg(state_dtype)
    R = slot_ids.numel()
    if R % n_rows_per_slot != 0:
        raise ValueError("slot_ids holds %d rows, not a multiple of %d" % (R, n_rows_per_slot))
    n_req = R // n_rows_per_slot
    if scale is None:
        scale = 1.0 / math.sqrt(pool.shape[2])
    H = pool.shape[1]
    for t, name, n in ((x, "x", R * 3 * H * KDA_HEAD_K), (conv_w, "conv_w", 3 * H * KDA_HEAD_K * 4),
                       (g, "g", R * H * KDA_HEAD_K), (out, "out", R * H * KDA_HEAD_K),
                       (b, "b", R * H), (init_slot_ids, "init_slot_ids", n_req)):
        _need_numel(t, name, n)
    opts = kda_launch_opts(int(waves_per_tile), int(bv), int(bool(block_rows)), int(rows_layout),
                           int(bool(g_raw)))
    args = (ctypes.byref(P), ctypes.byref(Cv), _dev(slot_ids, "slot_ids", torch.int32, dv),
            _dev(init_slot_ids, "init_slot_ids", torch.int32, dv), _dev(x, "x", torch.float32, dv),
            _dev(conv_w, "conv_w", torch.float32, dv), _dev(g, "g", torch.float32, dv),
            _dev(b, "b", torch.float32, dv), _dev(out, "out", torch.float32, dv), n_req,
            n_rows_per_slot, sd, float(scale))
    if noalloc:
        rc = library().kda_decode_step_conv_noalloc(*args, ctypes.byref(opts), _stream_ptr(stream))
        _check(rc, "kda_decode_step_conv_noalloc")
    elif pair_counts is None:
        rc = library().kda_decode_step_conv(*args, ctypes.byref(opts), _stream_ptr(stream))
        _check(rc, "kda_decode_step_conv")
    else:
        rc = library().kda_decode_step_conv_ws(*args, _dev(pair_counts, "pair_counts", torch.int32, dv),
                                               pair_counts.numel(), ctypes.byref(opts), _stream_ptr(stream))
        _check(rc, "kda_decode_step_conv_ws")


def kda_prefill(pool, init_slot_ids, cu_seqlens, q, k, v, g, b, out, dst_slot_ids=None,
                state_dtype=None, scale: float | None = None, chunk: int = 0, stream=None) -> None:
    """Chunked prefill (see kda_prefill in include/kda_decode.h).  pool: device
    tensor [n_slots, H, 128, 128]; init_slot_ids, dst_slot_ids (optional):
    device int32 [n_seq]; cu_seqlens: device int32 [n_seq + 1]; q, k, g, v,
    out: device float32 [T, H, 128]; b: [T, H]."""
    import torch
    P = make_pool(pool)
    dv = pool.device
    sd = P.dtype if state_dtype is None else _dtype_arg(state_dtype)
    n_seq = init_slot_ids.numel()
    H = pool.shape[1]
    T = q.shape[0]
    for t, name, n in ((cu_seqlens, "cu_seqlens", n_seq + 1), (dst_slot_ids, "dst_slot_ids", n_seq),
                       (q, "q", T * H * KDA_HEAD_K), (k, "k", T * H * KDA_HEAD_K),
                       (g, "g", T * H * KDA_HEAD_K), (v, "v", T * H * KDA_HEAD_V),
                       (out, "out", T * H * KDA_HEAD_V), (b, "b", T * H)):
        _need_numel(t, name, n)
    if scale is None:
        scale = 1.0 / math.sqrt(pool.shape[2])
    opts = kda_prefill_opts(int(chunk))
    rc = library().kda_prefill(ctypes.byref(P), _dev(init_slot_ids, "init_slot_ids", torch.int32, dv),
                               _dev(dst_slot_ids, "dst_slot_ids", torch.int32, dv),
                               _dev(cu_seqlens, "cu_seqlens", torch.int32, dv),
                               _dev(q, "q", torch.float32, dv), _dev(k, "k", torch.float32, dv),
                               _dev(v, "v", torch.float32, dv), _dev(g, "g", torch.float32, dv),
                               _dev(b, "b", torch.float32, dv), _dev(out, "out", torch.float32, dv),
                               n_seq, T, sd, float(scale), ctypes.byref(opts), _stream_ptr(stream))
    _check(rc, "kda_prefill")


def kda_prefill_validate(pool_desc: kda_pool, init_slot_ids_host, cu_seqlens_host, n_tokens: int,
                         state_dtype, dst_slot_ids_host=None) -> int:
    """Host-side check of a prefill's tables; returns the kda_status code."""
    init = np.ascontiguousarray(init_slot_ids_host, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    dst = None if dst_slot_ids_host is None else np.ascontiguousarray(dst_slot_ids_host, dtype=np.int32)
    if cu.size != init.size + 1 or (dst is not None and dst.size != init.size):
        raise ValueError("cu_seqlens needs n_seq + 1 entries, dst_slot_ids n_seq")
    return int(library().kda_prefill_validate(
        ctypes.byref(pool_desc), init.ctypes.data_as(ctypes.c_void_p),
        None if dst is None else dst.ctypes.data_as(ctypes.c_void_p),
        cu.ctypes.data_as(ctypes.c_void_p), init.size, int(n_tokens), _dtype_arg(state_dtype)))


def kda_validate(pool_desc: kda_pool, slot_ids_host, n_req: int, n_rows: int, state_dtype,
                 init_slot_ids_host=None) -> int:
    """Host-side validation; returns the kda_status code (0 = OK)."""
    ids = np.ascontiguousarray(slot_ids_host, dtype=np.int32)
    init = None if init_slot_ids_host is None else np.ascontiguousarray(init_slot_ids_host, dtype=np.int32)
    return int(library().kda_validate(ctypes.byref(pool_desc), ids.ctypes.data_as(ctypes.c_void_p),
                                      None if init is None else init.ctypes.data_as(ctypes.c_void_p),
                                      n_req, n_rows, _dtype_arg(state_dtype)))


def kda_state_copy(pool, src_slot_ids, dst_slot_ids, state_dtype=None, stream=None) -> None:
    """Copy whole slots: pool[dst[i]] = pool[src[i]] (device int32 id tensors)."""
    import torch
    P = make_pool(pool)
    dv = pool.device
    sd = P.dtype if state_dtype is None else _dtype_arg(state_dtype)
    n = src_slot_ids.numel()
    if dst_slot_ids.numel() != n:
        raise ValueError("src and dst slot tables differ in length")
    _check(library().kda_state_copy(ctypes.byref(P), _dev(src_slot_ids, "src_slot_ids", torch.int32, dv),
                                    _dev(dst_slot_ids, "dst_slot_ids", torch.int32, dv), n, sd,
                                    _stream_ptr(stream)), "kda_state_copy")


def kda_state_at(pool_desc: kda_pool, slot_ids_host, n_rows: int, req: int, row: int) -> int:
    """Element offset of the [H, K, V] block of (req, row); negative status on error."""
    ids = np.ascontiguousarray(slot_ids_host, dtype=np.int32)
    return int(library().kda_state_at(ctypes.byref(pool_desc), ids.ctypes.data_as(ctypes.c_void_p),
                                      n_rows, req, row))


def kda_pool_bytes(n_slots: int, H: int, K: int, V: int, dtype) -> int:
    return int(library().kda_pool_bytes(n_slots, H, K, V, _dtype_arg(dtype)))


def kda_tile_bv(dtype) -> int:
    return int(library().kda_tile_bv(_dtype_arg(dtype)))


def kda_describe_launch(n_req: int, n_rows: int, H: int, dtype, waves_per_tile: int = 0,
                        bv: int = 0, block_rows: bool = False, rows_layout: int = 0) -> dict:
    d = kda_launch_desc()
    opts = kda_launch_opts(int(waves_per_tile), int(bv), int(bool(block_rows)), int(rows_layout))
    _check(library().kda_describe_launch(n_req, n_rows, H, _dtype_arg(dtype), ctypes.byref(opts),
                                         ctypes.byref(d)), "kda_describe_launch")
    return {"bv": d.bv, "waves_per_tile": d.waves_per_tile, "threads": d.threads,
            "tiles": d.tiles, "blocks": d.blocks, "lds_bytes": d.lds_bytes,
            "kernel": d.kernel.decode(), "rows_layout": d.rows_layout}


def kda_tile_of_block(block: int, n_blocks: int) -> int:
    return int(library().kda_tile_of_block(block, n_blocks))


def kda_copy_probe(dst, src, nbytes: int | None = None, stream=None) -> None:
    """Device-to-device streaming copy of nbytes (default: all of src); nbytes
    may not exceed either tensor's size."""
    _on_gpu(dst, "dst")
    _on_gpu(src, "src")
    if dst.device != src.device:
        raise TypeError("dst is on %s, src on %s" % (dst.device, src.device))
    nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    cap = min(src.numel() * src.element_size(), dst.numel() * dst.element_size())
    if nb < 0 or nb > cap:
        raise ValueError("nbytes %d outside [0, %d], the smaller buffer's size" % (nb, cap))
    _check(library().kda_copy_probe(_dev(dst, "dst"), _dev(src, "src"), nb, _stream_ptr(stream)),
           "kda_copy_probe")


def kda_bw_probe(dst, src, nbytes: int, mode: int = KDA_PROBE_COPY, vectors_per_thread: int = 1,
                 nontemporal: bool = True, stream=None) -> None:
    """Streaming bandwidth probe over nbytes (see kda_bw_probe in
    include/kda_decode.h): copy src -> dst, read src only, or write dst
    only.  nbytes may not exceed the buffers it reads or writes (dst: 16
    bytes for a read-only probe)."""
    _on_gpu(dst, "dst")
    nb = int(nbytes)
    dst_need = 16 if mode == KDA_PROBE_READ else nb
    if nb < 0 or dst.numel() * dst.element_size() < dst_need:
        raise ValueError("dst holds fewer than the %d bytes the probe writes" % dst_need)
    if mode != KDA_PROBE_WRITE:
        _on_gpu(src, "src")
        if src.device != dst.device:
            raise TypeError("dst is on %s, src on %s" % (dst.device, src.device))
        if src.numel() * src.element_size() < nb:
            raise ValueError("src holds fewer than the %d bytes the probe reads" % nb)
    _check(library().kda_bw_probe(_dev(dst, "dst"), None if mode == KDA_PROBE_WRITE else _dev(src, "src"),
                                  nb, int(mode), int(vectors_per_thread), int(bool(nontemporal)),
                                  _stream_ptr(stream)), "kda_bw_probe")


def kda_tile_probe(pool, slot_ids, stream=None) -> None:
    """The single-row decode launch's state traffic without its arithmetic
    (see kda_tile_probe in include/kda_decode.h): each request's tiles of
    slot slot_ids[r] are read and written back unchanged."""
    import torch
    P = make_pool(pool)
    n_req = slot_ids.numel()
    _check(library().kda_tile_probe(ctypes.byref(P), _dev(slot_ids, "slot_ids", torch.int32, pool.device),
                                    n_req, P.dtype, _stream_ptr(stream)), "kda_tile_probe")


def kda_rows_probe(pool, slot_ids, n_rows: int, init_slot_ids=None, tile_cols: int = 0, waves: int = 0,
                   stream=None) -> None:
    """The chained-row launch's state traffic (matrix-core block form)
    without its arithmetic (see kda_rows_probe in include/kda_decode.h): each
    request's initial state is written unchanged to its rows' slots.
    tile_cols, waves: 0, 0 for the block form's 64 columns over 8 waves, or
    32 / 128 over 8, or 128 over 16."""
    import torch
    P = make_pool(pool)
    n_rows = int(n_rows)
    if n_rows < 1 or slot_ids.numel() % n_rows:
        raise ValueError("slot_ids holds %d ids, not a multiple of n_rows = %d" % (slot_ids.numel(), n_rows))
    n_req = slot_ids.numel() // n_rows
    if init_slot_ids is not None:
        _need_numel(init_slot_ids, "init_slot_ids", n_req)
    dv = pool.device
    _check(library().kda_rows_probe(ctypes.byref(P), _dev(slot_ids, "slot_ids", torch.int32, dv),
                                    _dev(init_slot_ids, "init_slot_ids", torch.int32, dv), n_req, n_rows,
                                    int(tile_cols), int(waves), P.dtype, _stream_ptr(stream)), "kda_rows_probe")


def kda_strerror(code: int) -> str:
    return library().kda_strerror(int(code)).decode()


def kda_abi_version() -> int:
    return int(library().kda_abi_version())
