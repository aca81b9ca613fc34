"""C-ABI tests that need no GPU: the library loads, exports every function
include/kda_decode.h declares, and refuses bad calls on the host before any
HIP call (ROCm/ATOM PR #2945, Changes and Testing: bf16 refused, a pool of
the other dtype refused, every build key carries the dtype)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda_decode.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

K = pytest.importorskip("kda_gated_delta_decode_amd")
from kda_gated_delta_decode_amd import binding as B  # noqa: E402

FAKE = 0x10000   # an aligned non-null address: only ever passed to calls that
                 # the host validation refuses, so it is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(kda_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_abi():
    names = declared_functions()
    for expected in ["kda_decode_step", "kda_decode_step_ex", "kda_validate", "kda_state_at",
                     "kda_state_copy", "kda_decode_step_conv", "kda_decode_step_conv_ws",
                     "kda_decode_step_conv_noalloc", "kda_prefill",
                     "kda_prefill_validate",
                     "kda_pool_bytes", "kda_tile_bv", "kda_describe_launch", "kda_tile_of_block",
                     "kda_copy_probe", "kda_bw_probe", "kda_tile_probe", "kda_rows_probe",
                     "kda_strerror",
                     "kda_abi_version"]:
        assert expected in names


def test_library_exports_every_declared_symbol():
    lib = B.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in B.SIGNATURES, "binding lacks a signature for %s" % name
    assert B.kda_abi_version() == 11


def pool(n_slots=96, H=12, Kd=128, V=128, dtype=B.KDA_F32, base=FAKE):
    return B.kda_pool(ctypes.c_void_p(base), n_slots, H, Kd, V, dtype)


def step(P, n_req=4, n_rows=1, state_dtype=None, scale=0.0883883, ptrs=None, opts=None, init=None):
    p = [FAKE] * 7 if ptrs is None else ptrs
    sd = P.dtype if state_dtype is None else state_dtype
    if opts is None and init is None:
        args = (ctypes.byref(P), *[ctypes.c_void_p(x) for x in p], n_req, n_rows, sd, scale)
        return B.library().kda_decode_step(*args, None)
    args = (ctypes.byref(P), ctypes.c_void_p(p[0]), ctypes.c_void_p(init),
            *[ctypes.c_void_p(x) for x in p[1:]], n_req, n_rows, sd, scale)
    return B.library().kda_decode_step_ex(*args, None if opts is None else ctypes.byref(opts), None)


def test_refusals_before_any_hip_call():
    assert step(pool(dtype=B.KDA_BF16)) == B.KDA_ERR_DTYPE_REFUSED
    assert step(pool(dtype=7)) == B.KDA_ERR_DTYPE_REFUSED
    assert step(pool(dtype=B.KDA_F16), state_dtype=B.KDA_F32) == B.KDA_ERR_DTYPE_MISMATCH
    assert step(pool(dtype=B.KDA_F32), state_dtype=B.KDA_F16) == B.KDA_ERR_DTYPE_MISMATCH
    assert step(pool(Kd=64)) == B.KDA_ERR_SHAPE
    assert step(pool(V=256)) == B.KDA_ERR_SHAPE
    assert step(pool(H=0)) == B.KDA_ERR_SHAPE
    assert step(pool(H=65536)) == B.KDA_ERR_SHAPE
    assert step(pool(), n_rows=0) == B.KDA_ERR_ROWS
    assert step(pool(), n_rows=9) == B.KDA_ERR_ROWS
    assert step(pool(), n_req=-1) == B.KDA_ERR_ARG
    assert step(pool(n_slots=10), n_req=3, n_rows=4) == B.KDA_ERR_SLOT
    assert step(pool(), scale=float("nan")) == B.KDA_ERR_ARG
    assert step(pool(), scale=float("inf")) == B.KDA_ERR_ARG
    assert step(pool(), opts=B.kda_launch_opts(3, 0)) == B.KDA_ERR_ARG
    assert step(pool(), opts=B.kda_launch_opts(0, 48)) == B.KDA_ERR_ARG
    assert step(pool(dtype=B.KDA_F16), opts=B.kda_launch_opts(0, 32)) == B.KDA_ERR_ARG
    assert step(pool(dtype=B.KDA_F16), opts=B.kda_launch_opts(1, 128)) == B.KDA_ERR_ARG  # spills
    # chained-row layouts: an unknown layout, the block form in the whole-K
    # layout, a whole-K shape with 1 lane per row piece or 1 wave
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(0, 0, 0, 4)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(0, 0, 0, -1)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(0, 0, 1, B.KDA_ROWS_WAVE_K)) == B.KDA_ERR_ARG
    # the block form with one wave is refused for fp16 pools (it would spill)
    assert step(pool(dtype=B.KDA_F16), n_rows=8, opts=B.kda_launch_opts(1, 64, 1)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(4, 16, 0, B.KDA_ROWS_WAVE_K)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(1, 16, 0, B.KDA_ROWS_WAVE_K)) == B.KDA_ERR_ARG
    # the matrix-core block form: 64 columns over 8 (default) or 4 waves
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(0, 32, 0, B.KDA_ROWS_MATRIX)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(2, 0, 0, B.KDA_ROWS_MATRIX)) == B.KDA_ERR_ARG
    # the raw gate belongs to the fused front end only
    assert step(pool(), opts=B.kda_launch_opts(0, 0, 0, 0, 1)) == B.KDA_ERR_ARG
    assert step(pool(), n_rows=8, opts=B.kda_launch_opts(0, 0, 0, B.KDA_ROWS_MATRIX, 1)) == B.KDA_ERR_ARG
    assert step(pool(base=FAKE + 4)) == B.KDA_ERR_ALIGN
    assert step(pool(), ptrs=[FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE]) == B.KDA_ERR_ALIGN
    assert step(pool(), ptrs=[FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE]) == B.KDA_ERR_ALIGN
    assert step(pool(), init=FAKE + 2) == B.KDA_ERR_ALIGN
    assert step(pool(dtype=B.KDA_BF16), init=FAKE) == B.KDA_ERR_DTYPE_REFUSED


@pytest.mark.parametrize("which", range(7))
def test_null_pointers_refused(which):
    ptrs = [FAKE] * 7
    ptrs[which] = 0
    assert step(pool(), ptrs=ptrs) == B.KDA_ERR_NULL
    assert step(pool(base=0)) == B.KDA_ERR_NULL
    assert B.library().kda_decode_step(None, *[ctypes.c_void_p(FAKE)] * 7, 1, 1, 0, 0.1, None) == B.KDA_ERR_NULL


def test_empty_launch_is_a_no_op():
    # n_req == 0 passes validation and returns before any HIP call; the row
    # buffers of an empty launch may be NULL
    assert step(pool(), n_req=0) == B.KDA_OK
    assert step(pool(dtype=B.KDA_F16), n_req=0, n_rows=8) == B.KDA_OK
    assert step(pool(), n_req=0, ptrs=[0] * 7) == B.KDA_OK
    assert step(pool(base=0), n_req=0) == B.KDA_ERR_NULL


def test_validate_initial_slots():
    P = pool(n_slots=10)
    ids = np.array([3, 1, 4, 0, 9, 2], dtype=np.int32)    # 3 requests x 2 rows
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[5, 6, 7]) == B.KDA_OK
    # a request may resume from one of its own snapshot slots ...
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[1, 4, 2]) == B.KDA_OK
    # ... and requests may share a read-only initial slot ...
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[5, 5, 5]) == B.KDA_OK
    # ... but not read a slot another request writes
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[4, 6, 7]) == B.KDA_ERR_SLOT
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[5, 6, 10]) == B.KDA_ERR_SLOT
    assert B.kda_validate(P, ids, 3, 2, B.KDA_F32, init_slot_ids_host=[-1, 6, 7]) == B.KDA_ERR_SLOT


def test_state_copy_refusals():
    L = B.library()
    P = pool(n_slots=10)
    f = ctypes.c_void_p(FAKE)
    assert L.kda_state_copy(ctypes.byref(P), f, f, 0, B.KDA_F32, None) == B.KDA_OK
    assert L.kda_state_copy(ctypes.byref(P), f, f, -1, B.KDA_F32, None) == B.KDA_ERR_ARG
    assert L.kda_state_copy(ctypes.byref(P), f, f, 70000, B.KDA_F32, None) == B.KDA_ERR_ARG
    assert L.kda_state_copy(ctypes.byref(P), None, f, 2, B.KDA_F32, None) == B.KDA_ERR_NULL
    assert L.kda_state_copy(ctypes.byref(P), f, f, 2, B.KDA_F16, None) == B.KDA_ERR_DTYPE_MISMATCH
    P16 = pool(n_slots=10, dtype=B.KDA_BF16)
    assert L.kda_state_copy(ctypes.byref(P16), f, f, 2, B.KDA_BF16, None) == B.KDA_ERR_DTYPE_REFUSED
    assert L.kda_state_copy(ctypes.byref(P), ctypes.c_void_p(FAKE + 1), f, 2, B.KDA_F32, None) == B.KDA_ERR_ALIGN


def test_validate_slot_table():
    P = pool(n_slots=10)
    ok = np.array([3, 1, 4, 0, 9, 2], dtype=np.int32)
    assert B.kda_validate(P, ok, 3, 2, B.KDA_F32) == B.KDA_OK
    assert B.kda_validate(P, np.array([3, 1, 3, 0], np.int32), 2, 2, B.KDA_F32) == B.KDA_ERR_SLOT
    assert B.kda_validate(P, np.array([3, 10], np.int32), 2, 1, B.KDA_F32) == B.KDA_ERR_SLOT
    assert B.kda_validate(P, np.array([-1, 2], np.int32), 2, 1, B.KDA_F32) == B.KDA_ERR_SLOT
    assert B.kda_validate(P, ok, 3, 2, B.KDA_BF16) == B.KDA_ERR_DTYPE_REFUSED
    assert B.kda_validate(P, ok, 3, 2, B.KDA_F16) == B.KDA_ERR_DTYPE_MISMATCH
    assert B.library().kda_validate(ctypes.byref(P), None, None, 3, 2, 0) == B.KDA_ERR_NULL


def test_state_at_addresses_initial_and_snapshot_slots():
    # ROCm/ATOM PR #2945, Changes: one address function for the initial
    # state (row 0) and every row's snapshot slot.
    P = pool(n_slots=96, H=12)
    ids = np.arange(64, dtype=np.int32)[::-1].copy()   # 8 requests x 8 rows
    block = 12 * 128 * 128
    for req in range(8):
        for row in range(8):
            assert B.kda_state_at(P, ids, 8, req, row) == int(ids[req * 8 + row]) * block
    assert B.kda_state_at(P, ids, 8, 0, 8) == -B.KDA_ERR_ARG
    assert B.kda_state_at(P, ids, 9, 0, 0) == -B.KDA_ERR_ROWS
    bad = ids.copy()
    bad[5] = 96
    assert B.kda_state_at(P, bad, 8, 0, 5) == -B.KDA_ERR_SLOT


def test_pool_sizing_matches_the_pages_memory_table():
    gold = json.load(open(os.path.join(GOLDEN, "pages_memory_table.json")))
    L, H, Kd, V = gold["layers"], gold["H"], gold["K"], gold["V"]
    f32 = L * B.kda_pool_bytes(1, H, Kd, V, "f32")
    f16 = L * B.kda_pool_bytes(1, H, Kd, V, "f16")
    diff_mb = gold["state_per_slot_MB"]["f32"] - gold["state_per_slot_MB"]["f16"]
    assert abs((f32 - f16) / 1e6 - diff_mb) <= 2 * gold["printed_precision_MB"]
    # what is left is the same for both dtypes (the conv state)
    rest32 = gold["state_per_slot_MB"]["f32"] - f32 / 1e6
    rest16 = gold["state_per_slot_MB"]["f16"] - f16 / 1e6
    assert abs(rest32 - rest16) <= 2 * gold["printed_precision_MB"]
    # 64-slot pools, in GiB
    for dt in ("f32", "f16"):
        gib = 64 * gold["state_per_slot_MB"][dt] * 1e6 / 2 ** 30
        assert abs(gib - gold["state_pool_64_slots_GB"][dt]) < 0.006
    assert B.kda_pool_bytes(64, 12, 128, 128, "bf16") == 0
    assert B.kda_pool_bytes(-1, 12, 128, 128, "f32") == 0


def test_pages_tile_widths_are_supported_shapes():
    # The pages' portable kernel caps the V block at 32 columns for a 4-byte
    # state and 64 for a 2-byte one; both widths are launchable here (their
    # tile row is one 128-byte line), though the default tile is wider.
    gold = json.load(open(os.path.join(GOLDEN, "pages_tiling.json")))
    for dt in ("f32", "f16"):
        bv = gold["bv_cap"][dt]
        d = B.kda_describe_launch(64, 1, 12, dt, waves_per_tile=1, bv=bv)
        assert d["bv"] == bv and d["tiles"] == 64 * 12 * (128 // bv)
        assert bv * (4 if dt == "f32" else 2) == 128
    assert B.kda_tile_bv("f32") == 128 and B.kda_tile_bv("f16") == 64
    assert B.kda_tile_bv("bf16") == -B.KDA_ERR_DTYPE_REFUSED


@pytest.mark.parametrize("n", [1, 7, 8, 9, 96, 192, 1536, 3072, 3073, 12345])
def test_block_to_tile_map_is_a_bijection(n):
    tiles = [B.kda_tile_of_block(b, n) for b in range(n)]
    assert sorted(tiles) == list(range(n))
    # the blocks of one XCD (b % 8 equal) hold consecutive tiles
    for x in range(min(8, n)):
        mine = [tiles[b] for b in range(x, n, 8)]
        assert mine == list(range(mine[0], mine[0] + len(mine)))
    assert B.kda_tile_of_block(n, n) == -1


SHAPES_F32 = {(32, 1), (32, 2), (32, 4), (32, 8), (64, 1), (64, 2), (64, 4), (64, 8),
              (128, 2), (128, 4), (128, 8)}
SHAPES_F16 = {(64, 1), (64, 2), (64, 4), (64, 8), (128, 2), (128, 4), (128, 8)}


@pytest.mark.parametrize("dtype,shapes", [("f32", SHAPES_F32), ("f16", SHAPES_F16)])
def test_supported_launch_shapes(dtype, shapes):
    got = set()
    for bv in (16, 32, 48, 64, 128, 256):
        for w in (1, 2, 3, 4, 8, 16):
            try:
                d = B.kda_describe_launch(64, 1, 12, dtype, waves_per_tile=w, bv=bv)
            except B.KdaError as e:
                assert e.code == B.KDA_ERR_ARG
                continue
            assert (d["bv"], d["waves_per_tile"]) == (bv, w)
            assert d["tiles"] == 64 * 12 * (128 // bv)
            got.add((bv, w))
    assert got == shapes


WAVE_K_F32 = {(16, 2), (32, 2), (32, 4), (64, 4), (64, 8), (128, 8)}
WAVE_K_F16 = {(32, 2), (64, 2), (64, 4), (128, 4), (128, 8)}


@pytest.mark.parametrize("dtype,shapes", [("f32", WAVE_K_F32), ("f16", WAVE_K_F16)])
def test_supported_whole_k_shapes(dtype, shapes):
    got = set()
    for bv in (8, 16, 32, 48, 64, 128, 256):
        for w in (1, 2, 3, 4, 8, 16):
            try:
                d = B.kda_describe_launch(8, 8, 12, dtype, waves_per_tile=w, bv=bv,
                                          rows_layout=B.KDA_ROWS_WAVE_K)
            except B.KdaError as e:
                assert e.code == B.KDA_ERR_ARG
                continue
            assert (d["bv"], d["waves_per_tile"], d["rows_layout"]) == (bv, w, B.KDA_ROWS_WAVE_K)
            assert d["tiles"] == 8 * 12 * (128 // bv) and d["kernel"] == "kda_rows_kernel"
            assert d["lds_bytes"] == 4 * 8 * (3 * 128 + bv + 2)
            got.add((bv, w))
    assert got == shapes


def test_describe_launch():
    d = B.kda_describe_launch(64, 1, 12, "f32")
    assert (d["bv"], d["waves_per_tile"], d["tiles"], d["blocks"]) == (128, 2, 768, 768)
    assert (d["kernel"], d["rows_layout"]) == ("kda_decode_tile", B.KDA_ROWS_K_SPLIT)
    d = B.kda_describe_launch(64, 1, 12, "f16")
    assert (d["bv"], d["waves_per_tile"], d["tiles"]) == (64, 1, 1536)
    # small single-row launches (requests x heads): narrower tiles or more waves
    for n_req, dt, want in ((1, "f32", (32, 1)), (4, "f32", (32, 1)), (5, "f32", (64, 8)), (10, "f32", (64, 8)),
                            (11, "f32", (128, 2)), (1, "f16", (64, 4)), (8, "f16", (64, 4)),
                            (9, "f16", (64, 1))):
        d = B.kda_describe_launch(n_req, 1, 12, dt)
        assert (d["bv"], d["waves_per_tile"]) == want, (n_req, dt)
    assert (B.kda_describe_launch(1, 1, 12, "f32", waves_per_tile=2)["bv"]) == 32   # bv stays the small default
    # one row: the layout option is ignored
    d = B.kda_describe_launch(64, 1, 12, "f16", rows_layout=B.KDA_ROWS_WAVE_K)
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (64, 1, "kda_decode_tile")
    # chained rows: the matrix-core block form for fp16 pools (the whole-K
    # layout when a shape option is set), the K split for fp32
    d = B.kda_describe_launch(8, 8, 12, "f16")
    assert (d["bv"], d["waves_per_tile"], d["tiles"]) == (64, 8, 8 * 12 * 2)
    assert (d["kernel"], d["rows_layout"]) == ("kda_rows_mfma8_kernel", B.KDA_ROWS_MATRIX)
    d = B.kda_describe_launch(8, 8, 12, "f16", waves_per_tile=2)
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (64, 2, "kda_rows_kernel")
    d = B.kda_describe_launch(8, 8, 12, "f16", bv=128)
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (128, 4, "kda_rows_kernel")
    d = B.kda_describe_launch(8, 8, 12, "f32")
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (64, 8, "kda_decode_tile")
    # small fp32 chained-row launches of 6 rows or more take the matrix-core
    # block form
    assert B.kda_describe_launch(4, 8, 12, "f32")["kernel"] == "kda_rows_mfma8_kernel"
    assert B.kda_describe_launch(4, 6, 12, "f32")["kernel"] == "kda_rows_mfma8_kernel"
    assert B.kda_describe_launch(4, 5, 12, "f32")["kernel"] == "kda_decode_tile"
    assert B.kda_describe_launch(1, 2, 12, "f32")["kernel"] == "kda_decode_tile"
    assert B.kda_describe_launch(5, 8, 12, "f32")["kernel"] == "kda_decode_tile"
    # fp16: the block form from 3 rows up to 240 requests x heads; 2 rows
    # whole-K up to 48, then the K split, as are larger launches
    assert B.kda_describe_launch(20, 8, 12, "f16")["kernel"] == "kda_rows_mfma8_kernel"
    assert B.kda_describe_launch(20, 3, 12, "f16")["kernel"] == "kda_rows_mfma8_kernel"
    assert B.kda_describe_launch(21, 8, 12, "f16")["rows_layout"] == B.KDA_ROWS_K_SPLIT
    assert B.kda_describe_launch(4, 2, 12, "f16")["rows_layout"] == B.KDA_ROWS_WAVE_K
    assert B.kda_describe_launch(5, 2, 12, "f16")["rows_layout"] == B.KDA_ROWS_K_SPLIT
    assert B.kda_describe_launch(4, 8, 12, "f32", waves_per_tile=8)["kernel"] == "kda_decode_tile"
    d = B.kda_describe_launch(8, 8, 12, "f16", waves_per_tile=8, rows_layout=B.KDA_ROWS_K_SPLIT)
    assert (d["waves_per_tile"], d["threads"], d["kernel"]) == (8, 512, "kda_decode_tile")
    d = B.kda_describe_launch(8, 8, 12, "f16", block_rows=True)
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (64, 4, "kda_decode_tile")
    # the block form with one wave: fp32 admitted, fp16 refused (it would spill registers)
    d = B.kda_describe_launch(8, 8, 12, "f32", block_rows=True, waves_per_tile=1, bv=32)
    assert (d["bv"], d["waves_per_tile"]) == (32, 1)
    with pytest.raises(B.KdaError):
        B.kda_describe_launch(8, 8, 12, "f16", block_rows=True, waves_per_tile=1, bv=64)
    d = B.kda_describe_launch(8, 8, 12, "f16", block_rows=True, waves_per_tile=2, bv=64)
    assert (d["bv"], d["waves_per_tile"]) == (64, 2)
    # the matrix-core block form: 64 columns over 8 waves (or 4 on request),
    # either dtype, block_rows implied
    for dt in ("f32", "f16"):
        for blk in (False, True):
            d = B.kda_describe_launch(8, 8, 12, dt, rows_layout=B.KDA_ROWS_MATRIX, block_rows=blk)
            assert (d["bv"], d["waves_per_tile"], d["threads"], d["tiles"]) == (64, 8, 512, 8 * 12 * 2)
            assert (d["kernel"], d["rows_layout"]) == ("kda_rows_mfma8_kernel", B.KDA_ROWS_MATRIX)
            assert d["lds_bytes"] == 52128
    d = B.kda_describe_launch(8, 8, 12, "f16", rows_layout=B.KDA_ROWS_MATRIX, waves_per_tile=4, bv=64)
    assert (d["bv"], d["waves_per_tile"], d["kernel"]) == (64, 4, "kda_rows_mfma_kernel")
    # H is packed into 16 bits of a kernel argument: more heads are refused
    with pytest.raises(B.KdaError):
        B.kda_describe_launch(1, 8, 70000, "f16")
    for w, bv in ((2, 0), (0, 128)):
        with pytest.raises(B.KdaError):
            B.kda_describe_launch(8, 8, 12, "f16", rows_layout=B.KDA_ROWS_MATRIX, waves_per_tile=w, bv=bv)
    # one row: the layout option is ignored
    d = B.kda_describe_launch(64, 1, 12, "f32", rows_layout=B.KDA_ROWS_MATRIX)
    assert d["kernel"] == "kda_decode_tile"
    with pytest.raises(B.KdaError):
        B.kda_describe_launch(8, 9, 12, "f16")
    with pytest.raises(B.KdaError):
        B.kda_describe_launch(8, 1, 12, "bf16")


def test_strerror_names_every_code():
    msgs = {c: B.kda_strerror(c) for c in range(10)}
    assert len(set(msgs.values())) == 10
    assert "bf16" in msgs[B.KDA_ERR_DTYPE_REFUSED]
    assert B.kda_strerror(1234) == "unknown kda status code"


def conv_step(P, conv, n_req=4, n_rows=1, ptrs=None, opts=None, scale=0.0883883):
    p = [FAKE] * 7 if ptrs is None else ptrs     # slot_ids, x, conv_w, g, b, out, init
    f = [ctypes.c_void_p(v) for v in p]
    return B.library().kda_decode_step_conv(
        ctypes.byref(P), None if conv is None else ctypes.byref(conv), f[0], f[6], f[1], f[2],
        f[3], f[4], f[5], n_req, n_rows, P.dtype, scale,
        None if opts is None else ctypes.byref(opts), None)


def test_conv_step_refusals():
    P = pool(n_slots=16)
    Cv = B.kda_conv_pool(ctypes.c_void_p(FAKE), 16, 12)
    assert conv_step(P, None) == B.KDA_ERR_NULL
    assert conv_step(P, B.kda_conv_pool(None, 16, 12)) == B.KDA_ERR_NULL
    assert conv_step(P, B.kda_conv_pool(ctypes.c_void_p(FAKE), 15, 12)) == B.KDA_ERR_SHAPE
    assert conv_step(P, B.kda_conv_pool(ctypes.c_void_p(FAKE), 16, 8)) == B.KDA_ERR_SHAPE
    assert conv_step(pool(n_slots=16, dtype=B.KDA_BF16), Cv) == B.KDA_ERR_DTYPE_REFUSED
    assert conv_step(P, Cv, n_rows=9) == B.KDA_ERR_ROWS
    assert conv_step(P, Cv, n_req=0) == B.KDA_OK
    for which in range(6):
        ptrs = [FAKE] * 7
        ptrs[which] = 0
        assert conv_step(P, Cv, ptrs=ptrs) == B.KDA_ERR_NULL
    assert conv_step(P, Cv, opts=B.kda_launch_opts(0, 64)) == B.KDA_ERR_ARG   # whole heads only
    assert conv_step(P, Cv, opts=B.kda_launch_opts(1, 0)) == B.KDA_ERR_ARG
    assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(0, 0, 0, B.KDA_ROWS_WAVE_K)) == B.KDA_ERR_ARG
    # the matrix-core block form with the convolution: whole heads over 16
    # waves (or 8: two halves of 4) only
    for nw in (2, 4, 32):
        assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(nw, 0, 0, B.KDA_ROWS_MATRIX)) == B.KDA_ERR_ARG
    # 16 waves ask for the matrix-core form: refused in the K-split layout
    assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(16, 0, 0, B.KDA_ROWS_K_SPLIT)) == B.KDA_ERR_ARG
    assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(16, 0)) == B.KDA_ERR_ARG
    assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(0, 64, 0, B.KDA_ROWS_MATRIX)) == B.KDA_ERR_ARG
    assert conv_step(P, Cv, n_rows=2, opts=B.kda_launch_opts(0, 0, 0, 4)) == B.KDA_ERR_ARG
    assert conv_step(P, Cv, scale=float("nan")) == B.KDA_ERR_ARG
    # the raw gate: 0 or 1 on the fused entries, 0 elsewhere
    assert conv_step(P, Cv, n_req=0, opts=B.kda_launch_opts(0, 0, 0, 0, 1)) == B.KDA_OK
    for bad in (2, -1):
        assert conv_step(P, Cv, opts=B.kda_launch_opts(0, 0, 0, 0, bad)) == B.KDA_ERR_ARG
        assert conv_step(P, Cv, n_rows=4, opts=B.kda_launch_opts(0, 0, 0, B.KDA_ROWS_MATRIX, bad)) == B.KDA_ERR_ARG
    assert conv_step(P, B.kda_conv_pool(ctypes.c_void_p(FAKE + 8), 16, 12)) == B.KDA_ERR_ALIGN


def conv_step_ws(P, conv, counts, n_counts, n_req=4, n_rows=2, opts=None, ptrs=None):
    p = [FAKE] * 7 if ptrs is None else ptrs     # slot_ids, x, conv_w, g, b, out, init
    f = [ctypes.c_void_p(v) for v in p]
    return B.library().kda_decode_step_conv_ws(
        ctypes.byref(P), ctypes.byref(conv), f[0], f[6], f[1], f[2], f[3], f[4], f[5], n_req, n_rows,
        P.dtype, 0.0883883, None if counts is None else ctypes.c_void_p(counts), n_counts,
        None if opts is None else ctypes.byref(opts), None)


def test_conv_step_with_pair_counters_refusals():
    P = pool(n_slots=16)
    Cv = B.kda_conv_pool(ctypes.c_void_p(FAKE), 16, 12)
    M = B.KDA_ROWS_MATRIX
    assert conv_step_ws(P, Cv, None, 48) == B.KDA_ERR_NULL          # no counters but a count
    assert conv_step_ws(P, Cv, FAKE, -1) == B.KDA_ERR_ARG
    assert conv_step_ws(P, Cv, FAKE, 4 * 12 - 1) == B.KDA_ERR_ARG   # one per (request, head)
    assert conv_step_ws(P, Cv, FAKE + 2, 48) == B.KDA_ERR_ALIGN
    assert conv_step_ws(P, Cv, FAKE, 48, n_req=0) == B.KDA_OK
    # the halves: the matrix-core form over 8 waves, chained rows only
    assert conv_step_ws(P, Cv, FAKE, 48, opts=B.kda_launch_opts(16, 64, 0, M)) == B.KDA_ERR_ARG
    assert conv_step_ws(P, Cv, FAKE, 48, opts=B.kda_launch_opts(4, 64, 0, M)) == B.KDA_ERR_ARG
    assert conv_step_ws(P, Cv, FAKE, 48, n_rows=1, opts=B.kda_launch_opts(0, 64)) == B.KDA_ERR_ARG
    assert conv_step_ws(P, Cv, FAKE, 48, opts=B.kda_launch_opts(0, 64, 0, B.KDA_ROWS_K_SPLIT)) == B.KDA_ERR_ARG
    assert conv_step_ws(P, Cv, FAKE, 48, opts=B.kda_launch_opts(0, 32, 0, M)) == B.KDA_ERR_ARG
    # without counters the halves are refused
    assert conv_step_ws(P, Cv, None, 0, opts=B.kda_launch_opts(0, 64, 0, M)) == B.KDA_ERR_ARG


def conv_step_noalloc(P, conv, n_req=4, n_rows=2, opts=None, ptrs=None):
    p = [FAKE] * 7 if ptrs is None else ptrs     # slot_ids, x, conv_w, g, b, out, init
    f = [ctypes.c_void_p(v) for v in p]
    return B.library().kda_decode_step_conv_noalloc(
        ctypes.byref(P), None if conv is None else ctypes.byref(conv), f[0], f[6], f[1], f[2], f[3], f[4],
        f[5], n_req, n_rows, P.dtype, 0.0883883, None if opts is None else ctypes.byref(opts), None)


def test_conv_step_noalloc_refusals():
    # every refusal comes before any device work (no GPU here)
    P = pool(n_slots=1024, H=12)
    Cv = B.kda_conv_pool(ctypes.c_void_p(FAKE), 1024, 12)
    assert B.KDA_NOALLOC_MAX_PAIRS == 4096
    assert conv_step_noalloc(P, Cv, n_req=4096 // 12 + 1) == B.KDA_ERR_ARG   # beyond the counters
    assert conv_step_noalloc(P, Cv, n_req=0) == B.KDA_OK
    assert conv_step_noalloc(P, None) == B.KDA_ERR_NULL
    assert conv_step_noalloc(pool(n_slots=1024, H=12, dtype=B.KDA_BF16), Cv) == B.KDA_ERR_DTYPE_REFUSED
    assert conv_step_noalloc(P, Cv, n_rows=9) == B.KDA_ERR_ROWS
    assert conv_step_noalloc(P, Cv, opts=B.kda_launch_opts(16, 64, 0, B.KDA_ROWS_MATRIX)) == B.KDA_ERR_ARG
    ptrs = [FAKE] * 7
    ptrs[1] = FAKE + 4                                                          # x misaligned
    assert conv_step_noalloc(P, Cv, ptrs=ptrs) == B.KDA_ERR_ALIGN


def prefill(P, n_seq=4, n_tokens=100, ptrs=None, chunk=0, scale=0.0883883, dtype=None):
    p = [FAKE] * 9 if ptrs is None else ptrs     # init, cu, q, k, v, g, b, out, dst
    f = [ctypes.c_void_p(v) for v in p]
    return B.library().kda_prefill(
        ctypes.byref(P), f[0], f[8], f[1], f[2], f[3], f[4], f[5], f[6], f[7], n_seq, n_tokens,
        P.dtype if dtype is None else dtype, scale, ctypes.byref(B.kda_prefill_opts(chunk)), None)


def test_prefill_refusals():
    P = pool(n_slots=16)
    assert prefill(pool(n_slots=16, base=0)) == B.KDA_ERR_NULL
    assert prefill(pool(n_slots=16, dtype=B.KDA_BF16)) == B.KDA_ERR_DTYPE_REFUSED
    assert prefill(P, dtype=B.KDA_F16) == B.KDA_ERR_DTYPE_MISMATCH
    assert prefill(pool(n_slots=16, Kd=64)) == B.KDA_ERR_SHAPE
    # byte offsets within a chunk stay below 2^31: at most 16384 heads (refused
    # before any launch; the accepted side would launch, so it is not called here)
    assert prefill(pool(n_slots=16, H=16385)) == B.KDA_ERR_SHAPE
    assert prefill(P, n_seq=17) == B.KDA_ERR_SLOT          # more sequences than slots
    assert prefill(P, n_seq=-1) == B.KDA_ERR_ARG
    assert prefill(P, n_tokens=-1) == B.KDA_ERR_ARG
    assert prefill(P, chunk=48) == B.KDA_ERR_ARG
    assert prefill(P, scale=float("inf")) == B.KDA_ERR_ARG
    assert prefill(P, n_seq=0) == B.KDA_OK
    for which in range(8):
        ptrs = [FAKE] * 9
        ptrs[which] = 0
        assert prefill(P, ptrs=ptrs) == B.KDA_ERR_NULL, which
    ptrs = [FAKE] * 9
    ptrs[2] = FAKE + 4                                     # q must be 16-byte aligned
    assert prefill(P, ptrs=ptrs) == B.KDA_ERR_ALIGN


@pytest.mark.parametrize("init,dst,cu,n_tokens,code", [
    ([0, 1], [2, 3], [0, 3, 7], 7, 0),
    ([0, 1], None, [0, 0, 0], 0, 0),                        # empty sequences, in place
    ([0, 1], [2, 2], [0, 3, 7], 7, B.KDA_ERR_SLOT),         # one slot stored twice
    ([0, 1], [1, 3], [0, 3, 7], 7, B.KDA_ERR_SLOT),         # destination is another's initial slot
    ([0, 16], None, [0, 3, 7], 7, B.KDA_ERR_SLOT),          # slot out of range
    ([0, 1], None, [0, 5, 3], 7, B.KDA_ERR_ARG),            # cu_seqlens decreasing
    ([0, 1], None, [0, 3, 8], 7, B.KDA_ERR_ARG),            # past the token arrays
    ([0, 1], None, [-1, 3, 7], 7, B.KDA_ERR_ARG),
])
def test_prefill_validate(init, dst, cu, n_tokens, code):
    assert B.kda_prefill_validate(pool(n_slots=16), init, cu, n_tokens, B.KDA_F32,
                                  dst_slot_ids_host=dst) == code


def test_binding_refuses_host_tensors():
    """The library dereferences device addresses only: the binding refuses a
    CPU tensor for any buffer with a TypeError before the library is
    called, and a copy length past either buffer with a ValueError."""
    torch = pytest.importorskip("torch")
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)  # noqa: E731
    ids = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.kda_decode_step(f(8, 2, 128, 128), ids, f(4, 2, 128), f(4, 2, 128), f(4, 2, 128),
                          f(4, 2, 128), f(4, 2), f(4, 2, 128))
    with pytest.raises(TypeError, match="GPU tensor"):
        B.make_pool(f(8, 2, 128, 128))
    with pytest.raises(TypeError, match="GPU tensor"):
        B._dev(f(4), "q")
    with pytest.raises(TypeError, match="torch tensor"):
        B._dev(np.zeros(4, np.float32), "q")
    with pytest.raises(TypeError, match="GPU tensor"):
        B.kda_prefill(f(8, 2, 128, 128), ids, torch.zeros(5, dtype=torch.int32), f(4, 2, 128),
                      f(4, 2, 128), f(4, 2, 128), f(4, 2, 128), f(4, 2), f(4, 2, 128))
    with pytest.raises(TypeError, match="GPU tensor"):
        B.kda_state_copy(f(8, 2, 128, 128), ids, ids)
    with pytest.raises(TypeError, match="GPU tensor"):
        B.kda_copy_probe(f(16), f(16))


def test_probe_refusals_before_any_hip_call():
    lib = B.library()
    f = ctypes.c_void_p(FAKE)
    assert lib.kda_bw_probe(f, f, 64, 3, 1, 1, None) == B.KDA_ERR_ARG        # mode
    assert lib.kda_bw_probe(f, f, 64, 0, 3, 1, None) == B.KDA_ERR_ARG        # vectors per thread
    assert lib.kda_bw_probe(f, f, 60, 0, 1, 1, None) == B.KDA_ERR_ARG        # not whole vectors
    assert lib.kda_bw_probe(None, f, 64, 0, 1, 1, None) == B.KDA_ERR_NULL
    assert lib.kda_bw_probe(f, None, 64, 1, 1, 1, None) == B.KDA_ERR_NULL    # a read needs src
    assert lib.kda_bw_probe(ctypes.c_void_p(FAKE + 4), f, 64, 0, 1, 1, None) == B.KDA_ERR_ALIGN
    assert lib.kda_bw_probe(f, f, 0, 0, 4, 0, None) == B.KDA_OK             # empty: no launch
    ids = ctypes.c_void_p(FAKE)
    assert lib.kda_tile_probe(None, ids, 4, B.KDA_F32, None) == B.KDA_ERR_NULL
    assert lib.kda_tile_probe(ctypes.byref(pool(dtype=B.KDA_BF16)), ids, 4, B.KDA_BF16, None) == \
        B.KDA_ERR_DTYPE_REFUSED
    assert lib.kda_tile_probe(ctypes.byref(pool()), ids, 4, B.KDA_F16, None) == B.KDA_ERR_DTYPE_MISMATCH
    assert lib.kda_tile_probe(ctypes.byref(pool(Kd=64)), ids, 4, B.KDA_F32, None) == B.KDA_ERR_SHAPE
    assert lib.kda_tile_probe(ctypes.byref(pool(n_slots=3)), ids, 4, B.KDA_F32, None) == B.KDA_ERR_ARG
    assert lib.kda_tile_probe(ctypes.byref(pool()), None, 4, B.KDA_F32, None) == B.KDA_ERR_NULL
    assert lib.kda_tile_probe(ctypes.byref(pool()), ids, 0, B.KDA_F32, None) == B.KDA_OK
    rp = lambda P, n_req=4, n_rows=8, ids=ids, init=None, dt=None, cols=0, nw=0: lib.kda_rows_probe(
        ctypes.byref(P) if P is not None else None, ids, init, n_req, n_rows, cols, nw,
        P.dtype if dt is None else dt, None)
    assert rp(None, dt=B.KDA_F16) == B.KDA_ERR_NULL
    assert rp(pool(dtype=B.KDA_BF16)) == B.KDA_ERR_DTYPE_REFUSED
    assert rp(pool(), dt=B.KDA_F16) == B.KDA_ERR_DTYPE_MISMATCH
    assert rp(pool(Kd=64)) == B.KDA_ERR_SHAPE
    assert rp(pool(), n_rows=0) == B.KDA_ERR_ROWS
    assert rp(pool(), n_rows=9) == B.KDA_ERR_ROWS
    assert rp(pool(n_slots=31), n_rows=8) == B.KDA_ERR_ARG              # 4 x 8 rows need 32 slots
    assert rp(pool(), n_req=-1) == B.KDA_ERR_ARG
    assert rp(pool(), ids=None) == B.KDA_ERR_NULL
    assert rp(pool(), init=ctypes.c_void_p(FAKE + 2)) == B.KDA_ERR_ALIGN
    assert rp(pool(), n_req=0) == B.KDA_OK                              # no launch
    # tile shapes: 32, 64 or 128 columns over 8 waves, 128 over 16
    for cols, nw in ((32, 8), (64, 8), (128, 8), (128, 16), (0, 0), (64, 0), (0, 8)):
        assert rp(pool(), n_req=0, cols=cols, nw=nw) == B.KDA_OK
    for cols, nw in ((16, 8), (64, 16), (32, 16), (128, 4), (96, 8), (64, 4)):
        assert rp(pool(), n_req=0, cols=cols, nw=nw) == B.KDA_ERR_ARG, (cols, nw)


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defines = dict(re.findall(r"^#define (KDA_\w+) (-?\d+)", text, flags=re.M))
    assert "KDA_NOALLOC_MAX_PAIRS" in defines
    for name, val in defines.items():
        if hasattr(B, name):
            assert getattr(B, name) == int(val), name
