"""GPU parity: the gfx950 kernels against the CPU oracle, through the C ABI.

Workloads: the named configurations at full size (single slot fp32; 64 of
96 slots fp32 and fp16; 8 requests x 8 speculative rows fp16), ragged small
shapes that span several tiles in every wave layout, and the edge cases:
an empty launch, out-of-range slot ids, the identity gate, a zero state,
zero q / k, 64-bit pool offsets.  Structural checks: the fp32 twin of an
fp16 launch (ROCm/ATOM PR #2945, Testing: outputs bit-equal, the fp16 pool
equal to the twin's fp32 pool rounded to fp16), chained rows equal to
single-row launches, permutation equivariance, determinism.
"""
import sys

import numpy as np
import pytest

import kda_inputs
from gpu_helpers import (B, F16_ULP, OUT_REL, check_parity, device_inputs, need_gpu,
                         out_rel_err, pool_to_host, run_gpu, run_oracle_f32, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# --- named workloads at full size, in the launch shape the bench times -----

@pytest.mark.parametrize("name", list(kda_inputs.WORKLOADS))
def test_named_workload_parity(oracle, name):
    inp = kda_inputs.WORKLOADS[name](seed=0)
    say("workload", name, inp.pool.shape, inp.dtype, "rows", inp.n_rows)
    gp, go = run_gpu(inp)
    res = check_parity(oracle, inp, gp, go, label=name)
    say(name, res)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_full_size_other_dtype_and_rows(oracle, dtype):
    # the multi-row shape on an fp32 pool and the batched shape on both
    inp = kda_inputs.make_inputs("spec-verify 8x8 " + dtype, 96, 8, 8, dtype, seed=3)
    gp, go = run_gpu(inp)
    say("spec-verify", dtype, check_parity(oracle, inp, gp, go, label="spec " + dtype))


# --- ragged small shapes over every wave layout ----------------------------

SHAPES = [(1, 1, 1), (3, 1, 1), (5, 2, 1), (2, 12, 1), (1, 1, 8), (3, 2, 3), (2, 5, 8), (4, 3, 7)]


LAUNCH_SHAPES = [("f32", bv, w) for bv, w in [(32, 1), (32, 2), (32, 4), (32, 8), (64, 1), (64, 2),
                                              (64, 4), (64, 8), (128, 2), (128, 4), (128, 8)]] + \
                [("f16", bv, w) for bv, w in [(64, 1), (64, 2), (64, 4), (64, 8), (128, 2), (128, 4),
                                              (128, 8)]]


@pytest.mark.parametrize("dtype,bv,waves", LAUNCH_SHAPES)
@pytest.mark.parametrize("n_req,H,n_rows", SHAPES)
def test_small_shapes_every_launch_shape(oracle, dtype, bv, waves, n_req, H, n_rows):
    n_slots = n_req * n_rows + 3
    inp = kda_inputs.make_inputs("small", n_slots, n_req, n_rows, dtype, H=H,
                                 seed=1000 + 7 * n_req + 31 * H + n_rows)
    gp, go = run_gpu(inp, waves_per_tile=waves, bv=bv, rows_layout=B.KDA_ROWS_K_SPLIT)
    check_parity(oracle, inp, gp, go,
                 label="small %s bv%d w%d %dx%dx%d" % (dtype, bv, waves, n_req, H, n_rows))


# whole-K chained-row layout: (bv, waves) with 2 or 4 lanes per row piece
WAVE_K_SHAPES = [("f32", bv, w) for bv, w in [(16, 2), (32, 2), (32, 4), (64, 4), (64, 8),
                                              (128, 8)]] + \
                [("f16", bv, w) for bv, w in [(32, 2), (64, 2), (64, 4), (128, 4), (128, 8)]]


@pytest.mark.parametrize("dtype,bv,waves", WAVE_K_SHAPES)
@pytest.mark.parametrize("n_req,H,n_rows", [s for s in SHAPES if s[2] > 1] + [(2, 3, 2)])
def test_small_shapes_whole_k_layout(oracle, dtype, bv, waves, n_req, H, n_rows):
    n_slots = n_req * n_rows + 3
    inp = kda_inputs.make_inputs("small wk", n_slots, n_req, n_rows, dtype, H=H,
                                 seed=2000 + 7 * n_req + 31 * H + n_rows)
    gp, go = run_gpu(inp, waves_per_tile=waves, bv=bv, rows_layout=B.KDA_ROWS_WAVE_K)
    check_parity(oracle, inp, gp, go,
                 label="small wk %s bv%d w%d %dx%dx%d" % (dtype, bv, waves, n_req, H, n_rows))


# --- edge cases -----------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_empty_launch_changes_nothing(dtype):
    inp = kda_inputs.make_inputs("empty", 4, 1, 1, dtype, H=2, seed=5)
    pool, ids, t, out = device_inputs(inp)
    before = pool.clone()
    empty = torch.empty((0, 2, 128), dtype=torch.float32, device=pool.device)
    B.kda_decode_step(pool, ids[:0], empty, empty, empty, empty, t["b"][:0], empty)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)


@pytest.mark.parametrize("n_rows", [1, 4])
def test_out_of_range_slot_is_skipped_on_device(oracle, n_rows):
    inp = kda_inputs.make_inputs("bad id", 16, 3, n_rows, "f16", H=2, seed=7)
    bad_req = 1
    ids = inp.slot_ids.copy()
    ids[bad_req * n_rows + n_rows - 1] = 16          # one past the end
    pool, dids, t, out = device_inputs(inp)
    dids.copy_(torch.from_numpy(ids))
    before = pool_to_host(pool).copy()
    B.kda_decode_step(pool, dids, t["q"], t["k"], t["v"], t["g"], t["b"], out, n_rows_per_slot=n_rows)
    torch.cuda.synchronize()
    after, o = pool_to_host(pool), out.cpu().numpy()
    rows = slice(bad_req * n_rows, (bad_req + 1) * n_rows)
    assert np.all(np.isnan(o[rows]))
    np.testing.assert_array_equal(after[inp.slot_ids[rows]], before[inp.slot_ids[rows]])
    # the other requests are processed as usual
    good = [r for r in range(3) if r != bad_req]
    sel = np.concatenate([np.arange(r * n_rows, (r + 1) * n_rows) for r in good])
    sub = kda_inputs.DecodeInputs("good", "f16", inp.pool.copy(), inp.slot_ids[sel], inp.q[sel],
                                  inp.k[sel], inp.v[sel], inp.g[sel], inp.b[sel], n_rows, inp.scale)
    o_pool, o_out = run_oracle_f32(oracle, sub)
    assert out_rel_err(o[sel], o_out) <= OUT_REL
    from gpu_helpers import f16_ulp_distance
    assert f16_ulp_distance(after[sub.slot_ids], o_pool[sub.slot_ids]).max() <= F16_ULP


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_rows", [1, 8])
def test_identity_gate_keeps_state_bits(oracle, dtype, n_rows):
    # g = 0 -> a = 1 exactly; b = -1e4 -> beta = 0 exactly: S unchanged
    inp = kda_inputs.make_inputs("identity", 24, 3, n_rows, dtype, seed=11)
    inp.g[:] = 0.0
    inp.b[:] = -1e4
    gp, go = run_gpu(inp)
    # unchanged in value: a -0 may come back as +0 ((-0) + (+0) * u = +0),
    # exactly as the oracle computes it
    as_float = (lambda x: x) if dtype == "f32" else (lambda x: x.view(np.float16))
    for r in range(3):
        s0 = inp.slot_ids[r * n_rows]
        for t in range(n_rows):
            got, want = as_float(gp[inp.slot_ids[r * n_rows + t]]), as_float(inp.pool[s0])
            assert np.array_equal(got, want)
    check_parity(oracle, inp, gp, go, label="identity")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_zero_state_closed_form(dtype):
    inp = kda_inputs.make_inputs("zero", 8, 8, 1, dtype, seed=13)
    inp.pool[:] = 0
    gp, go = run_gpu(inp)
    for r in range(8):
        for h in range(12):
            q, k, v = (x[r, h].astype(np.float64) for x in (inp.q, inp.k, inp.v))
            qn, kn = q / np.sqrt(q @ q + 1e-6), k / np.sqrt(k @ k + 1e-6)
            beta = 1.0 / (1.0 + np.exp(-float(inp.b[r, h])))
            S1 = beta * np.outer(kn, v)
            o = inp.scale * beta * (qn @ kn) * v
            got = gp[inp.slot_ids[r], h]
            got = got.astype(np.float64) if dtype == "f32" else got.view(np.float16).astype(np.float64)
            tol = 1e-6 if dtype == "f32" else 2.0 ** -10 * np.abs(S1) + 2.0 ** -24
            assert np.all(np.abs(got - S1) <= tol)
            np.testing.assert_allclose(go[r, h], o, rtol=1e-5, atol=1e-6)


def test_zero_q_and_k_stay_finite(oracle):
    inp = kda_inputs.make_inputs("zero q k", 8, 4, 1, "f32", seed=17)
    inp.q[0] = 0.0
    inp.k[1] = 0.0
    gp, go = run_gpu(inp)
    assert np.all(go[0] == 0.0)
    check_parity(oracle, inp, gp, go, label="zero q k")


def test_64bit_pool_offsets(oracle):
    # slot * H * K * V beyond 2^31 elements: an fp16 pool of 11,000 slots
    # (4.3 GB); the launch touches slots near the top only
    n_slots, H = 11000, 12
    pool = torch.zeros((n_slots, H, 128, 128), dtype=torch.float16, device="cuda")
    inp = kda_inputs.make_inputs("high slots", 6, 6, 1, "f16", seed=19)
    ids = np.array([10999, 10990, 10950, 10925, 11, 10998], dtype=np.int32)
    for i, s in enumerate(ids):
        pool[s] = torch.from_numpy(inp.pool[inp.slot_ids[i]].view(np.float16)).cuda()
    dev = {n: torch.from_numpy(getattr(inp, n)).cuda() for n in ("q", "k", "v", "g", "b")}
    out = torch.empty((6, H, 128), dtype=torch.float32, device="cuda")
    B.kda_decode_step(pool, torch.from_numpy(ids).cuda(), dev["q"], dev["k"], dev["v"], dev["g"],
                      dev["b"], out)
    torch.cuda.synchronize()
    got = pool[torch.from_numpy(ids).long().cuda()].cpu().numpy().view(np.uint16)
    o_pool, o_out = run_oracle_f32(oracle, inp)
    from gpu_helpers import f16_ulp_distance
    assert f16_ulp_distance(got, o_pool[inp.slot_ids]).max() <= F16_ULP
    assert out_rel_err(out.cpu().numpy(), o_out) <= OUT_REL
    assert int(ids.max()) * H * 128 * 128 > 2 ** 31
    del pool
    torch.cuda.empty_cache()


# --- structure ------------------------------------------------------------

# Lane layouts (lanes per tile row, waves per tile) that both dtypes build:
# an fp16 tile of 8 * lanes columns and an fp32 tile of 4 * lanes columns
# put the same rows in the same lanes, so their column sums are identical.
TWIN_LAYOUTS = [(8, 1), (8, 2), (8, 4), (8, 8), (16, 2), (16, 4), (16, 8)]


@pytest.mark.parametrize("n_rows", [1, 8])
@pytest.mark.parametrize("lanes,waves", TWIN_LAYOUTS)
def test_fp32_twin_of_fp16_launch(n_rows, lanes, waves):
    """fp16 launch vs the same launch on the exactly widened fp32 pool, same
    lane layout: outputs bit-equal; each fp16 snapshot = RNE(fp32 snapshot)
    (ROCm/ATOM PR #2945, Testing)."""
    inp16 = kda_inputs.make_inputs("twin", 96, 64 // n_rows, n_rows, "f16", seed=23)
    inp32 = kda_inputs.DecodeInputs("twin32", "f32", inp16.pool.view(np.float16).astype(np.float32),
                                    inp16.slot_ids, inp16.q, inp16.k, inp16.v, inp16.g, inp16.b,
                                    n_rows, inp16.scale)
    p16, o16 = run_gpu(inp16, waves_per_tile=waves, bv=8 * lanes, rows_layout=B.KDA_ROWS_K_SPLIT)
    p32, o32 = run_gpu(inp32, waves_per_tile=waves, bv=4 * lanes, rows_layout=B.KDA_ROWS_K_SPLIT)
    np.testing.assert_array_equal(o16.view(np.uint32), o32.view(np.uint32))
    np.testing.assert_array_equal(p16, p32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("lanes,waves", [(2, 2), (2, 4), (2, 8), (4, 2), (4, 4)])
def test_fp32_twin_of_fp16_launch_whole_k(lanes, waves):
    """The twin property in the whole-K layout: the same lanes per row piece
    give the same rows per lane and the same exchange tree over the row
    groups, so outputs are bit-equal and each fp16 snapshot is the RNE of
    the fp32 one."""
    inp16 = kda_inputs.make_inputs("twin wk", 96, 8, 8, "f16", seed=25)
    inp32 = kda_inputs.DecodeInputs("twin32", "f32", inp16.pool.view(np.float16).astype(np.float32),
                                    inp16.slot_ids, inp16.q, inp16.k, inp16.v, inp16.g, inp16.b,
                                    8, inp16.scale)
    p16, o16 = run_gpu(inp16, waves_per_tile=waves, bv=8 * lanes * waves,
                       rows_layout=B.KDA_ROWS_WAVE_K)
    p32, o32 = run_gpu(inp32, waves_per_tile=waves, bv=4 * lanes * waves,
                       rows_layout=B.KDA_ROWS_WAVE_K)
    np.testing.assert_array_equal(o16.view(np.uint32), o32.view(np.uint32))
    np.testing.assert_array_equal(p16, p32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("lanes,waves", [(8, 2), (8, 4), (16, 8)])
def test_fp32_twin_of_fp16_launch_rows_as_block(lanes, waves):
    """The same twin property for the block form of chained rows."""
    inp16 = kda_inputs.make_inputs("twin block", 96, 8, 8, "f16", seed=24)
    inp32 = kda_inputs.DecodeInputs("twin32", "f32", inp16.pool.view(np.float16).astype(np.float32),
                                    inp16.slot_ids, inp16.q, inp16.k, inp16.v, inp16.g, inp16.b,
                                    8, inp16.scale)
    p16, o16 = run_gpu(inp16, waves_per_tile=waves, bv=8 * lanes, block_rows=True)
    p32, o32 = run_gpu(inp32, waves_per_tile=waves, bv=4 * lanes, block_rows=True)
    np.testing.assert_array_equal(o16.view(np.uint32), o32.view(np.uint32))
    np.testing.assert_array_equal(p16, p32.astype(np.float16).view(np.uint16))


F32_SHAPES = [(32, 1), (32, 2), (32, 4), (32, 8), (64, 1), (64, 2), (64, 4), (64, 8),
              (128, 2), (128, 4), (128, 8)]


@pytest.mark.parametrize("bv,waves", F32_SHAPES)
def test_chained_rows_equal_single_row_launches_fp32(bv, waves):
    """Rows run one after the other do the single-row launch's arithmetic
    per row, so n chained single-row launches reproduce them bit for bit."""
    n_req, n = 4, 6
    inp = kda_inputs.make_inputs("chain", 40, n_req, n, "f32", seed=29)
    pm, om = run_gpu(inp, waves_per_tile=waves, bv=bv, rows_layout=B.KDA_ROWS_K_SPLIT)
    pool, ids, t, out = device_inputs(inp)
    for step in range(n):
        rows = torch.arange(n_req, device="cuda") * n + step
        if step > 0:   # carry each request's state into this row's slot
            src = ids[rows - 1].long()
            pool[ids[rows].long()] = pool[src]
        sub_out = torch.empty((n_req, 12, 128), dtype=torch.float32, device="cuda")
        B.kda_decode_step(pool, ids[rows].contiguous(), t["q"][rows].contiguous(),
                          t["k"][rows].contiguous(), t["v"][rows].contiguous(),
                          t["g"][rows].contiguous(), t["b"][rows].contiguous(), sub_out,
                          n_rows_per_slot=1, waves_per_tile=waves, bv=bv)
        out[rows] = sub_out
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool_to_host(pool).view(np.uint32), pm.view(np.uint32))
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), om.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_rows", [2, 5, 8])
@pytest.mark.parametrize("bv,waves", [(64, 1), (64, 4), (64, 8), (128, 2), (128, 8)])
def test_rows_as_block_and_row_after_row_both_match_the_oracle(oracle, dtype, n_rows, bv, waves):
    """The block form of a request's rows (one pass of 2 n column sums, an
    n x n triangular solve, element-wise snapshots) and the row-after-row
    chain compute the same recurrence: both within the oracle tolerances."""
    inp = kda_inputs.make_inputs("rows", 40, 40 // 8, n_rows, dtype, H=3, seed=41 + n_rows)
    for blk in (False, True):
        if blk and dtype == "f16" and waves == 1:
            continue  # refused: the one-wave fp16 block form would spill (test_abi_cpu)
        gp, go = run_gpu(inp, waves_per_tile=waves, bv=bv, block_rows=blk,
                         rows_layout=B.KDA_ROWS_K_SPLIT)
        check_parity(oracle, inp, gp, go, label="block" if blk else "sequential")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_permutation_equivariance_and_determinism(dtype):
    inp = kda_inputs.make_inputs("perm", 96, 64, 1, dtype, seed=31)
    p1, o1 = run_gpu(inp)
    p1b, o1b = run_gpu(inp)
    np.testing.assert_array_equal(p1, p1b)
    np.testing.assert_array_equal(o1.view(np.uint32), o1b.view(np.uint32))
    perm = np.random.default_rng(3).permutation(64)
    inp2 = kda_inputs.DecodeInputs("perm2", dtype, inp.pool, inp.slot_ids[perm], inp.q[perm],
                                   inp.k[perm], inp.v[perm], inp.g[perm], inp.b[perm], 1, inp.scale)
    p2, o2 = run_gpu(inp2)
    np.testing.assert_array_equal(p2, p1)
    np.testing.assert_array_equal(o2.view(np.uint32), o1[perm].view(np.uint32))


def test_launch_shapes_agree_within_rounding():
    inp = kda_inputs.make_inputs("layouts", 96, 64, 1, "f32", seed=37)
    res = [run_gpu(inp, waves_per_tile=w, bv=bv) for bv, w in F32_SHAPES]
    for p, o in res[1:]:
        assert np.max(np.abs(p - res[0][0])) <= 1e-6
        assert out_rel_err(o, res[0][1]) <= OUT_REL


def test_column_norm_growth_bound_on_gpu():
    # ROCm/ATOM PR #2945, Limitations: with unit k, beta in (0, 1) and decay
    # <= 1 a token adds at most v_j^2 to the squared norm of column j
    inp = kda_inputs.make_inputs("bound", 96, 64, 1, "f32", seed=41)
    gp, _ = run_gpu(inp)
    s = inp.slot_ids
    grow = (gp[s].astype(np.float64) ** 2).sum(2) - (inp.pool[s].astype(np.float64) ** 2).sum(2)
    assert np.all(grow <= inp.v.astype(np.float64) ** 2 + 1e-6)


def test_non_default_stream():
    inp = kda_inputs.make_inputs("stream", 16, 8, 1, "f16", seed=43)
    ref_pool, ref_out = run_gpu(inp)
    pool, ids, t, out = device_inputs(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        B.kda_decode_step(pool, ids, t["q"], t["k"], t["v"], t["g"], t["b"], out, stream=s)
    s.synchronize()
    np.testing.assert_array_equal(pool_to_host(pool), ref_pool)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref_out.view(np.uint32))


def test_binding_refuses_before_launch():
    inp = kda_inputs.make_inputs("refuse", 8, 2, 1, "f16", seed=47)
    pool, ids, t, out = device_inputs(inp)
    with pytest.raises(B.KdaError) as e:
        B.kda_decode_step(pool.view(torch.bfloat16), ids, t["q"], t["k"], t["v"], t["g"], t["b"], out)
    assert e.value.code == B.KDA_ERR_DTYPE_REFUSED
    with pytest.raises(B.KdaError) as e:
        B.kda_decode_step(pool, ids, t["q"], t["k"], t["v"], t["g"], t["b"], out, state_dtype="f32")
    assert e.value.code == B.KDA_ERR_DTYPE_MISMATCH
