"""GPU parity of the matrix-core block form of chained rows
(KDA_ROWS_MATRIX, kda_rows_mfma_kernel) against the CPU oracle.

The block form computes the same recurrence as the token-by-token oracle,
reassociated: the column sums of every row come from one product of the
initial state with the stacked weights gamma_t kn_t, gamma_t qn_t (fp32 on
the matrix cores), the n x n couplings and a triangular solve per column.
It is graded with the decode bounds (fp32: 1e-6 abs state against the fp32
and fp64 oracles, 1e-5 relative output; fp16: 1 ulp of the oracle's RNE
state).  Cases: the 8 x 8 fp16 workload and its fp32 pool at full size,
every row count 2..8, ragged small shapes, the fp16/fp32 twin (same
arithmetic on the exactly widened state: outputs bit-equal, fp16 snapshots
the RNE of the fp32 ones), initial states from other slots, an out-of-range
slot id, the identity gate, strong decays whose cumulative products
underflow, decays of about -5 per row on every channel, heads in different
decay regimes in one launch, zero q and k, slots beyond 2^31 pool elements.
"""
import sys

import numpy as np
import pytest

import kda_inputs
from gpu_helpers import (B, F16_ULP, OUT_REL, STATE_ABS_F32, check_parity, device_inputs,
                         f16_ulp_distance, need_gpu, out_rel_err, pool_to_host, run_gpu,
                         run_oracle_f32, run_oracle_f64, torch)

pytestmark = pytest.mark.gpu

MATRIX = dict(rows_layout=B.KDA_ROWS_MATRIX)


def strong_decay_bound(oracle_err64: float) -> float:
    """Output bound against fp64 where decays are strong enough that the
    fp32 oracle's own outputs leave 1e-5: the kernel may be at most half as
    far again from fp64 as the oracle's own rounding (and always 1e-5)."""
    return max(OUT_REL, 1.5 * oracle_err64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# the default form (K over 8 waves) and the 4-wave form (waves_per_tile = 4)
FORMS = [0, 4]


@pytest.mark.parametrize("waves", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_full_size_spec_verify(oracle, dtype, waves):
    inp = kda_inputs.make_inputs("matrix 8x8", 96, 8, 8, dtype, seed=0)
    say("matrix block form, 8 req x 8 rows, H=12,", dtype, "waves", waves or 8)
    gp, go = run_gpu(inp, waves_per_tile=waves, **MATRIX)
    say(check_parity(oracle, inp, gp, go, label="matrix 8x8 %s" % dtype))


@pytest.mark.parametrize("waves", FORMS)
@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_rows", [2, 3, 4, 5, 6, 7, 8])
def test_every_row_count(oracle, dtype, n_rows, waves):
    inp = kda_inputs.make_inputs("matrix rows", 40, 40 // n_rows, n_rows, dtype, H=3,
                                 seed=300 + n_rows)
    gp, go = run_gpu(inp, waves_per_tile=waves, **MATRIX)
    check_parity(oracle, inp, gp, go, label="matrix %s n=%d waves %d" % (dtype, n_rows, waves or 8))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_req,H,n_rows", [(1, 1, 8), (3, 2, 3), (2, 5, 8), (4, 3, 7), (2, 3, 2),
                                            (5, 1, 4)])
def test_small_shapes(oracle, dtype, n_req, H, n_rows):
    n_slots = n_req * n_rows + 3
    inp = kda_inputs.make_inputs("matrix small", n_slots, n_req, n_rows, dtype, H=H,
                                 seed=3000 + 7 * n_req + 31 * H + n_rows)
    gp, go = run_gpu(inp, **MATRIX)
    check_parity(oracle, inp, gp, go, label="matrix small %s %dx%dx%d" % (dtype, n_req, H, n_rows))


@pytest.mark.parametrize("waves", FORMS)
@pytest.mark.parametrize("n_rows", [2, 8])
def test_fp32_twin_of_fp16_launch(n_rows, waves):
    """One kernel template for both pools, in either form: on the exactly
    widened state the fp32 arithmetic is identical, so outputs are
    bit-equal and every fp16 snapshot is the RNE of the fp32 one (ROCm/ATOM
    PR #2945, Testing: the fp32 twin of spec-verify launches)."""
    inp16 = kda_inputs.make_inputs("twin matrix", 96, 64 // n_rows, n_rows, "f16", seed=26 + n_rows)
    inp32 = kda_inputs.DecodeInputs("twin32", "f32", inp16.pool.view(np.float16).astype(np.float32),
                                    inp16.slot_ids, inp16.q, inp16.k, inp16.v, inp16.g, inp16.b,
                                    n_rows, inp16.scale)
    p16, o16 = run_gpu(inp16, waves_per_tile=waves, **MATRIX)
    p32, o32 = run_gpu(inp32, waves_per_tile=waves, **MATRIX)
    np.testing.assert_array_equal(o16.view(np.uint32), o32.view(np.uint32))
    np.testing.assert_array_equal(p16, p32.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_agrees_with_the_other_layouts(dtype):
    """The same launch in the row-after-row layouts: every result within
    rounding (fp32 state 1e-6, fp16 1 ulp, outputs 1e-5)."""
    inp = kda_inputs.make_inputs("layouts", 96, 8, 8, dtype, seed=44)
    gm, om = run_gpu(inp, **MATRIX)
    for layout in (B.KDA_ROWS_K_SPLIT, B.KDA_ROWS_WAVE_K):
        gp, go = run_gpu(inp, rows_layout=layout)
        if dtype == "f32":
            assert np.max(np.abs(gp - gm)) <= STATE_ABS_F32
        else:
            assert f16_ulp_distance(gp, gm).max() <= F16_ULP
        assert out_rel_err(go, om) <= OUT_REL


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_initial_state_from_other_slots(oracle, dtype):
    n_req, n_rows = 8, 8
    inp = kda_inputs.make_inputs("matrix init", 128, n_req, n_rows, dtype, seed=62)
    free = np.setdiff1d(np.arange(128), inp.slot_ids)
    init = np.random.default_rng(3).permutation(free)[:n_req].astype(np.int32)
    pool, ids, t, out = device_inputs(inp)
    B.kda_decode_step(pool, ids, t["q"], t["k"], t["v"], t["g"], t["b"], out, n_rows_per_slot=n_rows,
                      scale=inp.scale, init_slot_ids=torch.from_numpy(init).cuda(), **MATRIX)
    torch.cuda.synchronize()
    gp, go = pool_to_host(pool), out.cpu().numpy()
    op = inp.pool.copy()
    oo = oracle.step_f32(op, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=n_rows,
                         scale=inp.scale, init_slot_ids=init)
    if dtype == "f32":
        assert np.max(np.abs(gp - op)) <= STATE_ABS_F32
    else:
        assert f16_ulp_distance(gp, op).max() <= F16_ULP
    assert out_rel_err(go, oo) <= OUT_REL
    np.testing.assert_array_equal(gp[init], inp.pool[init])   # initial slots only read


def test_out_of_range_slot_is_skipped(oracle):
    n_req, n_rows = 3, 4
    inp = kda_inputs.make_inputs("matrix bad id", 16, n_req, n_rows, "f16", H=2, seed=8)
    ids = inp.slot_ids.copy()
    ids[1 * n_rows + 2] = 16  # one past the end, request 1
    pool, dids, t, out = device_inputs(inp)
    dids.copy_(torch.from_numpy(ids))
    before = pool_to_host(pool).copy()
    B.kda_decode_step(pool, dids, t["q"], t["k"], t["v"], t["g"], t["b"], out,
                      n_rows_per_slot=n_rows, **MATRIX)
    torch.cuda.synchronize()
    after, o = pool_to_host(pool), out.cpu().numpy()
    bad = slice(n_rows, 2 * n_rows)
    assert np.all(np.isnan(o[bad]))
    np.testing.assert_array_equal(after[inp.slot_ids[bad]], before[inp.slot_ids[bad]])
    good = np.r_[0:n_rows, 2 * n_rows:3 * n_rows]
    sub = kda_inputs.DecodeInputs("good", "f16", inp.pool.copy(), inp.slot_ids[good], inp.q[good],
                                  inp.k[good], inp.v[good], inp.g[good], inp.b[good], n_rows,
                                  inp.scale)
    op = sub.pool.copy()
    oo = oracle.step_f32(op, sub.slot_ids, sub.q, sub.k, sub.v, sub.g, sub.b, n_rows=n_rows,
                         scale=sub.scale)
    assert out_rel_err(o[good], oo) <= OUT_REL
    assert f16_ulp_distance(after[sub.slot_ids], op[sub.slot_ids]).max() <= F16_ULP


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_identity_gate_keeps_state_bits(oracle, dtype):
    # a = 1 and beta = 0 exactly: Delta = 0, every snapshot equals S0
    inp = kda_inputs.make_inputs("matrix identity", 24, 3, 8, dtype, seed=12)
    inp.g[:] = 0.0
    inp.b[:] = -1e4
    gp, go = run_gpu(inp, **MATRIX)
    as_float = (lambda x: x) if dtype == "f32" else (lambda x: x.view(np.float16))
    for r in range(3):
        s0 = inp.slot_ids[r * 8]
        for t in range(8):
            assert np.array_equal(as_float(gp[inp.slot_ids[r * 8 + t]]), as_float(inp.pool[s0]))
    check_parity(oracle, inp, gp, go, label="matrix identity")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_strong_decays_underflow_cleanly(oracle, dtype):
    """Log-decays down to -60 per row: the cumulative products gamma_t and
    E_ts underflow to zero (no division, so no inf or NaN) and the results
    stay within the bounds."""
    inp = kda_inputs.make_inputs("matrix strong decay", 40, 5, 8, dtype, H=3, seed=71)
    rng = np.random.default_rng(72)
    strong = rng.random(inp.g.shape) < 0.3
    inp.g[strong] = -rng.uniform(20.0, 60.0, size=int(strong.sum())).astype(np.float32)
    gp, go = run_gpu(inp, **MATRIX)
    assert np.all(np.isfinite(go))
    check_parity(oracle, inp, gp, go, label="matrix strong decay %s" % dtype)


def test_zero_q_and_k_stay_finite(oracle):
    inp = kda_inputs.make_inputs("matrix zero qk", 40, 5, 8, "f32", H=2, seed=73)
    inp.q[3] = 0.0
    inp.k[3] = 0.0
    inp.k[10, 1] = 0.0
    gp, go = run_gpu(inp, **MATRIX)
    assert np.all(np.isfinite(gp)) and np.all(np.isfinite(go))
    check_parity(oracle, inp, gp, go, label="matrix zero qk")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_decays_of_minus_5_per_row(oracle, dtype):
    """Log-decays of about -5 per row on every channel: after 8 rows the
    cumulative decay is about e^-40 (2^-58), so the stacked weights span 58
    binades while the couplings stay of order one."""
    inp = kda_inputs.make_inputs("matrix edge decay", 40, 5, 8, dtype, H=3, seed=74)
    rng = np.random.default_rng(75)
    inp.g[:] = -rng.uniform(4.8, 5.1, size=inp.g.shape).astype(np.float32)
    gp, go = run_gpu(inp, **MATRIX)
    written = np.unique(inp.slot_ids)
    o_pool32, o_out32 = run_oracle_f32(oracle, inp)
    _, o_out64 = run_oracle_f64(oracle, inp)
    if dtype == "f32":
        assert np.max(np.abs(gp[written] - o_pool32[written])) <= STATE_ABS_F32
    else:
        assert f16_ulp_distance(gp[written], o_pool32[written]).max() <= F16_ULP
    # Under decays this strong the fp32 oracle's own outputs are about 1.5e-5
    # from fp64 here, so outputs are graded against fp64 relative to the
    # oracle's own error; the row-after-row layout is held to the same bound.
    o_err = out_rel_err(o_out32, o_out64)
    bound = strong_decay_bound(o_err)
    err = out_rel_err(go, o_out64)
    _, go_seq = run_gpu(inp, rows_layout=B.KDA_ROWS_K_SPLIT)
    err_seq = out_rel_err(go_seq, o_out64)
    say("edge decay %s: out rel vs fp64 %.3g (row after row %.3g, fp32 oracle %.3g, bound %.3g)" % (
        dtype, err, err_seq, o_err, bound))
    assert err <= bound
    assert err_seq <= bound


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_heads_in_different_decay_regimes(oracle, dtype):
    """One head with decays of -12 per row (its cumulative decays underflow
    within the request) and two with the usual draws, in one launch."""
    inp = kda_inputs.make_inputs("matrix mixed decay", 40, 5, 8, dtype, H=3, seed=76)
    inp.g[:, 1, :] = -12.0
    gp, go = run_gpu(inp, **MATRIX)
    written = np.unique(inp.slot_ids)
    o_pool32, o_out32 = run_oracle_f32(oracle, inp)
    _, o_out64 = run_oracle_f64(oracle, inp)
    if dtype == "f32":
        assert np.max(np.abs(gp[written] - o_pool32[written])) <= STATE_ABS_F32
    else:
        assert f16_ulp_distance(gp[written], o_pool32[written]).max() <= F16_ULP
    # heads 0 and 2: the decode bound; head 1 (decays of -12 per row: the
    # fp32 oracle's outputs are 2e-5 from fp64) the strong-decay bound
    # against fp64, relative to the oracle's own error; the row-after-row
    # layout is held to the same bounds
    both = [0, 2]
    _, go_seq = run_gpu(inp, rows_layout=B.KDA_ROWS_K_SPLIT)
    bound = strong_decay_bound(out_rel_err(o_out32[:, 1:2], o_out64[:, 1:2]))
    say("mixed decay %s: head 1 out rel vs fp64 %.3g (row after row %.3g, bound %.3g)" % (
        dtype, out_rel_err(go[:, 1:2], o_out64[:, 1:2]), out_rel_err(go_seq[:, 1:2], o_out64[:, 1:2]),
        bound))
    for o in (go, go_seq):
        assert out_rel_err(o[:, both], o_out32[:, both]) <= OUT_REL
        assert out_rel_err(o[:, both], o_out64[:, both]) <= OUT_REL
        assert out_rel_err(o[:, 1:2], o_out64[:, 1:2]) <= bound


def test_64bit_pool_offsets(oracle):
    """Snapshot and initial slots beyond 2^31 pool elements: an fp16 pool of
    11,000 slots (4.3 GB), 2 requests x 4 rows near its top."""
    n_slots, H, n_req, n_rows = 11000, 12, 2, 4
    inp = kda_inputs.make_inputs("matrix high slots", 8, n_req, n_rows, "f16", seed=77)
    high = np.array([10999, 10990, 10950, 10925, 10930, 10998, 10960, 10940], dtype=np.int32)
    remap = dict(zip(inp.slot_ids.tolist(), high.tolist()))   # compact slot -> high slot
    pool = torch.zeros((n_slots, H, 128, 128), dtype=torch.float16, device="cuda")
    for s_small, s_big in remap.items():
        pool[s_big] = torch.from_numpy(inp.pool[s_small].view(np.float16)).cuda()
    ids = torch.from_numpy(np.array([remap[s] for s in inp.slot_ids.tolist()], dtype=np.int32)).cuda()
    dev = {n: torch.from_numpy(getattr(inp, n)).cuda() for n in ("q", "k", "v", "g", "b")}
    out = torch.empty((n_req * n_rows, H, 128), dtype=torch.float32, device="cuda")
    B.kda_decode_step(pool, ids, dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], out,
                      n_rows_per_slot=n_rows, **MATRIX)
    torch.cuda.synchronize()
    got = pool[ids.long()].cpu().numpy().view(np.uint16)
    o_pool, o_out = run_oracle_f32(oracle, inp)
    assert f16_ulp_distance(got, o_pool[inp.slot_ids]).max() <= F16_ULP
    assert out_rel_err(out.cpu().numpy(), o_out) <= OUT_REL
    assert int(high.min()) * H * 128 * 128 > 2 ** 31
    del pool
    torch.cuda.empty_cache()
