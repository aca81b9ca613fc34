"""GPU parity of the decode step with the short causal convolution fused in
front (kda_decode_step_conv) against the oracle's composition: the
convolution (oracle.conv_f32) and then the decode (oracle.step_f32).

State and outputs to the decode tolerances; the convolution histories the
launch writes (RNE bfloat16 of raw inputs) bit for bit; slots not named
untouched in both pools."""
import numpy as np
import pytest

import kda_inputs
from gpu_helpers import (B, F16_ULP, OUT_REL, STATE_ABS_F32, f16_ulp_distance, need_gpu,
                         out_rel_err, pool_to_host, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def gpu_conv(ci, init=None, waves=0, block_rows=False, rows_layout=0, counts=None, bv=0):
    d = ci.dec
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(d.pool if d.dtype == "f32" else d.pool.view(np.float16)).to(dev)
    conv = torch.from_numpy(ci.conv).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(d.slot_ids).to(dev)
    x = torch.from_numpy(ci.x).to(dev)
    w = torch.from_numpy(ci.w).to(dev)
    g = torch.from_numpy(d.g).to(dev)
    b = torch.from_numpy(d.b).to(dev)
    out = torch.full((d.slot_ids.size, d.pool.shape[1], 128), float("nan"), device=dev)
    init_d = None if init is None else torch.from_numpy(np.asarray(init, np.int32)).to(dev)
    B.kda_decode_step_conv(pool, conv, ids, x, w, g, b, out, n_rows_per_slot=d.n_rows,
                           scale=d.scale, init_slot_ids=init_d, waves_per_tile=waves,
                           block_rows=block_rows, rows_layout=rows_layout, pair_counts=counts, bv=bv)
    torch.cuda.synchronize()
    return pool_to_host(pool), conv.view(torch.int16).cpu().numpy().view(np.uint16), out.cpu().numpy()


def oracle_conv(oracle, ci, init=None):
    d = ci.dec
    n_slots, H = d.pool.shape[0], d.pool.shape[1]
    C = 3 * H * 128
    conv = ci.conv.reshape(n_slots, 3, C).copy()
    R = d.slot_ids.size
    y = oracle.conv_f32(conv, d.slot_ids, ci.x.reshape(R, C), ci.w.reshape(C, 4),
                        n_rows=d.n_rows, init_slot_ids=init).reshape(R, 3, H, 128)
    pool = d.pool.copy()
    out = oracle.step_f32(pool, d.slot_ids, np.ascontiguousarray(y[:, 0]), np.ascontiguousarray(y[:, 1]),
                          np.ascontiguousarray(y[:, 2]), d.g, d.b, n_rows=d.n_rows, scale=d.scale,
                          init_slot_ids=init)
    return pool, conv.reshape(ci.conv.shape), out


def check(oracle, ci, init=None, waves=0, block_rows=False, rows_layout=0, counts=None, bv=0):
    gp, gc, go = gpu_conv(ci, init, waves, block_rows, rows_layout, counts, bv)
    op, oc, oo = oracle_conv(oracle, ci, init)
    d = ci.dec
    if d.dtype == "f32":
        assert np.max(np.abs(gp - op)) <= STATE_ABS_F32
    else:
        assert f16_ulp_distance(gp, op).max() <= F16_ULP
    assert out_rel_err(go, oo) <= OUT_REL
    np.testing.assert_array_equal(gc, oc)
    untouched = np.setdiff1d(np.arange(d.pool.shape[0]), np.concatenate(
        [d.slot_ids, [] if init is None else np.asarray(init)]).astype(int))
    np.testing.assert_array_equal(gc[untouched], ci.conv[untouched])
    np.testing.assert_array_equal(gp[untouched], d.pool[untouched])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_req,n_rows", [(64, 1), (8, 8), (3, 5)])
def test_fused_conv_parity(oracle, dtype, n_req, n_rows):
    ci = kda_inputs.make_conv_inputs("conv", 96, n_req, n_rows, dtype, seed=101 + n_rows)
    check(oracle, ci)


@pytest.mark.parametrize("waves", [2, 4, 8])
@pytest.mark.parametrize("n_rows", [1, 6])
def test_fused_conv_every_wave_count(oracle, waves, n_rows):
    ci = kda_inputs.make_conv_inputs("conv waves", 40, 4, n_rows, "f16", H=3, seed=131 + waves)
    check(oracle, ci, waves=waves)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_fused_conv_rows_as_block(oracle, dtype):
    ci = kda_inputs.make_conv_inputs("conv block", 64, 6, 7, dtype, H=4, seed=161)
    check(oracle, ci, block_rows=True)


@pytest.mark.parametrize("n_rows", [1, 4])
def test_fused_conv_initial_slots(oracle, n_rows):
    ci = kda_inputs.make_conv_inputs("conv init", 64, 6, n_rows, "f32", seed=141)
    free = np.setdiff1d(np.arange(64), ci.dec.slot_ids)
    init = np.random.default_rng(3).permutation(free)[:6].astype(np.int32)
    check(oracle, ci, init=init)


def test_fused_conv_identity_taps_equal_plain_decode_of_silu(oracle):
    # taps (0, 0, 0, 1): q, k, v = silu(x); the state update must then equal
    # the plain decode launched on silu(x) (same kernels downstream)
    ci = kda_inputs.make_conv_inputs("conv id", 32, 8, 1, "f32", seed=151)
    ci.w[:] = 0.0
    ci.w[..., 3] = 1.0
    gp, gc, go = gpu_conv(ci)
    d = ci.dec
    xs = ci.x.astype(np.float64)
    y = (xs / (1.0 + np.exp(-xs))).astype(np.float32)
    op = d.pool.copy()
    oo = oracle.step_f32(op, d.slot_ids, np.ascontiguousarray(y[:, 0]), np.ascontiguousarray(y[:, 1]),
                         np.ascontiguousarray(y[:, 2]), d.g, d.b, n_rows=1, scale=d.scale)
    assert np.max(np.abs(gp - op)) <= STATE_ABS_F32
    assert out_rel_err(go, oo) <= OUT_REL


# (waves, rows_layout, pair counters) of the layouts chained rows can take
# with the convolution fused: the matrix-core block form over whole heads of
# 16 waves (two halves of 8, the default without counters) or of 8 (two
# halves of 4), over 64-column halves of 8 waves (the default with
# counters), and the K-split layout
LAYOUTS = {"matrix16": (0, B.KDA_ROWS_MATRIX, False), "matrix8": (8, B.KDA_ROWS_MATRIX, False),
           "halves": (0, B.KDA_ROWS_MATRIX, True), "k_split": (0, B.KDA_ROWS_K_SPLIT, False)}


def counters(ci):
    return B.conv_pair_counts(ci.dec.n_req, ci.dec.pool.shape[1], torch.device("cuda", 0))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("n_req,n_rows", [(8, 8), (3, 5), (5, 2)])
@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_fused_conv_chained_rows_in_every_layout(oracle, dtype, n_req, n_rows, layout):
    """Chained rows with the convolution fused in front, in both matrix-core
    block forms (whole heads) and in the K-split layout."""
    ci = kda_inputs.make_conv_inputs("conv layouts", 72, n_req, n_rows, dtype, H=12 if n_req == 8 else 3,
                                     seed=150 + 7 * n_req + n_rows)
    waves, rows_layout, pairs = LAYOUTS[layout]
    check(oracle, ci, waves=waves, rows_layout=rows_layout, counts=counters(ci) if pairs else None)


@pytest.mark.parametrize("dtype,n_req,n_rows", [("f16", 20, 6), ("f16", 21, 8), ("f32", 8, 4), ("f32", 8, 3)])
def test_fused_conv_default_layout_with_counters_at_its_bounds(oracle, dtype, n_req, n_rows):
    """The default layout with pair counters on either side of the halves'
    bounds (fp16: 240 requests x heads from 6 rows, then the K split; fp32:
    96 from 4 rows, then the K split), requests in place at row 0."""
    ci = kda_inputs.make_conv_inputs("conv bounds", n_req * n_rows + 8, n_req, n_rows, dtype,
                                     seed=170 + n_req + n_rows)
    init = ci.dec.slot_ids.reshape(n_req, n_rows)[:, 0].copy()
    check(oracle, ci, init=init, counts=counters(ci))


MATRIX_FORMS = ["matrix16", "matrix8", "halves"]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("form", MATRIX_FORMS)
def test_fused_conv_matrix_initial_slots_and_in_place_history(oracle, dtype, form):
    """The matrix-core forms read the history at the initial slot and write
    row 0's history at the same slot (in place) or at another one."""
    ci = kda_inputs.make_conv_inputs("conv matrix init", 64, 4, 6, dtype, H=3, seed=171)
    free = np.setdiff1d(np.arange(64), ci.dec.slot_ids)
    init = np.random.default_rng(5).permutation(free)[:4].astype(np.int32)
    waves, rows_layout, pairs = LAYOUTS[form]
    counts = counters(ci) if pairs else None
    check(oracle, ci, init=init, waves=waves, rows_layout=rows_layout, counts=counts)
    check(oracle, ci, waves=waves, rows_layout=rows_layout, counts=counts)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_fused_conv_halves_in_place_at_any_row(oracle, dtype):
    """The halves hand over the history of whichever row's slot is the
    initial slot (row 0 of one request, a later row of another, none of a
    third), and their counters stay even: 2 per launch where a row is in
    place, untouched elsewhere."""
    n_req, n_rows, H = 3, 5, 3
    ci = kda_inputs.make_conv_inputs("conv halves rows", 48, n_req, n_rows, dtype, H=H, seed=191)
    ids = ci.dec.slot_ids.reshape(n_req, n_rows)
    free = np.setdiff1d(np.arange(48), ids)
    init = np.array([ids[0, 0], ids[1, 3], free[0]], np.int32)
    counts = counters(ci)
    for launch in range(3):
        check(oracle, ci, init=init, counts=counts)
        c = counts.cpu().numpy().reshape(n_req, H)
        np.testing.assert_array_equal(c, np.array([2, 2, 0])[:, None] * (launch + 1) * np.ones((1, H)))


def test_fused_conv_halves_on_counters_left_by_earlier_launches(oracle):
    """Counters serve launches of any size in a row (each launch adds 0 or 2,
    so they stay even), the buffer may be longer than a launch needs, and an
    explicit bv of 128 keeps whole heads with counters given."""
    ci8 = kda_inputs.make_conv_inputs("conv halves big", 96, 8, 8, "f16", H=12, seed=193)
    ci3 = kda_inputs.make_conv_inputs("conv halves small", 40, 3, 4, "f16", H=3, seed=194)
    counts = B.conv_pair_counts(8, 12, torch.device("cuda", 0))
    counts.fill_(6)  # even, as an earlier sequence of launches leaves them
    check(oracle, ci8, counts=counts)
    check(oracle, ci3, counts=counts)
    check(oracle, ci3, counts=counts, bv=128)
    check(oracle, ci8, counts=counts)
    assert bool((counts.remainder(2) == 0).all())


@pytest.mark.parametrize("form", MATRIX_FORMS)
@pytest.mark.parametrize("n_rows", [2, 8])
def test_fused_conv_matrix_skips_a_request_with_a_bad_id(oracle, form, n_rows):
    """A request with a slot id out of range gets NaN outputs and leaves its
    slots' state and history untouched; the others are processed as usual."""
    n_req, bad = 3, 1
    ci = kda_inputs.make_conv_inputs("conv matrix bad id", 40, n_req, n_rows, "f16", H=3,
                                     seed=181 + n_rows)
    d = ci.dec
    ids = d.slot_ids.copy()
    ids[bad * n_rows + n_rows - 1] = 40              # one past the end
    d.slot_ids = ids
    waves, rows_layout, pairs = LAYOUTS[form]
    counts = counters(ci) if pairs else None
    gp, gc, go = gpu_conv(ci, waves=waves, rows_layout=rows_layout, counts=counts)
    if pairs:  # the skipped request took no counter
        assert int(counts.view(-1)[bad * 3:(bad + 1) * 3].abs().sum()) == 0
    rows = slice(bad * n_rows, (bad + 1) * n_rows)
    assert np.all(np.isnan(go[rows]))
    named = ids[rows][:-1]
    np.testing.assert_array_equal(gp[named], ci.dec.pool.view(np.uint16)[named])
    np.testing.assert_array_equal(gc[named], ci.conv[named])
    good = [r for r in range(n_req) if r != bad]
    sel = np.concatenate([np.arange(r * n_rows, (r + 1) * n_rows) for r in good])
    sub_dec = kda_inputs.DecodeInputs("good", "f16", d.pool.copy(), ids[sel], d.q[sel], d.k[sel],
                                      d.v[sel], d.g[sel], d.b[sel], n_rows, d.scale)
    sub = kda_inputs.ConvInputs(sub_dec, ci.conv.copy(), ci.x[sel], ci.w)
    op, oc, oo = oracle_conv(oracle, sub)
    assert out_rel_err(go[sel], oo) <= OUT_REL
    assert f16_ulp_distance(gp[ids[sel]], op[ids[sel]]).max() <= F16_ULP
    np.testing.assert_array_equal(gc[ids[sel]], oc[ids[sel]])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("layout", ["single_row", "halves", "matrix16", "matrix8", "k_split"])
def test_fused_conv_with_the_raw_gate(oracle, dtype, layout):
    """g_raw: the launch gets the raw gate x and takes the log-decay
    -softplus(x) itself; the oracle forms g from x (log_decay_from_gate)
    and runs the usual composition.  Every fused layout."""
    n_rows = 1 if layout == "single_row" else 5
    ci = kda_inputs.make_conv_inputs("conv gate", 48, 4, n_rows, dtype, H=3, seed=221 + n_rows)
    raw = np.random.default_rng(7).standard_normal(ci.dec.g.shape).astype(np.float32) * np.float32(2.0)
    waves, rows_layout, pairs = (0, 0, False) if layout == "single_row" else LAYOUTS[layout]
    d = ci.dec
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(d.pool if d.dtype == "f32" else d.pool.view(np.float16)).to(dev)
    conv = torch.from_numpy(ci.conv).to(dev).view(torch.bfloat16)
    t = {n: torch.from_numpy(getattr(src, n)).to(dev) for src, n in ((d, "slot_ids"), (ci, "x"), (ci, "w"), (d, "b"))}
    out = torch.full((d.slot_ids.size, d.pool.shape[1], 128), float("nan"), device=dev)
    counts = counters(ci) if pairs else None
    B.kda_decode_step_conv(pool, conv, t["slot_ids"], t["x"], t["w"], torch.from_numpy(raw).to(dev), t["b"], out,
                           n_rows_per_slot=n_rows, scale=d.scale, waves_per_tile=waves, rows_layout=rows_layout,
                           pair_counts=counts, g_raw=True)
    torch.cuda.synchronize()
    gp, gc, go = pool_to_host(pool), conv.view(torch.int16).cpu().numpy().view(np.uint16), out.cpu().numpy()
    d.g = oracle.log_decay_from_gate(raw)
    op, oc, oo = oracle_conv(oracle, ci)
    if dtype == "f32":
        assert np.max(np.abs(gp - op)) <= STATE_ABS_F32
    else:
        assert f16_ulp_distance(gp, op).max() <= F16_ULP
    assert out_rel_err(go, oo) <= OUT_REL
    np.testing.assert_array_equal(gc, oc)
