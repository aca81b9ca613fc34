"""Pins of the CPU oracle against things other than itself.

The oracle (oracle/kda_oracle.c, an element loop) is checked against:
  * an independent dense-matrix formulation in fp64 (oracle/dense.py);
  * closed forms of the update (zero state, identity gate, the component
    along kn, the orthogonal complement);
  * the per-column norm-growth bound stated on ROCm/ATOM PR #2945
    (Limitations: unit k, beta in (0, 1), decay <= 1 -> a token adds at most
    v_j^2 to the squared norm of value column j);
  * the x86 F16C hardware conversion (exhaustive) and NumPy's float16 cast
    for the round-to-nearest-even store (ROCm/ATOM PR #2945, Changes);
  * structural facts: slots not named are untouched, a permutation of the
    requests permutes the results, a multi-row launch is its tokens chained.
Finally, planted mistakes in the oracle must each fail at least one pin.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import kda_inputs
from oracle import dense

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def small(n_slots=6, n_req=2, n_rows=1, dtype="f32", H=2, K=8, V=8, seed=1):
    return kda_inputs.make_inputs("small", n_slots, n_req, n_rows, dtype, H=H, K=K, V=V, seed=seed)


def f64_pool(inp):
    if inp.dtype == "f32":
        return inp.pool.astype(np.float64)
    return inp.pool.view(np.float16).astype(np.float64)


def run_f64(oracle, inp, pool=None, **kw):
    pool = f64_pool(inp) if pool is None else pool
    out = oracle.step_f64(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                          n_rows=inp.n_rows, scale=inp.scale, **kw)
    return pool, out


def run_f32(oracle, inp, pool=None):
    pool = inp.pool.copy() if pool is None else pool
    out = oracle.step_f32(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                          n_rows=inp.n_rows, scale=inp.scale)
    return pool, out


def run_dense(inp):
    pool = f64_pool(inp)
    out = dense.dense_launch(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                             n_rows=inp.n_rows, scale=inp.scale)
    return pool, out


# ---------------------------------------------------------------------------
# binary16 rounding
# ---------------------------------------------------------------------------

def _has_f16c():
    try:
        with open("/proc/cpuinfo") as f:
            return " f16c" in f.read()
    except OSError:
        return False


@pytest.mark.skipif(not _has_f16c() or shutil.which("gcc") is None,
                    reason="needs gcc and an x86 CPU with F16C")
def test_rne_exhaustive_against_f16c(tmp_path):
    exe = tmp_path / "rne_exhaustive"
    subprocess.run(["gcc", "-O2", "-mf16c", "-fopenmp", "-ffp-contract=off",
                    os.path.join(ROOT, "tests", "rne_exhaustive.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", str(exe), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "narrow_mismatches=0 widen_mismatches=0" in r.stdout


# Hand-derived binary16 encodings (IEEE 754: bias 15, 10 fraction bits).
TEXTBOOK = [
    (1.0, 0x3C00),
    (-2.0, 0xC000),
    (1.0 + 2.0 ** -11, 0x3C00),          # tie between 1 and 1+2^-10 -> even (1)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),      # tie between 1+2^-10 and 1+2^-9 -> even
    (1.0 + 2.0 ** -11 + 2.0 ** -20, 0x3C01),  # just above the tie -> up
    (65504.0, 0x7BFF),                   # largest finite
    (65519.0, 0x7BFF),                   # below the overflow midpoint
    (65520.0, 0x7C00),                   # midpoint, odd neighbour -> overflow
    (2.0 ** -14, 0x0400),                # smallest normal
    (2.0 ** -24, 0x0001),                # smallest subnormal
    (2.0 ** -25, 0x0000),                # tie between 0 and 2^-24 -> even (0)
    (3 * 2.0 ** -25, 0x0002),            # tie between 1 and 2 units -> even (2)
    (2.0 ** -25 * 1.0000001, 0x0001),    # above the tie -> up
    (-0.0, 0x8000),
    (float("inf"), 0x7C00),
    (float("-inf"), 0xFC00),
]


@pytest.mark.parametrize("x,bits", TEXTBOOK)
def test_rne_textbook_values(oracle, x, bits):
    got = int(oracle.f32_to_f16_rne(np.array([x], dtype=np.float32))[0])
    assert got == bits, "%r -> %#06x, expected %#06x" % (x, got, bits)


def test_rne_nan_stays_nan(oracle):
    x = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.all(np.isnan(oracle.f32_to_f16_rne(x).view(np.float16)))


def test_rne_random_and_boundaries_against_numpy(oracle):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-30, 18, 1 << 20))).astype(np.float32)
    # every binary16 value, and the binary32 neighbours of the midpoints
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), h])
    x = np.concatenate([x, near, -near])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16_rne(x), ref)


def test_widen_exhaustive_against_numpy(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------------------
# loop vs dense algebra
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("K,V", [(1, 1), (2, 4), (4, 2), (8, 8), (16, 16), (5, 3), (128, 128)])
@pytest.mark.parametrize("n_rows", [1, 3])
def test_loop_f64_matches_dense(oracle, K, V, n_rows):
    H = 2 if K < 128 else 3
    inp = small(n_slots=3 * n_rows + 1, n_req=3, n_rows=n_rows, H=H, K=K, V=V, seed=K * 10 + V)
    p_loop, o_loop = run_f64(oracle, inp)
    p_dense, o_dense = run_dense(inp)
    np.testing.assert_allclose(p_loop, p_dense, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o_loop, o_dense, rtol=1e-12, atol=1e-14)


def test_loop_f32_within_rounding_of_f64(oracle):
    inp = kda_inputs.make_inputs("f32 vs f64", 8, 4, 2, "f32", seed=3)
    p32, o32 = run_f32(oracle, inp)
    p64, o64 = run_f64(oracle, inp)
    # fp32 sums of 128 terms of size ~0.05: a few ulp of 0.1 (~1e-8 each)
    assert np.max(np.abs(p32 - p64)) < 2e-7
    rel = np.linalg.norm(o32 - o64, axis=-1) / np.linalg.norm(o64, axis=-1)
    assert rel.max() < 2e-6


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _unit(x):
    x = x.astype(np.float64)
    return x / np.sqrt(x @ x + dense.EPS)


def test_zero_state_closed_form(oracle):
    inp = kda_inputs.make_inputs("zero state", 4, 4, 1, "f32", seed=5)
    inp.pool[:] = 0.0
    pool, out = run_f64(oracle, inp)
    for r in range(4):
        for h in range(12):
            qn, kn = _unit(inp.q[r, h]), _unit(inp.k[r, h])
            beta = 1.0 / (1.0 + np.exp(-float(inp.b[r, h])))
            S1 = beta * np.outer(kn, inp.v[r, h].astype(np.float64))
            o = inp.scale * beta * (qn @ kn) * inp.v[r, h].astype(np.float64)
            np.testing.assert_allclose(pool[inp.slot_ids[r], h], S1, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(out[r, h], o, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_identity_gate_leaves_state_bit_unchanged(oracle, dtype):
    # g = 0 -> a = exp(0) = 1 exactly; b = -1e4 -> exp(1e4) = inf, beta = 0
    inp = kda_inputs.make_inputs("identity", 6, 2, 2, dtype, seed=9)
    inp.g[:] = 0.0
    inp.b[:] = -1e4
    before = inp.pool.copy()
    pool, out = run_f32(oracle, inp)
    for r in range(inp.n_req):
        s0 = inp.slot_ids[r * inp.n_rows]
        for t in range(inp.n_rows):
            np.testing.assert_array_equal(pool[inp.slot_ids[r * inp.n_rows + t]], before[s0])
    # o = scale * S0^T qn
    S0 = f64_pool(inp)
    for rho in range(inp.slot_ids.size):
        r = rho // inp.n_rows
        for h in range(12):
            ref = inp.scale * S0[inp.slot_ids[r * inp.n_rows], h].T @ _unit(inp.q[rho, h])
            np.testing.assert_allclose(out[rho, h], ref, rtol=1e-5, atol=1e-7)


def test_full_gate_writes_v_along_k(oracle):
    # b = +1e4 -> beta = 1/(1 + exp(-1e4)) = 1, g = 0 -> a = 1: kn^T S1 = v
    inp = kda_inputs.make_inputs("beta one", 4, 4, 1, "f32", seed=11)
    inp.g[:] = 0.0
    inp.b[:] = 1e4
    pool, _ = run_f64(oracle, inp)
    for r in range(4):
        for h in range(12):
            kn = _unit(inp.k[r, h])
            # kn has norm sqrt(s/(s+eps)), 1 - 1e-8 relative: allow for it
            np.testing.assert_allclose(kn @ pool[inp.slot_ids[r], h], inp.v[r, h], rtol=1e-7, atol=1e-7)


def test_orthogonal_complement_only_decays(oracle):
    inp = kda_inputs.make_inputs("complement", 4, 4, 1, "f32", seed=13)
    S0 = f64_pool(inp)
    pool, _ = run_f64(oracle, inp)
    for r in range(4):
        for h in range(12):
            kn = _unit(inp.k[r, h])
            kn = kn / np.linalg.norm(kn)
            P = np.eye(128) - np.outer(kn, kn)
            s = inp.slot_ids[r]
            Sp = np.exp(inp.g[r, h].astype(np.float64))[:, None] * S0[s, h]
            np.testing.assert_allclose(P @ pool[s, h], P @ Sp, rtol=1e-9, atol=1e-11)


def test_zero_vectors_give_zero_not_nan(oracle):
    inp = kda_inputs.make_inputs("zero q k", 2, 2, 1, "f32", seed=17)
    inp.q[0] = 0.0
    inp.k[1] = 0.0
    before = inp.pool.copy()
    pool, out = run_f32(oracle, inp)
    assert np.all(np.isfinite(pool)) and np.all(np.isfinite(out))
    assert np.all(out[0] == 0.0)
    # kn = 0: no correction, the state is only decayed
    s = inp.slot_ids[1]
    a = np.exp(inp.g[1].astype(np.float32))
    np.testing.assert_allclose(pool[s], a[:, :, None] * before[s], rtol=1e-6, atol=1e-9)


# ---------------------------------------------------------------------------
# the norm-growth bound (ROCm/ATOM PR #2945, Limitations)
# ---------------------------------------------------------------------------

def test_column_norm_growth_bound(oracle):
    inp = kda_inputs.make_inputs("bound", 16, 16, 1, "f32", seed=19)
    S0 = f64_pool(inp)
    pool, _ = run_f64(oracle, inp)
    for r in range(16):
        s = inp.slot_ids[r]
        for h in range(12):
            kn = _unit(inp.k[r, h])
            beta = 1.0 / (1.0 + np.exp(-float(inp.b[r, h])))
            Sp = np.exp(inp.g[r, h].astype(np.float64))[:, None] * S0[s, h]
            c = kn @ Sp
            v = inp.v[r, h].astype(np.float64)
            grow = (pool[s, h] ** 2).sum(0) - (S0[s, h] ** 2).sum(0)
            assert np.all(grow <= beta * (v ** 2 - c ** 2) + 1e-12)
            assert np.all(grow <= v ** 2 + 1e-12)


def test_column_norm_growth_bound_fp32_loop(oracle):
    inp = kda_inputs.make_inputs("bound f32", 16, 16, 1, "f32", seed=23)
    S0 = inp.pool.astype(np.float64)
    pool, _ = run_f32(oracle, inp)
    grow = (pool.astype(np.float64) ** 2).sum(2) - (S0 ** 2).sum(2)   # [slot, H, V]
    v2 = inp.v.astype(np.float64) ** 2
    for r in range(16):
        assert np.all(grow[inp.slot_ids[r]] <= v2[r] + 1e-6)


# ---------------------------------------------------------------------------
# fp16 pool = RNE of the fp32 chain; multi-row = chained tokens
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_req,n_rows", [(4, 1), (3, 4)])
def test_fp16_pool_is_rne_of_fp32_twin(oracle, n_req, n_rows):
    inp = kda_inputs.make_inputs("twin", 16, n_req, n_rows, "f16", seed=29)
    p16, o16 = run_f32(oracle, inp)
    twin = oracle.f16_to_f32(inp.pool)          # exact widening of the pool
    p32, o32 = run_f32(oracle, inp, pool=twin)
    np.testing.assert_array_equal(o16.view(np.uint32), o32.view(np.uint32))
    np.testing.assert_array_equal(p16, oracle.f32_to_f16_rne(p32))


def test_multirow_equals_chained_single_rows_fp32(oracle):
    inp = kda_inputs.make_inputs("chain", 20, 3, 5, "f32", seed=31)
    pool_m, out_m = run_f32(oracle, inp)
    pool_c = inp.pool.copy()
    out_c = np.zeros_like(out_m)
    for r in range(3):
        for t in range(5):
            rho = r * 5 + t
            if t > 0:   # carry the previous token's state into this row's slot
                pool_c[inp.slot_ids[rho]] = pool_c[inp.slot_ids[rho - 1]]
            sl = slice(rho, rho + 1)
            out_c[sl] = oracle.step_f32(pool_c, inp.slot_ids[sl], inp.q[sl], inp.k[sl], inp.v[sl],
                                        inp.g[sl], inp.b[sl], n_rows=1, scale=inp.scale)
    np.testing.assert_array_equal(pool_m.view(np.uint32), pool_c.view(np.uint32))
    np.testing.assert_array_equal(out_m.view(np.uint32), out_c.view(np.uint32))


def test_untouched_slots_and_permutation(oracle):
    inp = kda_inputs.make_inputs("perm", 12, 8, 1, "f16", seed=37)
    pool, out = run_f32(oracle, inp)
    named = set(int(s) for s in inp.slot_ids)
    for s in range(12):
        if s not in named:
            np.testing.assert_array_equal(pool[s], inp.pool[s])
    perm = np.random.default_rng(1).permutation(8)
    pool2 = inp.pool.copy()
    out2 = oracle.step_f32(pool2, inp.slot_ids[perm], inp.q[perm], inp.k[perm], inp.v[perm],
                           inp.g[perm], inp.b[perm], n_rows=1, scale=inp.scale)
    np.testing.assert_array_equal(pool2, pool)
    np.testing.assert_array_equal(out2, out[perm])


def test_oracle_rejects_bad_slot(oracle):
    inp = small()
    inp.slot_ids[0] = 99
    with pytest.raises(ValueError):
        run_f32(oracle, inp)


# ---------------------------------------------------------------------------
# planted mistakes must be caught
# ---------------------------------------------------------------------------

def _pins_pass(oracle) -> bool:
    """A compact battery of the pins above; False as soon as one fails."""
    for n_rows, K, V in [(1, 8, 8), (3, 8, 8), (2, 6, 6)]:
        inp = small(n_slots=10, n_req=3, n_rows=n_rows, K=K, V=V, seed=41 + n_rows)
        p64, o64 = run_f64(oracle, inp)
        pd, od = run_dense(inp)
        if not (np.allclose(p64, pd, rtol=1e-10, atol=1e-12) and np.allclose(o64, od, rtol=1e-10, atol=1e-12)):
            return False
        p32, o32 = run_f32(oracle, inp)
        if not (np.allclose(p32, pd, rtol=1e-4, atol=1e-5) and np.allclose(o32, od, rtol=1e-4, atol=1e-5)):
            return False
    return True


@pytest.mark.parametrize("mutation", list(range(1, 12)))
def test_planted_mistakes_are_caught(oracle, mutation):
    assert _pins_pass(oracle)
    oracle.set_mutation(mutation)
    try:
        caught = not _pins_pass(oracle)
    finally:
        oracle.set_mutation(0)
    assert caught, "planted mistake %d passed every pin" % mutation


# ---------------------------------------------------------------------------
# initial state read from a separate slot (accepted-count / checkpoint load)
# ---------------------------------------------------------------------------

def test_init_slot_equal_to_row0_slot_changes_nothing(oracle):
    inp = kda_inputs.make_inputs("init same", 20, 3, 4, "f16", seed=51)
    p1, o1 = run_f32(oracle, inp)
    p2 = inp.pool.copy()
    o2 = oracle.step_f32(p2, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=4,
                         scale=inp.scale, init_slot_ids=inp.slot_ids[::4])
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(o1.view(np.uint32), o2.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_init_slot_is_copy_then_launch(oracle, dtype):
    # reading the initial state from slot i is the same as first copying
    # slot i into the request's row-0 slot (NumPy copy) and launching as usual
    inp = kda_inputs.make_inputs("init other", 24, 3, 2, dtype, seed=53)
    free = np.setdiff1d(np.arange(24), inp.slot_ids)
    init = free[:3].astype(np.int32)
    p_init = inp.pool.copy()
    o_init = oracle.step_f32(p_init, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=2,
                             scale=inp.scale, init_slot_ids=init)
    p_copy = inp.pool.copy()
    for r in range(3):
        p_copy[inp.slot_ids[2 * r]] = p_copy[init[r]]
    o_copy = oracle.step_f32(p_copy, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=2,
                             scale=inp.scale)
    np.testing.assert_array_equal(p_init, p_copy)
    np.testing.assert_array_equal(o_init.view(np.uint32), o_copy.view(np.uint32))
    # and the init slots themselves are only read
    np.testing.assert_array_equal(p_init[init], inp.pool[init])


def test_init_slot_loop_matches_dense(oracle):
    inp = small(n_slots=12, n_req=3, n_rows=3, K=8, V=8, seed=57)
    init = np.array([11, 10, 9], dtype=np.int32)
    pool = f64_pool(inp)
    o_loop = oracle.step_f64(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=3,
                             scale=inp.scale, init_slot_ids=init)
    pd = f64_pool(inp)
    o_dense = dense.dense_launch(pd, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b, n_rows=3,
                                 scale=inp.scale, init_slot_ids=init)
    np.testing.assert_allclose(pool, pd, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o_loop, o_dense, rtol=1e-12, atol=1e-14)


def test_oracle_rejects_bad_init_slot(oracle):
    inp = small()
    with pytest.raises(ValueError):
        oracle.step_f32(inp.pool.copy(), inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                        init_slot_ids=np.array([0, 6], dtype=np.int32))
