"""Pins of the oracle's short causal convolution (the front end of the KDA
layer: q, k, v each pass a 4-tap depthwise causal conv, then SiLU; the slot
keeps the last 3 raw inputs per channel in bfloat16).

Sources: ROCm/ATOM PR #2130, Memory (1.91 MB per slot over 69 layers that
does not follow the state dtype = 3 entries x 4608 channels x 2 bytes);
ROCm/ATOM PR #2894, the two-node trial (a 3-entry history is read, then the
old entries and the step's inputs are written back).  Activation (SiLU), tap
order and the absence of a bias are readings; see the design notes.
"""
import json
import os

import numpy as np
import pytest

from numpy.lib.stride_tricks import sliding_window_view

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bf16_to_f32(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def make(n_slots, n_req, n_rows, C, seed):
    rng = np.random.default_rng(seed)
    pool = f32_to_bf16(rng.standard_normal((n_slots, 3, C), dtype=np.float32))
    x = rng.standard_normal((n_req * n_rows, C), dtype=np.float32)
    w = (rng.standard_normal((C, 4), dtype=np.float32) * 0.5).astype(np.float32)
    ids = rng.permutation(n_slots)[:n_req * n_rows].astype(np.int32)
    return pool, x, w, ids


def numpy_conv(pool, x, w, ids, n_rows, init=None):
    """fp64 sliding-window form of the same definition, and the expected
    bf16 snapshots."""
    R, C = x.shape
    y = np.zeros((R, C))
    snaps = {}
    for r in range(R // n_rows):
        s0 = ids[r * n_rows] if init is None else init[r]
        seq = np.concatenate([bf16_to_f32(pool[s0]).astype(np.float64),
                              x[r * n_rows:(r + 1) * n_rows].astype(np.float64)], axis=0)  # [3+n, C]
        win = sliding_window_view(seq, 4, axis=0)          # [n, C, 4]
        s = np.einsum("tcj,cj->tc", win, w.astype(np.float64))
        y[r * n_rows:(r + 1) * n_rows] = s / (1.0 + np.exp(-s))
        for t in range(n_rows):
            snaps[ids[r * n_rows + t]] = f32_to_bf16(seq[t + 1:t + 4].astype(np.float32))
    return y, snaps


@pytest.mark.parametrize("n_req,n_rows", [(3, 1), (2, 5), (4, 8)])
def test_conv_matches_sliding_window(oracle, n_req, n_rows):
    pool, x, w, ids = make(40, n_req, n_rows, 48, seed=n_req * 7 + n_rows)
    before = pool.copy()
    y = oracle.conv_f32(pool, ids, x, w, n_rows=n_rows)
    y_ref, snaps = numpy_conv(before, x, w, ids, n_rows)
    np.testing.assert_allclose(y, y_ref, rtol=2e-6, atol=1e-6)
    for s, h in snaps.items():
        np.testing.assert_array_equal(pool[s], h)
    untouched = np.setdiff1d(np.arange(40), ids)
    np.testing.assert_array_equal(pool[untouched], before[untouched])


def test_conv_with_initial_slots(oracle):
    pool, x, w, ids = make(40, 3, 4, 16, seed=3)
    init = np.setdiff1d(np.arange(40), ids)[:3].astype(np.int32)
    before = pool.copy()
    y = oracle.conv_f32(pool, ids, x, w, n_rows=4, init_slot_ids=init)
    y_ref, snaps = numpy_conv(before, x, w, ids, 4, init=init)
    np.testing.assert_allclose(y, y_ref, rtol=2e-6, atol=1e-6)
    for s, h in snaps.items():
        np.testing.assert_array_equal(pool[s], h)


def test_identity_taps_give_silu_of_input(oracle):
    pool, x, w, ids = make(8, 4, 2, 32, seed=5)
    w[:] = 0.0
    w[:, 3] = 1.0
    y = oracle.conv_f32(pool, ids, x, w, n_rows=2)
    xs = x.astype(np.float64)
    np.testing.assert_allclose(y, xs / (1.0 + np.exp(-xs)), rtol=1e-6, atol=1e-7)


def test_oldest_tap_reads_the_history(oracle):
    pool, x, w, ids = make(8, 2, 3, 32, seed=6)
    hist = bf16_to_f32(pool[ids[::3]]).astype(np.float64)     # [2, 3, C]
    w[:] = 0.0
    w[:, 0] = 1.0
    y = oracle.conv_f32(pool, ids, x, w, n_rows=3)
    for r in range(2):
        for t in range(3):
            h = hist[r, t]
            np.testing.assert_allclose(y[r * 3 + t], h / (1.0 + np.exp(-h)), rtol=1e-6, atol=1e-7)


def test_one_launch_equals_chained_launches_for_bf16_inputs(oracle):
    # with inputs already representable in bf16, storing the history between
    # launches loses nothing, so n rows at once = n single-row launches
    pool, x, w, ids = make(30, 2, 6, 24, seed=8)
    x = bf16_to_f32(f32_to_bf16(x))
    p1 = pool.copy()
    y1 = oracle.conv_f32(p1, ids, x, w, n_rows=6)
    p2 = pool.copy()
    y2 = np.zeros_like(y1)
    for r in range(2):
        for t in range(6):
            rho = r * 6 + t
            prev = ids[r * 6] if t == 0 else ids[rho - 1]
            y2[rho] = oracle.conv_f32(p2, ids[rho:rho + 1], x[rho:rho + 1], w, n_rows=1,
                                      init_slot_ids=np.array([prev], np.int32))[0]
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))
    np.testing.assert_array_equal(p1, p2)


def test_conv_state_size_matches_the_pages_memory_table():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_memory_table.json")))
    L, H, K, V = gold["layers"], gold["H"], gold["K"], gold["V"]
    rest_mb = gold["state_per_slot_MB"]["f32"] - L * H * K * V * 4 / 1e6
    conv_bytes = L * 3 * (3 * H * 128) * 2       # 3 entries x (q|k|v channels) x bf16
    assert abs(conv_bytes / 1e6 - rest_mb) <= 2 * gold["printed_precision_MB"]


def test_dropped_silu_is_caught(oracle):
    pool, x, w, ids = make(16, 2, 3, 16, seed=9)
    y_ref, _ = numpy_conv(pool.copy(), x, w, ids, 3)
    oracle.set_mutation(12)
    try:
        y = oracle.conv_f32(pool.copy(), ids, x, w, n_rows=3)
    finally:
        oracle.set_mutation(0)
    assert not np.allclose(y, y_ref, rtol=1e-4, atol=1e-5)


def test_log_decay_from_gate_closed_forms(oracle):
    # softplus(0) = ln 2; softplus(ln(e - 1)) = ln e = 1; softplus(x) -> x
    # for large x and -> e^x for very negative x
    g = oracle.log_decay_from_gate(np.array([0.0, np.log(np.e - 1.0), 40.0, -40.0]))
    assert g.dtype == np.float32
    assert g[0] == np.float32(-np.log(2.0))
    assert g[1] == np.float32(-1.0)
    assert g[2] == np.float32(-40.0)
    assert g[3] == np.float32(-np.exp(-40.0))


def test_log_decay_from_gate_identities(oracle):
    # softplus(x) - softplus(-x) = x, and e^g = 1 / (1 + e^x) (the decay the
    # kernels form without the logarithm), over a wide range of x
    x = np.linspace(-30.0, 30.0, 6001)
    g_pos = oracle.log_decay_from_gate(x).astype(np.float64)
    g_neg = oracle.log_decay_from_gate(-x).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(g_pos), np.abs(g_neg)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs((g_neg - g_pos) - x) <= 2 * ulp + 1e-300)
    a = np.exp(g_pos)
    ref = 1.0 / (1.0 + np.exp(x))
    assert np.all(np.abs(a - ref) <= 1.2e-7 * (1.0 + np.abs(x)) * ref)   # g's fp32 rounding, times |g|
    assert np.all(g_pos <= 0) and np.all(np.diff(g_pos) <= 0)   # a decay in (0, 1], falling with x
