"""Pins of the oracle's prefill (whole sequences through the decode
recurrence; ROCm/ATOM PR #2130, What and Depends on: the prefill kernel takes
its initial state from the pool in the pool's dtype and the recurrence runs
in fp32 whatever the pool stores).

- The prefill oracle equals the decode oracle run one token per launch
  (bitwise in fp32): the sequence bookkeeping (cu_seqlens, initial and
  destination slots, empty sequences) is what is new here.
- Its fp64 twin equals the dense matrix form token after token.
- The chunked form that a parallel prefill computes (per-channel cumulative
  log-decay, a unit lower-triangular solve per chunk, matrix products for
  the outputs and the chunk-end state) equals the recurrence in fp64 to
  rounding.  It is written here from the algebra, with the same block
  references that keep every exponential bounded, so the algebra the GPU
  kernel relies on is pinned independently of any kernel.
"""
import numpy as np
import pytest

import kda_inputs
from oracle import dense

EPS = 1e-6


def chained_decode_f32(oracle, inp):
    """The decode oracle, one token per launch, on a one-slot pool per
    sequence; returns (pool after, out)."""
    pool = inp.pool.copy()
    T = inp.n_tokens
    _, H, K, V = pool.shape
    out = np.zeros((T, H, V), dtype=np.float32)
    finals = []
    for s in range(inp.init_slot_ids.size):
        # the chain runs in fp32 (an fp16 pool is widened exactly) and only
        # the final state rounds, so the decode launches run on an fp32 copy
        one = pool[inp.init_slot_ids[s]][None].copy()
        if inp.dtype == "f16":
            one = oracle.f16_to_f32(one)
        for t in range(inp.cu_seqlens[s], inp.cu_seqlens[s + 1]):
            out[t] = oracle.step_f32(one, np.zeros(1, np.int32), inp.q[t:t + 1], inp.k[t:t + 1],
                                     inp.v[t:t + 1], inp.g[t:t + 1], inp.b[t:t + 1],
                                     scale=inp.scale)[0]
        finals.append(one[0])
    for s, st in enumerate(finals):
        pool[inp.dst_slot_ids[s]] = oracle.f32_to_f16_rne(st) if inp.dtype == "f16" else st
    return pool, out


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("in_place", [True, False])
def test_prefill_equals_chained_decode(oracle, dtype, in_place):
    inp = kda_inputs.make_prefill_inputs("pin", [5, 0, 1, 9, 3], 12, dtype, H=2, K=16, V=8,
                                         seed=3, in_place=in_place)
    ref_pool, ref_out = chained_decode_f32(oracle, inp)
    pool = inp.pool.copy()
    out = oracle.prefill_f32(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g,
                             inp.b, dst_slot_ids=inp.dst_slot_ids, scale=inp.scale)
    np.testing.assert_array_equal(pool, ref_pool)
    np.testing.assert_array_equal(out, ref_out)


def test_prefill_f64_equals_dense(oracle):
    inp = kda_inputs.make_prefill_inputs("pin", [4, 7, 0, 2], 8, "f32", H=2, K=8, V=5, seed=5,
                                         in_place=False)
    pool = inp.pool.astype(np.float64)
    out = oracle.prefill_f64(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g,
                             inp.b, dst_slot_ids=inp.dst_slot_ids, scale=inp.scale)
    ref = inp.pool.astype(np.float64)
    for s in range(inp.init_slot_ids.size):
        for h in range(2):
            S = ref[inp.init_slot_ids[s], h].copy()
            for t in range(inp.cu_seqlens[s], inp.cu_seqlens[s + 1]):
                S, o = dense.dense_token(S, inp.q[t, h], inp.k[t, h], inp.v[t, h], inp.g[t, h],
                                         inp.b[t, h], inp.scale)
                assert np.max(np.abs(o - out[t, h])) <= 1e-12
            assert np.max(np.abs(S - pool[inp.dst_slot_ids[s], h])) <= 1e-12


def test_empty_sequence_copies_state_and_untouched_slots(oracle):
    inp = kda_inputs.make_prefill_inputs("pin", [0, 3, 0], 10, "f16", H=2, K=16, V=8, seed=9,
                                         in_place=False)
    pool = inp.pool.copy()
    oracle.prefill_f32(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g, inp.b,
                       dst_slot_ids=inp.dst_slot_ids, scale=inp.scale)
    for s in (0, 2):      # empty: the fp16 bits come back unchanged (exact widen, RNE of an fp16)
        np.testing.assert_array_equal(pool[inp.dst_slot_ids[s]], inp.pool[inp.init_slot_ids[s]])
    named = set(inp.dst_slot_ids.tolist())
    for slot in range(10):
        if slot not in named:
            np.testing.assert_array_equal(pool[slot], inp.pool[slot])


@pytest.mark.parametrize("init,dst,cu", [
    ([0, 1], [2, 2], [0, 1, 2]),        # two sequences store to one slot
    ([0, 1], [1, 3], [0, 1, 2]),        # a destination is another sequence's initial slot
    ([0, 1], [2, 3], [0, 2, 1]),        # cu_seqlens decreasing
    ([0, 12], [2, 3], [0, 1, 2]),       # slot out of range
])
def test_prefill_refusals(oracle, init, dst, cu):
    inp = kda_inputs.make_prefill_inputs("pin", [1, 1], 12, "f32", H=1, K=4, V=4, seed=1)
    with pytest.raises(ValueError):
        oracle.prefill_f32(inp.pool.copy(), init, cu, inp.q, inp.k, inp.v, inp.g, inp.b,
                           dst_slot_ids=dst)


# ---------------------------------------------------------------------------
# the chunked form, fp64, from the algebra
# ---------------------------------------------------------------------------

def chunk_form(S0, q, k, v, g, b, scale, C=64, Bk=16):
    """One head, one sequence: S0 [K, V]; q, k, g [L, K]; v [L, V]; b [L].

    Within a chunk, with G_t the inclusive cumulative log-decay from the
    chunk start (per key channel), Delta_t = beta_t u_t satisfies
        (I + A) Delta = beta V - (beta Kn e^G) S0,
        A_ts = beta_t sum_i kn_ti kn_si e^(G_ti - G_si)   (s < t),
    the outputs are o_t = scale (sum_i qn_ti e^G_ti S0_i. + sum_{s<=t} P_ts Delta_s),
        P_ts = sum_i qn_ti kn_si e^(G_ti - G_si),
    and the chunk-end state is e^G_C S0 + sum_s (kn_s e^(G_C - G_s)) Delta_s^T.
    The exponentials of A and P are taken as products of two factors around a
    reference: the end of the previous block of Bk tokens (for a pair in
    different blocks both factors are <= 1; inside a block the right factor is
    e^(-G_s + G_ref) >= 1, bounded by the block's own decay)."""
    S = np.asarray(S0, np.float64).copy()
    L, K = q.shape
    qn = q.astype(np.float64) / np.sqrt((q.astype(np.float64) ** 2).sum(1, keepdims=True) + EPS)
    kn = k.astype(np.float64) / np.sqrt((k.astype(np.float64) ** 2).sum(1, keepdims=True) + EPS)
    beta = 1.0 / (1.0 + np.exp(-b.astype(np.float64)))
    out = np.zeros((L, S.shape[1]))
    for c0 in range(0, L, C):
        n = min(C, L - c0)
        sl = slice(c0, c0 + n)
        G = np.cumsum(g[sl].astype(np.float64), axis=0)           # [n, K]
        Qn, Kn, Bt, Vc = qn[sl], kn[sl], beta[sl], v[sl].astype(np.float64)
        A = np.zeros((n, n))
        P = np.zeros((n, n))
        for bt in range(0, n, Bk):
            ref = G[bt - 1] if bt > 0 else np.zeros(K)
            rows = slice(bt, min(bt + Bk, n))
            left_q = Qn[rows] * np.exp(G[rows] - ref)
            left_k = (Bt[rows, None] * Kn[rows]) * np.exp(G[rows] - ref)
            right = Kn[:rows.stop] * np.exp(ref - G[:rows.stop])
            P[rows, :rows.stop] = left_q @ right.T
            A[rows, :rows.stop] = left_k @ right.T
        P = np.tril(P)
        A = np.tril(A, -1)
        Kb = (Bt[:, None] * Kn) * np.exp(G)
        R = Bt[:, None] * Vc - Kb @ S
        Delta = np.linalg.solve(np.eye(n) + A, R)
        out[sl] = scale * ((Qn * np.exp(G)) @ S + P @ Delta)
        Kd = Kn * np.exp(G[-1] - G)
        S = np.exp(G[-1])[:, None] * S + Kd.T @ Delta
    return S, out


@pytest.mark.parametrize("L", [1, 15, 16, 17, 64, 65, 150])
def test_chunked_form_equals_recurrence(oracle, L):
    inp = kda_inputs.make_prefill_inputs("chunk", [L], 2, "f32", H=1, K=128, V=128, seed=L)
    pool = inp.pool.astype(np.float64)
    out = oracle.prefill_f64(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g,
                             inp.b, scale=inp.scale)
    S, o = chunk_form(inp.pool[inp.init_slot_ids[0], 0], inp.q[:, 0], inp.k[:, 0], inp.v[:, 0],
                      inp.g[:, 0], inp.b[:, 0], inp.scale)
    assert np.max(np.abs(S - pool[inp.init_slot_ids[0], 0])) <= 1e-10
    assert np.max(np.abs(o - out[:, 0])) <= 1e-10


def test_chunked_form_with_strong_decay(oracle):
    # log-decays of -3 .. -8 per token: the cumulative decay over a 64-token
    # chunk reaches far below fp64's range of e^x; the block references keep
    # every factor finite and the result still equals the recurrence
    inp = kda_inputs.make_prefill_inputs("chunk", [130], 2, "f32", H=1, K=32, V=16, seed=2)
    inp.g[:] = -np.random.default_rng(0).uniform(3.0, 8.0, inp.g.shape).astype(np.float32)
    pool = inp.pool.astype(np.float64)
    out = oracle.prefill_f64(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g,
                             inp.b, scale=inp.scale)
    S, o = chunk_form(inp.pool[inp.init_slot_ids[0], 0], inp.q[:, 0], inp.k[:, 0], inp.v[:, 0],
                      inp.g[:, 0], inp.b[:, 0], inp.scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert np.max(np.abs(S - pool[inp.init_slot_ids[0], 0])) <= 1e-10
    assert np.max(np.abs(o - out[:, 0])) <= 1e-10


def test_planted_mistake_in_prefill_is_caught(oracle):
    # exp(-g) instead of exp(g): the prefill must stop matching the dense form
    inp = kda_inputs.make_prefill_inputs("pin", [6], 2, "f32", H=1, K=8, V=4, seed=4)
    oracle.set_mutation(8)
    try:
        pool = inp.pool.astype(np.float64)
        oracle.prefill_f64(pool, inp.init_slot_ids, inp.cu_seqlens, inp.q, inp.k, inp.v, inp.g,
                           inp.b, scale=inp.scale)
    finally:
        oracle.set_mutation(0)
    S = inp.pool[inp.init_slot_ids[0], 0].astype(np.float64)
    for t in range(6):
        S, _ = dense.dense_token(S, inp.q[t, 0], inp.k[t, 0], inp.v[t, 0], inp.g[t, 0], inp.b[t, 0],
                                 inp.scale)
    assert np.max(np.abs(S - pool[inp.init_slot_ids[0], 0])) > 1e-3
