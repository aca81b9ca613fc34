"""bf16-pool error study (CPU, oracle only; the library refuses bf16 pools).

ROCm/ATOM PR #2130, What: fp16 rather than bf16 for the narrow state, because
q and k are L2-normalised in-kernel so the state is O(1) and bf16's wider
range buys nothing, while its 3 fewer mantissa bits cost roughly 8x the
error; Note on the default: that long-context error does not grow is offline
numerics.  Here both claims are measured at the long-run shape (one slot,
8192 decode tokens, H = 12, K = V = 128, fresh seeded inputs per token): the
pool stored in fp16 and, separately, in bf16 (each token's state rounded to
nearest even on store, the next token reading the rounded state), each
against the fp64 oracle run from the same initial state, token by token.
Reported per 1024-token chunk: RMS and max abs state error of each pool.
Graded: the ratio of the RMS errors over the second half of the run is near
2^3 = 8 (accepted: 4..16), and neither error grows from the first chunk to
the last (at most 1.5x).  Set KDA_BF16_REPORT=<path> to write the figures as
JSON.
"""
import json
import os

import numpy as np
import pytest

import kda_inputs

torch = pytest.importorskip("torch")

T = 2048
H = 2


def test_bf16_converter_matches_torch(oracle):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-60, 60, 1 << 20))).astype(np.float32)
    # values exactly halfway between bf16 neighbours, and their neighbours
    hb = (rng.integers(0, 1 << 15, 1 << 16).astype(np.uint32) << 16) | 0x8000
    mids = hb.view(np.float32)
    with np.errstate(invalid="ignore"):
        x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                            np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16_rne(x)
    nan = np.isnan(x)       # NaN payloads differ between implementations; NaN-ness must not
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))


T = 8192
H = 12
CHUNK = 1024


def _rms(x):
    return float(np.sqrt(np.mean(np.square(x))))


@pytest.mark.slow
def test_bf16_costs_about_8x_the_fp16_error(oracle):
    """About 20 s: the three pools (fp64, fp16, bf16) advance token by token
    in three threads (the C oracle releases the GIL), and each token's
    errors are reduced at once, so no trajectory is kept."""
    from concurrent.futures import ThreadPoolExecutor

    s0, q, k, v, g, b = kda_inputs.drift_tokens(T, seed=0, H=H)
    ids = np.zeros(1, dtype=np.int32)
    pools = {"f64": s0.astype(np.float64), "f16": s0.astype(np.float16).view(np.uint16),
             "bf16": oracle.f32_to_bf16_rne(s0)}

    def advance(kind, t):
        sl = slice(t, t + 1)
        if kind == "f64":
            oracle.step_f64(pools[kind], ids, q[sl], k[sl], v[sl], g[sl], b[sl])
            return pools[kind][0]
        oracle.step_f32(pools[kind], ids, q[sl], k[sl], v[sl], g[sl], b[sl], bf16=(kind == "bf16"))
        st = pools[kind][0]
        return st.view(np.float16).astype(np.float64) if kind == "f16" else \
            (st.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    sq = {kind: np.zeros(T) for kind in ("f16", "bf16")}
    mx = {kind: np.zeros(T) for kind in ("f16", "bf16")}
    state_sq = np.zeros(T)
    with ThreadPoolExecutor(3) as ex:
        for t in range(T):
            futs = {kind: ex.submit(advance, kind, t) for kind in ("f64", "f16", "bf16")}
            ref = futs["f64"].result()
            state_sq[t] = np.mean(np.square(ref))
            for kind in ("f16", "bf16"):
                d = futs[kind].result() - ref
                sq[kind][t] = np.mean(np.square(d))
                mx[kind][t] = np.abs(d).max()
    res = {"tokens": T, "heads": H, "chunk": CHUNK, "chunks": {}}
    for kind in ("f16", "bf16"):
        res["chunks"][kind] = [{"tokens": [c, c + CHUNK],
                                "rms": float(np.sqrt(sq[kind][c:c + CHUNK].mean())),
                                "max_abs": float(mx[kind][c:c + CHUNK].max())}
                               for c in range(0, T, CHUNK)]
        res[kind] = {"rms_last_half": float(np.sqrt(sq[kind][T // 2:].mean())),
                     "max_abs": float(mx[kind].max())}
    res["ratio_rms"] = res["bf16"]["rms_last_half"] / res["f16"]["rms_last_half"]
    res["state_rms"] = float(np.sqrt(state_sq[T // 2:].mean()))
    path = os.environ.get("KDA_BF16_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(res, f, indent=1)
    print(json.dumps({"ratio_rms": res["ratio_rms"], "f16": res["f16"], "bf16": res["bf16"],
                      "state_rms": res["state_rms"]}))
    assert 4.0 <= res["ratio_rms"] <= 16.0
    # neither error grows over the run
    for kind in ("f16", "bf16"):
        first, last = res["chunks"][kind][0]["rms"], res["chunks"][kind][-1]["rms"]
        assert last <= 1.5 * first, (kind, first, last)
