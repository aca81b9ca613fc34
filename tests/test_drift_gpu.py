"""Long single-slot run: 8192 decode launches of one token each on one slot
(H = 12, K = V = 128, fresh seeded inputs per token), fp32 and fp16 pools.

Graded:
  * fp32 pool, free-running: every token's state within 1e-6 (max abs) of
    the fp32 oracle run free over the same 8192 tokens, and every output
    within 1e-5 (relative, per head).  Decay <= 1 and (I - beta kn kn^T) are
    contractions, so rounding differences do not grow.
  * fp16 pool, one step at a time: for every token, the oracle's step applied
    to the GPU's own previous stored state must match the GPU's stored state
    within 1 fp16 ulp and its output within 1e-5.  (Free-running fp16
    trajectories may legitimately part by an ulp and then differ in later
    roundings, so they are not compared element by element.)
Reported, not graded: the drift of the GPU's fp32 and fp16 trajectories from
the fp64 oracle over the run (ROCm/ATOM PR #2130, Note on the default: the
evidence that the error does not grow with sequence length is offline
numerics).  Set KDA_DRIFT_REPORT=<path> to write the report as JSON.
"""
import json
import os
import sys

import numpy as np
import pytest

import kda_inputs
from gpu_helpers import B, f16_ulp_distance, need_gpu, torch

pytestmark = pytest.mark.gpu

T = 8192
CHUNK = 1024
H = 12


@pytest.fixture(scope="module")
def tokens():
    need_gpu()
    return kda_inputs.drift_tokens(T, seed=0)


def gpu_run(dtype, s0, q, k, v, g, b, t0, t1, pool, out_dev):
    """Launch tokens t0..t1-1 on the 1-slot device pool; return the
    trajectory [t1-t0, H, 128, 128] and outputs, on the host."""
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    traj = torch.empty((t1 - t0, H, 128, 128), dtype=pool.dtype, device="cuda")
    for t in range(t0, t1):
        sl = slice(t, t + 1)
        B.kda_decode_step(pool, ids, q[sl], k[sl], v[sl], g[sl], b[sl], out_dev[sl])
        traj[t - t0].copy_(pool[0])
    torch.cuda.synchronize()
    x = traj.cpu().numpy()
    return (x.view(np.uint16) if dtype == "f16" else x), out_dev[t0:t1].cpu().numpy()


def test_8192_token_run(oracle, tokens):
    s0, q, k, v, g, b = tokens
    dev = {n: torch.from_numpy(a).cuda() for n, a in zip("qkvgb", (q, k, v, g, b))}
    report = {"tokens": T, "heads": H, "chunks": []}

    pool32 = torch.from_numpy(s0.copy()).cuda()
    pool16 = torch.from_numpy(s0.astype(np.float16)).cuda()
    out32 = torch.empty((T, H, 128), device="cuda")
    out16 = torch.empty((T, H, 128), device="cuda")

    # oracle free runs: fp32 (graded) and fp64 (drift reference), chained
    # through the multi-row path one chunk at a time (identity stores)
    o32_state = s0[0].copy()
    o64_state = s0[0].astype(np.float64)
    prev16 = s0.astype(np.float16).view(np.uint16)[0].copy()  # GPU fp16 state before the chunk
    ids_chain = np.arange(1, CHUNK + 1, dtype=np.int32)
    worst = {"f32_state_abs": 0.0, "f32_out_rel": 0.0, "f16_step_ulp": 0, "f16_out_rel": 0.0}
    for c0 in range(0, T, CHUNK):
        c1 = c0 + CHUNK
        print("drift chunk", c0, c1, flush=True)
        sl = slice(c0, c1)
        g32, go32 = gpu_run("f32", s0, dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], c0, c1, pool32, out32)
        g16, go16 = gpu_run("f16", s0, dev["q"], dev["k"], dev["v"], dev["g"], dev["b"], c0, c1, pool16, out16)

        # fp32 oracle, free-running over the chunk
        p = np.empty((CHUNK + 1, H, 128, 128), dtype=np.float32)
        p[1] = o32_state
        oo32 = oracle.step_f32(p, ids_chain, q[sl], k[sl], v[sl], g[sl], b[sl], n_rows=CHUNK)
        o32 = p[1:]
        o32_state = o32[-1].copy()
        p64 = np.empty((CHUNK + 1, H, 128, 128), dtype=np.float64)
        p64[1] = o64_state
        oracle.step_f64(p64, ids_chain, q[sl], k[sl], v[sl], g[sl], b[sl], n_rows=CHUNK)
        o64 = p64[1:]
        o64_state = o64[-1].copy()
        del p, p64

        e32 = np.abs(g32.astype(np.float64) - o32).reshape(CHUNK, -1).max(1)
        rel = (np.linalg.norm(go32 - oo32, axis=-1) / np.linalg.norm(oo32, axis=-1)).max()
        worst["f32_state_abs"] = max(worst["f32_state_abs"], float(e32.max()))
        worst["f32_out_rel"] = max(worst["f32_out_rel"], float(rel))

        # fp16: each token's oracle step from the GPU's own previous state
        before = np.concatenate([prev16[None], g16[:-1]], axis=0)      # [CHUNK, H, K, V]
        ids_step = np.arange(CHUNK, dtype=np.int32)
        ps = before.copy()
        os16 = oracle.step_f32(ps, ids_step, q[sl], k[sl], v[sl], g[sl], b[sl], n_rows=1)
        ulp = f16_ulp_distance(g16, ps)
        rel16 = (np.linalg.norm(go16 - os16, axis=-1) / np.linalg.norm(os16, axis=-1)).max()
        worst["f16_step_ulp"] = max(worst["f16_step_ulp"], int(ulp.max()))
        worst["f16_out_rel"] = max(worst["f16_out_rel"], float(rel16))
        prev16 = g16[-1].copy()
        del before, ps

        d32 = np.abs(g32.astype(np.float64) - o64).reshape(CHUNK, -1).max(1)
        d16 = np.abs(g16.view(np.float16).astype(np.float64) - o64).reshape(CHUNK, -1).max(1)
        rms16 = np.sqrt(((g16.view(np.float16).astype(np.float64) - o64) ** 2).reshape(CHUNK, -1).mean(1))
        report["chunks"].append({
            "tokens": [c0, c1],
            "gpu_f32_vs_oracle_f32_state_max_abs": float(e32.max()),
            "gpu_f32_vs_oracle_f64_state_max_abs": float(d32.max()),
            "gpu_f16_vs_oracle_f64_state_max_abs": float(d16.max()),
            "gpu_f16_vs_oracle_f64_state_rms": float(rms16.mean()),
            "state_max_abs": float(np.abs(o64).max()),
            "f16_step_max_ulp": int(ulp.max()),
            "f16_step_frac_1ulp": float((ulp > 0).mean()),
        })
        del g32, g16, o32, o64
    report["worst"] = worst
    path = os.environ.get("KDA_DRIFT_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(worst), flush=True)
    sys.stdout.flush()
    assert worst["f32_state_abs"] <= 1e-6
    assert worst["f32_out_rel"] <= 1e-5
    assert worst["f16_step_ulp"] <= 1
    assert worst["f16_out_rel"] <= 1e-5
