"""Helpers for the GPU tests: move seeded host inputs to the device, launch
through the C ABI, bring results back, and measure errors against the
oracle with the tolerances the tests state."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kda_inputs  # noqa: E402
from kda_gated_delta_decode_amd import binding as B  # noqa: E402

# Tolerances.  fp32 pool: max abs state error <= 1e-6 over every written
# slot, and per (row, head) ||o - o_ref|| / ||o_ref|| <= 1e-5.  fp16 pool:
# every stored element within 1 fp16 ulp of the oracle's RNE-rounded fp32
# state (same output bound as fp32: the recurrence is fp32 on the same
# widened state).
STATE_ABS_F32 = 1e-6
OUT_REL = 1e-5
F16_ULP = 1


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.library()


def device_inputs(inp: kda_inputs.DecodeInputs):
    """Device tensors for a DecodeInputs (pool as float32 or float16)."""
    dev = torch.device("cuda", 0)
    if inp.dtype == "f32":
        pool = torch.from_numpy(inp.pool).to(dev)
    else:
        pool = torch.from_numpy(inp.pool.view(np.float16)).to(dev)
    t = {n: torch.from_numpy(getattr(inp, n)).to(dev) for n in ("q", "k", "v", "g", "b")}
    ids = torch.from_numpy(inp.slot_ids).to(dev)
    out = torch.full((inp.slot_ids.size, inp.pool.shape[1], inp.pool.shape[3]), float("nan"),
                     dtype=torch.float32, device=dev)
    return pool, ids, t, out


def pool_to_host(pool) -> np.ndarray:
    x = pool.cpu().numpy()
    return x.view(np.uint16) if x.dtype == np.float16 else x


def run_gpu(inp: kda_inputs.DecodeInputs, waves_per_tile: int = 0, bv: int = 0,
            block_rows: bool = False, rows_layout: int = 0):
    """One launch on the device; returns (pool after [host], out [host])."""
    pool, ids, t, out = device_inputs(inp)
    B.kda_decode_step(pool, ids, t["q"], t["k"], t["v"], t["g"], t["b"], out,
                      n_rows_per_slot=inp.n_rows, scale=inp.scale, waves_per_tile=waves_per_tile,
                      bv=bv, block_rows=block_rows, rows_layout=rows_layout)
    torch.cuda.synchronize()
    return pool_to_host(pool), out.cpu().numpy()


def run_oracle_f32(oracle, inp, pool=None):
    pool = inp.pool.copy() if pool is None else pool
    out = oracle.step_f32(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                          n_rows=inp.n_rows, scale=inp.scale)
    return pool, out


def run_oracle_f64(oracle, inp):
    if inp.dtype == "f32":
        pool = inp.pool.astype(np.float64)
    else:
        pool = inp.pool.view(np.float16).astype(np.float64)
    out = oracle.step_f64(pool, inp.slot_ids, inp.q, inp.k, inp.v, inp.g, inp.b,
                          n_rows=inp.n_rows, scale=inp.scale)
    return pool, out


def f16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """|a - b| in units in the last place of binary16, +0 and -0 equal:
    bit patterns mapped to an ordered integer line."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def out_rel_err(out, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(np.asarray(out, dtype=np.float64) - ref, axis=-1)
    n = np.linalg.norm(ref, axis=-1)
    return float(np.max(d / np.maximum(n, 1e-30)))


def check_parity(oracle, inp, gpu_pool, gpu_out, label=""):
    """Assert the GPU results match the oracle within the stated bounds;
    returns a dict of the measured errors."""
    written = np.unique(inp.slot_ids)
    untouched = np.setdiff1d(np.arange(inp.pool.shape[0]), written)
    np.testing.assert_array_equal(gpu_pool[untouched], inp.pool[untouched],
                                  err_msg="%s: a slot not named was modified" % label)
    assert np.all(np.isfinite(gpu_out)), "%s: non-finite output" % label
    o_pool32, o_out32 = run_oracle_f32(oracle, inp)
    res = {}
    if inp.dtype == "f32":
        o_pool64, o_out64 = run_oracle_f64(oracle, inp)
        err64 = float(np.max(np.abs(gpu_pool[written].astype(np.float64) - o_pool64[written])))
        err32 = float(np.max(np.abs(gpu_pool[written] - o_pool32[written])))
        res.update(state_abs_vs_f64=err64, state_abs_vs_f32=err32,
                   out_rel_vs_f64=out_rel_err(gpu_out, o_out64))
        assert err64 <= STATE_ABS_F32, "%s: state error %.3g vs fp64 oracle" % (label, err64)
        assert err32 <= STATE_ABS_F32, "%s: state error %.3g vs fp32 oracle" % (label, err32)
        assert res["out_rel_vs_f64"] <= OUT_REL, "%s: out rel error %.3g" % (label, res["out_rel_vs_f64"])
    else:
        ulp = f16_ulp_distance(gpu_pool[written], o_pool32[written])
        res.update(state_max_ulp=int(ulp.max()), state_frac_ulp1=float((ulp > 0).mean()))
        assert ulp.max() <= F16_ULP, "%s: fp16 state %d ulp from the oracle" % (label, ulp.max())
    res["out_rel_vs_f32"] = out_rel_err(gpu_out, o_out32)
    assert res["out_rel_vs_f32"] <= OUT_REL, "%s: out rel error %.3g vs fp32 oracle" % (label, res["out_rel_vs_f32"])
    return res
