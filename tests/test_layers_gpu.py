"""GPU parity of the 69-layer decode step: 69 independent layer pools of 64
slots (every slot updated, one token each; inputs drawn on the GPU from one
seeded generator, slots permuted by a generator seeded with the layer index), launched back
to back on one stream with no synchronisation in between, as the bench times
the step; then every layer's pool and outputs against the fp32 oracle, with
the decode bounds.  fp32 and fp16 pools."""
import sys

import numpy as np
import pytest

import kda_inputs
from gpu_helpers import (B, F16_ULP, OUT_REL, STATE_ABS_F32, f16_ulp_distance, need_gpu,
                         out_rel_err, pool_to_host, run_oracle_f32, torch)

pytestmark = pytest.mark.gpu

N_LAYERS = 69


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def layer_inputs(layer, dtype, gen, H=12, n=64):
    """One layer's inputs, drawn on the GPU with the documented distributions
    (state N(0, 0.05^2), rounded to nearest even for fp16 pools; q, k, v, b
    N(0, 1); g = -softplus(N(0, 1)); slots a permutation of the 64), and the
    same arrays on the host for the oracle."""
    tdt = torch.float32 if dtype == "f32" else torch.float16
    pool = (torch.randn((n, H, 128, 128), generator=gen, device="cuda") * 0.05).to(tdt)
    q, k, v = (torch.randn((n, H, 128), generator=gen, device="cuda") for _ in range(3))
    g = -torch.nn.functional.softplus(torch.randn((n, H, 128), generator=gen, device="cuda"))
    b = torch.randn((n, H), generator=gen, device="cuda")
    ids = np.random.default_rng(layer).permutation(n).astype(np.int32)
    host_pool = pool.cpu().numpy()
    if dtype == "f16":
        host_pool = host_pool.view(np.uint16)
    inp = kda_inputs.DecodeInputs("layer %d" % layer, dtype, host_pool, ids, q.cpu().numpy(), k.cpu().numpy(),
                                  v.cpu().numpy(), g.cpu().numpy(), b.cpu().numpy(), 1, float(1.0 / np.sqrt(128)))
    dev = dict(pool=pool, ids=torch.from_numpy(ids).cuda(), q=q, k=k, v=v, g=g, b=b,
               out=torch.full((n, H, 128), float("nan"), device="cuda"))
    return inp, dev


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_69_layer_step(oracle, dtype):
    print("69 layers x 64 slots, back to back,", dtype, flush=True)
    sys.stdout.flush()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(69)
    layers = [layer_inputs(layer, dtype, gen) for layer in range(N_LAYERS)]
    torch.cuda.synchronize()
    for inp, d in layers:
        B.kda_decode_step(d["pool"], d["ids"], d["q"], d["k"], d["v"], d["g"], d["b"], d["out"],
                          scale=inp.scale)
    torch.cuda.synchronize()
    worst_state, worst_out = 0.0, 0.0
    for layer, (inp, d) in enumerate(layers):
        gp, go = pool_to_host(d["pool"]), d["out"].cpu().numpy()
        op, oo = run_oracle_f32(oracle, inp)
        if dtype == "f32":
            err = float(np.max(np.abs(gp - op)))
            assert err <= STATE_ABS_F32, "layer %d: state error %.3g" % (layer, err)
        else:
            err = float(f16_ulp_distance(gp, op).max())
            assert err <= F16_ULP, "layer %d: fp16 state %d ulp from the oracle" % (layer, err)
        rel = out_rel_err(go, oo)
        assert rel <= OUT_REL, "layer %d: out rel error %.3g" % (layer, rel)
        worst_state, worst_out = max(worst_state, err), max(worst_out, rel)
    print("worst state error %.3g, worst out rel error %.3g" % (worst_state, worst_out), flush=True)
    del layers
    torch.cuda.empty_cache()
