"""GPU test of kda_decode_step_conv_noalloc, the fused step for callers that
cannot allocate (its pair counters live in the library's static device
array), against kda_decode_step_conv_ws with caller-owned counters.  Both run
the same kernels, so states, convolution histories and outputs must agree
bit for bit, on two calls in a row, the second with a smaller launch (the
static counters keep what the first call left)."""
import numpy as np
import pytest

import kda_inputs
from gpu_helpers import B, need_gpu, pool_to_host, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def launch(ci, counts=None):
    d = ci.dec
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(d.pool if d.dtype == "f32" else d.pool.view(np.float16)).to(dev)
    conv = torch.from_numpy(ci.conv).to(dev).view(torch.bfloat16)
    t = {n: torch.from_numpy(getattr(src, n)).to(dev)
         for src, n in ((d, "slot_ids"), (ci, "x"), (ci, "w"), (d, "g"), (d, "b"))}
    out = torch.full((d.slot_ids.size, d.pool.shape[1], 128), float("nan"), device=dev)
    args = (pool, conv, t["slot_ids"], t["x"], t["w"], t["g"], t["b"], out)
    if counts is None:
        B.kda_decode_step_conv_noalloc(*args, n_rows_per_slot=d.n_rows, scale=d.scale)
    else:
        B.kda_decode_step_conv(*args, n_rows_per_slot=d.n_rows, scale=d.scale, pair_counts=counts)
    torch.cuda.synchronize()
    return (pool_to_host(pool).view(np.uint8), conv.view(torch.int16).cpu().numpy(),
            out.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_noalloc_matches_caller_counters_on_two_calls(dtype):
    dev = torch.device("cuda", 0)
    big = kda_inputs.make_conv_inputs("noalloc big", 96, 8, 8, dtype, H=12, seed=201)
    small = kda_inputs.make_conv_inputs("noalloc small", 24, 3, 4, dtype, H=3, seed=202)
    # both launches take the halves, whose in-place rows use the counters
    for ci in (big, small):
        units = ci.dec.n_req * ci.dec.pool.shape[1]
        assert units <= B.KDA_NOALLOC_MAX_PAIRS
        counts = B.conv_pair_counts(ci.dec.n_req, ci.dec.pool.shape[1], dev)
        want = launch(ci, counts)
        got = launch(ci)
        for name, w, g in zip(("state", "history", "out"), want, got):
            np.testing.assert_array_equal(g, w, err_msg="%s, %s" % (ci.dec.name, name))
        assert not np.isnan(got[2].view(np.float32)).any()
        # the caller's counters: 2 per (request, head), every row 0 in place
        assert bool((counts == 2).all())
