"""GPU tests of the library's launches replayed from HIP graphs, the way the
bench times them and a serving step launches them.  Each launch is captured
once and replayed several times; before every replay the buffers it updates
are restored by eager copies (outside the graph), and every replay must
equal the eager launch bit for bit: the same kernels on the same inputs.
The fused step's pair counters (caller-owned, or the library's own for the
allocation-free entry) must stay even across replays, as each launch adds 2
to every counter it uses."""
import numpy as np
import pytest

import kda_inputs
from gpu_helpers import B, device_inputs, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def replays_match_eager(launch, written, n_replays=3, check=None):
    """launch() enqueues one step on the current stream; written: the
    tensors it updates.  check() (optional) runs after every run."""
    start = [t.clone() for t in written]

    def restore():
        for t, t0 in zip(written, start):
            t.copy_(t0)

    launch()
    torch.cuda.synchronize()
    want = [t.clone() for t in written]
    if check:
        check()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the warm-up launch torch asks for before a capture
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for i in range(n_replays):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, w in zip(written, want):
            assert torch.equal(bits(t), bits(w)), "replay %d" % i
        if check:
            check()
    del graph


def decode_launch(inp, **opts):
    pool, ids, t, out = device_inputs(inp)

    def launch():
        B.kda_decode_step(pool, ids, t["q"], t["k"], t["v"], t["g"], t["b"], out, n_rows_per_slot=inp.n_rows,
                          scale=inp.scale, **opts)
    return launch, [pool, out]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_batched_decode_replays(dtype):
    inp = kda_inputs.make_inputs("graph batched", 96, 64, 1, dtype, seed=301)
    launch, written = decode_launch(inp)
    replays_match_eager(launch, written)


@pytest.mark.parametrize("layout", ["matrix", "k_split"])
def test_chained_rows_replay(layout):
    inp = kda_inputs.make_inputs("graph rows", 96, 8, 8, "f16", seed=302)
    launch, written = decode_launch(
        inp, rows_layout=B.KDA_ROWS_MATRIX if layout == "matrix" else B.KDA_ROWS_K_SPLIT)
    replays_match_eager(launch, written)


def conv_launch(ci, entry, **opts):
    d = ci.dec
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(d.pool if d.dtype == "f32" else d.pool.view(np.float16)).to(dev)
    conv = torch.from_numpy(ci.conv).to(dev).view(torch.bfloat16)
    t = {n: torch.from_numpy(getattr(src, n)).to(dev)
         for src, n in ((d, "slot_ids"), (ci, "x"), (ci, "w"), (d, "g"), (d, "b"))}
    out = torch.full((d.slot_ids.size, d.pool.shape[1], 128), float("nan"), device=dev)

    def launch():
        entry(pool, conv, t["slot_ids"], t["x"], t["w"], t["g"], t["b"], out, n_rows_per_slot=d.n_rows,
              scale=d.scale, **opts)
    return launch, [pool, conv, out]


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_fused_halves_replay_with_caller_counters(dtype):
    ci = kda_inputs.make_conv_inputs("graph conv halves", 96, 8, 8, dtype, seed=303)
    counts = B.conv_pair_counts(8, 12, torch.device("cuda", 0))
    launch, written = conv_launch(ci, B.kda_decode_step_conv, pair_counts=counts, rows_layout=B.KDA_ROWS_MATRIX)

    def even():
        assert bool((counts.remainder(2) == 0).all()) and int(counts.min()) > 0

    replays_match_eager(launch, written, check=even)


def test_fused_noalloc_replays():
    # the first call (eager) looks the library's counters up on the device;
    # the captured calls then allocate nothing
    ci = kda_inputs.make_conv_inputs("graph conv noalloc", 96, 8, 8, "f16", seed=304)
    launch, written = conv_launch(ci, B.kda_decode_step_conv_noalloc)
    replays_match_eager(launch, written)


def test_prefill_replays():
    inp = kda_inputs.make_prefill_inputs("graph prefill", [37, 1, 96, 64], 16, "f32", H=3, seed=305,
                                         in_place=False)
    dev = torch.device("cuda", 0)
    pool = torch.from_numpy(inp.pool).to(dev)
    t = {n: torch.from_numpy(getattr(inp, n)).to(dev) for n in ("q", "k", "v", "g", "b")}
    init = torch.from_numpy(inp.init_slot_ids).to(dev)
    dst = torch.from_numpy(inp.dst_slot_ids).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens).to(dev)
    out = torch.full((inp.q.shape[0], inp.pool.shape[1], 128), float("nan"), device=dev)

    def launch():
        B.kda_prefill(pool, init, cu, t["q"], t["k"], t["v"], t["g"], t["b"], out, dst_slot_ids=dst,
                      scale=inp.scale)
    replays_match_eager(launch, [pool, out])
