"""GPU tests of the measurement helpers the bench sets the kernels against:
kda_bw_probe (streaming copy, read-only and write-only streams),
kda_tile_probe (the single-row decode's state traffic, written back in
place) and kda_rows_probe (the chained rows' traffic: the initial state
written to every row's slot, in every tile shape it takes).  Each must move exactly the bytes it claims
and touch nothing else, or the ceilings the bench reports would be wrong."""
import numpy as np
import pytest

from gpu_helpers import B, need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def rand_bytes(n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)


@pytest.mark.parametrize("v", [1, 2, 4])
@pytest.mark.parametrize("nt", [False, True])
def test_bw_probe_copy_moves_exactly_the_bytes(v, nt):
    # a size that leaves a ragged last workgroup for every vector count
    nbytes = 16 * (3 * 256 * 4 + 37)
    src = rand_bytes(nbytes + 64, 1)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    B.kda_bw_probe(dst, src, nbytes, B.KDA_PROBE_COPY, v, nt)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert int(dst[nbytes:].count_nonzero()) == 0


@pytest.mark.parametrize("nt", [False, True])
def test_bw_probe_write_and_read(nt):
    n = 3 * 256 * 2 + 5                       # 16-byte vectors
    dst = torch.full((n + 4, 4), -1.0, device="cuda")
    B.kda_bw_probe(dst, None, 16 * n, B.KDA_PROBE_WRITE, 2, nt)
    torch.cuda.synchronize()
    idx = torch.arange(n, device="cuda", dtype=torch.float32)
    assert torch.equal(dst[:n], idx[:, None].expand(n, 4))
    assert bool((dst[n:] == -1.0).all())      # nothing past the range
    # a read-only stream over random bits writes nothing (the fold never
    # equals the probe's tag)
    src = rand_bytes(16 * n, 2)
    sink = torch.full((4,), 7.0, device="cuda")
    B.kda_bw_probe(sink, src, 16 * n, B.KDA_PROBE_READ, 4, nt)
    torch.cuda.synchronize()
    assert bool((sink == 7.0).all())


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_tile_probe_writes_every_tile_back_unchanged(dtype):
    tdt = torch.float32 if dtype == "f32" else torch.float16
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    pool = torch.randn((10, 3, 128, 128), generator=g, device="cuda").to(tdt)
    before = pool.clone()
    ids = torch.tensor([7, 2, 9, 0], dtype=torch.int32, device="cuda")
    B.kda_tile_probe(pool, ids)
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int16 if dtype == "f16" else torch.int32),
                       before.view(torch.int16 if dtype == "f16" else torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("with_init", [False, True])
@pytest.mark.parametrize("cols,waves", [(0, 0), (32, 8), (128, 8), (128, 16)])
def test_rows_probe_copies_the_initial_state_to_every_row(dtype, with_init, cols, waves):
    tdt = torch.float32 if dtype == "f32" else torch.float16
    itype = torch.int32 if dtype == "f32" else torch.int16
    n_slots, H, n_rows = 40, 3, 8
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    pool = torch.randn((n_slots, H, 128, 128), generator=g, device="cuda").to(tdt)
    before = pool.clone()
    perm = np.random.default_rng(5).permutation(n_slots).astype(np.int32)
    ids = perm[:3 * n_rows].reshape(3, n_rows).copy()
    init = perm[3 * n_rows:3 * n_rows + 3].copy() if with_init else ids[:, 0].copy()
    ids[2, 5] = n_slots                       # request 2 has a bad id: skipped
    B.kda_rows_probe(pool, torch.from_numpy(ids.reshape(-1)).cuda(), n_rows,
                     init_slot_ids=torch.from_numpy(init).cuda() if with_init else None,
                     tile_cols=cols, waves=waves)
    torch.cuda.synchronize()
    got, ref = pool.view(itype).cpu(), before.view(itype).cpu()
    expect = ref.clone()
    for r in range(2):
        for t in range(n_rows):
            expect[int(ids[r, t])] = ref[int(init[r])]
    assert torch.equal(got, expect)
