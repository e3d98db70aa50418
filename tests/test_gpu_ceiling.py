"""The gather-copy ceiling (libibp_ceiling) moves the bytes it claims: output
row i = the first src_bytes[i] bytes (rounded up to 16) of slot ids[i],
zeros after; an id outside the table gives a zero row.  Rows of 16 B to
4 KiB (one task each), chunked rows (8 and 28 KiB), several tensors in one
launch, a capped grid, a pinned host source.  The benchmark times this copy as the floor of each
decompression, so it has to read and write exactly that.  The plain tile
copy (ibp_ceiling_copy) equals its source and writes nothing past it."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ceiling():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_level_amd import ceiling as c
    c.lib()
    return c


def expected(table: np.ndarray, src_bytes: np.ndarray, ids) -> np.ndarray:
    n_rows, S = table.shape
    rows = np.arange(n_rows) if ids is None else ids
    out = np.zeros((len(rows), S), np.uint8)
    for i, r in enumerate(rows):
        if 0 <= r < n_rows:
            nb = min(S, (int(src_bytes[i]) + 15) // 16 * 16)
            out[i, :nb] = table[r, :nb]
    return out


def case(rng, n_rows, S, n_ids):
    table = rng.integers(0, 256, (n_rows, S), dtype=np.uint8)
    ids = None
    if n_ids is not None:
        ids = rng.integers(-2, n_rows + 3, n_ids).astype(np.int64)
    n_out = n_rows if ids is None else n_ids
    src_bytes = (rng.integers(0, S // 4 + 40, n_out) * 4).astype(np.int32)
    src_bytes[:3] = [0, S, 4]
    return table, src_bytes, ids


@pytest.mark.parametrize("pack,stream_loads", [(False, False), (True, False), (False, True),
                                               (True, True)])
@pytest.mark.parametrize("cap", [0, 1, 7])
@pytest.mark.parametrize("S,n_rows,n_ids", [(512, 3000, 5000), (1024, 700, 4097),
                                            (2048, 513, 1000), (4096, 300, 999),
                                            (16, 100, 77), (8192, 65, None),
                                            (28672, 33, None), (1040, 40, 90)])
def test_gather_copy_single(ceiling, S, n_rows, n_ids, cap, pack, stream_loads):
    rng = np.random.default_rng(S + n_rows)
    table, sb, ids = case(rng, n_rows, S, n_ids)
    tg = torch.from_numpy(table).cuda()
    sbg = torch.from_numpy(sb).cuda()
    idg = torch.from_numpy(ids).cuda() if ids is not None else None
    n_out = len(ids) if ids is not None else n_rows
    out = torch.full((n_out, S), 0xAB, dtype=torch.uint8, device="cuda")
    ceiling.gather_copy_launcher([(tg, sbg, idg, out)], max_workgroups=cap, pack=pack,
                                 stream_loads=stream_loads)()
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), expected(table, sb, ids))


def test_gather_copy_batch_and_host_source(ceiling):
    rng = np.random.default_rng(7)
    parts, want = [], []
    for S, n_rows, n_ids, host in [(8192, 40, None, False), (28672, 20, None, True),
                                   (2048, 100, 300, True), (512, 64, 1000, False)]:
        table, sb, ids = case(rng, n_rows, S, n_ids)
        tg = torch.from_numpy(table)
        tg = tg.pin_memory() if host else tg.cuda()
        idg = torch.from_numpy(ids).cuda() if ids is not None else None
        n_out = len(ids) if ids is not None else n_rows
        out = torch.full((n_out, S), 0xCD, dtype=torch.uint8, device="cuda")
        parts.append((tg, torch.from_numpy(sb).cuda(), idg, out))
        want.append(expected(table, sb, ids))
    for cap, pack, nt in ((0, False, False), (3, False, True), (0, True, True), (5, True, False)):
        for _, _, _, out in parts:
            out.fill_(0xCD)
        ceiling.gather_copy_launcher(parts, max_workgroups=cap, pack=pack, stream_loads=nt)()
        torch.cuda.synchronize()
        for (_, _, _, out), w in zip(parts, want):
            assert np.array_equal(out.cpu().numpy(), w)


@pytest.mark.parametrize("cap", [0, 1, 5])
@pytest.mark.parametrize("n_bytes", [16, 16368, 16384, 16400, 37 * 16384 + 80, (64 << 20) + 48])
def test_tile_copy(ceiling, n_bytes, cap):
    """The plain contiguous copy the benchmark quotes as the practical
    read/write rate: whole 16 KiB tiles, a partial last tile, a capped grid
    (workgroups looping over tiles); nothing is written past n_bytes."""
    rng = np.random.default_rng(n_bytes + cap)
    src = torch.from_numpy(rng.integers(0, 256, n_bytes, dtype=np.uint8)).cuda()
    dst = torch.full((n_bytes + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    ceiling.copy_launcher(src, dst[:n_bytes], max_workgroups=cap)()
    torch.cuda.synchronize()
    assert torch.equal(dst[:n_bytes], src)
    assert bool((dst[n_bytes:] == 0xA5).all())
