"""A seeded sweep of random tables against the oracle.

Each case draws a block width (16, 32 or 64 bits), a row length (the lengths
the specialised kernels take -- 512 B to 32 KiB -- or any multiple of the
block pair, up to the 96 KiB limit), a row count, a Mask with a random
number of invariant bits (none and all included), a Bitval inside it, a
match rate and a few raw rows.  The GPU image (every row's flag, C and
stored words) must equal the oracle's, the full decompress and the batched
decompress must return the source, and a gather with repeated ids and ids
outside the table must equal the oracle's gather.  Every fourth 32-bit case
also runs per-position metadata with a random table.  Cases are fixed by
their index: the same inputs on every run."""
import numpy as np
import pytest

from oracle import oracle as orc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 48
SPECIAL_ROWS = (512, 1024, 2048, 4096, 8192, 16384, 28672, 32768)
MAX_BYTES = 4 << 20  # per table, so that the oracle runs in a fraction of a second


@pytest.fixture(scope="module")
def ibp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_level_amd import ibp as b
    b.lib()
    return b


def draw_case(k):
    rng = np.random.default_rng([7, k])
    w = (16, 32, 64)[k % 3]
    unit = 8 if w == 64 else 4
    if rng.random() < 0.5:
        row_bytes = int(rng.choice(SPECIAL_ROWS))
    else:
        row_bytes = int(rng.integers(1, 98304 // unit + 1)) * unit
    n_rows = int(rng.integers(1, max(2, min(300, MAX_BYTES // row_bytes)) + 1))
    p = int(rng.choice([0, w, int(rng.integers(1, w))]))
    bits = rng.permutation(w)[:p]
    mask = sum(1 << int(b) for b in bits)
    bitval = mask & int.from_bytes(rng.bytes(8), "little")
    match_p = float(rng.choice([0.0, 0.5, 0.9, 0.99, 1.0]))
    return rng, w, row_bytes, n_rows, mask, bitval, match_p


def make_table(rng, w, row_bytes, n_rows, mask, bitval, match_p):
    dt = {16: np.uint16, 32: np.uint32, 64: np.uint64}[w]
    x = rng.integers(0, 256, (n_rows, row_bytes), dtype=np.uint8).view(dt)
    force = rng.random(x.shape) < match_p
    keep = dt(~mask & ((1 << w) - 1))
    x = np.where(force, (x & keep) | dt(bitval), x).astype(dt)
    for r in rng.integers(0, n_rows, min(3, n_rows)):
        x[r] = rng.integers(0, 256, row_bytes, dtype=np.uint8).view(dt)
    return np.ascontiguousarray(x).view(np.uint8).reshape(n_rows, row_bytes)


def metadata(ibp, w, mask, bitval):
    md = ibp.ibp_metadata()
    md.width_bits, md.mask, md.bitval, md.t_ppm = w, mask, bitval, 900000
    md.invariant_bits = bin(mask).count("1")
    return md


def flags_of(flags, n_rows):
    f = flags.cpu().numpy().view(np.uint64)[:(n_rows + 63) // 64].copy()
    if n_rows % 64:
        f[-1] &= np.uint64((1 << (n_rows % 64)) - 1)
    return f


def assert_image(slots, flags, rb, slots_o, flags_o, rb_o, n_rows, row_bytes):
    fg = flags_of(flags, n_rows)
    assert np.array_equal(fg, flags_o)
    rg = rb.cpu().numpy()[:n_rows].view(np.uint32).astype(np.uint64)
    assert np.array_equal(rg, rb_o)
    ok = orc.image_bytes_equal(slots.cpu().numpy(), slots_o, flags_o, rb_o)
    assert ok.all(), f"rows {np.flatnonzero(~ok)[:8]} differ"


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_table(ibp, k):
    rng, w, row_bytes, n_rows, mask, bitval, match_p = draw_case(k)
    print(f"case {k}: W={w} rows={n_rows} row_bytes={row_bytes} mask={mask:x} "
          f"bitval={bitval:x} match={match_p}", flush=True)
    x = make_table(rng, w, row_bytes, n_rows, mask, bitval, match_p)
    md = metadata(ibp, w, mask, bitval)
    md_o = orc.Metadata(w, mask, bitval, 900000)
    xg = torch.from_numpy(x).cuda()
    slots, flags, rb = ibp.ibp_compress(md, xg)
    torch.cuda.synchronize()
    slots_o, flags_o, rb_o = orc.compress(md_o, x)
    assert_image(slots, flags, rb, slots_o, flags_o, rb_o, n_rows, row_bytes)
    assert torch.equal(ibp.ibp_decompress(md, slots, flags), xg)
    # batched: the table twice (two entries of one launch)
    outs = ibp.ibp_decompress_batch(md, [(slots, flags), (slots, flags)])
    torch.cuda.synchronize()
    assert torch.equal(outs[0], xg) and torch.equal(outs[1], xg)
    ids = rng.integers(-2, n_rows + 2, 2 * n_rows + 7).astype(np.int64)
    ids[:2] = [n_rows - 1, n_rows - 1]
    inside = (ids >= 0) & (ids < n_rows)
    want = np.zeros((ids.size, row_bytes), np.uint8)
    want[inside] = orc.gather_decompress(md_o, slots_o, flags_o, ids[inside])
    got = ibp.ibp_gather_decompress(md, slots, flags, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)

    if w == 32 and k % 4 == 2:
        n = row_bytes // 4
        pm = np.zeros(n, np.uint64)
        for j in range(n):
            bits = rng.permutation(32)[:int(rng.integers(0, 33))]
            pm[j] = sum(1 << int(b) for b in bits)
        pb = pm & rng.integers(0, 2**32, n, dtype=np.uint64)
        xp = x.view(np.uint32).copy()
        force = rng.random(xp.shape) < match_p
        xp = np.where(force, (xp & ~pm.astype(np.uint32)) | pb.astype(np.uint32), xp)
        xp = np.ascontiguousarray(xp.astype(np.uint32)).view(np.uint8).reshape(n_rows, row_bytes)
        table = ibp.ibp_positional_table(pm, pb).cuda()
        xpg = torch.from_numpy(xp).cuda()
        s2, f2, r2 = ibp.ibp_compress_positional(table, xpg)
        torch.cuda.synchronize()
        pmd = orc.PositionalMetadata(32, pm.astype(np.uint64), pb.astype(np.uint64))
        s2o, f2o, r2o = orc.compress_positional(pmd, xp)
        assert_image(s2, f2, r2, s2o, f2o, r2o, n_rows, row_bytes)
        assert torch.equal(ibp.ibp_decompress_positional(table, s2, f2), xpg)
        got = ibp.ibp_gather_decompress_positional(table, s2, f2, torch.from_numpy(ids).cuda())
        torch.cuda.synchronize()
        want = np.zeros((ids.size, row_bytes), np.uint8)
        want[inside] = xp[ids[inside]]
        assert np.array_equal(got.cpu().numpy(), want)
