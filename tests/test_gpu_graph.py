"""The hot-path entry points inside a captured HIP graph.

ibp_compress_batch, ibp_decompress_batch, ibp_gather_decompress and the
per-position compress and gather allocate nothing and never synchronize, so
a caller can capture them once and replay them.  One graph holds all of them
on bf16 tables with 4, 8, 14 and 28 KiB rows; it is replayed four times,
with the tables, ids and outputs rewritten by ordinary (eager) work between
replays, and every replay is checked against eager calls on the same inputs
(images, flags and C values) and against the source rows (lossless round
trip).  The graph records kernel launches only: none of these calls clears
memory with a memset, and the flag words are written by the compression
kernels themselves."""
import numpy as np
import pytest

import synthetic as syn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(1000, 2048), (80, 4096), (300, 7168), (96, 14336)]  # bf16 elements per row


@pytest.fixture(scope="module")
def ibp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_level_amd import ibp as b
    b.lib()
    return b


def bf16_rows(rng, shape, sigma):
    x = (rng.standard_normal(shape, dtype=np.float32) * sigma).astype(np.float32)
    return syn.f32_to_bf16_bits(x).view(np.uint8).reshape(shape[0], -1)


def flag_bits(flags, n_rows):
    f = flags.cpu().numpy().view(np.uint64)
    return ((f[np.arange(n_rows) // 64] >> (np.arange(n_rows) % 64).astype(np.uint64)) & 1
            ).astype(bool)


def assert_same_image(got, want, n_rows, row_bytes):
    """Same flag bits, same C values and the same stored words in every row."""
    (gs, gf, gb), (ws, wf, wb) = got, want
    fg, fw = flag_bits(gf, n_rows), flag_bits(wf, n_rows)
    assert np.array_equal(fg, fw)
    cg, cw = gb.cpu().numpy()[:n_rows], wb.cpu().numpy()[:n_rows]
    assert np.array_equal(cg, cw)
    sg, sw = gs.cpu().numpy(), ws.cpu().numpy()
    stored = np.where(fw, 4 * ((cw.astype(np.int64) + 31) // 32), row_bytes)
    for r in range(n_rows):
        assert np.array_equal(sg[r, :stored[r]], sw[r, :stored[r]]), f"row {r}"


def test_graph_replays_match_eager(ibp):
    dev = torch.device("cuda")
    rng = np.random.default_rng(11)
    tables = [torch.from_numpy(bf16_rows(rng, s, 0.02)).to(dev) for s in SHAPES]
    md, _ = ibp.ibp_build_metadata(tables[0][:512])
    assert md.invariant_bits > 0
    # per-position metadata over the 4 KiB rows
    ptab, _, _ = ibp.ibp_build_metadata_positional(tables[0][:512])

    imgs = [(torch.empty_like(t),
             torch.empty(max(1, ibp.ibp_flag_words(t.shape[0])), dtype=torch.int64, device=dev),
             torch.empty(t.shape[0], dtype=torch.int32, device=dev)) for t in tables]
    outs = [torch.empty_like(t) for t in tables]
    n0, S0 = tables[0].shape
    ids = torch.empty(777, dtype=torch.int64, device=dev)
    gout = torch.empty((ids.numel(), S0), dtype=torch.uint8, device=dev)
    pimg = (torch.empty_like(tables[0]),
            torch.empty(ibp.ibp_flag_words(n0), dtype=torch.int64, device=dev),
            torch.empty(n0, dtype=torch.int32, device=dev))
    pout = torch.empty_like(gout)

    def calls():
        ibp.ibp_compress_batch(md, tables, imgs)
        ibp.ibp_decompress_batch(md, [(s, f) for s, f, _ in imgs], outs)
        ibp.ibp_gather_decompress(md, imgs[0][0], imgs[0][1], ids, out=gout)
        ibp.ibp_compress_positional(ptab, tables[0], *pimg)
        ibp.ibp_gather_decompress_positional(ptab, pimg[0], pimg[1], ids, out=pout)

    ids.copy_(torch.from_numpy(rng.integers(0, n0, ids.numel())))
    calls()  # eager once: every kernel is loaded before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()

    for rep in range(4):
        # ordinary work between replays: new rows (the last replay with wider
        # values, so that some rows stay raw), new ids with a repeat and an id
        # outside the table, poisoned outputs
        sigma = 0.02 if rep < 3 else 0.02 * 2.0 ** 40
        for t, s in zip(tables, SHAPES):
            t.copy_(torch.from_numpy(bf16_rows(rng, s, sigma)))
        new_ids = rng.integers(0, n0, ids.numel())
        new_ids[5] = new_ids[4]
        new_ids[6] = -1
        ids.copy_(torch.from_numpy(new_ids))
        for o in outs + [gout, pout]:
            o.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()

        ref_imgs = ibp.ibp_compress_batch(md, tables)
        ref_outs = ibp.ibp_decompress_batch(md, [(s, f) for s, f, _ in ref_imgs])
        ref_g = ibp.ibp_gather_decompress(md, ref_imgs[0][0], ref_imgs[0][1], ids)
        ref_p = ibp.ibp_compress_positional(ptab, tables[0])
        ref_pg = ibp.ibp_gather_decompress_positional(ptab, ref_p[0], ref_p[1], ids)
        torch.cuda.synchronize()

        for t, img, ref, o, ro in zip(tables, imgs, ref_imgs, outs, ref_outs):
            assert_same_image(img, ref, t.shape[0], t.shape[1])
            assert torch.equal(o, t) and torch.equal(ro, t)
        assert_same_image(pimg, ref_p, n0, S0)
        src = tables[0].cpu().numpy()
        want = np.where((new_ids >= 0)[:, None], src[np.clip(new_ids, 0, n0 - 1)], 0)
        for got in (gout, ref_g, pout, ref_pg):
            assert np.array_equal(got.cpu().numpy(), want)
        if rep == 3:  # wide values: the raw-row path ran in the graph too
            assert not flag_bits(imgs[0][1], n0).all()
