"""ibp_build_metadata_noalloc (static device scratch, no hipMalloc) against
ibp_build_metadata on the same samples, through the C ABI: metadata and
per-bit counts equal, and equal to the oracle's; two calls in a row, the
second on a smaller sample, so that nothing carries over from the first."""
import ctypes

import numpy as np
import pytest

from oracle import oracle as orc
import synthetic as syn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ibp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_bit_level_amd import ibp as b
    b.lib()
    return b


def both(ibp, x: np.ndarray, w: int, n_blocks: int):
    """(allocating result, no-alloc result) through the C ABI on cuda:0."""
    xg = torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.uint8)).cuda()
    L = ibp.lib()
    res = []
    for fn in (L.ibp_build_metadata, L.ibp_build_metadata_noalloc):
        md = ibp.ibp_metadata()
        ones = (ctypes.c_uint64 * w)()
        rc = fn(ctypes.c_void_p(xg.data_ptr()), n_blocks, w, 900000, ctypes.byref(md), ones,
                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == ibp.IBP_OK, ibp.status_string(rc)
        res.append(((md.width_bits, md.invariant_bits, md.mask, md.bitval, md.t_ppm),
                    list(ones)))
    return res


@pytest.mark.parametrize("w", [32, 16, 64])
def test_noalloc_matches_allocating_call_twice(ibp, w):
    big = syn.dense_gnn_rows(0, 65536)                 # 64 MiB, 2^24 words
    small = syn.tiny_dense()[:777]                     # ragged: 99,456 words
    for x in (big, small):
        n_blocks = x.nbytes * 8 // w
        if w == 16:
            n_blocks -= 1                              # an odd 16-bit block count
        print(f"W={w}: {n_blocks} blocks", flush=True)
        (md_a, ones_a), (md_n, ones_n) = both(ibp, x, w, n_blocks)
        assert md_n == md_a
        assert ones_n == ones_a
        md_o, ones_o = orc.build_metadata(x.reshape(-1).view(np.uint8), w, n_blocks=n_blocks)
        assert (md_n[2], md_n[3]) == (md_o.mask, md_o.bitval)
        assert np.array_equal(np.array(ones_n, np.uint64), ones_o)


def test_noalloc_binding_and_stream_order(ibp):
    """The Python binding, a sample written on the same stream just before."""
    x = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    x.fill_(0x3C000001)
    md, ones = ibp.ibp_build_metadata_noalloc(x)
    assert (md.mask, md.bitval) == (0xFFFFFFFF, 0x3C000001)
    assert ones == [(1 << 20) if (0x3C000001 >> b) & 1 else 0 for b in range(32)]
