"""Host-side checks of the C ABI (no GPU needed).

* libibp.so loads and exports every function include/ibp.h declares;
* argument validation returns the documented status before anything is
  enqueued (these calls never reach HIP);
* the host half of the metadata step (ibp_metadata_from_counts) agrees with
  the oracle's rule on the oracle's own counts.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import oracle as orc
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "lossless_bit_level_amd", "libibp.so")
HEADER = os.path.join(ROOT, "include", "ibp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB),
                                reason="libibp.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def ibp():
    from lossless_bit_level_amd import ibp as b
    return b


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ibp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"ibp_build_metadata", "ibp_build_metadata_noalloc", "ibp_compress",
            "ibp_decompress", "ibp_gather_decompress"} <= set(names)
    L = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(L, n), n


def test_ceiling_library_exports_and_validation():
    """libibp_ceiling (the benchmark's gather-copy floor) exports what
    include/ibp_ceiling.h declares and rejects bad layouts before any HIP
    call."""
    lib = os.path.join(ROOT, "lossless_bit_level_amd", "libibp_ceiling.so")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ibp_ceiling.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(ibp_[a-z_]+)\s*\(", text)))
    assert names == ["ibp_ceiling_copy", "ibp_ceiling_gather_copy"]
    L = ctypes.CDLL(lib)
    for n in names:
        assert hasattr(L, n), n
    from lossless_bit_level_amd import ceiling
    T = ceiling.ibp_copy_tensor
    f = ceiling.lib().ibp_ceiling_gather_copy
    fake = 0x10000
    assert f(None, 0, 0, 0, None) == 0
    assert f((T * 1)(T(4, 4096, fake, fake, None, 0, fake)), 1, 0, 0, None) == 0   # nothing to copy
    for bad in [T(4, 4100, fake, fake, None, 4, fake),       # row_bytes % 16
                T(4, 4096, fake + 4, fake, None, 4, fake),   # misaligned src
                T(4, 4096, fake, fake, None, 5, fake),       # n_out > n_rows without ids
                T(4, 4096, fake, None, None, 4, fake),       # no src_bytes
                T(4, 4096, fake, fake, fake + 4, 4, fake)]:  # misaligned ids
        assert f((T * 1)(bad), 1, 0, 0, None) == -1
    assert f((T * 17)(), 17, 0, 0, None) == -1
    assert f((T * 1)(T(4, 4096, fake, fake, None, 4, fake)), 1, 0, 4, None) == -1  # unknown flag
    c = ceiling.lib().ibp_ceiling_copy
    assert c(None, None, 0, 0, None) == 0                   # nothing to copy
    assert c(fake, fake + 4096, 40, 0, None) == -1          # not a multiple of 16 bytes
    assert c(fake + 8, fake + 4096, 64, 0, None) == -1      # misaligned src
    assert c(fake, fake + 4100, 64, 0, None) == -1          # misaligned dst
    assert c(None, fake, 64, 0, None) == -1                 # null src


def test_flag_words_and_status_strings(ibp):
    assert [ibp.ibp_flag_words(n) for n in (0, 1, 63, 64, 65, 128, 129)] == \
        [0, 1, 1, 1, 2, 2, 3]
    for s in (0, -1, -2, -3, -4, -5):
        assert ibp.status_string(s) and ibp.status_string(s) != "unknown status"
    assert ibp.status_string(7) == "unknown status"


def _md(ibp, mask=0x7C000000, bitval=0x3C000000, w=32, p=None):
    md = ibp.ibp_metadata()
    md.width_bits, md.mask, md.bitval, md.t_ppm = w, mask, bitval, 900000
    md.invariant_bits = bin(mask).count("1") if p is None else p
    return md


def test_batch_validation_before_enqueue(ibp):
    """ibp_decompress_batch checks every tensor before it enqueues anything."""
    L = ibp.lib()
    md = _md(ibp)
    byref = ctypes.byref
    fake = 0x10000  # never dereferenced
    T = ibp.ibp_tensor
    good = T(4, 4096, fake, fake, fake)
    arr = (T * 3)(good, T(4, 4098, fake, fake, fake), good)       # row_bytes % 4
    assert L.ibp_decompress_batch(byref(md), arr, 3, None) == ibp.IBP_ERR_LAYOUT
    arr = (T * 2)(good, T(4, 4096, fake, None, fake))              # null flags
    assert L.ibp_decompress_batch(byref(md), arr, 2, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    arr = (T * 2)(good, T(4, 4096, fake, fake + 4, fake))          # misaligned flags
    assert L.ibp_decompress_batch(byref(md), arr, 2, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_decompress_batch(byref(md), None, 1, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_decompress_batch(None, arr, 1, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_decompress_batch(byref(md), None, 0, None) == ibp.IBP_OK
    empty = (T * 1)(T(0, 4096, None, None, None))                 # empty tensors: no-op
    assert L.ibp_decompress_batch(byref(md), empty, 1, None) == ibp.IBP_OK


def test_compress_batch_validation_before_enqueue(ibp):
    """ibp_compress_batch checks every tensor (ibp_compress's rules) before it
    enqueues anything."""
    L = ibp.lib()
    md = _md(ibp)
    byref = ctypes.byref
    fake = 0x10000  # never dereferenced
    T = ibp.ibp_compress_tensor
    good = T(4, 8192, fake, fake + (1 << 20), fake, None)
    arr = (T * 3)(good, T(4, 8194, fake, fake, fake, None), good)   # row_bytes % 4
    assert L.ibp_compress_batch(byref(md), arr, 3, None) == ibp.IBP_ERR_LAYOUT
    arr = (T * 2)(good, T(4, 8192, fake, fake, None, None))         # null flags
    assert L.ibp_compress_batch(byref(md), arr, 2, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    arr = (T * 2)(good, T(4, 8192, fake, fake + 8192, fake, None))  # src and slots overlap
    assert L.ibp_compress_batch(byref(md), arr, 2, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    arr = (T * 2)(good, T(4, 8192, fake, fake + (1 << 20), fake, fake + 2))  # row_bits
    assert L.ibp_compress_batch(byref(md), arr, 2, None) == ibp.IBP_ERR_LAYOUT
    big = T(4, (1 << 20) + 4, fake, fake + (1 << 24), fake, None)   # row too long
    assert L.ibp_compress_batch(byref(md), (T * 1)(big), 1, None) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_compress_batch(byref(md), None, 1, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress_batch(None, arr, 1, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress_batch(byref(md), None, 0, None) == ibp.IBP_OK
    empty = (T * 1)(T(0, 8192, None, None, None, None))            # empty tensors: no-op
    assert L.ibp_compress_batch(byref(md), empty, 1, None) == ibp.IBP_OK


def test_validation_before_enqueue(ibp):
    L = ibp.lib()
    md = _md(ibp)
    byref = ctypes.byref
    fake = 0x10000  # never dereferenced: every call below fails validation
    # null metadata / bad metadata
    assert L.ibp_compress(None, 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(_md(ibp, w=8)), 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_UNSUPPORTED
    # a 16-bit mask must fit 16 bits; 64-bit blocks need 8-byte rows and buffers
    assert L.ibp_compress(byref(_md(ibp, w=16)), 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(_md(ibp, 0x7C00, 0x3C00, w=16)), 0, 16, None, None, None, None, None) == ibp.IBP_OK
    assert L.ibp_compress(byref(_md(ibp, w=64)), 4, 12, fake, fake, fake, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(_md(ibp, w=64)), 4, 16, fake + 4, fake + 4096, fake, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_decompress(byref(_md(ibp, w=64)), 4, 16, fake, fake, fake + 4, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(_md(ibp, bitval=0x1)), 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(_md(ibp, p=3)), 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(_md(ibp, mask=1 << 40, bitval=0)), 4, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    # layout
    assert L.ibp_compress(byref(md), 4, 6, fake, fake, fake, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(md), 4, 0, fake, fake, fake, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(md), 4, 16, fake + 2, fake, fake, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(md), 4, 16, fake, fake, fake + 4, None, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_compress(byref(md), 4, ibp.IBP_MAX_COMPRESS_ROW_BYTES + 4, fake, fake, fake, None, None) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_compress(byref(md), 4, 16, None, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(md), 1 << 62, 16, fake, fake, fake, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    # src and slots may coincide (in place) but must not partly overlap
    assert L.ibp_compress(byref(md), 4, 16, fake, fake + 16, fake + 1024, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_compress(byref(md), 4, 16, fake + 48, fake, fake + 1024, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    # empty work is a no-op that needs no pointers
    assert L.ibp_compress(byref(md), 0, 16, None, None, None, None, None) == ibp.IBP_OK
    assert L.ibp_gather_decompress(byref(md), 10, 16, fake, fake, fake, 0, fake, None) == ibp.IBP_OK
    assert L.ibp_decompress(byref(md), 0, 16, None, None, None, None) == ibp.IBP_OK
    # decode validation
    assert L.ibp_decompress(byref(md), 4, 16, None, fake, fake, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_gather_decompress(byref(md), 4, 16, fake, fake, None, 3, fake, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_gather_decompress(byref(md), 0, 16, fake, fake, fake, 3, fake, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_gather_decompress(byref(md), 4, 16, fake, fake, fake + 4, 3, fake, None) == ibp.IBP_ERR_LAYOUT
    assert L.ibp_gather_decompress(byref(md), 4, 1 << 27, fake, fake, fake, 3, fake, None) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_gather_decompress(byref(md), 4, 16, fake, fake, fake, 1 << 61, fake, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    # metadata build
    out = ibp.ibp_metadata()
    assert L.ibp_build_metadata(fake, 0, 32, 900000, byref(out), None, None) == ibp.IBP_ERR_EMPTY
    assert L.ibp_build_metadata(fake, 10, 8, 900000, byref(out), None, None) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_build_metadata(fake, 10, 32, 1000001, byref(out), None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_build_metadata(None, 10, 32, 900000, byref(out), None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_build_metadata(fake + 1, 10, 32, 900000, byref(out), None, None) == ibp.IBP_ERR_LAYOUT
    # the no-allocation variant reports the same argument errors, before any HIP call
    nl = L.ibp_build_metadata_noalloc
    assert nl(fake, 0, 32, 900000, byref(out), None, None) == ibp.IBP_ERR_EMPTY
    assert nl(fake, 10, 8, 900000, byref(out), None, None) == ibp.IBP_ERR_UNSUPPORTED
    assert nl(fake, 10, 32, 1000001, byref(out), None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert nl(None, 10, 32, 900000, byref(out), None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert nl(fake, 10, 32, 900000, None, None, None) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_host_device_pointer(None, byref(ctypes.c_void_p())) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_last_hip_error() == 0


@pytest.mark.parametrize("t_ppm", [0, 500000, 500001, 900000, 999999, 1000000])
def test_metadata_from_counts_matches_oracle(ibp, t_ppm):
    rng = np.random.default_rng(t_ppm)
    samples = [syn.tiny_dense()[:256], syn.sparse_gnn_rows(0, 64),
               rng.integers(0, 2**32, 4096, dtype=np.uint64).astype(np.uint32),
               np.array([0x80000001, 0x80000001, 0x00000001, 0xFFFFFFFF], np.uint32)]
    for x in samples:
        md_o, ones = orc.build_metadata(x, 32, t_ppm=t_ppm)
        md = ibp.ibp_metadata_from_counts(ones, x.nbytes // 4, t_ppm=t_ppm)
        assert (md.mask, md.bitval, md.invariant_bits, md.t_ppm) == \
            (md_o.mask, md_o.bitval, md_o.invariant_bits, t_ppm)


def test_metadata_from_counts_rejects(ibp):
    L = ibp.lib()
    ones = (ctypes.c_uint64 * 32)(*([5] * 32))
    out = ibp.ibp_metadata()
    assert L.ibp_metadata_from_counts(ones, 4, 32, 900000, ctypes.byref(out)) == ibp.IBP_ERR_INVALID_ARGUMENT
    assert L.ibp_metadata_from_counts(ones, 0, 32, 900000, ctypes.byref(out)) == ibp.IBP_ERR_EMPTY
    assert L.ibp_metadata_from_counts(ones, 8, 8, 900000, ctypes.byref(out)) == ibp.IBP_ERR_UNSUPPORTED
    assert L.ibp_metadata_from_counts(None, 8, 32, 900000, ctypes.byref(out)) == ibp.IBP_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("w", [16, 64])
def test_metadata_from_counts_other_widths(ibp, w):
    rng = np.random.default_rng(w)
    dt = {16: np.uint16, 64: np.uint64}[w]
    x = rng.standard_normal(3000).astype(np.float32).view(np.uint32)
    samples = [x.view(dt), rng.integers(0, 2**63, 1000, dtype=np.int64).view(dt)]
    for t_ppm in (500000, 900000, 1000000):
        for smp in samples:
            md_o, ones = orc.build_metadata(smp, w, t_ppm=t_ppm)
            md = ibp.ibp_metadata_from_counts(ones, smp.size, t_ppm=t_ppm, width_bits=w)
            assert (md.mask, md.bitval, md.invariant_bits, md.width_bits) == \
                (md_o.mask, md_o.bitval, md_o.invariant_bits, w)


def test_positional_table_drives_extract_and_deposit(ibp):
    """The host-built position table: mask/bitval/p per entry, the planes of p
    per 64-position chunk, and five shift masks with which the kernels'
    extract and deposit steps (replayed here) equal bit-serial PEXT/PDEP."""
    rng = np.random.default_rng(8)
    n = 150
    mask = rng.integers(0, 2**32, n, dtype=np.uint64)
    mask[:6] = [0, 0xFFFFFFFF, 0x80000000, 1, 0x83FF83FF, 0x7C007C00]
    bitval = mask & rng.integers(0, 2**32, n, dtype=np.uint64)
    tab = ibp.ibp_positional_table(mask, bitval).numpy()
    assert tab.size >= ibp.ibp_positional_table_bytes(n) == 32 * n + 64 * 3
    ent = tab[:32 * n].view(np.uint32).reshape(n, 8)
    planes = tab[32 * n:32 * n + 64 * 3].view(np.uint64).reshape(3, 8)
    M = 0xFFFFFFFF
    for k in range(n):
        m, bv, p = int(ent[k, 0]), int(ent[k, 1]), int(ent[k, 2])
        assert (m, bv, p) == (int(mask[k]), int(bitval[k]), bin(int(mask[k])).count("1"))
        for t in range(8):
            assert (int(planes[k // 64, t]) >> (k % 64)) & 1 == ((p >> t) & 1 if t < 6 else 0)
        sfx = [int(v) for v in ent[k, 3:8]]
        keep = ~m & M
        for x in [int(v) for v in rng.integers(0, 2**32, 40)]:
            y = x & keep
            for i in range(5):
                t = y & sfx[i]
                y = ((y ^ t) | (t >> (1 << i))) & M
            assert y == orc.pext(x, keep)
            v = y
            for i in range(4, -1, -1):
                v = (((v << (1 << i)) & M) & sfx[i]) | (v & ~sfx[i] & M)
            assert ((v & keep) | bv) == ((x & keep) | bv)
    with pytest.raises(ibp.IBPError):
        ibp.ibp_positional_table([0x0F], [0x10])
