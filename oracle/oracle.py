"""Python face of the CPU oracle for Invariant Bit Packing.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU
baseline of the benchmark use this module; the product library never does.
The method's arithmetic (metadata, compression, decompression, gather,
global and per-position) lives in ``ibp_oracle.c`` (plain bit-serial C, see
its header for the method's source and the readings of it); for those this
file only compiles the C with gcc, loads it with ctypes and moves numpy
arrays in and out.  One part is written here in Python instead: the packed
layout of the compressed GPU cache (cache_pack, cache_gather), which is plain
byte bookkeeping around the C decoder -- each cached row's stored words
copied back to back at 16-byte boundaries, with a 64-bit locator per row.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ibp_oracle.c")
_LIB = os.path.join(_HERE, "libibp_oracle.so")

GCC_CMD = ["gcc", "-O2", "-std=gnu11", "-Wall", "-Wextra", "-shared", "-fPIC",
           _SRC, "-o", _LIB]


def build(force: bool = False) -> str:
    """Compile the oracle shared object (gcc, no GPU headers).

    IBP_ORACLE_LIB names another build of the same source (the pin tests use
    it to run deliberately broken copies of the oracle)."""
    override = os.environ.get("IBP_ORACLE_LIB")
    if override:
        return override
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        i64p = ctypes.POINTER(ctypes.c_int64)
        u64, u32, c_uint, c_int = (ctypes.c_uint64, ctypes.c_uint32,
                                   ctypes.c_uint, ctypes.c_int)
        L.orc_pext.restype = u64
        L.orc_pext.argtypes = [u64, u64]
        L.orc_pdep.restype = u64
        L.orc_pdep.argtypes = [u64, u64]
        L.orc_build_metadata.restype = c_int
        L.orc_build_metadata.argtypes = [u8p, u64, c_uint, u32, u64p, u64p, u64p]
        L.orc_stored_bytes.restype = u64
        L.orc_stored_bytes.argtypes = [u64, u64, c_int]
        L.orc_compress_row.restype = c_int
        L.orc_compress_row.argtypes = [u8p, u64, c_uint, u64, u64, u8p, u64p,
                                       ctypes.POINTER(c_int)]
        L.orc_decompress_row.restype = c_int
        L.orc_decompress_row.argtypes = [u8p, u64, c_uint, u64, u64, c_int, u8p]
        L.orc_compress_table.restype = c_int
        L.orc_compress_table.argtypes = [u8p, u64, u64, c_uint, u64, u64, u8p,
                                         u64p, u64p]
        L.orc_gather_decompress.restype = c_int
        L.orc_gather_decompress.argtypes = [u8p, u64p, u64, u64, c_uint, u64,
                                            u64, i64p, u64, u8p]
        L.orc_build_metadata_positional.restype = c_int
        L.orc_build_metadata_positional.argtypes = [u8p, u64, u64, c_uint, u32, u64p, u64p]
        L.orc_compress_row_positional.restype = c_int
        L.orc_compress_row_positional.argtypes = [u8p, u64, c_uint, u64p, u64p, u8p, u64p,
                                                  ctypes.POINTER(c_int)]
        L.orc_decompress_row_positional.restype = c_int
        L.orc_decompress_row_positional.argtypes = [u8p, u64, c_uint, u64p, u64p, c_int, u8p]
        L.orc_compress_table_positional.restype = c_int
        L.orc_compress_table_positional.argtypes = [u8p, u64, u64, c_uint, u64p, u64p, u8p,
                                                    u64p, u64p]
        L.orc_gather_decompress_positional.restype = c_int
        L.orc_gather_decompress_positional.argtypes = [u8p, u64p, u64, u64, c_uint, u64p,
                                                       u64p, i64p, u64, u8p]
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _bytes2d(x: np.ndarray) -> np.ndarray:
    """View a 2-D array of any dtype as [rows, row_bytes] uint8."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    return x.reshape(x.shape[0], -1).view(np.uint8)


@dataclass(frozen=True)
class Metadata:
    width_bits: int
    mask: int
    bitval: int
    t_ppm: int

    @property
    def invariant_bits(self) -> int:
        return bin(self.mask).count("1")


def t_to_ppm(t: float) -> int:
    """Threshold T as an integer number of parts per million."""
    return int(round(t * 1_000_000))


def pext(x: int, m: int) -> int:
    return int(lib().orc_pext(x, m))


def pdep(v: int, m: int) -> int:
    return int(lib().orc_pdep(v, m))


def build_metadata(sample: np.ndarray, width_bits: int = 32, t: float = 0.9,
                   t_ppm: int | None = None, n_blocks: int | None = None):
    """Mask/Bitval over the blocks of ``sample`` (read as a flat bit string).

    Returns (Metadata, ones) where ones[b] counts the sample blocks with bit b
    set.  ``n_blocks`` defaults to every whole block of the buffer.
    """
    raw = np.ascontiguousarray(sample).reshape(-1).view(np.uint8)
    if n_blocks is None:
        n_blocks = raw.size * 8 // width_bits
    ppm = t_to_ppm(t) if t_ppm is None else int(t_ppm)
    ones = np.zeros(64, np.uint64)
    mask = ctypes.c_uint64()
    bitval = ctypes.c_uint64()
    buf = raw if raw.size else np.zeros(1, np.uint8)
    rc = lib().orc_build_metadata(_p(buf, ctypes.c_uint8), n_blocks, width_bits,
                                  ppm, _p(ones, ctypes.c_uint64),
                                  ctypes.byref(mask), ctypes.byref(bitval))
    if rc:
        raise ValueError(f"orc_build_metadata failed: {rc}")
    md = Metadata(width_bits, int(mask.value), int(bitval.value), ppm)
    return md, ones[:width_bits].copy()


def stored_bytes(row_bytes: int, c_bits: int, flag: int) -> int:
    return int(lib().orc_stored_bytes(row_bytes, c_bits, int(flag)))


def compress(md: Metadata, x: np.ndarray):
    """Compress a table (rows = first axis).  Returns (slots, flags, row_bits).

    slots: uint8 [n_rows, row_bytes]; flags: uint64 [ceil(n_rows/64)];
    row_bits: uint64 [n_rows] (C of every row, raw rows included).
    """
    src = _bytes2d(x)
    n_rows, row_bytes = src.shape
    slots = np.zeros((n_rows, row_bytes), np.uint8)
    flags = np.zeros(max(1, (n_rows + 63) // 64), np.uint64)
    row_bits = np.zeros(max(1, n_rows), np.uint64)
    rc = lib().orc_compress_table(
        _p(src, ctypes.c_uint8) if n_rows else None, n_rows, row_bytes,
        md.width_bits, md.mask, md.bitval,
        _p(slots, ctypes.c_uint8) if n_rows else None,
        _p(flags, ctypes.c_uint64), _p(row_bits, ctypes.c_uint64))
    if rc:
        raise ValueError(f"orc_compress_table failed: {rc}")
    return slots, flags[:(n_rows + 63) // 64], row_bits[:n_rows]


def compress_row(md: Metadata, row: np.ndarray):
    """One row -> (slot bytes, C, flag)."""
    r = np.ascontiguousarray(row).reshape(-1).view(np.uint8)
    slot = np.zeros_like(r)
    c = ctypes.c_uint64()
    f = ctypes.c_int()
    rc = lib().orc_compress_row(_p(r, ctypes.c_uint8), r.size, md.width_bits,
                                md.mask, md.bitval, _p(slot, ctypes.c_uint8),
                                ctypes.byref(c), ctypes.byref(f))
    if rc:
        raise ValueError(f"orc_compress_row failed: {rc}")
    return slot, int(c.value), int(f.value)


def decompress_row(md: Metadata, slot: np.ndarray, flag: int) -> np.ndarray:
    s = np.ascontiguousarray(slot).reshape(-1).view(np.uint8)
    out = np.zeros_like(s)
    rc = lib().orc_decompress_row(_p(s, ctypes.c_uint8), s.size, md.width_bits,
                                  md.mask, md.bitval, int(flag),
                                  _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError(f"orc_decompress_row failed: {rc}")
    return out


def gather_decompress(md: Metadata, slots: np.ndarray, flags: np.ndarray,
                      ids: np.ndarray) -> np.ndarray:
    """out[i] = decompressed row ids[i] (uint8 [n_ids, row_bytes])."""
    s = _bytes2d(slots)
    n_rows, row_bytes = s.shape
    ids = np.ascontiguousarray(ids, dtype=np.int64).reshape(-1)
    fl = np.ascontiguousarray(flags, dtype=np.uint64)
    if fl.size == 0:
        fl = np.zeros(1, np.uint64)
    out = np.zeros((ids.size, row_bytes), np.uint8)
    if ids.size == 0:
        return out
    rc = lib().orc_gather_decompress(
        _p(s, ctypes.c_uint8), _p(fl, ctypes.c_uint64), n_rows, row_bytes,
        md.width_bits, md.mask, md.bitval, _p(ids, ctypes.c_int64), ids.size,
        _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError(f"orc_gather_decompress failed: {rc}")
    return out


def decompress(md: Metadata, slots: np.ndarray, flags: np.ndarray) -> np.ndarray:
    n_rows = _bytes2d(slots).shape[0]
    return gather_decompress(md, slots, flags, np.arange(n_rows, dtype=np.int64))


def image_bytes_equal(slots_a: np.ndarray, slots_b: np.ndarray,
                      flags: np.ndarray, row_bits: np.ndarray) -> np.ndarray:
    """Per-row equality of two images over the bytes that belong to the image.

    Returns a bool array; bytes of a compressed slot past its padded stream
    are ignored.
    """
    a, b = _bytes2d(slots_a), _bytes2d(slots_b)
    n_rows, row_bytes = a.shape
    ok = np.empty(n_rows, bool)
    for r in range(n_rows):
        f = int((int(flags[r >> 6]) >> (r & 63)) & 1)
        nb = stored_bytes(row_bytes, int(row_bits[r]), f)
        ok[r] = np.array_equal(a[r, :nb], b[r, :nb])
    return ok


# ----------------------------------------------------------- packed cache --
# Cache compression ([IBP] System integration): rows held in a GPU software
# cache are kept in their stored form.  The page fixes no layout for it; this
# is the library's, written out from its definition:
#   * entry e holds the stored words of row ids[e] (ceil(C/32) words of a
#     compressed row, all S/4 words of a raw row), zero padded to a multiple
#     of 16 bytes; entries follow each other in id order from offset 0;
#   * its locator is resident (bit 63) | compressed (bit 62) | words << 36 |
#     offset in 16-byte units (bits 0..35); an id outside the table gets
#     locator 0 and no space.
LOC_RESIDENT = 1 << 63
LOC_COMPRESSED = 1 << 62
LOC_WORDS_SHIFT = 36
LOC_WORDS_MASK = (1 << 26) - 1
LOC_OFFSET_MASK = (1 << 36) - 1


def cache_pack(slots: np.ndarray, flags: np.ndarray, row_bits: np.ndarray,
               ids: np.ndarray):
    """(entry locators uint64 [n_ids], arena uint8) for rows ids of an image."""
    s = _bytes2d(slots)
    n_rows, row_bytes = s.shape
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    locs = np.zeros(ids.size, np.uint64)
    parts = []
    off = 0
    for e, r in enumerate(ids):
        r = int(r)
        if not 0 <= r < n_rows:
            continue
        f = (int(flags[r >> 6]) >> (r & 63)) & 1
        nb = stored_bytes(row_bytes, int(row_bits[r]), f)
        padded = (nb + 15) // 16 * 16
        entry = np.zeros(padded, np.uint8)
        entry[:nb] = s[r, :nb]
        parts.append(entry)
        locs[e] = LOC_RESIDENT | (f * LOC_COMPRESSED) | ((nb // 4) << LOC_WORDS_SHIFT) | off
        off += padded // 16
    arena = np.concatenate(parts) if parts else np.zeros(0, np.uint8)
    return locs, arena


def cache_gather(md: Metadata, arena: np.ndarray, cache_loc: np.ndarray,
                 slots: np.ndarray, flags: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """out[i] = row ids[i] restored from its arena entry when cache_loc marks
    it resident, else from the image; zero for an id outside the table."""
    s = _bytes2d(slots)
    n_rows, row_bytes = s.shape
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.zeros((ids.size, row_bytes), np.uint8)
    for i, r in enumerate(ids):
        r = int(r)
        if not 0 <= r < n_rows:
            continue
        loc = int(cache_loc[r])
        if loc & LOC_RESIDENT:
            words = (loc >> LOC_WORDS_SHIFT) & LOC_WORDS_MASK
            at = (loc & LOC_OFFSET_MASK) * 16
            slot = np.zeros(row_bytes, np.uint8)
            slot[:words * 4] = arena[at:at + words * 4]
            out[i] = decompress_row(md, slot, int(bool(loc & LOC_COMPRESSED)))
        else:
            out[i] = decompress_row(md, s[r], (int(flags[r >> 6]) >> (r & 63)) & 1)
    return out



# ---------------------------------------------------- per-position metadata --
# One Mask/Bitval per block position k of a row (the kilobyte-sized reading
# of the page's fixed-size metadata); arithmetic in ibp_oracle.c.

@dataclass
class PositionalMetadata:
    width_bits: int
    mask: np.ndarray      # uint64 [n]
    bitval: np.ndarray    # uint64 [n]
    t_ppm: int = 900000

    @property
    def invariant_bits(self) -> np.ndarray:
        return np.array([bin(int(m)).count("1") for m in self.mask], np.int64)


def build_metadata_positional(sample_rows: np.ndarray, width_bits: int = 32,
                              t: float = 0.9, t_ppm: int | None = None) -> PositionalMetadata:
    """Per-position metadata from the rows of a sample (first axis = rows)."""
    s = _bytes2d(sample_rows)
    n_rows, row_bytes = s.shape
    n = row_bytes * 8 // width_bits
    ppm = t_to_ppm(t) if t_ppm is None else int(t_ppm)
    mask = np.zeros(n, np.uint64)
    bitval = np.zeros(n, np.uint64)
    rc = lib().orc_build_metadata_positional(
        _p(s, ctypes.c_uint8), n_rows, row_bytes, width_bits, ppm,
        _p(mask, ctypes.c_uint64), _p(bitval, ctypes.c_uint64))
    if rc:
        raise ValueError(f"orc_build_metadata_positional failed: {rc}")
    return PositionalMetadata(width_bits, mask, bitval, ppm)


def _pm_arrays(pm: PositionalMetadata):
    return (np.ascontiguousarray(pm.mask, dtype=np.uint64),
            np.ascontiguousarray(pm.bitval, dtype=np.uint64))


def compress_positional(pm: PositionalMetadata, x: np.ndarray):
    """Like compress(), with per-position metadata."""
    src = _bytes2d(x)
    n_rows, row_bytes = src.shape
    m, b = _pm_arrays(pm)
    slots = np.zeros((n_rows, row_bytes), np.uint8)
    flags = np.zeros(max(1, (n_rows + 63) // 64), np.uint64)
    row_bits = np.zeros(max(1, n_rows), np.uint64)
    rc = lib().orc_compress_table_positional(
        _p(src, ctypes.c_uint8) if n_rows else None, n_rows, row_bytes, pm.width_bits,
        _p(m, ctypes.c_uint64), _p(b, ctypes.c_uint64),
        _p(slots, ctypes.c_uint8) if n_rows else None,
        _p(flags, ctypes.c_uint64), _p(row_bits, ctypes.c_uint64))
    if rc:
        raise ValueError(f"orc_compress_table_positional failed: {rc}")
    return slots, flags[:(n_rows + 63) // 64], row_bits[:n_rows]


def compress_row_positional(pm: PositionalMetadata, row: np.ndarray):
    r = np.ascontiguousarray(row).reshape(-1).view(np.uint8)
    m, b = _pm_arrays(pm)
    slot = np.zeros_like(r)
    c = ctypes.c_uint64()
    f = ctypes.c_int()
    rc = lib().orc_compress_row_positional(
        _p(r, ctypes.c_uint8), r.size, pm.width_bits, _p(m, ctypes.c_uint64),
        _p(b, ctypes.c_uint64), _p(slot, ctypes.c_uint8), ctypes.byref(c), ctypes.byref(f))
    if rc:
        raise ValueError(f"orc_compress_row_positional failed: {rc}")
    return slot, int(c.value), int(f.value)


def gather_decompress_positional(pm: PositionalMetadata, slots: np.ndarray,
                                 flags: np.ndarray, ids: np.ndarray) -> np.ndarray:
    s = _bytes2d(slots)
    n_rows, row_bytes = s.shape
    m, b = _pm_arrays(pm)
    ids = np.ascontiguousarray(ids, dtype=np.int64).reshape(-1)
    fl = np.ascontiguousarray(flags, dtype=np.uint64)
    if fl.size == 0:
        fl = np.zeros(1, np.uint64)
    out = np.zeros((ids.size, row_bytes), np.uint8)
    if ids.size == 0:
        return out
    rc = lib().orc_gather_decompress_positional(
        _p(s, ctypes.c_uint8), _p(fl, ctypes.c_uint64), n_rows, row_bytes, pm.width_bits,
        _p(m, ctypes.c_uint64), _p(b, ctypes.c_uint64), _p(ids, ctypes.c_int64), ids.size,
        _p(out, ctypes.c_uint8))
    if rc:
        raise ValueError(f"orc_gather_decompress_positional failed: {rc}")
    return out


def decompress_positional(pm: PositionalMetadata, slots: np.ndarray,
                          flags: np.ndarray) -> np.ndarray:
    n_rows = _bytes2d(slots).shape[0]
    return gather_decompress_positional(pm, slots, flags, np.arange(n_rows, dtype=np.int64))
