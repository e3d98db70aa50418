"""Thin ctypes binding of libibp (include/ibp.h), same names as the C ABI.

Argument marshalling only: every step of compression and decompression runs
in the HIP kernels of libibp.so.  PyTorch supplies device memory and the
current HIP stream.  If libibp.so has not been built this module raises on
first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libibp.so")

IBP_OK = 0
IBP_ERR_INVALID_ARGUMENT = -1
IBP_ERR_UNSUPPORTED = -2
IBP_ERR_LAYOUT = -3
IBP_ERR_EMPTY = -4
IBP_ERR_HIP = -5
IBP_MAX_COMPRESS_ROW_BYTES = 98304
IBP_LOC_RESIDENT = 1 << 63
IBP_LOC_COMPRESSED = 1 << 62
IBP_LOC_WORDS_SHIFT = 36
IBP_LOC_WORDS_MASK = (1 << 26) - 1
IBP_LOC_OFFSET_MASK = (1 << 36) - 1


class ibp_tensor(ctypes.Structure):
    """One tensor of ibp_decompress_batch (see include/ibp.h)."""
    _fields_ = [("n_rows", ctypes.c_uint64),
                ("row_bytes", ctypes.c_uint64),
                ("slots", ctypes.c_void_p),
                ("flags", ctypes.c_void_p),
                ("dst", ctypes.c_void_p)]


class ibp_compress_tensor(ctypes.Structure):
    """One tensor of ibp_compress_batch (see include/ibp.h)."""
    _fields_ = [("n_rows", ctypes.c_uint64),
                ("row_bytes", ctypes.c_uint64),
                ("src", ctypes.c_void_p),
                ("slots", ctypes.c_void_p),
                ("flags", ctypes.c_void_p),
                ("row_bits", ctypes.c_void_p)]


class ibp_metadata(ctypes.Structure):
    _fields_ = [("width_bits", ctypes.c_uint32),
                ("invariant_bits", ctypes.c_uint32),
                ("mask", ctypes.c_uint64),
                ("bitval", ctypes.c_uint64),
                ("t_ppm", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]

    def __repr__(self):
        return (f"ibp_metadata(W={self.width_bits}, p={self.invariant_bits}, "
                f"mask=0x{self.mask:08X}, bitval=0x{self.bitval:08X}, "
                f"t_ppm={self.t_ppm})")


class IBPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn}: {status_string(status)} ({status})"
        if status == IBP_ERR_HIP:
            msg += f", hipError {lib().ibp_last_hip_error()}"
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libibp.so (built in-tree by lossless_bit_level_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m lossless_bit_level_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, u64, u32, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        mdp = ctypes.POINTER(ibp_metadata)
        L.ibp_metadata_from_counts.argtypes = [vp, u64, u32, u32, mdp]
        L.ibp_build_metadata.argtypes = [vp, u64, u32, u32, mdp, vp, vp]
        L.ibp_build_metadata_noalloc.argtypes = [vp, u64, u32, u32, mdp, vp, vp]
        L.ibp_compress.argtypes = [mdp, u64, u64, vp, vp, vp, vp, vp]
        L.ibp_decompress.argtypes = [mdp, u64, u64, vp, vp, vp, vp]
        L.ibp_gather_decompress.argtypes = [mdp, u64, u64, vp, vp, vp, u64, vp, vp]
        L.ibp_decompress_batch.argtypes = [mdp, ctypes.POINTER(ibp_tensor), u64, vp]
        L.ibp_compress_batch.argtypes = [mdp, ctypes.POINTER(ibp_compress_tensor), u64, vp]
        L.ibp_cache_plan.argtypes = [mdp, u64, u64, vp, vp, vp, u64, vp, ctypes.POINTER(u64), vp]
        L.ibp_cache_fill.argtypes = [mdp, u64, u64, vp, vp, vp, u64, vp, vp, u64, vp, vp]
        L.ibp_gather_decompress_cached.argtypes = [mdp, u64, u64, vp, vp, vp, vp, vp, u64, vp, vp]
        L.ibp_positional_table_bytes.argtypes = [u64]
        L.ibp_positional_table_bytes.restype = u64
        L.ibp_positional_table.argtypes = [vp, vp, u64, vp]
        L.ibp_build_metadata_positional.argtypes = [vp, u64, u64, u32, vp, vp, vp, vp]
        L.ibp_compress_positional.argtypes = [vp, u64, u64, vp, vp, vp, vp, vp]
        L.ibp_decompress_positional.argtypes = [vp, u64, u64, vp, vp, vp, vp]
        L.ibp_gather_decompress_positional.argtypes = [vp, u64, u64, vp, vp, vp, u64, vp, vp]
        L.ibp_flag_words.argtypes = [u64]
        L.ibp_flag_words.restype = u64
        L.ibp_host_device_pointer.argtypes = [vp, ctypes.POINTER(vp)]
        L.ibp_status_string.argtypes = [i32]
        L.ibp_status_string.restype = ctypes.c_char_p
        L.ibp_last_hip_error.argtypes = []
        for f in ("ibp_metadata_from_counts", "ibp_build_metadata",
                  "ibp_build_metadata_noalloc", "ibp_compress",
                  "ibp_decompress", "ibp_decompress_batch", "ibp_gather_decompress",
                  "ibp_host_device_pointer",
                  "ibp_last_hip_error", "ibp_cache_plan", "ibp_cache_fill",
                  "ibp_gather_decompress_cached", "ibp_positional_table",
                  "ibp_build_metadata_positional", "ibp_compress_positional",
                  "ibp_decompress_positional", "ibp_gather_decompress_positional"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ibp_status_string(status).decode()


def _check(fn: str, status: int):
    if status != IBP_OK:
        raise IBPError(fn, status)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dptr(t: torch.Tensor) -> int:
    """Device-visible address of a CUDA tensor or of a pinned host tensor."""
    if t.is_cuda:
        return t.data_ptr()
    if t.is_pinned():
        return ibp_host_device_pointer(t)
    raise ValueError("tensor must be on the GPU or in pinned host memory")


def _need_cuda(t: torch.Tensor, name: str):
    """Arguments the kernels write, or read as device memory, must be GPU
    tensors (a CPU pointer there would fault the GPU)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t


def _rows(t: torch.Tensor):
    """(n_rows, row_bytes) of a tensor whose first axis is the row axis."""
    if t.dim() == 0:
        raise ValueError("need at least one dimension")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    n_rows = t.shape[0]
    row_bytes = (t.numel() // n_rows) * t.element_size() if n_rows else \
        int(torch.tensor(t.shape[1:]).prod().item()) * t.element_size()
    return n_rows, row_bytes


def ibp_flag_words(n_rows: int) -> int:
    return int(lib().ibp_flag_words(n_rows))


def ibp_host_device_pointer(t: torch.Tensor) -> int:
    dev = ctypes.c_void_p()
    _check("ibp_host_device_pointer",
           lib().ibp_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(dev)))
    return int(dev.value)


def ibp_metadata_from_counts(ones, n_blocks: int, t_ppm: int = 900000,
                             width_bits: int = 32) -> ibp_metadata:
    arr = (ctypes.c_uint64 * width_bits)(*[int(v) for v in ones])
    md = ibp_metadata()
    _check("ibp_metadata_from_counts",
           lib().ibp_metadata_from_counts(arr, n_blocks, width_bits, t_ppm, ctypes.byref(md)))
    return md


def ibp_build_metadata(sample: torch.Tensor, t: float = 0.9, width_bits: int = 32,
                       n_blocks: int | None = None, t_ppm: int | None = None,
                       stream=None, _fn: str = "ibp_build_metadata"):
    """Mask/Bitval over the width_bits-bit blocks of `sample` (GPU or pinned
    host memory).

    Returns (ibp_metadata, ones) with ones a list of the per-bit counts.
    Synchronous."""
    avail = sample.numel() * sample.element_size() * 8 // width_bits
    if n_blocks is None:
        n_blocks = avail
    if not 0 <= n_blocks <= avail:
        raise ValueError(f"n_blocks={n_blocks} but the sample holds {avail} blocks")
    if not sample.is_contiguous():
        raise ValueError("sample must be contiguous")
    ppm = int(round(t * 1_000_000)) if t_ppm is None else int(t_ppm)
    md = ibp_metadata()
    ones = (ctypes.c_uint64 * width_bits)()
    _check(_fn, getattr(lib(), _fn)(_dptr(sample), n_blocks, width_bits, ppm,
                                    ctypes.byref(md), ones, _stream(stream)))
    return md, list(ones)


def ibp_build_metadata_noalloc(sample: torch.Tensor, t: float = 0.9, width_bits: int = 32,
                               n_blocks: int | None = None, t_ppm: int | None = None,
                               stream=None):
    """ibp_build_metadata with the library's static scratch instead of a
    per-call device allocation (for callers that cannot allocate)."""
    return ibp_build_metadata(sample, t, width_bits, n_blocks, t_ppm, stream,
                              _fn="ibp_build_metadata_noalloc")


def ibp_compress(md: ibp_metadata, src: torch.Tensor, slots: torch.Tensor | None = None,
                 flags: torch.Tensor | None = None, row_bits: torch.Tensor | None = None,
                 want_row_bits: bool = True, stream=None):
    """Compress the rows of `src` (first axis = rows).  Returns
    (slots uint8 [n_rows, row_bytes], flags int64 [flag words], row_bits
    int32 [n_rows] or None).  Asynchronous on the current stream."""
    n_rows, row_bytes = _rows(src)
    dev = src.device if src.is_cuda else torch.device("cuda")
    if slots is None:
        slots = torch.empty((n_rows, row_bytes), dtype=torch.uint8, device=dev)
    if flags is None:
        flags = torch.empty(max(1, ibp_flag_words(n_rows)), dtype=torch.int64, device=dev)
    if row_bits is None and want_row_bits:
        row_bits = torch.empty(max(1, n_rows), dtype=torch.int32, device=dev)
    _need_cuda(flags, "flags")
    if row_bits is not None:
        _need_cuda(row_bits, "row_bits")
    _check("ibp_compress",
           lib().ibp_compress(ctypes.byref(md), n_rows, row_bytes, _dptr(src), _dptr(slots),
                              flags.data_ptr(),
                              row_bits.data_ptr() if row_bits is not None else None,
                              _stream(stream)))
    return slots, flags, row_bits


def _compress_batch_args(srcs, outs):
    arr = (ibp_compress_tensor * max(1, len(srcs)))()
    for k, (src, (slots, flags, row_bits)) in enumerate(zip(srcs, outs)):
        n_rows, row_bytes = _rows(src)
        _need_cuda(flags, "flags")
        if row_bits is not None:
            _need_cuda(row_bits, "row_bits")
        arr[k] = ibp_compress_tensor(n_rows, row_bytes, _dptr(src), _dptr(slots),
                                     flags.data_ptr(),
                                     row_bits.data_ptr() if row_bits is not None else None)
    return arr


def ibp_compress_batch(md: ibp_metadata, srcs, outs=None, stream=None):
    """Compress several tensors sharing `md` (one launch per row length and 16
    tensors where the library batches them): srcs is a list of tables; outs
    (optional) the matching (slots, flags, row_bits) buffers.  Returns outs."""
    srcs = list(srcs)
    if outs is None:
        outs = []
        for src in srcs:
            n_rows, row_bytes = _rows(src)
            dev = src.device if src.is_cuda else torch.device("cuda")
            outs.append((torch.empty((n_rows, row_bytes), dtype=torch.uint8, device=dev),
                         torch.empty(max(1, ibp_flag_words(n_rows)), dtype=torch.int64, device=dev),
                         torch.empty(max(1, n_rows), dtype=torch.int32, device=dev)))
    if len(outs) != len(srcs):
        raise ValueError("one output per table")
    arr = _compress_batch_args(srcs, outs)
    _check("ibp_compress_batch",
           lib().ibp_compress_batch(ctypes.byref(md), arr, len(srcs), _stream(stream)))
    return outs


def ibp_compress_batch_launcher(md: ibp_metadata, srcs, outs, stream=None):
    """ibp_compress_batch with its arguments converted once."""
    srcs, outs = list(srcs), list(outs)
    if len(outs) != len(srcs):
        raise ValueError("one output per table")
    arr = _compress_batch_args(srcs, outs)
    fn = lib().ibp_compress_batch
    args = (ctypes.byref(md), arr, ctypes.c_uint64(len(srcs)), ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_compress_batch", rc)
    launch.keep = (arr, srcs, outs)
    return launch


def ibp_decompress(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                   out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Restore every row; `out` defaults to uint8 [n_rows, row_bytes] on the GPU."""
    n_rows, row_bytes = _rows(slots)
    if out is None:
        out = torch.empty((n_rows, row_bytes), dtype=torch.uint8, device="cuda")
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    _check("ibp_decompress",
           lib().ibp_decompress(ctypes.byref(md), n_rows, row_bytes, _dptr(slots),
                                flags.data_ptr(), out.data_ptr(), _stream(stream)))
    return out


def _batch_args(images, outs):
    arr = (ibp_tensor * max(1, len(images)))()
    for k, ((slots, flags), out) in enumerate(zip(images, outs)):
        n_rows, row_bytes = _rows(slots)
        _need_cuda(flags, "flags")
        _need_cuda(out, "out")
        _need_size(out, n_rows * row_bytes, "out")
        arr[k] = ibp_tensor(n_rows, row_bytes, _dptr(slots), flags.data_ptr(), out.data_ptr())
    return arr


def ibp_decompress_batch(md: ibp_metadata, images, outs=None, stream=None):
    """Restore several tensors sharing `md` in one launch: images is a list of
    (slots, flags); outs (optional) the matching uint8 [n_rows, row_bytes]
    outputs.  Returns the outputs."""
    images = list(images)
    if outs is None:
        outs = [torch.empty(_rows(sl), dtype=torch.uint8, device="cuda") for sl, _ in images]
    if len(outs) != len(images):
        raise ValueError("one output per image")
    arr = _batch_args(images, outs)
    _check("ibp_decompress_batch",
           lib().ibp_decompress_batch(ctypes.byref(md), arr, len(images), _stream(stream)))
    return outs


def ibp_decompress_batch_launcher(md: ibp_metadata, images, outs, stream=None):
    """ibp_decompress_batch with its arguments converted once."""
    images = list(images)
    arr = _batch_args(images, outs)
    fn = lib().ibp_decompress_batch
    args = (ctypes.byref(md), arr, ctypes.c_uint64(len(images)), ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_decompress_batch", rc)
    launch.keep = (arr, images, outs)
    return launch


def ibp_gather_decompress(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                          row_ids: torch.Tensor, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """out[i] = restored row row_ids[i] (row_ids: int64 on the GPU)."""
    n_rows, row_bytes = _rows(slots)
    if row_ids.dtype != torch.int64 or not row_ids.is_cuda:
        raise ValueError("row_ids must be an int64 GPU tensor")
    n_ids = row_ids.numel()
    if out is None:
        out = torch.empty((n_ids, row_bytes), dtype=torch.uint8, device="cuda")
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    _check("ibp_gather_decompress",
           lib().ibp_gather_decompress(ctypes.byref(md), n_rows, row_bytes, _dptr(slots),
                                       flags.data_ptr(), row_ids.data_ptr(), n_ids,
                                       out.data_ptr(), _stream(stream)))
    return out


def ibp_gather_decompress_launcher(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                                   row_ids: torch.Tensor, out: torch.Tensor, stream=None):
    """ibp_gather_decompress with every argument converted once: returns a
    no-argument callable that enqueues the same call again (for loops that
    launch the same gather many times).  The tensors must stay alive."""
    n_rows, row_bytes = _rows(slots)
    if row_ids.dtype != torch.int64 or not row_ids.is_cuda:
        raise ValueError("row_ids must be an int64 GPU tensor")
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    fn = lib().ibp_gather_decompress
    args = (ctypes.byref(md), ctypes.c_uint64(n_rows), ctypes.c_uint64(row_bytes),
            ctypes.c_void_p(_dptr(slots)), ctypes.c_void_p(flags.data_ptr()),
            ctypes.c_void_p(row_ids.data_ptr()), ctypes.c_uint64(row_ids.numel()),
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_gather_decompress", rc)
    return launch


def ibp_decompress_launcher(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                            out: torch.Tensor, stream=None):
    """ibp_decompress with its arguments converted once (see above)."""
    n_rows, row_bytes = _rows(slots)
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    fn = lib().ibp_decompress
    args = (ctypes.byref(md), ctypes.c_uint64(n_rows), ctypes.c_uint64(row_bytes),
            ctypes.c_void_p(_dptr(slots)), ctypes.c_void_p(flags.data_ptr()),
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_decompress", rc)
    return launch


def _ids(row_ids: torch.Tensor) -> torch.Tensor:
    if row_ids.dtype != torch.int64 or not row_ids.is_cuda or not row_ids.is_contiguous():
        raise ValueError("row_ids must be a contiguous int64 GPU tensor")
    return row_ids


def _need_size(t: torch.Tensor, nbytes: int, name: str):
    if t.numel() * t.element_size() < nbytes or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous and hold at least {nbytes} bytes")


def ibp_cache_plan(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                   row_ids: torch.Tensor, entry_loc: torch.Tensor | None = None,
                   stream=None):
    """Plan a packed cache of rows row_ids of the image (slots, flags).
    Returns (entry_loc int64 [n_ids] on the GPU, arena_bytes).  Synchronous."""
    n_rows, row_bytes = _rows(slots)
    _ids(row_ids)
    _need_cuda(flags, "flags")
    _need_size(flags, 8 * ibp_flag_words(n_rows), "flags")
    n_ids = row_ids.numel()
    if entry_loc is None:
        entry_loc = torch.empty(max(1, n_ids), dtype=torch.int64, device=row_ids.device)
    _need_cuda(entry_loc, "entry_loc")
    _need_size(entry_loc, 8 * n_ids, "entry_loc")
    total = ctypes.c_uint64()
    _check("ibp_cache_plan",
           lib().ibp_cache_plan(ctypes.byref(md), n_rows, row_bytes, _dptr(slots),
                                flags.data_ptr(), row_ids.data_ptr(), n_ids,
                                entry_loc.data_ptr(), ctypes.byref(total), _stream(stream)))
    return entry_loc, int(total.value)


def ibp_cache_fill(md: ibp_metadata, slots: torch.Tensor, flags: torch.Tensor,
                   row_ids: torch.Tensor, entry_loc: torch.Tensor, arena_bytes: int,
                   arena: torch.Tensor | None = None, cache_loc: torch.Tensor | None = None,
                   stream=None):
    """Fill the planned arena and the table's locators.  Returns
    (arena uint8 [arena_bytes] on the GPU, cache_loc int64 [n_rows])."""
    n_rows, row_bytes = _rows(slots)
    _ids(row_ids)
    _need_cuda(flags, "flags")
    _need_size(flags, 8 * ibp_flag_words(n_rows), "flags")
    n_ids = row_ids.numel()
    _need_cuda(entry_loc, "entry_loc")
    _need_size(entry_loc, 8 * n_ids, "entry_loc")
    if arena is None:
        arena = torch.empty(max(16, arena_bytes), dtype=torch.uint8, device=row_ids.device)
    if cache_loc is None:
        cache_loc = torch.empty(max(1, n_rows), dtype=torch.int64, device=row_ids.device)
    _need_cuda(arena, "arena")
    _need_size(arena, arena_bytes, "arena")
    _need_cuda(cache_loc, "cache_loc")
    _need_size(cache_loc, 8 * n_rows, "cache_loc")
    _check("ibp_cache_fill",
           lib().ibp_cache_fill(ctypes.byref(md), n_rows, row_bytes, _dptr(slots),
                                flags.data_ptr(), row_ids.data_ptr(), n_ids,
                                entry_loc.data_ptr(), arena.data_ptr(), arena_bytes,
                                cache_loc.data_ptr(), _stream(stream)))
    return arena, cache_loc


def ibp_gather_decompress_cached(md: ibp_metadata, arena: torch.Tensor,
                                 cache_loc: torch.Tensor, slots: torch.Tensor,
                                 flags: torch.Tensor, row_ids: torch.Tensor,
                                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[i] = restored row row_ids[i], from the arena for cached rows, else
    from the image (slots on the GPU or pinned host)."""
    return ibp_gather_decompress_cached_launcher(md, arena, cache_loc, slots, flags, row_ids,
                                                 out, stream, _run=True)


def ibp_gather_decompress_cached_launcher(md: ibp_metadata, arena: torch.Tensor,
                                          cache_loc: torch.Tensor, slots: torch.Tensor,
                                          flags: torch.Tensor, row_ids: torch.Tensor,
                                          out: torch.Tensor | None = None, stream=None,
                                          _run: bool = False):
    """ibp_gather_decompress_cached with its arguments converted once: returns
    a no-argument callable that enqueues the call (or, internally, the output
    after one call)."""
    n_rows, row_bytes = _rows(slots)
    _ids(row_ids)
    for t, name in ((flags, "flags"), (arena, "arena"), (cache_loc, "cache_loc")):
        _need_cuda(t, name)
    _need_size(flags, 8 * ibp_flag_words(n_rows), "flags")
    _need_size(cache_loc, 8 * n_rows, "cache_loc")
    n_ids = row_ids.numel()
    if out is None:
        out = torch.empty((n_ids, row_bytes), dtype=torch.uint8, device=row_ids.device)
    _need_cuda(out, "out")
    _need_size(out, n_ids * row_bytes, "out")
    fn = lib().ibp_gather_decompress_cached
    args = (ctypes.byref(md), ctypes.c_uint64(n_rows), ctypes.c_uint64(row_bytes),
            ctypes.c_void_p(arena.data_ptr()), ctypes.c_void_p(cache_loc.data_ptr()),
            ctypes.c_void_p(_dptr(slots)), ctypes.c_void_p(flags.data_ptr()),
            ctypes.c_void_p(row_ids.data_ptr()), ctypes.c_uint64(n_ids),
            ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_gather_decompress_cached", rc)
    if _run:
        launch()
        return out
    return launch



# ---------------------------------------------------- per-position metadata --

def ibp_positional_table_bytes(n_positions: int) -> int:
    return int(lib().ibp_positional_table_bytes(n_positions))


def ibp_positional_table(mask, bitval) -> torch.Tensor:
    """Position table (host uint8 tensor) from per-position mask/bitval
    sequences of 32-bit values; move it to the GPU before use."""
    import numpy as np
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint64).astype(np.uint32))
    b = np.ascontiguousarray(np.asarray(bitval, dtype=np.uint64).astype(np.uint32))
    if m.shape != b.shape or m.ndim != 1:
        raise ValueError("mask and bitval must be 1-D of equal length")
    out = torch.zeros(max(16, ibp_positional_table_bytes(m.size)), dtype=torch.uint8)
    _check("ibp_positional_table",
           lib().ibp_positional_table(m.ctypes.data, b.ctypes.data, m.size, out.data_ptr()))
    return out


def ibp_build_metadata_positional(sample: torch.Tensor, t: float = 0.9,
                                  n_sample_rows: int | None = None,
                                  t_ppm: int | None = None, stream=None):
    """Per-position metadata over the rows of `sample` (first axis = rows; GPU
    or pinned host).  Returns (table uint8 on the GPU, mask, bitval) with
    mask/bitval numpy uint32 arrays.  Synchronous."""
    import numpy as np
    n_rows, row_bytes = _rows(sample)
    if n_sample_rows is None:
        n_sample_rows = n_rows
    if not 0 <= n_sample_rows <= n_rows:
        raise ValueError(f"n_sample_rows={n_sample_rows} but the sample holds {n_rows} rows")
    n = row_bytes // 4
    ppm = int(round(t * 1_000_000)) if t_ppm is None else int(t_ppm)
    table = torch.empty(max(16, ibp_positional_table_bytes(n)), dtype=torch.uint8,
                        device="cuda")
    mask = np.zeros(n, np.uint32)
    bitval = np.zeros(n, np.uint32)
    _check("ibp_build_metadata_positional",
           lib().ibp_build_metadata_positional(_dptr(sample), n_sample_rows, row_bytes, ppm,
                                               table.data_ptr(), mask.ctypes.data,
                                               bitval.ctypes.data, _stream(stream)))
    return table, mask, bitval


def _need_table(table: torch.Tensor, row_bytes: int):
    _need_cuda(table, "table")
    _need_size(table, ibp_positional_table_bytes(row_bytes // 4), "table")
    if table.data_ptr() % 16:
        raise ValueError("table must be 16-byte aligned")


def ibp_compress_positional(table: torch.Tensor, src: torch.Tensor,
                            slots: torch.Tensor | None = None,
                            flags: torch.Tensor | None = None,
                            row_bits: torch.Tensor | None = None,
                            want_row_bits: bool = True, stream=None):
    """ibp_compress with a position table.  Returns (slots, flags, row_bits)."""
    n_rows, row_bytes = _rows(src)
    _need_table(table, row_bytes)
    dev = src.device if src.is_cuda else torch.device("cuda")
    if slots is None:
        slots = torch.empty((n_rows, row_bytes), dtype=torch.uint8, device=dev)
    if flags is None:
        flags = torch.empty(max(1, ibp_flag_words(n_rows)), dtype=torch.int64, device=dev)
    if row_bits is None and want_row_bits:
        row_bits = torch.empty(max(1, n_rows), dtype=torch.int32, device=dev)
    _need_cuda(flags, "flags")
    _need_size(flags, 8 * ibp_flag_words(n_rows), "flags")
    if row_bits is not None:
        _need_cuda(row_bits, "row_bits")
        _need_size(row_bits, 4 * n_rows, "row_bits")
    _need_size(slots, n_rows * row_bytes, "slots")
    _check("ibp_compress_positional",
           lib().ibp_compress_positional(table.data_ptr(), n_rows, row_bytes, _dptr(src),
                                         _dptr(slots), flags.data_ptr(),
                                         row_bits.data_ptr() if row_bits is not None else None,
                                         _stream(stream)))
    return slots, flags, row_bits


def ibp_decompress_positional(table: torch.Tensor, slots: torch.Tensor, flags: torch.Tensor,
                              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    n_rows, row_bytes = _rows(slots)
    _need_table(table, row_bytes)
    if out is None:
        out = torch.empty((n_rows, row_bytes), dtype=torch.uint8, device="cuda")
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    _need_size(out, n_rows * row_bytes, "out")
    _check("ibp_decompress_positional",
           lib().ibp_decompress_positional(table.data_ptr(), n_rows, row_bytes, _dptr(slots),
                                           flags.data_ptr(), out.data_ptr(), _stream(stream)))
    return out


def ibp_gather_decompress_positional_launcher(table: torch.Tensor, slots: torch.Tensor,
                                              flags: torch.Tensor, row_ids: torch.Tensor,
                                              out: torch.Tensor, stream=None):
    """ibp_gather_decompress_positional with its arguments converted once."""
    n_rows, row_bytes = _rows(slots)
    _need_table(table, row_bytes)
    _ids(row_ids)
    _need_cuda(flags, "flags")
    _need_cuda(out, "out")
    _need_size(out, row_ids.numel() * row_bytes, "out")
    fn = lib().ibp_gather_decompress_positional
    args = (ctypes.c_void_p(table.data_ptr()), ctypes.c_uint64(n_rows),
            ctypes.c_uint64(row_bytes), ctypes.c_void_p(_dptr(slots)),
            ctypes.c_void_p(flags.data_ptr()), ctypes.c_void_p(row_ids.data_ptr()),
            ctypes.c_uint64(row_ids.numel()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(_stream(stream)))

    def launch():
        rc = fn(*args)
        if rc:
            raise IBPError("ibp_gather_decompress_positional", rc)
    return launch


def ibp_gather_decompress_positional(table: torch.Tensor, slots: torch.Tensor,
                                     flags: torch.Tensor, row_ids: torch.Tensor,
                                     out: torch.Tensor | None = None,
                                     stream=None) -> torch.Tensor:
    n_rows, row_bytes = _rows(slots)
    if out is None:
        out = torch.empty((row_ids.numel(), row_bytes), dtype=torch.uint8, device="cuda")
    ibp_gather_decompress_positional_launcher(table, slots, flags, row_ids, out, stream)()
    return out
