"""ctypes binding of libibp_ceiling (include/ibp_ceiling.h): the gather-copy
floor the benchmark times beside each decompression, and a plain contiguous
copy.  Argument marshalling
only; raises if the library has not been built."""
from __future__ import annotations

import ctypes
import os

import torch

from . import ibp

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libibp_ceiling.so")
IBP_CEILING_MAX_TENSORS = 16
IBP_CEILING_PACK = 1
IBP_CEILING_STREAM_LOADS = 2


class ibp_copy_tensor(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_uint64),
                ("row_bytes", ctypes.c_uint64),
                ("src", ctypes.c_void_p),
                ("src_bytes", ctypes.c_void_p),
                ("ids", ctypes.c_void_p),
                ("n_out", ctypes.c_uint64),
                ("dst", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m lossless_bit_level_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.ibp_ceiling_gather_copy.argtypes = [ctypes.POINTER(ibp_copy_tensor), ctypes.c_uint64,
                                              ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p]
        L.ibp_ceiling_gather_copy.restype = ctypes.c_int
        L.ibp_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_uint32, ctypes.c_void_p]
        L.ibp_ceiling_copy.restype = ctypes.c_int
        _lib = L
    return _lib


def gather_copy_launcher(parts, max_workgroups: int = 0, pack: bool = False,
                         stream_loads: bool = False, stream=None):
    """parts: list of (slots, src_bytes, ids or None, out) with slots a
    [n_rows, S] uint8 tensor (GPU or pinned host), src_bytes an int32 GPU
    tensor of the n_out stored lengths of the output rows' source rows, ids
    an int64 GPU tensor and out a GPU tensor of n_out x S bytes;
    max_workgroups caps the grid (0: none); pack puts several short rows in
    one 4 KiB task; stream_loads makes the slot loads non-temporal.
    Returns a no-argument callable that enqueues the copy (one launch) on
    the current stream."""
    if not 0 < len(parts) <= IBP_CEILING_MAX_TENSORS:
        raise ValueError("1 to 16 tensors per copy")
    arr = (ibp_copy_tensor * len(parts))()
    for k, (slots, src_bytes, ids, out) in enumerate(parts):
        n_rows, row_bytes = ibp._rows(slots)
        if ids is not None:
            ibp._ids(ids)
        n_out = ids.numel() if ids is not None else n_rows
        if src_bytes.dtype != torch.int32 or not src_bytes.is_cuda or src_bytes.numel() < n_out:
            raise ValueError("src_bytes must be an int32 GPU tensor of n_out entries")
        ibp._need_cuda(out, "out")
        ibp._need_size(out, n_out * row_bytes, "out")
        arr[k] = ibp_copy_tensor(n_rows, row_bytes, ibp._dptr(slots), src_bytes.data_ptr(),
                                 ids.data_ptr() if ids is not None else None, n_out,
                                 out.data_ptr())
    fn = lib().ibp_ceiling_gather_copy
    s = ctypes.c_void_p((torch.cuda.current_stream() if stream is None else stream).cuda_stream)
    n = ctypes.c_uint64(len(parts))
    cap = ctypes.c_uint32(max_workgroups)
    pk = ctypes.c_uint32((IBP_CEILING_PACK if pack else 0) |
                         (IBP_CEILING_STREAM_LOADS if stream_loads else 0))

    def launch():
        rc = fn(arr, n, cap, pk, s)
        if rc:
            raise RuntimeError(f"ibp_ceiling_gather_copy failed ({rc})")
    launch.keep = (arr, parts)
    return launch


def copy_launcher(src, dst, max_workgroups: int = 0, stream=None):
    """A plain contiguous copy of src into dst (GPU tensors of the same byte
    size, 16-byte aligned, a multiple of 16 bytes): workgroups stride over 16
    KiB tiles with non-temporal 16-byte loads and stores; max_workgroups caps
    the grid (0: one workgroup per tile).  Returns a no-argument callable
    that enqueues the copy (one launch) on the current stream."""
    ibp._need_cuda(src, "src")
    ibp._need_cuda(dst, "dst")
    n = src.numel() * src.element_size()
    ibp._need_size(src, n, "src")
    ibp._need_size(dst, n, "dst")
    fn = lib().ibp_ceiling_copy
    s = ctypes.c_void_p((torch.cuda.current_stream() if stream is None else stream).cuda_stream)
    a, b = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())
    nb, cap = ctypes.c_uint64(n), ctypes.c_uint32(max_workgroups)

    def launch():
        rc = fn(a, b, nb, cap, s)
        if rc:
            raise RuntimeError(f"ibp_ceiling_copy failed ({rc})")
    launch.keep = (src, dst)
    return launch
