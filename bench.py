"""Benchmark of IBP decompression on one MI355X.

Default run (python bench.py): the LLM-weight workload, 32 layers x (4 x
[4096, 4096] + 3 x [4096, 14336]) bf16 weights ~ N(0, 0.02^2), all 32
layers compressed with Invariant Bit Packing and resident in HBM (15.6 GB
raw, uploaded and compressed layer by layer).  One step = the full
decompression of one layer, its 7 matrices in one batched launch, layer
after layer (the layer-by-layer weight load of the IBP page's offloaded LLM
inference, section "Results").  Outputs rotate over >= 1 GiB.

The same line then carries, under "configs", every other workload on the
page's data kinds, each with its own kernel, launch time, fraction of the
HBM (or host-link) roofline and fraction of a measured gather-copy ceiling:
  tiny_dense   4096 x 128 fp32: compress, full decompress, round trip
  sparse_gnn   1M x 512 fp32 bag-of-words rows, 8 x 65,536 uniform ids
  dense_gnn    2M x 256 fp32 N(0, 0.5^2), 8 x 65,536 Zipf(1.05) ids
  dlrm_emb     4M x 128 fp32 U(-0.05, 0.05), 8 x 65,536 Zipf(1.05) ids
  llm_kv       [16, 32, 4096, 128] bf16 KV cache, 4 KiB pages, 8 x 16,384 ids
  llm_kv_host, llm_weights_host: the same images in pinned host memory,
               decoded across the host link (zero-copy)

Prints one JSON line:
  value        GB/s of uncompressed output over the K timed steps
  roofline     algorithmic bytes of one launch / its mean duration (HIP
               events on the launch stream) against the 8 TB/s HBM peak;
               "ceiling": the gather-copy floor of the same transfer, timed
               the same way on the same ids, images and outputs;
               "device_copy" (headline): a plain contiguous 1 GiB device-to-
               device copy, read + written bytes per second (hipMemcpy and
               two copy kernels, the best of each), the practical rate of a
               streaming read/write mix on the GPU at hand
  cpu_baseline the CPU oracle on the host cores: full decompress and
               compress of one layer on every host thread of this GPU's share,
               plus single-thread figures on the tiny table and a 256 MiB
               slice of the model
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time
from collections import deque
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IBP decompress GB/s (uncompressed out), % of HBM roofline; compression ratio"
HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "lossless_bit_level_amd", "csrc", "ibp.hip")
ROTATE_BYTES = 1 << 30           # outputs rotate over at least this much memory
CEILING_GRIDS = (2, 4, 8, 16, 64)   # workgroups per CU tried for the gather-copy ceiling
COMPRESS_GROUP_BYTES = 400 << 20  # compression timed over groups of this much raw input (a layer)
COMPRESS_SPIN_CYCLES = 1_000_000  # spin before a timed compress group (~0.5 ms of GPU clock)
GiB = float(1 << 30)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_threads():
    """(threads to use, CPUs the affinity mask allows): the affinity mask,
    capped at the share OMP_NUM_THREADS announces (a host may give one GPU
    a share of its threads smaller than the mask shows)."""
    allowed = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS") or allowed)
    return max(1, min(allowed, share)), allowed


def cu_count() -> int:
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------- workloads --

class Workload:
    """n_tables tables (rows on axis 0) produced by table(i); steps: list of
    (table index, ids or None); groups of layer_size consecutive steps may go
    in one batched launch; sample: numpy bytes for the metadata."""

    def __init__(self, name, desc, n_tables, make_table, steps, sample, layer_size=1,
                 hot=None, keep=True):
        self.name, self.desc = name, desc
        self.n_tables, self._make, self.steps = n_tables, make_table, steps
        self.sample, self.layer_size, self.hot, self.keep = sample, layer_size, hot, keep
        self._cache = {}

    def table(self, i):
        if i in self._cache:
            return self._cache[i]
        x = self._make(i)
        if self.keep:
            self._cache[i] = x
        return x

    def source_rows(self, i, rows):
        """Rows of table i as uint8 [len(rows), S]."""
        x = self.table(i)
        return x.reshape(x.shape[0], -1).view(np.uint8)[rows]


def make_workload(name: str, threads: int) -> Workload:
    import synthetic as syn
    if name == "tiny_dense":
        x = syn.tiny_dense()
        return Workload(name, "tiny dense 4096 x 128 fp32 N(0, 0.1^2), full decompress",
                        1, lambda i: x, [(0, None)], x)
    if name == "sparse_gnn":
        x = syn.sparse_gnn_rows(threads=threads)
        ids = syn.uniform_ids(syn.SPARSE_GNN_ROWS, 8, 65536)
        return Workload(name, "sparse GNN features 1048576 x 512 fp32, gather 8 x 65536 "
                        "uniform ids", 1, lambda i: x, [(0, b) for b in ids], x,
                        hot=np.arange(x.shape[0], dtype=np.int64))
    if name in ("dense_gnn", "dlrm_emb"):
        if name == "dense_gnn":
            x = syn.dense_gnn_rows(threads=threads)
            ids = syn.zipf_ids(syn.DENSE_GNN_ROWS, 8, 65536)
            desc = "dense GNN features 2097152 x 256 fp32 N(0,0.25)"
        else:
            x = syn.dlrm_emb_rows(threads=threads)
            ids = syn.zipf_ids(syn.DLRM_EMB_ROWS, 8, 65536, seed=2)
            desc = "DLRM embedding 4194304 x 128 fp32 U(-0.05,0.05)"
        return Workload(name, desc + ", gather 8 x 65536 Zipf(1.05) ids", 1, lambda i: x,
                        [(0, b) for b in ids], x, hot=syn.zipf_hot_order(x.shape[0]))
    if name == "llm_kv":
        x = syn.llm_kv_pages(threads=threads)
        ids = syn.kv_page_ids()
        return Workload(name, "LLM KV cache [16,32,4096,128] bf16, 4 KiB pages, gather "
                        "8 x 16384 page ids", 1, lambda i: x, [(0, b) for b in ids], x,
                        hot=np.arange(x.shape[0], dtype=np.int64))
    if name == "llm_weights":
        n = syn.LLM_LAYERS * syn.LLM_MATRICES
        # the first 2^24 blocks of the model in storage order: layer 0's
        # first two matrices
        sample = np.concatenate([syn.llm_weight(0, 0).reshape(-1), syn.llm_weight(0, 1).reshape(-1)])
        return Workload(name, "LLM weights bf16, 32 layers x (4 x [4096,4096] + 3 x "
                        "[4096,14336]), all resident; full decompress layer by layer (the 7 "
                        "matrices of a layer in one batched call)", n,
                        lambda i: syn.llm_weight(i // syn.LLM_MATRICES, i % syn.LLM_MATRICES),
                        [(t, None) for t in range(n)], sample, layer_size=syn.LLM_MATRICES,
                        keep=False)
    raise SystemExit(f"unknown workload {name}")


def iter_tables(wl: Workload, threads: int):
    """(index, table) in order, generated ahead on a thread pool."""
    if wl.n_tables == 1:
        yield 0, wl.table(0)
        return
    with ThreadPoolExecutor(threads) as ex:
        futs = deque()
        nxt = 0
        while nxt < wl.n_tables and len(futs) < threads:
            futs.append(ex.submit(wl.table, nxt))
            nxt += 1
        for i in range(wl.n_tables):
            x = futs.popleft().result()
            if nxt < wl.n_tables:
                futs.append(ex.submit(wl.table, nxt))
                nxt += 1
            yield i, x


# ----------------------------------------------------------- helpers ----

def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def decode_kernel_name(row_bytes: int, width: int = 32, positional: bool = False,
                       invariant_bits: int = 0, cached: bool = False,
                       host_image: bool = False, batched: bool = False) -> str:
    """The decode kernel libibp launches for rows of this size (16-byte
    aligned buffers)."""
    if positional:
        return ("decode_pos_pipe_kernel" if row_bytes in (512, 1024, 2048, 4096)
                else "decode_positional_kernel")
    if width == 64 and row_bytes in (512, 1024, 2048) and not cached:
        return "decode_pipe64_kernel"
    if width != 32:
        return "decode_wide_batch_kernel" if batched else "decode_wide_kernel"
    if batched:
        return "decode_batch_kernel"
    if host_image and invariant_bits < 32 and row_bytes >= 4096 and not cached:
        return "decode_segments_kernel"   # 256-block tasks for an image in host memory
    if row_bytes in (512, 1024, 2048) and invariant_bits < 32 and not cached:
        return "decode_pipe_kernel"
    return "decode_rows_kernel" if row_bytes <= 4096 else "decode_segments_kernel"


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, only
    if it was taken on the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def stored_bytes_per_row(row_bits: np.ndarray, row_bytes: int) -> np.ndarray:
    n = row_bytes // 4
    c = row_bits.astype(np.int64)
    comp = c < 32 * n
    return np.where(comp, 4 * ((c + 31) // 32), row_bytes)


class Opts:
    def __init__(self, source="device", width=32, positional=False, cache_mib=0,
                 per_tensor=False):
        self.source, self.width, self.positional = source, width, positional
        self.cache_mib, self.per_tensor = cache_mib, per_tensor


def time_region(stream, launch, K):
    """(wall seconds, event seconds) of K launches back to back, bracketed by
    a synchronize on both sides and by HIP events on the launch stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(K):
        launch(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3


def link_ceiling(dev, stream):
    """Host-link ceiling, 1 GiB from pinned host memory to the device: the
    better of hipMemcpyAsync and a zero-copy streaming read kernel (the
    gather-copy kernel of libibp_ceiling reading the pinned buffer as 4 KiB
    rows in order; the best of a few grids and both load policies).  Returns
    (GB/s, record)."""
    import torch
    from lossless_bit_level_amd import ceiling
    n = 1 << 30
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    h.view(torch.int64).fill_(0x0123456789ABCDEF)
    d = torch.empty(n, dtype=torch.uint8, device=dev)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    memcpy = n / timed(lambda: d.copy_(h, non_blocking=True)) / 1e9
    rows = h.view(n // 4096, 4096)
    lens = torch.full((n // 4096,), 4096, dtype=torch.int32, device=dev)
    best = None
    for per_cu in (4, 16, 64):
        for nt in (False, True):
            fn = ceiling.gather_copy_launcher([(rows, lens, None, d)],
                                              max_workgroups=per_cu * cu_count(),
                                              stream_loads=nt)
            t = timed(fn)
            if best is None or t < best[0]:
                best = (t, per_cu, nt)
    if not torch.equal(d[:1 << 20].cpu(), h[:1 << 20]):
        raise SystemExit("bench: the zero-copy read differs from its source")
    zero_copy = n / best[0] / 1e9
    del h, d, rows, lens
    rate = max(memcpy, zero_copy)
    return rate, {"hipMemcpy_GB_per_s": round(memcpy, 2),
                  "zero_copy_read_GB_per_s": round(zero_copy, 2),
                  "zero_copy_kernel": {"kernel": "gather_copy_kernel", "workgroups_per_cu": best[1],
                                       "loads": "non-temporal" if best[2] else "default"},
                  "ceiling_GB_per_s": round(rate, 2),
                  "what": "1 GiB pinned host -> device; the ceiling is the better of the two"}


def device_copy_reference(dev, stream, reps: int = 5):
    """Read + write bytes per second of a plain contiguous 1 GiB device-to-
    device copy, the practical rate of a streaming read/write mix on this
    GPU: torch's copy_ (hipMemcpyAsync), the tile copy of libibp_ceiling
    (16 KiB tiles, non-temporal 16-byte loads and stores; the best of a few
    grids) and its gather-copy kernel on the same buffers as 4 KiB rows in
    order (no ids; the best of a few grids and both load policies).  Context
    for the headline's roofline fraction, which is against the nominal 8
    TB/s."""
    import torch
    from lossless_bit_level_amd import ceiling
    n = 1 << 30
    a = torch.randint(0, 255, (n,), dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    def check(what):
        if not torch.equal(a, b):
            raise SystemExit(f"bench: the reference copy ({what}) differs from its source")
        b.zero_()

    t_memcpy = timed(lambda: b.copy_(a))
    check("hipMemcpy")
    tile = None
    for per_cu in (16, 32, 64):
        t = timed(ceiling.copy_launcher(a, b, max_workgroups=per_cu * cu_count()))
        if tile is None or t < tile[0]:
            tile = (t, per_cu)
    check("tile copy")
    rows = a.view(n // 4096, 4096)
    lens = torch.full((n // 4096,), 4096, dtype=torch.int32, device=dev)
    best = None
    for per_cu in (8, 16, 64):
        for nt in (False, True):
            fn = ceiling.gather_copy_launcher([(rows, lens, None, b)],
                                              max_workgroups=per_cu * cu_count(),
                                              stream_loads=nt)
            t = timed(fn)
            if best is None or t < best[0]:
                best = (t, per_cu, nt)
    check("gather copy")
    del a, b, rows, lens
    r_memcpy = 2 * n / t_memcpy / 1e9
    r_tile = 2 * n / tile[0] / 1e9
    r_kernel = 2 * n / best[0] / 1e9
    return {"what": "contiguous 1 GiB device-to-device copy, read + written bytes per second",
            "hipMemcpy_GB_per_s": round(r_memcpy, 1),
            "tile_copy_GB_per_s": round(r_tile, 1),
            "tile_copy": {"kernel": "tile_copy_kernel", "workgroups_per_cu": tile[1]},
            "copy_kernel_GB_per_s": round(r_kernel, 1),
            "copy_kernel": {"kernel": "gather_copy_kernel", "workgroups_per_cu": best[1],
                            "loads": "non-temporal" if best[2] else "default"},
            "best_GB_per_s": round(max(r_memcpy, r_tile, r_kernel), 1),
            "best_frac_of_peak": round(max(r_memcpy, r_tile, r_kernel) / HBM_PEAK_GBPS, 4)}


# ------------------------------------------------------------- measure ----

def measure(wl: Workload, opt: Opts, sources, K: int, W: int, threads: int, dev,
            link_rate=None):
    """Metadata, compression and timed decompression of one workload, from
    each image location in `sources` ("device", "host").  Returns
    {source: result dict}."""
    import torch
    from lossless_bit_level_amd import ibp
    from lossless_bit_level_amd import ceiling
    stream = torch.cuda.current_stream()
    width = opt.width

    # metadata over the first min(N, 2^24) blocks, timed apart
    samp = torch.from_numpy(np.ascontiguousarray(wl.sample).reshape(-1).view(np.uint8)).to(dev)
    n_blocks = min(samp.numel() * 8 // width, 1 << 24)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    md, _ = ibp.ibp_build_metadata(samp, n_blocks=n_blocks, width_bits=width)
    meta_first_ms = (time.perf_counter() - t0) * 1e3   # includes first-use setup
    t0 = time.perf_counter()
    md, _ = ibp.ibp_build_metadata(samp, n_blocks=n_blocks, width_bits=width)
    meta_ms = (time.perf_counter() - t0) * 1e3
    del samp
    pos_table = pmask = pbitval = None
    if opt.positional:
        if width != 32 or opt.cache_mib:
            raise SystemExit("--positional runs with W = 32 and without --cache-mib")
        x0 = wl.table(0)
        S0 = x0.nbytes // x0.shape[0]
        s_rows = max(1, min(x0.shape[0], (1 << 24) // (S0 // 4)))
        samp = torch.from_numpy(x0[:s_rows].reshape(s_rows, -1).view(np.uint8)).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pos_table, pmask, pbitval = ibp.ibp_build_metadata_positional(samp)
        meta_ms = (time.perf_counter() - t0) * 1e3
        del samp
        log(f"positional metadata over {s_rows} rows in {meta_ms:.1f} ms; "
            f"{len(set(pmask.tolist()))} distinct masks")

    def compress(tg, out=(None, None, None)):
        slots, flags, rb = out
        if pos_table is not None:
            return ibp.ibp_compress_positional(pos_table, tg, slots=slots, flags=flags,
                                               row_bits=rb)
        return ibp.ibp_compress(md, tg, slots=slots, flags=flags, row_bits=rb)

    def time_compress(groups, batch=False, reps=1):
        """GPU seconds of compressing the staged tables again into their
        outputs: each group (a list of (staged table, outputs)) with one
        ibp_compress_batch, or table by table, back to back on the stream,
        reps times.  The calls' arguments are converted first, and a spin
        kernel runs before the region, so that the calls are queued before it
        starts and the host's own per-call work is not timed (the GPU time of
        a pipeline of such calls).  No table generator runs meanwhile."""
        if batch:
            calls = [ibp.ibp_compress_batch_launcher(md, [tg for tg, _ in g], [o for _, o in g])
                     for g in groups]
        else:
            calls = [(lambda tg=tg, o=o: compress(tg, o)) for g in groups for tg, o in g]
        torch.cuda.synchronize()
        torch.cuda._sleep(COMPRESS_SPIN_CYCLES)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for call in calls:
                call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    # upload and compress every table (out of place from a staging upload),
    # keeping the staged tables; then, with no table generator running, time
    # their compression again into the same buffers: the tables of a layer
    # (up to COMPRESS_GROUP_BYTES of raw input) in one batched call, layer
    # after layer, or a one-table workload three times back to back
    images = []          # (slots, flags, stored bytes per row numpy, stored bytes int32 GPU)
    shapes = []
    raw_bytes = stored = bits_total = side_bytes = 0
    t_up = time.perf_counter()
    groups, group_bytes = [[]], 0
    for i, x in iter_tables(wl, threads):
        tg = torch.from_numpy(x.reshape(x.shape[0], -1).view(np.uint8)).to(dev)
        shapes.append(tuple(tg.shape))
        out = compress(tg)
        slots, flags, rb = out
        groups[-1].append((tg, out))
        group_bytes += tg.numel()
        if group_bytes >= COMPRESS_GROUP_BYTES and i < wl.n_tables - 1:
            groups.append([])
            group_bytes = 0
        del tg
        rbn = rb.cpu().numpy()[:shapes[-1][0]]
        sb = stored_bytes_per_row(rbn, shapes[-1][1])
        images.append((slots, flags, sb, torch.from_numpy(sb.astype(np.int32)).to(dev)))
        raw_bytes += shapes[-1][0] * shapes[-1][1]
        stored += int(sb.sum())
        side_bytes += 8 * ((shapes[-1][0] + 63) // 64)
        bits_total += int(np.minimum(rbn.astype(np.int64), 8 * shapes[-1][1]).sum())
    # a layer's tables in one ibp_compress_batch (global metadata)
    comp_s = time_compress(groups, batch=wl.n_tables > 1 and pos_table is None,
                           reps=3 if wl.n_tables == 1 else 1)
    del groups
    log(f"{wl.name}: {len(images)} tables uploaded and compressed in "
        f"{time.perf_counter() - t_up:.1f} s; {md}; compress {comp_s * 1e3:.2f} ms "
        f"({raw_bytes / comp_s / 1e9:.0f} GB/s); ratio {raw_bytes / stored:.4f}")
    compress_rec = {"ms": round(comp_s * 1e3, 3), "GB_per_s_raw_in": round(raw_bytes / comp_s / 1e9, 1),
                    # raw bytes read plus stored bytes written, against the HBM peak
                    "frac": round((raw_bytes + stored) / comp_s / 1e9 / HBM_PEAK_GBPS, 4),
                    "timed": ("one table, three calls back to back" if wl.n_tables == 1 else
                              "each layer's tables in one batched call"
                              if pos_table is None else "each layer's tables back to back") +
                             ", after a spin kernel; HIP events"}
    common = {
        "desc": wl.desc,
        "compression_ratio": round(raw_bytes / stored, 4),
        "compression_ratio_bits": round(raw_bytes * 8 / bits_total, 4),
        # with the flag words and the metadata (32 bytes, or the position table)
        "compression_ratio_with_side_data": round(raw_bytes / (stored + side_bytes + (
            pos_table.numel() if pos_table is not None else 32)), 4),
        "metadata": {"mask": f"0x{md.mask:0{width // 4}X}",
                     "bitval": f"0x{md.bitval:0{width // 4}X}",
                     "invariant_bits": md.invariant_bits, "build_ms": round(meta_ms, 3),
                     "first_call_ms": round(meta_first_ms, 3)},
        "compress": compress_rec,
    }

    results = {}
    for source in sources:
        host = source == "host"
        if host:
            # [IBP] System integration: host tensors compressed in place, each
            # row in its own fixed-size buffer, by the GPU over the host link
            t_ip = 0.0
            raw_ip = 0
            n_ip = min(wl.n_tables, wl.layer_size)
            with ThreadPoolExecutor(threads) as ex:
                first = list(ex.map(wl.table, range(n_ip)))
            for x in first:
                h = torch.from_numpy(x.reshape(x.shape[0], -1).view(np.uint8)).pin_memory()

                def in_place():
                    if pos_table is not None:
                        ibp.ibp_compress_positional(pos_table, h, slots=h, want_row_bits=False)
                    else:
                        ibp.ibp_compress(md, h, slots=h, want_row_bits=False)
                in_place()
                torch.cuda.synchronize()
                h.copy_(torch.from_numpy(x.reshape(x.shape[0], -1).view(np.uint8)))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                in_place()
                e1.record(stream)
                torch.cuda.synchronize()
                t_ip += e0.elapsed_time(e1) / 1e3
                raw_ip += h.numel()
                del h
            del first
            inplace = {"tables": n_ip, "ms": round(t_ip * 1e3, 3),
                       "GB_per_s_raw": round(raw_ip / t_ip / 1e9, 2)}
            log(f"in-place compression of {inplace['tables']} pinned host table(s): "
                f"{t_ip * 1e3:.2f} ms ({raw_ip / t_ip / 1e9:.1f} GB/s raw)")
            imgs = []
            for slots, flags, sb, sbg in images:
                hs = torch.empty(slots.shape, dtype=torch.uint8, pin_memory=True)
                hs.copy_(slots)
                imgs.append((hs, flags, sb, sbg))
            torch.cuda.synchronize()
        else:
            inplace = None
            imgs = images
        results[source] = measure_decode(wl, opt, imgs, shapes, md, pos_table, K, W, dev,
                                         stream, host, link_rate)
        results[source].update(common)
        if inplace is not None:
            results[source]["compress"] = dict(compress_rec, in_place_pinned_host=inplace)
        if host:
            del imgs
            torch.cuda.synchronize()
    return results


def measure_decode(wl, opt, images, shapes, md, pos_table, K, W, dev, stream, host, link_rate):
    import torch
    from lossless_bit_level_amd import ibp
    from lossless_bit_level_amd import ceiling

    # [IBP] System integration, cache compression: the most popular rows that
    # fit the budget, in their stored form, packed into a GPU arena
    cache = None
    resident = None
    arena = cache_loc = None
    if opt.cache_mib:
        if wl.n_tables != 1 or wl.hot is None or any(ids is None for _, ids in wl.steps):
            raise SystemExit("--cache-mib needs a gather workload over one table")
        slots, flags, sb, _ = images[0]
        n_rows, S = shapes[0]
        budget = opt.cache_mib << 20
        k = int(np.searchsorted(np.cumsum((sb[wl.hot] + 15) // 16 * 16), budget, side="right"))
        cached = torch.from_numpy(wl.hot[:k].copy()).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        entry_loc, arena_bytes = ibp.ibp_cache_plan(md, slots, flags, cached)
        plan_ms = (time.perf_counter() - t0) * 1e3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        arena = torch.empty(max(16, arena_bytes), dtype=torch.uint8, device=dev)
        cache_loc = torch.empty(n_rows, dtype=torch.int64, device=dev)
        e0.record(stream)
        ibp.ibp_cache_fill(md, slots, flags, cached, entry_loc, arena_bytes, arena=arena,
                           cache_loc=cache_loc)
        e1.record(stream)
        torch.cuda.synchronize()
        del entry_loc
        resident = np.zeros(n_rows, bool)
        resident[wl.hot[:k]] = True
        all_ids = np.concatenate([ids for _, ids in wl.steps])
        counts = np.bincount(all_ids, minlength=n_rows)
        raw_rows = min(n_rows, budget // S)
        cache = {"budget_mib": opt.cache_mib, "rows": k, "rows_fraction": round(k / n_rows, 4),
                 "arena_mib": round(arena_bytes / 2**20, 2),
                 "hit_rate": round(float(resident[all_ids].mean()), 4),
                 "raw_cache_rows": int(raw_rows),
                 "raw_cache_hit_rate": round(float(counts[wl.hot[:raw_rows]].sum() /
                                                   counts.sum()), 4),
                 "plan_ms": round(plan_ms, 3), "fill_ms": round(e0.elapsed_time(e1), 3)}
        log(f"cache: {cache}")

    # step groups: the weight matrices of a layer are one step (layer-by-layer
    # loading), from a device image in one batched launch; from a host image
    # one launch per matrix (its rows are cut into the small tasks that suit
    # the host link).  Every other step is one launch.
    steps = wl.steps
    layered = wl.layer_size > 1 and not opt.per_tensor
    batched = layered and not host and pos_table is None and not opt.cache_mib
    if layered:
        groups = [list(range(g, min(g + wl.layer_size, len(steps))))
                  for g in range(0, len(steps), wl.layer_size)]
    else:
        groups = [[k] for k in range(len(steps))]
    ids_g = [torch.from_numpy(np.ascontiguousarray(ids)).to(dev) if ids is not None else None
             for _, ids in steps]

    def out_shape(k):
        ti, ids = steps[k]
        n_rows, S = shapes[ti]
        return (len(ids) if ids is not None else n_rows, S)

    group_shapes = [[out_shape(k) for k in g] for g in groups]
    group_out = [sum(a * b for a, b in gs) for gs in group_shapes]
    # output sets: every group of a workload has the same shapes here; enough
    # sets that the outputs rotate over >= 1 GiB
    n_sets = max(1, math.ceil(ROTATE_BYTES / min(group_out)))
    max_shapes = group_shapes[int(np.argmax(group_out))]
    out_sets = [[torch.empty(s, dtype=torch.uint8, device=dev) for s in max_shapes]
                for _ in range(n_sets)]

    def algo_bytes(k):
        """(bytes the launch must move, duplicates counted; bytes of it read
        from the image; bytes of distinct image rows, which is what must cross
        the host link when the image is in host memory: a repeated row is
        served from the GPU's caches)."""
        ti, ids = steps[k]
        sb = images[ti][2]
        n_rows, S = shapes[ti]
        if ids is None:
            img = int(sb.sum())
            return img + n_rows * S + 8 * ((n_rows + 63) // 64), img, img
        if resident is None:
            img = int(sb[ids].sum())
            return (img + len(ids) * S + 8 * len(ids) + 8 * len(np.unique(ids >> 6)), img,
                    int(sb[np.unique(ids)].sum()))
        hit = resident[ids]
        miss_ids = ids[~hit]
        img = int(sb[miss_ids].sum())
        # hits: the arena entry (16-byte padded) and the locator; misses: the
        # locator, the flag word and the stored row from the image
        return (img + int(((sb[ids[hit]] + 15) // 16 * 16).sum()) + len(ids) * S +
                16 * len(ids) + 8 * len(np.unique(miss_ids >> 6))), img, \
            int(sb[np.unique(miss_ids)].sum())

    split = [algo_bytes(k) for k in range(len(steps))]
    g_bytes = [sum(split[k][0] for k in g) for g in groups]
    g_img = [sum(split[k][1] for k in g) for g in groups]
    g_link = [sum(split[k][2] for k in g) for g in groups]

    def make_decode(gi, oi):
        g = groups[gi]
        outs = [out_sets[oi][j].view(-1)[:group_shapes[gi][j][0] * group_shapes[gi][j][1]]
                .view(group_shapes[gi][j]) for j in range(len(g))]
        if batched:
            return ibp.ibp_decompress_batch_launcher(
                md, [(images[steps[k][0]][0], images[steps[k][0]][1]) for k in g], outs)
        if len(g) > 1:
            each = [make_single(k, out) for k, out in zip(g, outs)]

            def all_of_group():
                for f in each:
                    f()
            return all_of_group
        return make_single(g[0], outs[0])

    def make_single(k, out):
        slots, flags = images[steps[k][0]][:2]
        idg = ids_g[k]
        if pos_table is not None:
            if idg is None:
                return lambda: ibp.ibp_decompress_positional(pos_table, slots, flags, out=out)
            return ibp.ibp_gather_decompress_positional_launcher(pos_table, slots, flags, idg, out)
        if idg is None:
            return ibp.ibp_decompress_launcher(md, slots, flags, out)
        if arena is not None:
            return ibp.ibp_gather_decompress_cached_launcher(md, arena, cache_loc, slots, flags,
                                                             idg, out)
        return ibp.ibp_gather_decompress_launcher(md, slots, flags, idg, out)

    # stored bytes of each output row's source row, the copy's read lengths
    out_sb = []
    for ti, ids in steps:
        sb = images[ti][2]
        out_sb.append(images[ti][3] if ids is None else
                      torch.from_numpy(sb[ids].astype(np.int32)).to(dev))

    def make_copy(gi, oi, cap, pack, nt):
        parts = []
        for j, k in enumerate(groups[gi]):
            slots = images[steps[k][0]][0]
            n, S = group_shapes[gi][j]
            parts.append((slots, out_sb[k], ids_g[k], out_sets[oi][j].view(-1)[:n * S].view(n, S)))
        return ceiling.gather_copy_launcher(parts, max_workgroups=cap, pack=pack,
                                            stream_loads=nt)

    def launcher(make):
        # every (group, output set) pair the warm-up, the timed region and
        # the event-pair pass use, converted before any timing
        n_keys = max(K, W, 64) + 1
        memo = {}
        for k in range(n_keys):
            key = (k % len(groups), k % n_sets)
            if key not in memo:
                memo[key] = make(*key)

        def launch(k):
            memo[(k % len(groups), k % n_sets)]()
        return launch

    decode = launcher(make_decode)
    G = len(groups)
    for k in range(W):
        decode(k)
    torch.cuda.synchronize()
    wall, region_s = time_region(stream, decode, K)
    # per-launch event pairs in a second, untimed pass: min / median
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(K, 64))]
    for k, (a, b) in enumerate(ev):
        a.record(stream)
        decode(k)
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    out_bytes = sum(group_out[k % G] for k in range(K))
    a_bytes = sum(g_bytes[k % G] for k in range(K)) / K
    mean_launch_s = region_s / K
    value = out_bytes / wall / 1e9
    achieved = a_bytes / mean_launch_s / 1e9

    # correctness spot check of the timed path against the source rows: the
    # last group launched and the output set it wrote
    gi, oi = (K - 1) % G, (K - 1) % n_sets
    decode(K - 1)
    torch.cuda.synchronize()
    for j, k in enumerate(groups[gi]):
        ti, ids = steps[k]
        n, S = group_shapes[gi][j]
        out = out_sets[oi][j].view(-1)[:n * S].view(n, S)
        pick = np.random.default_rng(k).integers(0, n, 64)
        got = out[torch.from_numpy(pick).to(dev)].cpu().numpy()
        want = wl.source_rows(ti, ids[pick] if ids is not None else pick)
        if not np.array_equal(got, want):
            raise SystemExit(f"bench: decompressed rows of {wl.name} differ from the source")

    # the gather-copy ceiling on the same ids, images and output rotation:
    # the best of a few grid sizes (the copy's waves loop over their work),
    # task shapes and load policies
    ceil_rec = None
    if arena is None:
        best = None
        short = min(s[1] for s in shapes) < 4096
        for pack in ((False, True) if short else (False,)):
            for nt in (False, True):
                for per_cu in CEILING_GRIDS:
                    cap = per_cu * cu_count()
                    copy = launcher(lambda gi, oi, c=cap, p=pack, t=nt: make_copy(gi, oi, c, p, t))
                    for k in range(W):
                        copy(k)
                    torch.cuda.synchronize()
                    _, c_region = time_region(stream, copy, K)
                    if best is None or c_region < best[0]:
                        best = (c_region, per_cu, pack, nt)
                    del copy
        c_s = best[0] / K
        ceil_rec = {"kernel": "gather_copy_kernel", "workgroups_per_cu": best[1],
                    "rows_per_task": "4 KiB of rows" if best[2] else "one",
                    "loads": "non-temporal" if best[3] else "default",
                    "mean_launch_us": round(c_s * 1e6, 3),
                    "achieved": round(a_bytes / c_s / 1e9, 2),
                    "frac_of_peak": round(a_bytes / c_s / 1e9 / HBM_PEAK_GBPS, 4),
                    "decode_frac_of_ceiling": round(c_s / mean_launch_s, 4)}

    S0 = shapes[steps[0][0]][1]
    kernel = decode_kernel_name(S0, opt.width, pos_table is not None, md.invariant_bits,
                                bool(opt.cache_mib), host, batched)
    if host:
        link = link_rate
        link_read = sum(g_link[k % G] for k in range(K)) / K   # crosses the link
        hbm_bytes = a_bytes - sum(g_img[k % G] for k in range(K)) / K
        if link_read / link >= hbm_bytes / HBM_PEAK_GBPS:
            roof = {"bound": "host_link", "achieved": round(link_read / mean_launch_s / 1e9, 2),
                    "peak": round(link, 2), "unit": "GB/s",
                    "frac": round(link_read / mean_launch_s / 1e9 / link, 4), "traffic": None,
                    "peak_note": "measured host-link ceiling, 1 GiB: the better of the pinned "
                                 "host->device hipMemcpy and a zero-copy streaming read kernel"}
        else:  # cache hits dominate: the HBM side bounds the launch
            roof = {"bound": "hbm", "achieved": round(hbm_bytes / mean_launch_s / 1e9, 2),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(hbm_bytes / mean_launch_s / 1e9 / HBM_PEAK_GBPS, 4),
                    "traffic": None, "link_GB_per_s": round(link_read / mean_launch_s / 1e9, 2),
                    "link_peak": round(link, 2)}
        if ceil_rec is not None:
            ceil_rec["achieved"] = round(link_read / c_s / 1e9, 2)
            ceil_rec["frac_of_peak"] = round(link_read / c_s / 1e9 / link, 4)
            ceil_rec["unit"] = "GB/s of image read across the host link"
        # [IBP] Results: "ideal" rate = link ceiling x (output / image bytes)
        out_per_launch = out_bytes / K
        img_per_launch = link_read
        ideal = link * out_per_launch / max(1, img_per_launch)
        roof["ideal_output_GB_per_s"] = round(ideal, 2)
        roof["output_frac_of_ideal"] = round(out_per_launch / mean_launch_s / 1e9 / ideal, 4)
    else:
        traffic = None if opt.cache_mib or opt.width != 32 else \
            traffic_from_profiles(kernel, wl.name)
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic}
    if ceil_rec is not None:
        roof["ceiling"] = ceil_rec
    rec = {"value": round(value, 2), "unit": "GB/s", "steps": K, "warmup": W,
           "ms_per_step": round(wall / K * 1e3, 5),
           "source": "pinned_host" if host else "device",
           "row_bytes": sorted({s[1] for s in shapes}),
           "outputs_rotated_MiB": round(n_sets * max(group_out) / 2**20, 1),
           "kernel": {"name": kernel, "mean_launch_us": round(mean_launch_s * 1e6, 3),
                      "event_pair_median_us": round(float(np.median(launch_ms)) * 1e3, 3),
                      "event_pair_min_us": round(float(launch_ms.min()) * 1e3, 3),
                      "launches_per_step": 1 if batched else len(groups[0]),
                      "algorithmic_bytes_per_launch": int(a_bytes),
                      "source_sha256_16": kernel_source_hash()},
           "roofline": roof}
    if cache is not None:
        rec["cache"] = cache
    log(f"{wl.name} ({rec['source']}): {value:.0f} GB/s out, {kernel} "
        f"{mean_launch_s * 1e6:.2f} us, frac {roof['frac']}" +
        (f", ceiling {ceil_rec['mean_launch_us']} us" if ceil_rec else ""))
    del out_sets
    return rec


def measure_tiny(dev, reps: int = 50):
    """The tiny dense table (4096 x 128 fp32), reported only: compress, full
    decompress and the round trip of the 2 MiB table, each the median of
    `reps` calls."""
    import torch
    from lossless_bit_level_amd import ibp
    import synthetic as syn
    x = syn.tiny_dense()
    xg = torch.from_numpy(x.view(np.uint8)).to(dev)
    md, _ = ibp.ibp_build_metadata(xg)
    slots, flags, rb = ibp.ibp_compress(md, xg)
    out = ibp.ibp_decompress(md, slots, flags)
    torch.cuda.synchronize()
    if not torch.equal(out, xg):
        raise SystemExit("bench: tiny_dense round trip differs")
    stream = torch.cuda.current_stream()

    def med(fn):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        return float(np.median(ts))
    c = med(lambda: ibp.ibp_compress(md, xg, slots=slots, flags=flags, row_bits=rb))
    d = med(lambda: ibp.ibp_decompress(md, slots, flags, out=out))
    r = med(lambda: (ibp.ibp_compress(md, xg, slots=slots, flags=flags, row_bits=rb),
                     ibp.ibp_decompress(md, slots, flags, out=out)))
    sb = stored_bytes_per_row(rb.cpu().numpy()[:x.shape[0]], 512)
    nb = x.nbytes
    return {"desc": "tiny dense 4096 x 128 fp32 N(0, 0.1^2): compress, full decompress, round "
                    "trip (2 MiB: launch- and cache-bound; reported only)",
            "compress_us": round(c * 1e6, 2), "compress_GB_per_s": round(nb / c / 1e9, 1),
            "decompress_us": round(d * 1e6, 2), "decompress_GB_per_s": round(nb / d / 1e9, 1),
            "round_trip_us": round(r * 1e6, 2), "round_trip_GB_per_s": round(nb / r / 1e9, 1),
            "compression_ratio": round(nb / int(sb.sum()), 4),
            "metadata": {"mask": f"0x{md.mask:08X}", "bitval": f"0x{md.bitval:08X}",
                         "invariant_bits": md.invariant_bits}}


# --------------------------------------------------------- cpu baseline --

def cpu_baseline(wl: Workload, md, threads: int, allowed: int):
    """The CPU oracle (plain bit-serial C, test infrastructure) on the host
    cores, on bounded samples of the workload:
      * every thread of the share: compress, then full decompress, of the
        first layer's tables (or, for a gather workload, of the rows the first
        gather ids reference, then the gather over those ids);
      * one thread: the tiny table (compress, decompress) and the first
        256 MiB of the workload's tables in storage order."""
    from oracle import oracle as orc
    import synthetic as syn
    md_o = orc.Metadata(int(md.width_bits), int(md.mask), int(md.bitval), int(md.t_ppm))
    ex = ThreadPoolExecutor(threads)

    def par_compress(x):
        parts = np.array_split(np.arange(x.shape[0]), threads)
        res = list(ex.map(lambda p: orc.compress(md_o, x[p]) if len(p) else None, parts))
        return [(p, r) for p, r in zip(parts, res) if r is not None]

    def par_decompress(pieces, S):
        outs = list(ex.map(lambda pr: orc.decompress(md_o, pr[1][0], pr[1][1]), pieces))
        return outs

    rec = {"unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "cpus_allowed": allowed}
    gather = wl.steps[0][1] is not None
    if not gather:
        tabs = [wl.table(i) for i in range(min(wl.n_tables, wl.layer_size))]
        raw = sum(t.nbytes for t in tabs)
        t0 = time.perf_counter()
        comp = [par_compress(t.reshape(t.shape[0], -1).view(np.uint8)) for t in tabs]
        tc = time.perf_counter() - t0
        t0 = time.perf_counter()
        outs = [par_decompress(c, t.nbytes // t.shape[0]) for c, t in zip(comp, tabs)]
        td = time.perf_counter() - t0
        for t, o in zip(tabs, outs):
            if not np.array_equal(np.concatenate(o), t.reshape(t.shape[0], -1).view(np.uint8)):
                raise SystemExit("bench: oracle round trip differs")
        rec["value"] = round(raw / td / 1e9, 4)
        rec["sample"] = (f"full decompress of the first {len(tabs)} table(s) "
                         f"({raw / 2**20:.0f} MiB out) on {threads} threads, {td:.2f} s")
        rec["compress_GB_per_s"] = round(raw / tc / 1e9, 4)
        del comp, outs
    else:
        x = wl.table(0)
        x2 = x.reshape(x.shape[0], -1).view(np.uint8)
        S = x2.shape[1]
        ids0 = np.concatenate([ids for _, ids in wl.steps])
        n_ids = min(len(ids0), 262144 if S <= 1024 else 131072)
        ids = ids0[:n_ids]
        uniq, inv = np.unique(ids, return_inverse=True)
        src = x2[uniq]
        t0 = time.perf_counter()
        pieces = par_compress(src)
        tc = time.perf_counter() - t0
        slots = np.concatenate([r[0] for _, r in pieces])
        flag_bits = np.concatenate([[(int(r[1][i >> 6]) >> (i & 63)) & 1 for i in range(len(p))]
                                    for p, r in pieces]).astype(np.uint8)
        pad = np.zeros(((len(uniq) + 63) // 64) * 64, np.uint8)
        pad[:len(uniq)] = flag_bits
        flags = np.packbits(pad, bitorder="little").view(np.uint64)
        id_parts = np.array_split(inv.astype(np.int64), threads)
        t0 = time.perf_counter()
        outs = list(ex.map(lambda p: orc.gather_decompress(md_o, slots, flags, p), id_parts))
        td = time.perf_counter() - t0
        if not np.array_equal(np.concatenate(outs), x2[ids]):
            raise SystemExit("bench: oracle gather differs")
        rec["value"] = round(n_ids * S / td / 1e9, 4)
        rec["sample"] = (f"gather of the first {n_ids} ids ({n_ids * S / 2**20:.0f} MiB out) on "
                         f"{threads} threads, {td:.2f} s; their {len(uniq)} distinct rows "
                         f"compressed first")
        rec["compress_GB_per_s"] = round(src.nbytes / tc / 1e9, 4)
    ex.shutdown()
    # one thread: the tiny table, then 256 MiB of the workload in storage order
    single = {}
    tiny = syn.tiny_dense()
    md_t, _ = orc.build_metadata(tiny, 32)
    t0 = time.perf_counter()
    s_t, f_t, _ = orc.compress(md_t, tiny)
    tc = time.perf_counter() - t0
    t0 = time.perf_counter()
    back = orc.decompress(md_t, s_t, f_t)
    td = time.perf_counter() - t0
    assert np.array_equal(back, tiny.view(np.uint8))
    single["tiny_dense"] = {"compress_GB_per_s": round(tiny.nbytes / tc / 1e9, 4),
                            "decompress_GB_per_s": round(tiny.nbytes / td / 1e9, 4)}
    budget = 256 << 20
    pieces, got = [], 0
    for i in range(wl.n_tables):
        x = wl.table(i)
        x2 = x.reshape(x.shape[0], -1).view(np.uint8)
        take = min(x2.shape[0], (budget - got) // x2.shape[1])
        if take <= 0:
            break
        pieces.append(x2[:take])
        got += take * x2.shape[1]
    tc = td = 0.0
    for p in pieces:
        t0 = time.perf_counter()
        s_p, f_p, _ = orc.compress(md_o, p)
        tc += time.perf_counter() - t0
        t0 = time.perf_counter()
        orc.decompress(md_o, s_p, f_p)
        td += time.perf_counter() - t0
    single["slice_256MiB"] = {"MiB": round(got / 2**20, 1),
                              "compress_GB_per_s": round(got / tc / 1e9, 4),
                              "decompress_GB_per_s": round(got / td / 1e9, 4)}
    rec["single_thread"] = single
    return rec


# --------------------------------------------------------------- main ----

SUBCONFIGS = [  # (key, workload, sources)
    ("sparse_gnn", "sparse_gnn", ("device",)),
    ("dense_gnn", "dense_gnn", ("device",)),
    ("dlrm_emb", "dlrm_emb", ("device",)),
    ("llm_kv", "llm_kv", ("device", "host")),
]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llm_weights",
                    choices=["llm_weights", "sparse_gnn", "dense_gnn", "dlrm_emb", "llm_kv",
                             "tiny_dense"])
    ap.add_argument("--source", default="device", choices=["device", "host"])
    ap.add_argument("--width", type=int, default=32, choices=[16, 32, 64],
                    help="block width W in bits (32: the tuned kernels)")
    ap.add_argument("--positional", action="store_true",
                    help="per-position Mask/Bitval (one pair per block position of a row) "
                         "instead of one global pair; W = 32")
    ap.add_argument("--cache-mib", type=int, default=0,
                    help="keep the most popular rows that fit this many MiB in a packed, "
                         "compressed GPU cache; the other rows come from the image "
                         "(--source host: pinned host memory)")
    ap.add_argument("--per-tensor", action="store_true",
                    help="llm_weights: one launch per matrix instead of one batched launch "
                         "per layer")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the chosen workload (the default run also times every "
                         "other workload under \"configs\")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy before the timed loop "
                         "(calibrates rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the IBP path here is single-GPU "
              "(multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from lossless_bit_level_amd import ibp, ceiling
    ibp.lib()
    ceiling.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    threads, allowed = cpu_threads()
    t_all = time.perf_counter()

    if args.pmc_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    default_run = (args.workload == "llm_weights" and args.source == "device" and
                   args.width == 32 and not args.positional and not args.cache_mib and
                   not args.per_tensor)
    with_configs = default_run and not args.no_configs
    link_rate, link_rec = (link_ceiling(dev, stream) if (args.source == "host" or with_configs)
                           else (None, None))
    opt = Opts(args.source, args.width, args.positional, args.cache_mib, args.per_tensor)
    if args.workload == "tiny_dense":
        raise SystemExit("tiny_dense is reported under \"configs\" of the default run")
    t_gen = time.perf_counter()
    wl = make_workload(args.workload, threads)
    log(f"workload {wl.name}: set up in {time.perf_counter() - t_gen:.1f} s")
    sources = [args.source] + (["host"] if with_configs else [])
    head_all = measure(wl, opt, sources, args.steps, args.warmup, threads, dev, link_rate)
    head = head_all[args.source]
    configs = {}
    if with_configs:
        configs["llm_weights_host"] = head_all["host"]
    torch.cuda.empty_cache()

    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": wl.name, "desc": wl.desc, "source": args.source,
                   "tables": wl.n_tables, "row_bytes": head["row_bytes"],
                   "block_bits": args.width, "cache_mib": args.cache_mib,
                   "metadata": "per_position" if args.positional else "global",
                   "outputs_rotated_MiB": head["outputs_rotated_MiB"],
                   "parallelism": "none (1 GPU)"},
        "compression_ratio": head["compression_ratio"],
        "compression_ratio_bits": head["compression_ratio_bits"],
        "compression_ratio_with_side_data": head["compression_ratio_with_side_data"],
        "metadata": head["metadata"],
        "compress": head["compress"],
        "kernel": head["kernel"],
        "roofline": head["roofline"],
    }
    if "cache" in head:
        res["cache"] = head["cache"]
    if args.source == "device":
        ref = device_copy_reference(dev, stream)
        ref["decode_over_best_copy"] = round(head["roofline"]["achieved"] / ref["best_GB_per_s"],
                                             4)
        res["roofline"]["device_copy"] = ref
    if link_rate is not None:
        res["host_link"] = link_rec

    # the CPU oracle on the headline workload, before its tables are dropped
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        from lossless_bit_level_amd import ibp as _b
        mdh = _b.ibp_metadata()
        mdh.width_bits = args.width
        mdh.mask = int(head["metadata"]["mask"], 16)
        mdh.bitval = int(head["metadata"]["bitval"], 16)
        mdh.t_ppm = 900000
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline(wl, mdh, threads, allowed)
        log(f"cpu baseline done in {time.perf_counter() - t0:.1f} s")
    del wl, head_all

    if with_configs:
        configs["tiny_dense"] = measure_tiny(dev)
        for key, name, srcs in SUBCONFIGS:
            t0 = time.perf_counter()
            w = make_workload(name, threads)
            r = measure(w, Opts(), srcs, 256, 8, threads, dev, link_rate)
            for s, rec in r.items():
                configs[key if s == "device" else key + "_host"] = rec
            del w, r
            torch.cuda.empty_cache()
            log(f"{key}: {time.perf_counter() - t0:.1f} s")
        res["configs"] = configs
    log(f"bench total {time.perf_counter() - t_all:.1f} s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
