"""Benchmark of IBP decompression on one MI355X.

Default workload: sparse GNN features, a 1,048,576 x 512 fp32 table (2 GiB,
entries 1.0 with probability 0.01) compressed with Invariant Bit Packing,
then gather-decompressed in batches of 65,536 uniform random row ids.  One
step = one gather-decompress launch over one batch (8 batches, 8 output
buffers of 128 MiB rotated so that neither L2 nor the 256 MiB MALL holds the
output).  Metadata building and compression run once before the timed region
(the method builds metadata once and compresses a table once; both are
timed and reported separately).

Prints one JSON line (rank 0):
  value      = GB/s of uncompressed output over the timed steps
  roofline   = algorithmic bytes of one launch / its mean duration (HIP
               events on the launch stream) against the 8 TB/s HBM peak
  cpu_baseline = the CPU oracle's gather over a bounded sample, all threads
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "IBP decompress GB/s (uncompressed out), % of HBM roofline; compression ratio"
HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "lossless_bit_level_amd", "csrc", "ibp.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------- workloads --

class Workload:
    """tables: list of numpy arrays (rows on axis 0); steps: list of
    (table index, ids or None); sample_for_metadata: numpy array."""

    def __init__(self, name, desc, tables, steps, sample, n_out_bytes, hot=None, layer_size=1):
        self.name, self.desc, self.tables, self.steps = name, desc, tables, steps
        self.sample = sample
        self.n_out_bytes = n_out_bytes
        self.hot = hot  # row ids by static popularity (cache fill order)
        self.layer_size = layer_size  # consecutive steps that one batched launch may take


def make_workload(name: str) -> Workload:
    import synthetic as syn
    if name == "sparse_gnn":
        x = syn.sparse_gnn_rows()
        ids = syn.uniform_ids(syn.SPARSE_GNN_ROWS, 8, 65536)
        return Workload(name, "sparse GNN features 1048576 x 512 fp32, gather 8 x 65536 "
                        "uniform ids", [x], [(0, b) for b in ids], x, 65536 * 2048,
                        hot=np.arange(x.shape[0], dtype=np.int64))
    if name in ("dense_gnn", "dlrm_emb"):
        if name == "dense_gnn":
            x = syn.dense_gnn_rows()
            ids = syn.zipf_ids(syn.DENSE_GNN_ROWS, 8, 65536)
            desc = "dense GNN features 2097152 x 256 fp32 N(0,0.25)"
        else:
            x = syn.dlrm_emb_rows()
            ids = syn.zipf_ids(syn.DLRM_EMB_ROWS, 8, 65536, seed=2)
            desc = "DLRM embedding 4194304 x 128 fp32 U(-0.05,0.05)"
        return Workload(name, desc + ", gather 8 x 65536 Zipf(1.05) ids", [x],
                        [(0, b) for b in ids], x, 65536 * x.shape[1] * 4,
                        hot=syn.zipf_hot_order(x.shape[0]))
    if name == "llm_kv":
        x = syn.llm_kv_pages()
        ids = syn.kv_page_ids()
        return Workload(name, "LLM KV cache [16,32,4096,128] bf16, 4 KiB pages, gather "
                        "8 x 16384 page ids", [x], [(0, b) for b in ids], x, 16384 * 4096,
                        hot=np.arange(x.shape[0], dtype=np.int64))
    if name == "llm_weights":
        tables = [syn.llm_weight(layer, j) for layer in (0, 1) for j in range(7)]
        steps = [(t, None) for t in range(len(tables))]
        return Workload(name, "LLM weights bf16, 4 x [4096,4096] + 3 x [4096,14336] per "
                        "layer, full decompress layer by layer (the 7 matrices of a layer in "
                        "one batched call; 2 resident layers)", tables,
                        steps, tables[0], None, layer_size=7)
    raise SystemExit(f"unknown workload {name}")


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
        return "decode_wide_kernel"
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


def cpu_baseline(wl: Workload, md, target_core_s: float = 20.0, pos_mask=None, pos_bitval=None):
    """Time the CPU oracle's gather-decompress on a bounded sample of the same
    workload: the rows the first ids of the gather batches reference are
    compressed by the oracle (untimed), then the oracle's gather over those
    ids is timed on every allowed core (one contiguous id range per thread)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as orc
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    md_o = orc.Metadata(int(md.width_bits), int(md.mask), int(md.bitval), int(md.t_ppm))
    if pos_mask is not None:   # per-position metadata: the oracle's positional codec
        pm = orc.PositionalMetadata(32, np.asarray(pos_mask, np.uint64),
                                    np.asarray(pos_bitval, np.uint64))
        comp = lambda rows: orc.compress_positional(pm, rows)
        gath = lambda sl, fl, ids: orc.gather_decompress_positional(pm, sl, fl, ids)
    else:
        comp = lambda rows: orc.compress(md_o, rows)
        gath = lambda sl, fl, ids: orc.gather_decompress(md_o, sl, fl, ids)
    t_idx, ids0 = wl.steps[0]
    table = wl.tables[t_idx]
    S = table.nbytes // table.shape[0]
    if ids0 is None:
        ids0 = np.arange(table.shape[0], dtype=np.int64)
    else:  # the gather batches back to back
        ids0 = np.concatenate([ids for ti, ids in wl.steps if ti == t_idx])
    # calibrate on 64 rows, size the sample for ~target_core_s core-seconds
    probe = np.unique(ids0[:64])
    local = table[probe]
    slots, flags, _ = comp(local)
    t0 = time.perf_counter()
    gath(slots, flags, np.arange(len(probe)))
    per_row = (time.perf_counter() - t0) / len(probe)
    n_ids = int(min(len(ids0), max(threads * 64, target_core_s / max(per_row, 1e-9))))
    ids = ids0[:n_ids]
    uniq, inv = np.unique(ids, return_inverse=True)
    src = table[uniq]
    parts = np.array_split(np.arange(len(uniq)), threads)
    with ThreadPoolExecutor(threads) as ex:   # oracle compress of the sample rows
        res = list(ex.map(lambda p: comp(src[p]), parts))
    slots = np.concatenate([r[0] for r in res])
    flag_bits = np.concatenate([[(int(r[1][i >> 6]) >> (i & 63)) & 1 for i in range(len(p))]
                                for r, p in zip(res, parts)]).astype(np.uint8)
    pad = np.zeros(((len(uniq) + 63) // 64) * 64, np.uint8)
    pad[:len(uniq)] = flag_bits
    flags = np.packbits(pad, bitorder="little").view(np.uint64)
    id_parts = np.array_split(inv.astype(np.int64), threads)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        outs = list(ex.map(lambda p: gath(slots, flags, p), id_parts))
    dt = time.perf_counter() - t0
    out = np.concatenate(outs)
    assert np.array_equal(out, table[ids].reshape(len(ids), -1).view(np.uint8))
    return {"value": round(n_ids * S / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"first {n_ids} ids of the gather batches ({n_ids * S / 2**20:.1f} MiB out), "
                      f"bit-serial C oracle, {threads} threads, {dt:.2f} s wall"}


# --------------------------------------------------------------- main ----

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="sparse_gnn",
                    choices=["sparse_gnn", "dense_gnn", "dlrm_emb", "llm_weights", "llm_kv"])
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
    from lossless_bit_level_amd import ibp
    ibp.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    wl = make_workload(args.workload)
    log(f"workload {wl.name}: generated in {time.perf_counter() - t_gen:.1f} s")

    tables_g = [torch.from_numpy(t.reshape(t.shape[0], -1).view(np.uint8)).to(dev)
                for t in wl.tables]
    S = tables_g[0].shape[1]
    stream = torch.cuda.current_stream()

    # metadata (first min(N, 2^24) blocks) and compression, timed apart
    samp = torch.from_numpy(wl.sample.reshape(-1).view(np.uint8)).to(dev)
    n_blocks = min(samp.numel() * 8 // args.width, 1 << 24)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    md, _ = ibp.ibp_build_metadata(samp, n_blocks=n_blocks, width_bits=args.width)
    meta_first_ms = (time.perf_counter() - t0) * 1e3   # includes the library's first-use setup
    t0 = time.perf_counter()
    md, _ = ibp.ibp_build_metadata(samp, n_blocks=n_blocks, width_bits=args.width)
    meta_ms = (time.perf_counter() - t0) * 1e3
    del samp
    pos_table = pmask = pbitval = None
    if args.positional:
        if args.width != 32 or args.cache_mib:
            raise SystemExit("--positional runs with W = 32 and without --cache-mib")
        # the same 2^24-block budget, as whole sample rows of the first table
        s_rows = max(1, min(wl.sample.shape[0], (1 << 24) // (wl.sample.nbytes // wl.sample.shape[0] // 4)))
        samp = torch.from_numpy(wl.sample[:s_rows].reshape(s_rows, -1).view(np.uint8)).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pos_table, pmask, pbitval = ibp.ibp_build_metadata_positional(samp)
        meta_ms = (time.perf_counter() - t0) * 1e3
        del samp
        log(f"positional metadata over {s_rows} rows in {meta_ms:.1f} ms; "
            f"{len(set(pmask.tolist()))} distinct masks")
    images = []
    comp_ms = 0.0
    raw_bytes = stored = 0
    bits_total = 0
    side_bytes = 0   # flag words of every table
    def compress(tg, out=(None, None, None)):
        slots, flags, rb = out
        if pos_table is not None:
            return ibp.ibp_compress_positional(pos_table, tg, slots=slots, flags=flags, row_bits=rb)
        return ibp.ibp_compress(md, tg, slots=slots, flags=flags, row_bits=rb)

    for tg in tables_g:
        out = compress(tg)                    # warm; allocates the image buffers
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(3):                    # the median of three calls into those buffers
            e0.record(stream)
            slots, flags, rb = compress(tg, out)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        comp_ms += sorted(times)[1]
        rbn = rb.cpu().numpy()[:tg.shape[0]]
        sb = stored_bytes_per_row(rbn, tg.shape[1])
        images.append((slots, flags, sb))
        raw_bytes += tg.numel()
        stored += int(sb.sum())
        side_bytes += 8 * ((tg.shape[0] + 63) // 64)
        bits_total += int(np.minimum(rbn.astype(np.int64), 8 * tg.shape[1]).sum())
    comp_GBps = raw_bytes / (comp_ms / 1e3) / 1e9
    log(f"metadata {md} in {meta_ms:.1f} ms; compress {comp_ms:.2f} ms ({comp_GBps:.0f} GB/s); "
        f"ratio {raw_bytes / stored:.4f}")

    inplace = None
    if args.source == "host":
        # [IBP] System integration: host tensors compressed in place, each in
        # its own fixed-size buffer, by the GPU over the host link (zero-copy)
        t_ip = 0.0
        raw_ip = 0
        for t in wl.tables:
            h = torch.from_numpy(t.reshape(t.shape[0], -1).view(np.uint8)).pin_memory()

            def in_place():
                if pos_table is not None:
                    ibp.ibp_compress_positional(pos_table, h, slots=h, want_row_bits=False)
                else:
                    ibp.ibp_compress(md, h, slots=h, want_row_bits=False)
            in_place()
            torch.cuda.synchronize()
            h.copy_(torch.from_numpy(t.reshape(t.shape[0], -1).view(np.uint8)))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            in_place()
            e1.record(stream)
            torch.cuda.synchronize()
            t_ip += e0.elapsed_time(e1) / 1e3
            raw_ip += h.numel()
            del h
        inplace = {"ms": round(t_ip * 1e3, 3), "GB_per_s_raw": round(raw_ip / t_ip / 1e9, 2)}
        log(f"in-place compression of the pinned host tables: {t_ip * 1e3:.2f} ms "
            f"({raw_ip / t_ip / 1e9:.1f} GB/s raw)")
        host_images = []
        for slots, flags, sb in images:
            h = torch.empty(slots.shape, dtype=torch.uint8, pin_memory=True)
            h.copy_(slots)
            host_images.append((h, flags, sb))
        images = host_images
    del tables_g

    # [IBP] System integration, cache compression: the most popular rows that
    # fit the budget, in their stored form, packed into a GPU arena
    cache = None
    resident = None
    if args.cache_mib:
        if len(wl.tables) != 1 or wl.hot is None or any(ids is None for _, ids in wl.steps):
            raise SystemExit("--cache-mib needs a gather workload over one table")
        slots, flags, sb = images[0]
        n_rows = wl.tables[0].shape[0]
        budget = args.cache_mib << 20
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
        cache = {"budget_mib": args.cache_mib, "rows": k, "rows_fraction": round(k / n_rows, 4),
                 "arena_mib": round(arena_bytes / 2**20, 2),
                 "hit_rate": round(float(resident[all_ids].mean()), 4),
                 "raw_cache_rows": int(raw_rows),
                 "raw_cache_hit_rate": round(float(counts[wl.hot[:raw_rows]].sum() /
                                                   counts.sum()), 4),
                 "plan_ms": round(plan_ms, 3), "fill_ms": round(e0.elapsed_time(e1), 3)}
        log(f"cache: {cache}")

    # per-step launch plan: (image index, ids tensor or None, output buffer)
    plan = []
    outs = []
    for i, (ti, ids) in enumerate(wl.steps):
        n_out = len(ids) if ids is not None else wl.tables[ti].shape[0]
        outs.append(torch.empty((n_out, S if ids is not None else
                                 wl.tables[ti].nbytes // wl.tables[ti].shape[0]),
                                dtype=torch.uint8, device=dev))
        idg = torch.from_numpy(np.ascontiguousarray(ids)).to(dev) if ids is not None else None
        plan.append((ti, idg, outs[-1], ids))

    def algo_bytes(ti, ids):
        """(bytes the launch must move, duplicates counted; bytes of it read
        from the image; bytes of distinct image rows, which is what must cross
        the host link when the image is in host memory: a repeated row is
        served from the GPU's caches)."""
        slots, flags, sb = images[ti]
        if ids is None:
            n = wl.tables[ti].shape[0]
            img = int(sb.sum())
            return img + wl.tables[ti].nbytes + 8 * ((n + 63) // 64), img, img
        row_out = wl.tables[ti].nbytes // wl.tables[ti].shape[0]
        if resident is None:
            img = int(sb[ids].sum())
            return (img + len(ids) * row_out + 8 * len(ids) + 8 * len(np.unique(ids >> 6)), img,
                    int(sb[np.unique(ids)].sum()))
        hit = resident[ids]
        miss_ids = ids[~hit]
        img = int(sb[miss_ids].sum())
        # hits: the arena entry (16-byte padded) and the locator; misses: the
        # locator, the flag word and the stored row from the image
        return (img + int(((sb[ids[hit]] + 15) // 16 * 16).sum()) + len(ids) * row_out +
                16 * len(ids) + 8 * len(np.unique(miss_ids >> 6))), img, \
            int(sb[np.unique(miss_ids)].sum())

    # launch groups: the weight matrices of a layer go in one batched call
    # (layer-by-layer loading), every other step is a launch of its own
    batch_layers = wl.layer_size > 1 and not args.per_tensor and pos_table is None and \
        args.width == 32 and args.source == "device" and not args.cache_mib
    if batch_layers:
        groups = [list(range(g, min(g + wl.layer_size, len(plan))))
                  for g in range(0, len(plan), wl.layer_size)]
    else:
        groups = [[k] for k in range(len(plan))]
    plan_split = [algo_bytes(ti, ids) for ti, _, _, ids in plan]
    plan_bytes = [sum(plan_split[k][0] for k in g) for g in groups]
    plan_img = [sum(plan_split[k][1] for k in g) for g in groups]
    plan_link = [sum(plan_split[k][2] for k in g) for g in groups]
    plan_out = [sum(plan[k][2].numel() for k in g) for g in groups]

    launchers = []
    for ti, idg, out, _ in (plan if not batch_layers else []):
        slots, flags, _ = images[ti]
        if pos_table is not None:
            if idg is None:
                launchers.append(lambda s=slots, f=flags, o=out:
                                 ibp.ibp_decompress_positional(pos_table, s, f, out=o))
            else:
                launchers.append(ibp.ibp_gather_decompress_positional_launcher(
                    pos_table, slots, flags, idg, out))
        elif idg is None:
            launchers.append(ibp.ibp_decompress_launcher(md, slots, flags, out))
        elif cache is not None:
            launchers.append(ibp.ibp_gather_decompress_cached_launcher(
                md, arena, cache_loc, slots, flags, idg, out))
        else:
            launchers.append(ibp.ibp_gather_decompress_launcher(md, slots, flags, idg, out))

    if batch_layers:
        for g in groups:
            launchers.append(ibp.ibp_decompress_batch_launcher(
                md, [(images[plan[k][0]][0], images[plan[k][0]][1]) for k in g],
                [plan[k][2] for k in g]))

    def launch(k):
        launchers[k % len(launchers)]()

    if args.pmc_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for k in range(args.warmup):
        launch(k)
    torch.cuda.synchronize()

    # Timed region: K launches back to back on one stream, bracketed by a
    # synchronize on both sides and by HIP events on the launch stream.  The
    # mean launch duration is the event time over the region divided by K
    # (it includes the gaps between kernels, so it is an upper bound).
    K = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for k in range(K):
        launch(k)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_s = e_start.elapsed_time(e_end) / 1e3
    # per-launch event pairs in a second, untimed pass: min/median durations
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(K, 64))]
    for k, (a, b) in enumerate(ev):
        a.record(stream)
        launch(k)
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    out_bytes = sum(plan_out[k % len(groups)] for k in range(K))
    a_bytes = sum(plan_bytes[k % len(groups)] for k in range(K)) / K
    value = out_bytes / wall / 1e9
    mean_launch_s = region_s / K
    achieved = a_bytes / mean_launch_s / 1e9

    # correctness spot check of the timed path against the source rows
    for pk in groups[(K - 1) % len(groups)]:
        ti, idg, out, ids = plan[pk]
        src = wl.tables[ti].reshape(wl.tables[ti].shape[0], -1).view(np.uint8)
        pick = np.random.default_rng(0).integers(0, out.shape[0], 256)
        got = out[torch.from_numpy(pick).to(dev)].cpu().numpy()
        want = src[ids[pick]] if ids is not None else src[pick]
        if not np.array_equal(got, want):
            raise SystemExit("bench: decompressed rows differ from the source table")

    if args.source == "host":
        # host-link ceiling: pinned host -> device copy of 1 GiB
        h = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
        d = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        d.copy_(h, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            d.copy_(h, non_blocking=True)
        e1.record(stream)
        torch.cuda.synchronize()
        link = 3 * (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
        del h, d
        link_read = sum(plan_link[k % len(groups)] for k in range(K)) / K  # crosses the link
        hbm_bytes = a_bytes - sum(plan_img[k % len(groups)] for k in range(K)) / K
        if link_read / link >= hbm_bytes / HBM_PEAK_GBPS:
            roof = {"bound": "host_link", "achieved": round(link_read / mean_launch_s / 1e9, 2),
                    "peak": round(link, 2), "unit": "GB/s",
                    "frac": round(link_read / mean_launch_s / 1e9 / link, 4), "traffic": None,
                    "peak_note": "measured pinned host->device hipMemcpy ceiling, 1 GiB"}
        else:  # cache hits dominate: the HBM side bounds the launch
            roof = {"bound": "hbm", "achieved": round(hbm_bytes / mean_launch_s / 1e9, 2),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(hbm_bytes / mean_launch_s / 1e9 / HBM_PEAK_GBPS, 4),
                    "traffic": None, "link_GB_per_s": round(link_read / mean_launch_s / 1e9, 2),
                    "link_peak": round(link, 2)}
    else:
        traffic = None if cache or args.width != 32 else \
            traffic_from_profiles(decode_kernel_name(S, positional=args.positional,
                                                     invariant_bits=md.invariant_bits,
                                                     batched=batch_layers), wl.name)
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": wl.name, "desc": wl.desc, "source": args.source,
                   "row_bytes": S, "block_bits": args.width, "cache_mib": args.cache_mib,
                   "metadata": "per_position" if args.positional else "global",
                   "parallelism": "none (1 GPU)"},
        "compression_ratio": round(raw_bytes / stored, 4),
        "compression_ratio_bits": round(raw_bytes * 8 / bits_total, 4),
        # with the flag words and the metadata (32 bytes, or the position table)
        "compression_ratio_with_side_data": round(raw_bytes / (stored + side_bytes + (
            pos_table.numel() if pos_table is not None else 32)), 4),
        "metadata": {"mask": f"0x{md.mask:0{args.width // 4}X}",
                     "bitval": f"0x{md.bitval:0{args.width // 4}X}",
                     "invariant_bits": md.invariant_bits, "build_ms": round(meta_ms, 3),
                     "first_call_ms": round(meta_first_ms, 3)},
        "compress": {"ms": round(comp_ms, 3), "GB_per_s_raw_in": round(comp_GBps, 1),
                     # raw bytes read plus stored bytes written, against the HBM peak
                     "frac": round((raw_bytes + stored) / (comp_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "in_place_pinned_host": inplace},
        "kernel": {"name": decode_kernel_name(S, args.width, args.positional, md.invariant_bits,
                                              bool(args.cache_mib), args.source == "host",
                                              batch_layers),
                   "mean_launch_us": round(mean_launch_s * 1e6, 3),
                   "event_pair_median_us": round(float(np.median(launch_ms)) * 1e3, 3),
                   "event_pair_min_us": round(float(launch_ms.min()) * 1e3, 3),
                   "algorithmic_bytes_per_launch": int(a_bytes),
                   "source_sha256_16": kernel_source_hash()},
        "roofline": roof,
    }
    if cache is not None:
        res["cache"] = cache
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(wl, md, pos_mask=pmask if pos_table is not None else None,
                                           pos_bitval=pbitval if pos_table is not None else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
