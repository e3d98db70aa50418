"""Seeded synthetic inputs shaped like the IBP page's workloads.

Shared by the oracle-side tests, the GPU tests and the benchmark.  This
module only draws random numbers (numpy PCG64) and lays them out; it holds
none of the compression method's arithmetic.

The page measures on real GNN feature tables, DLRM embedding tables and LLM
weights / KV caches (explainer page "Reducing the GPU Memory Bottleneck with
Lossless Compression for ML -- Extended", sections "Results" and
"Contributions").  None of those data sets is available, so each workload
below is a synthetic stand-in with the same dtype, shape and value
distribution family:

  tiny_dense    4096 x 128 fp32 ~ N(0, 0.1^2), seed 0
  sparse_gnn    1,048,576 x 512 fp32, each entry 1.0 with probability 0.01
                else 0.0 (bag-of-words features); 8 batches x 65,536 uniform
                row ids
  dense_gnn     2,097,152 x 256 fp32 ~ N(0, 0.5^2); Zipf(1.05) row ids
  dlrm_emb      4,194,304 x 128 fp32 ~ U(-0.05, 0.05); Zipf(1.05) row ids
  llm_weights   32 layers x (4 x [4096, 4096] + 3 x [4096, 14336]) bf16
                ~ N(0, 0.02^2)
  llm_kv        [16, 32, 4096, 128] bf16 ~ N(0, 1), 4 outlier channels per
                head scaled x20; 16-token pages (4 KiB) gathered by id
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 65536

# ------------------------------------------------------------- helpers --


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to IEEE fp16 (numpy's conversion: nearest, ties to even,
    subnormals kept, overflow to infinity); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _chunked(n_rows: int, row_start: int, row_count: int, make_chunk, threads: int = 1):
    """Rows [row_start, row_start+row_count) of a table built from 65,536-row
    chunks, chunk c drawn by make_chunk(c, rows_in_chunk).  With threads > 1
    the chunks are drawn concurrently (each has its own generator, so the
    values do not depend on the thread count)."""
    assert 0 <= row_start and row_start + row_count <= n_rows
    c0 = row_start // CHUNK_ROWS
    c1 = (row_start + row_count + CHUNK_ROWS - 1) // CHUNK_ROWS
    if c1 <= c0:
        return make_chunk(0, 0)[:0]

    def piece(c):
        rows = min(CHUNK_ROWS, n_rows - c * CHUNK_ROWS)
        lo = max(row_start - c * CHUNK_ROWS, 0)
        hi = min(row_start + row_count - c * CHUNK_ROWS, rows)
        return lo, hi, make_chunk(c, rows)

    if threads <= 1 or c1 - c0 == 1:
        parts = [p[2][p[0]:p[1]] for p in map(piece, range(c0, c1))]
        return np.concatenate(parts) if len(parts) > 1 else parts[0]
    first = piece(c0)
    out = np.empty((row_count,) + first[2].shape[1:], first[2].dtype)

    def place(c, p=None):
        lo, hi, chunk = p if p is not None else piece(c)
        at = c * CHUNK_ROWS + lo - row_start
        out[at:at + hi - lo] = chunk[lo:hi]

    place(c0, first)
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(place, range(c0 + 1, c1)))
    return out


# ------------------------------------------------------------ workloads --

def tiny_dense() -> np.ndarray:
    """4096 x 128 fp32 ~ N(0, 0.1^2), seed 0."""
    rng = np.random.default_rng(0)
    return rng.standard_normal((4096, 128), dtype=np.float32) * np.float32(0.1)


SPARSE_GNN_ROWS, SPARSE_GNN_COLS = 1 << 20, 512


def sparse_gnn_rows(row_start: int = 0, row_count: int | None = None,
                    n_rows: int = SPARSE_GNN_ROWS, threads: int = 1) -> np.ndarray:
    """Bag-of-words features: 1.0 with probability 0.01, else 0.0."""
    if row_count is None:
        row_count = n_rows - row_start

    def make(c, rows):
        rng = np.random.default_rng([0, c])
        u = rng.random((rows, SPARSE_GNN_COLS), dtype=np.float32)
        return (u < np.float32(0.01)).astype(np.float32)
    return _chunked(n_rows, row_start, row_count, make, threads)


def uniform_ids(n_rows: int, batches: int, per_batch: int, seed: int = 1):
    """Row ids drawn uniformly with replacement, [batches, per_batch] int64."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_rows, size=(batches, per_batch), dtype=np.int64)


DENSE_GNN_ROWS, DENSE_GNN_COLS = 1 << 21, 256
DLRM_EMB_ROWS, DLRM_EMB_COLS = 1 << 22, 128


def dense_gnn_rows(row_start: int = 0, row_count: int | None = None,
                   n_rows: int = DENSE_GNN_ROWS, threads: int = 1) -> np.ndarray:
    """Dense node features ~ N(0, 1) * 0.5, fp32."""
    if row_count is None:
        row_count = n_rows - row_start

    def make(c, rows):
        rng = np.random.default_rng([0, c])
        return rng.standard_normal((rows, DENSE_GNN_COLS),
                                   dtype=np.float32) * np.float32(0.5)
    return _chunked(n_rows, row_start, row_count, make, threads)


def dlrm_emb_rows(row_start: int = 0, row_count: int | None = None,
                  n_rows: int = DLRM_EMB_ROWS, threads: int = 1) -> np.ndarray:
    """Embedding table ~ U(-0.05, 0.05), drawn in fp64 and stored as fp32."""
    if row_count is None:
        row_count = n_rows - row_start

    def make(c, rows):
        rng = np.random.default_rng([1, c])
        return rng.uniform(-0.05, 0.05, (rows, DLRM_EMB_COLS)).astype(np.float32)
    return _chunked(n_rows, row_start, row_count, make, threads)


def zipf_ids(n_rows: int, batches: int, per_batch: int, a: float = 1.05,
             seed: int = 1, perm_seed: int = 3) -> np.ndarray:
    """Zipf(a) popularity bounded to ranks 1..n_rows (inverse CDF over
    k^-a), rank mapped to a row id through a fixed random permutation."""
    k = np.arange(1, n_rows + 1, dtype=np.float64)
    cdf = np.cumsum(k ** -a)
    cdf /= cdf[-1]
    rng = np.random.default_rng(seed)
    u = rng.random((batches, per_batch))
    rank = np.minimum(np.searchsorted(cdf, u, side="right"), n_rows - 1)
    perm = np.random.default_rng(perm_seed).permutation(n_rows)
    return perm[rank].astype(np.int64)


def zipf_hot_order(n_rows: int, perm_seed: int = 3) -> np.ndarray:
    """Row ids from most to least popular under zipf_ids (rank order): the
    static popularity a feature cache is filled by (like node degree)."""
    return np.random.default_rng(perm_seed).permutation(n_rows).astype(np.int64)


LLM_LAYERS = 32
LLM_HIDDEN, LLM_FFN = 4096, 14336
LLM_MATRICES = 7  # q, k, v, o as [4096, 4096]; three MLP matrices [4096, 14336]


def llm_weight_shape(j: int):
    return (LLM_HIDDEN, LLM_HIDDEN) if j < 4 else (LLM_HIDDEN, LLM_FFN)


def llm_weight(layer: int, j: int, rows: slice | None = None,
               fp16: bool = False) -> np.ndarray:
    """Matrix j of one layer, bf16 bits (uint16) ~ N(0, 0.02^2); with fp16
    the same draw rounded to IEEE fp16 instead."""
    shape = llm_weight_shape(j)
    rng = np.random.default_rng([0, layer, j])
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    if rows is not None:
        w = w[rows]
    return f32_to_fp16_bits(w) if fp16 else f32_to_bf16_bits(w)


KV_B, KV_H, KV_S, KV_D = 16, 32, 4096, 128
KV_PAGE_TOKENS = 16
KV_PAGES = KV_B * KV_H * (KV_S // KV_PAGE_TOKENS)   # 131,072 pages of 4 KiB


def kv_outlier_channels() -> np.ndarray:
    """[32, 4] channel indices per head (4 outlier channels each)."""
    rng = np.random.default_rng(2)
    return np.stack([rng.choice(KV_D, 4, replace=False) for _ in range(KV_H)])


def llm_kv_batch(b: int, seq: int = KV_S, fp16: bool = False) -> np.ndarray:
    """One batch entry of the KV cache: [32, seq, 128] bf16 bits (uint16).

    Values ~ N(0, 1); the 4 outlier channels of every head are scaled by 20
    before rounding to bf16 (to IEEE fp16 with fp16)."""
    rng = np.random.default_rng([0, b])
    x = rng.standard_normal((KV_H, seq, KV_D), dtype=np.float32)
    ch = kv_outlier_channels()
    for h in range(KV_H):
        x[h][:, ch[h]] *= np.float32(20.0)
    return f32_to_fp16_bits(x) if fp16 else f32_to_bf16_bits(x)


def llm_kv_pages(batches=range(KV_B), seq: int = KV_S, fp16: bool = False,
                 threads: int = 1) -> np.ndarray:
    """KV cache as pages: [n_pages, 16*128] uint16, page id
    (b*32 + h) * (seq/16) + t; each page is contiguous in [B, H, S, D]."""
    def one(b):
        return llm_kv_batch(b, seq, fp16).reshape(-1, KV_PAGE_TOKENS * KV_D)
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(one, batches))
    else:
        parts = [one(b) for b in batches]
    return np.concatenate(parts)


def kv_page_ids(batches: int = 8, n_pages: int = KV_PAGES, seed: int = 1):
    """One permutation of all page ids, split into equal batches."""
    perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int64)
    return perm.reshape(batches, -1)
