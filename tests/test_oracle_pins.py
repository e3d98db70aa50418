"""Pins of the CPU oracle to facts fixed outside the oracle itself.

The IBP explainer page ("Reducing the GPU Memory Bottleneck with Lossless
Compression for ML -- Extended") prints no worked example and no byte
layout, so the oracle is pinned by:
  * a hardware library routine (x86 BMI2 PEXT/PDEP, tests/native/bmi2_pin.c);
  * brute force over every tiny input (width 4 metadata, width 8 codec);
  * hand-derived worked examples (derivations written out below);
  * closed forms: per-row size n + nW - p*m, the sparse-feature image, the
    fp32/bf16/fp16 exponent-bit probabilities of the synthetic
    distributions and the space saved, (p q - 1)/W;
  * special cases that reduce to memcpy / fill / numpy bit packing;
  * round-trip identity on adversarial rows.
All tests here run on the CPU.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction
from itertools import combinations_with_replacement

import numpy as np
import pytest

from oracle import oracle as orc
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def has_bmi2():
    try:
        with open("/proc/cpuinfo") as f:
            return " bmi2" in f.read()
    except OSError:
        return False


# ------------------------------------------------- library routine pin --

@pytest.mark.skipif(not has_bmi2() or shutil.which("gcc") is None,
                    reason="needs gcc and a BMI2 CPU")
def test_bit_primitives_and_width8_codec_against_bmi2():
    so = orc.build()
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "bmi2_pin")
        subprocess.run(["gcc", "-O2", "-mbmi2", "-std=gnu11",
                        os.path.join(ROOT, "tests", "native", "bmi2_pin.c"),
                        so, "-Wl,-rpath," + os.path.dirname(so), "-o", exe],
                       check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bmi2 pin: ok" in r.stdout


# ------------------------------------------------ hand-derived examples --

def test_worked_example_width8():
    """Width 8, Mask 0xF0, Bitval 0x30, row bytes 35 47 3A FF.

    block 0: 0x35 & 0xF0 = 0x30 -> stripped, payload 0x5 (4 bits)
    block 1: 0x47 & 0xF0 = 0x40 -> raw 0x47 (8 bits)
    block 2: 0x3A & 0xF0 = 0x30 -> stripped, payload 0xA (4 bits)
    block 3: 0xFF & 0xF0 = 0xF0 -> raw 0xFF (8 bits)
    header bits (block order, 1 = stripped): 1,0,1,0 -> value 0x5 in bits 0-3
    stream: bits 0-3 = 0x5, 4-7 = 0x5, 8-15 = 0x47, 16-19 = 0xA, 20-27 = 0xFF
    word = 0x0FFA4755 -> bytes 55 47 FA 0F; C = 4+4+8+4+8 = 28 < 32 -> flag 1
    """
    md = orc.Metadata(8, 0xF0, 0x30, 900000)
    slot, c, flag = orc.compress_row(md, np.array([0x35, 0x47, 0x3A, 0xFF], np.uint8))
    assert (c, flag) == (28, 1)
    assert slot.tolist() == [0x55, 0x47, 0xFA, 0x0F]
    back = orc.decompress_row(md, slot, flag)
    assert back.tolist() == [0x35, 0x47, 0x3A, 0xFF]


def test_worked_example_width32_one_unmatched_block():
    """Width 32, Mask 0x7C000000 (exponent bits 30..26), Bitval 0x3C000000.

    32 blocks: block k = 0x3C000000 | k except block 5 = 0x40000000 (2.0f,
    exponent bit 30 set -> no match).  p = 5, payload of a stripped block =
    bits 0..25 of x, then bit 31 at position 26 (27 bits) = k here.
    header word = all ones but bit 5 = 0xFFFFFFDF, C = 32 + 31*27 + 32 = 901.
    payload offsets: k <= 5 at 32 + 27k; block 5 raw at 167 (32 bits);
    k >= 6 at 199 + 27(k - 6).  Stream = 29 words (ceil(901/32)).
    """
    x = np.array([0x3C000000 | k for k in range(32)], np.uint32)
    x[5] = 0x40000000
    md = orc.Metadata(32, 0x7C000000, 0x3C000000, 900000)
    slot, c, flag = orc.compress_row(md, x)
    assert (c, flag) == (901, 1)
    want = 0xFFFFFFDF
    for k in range(32):
        if k < 5:
            want |= k << (32 + 27 * k)
        elif k == 5:
            want |= 0x40000000 << 167
        else:
            want |= k << (199 + 27 * (k - 6))
    got = int.from_bytes(slot[:29 * 4].tobytes(), "little")
    assert got == want
    assert orc.stored_bytes(128, c, flag) == 116
    assert not slot[116:].any()
    assert np.array_equal(orc.decompress_row(md, slot, flag).view(np.uint32), x)


def test_stream_exactly_raw_size_stays_raw():
    """p = 1 and all 32 blocks match: C = 32 + 32*31 = 1024 = 8S, which
    saves nothing, so the row is kept raw (flag 0); with one more invariant
    bit (p = 2) C = 992 < 1024 and the row is stored compressed."""
    x = np.full(32, 0x00000001, np.uint32)
    slot, c, flag = orc.compress_row(orc.Metadata(32, 0x80000000, 0, 0), x)
    assert (c, flag) == (1024, 0) and np.array_equal(slot.view(np.uint32), x)
    slot, c, flag = orc.compress_row(orc.Metadata(32, 0xC0000000, 0, 0), x)
    assert (c, flag) == (992, 1)


def test_lay_example_bit3_always_one():
    """The page's lay summary illustrates the metadata with a data group in
    which bit 3 is always 1.  Random bytes with bit 3 forced on: only bit 3
    is invariant at T = 0.9, with value 1."""
    rng = np.random.default_rng(7)
    x = (rng.integers(0, 256, 4096, dtype=np.uint16).astype(np.uint8) | 0x08)
    md, ones = orc.build_metadata(x, width_bits=8, t=0.9)
    assert md.mask == 0x08 and md.bitval == 0x08
    assert ones[3] == 4096


# ----------------------------------------------------- metadata pins ----

def _pack4(blocks):
    """Width-4 blocks into bytes, block k in bits 4(k%2).. of byte k//2."""
    out = bytearray((len(blocks) + 1) // 2)
    for k, v in enumerate(blocks):
        out[k // 2] |= v << (4 * (k % 2))
    return np.frombuffer(bytes(out), np.uint8)


@pytest.mark.parametrize("t", [Fraction(1, 2), Fraction(3, 4), Fraction(9, 10),
                               Fraction(1)])
def test_metadata_bruteforce_width4(t):
    """Every multiset of 1..4 width-4 blocks, against the definition with
    exact fractions: bit b is invariant iff one value v in {0, 1} holds in
    at least a fraction T of the blocks; a 50/50 tie records v = 0."""
    ppm = int(t * 1_000_000)
    for n in range(1, 5):
        for combo in combinations_with_replacement(range(16), n):
            md, _ = orc.build_metadata(_pack4(combo), width_bits=4, t_ppm=ppm,
                                       n_blocks=n)
            mask = bitval = 0
            for b in range(4):
                k1 = sum((v >> b) & 1 for v in combo)
                k0 = n - k1
                q0, q1 = Fraction(k0, n) >= t, Fraction(k1, n) >= t
                if q0 or q1:
                    mask |= 1 << b
                    # when both values qualify (T <= 1/2) the more frequent
                    # one is recorded, 0 on an exact tie
                    if q1 and (not q0 or k1 > k0):
                        bitval |= 1 << b
            assert (md.mask, md.bitval) == (mask, bitval), (combo, t)


def test_metadata_threshold_boundary_exact():
    """N = 10 blocks, bit 0 set in exactly 9: 9/10 >= 0.9 qualifies (the
    comparison is >=), 900001 ppm does not; 8 of 10 does not qualify."""
    nine = np.array([1] * 9 + [0], np.uint8)
    assert orc.build_metadata(nine, 8, t_ppm=900000)[0].mask & 1 == 1
    assert orc.build_metadata(nine, 8, t_ppm=900000)[0].bitval & 1 == 1
    assert orc.build_metadata(nine, 8, t_ppm=900001)[0].mask & 1 == 0
    eight = np.array([1] * 8 + [0] * 2, np.uint8)
    assert orc.build_metadata(eight, 8, t_ppm=900000)[0].mask & 1 == 0
    assert orc.build_metadata(eight, 8, t_ppm=800000)[0].mask & 1 == 1


def test_metadata_tie_and_zero_threshold():
    """A 50/50 tie qualifies only when T <= 0.5 and records 0; T = 0 marks
    every bit, each with its majority value."""
    half = np.array([0xFF, 0x00, 0xF0, 0x0F], np.uint8)  # every bit: 2 of 4
    md, _ = orc.build_metadata(half, 8, t_ppm=500000)
    assert (md.mask, md.bitval) == (0xFF, 0x00)
    md, _ = orc.build_metadata(half, 8, t_ppm=500001)
    assert md.mask == 0
    three = np.array([0x81, 0x81, 0x80, 0x01], np.uint8)
    md, _ = orc.build_metadata(three, 8, t_ppm=0)
    assert (md.mask, md.bitval) == (0xFF, 0x81)


@pytest.mark.parametrize("w,dt", [(32, np.uint32), (64, np.uint64)])
def test_metadata_single_block_and_t1(w, dt):
    """N = 1: every bit is invariant and Bitval is the block.  T = 1: Mask is
    exactly the set of bits constant over the sample (bitwise AND == OR)."""
    rng = np.random.default_rng(3)
    one = rng.integers(0, np.iinfo(dt).max, 1, dtype=dt, endpoint=True)
    md, _ = orc.build_metadata(one, w, t=0.9)
    full = (1 << w) - 1
    assert md.mask == full and md.bitval == int(one[0])
    x = rng.integers(0, np.iinfo(dt).max, 5000, dtype=dt, endpoint=True)
    x = (x & dt(0x00FF00FF00FF00FF & full)) | dt(0x1200340056007800 & full)
    md, _ = orc.build_metadata(x, w, t=1.0)
    a, o = int(np.bitwise_and.reduce(x)), int(np.bitwise_or.reduce(x))
    const = ~(a ^ o) & full
    assert md.mask == const and md.bitval == (a & const)


def _binade_bit_prob(cdf_abs, exp_bits, mant_bits, bit, bias):
    """P(bit `bit` of the exponent field is 1) for a float whose |x| has
    CDF cdf_abs, summing P(2^(E-bias) <= |x| < 2^(E-bias+1)) over the
    exponent values E with that bit set (zeros/denormals have E = 0)."""
    tot = 0.0
    for e in range(1, (1 << exp_bits) - 1):
        if (e >> bit) & 1:
            lo, hi = 2.0 ** (e - bias), 2.0 ** (e - bias + 1)
            tot += cdf_abs(hi) - cdf_abs(lo)
    return tot


# (exponent bits, mantissa bits, bias) of the float formats
_FMT = {"f32": (8, 23, 127), "bf16": (8, 7, 127), "f16": (5, 10, 15)}


def _predicted_mask(cdf_abs, w_field, t=0.9, n=None, fmt=None):
    """Predicted Mask/Bitval for the sign+exponent bits of fp32 (w_field=32)
    or of each bf16 half (w_field=16; fmt="f16" for IEEE fp16 halves), plus
    the bits whose majority margin is too close to T to predict with n
    samples."""
    fmt = fmt or ("f32" if w_field == 32 else "bf16")
    exp_bits, mant, bias = _FMT[fmt]
    mask = val = 0
    unsure = 0
    for j in range(exp_bits):
        p1 = _binade_bit_prob(cdf_abs, exp_bits, mant, j, bias)
        maj = max(p1, 1 - p1)
        pos = mant + j
        sigma = (maj * (1 - maj) / n) ** 0.5 if n else 0.0
        if abs(maj - t) < 6 * sigma + 1e-3:
            unsure |= 1 << pos
        if maj >= t:
            mask |= 1 << pos
            if p1 > 0.5:
                val |= 1 << pos
    return mask, val, unsure


def test_metadata_matches_distribution_tiny_dense():
    """N(0, 0.1^2) fp32: exponent bits 30..26 are invariant (bit 26 is 1 for
    |x| >= 2^-7, probability 0.938); sign and mantissa bits are not."""
    from scipy.stats import norm
    x = syn.tiny_dense()
    md, ones = orc.build_metadata(x, 32, t=0.9)
    n = x.size
    cdf = lambda a: 2 * norm.cdf(a / 0.1) - 1
    mask, val, unsure = _predicted_mask(cdf, 32, n=n)
    assert unsure == 0
    assert (md.mask, md.bitval) == (mask, val) == (0x7C000000, 0x3C000000)
    p26 = _binade_bit_prob(cdf, 8, 23, 3, 127)
    sig = (p26 * (1 - p26) / n) ** 0.5
    assert abs(ones[26] / n - p26) < 5 * sig


@pytest.mark.parametrize("name", ["dense_gnn", "dlrm_emb", "llm_weights", "llm_kv",
                                  "llm_weights_fp16", "llm_kv_fp16"])
def test_metadata_matches_distribution_configs(name):
    """Predicted Mask/Bitval of the other synthetic workloads from their
    CDFs, on a 2^20-block sample (first rows in storage order).  Stored as
    IEEE fp16 (5 exponent bits, bias 15), the weights keep only the top
    exponent bit invariant (0: |x| < 2), the KV values also the next one."""
    from scipy.stats import norm
    fmt = "f16" if name.endswith("_fp16") else None
    if name == "llm_weights_fp16":
        x, w = syn.llm_weight(0, 0, rows=slice(0, 512), fp16=True), 16
        cdf = lambda a: 2 * norm.cdf(a / 0.02) - 1
    elif name == "llm_kv_fp16":
        x, w = syn.llm_kv_batch(0, seq=256, fp16=True).reshape(-1), 16
        f = 4 / 128
        cdf = lambda a: (1 - f) * (2 * norm.cdf(a) - 1) + f * (2 * norm.cdf(a / 20) - 1)
    elif name == "dense_gnn":
        x, w = syn.dense_gnn_rows(0, 4096), 32
        cdf = lambda a: 2 * norm.cdf(a / 0.5) - 1
    elif name == "dlrm_emb":
        x, w = syn.dlrm_emb_rows(0, 8192), 32
        cdf = lambda a: min(a / 0.05, 1.0)
    elif name == "llm_weights":
        x, w = syn.llm_weight(0, 0, rows=slice(0, 512)), 16
        cdf = lambda a: 2 * norm.cdf(a / 0.02) - 1
    else:
        x, w = syn.llm_kv_batch(0, seq=256)[:, :, :].reshape(-1), 16
        f = 4 / 128
        cdf = lambda a: (1 - f) * (2 * norm.cdf(a) - 1) + f * (2 * norm.cdf(a / 20) - 1)
    md, _ = orc.build_metadata(x, 32, t=0.9)
    n = x.nbytes // 4
    mask, val, unsure = _predicted_mask(cdf, w, n=n, fmt=fmt)
    if w == 16:  # both 16-bit halves of a 32-bit block share the prediction
        mask, val, unsure = (mask | mask << 16, val | val << 16,
                             unsure | unsure << 16)
    assert unsure == 0
    assert (md.mask, md.bitval) == (mask, val)
    expected = {"dense_gnn": (0x7C000000, 0x3C000000),
                "dlrm_emb": (0x78000000, 0x38000000),
                "llm_weights": (0x78007800, 0x38003800),
                "llm_kv": (0x7C007C00, 0x3C003C00),
                "llm_weights_fp16": (0x40004000, 0x00000000),
                "llm_kv_fp16": (0x60006000, 0x20002000)}[name]
    assert (md.mask, md.bitval) == expected


def _match_prob(cdf_abs, mask_e, val_e, fmt, rounded):
    """P((v & mask_e) == val_e) for one float v whose |x| has CDF cdf_abs,
    when mask_e covers exponent bits only: the sum of P(|v| in binade E)
    over the exponent values E that agree with val_e under the mask (E = 0:
    zero and subnormals).  For 16-bit values rounded from a continuous x
    (nearest, ties to even), |v| reaches 2^k once |x| passes 2^k less half
    a step, 2^k (1 - 2^-(mantissa bits + 2))."""
    exp_bits, mant, bias = _FMT[fmt]
    assert mask_e & ((1 << mant) - 1) == 0 and mask_e >> (mant + exp_bits) == 0
    adj = 1.0 - 2.0 ** -(mant + 2) if rounded else 1.0
    q = 0.0
    for e in range((1 << exp_bits) - 1):
        if ((e << mant) & mask_e) != val_e:
            continue
        lo = 0.0 if e == 0 else 2.0 ** (e - bias) * adj
        hi = 2.0 ** (e + 1 - bias) * adj
        q += cdf_abs(hi) - cdf_abs(lo)
    return q


def _page_savings():
    """tests/golden/page_savings.txt: class -> (low, high) percent."""
    bands = {}
    with open(os.path.join(ROOT, "tests", "golden", "page_savings.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                bands[line[0]] = (float(line[1]), float(line[2]))
    return bands


@pytest.mark.parametrize("name,w", [("tiny_dense", 32), ("dense_gnn", 32), ("dlrm_emb", 32),
                                    ("llm_weights", 32), ("llm_kv", 32),
                                    ("llm_weights_fp16", 32), ("llm_kv_fp16", 32),
                                    ("llm_kv_fp16", 16)])
def test_savings_closed_form_and_page_bands(name, w):
    """Space saved by the oracle's image against a number computed without
    it.  Every row of these tables is stored compressed, so its stored bits
    are n(1 + W) - p m: the saving is (p q - 1) / W, where q, the chance that
    a block matches Bitval under Mask, follows from the distribution the
    table is drawn from (for a bf16 block, both halves must match).  A lost
    header bit or a wrong p moves the saving by 1/32 or more, ~100 sigma
    here.  The result is then held to the savings the IBP page reports for
    real data of the same kind (Results section), within 1.5 points: the
    tables are synthetic stand-ins, not the page's datasets.  The page gives
    no figure for fp16 tables, which are held to the closed form only."""
    from scipy.stats import norm
    gauss = lambda s: (lambda a: 2 * norm.cdf(a / s) - 1)
    fp16 = name.endswith("_fp16")
    fmt16 = "f16" if fp16 else "bf16"

    def pair(q_elem):
        """Per 32-bit block of two 16-bit values: both must match (at W =
        16 a block is one value)."""
        def q_of(m, v):
            if w == 16:
                return q_elem(m, v)
            assert m >> 16 == m & 0xFFFF and v >> 16 == v & 0xFFFF
            return q_elem(m & 0xFFFF, v & 0xFFFF) ** 2
        return q_of

    if name == "tiny_dense":
        x, cls = syn.tiny_dense(), "dense_fp32"
        q_of = lambda m, v: _match_prob(gauss(0.1), m, v, "f32", False)
    elif name == "dense_gnn":
        x, cls = syn.dense_gnn_rows(0, 4096), "dense_fp32"
        q_of = lambda m, v: _match_prob(gauss(0.5), m, v, "f32", False)
    elif name == "dlrm_emb":
        x, cls = syn.dlrm_emb_rows(0, 8192), "dlrm_fp32"
        q_of = lambda m, v: _match_prob(lambda a: min(a / 0.05, 1.0), m, v, "f32", False)
    elif name.startswith("llm_weights"):
        x, cls = syn.llm_weight(0, 0, rows=slice(0, 512), fp16=fp16), "bf16_llm"
        q_of = pair(lambda m, v: _match_prob(gauss(0.02), m, v, fmt16, True))
    else:
        x, cls = syn.llm_kv_pages(batches=[0], seq=256, fp16=fp16), "bf16_llm"

        def q_of(m, v):
            halves = [(m, v)] if w == 16 else [(m >> 16, v >> 16), (m & 0xFFFF, v & 0xFFFF)]
            assert all(h == halves[0] for h in halves)
            q1 = _match_prob(gauss(1.0), *halves[0], fmt16, True)
            q20 = _match_prob(gauss(20.0), *halves[0], fmt16, True)
            # every head owns the same number of pages; a 32-bit block of a
            # page holds channels 2k and 2k + 1 of one token, a 16-bit one
            # a single channel
            tot = 0.0
            for ch in syn.kv_outlier_channels():
                out = np.zeros(syn.KV_D, bool)
                out[ch] = True
                qc = np.where(out, q20, q1)
                tot += float(np.mean(qc if w == 16 else qc[0::2] * qc[1::2]))
            return tot / syn.KV_H
    md, _ = orc.build_metadata(x, w, t=0.9)
    p = md.invariant_bits
    q = q_of(md.mask, md.bitval)
    _, flags, row_bits = orc.compress(md, x)
    rows = x.shape[0]
    n = x.nbytes // rows * 8 // w
    assert all(bool(int(flags[r >> 6]) >> (r & 63) & 1) for r in range(rows))
    blocks = rows * n
    saved = 1.0 - float(row_bits.astype(np.float64).sum()) / (blocks * w)
    predicted = (p * q - 1.0) / w
    sigma = p * (q * (1 - q) / blocks) ** 0.5 / w
    assert abs(saved - predicted) < 5 * sigma + 1e-6, (saved, predicted, sigma)
    if not fp16:
        lo, hi = _page_savings()[cls]
        assert lo - 1.5 <= 100 * saved <= hi + 1.5, (name, 100 * saved, lo, hi)


# ------------------------------------------------------- layout pins ----

def _numpy_stream(x_rows_u8, w, mask, bitval):
    """Expected stream bytes of each row from the format's definition,
    assembled with numpy bit matrices: header = match bits in block order,
    then per block its bits at the non-invariant positions in ascending
    order (all W bits for a raw block), LSB first, zero padded to 32 bits."""
    n_rows, S = x_rows_u8.shape
    n = S * 8 // w
    bits = np.unpackbits(x_rows_u8, axis=1, bitorder="little").reshape(n_rows, n, w)
    mbits = np.array([(mask >> b) & 1 for b in range(w)], bool)
    vbits = np.array([(bitval >> b) & 1 for b in range(w)], np.uint8)
    out = []
    for r in range(n_rows):
        match = np.all(bits[r][:, mbits] == vbits[mbits], axis=1)
        parts = [match.astype(np.uint8)]
        for k in range(n):
            parts.append(bits[r, k][~mbits] if match[k] else bits[r, k])
        s = np.concatenate(parts)
        c = s.size
        s = np.concatenate([s, np.zeros((-c) % 32, np.uint8)])
        out.append((np.packbits(s, bitorder="little"), c, int(match.sum())))
    return out


@pytest.mark.parametrize("w,S,mask,bitval", [
    (32, 148, 0x7C000000, 0x3C000000),   # n = 37: ragged header
    (32, 512, 0x78007800, 0x38003800),
    (32, 64, 0xFFFFFFFF, 0x00000000),
    (32, 256, 0x80F0000F, 0x00A00005),   # scattered invariant bits
    (16, 96, 0x7C00, 0x3C00),
    (8, 40, 0xF0, 0x30),
    (64, 256, 0x7FF0000000000000, 0x3FF0000000000000),
    (4, 9, 0xC, 0x4),
])
def test_stream_layout_against_numpy_bitmatrix(w, S, mask, bitval):
    rng = np.random.default_rng(w * 1000 + S)
    n_rows = 70
    x = rng.integers(0, 256, (n_rows, S), dtype=np.uint16).astype(np.uint8)
    # force most blocks to match so that compressed rows exist
    xb = np.unpackbits(x, axis=1, bitorder="little").reshape(n_rows, -1, w)
    force = rng.random(xb.shape[:2]) < 0.85
    for b in range(w):
        if (mask >> b) & 1:
            xb[:, :, b] = np.where(force, (bitval >> b) & 1, xb[:, :, b])
    x = np.packbits(xb.reshape(n_rows, -1), axis=1, bitorder="little")
    x[3] = 0xFF   # an all-ones row (matches only if Bitval covers it)
    md = orc.Metadata(w, mask, bitval, 900000)
    slots, flags, row_bits = orc.compress(md, x)
    p = bin(mask).count("1")
    n = S * 8 // w
    exp = _numpy_stream(x, w, mask, bitval)
    n_flag1 = 0
    for r in range(n_rows):
        stream, c, m = exp[r]
        assert row_bits[r] == c == n + n * w - p * m          # closed form
        f = int((int(flags[r >> 6]) >> (r & 63)) & 1)
        assert f == int(c < 8 * S)
        if f:
            n_flag1 += 1
            nb = orc.stored_bytes(S, c, 1)
            assert nb == min(S, 4 * ((c + 31) // 32))
            assert np.array_equal(slots[r, :nb], stream[:nb])
            hdr = np.unpackbits(slots[r], bitorder="little")[:n]
            assert hdr.sum() == m
        else:
            assert np.array_equal(slots[r], x[r])
    assert n_flag1 > 0
    assert int(flags[-1]) >> (n_rows - 64 * (len(flags) - 1)) == 0  # tail bits
    assert np.array_equal(orc.decompress(md, slots, flags), x)


def test_zero_invariant_bits_is_a_copy():
    """p = 0: every stream is n bits longer than the row, so every row is
    stored raw and the image is a byte copy of the input."""
    x = syn.tiny_dense()[:100]
    md = orc.Metadata(32, 0, 0, 900000)
    slots, flags, row_bits = orc.compress(md, x)
    assert not flags.any()
    assert np.array_equal(slots, x.view(np.uint8))
    assert (row_bits == 128 + 128 * 32).all()


def test_all_invariant_constant_rows_is_a_fill():
    """Mask = all ones and every block equal to Bitval: C = n, the stream is
    the all-ones header, and decompression is a fill with Bitval."""
    md = orc.Metadata(32, 0xFFFFFFFF, 0x3F800000, 900000)
    x = np.full((5, 96), 0x3F800000, np.uint32)
    slots, flags, row_bits = orc.compress(md, x)
    assert (row_bits == 96).all() and flags[0] == 0b11111
    assert (slots[:, :12] == 0xFF).all()
    assert np.array_equal(orc.decompress(md, slots, flags).view(np.uint32), x)


def test_sparse_features_image_closed_form():
    """Sparse 0/1 fp32 features: Mask = all ones, Bitval = 0 (0.0 covers 99%
    of blocks).  A row's stream is its header (bit k = 1 iff entry k is 0.0)
    followed by one word 0x3F800000 per 1.0 entry, in column order."""
    x = syn.sparse_gnn_rows(0, 2048)
    md, _ = orc.build_metadata(x, 32, t=0.9)
    assert (md.mask, md.bitval) == (0xFFFFFFFF, 0)
    slots, flags, row_bits = orc.compress(md, x)
    for r in range(x.shape[0]):
        hdr = np.packbits(x[r] == 0, bitorder="little")
        body = np.full(int((x[r] != 0).sum()), 0x3F800000, np.uint32).view(np.uint8)
        want = np.concatenate([hdr, body])
        assert np.array_equal(slots[r, :want.size], want)
        assert row_bits[r] == 512 + 32 * (x[r] != 0).sum()
    assert flags.all() or np.all(flags == np.uint64(0xFFFFFFFFFFFFFFFF))


def test_round_trip_adversarial_rows():
    rng = np.random.default_rng(11)
    rows = [
        rng.integers(0, 256, 512, dtype=np.uint16).astype(np.uint8),  # random
        np.zeros(512, np.uint8),
        np.full(512, 0xFF, np.uint8),
        np.full(128, 0x7FC00001, np.uint32).view(np.uint8),          # NaNs
        np.tile(np.array([0x55, 0xAA], np.uint8), 256),
        np.full(128, 0x3C000001, np.uint32).view(np.uint8),
    ]
    one_off = np.full(128, 0x3C000001, np.uint32)
    one_off[77] = 0xFFFFFFFF
    rows.append(one_off.view(np.uint8))
    neg0 = np.full(128, 0x80000000, np.uint32)                        # -0.0
    rows.append(neg0.view(np.uint8))
    x = np.stack(rows)
    for w in (4, 8, 16, 32, 64):
        for mask, bitval in [(0x7C000000, 0x3C000000), (0xFFFFFFFF, 0),
                             (0x80000000, 0x80000000), (0, 0), (0x5, 0x4)]:
            mask &= (1 << w) - 1
            bitval &= mask
            md = orc.Metadata(w, mask, bitval, 900000)
            slots, flags, _ = orc.compress(md, x)
            assert np.array_equal(orc.decompress(md, slots, flags), x)


def test_gather_order_duplicates_and_empty():
    x = syn.tiny_dense()[:300]
    md, _ = orc.build_metadata(x, 32, t=0.9)
    slots, flags, _ = orc.compress(md, x)
    ids = np.array([299, 0, 5, 5, 299, 64, 63], np.int64)
    out = orc.gather_decompress(md, slots, flags, ids)
    assert np.array_equal(out.view(np.float32), x[ids])
    assert orc.gather_decompress(md, slots, flags, ids[:0]).shape == (0, 512)
    with pytest.raises(ValueError):
        orc.gather_decompress(md, slots, flags, np.array([300]))


# ------------------------------------------------------------ packed cache --

def test_cache_pack_round_trip_and_layout():
    """The packed cache (cache compression of the page's System integration):
    each entry, put back in a slot, decodes to its source row with the page's
    decoder; entries tile the arena in id order at 16-byte boundaries with
    zero padding; the stored words follow the closed form C = n + nW - p*m
    with m counted by numpy; out-of-table ids get nothing."""
    rng = np.random.default_rng(21)
    mask, bitval = 0x7C000000, 0x3C000000
    md = orc.Metadata(32, mask, bitval, 900000)
    for S in (512, 148, 8):
        n = S // 4
        x = rng.standard_normal((40, n)).astype(np.float32).view(np.uint32)
        x[3] = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)  # raw row
        slots, flags, rb = orc.compress(md, x)
        ids = np.array([5, 3, 39, -1, 5, 40, 0, 17, 2**40], np.int64)
        locs, arena = orc.cache_pack(slots, flags, rb, ids)
        m = ((x & np.uint32(mask)) == np.uint32(bitval)).sum(1)
        c = n + 32 * n - 5 * m
        end = 0
        for e, r in enumerate(ids):
            loc = int(locs[e])
            if not 0 <= r < 40:
                assert loc == 0
                continue
            comp = bool(loc & orc.LOC_COMPRESSED)
            words = (loc >> orc.LOC_WORDS_SHIFT) & orc.LOC_WORDS_MASK
            at = (loc & orc.LOC_OFFSET_MASK) * 16
            assert loc & orc.LOC_RESIDENT and at == end
            assert comp == (c[r] < 32 * n)
            assert words == ((c[r] + 31) // 32 if comp else n)
            end = at + (words * 4 + 15) // 16 * 16
            assert not arena[at + words * 4:end].any()
            slot = np.zeros(S, np.uint8)
            slot[:words * 4] = arena[at:at + words * 4]
            assert np.array_equal(orc.decompress_row(md, slot, int(comp)),
                                  x[r].view(np.uint8)), (S, r)
        assert end == arena.size
        # the table's locators (one entry per row) and the gather through them
        cache_loc = np.zeros(40, np.uint64)
        for e, r in enumerate(ids):
            if 0 <= r < 40:
                cache_loc[r] = locs[e]
        q = np.array([5, 6, 3, -7, 39, 0, 40, 17, 17, 1], np.int64)
        want = np.zeros((q.size, S), np.uint8)
        for i, r in enumerate(q):
            if 0 <= r < 40:
                want[i] = x[r].view(np.uint8)
        assert np.array_equal(orc.cache_gather(md, arena, cache_loc, slots, flags, q), want)


def test_cache_locator_constants_match_header():
    """The oracle's locator layout is the one include/ibp.h declares."""
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "include", "ibp.h")).read()
    vals = {k: eval(v.replace("ull", ""), {}) for k, v in
            re.findall(r"#define (IBP_LOC_[A-Z_]+) (.+)", text)}
    assert vals == {"IBP_LOC_RESIDENT": orc.LOC_RESIDENT,
                    "IBP_LOC_COMPRESSED": orc.LOC_COMPRESSED,
                    "IBP_LOC_WORDS_SHIFT": orc.LOC_WORDS_SHIFT,
                    "IBP_LOC_WORDS_MASK": orc.LOC_WORDS_MASK,
                    "IBP_LOC_OFFSET_MASK": orc.LOC_OFFSET_MASK}


# ------------------------------------------------- per-position metadata --

def test_positional_worked_example_width8():
    """Two 8-bit blocks with their own masks, stream derived by hand:
    block 0 = 0x55 under Mask 0xF0 / Bitval 0x50 keeps its low nibble 0x5,
    block 1 = 0xF0 under Mask 0x0F / Bitval 0x00 keeps its high nibble 0xF.
    Header bits 1,1; payload 0101 (LSB first) at bits 2-5; 1111 at bits 6-9:
    C = 10 bits, bytes 0xD7 0x03."""
    pm = orc.PositionalMetadata(8, np.array([0xF0, 0x0F], np.uint64),
                                np.array([0x50, 0x00], np.uint64))
    row = np.array([0x55, 0xF0], np.uint8)
    slot, c, f = orc.compress_row_positional(pm, row)
    assert (c, f) == (10, 1) and list(slot) == [0xD7, 0x03]
    slots, flags, _ = orc.compress_positional(pm, row[None])
    assert np.array_equal(orc.decompress_positional(pm, slots, flags)[0], row)


@pytest.mark.parametrize("w", [8, 16, 32, 64])
def test_positional_with_equal_masks_is_the_global_image(w):
    """The same Mask/Bitval at every position gives the global image byte for
    byte (the global codec is pinned above)."""
    rng = np.random.default_rng(w)
    for _ in range(6):
        mask = int(rng.integers(0, 2**63)) & ((1 << w) - 1) if w < 64 else int(rng.integers(0, 2**63)) << 1
        bitval = mask & int(rng.integers(0, 2**63))
        S = w // 8 * int(rng.integers(1, 40))
        x = rng.integers(0, 256, (30, S), dtype=np.uint8)
        blocks = x.view({8: np.uint8, 16: np.uint16, 32: np.uint32, 64: np.uint64}[w])
        force = rng.random(blocks.shape) < 0.8
        blocks[force] = (blocks[force] & blocks.dtype.type(~mask & ((1 << w) - 1))) | \
            blocks.dtype.type(bitval)
        n = S * 8 // w
        pm = orc.PositionalMetadata(w, np.full(n, mask, np.uint64), np.full(n, bitval, np.uint64))
        g = orc.compress(orc.Metadata(w, mask, bitval, 900000), x)
        q = orc.compress_positional(pm, x)
        for a, b in zip(g, q):
            assert np.array_equal(a, b)


def test_positional_metadata_is_the_rule_per_column():
    """Per-position metadata against numpy column counts and the threshold
    rule in exact fractions (majority, ties to 0, count/N >= T)."""
    rng = np.random.default_rng(3)
    n_rows, n = 157, 24
    dens = rng.random((1, n, 32)) ** 3            # per position and bit
    dens[0, 5] = 0.5                              # exact ties at one position
    bits = rng.random((n_rows, n, 32)) < dens
    bits[:, 7] = False                            # a constant-zero column
    x = (bits.astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(2).astype(np.uint32)
    if n_rows % 2 == 0:
        x[0, 5] ^= 1
    ones = bits.sum(0)                            # [n, 32]
    for t_ppm in (500000, 900000, 1000000):
        pm = orc.build_metadata_positional(x, 32, t_ppm=t_ppm)
        T = Fraction(t_ppm, 1000000)
        for k in range(n):
            m = bv = 0
            for b in range(32):
                o = int(ones[k, b])
                z = n_rows - o
                maj = 1 if o > z else 0
                if Fraction(max(o, z), n_rows) >= T:
                    m |= 1 << b
                    bv |= maj << b
            assert (int(pm.mask[k]), int(pm.bitval[k])) == (m, bv), (t_ppm, k)


@pytest.mark.parametrize("w", [8, 32, 64])
def test_positional_sizes_closed_form_and_round_trip(w):
    """Masks that differ per position, including none (p = 0) and all (p = W):
    C = n + sum over blocks of (W - p_k if matched else W), with matches
    counted by numpy; every row decodes back; raw rows stay raw."""
    rng = np.random.default_rng(100 + w)
    dt = {8: np.uint8, 32: np.uint32, 64: np.uint64}[w]
    n = 37
    full = (1 << w) - 1
    masks = [int(rng.integers(0, 2**63)) & full for _ in range(n)]
    masks[0], masks[1] = 0, full
    bitvals = [m & int(rng.integers(0, 2**63)) for m in masks]
    x = rng.integers(0, 256, (60, n * w // 8), dtype=np.uint8).view(dt)
    force = rng.random(x.shape) < 0.9
    for k in range(n):
        col = x[:, k]
        col[force[:, k]] = (col[force[:, k]] & dt(~masks[k] & full)) | dt(bitvals[k])
    x[3] = rng.integers(0, 256, n * w // 8, dtype=np.uint8).view(dt)   # likely raw
    pm = orc.PositionalMetadata(w, np.array(masks, np.uint64), np.array(bitvals, np.uint64))
    slots, flags, rb = orc.compress_positional(pm, x)
    p = np.array([bin(m).count("1") for m in masks])
    match = (x & np.array(masks, np.uint64).astype(dt)) == np.array(bitvals, np.uint64).astype(dt)
    c = n + np.where(match, w - p, w).sum(1)
    assert np.array_equal(rb, c.astype(np.uint64))
    fl = [(int(flags[r >> 6]) >> (r & 63)) & 1 for r in range(60)]
    assert fl == [int(v < n * w) for v in c]
    assert np.array_equal(orc.decompress_positional(pm, slots, flags), x.view(np.uint8))


def test_positional_bruteforce_width4():
    """W = 4, rows of two blocks: random per-position (Mask, Bitval) pairs,
    every one of the 256 rows, round trip and C against direct counting."""
    rng = np.random.default_rng(4)
    rows = np.arange(256, dtype=np.uint8)[:, None]
    for _ in range(300):
        m = [int(v) for v in rng.integers(0, 16, 2)]
        b = [m[i] & int(rng.integers(0, 16)) for i in range(2)]
        pm = orc.PositionalMetadata(4, np.array(m, np.uint64), np.array(b, np.uint64))
        slots, flags, rb = orc.compress_positional(pm, rows)
        assert np.array_equal(orc.decompress_positional(pm, slots, flags), rows)
        for v in range(256):
            blk = [v & 15, v >> 4]
            c = 2 + sum(4 - bin(m[k]).count("1") if (blk[k] & m[k]) == b[k] else 4
                        for k in range(2))
            assert int(rb[v]) == c
