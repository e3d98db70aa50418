"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a temporary copy of the oracle's C
source (never in the oracle itself), builds it, and runs the CPU pin suite
against that build through IBP_ORACLE_LIB.  The suite has to fail for every
mutant; a mutant that passes would mean a part of the oracle is unpinned.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ibp_oracle.c")

MUTANTS = {
    "tie_picks_one": ("unsigned majority = ones[b] > zeros ? 1u : 0u;",
                      "unsigned majority = ones[b] >= zeros ? 1u : 0u;"),
    "strict_threshold": ("if (lhs >= rhs) {", "if (lhs > rhs) {"),
    "count_wrong_bit": ("ones[b] += get_bit(sample, i * w + b);",
                        "ones[b] += get_bit(sample, i * w + (b ^ 1));"),
    "header_polarity": ("put_bit(slot, cursor++, (x & mask) == bitval);",
                        "put_bit(slot, cursor++, (x & mask) != bitval);"),
    "payload_msb_first": ("put_bit(buf, pos + b, (unsigned)((v >> b) & 1u));",
                          "put_bit(buf, pos + (w - 1 - b), (unsigned)((v >> b) & 1u));"),
    "flag_rule_le": ("int f = c < row_bytes * 8;", "int f = c <= row_bytes * 8;"),
    "extract_by_mask": ("write_bits(slot, cursor, w - p, orc_pext(x, keep));",
                        "write_bits(slot, cursor, w - p, orc_pext(x, mask));"),
    "size_term_dropped": ("c += match ? (uint64_t)(w - p) : (uint64_t)w;",
                          "c += match ? (uint64_t)(w - p) : (uint64_t)(w - p);"),
    "bitval_not_restored": ("uint64_t x = stripped ? (orc_pdep(v, keep) | bitval) : v;",
                            "uint64_t x = stripped ? orc_pdep(v, keep) : v;"),
    "deposit_off_by_one": ("r |= ((v >> k) & 1u) << b;",
                           "r |= ((v >> (k + 1)) & 1u) << b;"),
    "flag_word_index": ("int f = (int)((flags[(uint64_t)id >> 6] >> ((uint64_t)id & 63)) & 1u);",
                        "int f = (int)((flags[(uint64_t)id >> 6] >> ((uint64_t)id & 31)) & 1u);"),
    "pad_to_byte": ("uint64_t b = ((c_bits + 31) / 32) * 4;",
                    "uint64_t b = (c_bits + 7) / 8;"),
    # per-position metadata
    "positional_first_mask": ("int match = (x & mask[k]) == bitval[k];",
                              "int match = (x & mask[0]) == bitval[0];"),
    "positional_len_neighbour": ("unsigned len = stripped ? w - popcount64(mask[k]) : w;",
                                 "unsigned len = stripped ? w - popcount64(mask[k ? k - 1 : 0]) : w;"),
    "positional_column_shift": ("write_bits(column, r * w, w, read_bits(sample + r * row_bytes, k * w, w));",
                                "write_bits(column, r * w, w, read_bits(sample + r * row_bytes, (k ^ 1) * w, w));"),
}


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation target for {name} not found once"
    path = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib{name}.so")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-shared", "-fPIC", path,
                    "-o", so], check=True)
    env = dict(os.environ, IBP_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                        "-p", "no:cacheprovider", "-k", "not bmi2",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
            res = list(ex.map(lambda kv: _run_mutant(kv[0], *kv[1], tmp),
                              MUTANTS.items()))
    survivors = [n for n, rc in res if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
