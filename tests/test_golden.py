"""Pins of the oracle's packed format against numbers the pages print.

tests/golden/decode_v2_linear_bench.tsv holds the per-launch bench table of the
deep-fold "Decode V2" page (section 6, Linear primitive).  The page defines
its GB/s column as packed codes + scales + x over the median time, so every
row fixes the bytes one GEMV reads.  The oracle's own packing of one row of
each K (codes bytes + 2 bytes per scale), times M, plus a bf16 x, must
reproduce all 13 printed GB/s values within the rounding of the printed
figures.  A format with another group size, scale width or activation width
misses at least one row (checked below), so this pins the 4-bit code plane,
the fp16 scale per 64 weights and the bf16 activation.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "decode_v2_linear_bench.tsv")


def _rows():
    out = []
    with open(GOLDEN) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            kind, M, K, us, gbs = line.split("\t")
            out.append((kind, int(M), int(K), float(us), float(gbs)))
    return out


def _consistent(nbytes, us, gbs):
    """Whether nbytes / us reproduces the printed GB/s, given that us and
    GB/s are printed to 0.1."""
    lo = nbytes / (us + 0.05) / 1e3
    hi = nbytes / (us - 0.05) / 1e3
    return lo - 0.05 <= gbs <= hi + 0.05


def _oracle_row_bytes(oracle_mod, K):
    """Bytes one packed row of K weights takes in the oracle's format."""
    w = np.random.default_rng(K).standard_normal((1, K)).astype(np.float32) * 0.02
    codes, scales, st = oracle_mod.pack(w)
    assert st == 0
    return codes.nbytes + scales.nbytes


def test_golden_table_has_the_pages_13_rows():
    rows = _rows()
    assert len(rows) == 13
    assert {r[0] for r in rows} >= {"down_proj", "lm_head", "gate_proj"}


@pytest.mark.parametrize("row", _rows(), ids=lambda r: r[0])
def test_oracle_format_reproduces_printed_gbs(oracle_mod, row):
    kind, M, K, us, gbs = row
    nbytes = M * _oracle_row_bytes(oracle_mod, K) + 2 * K  # codes + scales + bf16 x
    assert _consistent(nbytes, us, gbs), (kind, nbytes / us / 1e3, gbs)


@pytest.mark.parametrize("variant", [
    ("fp32 scale per 64", lambda M, K: M * K // 2 + M * K // 16 + 2 * K),
    ("fp16 scale per 32", lambda M, K: M * K // 2 + M * K // 16 + 2 * K),
    ("fp16 scale per 128", lambda M, K: M * K // 2 + M * K // 64 + 2 * K),
    ("fp32 x", lambda M, K: M * K // 2 + M * K // 32 + 4 * K),
    ("y counted too", lambda M, K: M * K // 2 + M * K // 32 + 2 * K + 4 * M),
], ids=lambda v: v[0])
def test_other_formats_miss_some_row(variant):
    _, nbytes = variant
    misses = [r[0] for r in _rows() if not _consistent(nbytes(r[1], r[2]), r[3], r[4])]
    assert misses, "the table would not distinguish this format"
