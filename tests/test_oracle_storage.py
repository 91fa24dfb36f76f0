"""Pins for the bit split and the storage formula against the memory figures
the pages print (see tests/golden/page_ratios.txt for the citations)."""
import numpy as np
import pytest

import oracle
from conftest import read_golden


def test_split_bits():
    assert oracle.split_bits(3.5) == (3, 4)
    assert oracle.split_bits(4) == (4, 4)
    assert oracle.split_bits(4.0) == (4, 4)
    assert oracle.split_bits(2.5) == (2, 3)
    # floor/ceil taken literally for non-half fractions
    assert oracle.split_bits(4.2) == (4, 5)


def test_row_words():
    assert oracle.row_words(128, 3) == 12
    assert oracle.row_words(128, 4) == 16
    assert oracle.row_words(64, 3) == 6
    assert oracle.row_words(64, 4) == 8
    assert oracle.row_words(32, 5) == 5
    assert oracle.row_words(32, 1) == 1


def test_bytes_per_token_head():
    # 3-bit K + 4-bit V at d=128: (48 + 4) + (64 + 4) = 120 bytes
    assert oracle.bytes_per_token_head(128, 3) + oracle.bytes_per_token_head(128, 4) == 120


def test_page_memory_figures():
    d = 128
    fp16 = 2 * d
    for row in read_golden("page_ratios.txt"):
        name, kb, vb, side, val, tol = row.split()
        kb, vb, val, tol = int(kb), int(vb), float(val), float(tol)
        if side == "kv":
            ours = oracle.bytes_per_token_head(d, kb) + oracle.bytes_per_token_head(d, vb)
            base = 2 * fp16
        else:
            ours = oracle.bytes_per_token_head(d, vb)
            base = fp16
        ratio = base / ours
        if name == "reduction_3p5":
            assert abs((1 - ours / base) - val) <= tol, 1 - ours / base
        elif name == "ratio_3p5_low":
            assert ratio >= val
        elif name == "ratio_3p5_high":
            assert ratio <= val
        else:
            assert abs(ratio - val) <= tol, (name, ratio)
