"""Byte counts printed on the pages, recomputed from the per-row storage sizes
(tests/golden/page_sizes.txt holds the printed figures with their citations)."""
import os

import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.txt")
UNIT = {"KiB": 2**10, "MiB": 2**20, "GiB": 2**30}


def rows():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fields, cite = line.split("|", 1)
        layers, heads, D, tK, tV, tokens, value, unit = fields.split()
        out.append((int(layers), int(heads), int(D), tK, tV, int(tokens), float(value), unit,
                    cite.strip()))
    return out


ROWS = rows()


def row_bytes(row_fn, t, D):
    return row_fn(t, D)


@pytest.mark.parametrize("layers,heads,D,tK,tV,tokens,value,unit,cite", ROWS,
                         ids=[f"{r[3]}-{r[4]}-{r[5]}-{r[2]}" for r in ROWS])
def test_oracle_layout_reproduces_page_sizes(layers, heads, D, tK, tV, tokens, value, unit, cite):
    per_row = lambda t: O.data_row_bytes(t, D) + O.scale_row_bytes(t, D)
    total = layers * heads * tokens * (per_row(tK) + per_row(tV))
    assert total / UNIT[unit] == pytest.approx(value, rel=1e-12), cite


def test_block_sizes():
    """34-byte q8_0 and 18-byte q4_0 blocks (8.5 and 4.5 bits per value)."""
    for t, blk in (("q8_0", 34), ("q4_0", 18)):
        assert O.data_row_bytes(t, 32) + O.scale_row_bytes(t, 32) == blk
    assert O.data_row_bytes("f16", 32) + O.scale_row_bytes("f16", 32) == 64
