"""The KV tier ladder (kvq_select_kv_tier, host-only) against the pages'
validation of the automatic tier choice (tests/golden/kv_tier_ladder.txt), and
its edges: f16 when everything fits, the last rung when nothing does."""
import os

import pytest

from quantised_kv_long_amd import _lib
from quantised_kv_long_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
MIB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    srcs = B.sources()
    if not os.path.exists(B.LIB) or os.path.getmtime(B.LIB) < max(os.path.getmtime(s) for s in srcs):
        B.build()
    return _lib.load()


def rows():
    out = []
    for line in open(os.path.join(HERE, "golden", "kv_tier_ladder.txt")):
        line = line.split("|")[0].strip()
        if not line or line.startswith("#"):
            continue
        L, H, D, n, target, tier, cache, budget = line.split()
        out.append((int(L), int(H), int(D), int(n), int(target), tier, int(cache), int(budget)))
    return out


RESIDENT_MIB = 15136   # from any one validation line: target - 1536 - budget


@pytest.mark.parametrize("row", rows())
def test_pages_validation(lib, row):
    L, H, D, n, target, tier, cache, budget = row
    free = 96 * 1024 * MIB                      # the card is larger than every target
    t, got_budget, got_cache = _lib.kvq_select_kv_tier(n, L, H, D, free, RESIDENT_MIB * MIB,
                                                       target * MIB)
    assert "/".join(_lib.TIERS[t]) == tier
    assert got_cache == cache * MIB
    assert got_budget == budget * MIB


def test_resident_size_is_consistent_across_the_lines():
    assert len({target - 1536 - budget for _, _, _, _, target, _, _, budget in rows()}) == 1


def test_every_rung_is_the_first_that_fits(lib):
    n, L, H, D = 32768, 48, 8, 128
    sizes = [_lib.kvq_tier_cache_bytes(t, n, L, H, D) for t in range(4)]
    assert sizes == sorted(sizes, reverse=True)
    assert sizes[0] == 2 * 48 * 8 * 32768 * 256          # f16: 2D bytes a row, K and V
    reserve = 1536 * MIB
    for t, size in enumerate(sizes):
        # a budget of exactly this rung's size picks it; one byte less picks the next
        got, budget, _ = _lib.kvq_select_kv_tier(n, L, H, D, size + reserve, 0, 0)
        assert got == t and budget == size
        if t < 3:
            assert _lib.kvq_select_kv_tier(n, L, H, D, size + reserve - 1, 0, 0)[0] == t + 1
    # nothing fits: the floor
    assert _lib.kvq_select_kv_tier(n, L, H, D, 1 << 30, 0, 0)[0] == 3


def test_target_only_caps_the_free_memory(lib):
    n, L, H, D = 32768, 48, 8, 128
    a = _lib.kvq_select_kv_tier(n, L, H, D, 30000 * MIB, 15136 * MIB, 0)
    b = _lib.kvq_select_kv_tier(n, L, H, D, 30000 * MIB, 15136 * MIB, 40000 * MIB)
    assert a == b and a[0] == 0


def test_tier_types_and_errors(lib):
    assert _lib.kvq_tier_types(0) == (_lib.F16, _lib.F16)
    assert _lib.kvq_tier_types(1) == (_lib.Q8_0, _lib.Q8_0)
    assert _lib.kvq_tier_types(2) == (_lib.Q8_0, _lib.Q4_0)
    assert _lib.kvq_tier_types(3) == (_lib.Q5_1, _lib.Q4_0)
    with pytest.raises(_lib.KVQError):
        _lib.kvq_tier_types(4)
    assert _lib.kvq_tier_cache_bytes(4, 1, 1, 1, 128) == -1
    assert _lib.kvq_tier_cache_bytes(0, 1, 1, 1, 100) == -1
    assert lib.kvq_select_kv_tier(0, 48, 8, 128, 1, 0, 0, None, None) == -2
    assert lib.kvq_select_kv_tier(1, 48, 8, 128, -1, 0, 0, None, None) == -2
