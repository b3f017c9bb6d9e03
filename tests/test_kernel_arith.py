"""Integer identities the attention kernel's address arithmetic relies on,
checked exhaustively on the host.

The kernel splits a flat context key g into (page, token) as
floor(fma(float(g), RN(1/pt), RN(1/pt)/2)) in fp32, for every page size pt
that the library accepts (multiples of 8) and every key below 2^22 - 1 (the
host rejects larger contexts). The fractional part of (g + 1/2)/pt is at
least 1/(2 pt) from an integer, so the worst cases are the first and last
token of every page; both are checked for every page of every page size up to
70,000 tokens. The fma is emulated exactly: g * RN(1/pt) + RN(1/pt)/2 needs
fewer than 53 significant bits, so it is exact in fp64 and one rounding to
fp32 is the fma's.
"""
import numpy as np

LIMIT = (1 << 22) - 1


def fp32_page_of(g, pt):
    r = np.float64(np.float32(1.0) / np.float32(pt))           # RN(1/pt)
    x = g.astype(np.float64) * r + r * 0.5                      # exact in fp64
    return np.floor(x.astype(np.float32)).astype(np.int64)      # one rounding = the fma's


def test_fp32_page_division_is_exact_at_every_page_boundary():
    for pt in range(8, 70001, 8):
        q = np.arange(0, LIMIT // pt + 1, dtype=np.int64)
        first = q * pt
        last = q * pt + (pt - 1)
        for g in (first[first < LIMIT], last[last < LIMIT]):
            assert np.array_equal(fp32_page_of(g, pt), g // pt), pt


def test_fp32_page_division_is_exact_for_every_key_of_the_wan_pages():
    g = np.arange(LIMIT, dtype=np.int64)
    for pt in (8, 24, 40, 64, 72, 104, 1560, 4680):
        assert np.array_equal(fp32_page_of(g, pt), g // pt), pt


def test_fp32_page_division_fails_beyond_the_limit():
    """The bound is not slack: with 2^24 keys some key lands on the wrong page."""
    g = np.arange(1 << 24, dtype=np.int64)
    bad = [pt for pt in (1560, 4680, 65528) if not np.array_equal(fp32_page_of(g, pt), g // pt)]
    assert bad
