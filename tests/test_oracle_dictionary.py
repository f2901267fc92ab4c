"""Pins of oracle/dictionary.py against the QMoE page and exact counting."""
import math
from fractions import Fraction
from itertools import product
from math import comb

import numpy as np
import pytest

from oracle import dictionary as D


def _exact_prob(seq, p0):
    p = Fraction(p0)
    q = (1 - p) / 2
    z = sum(1 for s in seq if s == 0)
    return p ** z * q ** (len(seq) - z)


def _colex_rank_by_sorting(L, n):
    """Rank of every n-subset of range(L) in colex order, by sorting subsets on
    their reversed tuples (no binomial arithmetic)."""
    from itertools import combinations
    subsets = sorted(combinations(range(L), n), key=lambda t: tuple(reversed(t)))
    return {t: i for i, t in enumerate(subsets)}


@pytest.mark.parametrize("p0,n_entries,max_len", [(0.885, 300, 8), (0.7, 500, 8), (0.886, 120, 6)])
def test_best_first_equals_exhaustive_sort(p0, n_entries, max_len):
    """Brute force on a reduced table: enumerate every even-length sequence,
    sort by exact probability (descending), break ties by the in-class reading
    (colex rank of positions by sorting, then sign index), take the top."""
    cands = []
    rank_cache = {}
    for L in range(2, max_len + 1, 2):
        for seq in product(range(3), repeat=L):
            nz = tuple(i for i, s in enumerate(seq) if s)
            key = (L, len(nz))
            if key not in rank_cache:
                rank_cache[key] = _colex_rank_by_sorting(L, len(nz))
            colex = rank_cache[key][nz]
            sidx = sum(1 << i for i, p in enumerate(nz) if seq[p] == 2)
            cands.append((-_exact_prob(seq, p0), colex, sidx, seq))
    cands.sort()
    expect = [c[3] for c in cands[:n_entries]]
    got = D.build_dictionary(p0, n_entries=n_entries, max_len=max_len)
    assert got == expect


def test_size_and_figure4_bytes(odict):
    seqs, words = odict["seqs"], odict["words"]
    assert len(seqs) == 65536 and len(set(seqs)) == 65536
    assert words.dtype == np.uint32 and words.nbytes == 512 * 1024  # 2^16 x 8 B
    assert all(len(s) % 2 == 0 and 2 <= len(s) <= 28 for s in seqs)


def test_class_counts_closed_form(odict):
    """Every class (L, n) holds C(L,n)*2^n equiprobable sequences; taking
    classes in decreasing probability until 2^16 fixes how many of each class
    are in the table.  Compare against the built table."""
    p0 = 0.885
    lp, lq = math.log(p0), math.log((1 - p0) / 2)
    classes = sorted(((L, n) for L in range(2, 29, 2) for n in range(L + 1)),
                     key=lambda c: -((c[0] - c[1]) * lp + c[1] * lq))
    left = 65536
    expect = {}
    for L, n in classes:
        take = min(left, comb(L, n) * 2 ** n)
        if take:
            expect[(L, n)] = take
        left -= take
    got = {}
    for s in odict["seqs"]:
        k = (len(s), sum(1 for v in s if v))
        got[k] = got.get(k, 0) + 1
    assert got == expect
    # the cut falls inside class (26, 3): 2490 of its 20800 sequences
    assert got[(26, 3)] == 2490
    by_len = {}
    by_n = {}
    for (L, n), v in got.items():
        by_len[L] = by_len.get(L, 0) + v
        by_n[n] = by_n.get(n, 0) + v
    assert by_n == {0: 14, 1: 420, 2: 7700, 3: 57402}
    assert by_len[28] == 1569 and by_len[26] == 3843 and by_len[2] == 9


def test_probability_non_increasing_and_prefix_closed(odict):
    seqs = odict["seqs"]
    p0 = 0.885
    lp, lq = math.log(p0), math.log((1 - p0) / 2)
    v = np.array([(len(s) - sum(1 for x in s if x)) * lp + sum(1 for x in s if x) * lq for s in seqs])
    assert np.all(np.diff(v) <= 1e-12)
    table = set(seqs)
    for s in seqs:
        for k in range(2, len(s), 2):
            assert s[:k] in table
    # any sequence outside the table is no more probable than the last entry
    last = v[-1]
    for L in range(2, 29, 2):
        for n in range(0, 5):
            if n > L:
                continue
            val = (L - n) * lp + n * lq
            inside = sum(1 for s in seqs if len(s) == L and sum(1 for x in s if x) == n)
            if inside < comb(L, n) * 2 ** n:
                assert val <= last + 1e-12


def test_figure4_packing_by_hand(odict):
    seqs, words = odict["seqs"], odict["words"]
    c = seqs.index((0, 0))
    assert c == 0 and words[0] == 1 and words[1] == 1           # k=1, all symbols 00
    c = seqs.index((2, 0))
    assert words[2 * c] == (1 | (2 << 4)) and words[2 * c + 1] == 1
    c = seqs.index((0,) * 28)
    assert words[2 * c] == 14 and words[2 * c + 1] == 14
    s = (0,) * 15 + (1,) + (0,) * 12                            # symbol 15 -> word 1, slot 1
    assert D.pack_entry(s) == (14, 14 | (1 << 6))
    s = (0,) * 13 + (2,) + (0,) * 14                            # symbol 13 -> word 0, bits 30-31
    assert D.pack_entry(s) == (14 | (2 << 30), 14)
    for c in range(0, 65536, 97):
        assert D.unpack_entry(int(words[2 * c]), int(words[2 * c + 1])) == seqs[c]


def test_page_entropy_numbers():
    """QMoE page, 'The entropy perspective': about 0.63 bit/weight at
    p0 = 0.885, a limit of about 25.4x against 16-bit weights."""
    p0 = 0.885
    q = (1 - p0) / 2
    H = -p0 * math.log2(p0) - 2 * q * math.log2(q)
    assert abs(H - 0.63) < 0.005
    assert abs(16 / H - 25.4) < 0.1


def test_same_table_for_0886(odict):
    assert D.build_dictionary(0.886) == odict["seqs"]


def test_first_codes_reading(odict):
    seqs = odict["seqs"]
    assert [len(s) for s in seqs[:12]] == list(range(2, 25, 2))
    assert all(not any(s) for s in seqs[:12])
    assert seqs[12:16] == [(1, 0), (2, 0), (0, 1), (0, 2)]
    assert seqs[16] == (0,) * 26 and seqs[25] == (0,) * 28


@pytest.mark.parametrize("p0", [0.857, 0.864])
def test_class_ranges_closed_form_other_p0(odict_for, p0):
    """Tables built for the sparsities the page reports for base128 and
    large128 (Table 4: 85.7%, 86.4%): classes (L, n) of C(L,n)*2^n
    equiprobable sequences taken in decreasing probability until 2^16, each
    occupying one contiguous codeword range in that order.  At p0 = 0.857 the
    4-nonzero classes are (4,4), (6,4), (8,4): 16 + 240 + 1120 = 1376 entries."""
    od = odict_for(p0)
    lp, lq = math.log(p0), math.log((1 - p0) / 2)
    classes = sorted(((L, n) for L in range(2, 29, 2) for n in range(L + 1)),
                     key=lambda c: -((c[0] - c[1]) * lp + c[1] * lq))
    left, start, ranges = 65536, 0, []
    for L, n in classes:
        take = min(left, comb(L, n) * 2 ** n)
        if take:
            ranges.append((L, n, start, start + take))
        start += take
        left -= take
    seqs = od["seqs"]
    for L, n, a, b in ranges:
        for c in (a, (a + b) // 2, b - 1):
            s = seqs[c]
            assert (len(s), sum(1 for v in s if v)) == (L, n), (p0, c, L, n)
    got4 = {(L, n): b - a for L, n, a, b in ranges if n == 4}
    n4 = sum(1 for s in seqs if sum(1 for v in s if v) == 4)
    assert n4 == sum(got4.values())
    assert max(sum(1 for v in s if v) for s in seqs) == 4
    if p0 == 0.857:
        assert got4 == {(4, 4): 16, (6, 4): 240, (8, 4): 1120} and n4 == 1376
        assert next(a for L, n, a, b in ranges if n == 4) == 34534
