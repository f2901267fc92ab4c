"""Dictionary generation and Figure-4 entry packing ([QMoE] "The Fixed-to-
Variable Dictionary Code").

The method: a static table of the 2^16 most probable ternary sequences of
length 1..28 under the i.i.d. model of Eq. 2 (P(0)=p0, P(1)=P(2)=(1-p0)/2),
grown from the empty sequence by a best-first search that repeatedly pops the
most probable candidate, records it when its length is 1..28, and pushes its
extensions by one more *pair* of symbols.  Codeword = position in the table,
the table being ordered from most to least probable.

Readings taken where the page is silent:
  * Extension is by pairs, so only even lengths 2..28 exist.
  * Equal probabilities: every sequence with z zeros and n nonzeros has the
    same probability ("class" (L, n), L = z + n).  Within a class the order is
    (a) the colexicographic rank of the nonzero-position tuple p_0<...<p_{n-1},
    i.e. sum_i C(p_i, i+1) (the combinatorial number system), then (b) the sign
    index sum_i [symbol at p_i == 2] * 2^i (lowest position = least significant
    bit).  Different classes are ordered by the value z*ln p0 + n*ln q; classes
    whose values agree to 1e-9 (exact ties, which do not occur at p0=0.885)
    order by shorter length, then fewer nonzeros.
  * Both pair-count nibbles of a packed entry hold the entry's total pair count;
    unused symbol slots are zero.

Pins (tests/test_oracle_dictionary.py): brute-force enumeration on a reduced
table, closed-form class counts, 512 KB size, prefix closure, monotone
probability, hand-packed Figure-4 words.
"""
from __future__ import annotations

import heapq
import math
from functools import cmp_to_key
from math import comb

import numpy as np

N_ENTRIES = 1 << 16
MAX_LEN = 28


def class_order(p0: float, max_len: int = MAX_LEN) -> dict:
    """Rank of every class (L, n) (L even, 2..max_len; 0 <= n <= L) in
    decreasing probability, with the tie rule above.  Returns {(L, n): rank}."""
    if not (0.0 < p0 < 1.0):
        raise ValueError("p0 must lie in (0, 1)")
    lp0 = math.log(p0)
    lq = math.log((1.0 - p0) / 2.0)
    classes = [(L, n) for L in range(2, max_len + 1, 2) for n in range(L + 1)]

    def value(c):
        L, n = c
        return (L - n) * lp0 + n * lq

    def cmp(a, b):
        va, vb = value(a), value(b)
        if abs(va - vb) > 1e-9 * max(1.0, abs(va), abs(vb)):
            return -1 if va > vb else 1          # more probable first
        if a[0] != b[0]:
            return -1 if a[0] < b[0] else 1      # shorter first
        return -1 if a[1] < b[1] else (1 if a[1] > b[1] else 0)

    ordered = sorted(classes, key=cmp_to_key(cmp))
    return {c: i for i, c in enumerate(ordered)}


def in_class_rank(seq) -> tuple:
    """(colex rank of the nonzero positions, sign index) of a symbol sequence."""
    nz = [i for i, s in enumerate(seq) if s != 0]
    colex = sum(comb(p, i + 1) for i, p in enumerate(nz))
    sidx = sum(1 << i for i, p in enumerate(nz) if seq[p] == 2)
    return colex, sidx


def build_dictionary(p0: float = 0.885, n_entries: int = N_ENTRIES, max_len: int = MAX_LEN) -> list:
    """Best-first search over pair extensions (Algorithm 1 of [QMoE]).

    Returns the list of n_entries symbol tuples; index = codeword."""
    rank = class_order(p0, max_len)
    pairs = [(a, b) for a in range(3) for b in range(3)]

    def key(seq):
        L = len(seq)
        n = sum(1 for s in seq if s)
        colex, sidx = in_class_rank(seq)
        return (rank[(L, n)], colex, sidx)

    heap = [((-1, 0, 0), ())]          # the empty sequence, probability 1
    out = []
    while heap and len(out) < n_entries:
        _, seq = heapq.heappop(heap)
        if 1 <= len(seq) <= max_len:
            out.append(seq)
        if len(seq) + 2 <= max_len:
            for a, b in pairs:
                child = seq + (a, b)
                heapq.heappush(heap, (key(child), child))
    if len(out) < n_entries:
        raise ValueError("fewer candidate sequences than table entries")
    return out


def pack_entry(seq) -> tuple:
    """Figure-4 packing of one entry into two uint32 words.

    Word 0: bits 0-3 = pair count k, bits 4+2i..5+2i = symbol i (i = 0..13).
    Word 1: bits 0-3 = k, bits 4+2i..5+2i = symbol 14+i."""
    L = len(seq)
    if L % 2 or not (2 <= L <= 28):
        raise ValueError("entry length must be even, 2..28")
    k = L // 2
    w0 = k
    w1 = k
    for i, s in enumerate(seq):
        if not (0 <= s <= 2):
            raise ValueError("symbols are 0, 1, 2")
        if i < 14:
            w0 |= s << (4 + 2 * i)
        else:
            w1 |= s << (4 + 2 * (i - 14))
    return w0, w1


def unpack_entry(w0: int, w1: int) -> tuple:
    """Inverse of pack_entry: the symbol tuple of length 2*k."""
    k = w0 & 0xF
    if (w1 & 0xF) != k or not (1 <= k <= 14):
        raise ValueError("corrupt pair count")
    L = 2 * k
    seq = []
    for i in range(L):
        w = w0 if i < 14 else w1
        j = i if i < 14 else i - 14
        seq.append((w >> (4 + 2 * j)) & 3)
    return tuple(seq)


def dictionary_words(seqs) -> np.ndarray:
    """uint32[2 * len(seqs)]: entry c occupies words 2c (symbols 0..13) and 2c+1."""
    out = np.zeros(2 * len(seqs), dtype=np.uint32)
    for c, s in enumerate(seqs):
        w0, w1 = pack_entry(s)
        out[2 * c] = w0
        out[2 * c + 1] = w1
    return out


def expansion_table(words: np.ndarray) -> tuple:
    """(symbols uint8[E, 28], lengths int32[E]) obtained by unpacking every
    packed entry; unused slots are 0."""
    E = len(words) // 2
    sym = np.zeros((E, 28), dtype=np.uint8)
    lens = np.zeros(E, dtype=np.int32)
    for c in range(E):
        s = unpack_entry(int(words[2 * c]), int(words[2 * c + 1]))
        lens[c] = len(s)
        sym[c, :len(s)] = s
    return sym, lens
