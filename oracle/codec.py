"""Trie encoder, reference decoder and offset tables ([QMoE] "The GPU Decoding
Kernel": per-row independent encoding with one offset per row; "Encoding":
trie built from the dictionary, greedy longest-prefix walk; [M8.5] 0x08A:
reference decoder expanding each row's codewords and mapping symbols through
[zero, negative, positive]).

Layout of an encoded matrix (rows x cols, cols even):
  codes   uint16[n]       rows' codeword streams concatenated in row order
  row_off uint32[rows+1]  row_off[0] = 0, row_off[r+1] = row_off[r] + #codes(r)
  bstart  uint32[nblk]    for block b of B consecutive codes (B a power of two),
                          the linear symbol position row*cols + col at which
                          code b*B starts ("per-block offset table"; the
                          spec interface's per-wavefront start offsets).

Readings: the walk stops at the row end (rows never share a codeword); an odd
row width is rejected.

Pins (tests/test_oracle_codec.py): round trip on random and edge-case
matrices, brute-force maximality of every emitted codeword, all-zero and
all-nonzero row code counts, long-row mean run length against the stationary
Markov-chain value, block offsets against cumulative decoded lengths.
"""
from __future__ import annotations

import numpy as np

ROOT = -1  # virtual trie root (the empty sequence)


def code_of(seqs) -> dict:
    """Map symbol tuple -> codeword."""
    return {s: c for c, s in enumerate(seqs)}


def trie_children(seqs) -> np.ndarray:
    """int32[E+1, 9]: child[node, 3a+b] = codeword of node's sequence extended
    by pair (a, b), or -1.  Row E is the root (empty sequence)."""
    lookup = code_of(seqs)
    E = len(seqs)
    child = np.full((E + 1, 9), -1, dtype=np.int32)
    for node in range(E + 1):
        base = () if node == E else seqs[node]
        if len(base) + 2 > 28:
            continue
        for a in range(3):
            for b in range(3):
                c = lookup.get(base + (a, b))
                if c is not None:
                    child[node, 3 * a + b] = c
    return child


def encode_row(row_syms, seqs) -> list:
    """Greedy longest-prefix encoding of one row by walking pairs while the
    extended sequence is a dictionary entry.  Plain loop; the definition."""
    lookup = code_of(seqs)
    cols = len(row_syms)
    if cols % 2:
        raise ValueError("odd row width")
    out = []
    pos = 0
    while pos < cols:
        cur = None
        L = 0
        while pos + L + 2 <= cols and L + 2 <= 28:
            cand = tuple(int(v) for v in row_syms[pos:pos + L + 2])
            c = lookup.get(cand)
            if c is None:
                break
            cur, L = c, L + 2
        if cur is None:
            raise ValueError("pair not in dictionary")
        out.append(cur)
        pos += L
    return out


def encode_matrix(sym: np.ndarray, child: np.ndarray) -> tuple:
    """Same walk as encode_row, run for all rows at once (rows are independent).
    Returns (codes uint16[n], row_off uint32[rows+1])."""
    sym = np.asarray(sym, dtype=np.uint8)
    rows, cols = sym.shape
    if cols % 2:
        raise ValueError("odd row width")
    E = child.shape[0] - 1
    if rows == 0:
        return np.zeros(0, np.uint16), np.zeros(1, np.uint32)
    pairs = (sym[:, 0::2].astype(np.int32) * 3 + sym[:, 1::2]).astype(np.int32)
    npairs = cols // 2
    pos = np.zeros(rows, dtype=np.int64)
    cur = np.full(rows, E, dtype=np.int64)          # at the root
    ev_row, ev_code = [], []
    active = np.arange(rows)
    while active.size:
        p = pos[active]
        c = cur[active]
        at_end = p >= npairs
        nxt = np.full(active.size, -1, dtype=np.int64)
        live = ~at_end
        nxt[live] = child[c[live], pairs[active[live], p[live]]]
        ext = nxt >= 0
        # extend: consume the pair
        cur[active[ext]] = nxt[ext]
        pos[active[ext]] += 1
        # stop: emit current node (extension missing or row end)
        stop = ~ext
        if np.any(stop & (c == E) & ~at_end):
            raise ValueError("pair not in dictionary")
        emit = stop & (c != E)
        ev_row.append(active[emit])
        ev_code.append(c[emit])
        cur[active[stop]] = E
        done = stop & at_end
        active = active[~done]
    rr = np.concatenate(ev_row)
    cc = np.concatenate(ev_code)
    order = np.argsort(rr, kind="stable")          # keep emission order per row
    codes = cc[order].astype(np.uint16)
    counts = np.bincount(rr, minlength=rows)
    row_off = np.zeros(rows + 1, dtype=np.uint32)
    row_off[1:] = np.cumsum(counts)
    return codes, row_off


def decode_symbols(codes, row_off, words, cols: int) -> np.ndarray:
    """Reference decode to symbols uint8[rows, cols]: expand each row's codes
    in order by unpacking the Figure-4 words; each row must total cols."""
    from .dictionary import expansion_table
    sym28, lens = expansion_table(words)
    return decode_symbols_with_table(codes, row_off, sym28, lens, cols)


def decode_symbols_with_table(codes, row_off, sym28, lens, cols: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int64)
    row_off = np.asarray(row_off, dtype=np.int64)
    rows = len(row_off) - 1
    out = np.zeros((rows, cols), dtype=np.uint8)
    for r in range(rows):
        cs = codes[row_off[r]:row_off[r + 1]]
        exp = sym28[cs]                                   # [k, 28]
        mask = np.arange(28)[None, :] < lens[cs][:, None]
        flat = exp[mask]                                  # row-major: in order
        if flat.size != cols:
            raise ValueError(f"row {r} decodes to {flat.size} symbols, expected {cols}")
        out[r] = flat
    return out


def dequantize(sym: np.ndarray, scales) -> np.ndarray:
    """fp64 weights: symbol 0 -> 0, 1 -> -s_r, 2 -> +s_r ([zero, negative,
    positive] with a symmetric per-row grid)."""
    s = np.asarray(scales, dtype=np.float64)[:, None]
    table = np.stack([np.zeros_like(s[:, 0]), -s[:, 0], s[:, 0]], axis=1)  # [rows, 3]
    return np.take_along_axis(table, sym.astype(np.int64), axis=1)


def dequantize_minmax(sym: np.ndarray, minmax) -> np.ndarray:
    """fp64 weights on the page's per-row grid {w_min, 0, w_max} ([QMoE]
    "Quantization grid"; the decode table of "The GPU Decoding Kernel" maps
    code 0 -> 0, 1 -> w_min, 2 -> w_max of the row).  minmax: [rows, 2] =
    (w_min, w_max) per row."""
    mm = np.asarray(minmax, dtype=np.float64).reshape(-1, 2)
    table = np.stack([np.zeros(mm.shape[0]), mm[:, 0], mm[:, 1]], axis=1)  # [rows, 3]
    return np.take_along_axis(table, sym.astype(np.int64), axis=1)


def code_lengths(codes, lens) -> np.ndarray:
    return np.asarray(lens, dtype=np.int64)[np.asarray(codes, dtype=np.int64)]


def block_starts(codes, lens, block: int) -> np.ndarray:
    """uint32 linear start position of codes 0, B, 2B, ...: the sum of the
    lengths of all earlier codes (rows are concatenated and each row's codes
    sum to cols, so the sum is row*cols + col)."""
    if block <= 0 or block & (block - 1):
        raise ValueError("block must be a power of two")
    L = code_lengths(codes, lens)
    starts = np.concatenate([[0], np.cumsum(L)])[:-1] if L.size else np.zeros(0, np.int64)
    return starts[::block].astype(np.uint32)
