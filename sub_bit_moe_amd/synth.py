"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module holds input generation only: ternary symbol matrices drawn i.i.d.
from the distribution of the QMoE page's Eq. 2 (P(0)=p0, the two nonzero values
equiprobable), per-row fp16 scales, fp16 activations, and top-1 Zipf routing
(expert popularity is Zipfian per the cache-amplification page, section
"Routing statistics"). None of the codec's or the product's arithmetic lives here.

Symbol convention used everywhere: 0 = zero, 1 = negative (w_min), 2 = positive
(w_max); the QMoE page's Figure 4 stores exactly these 2-bit values.

Two generators:
  * host matrices (small and mid configs): numpy PCG64, seeded;
  * counter-based matrices (configs too large for host memory): the published
    SplitMix64 generator (Steele, Lea, Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014; reference code by S. Vigna), whose i-th
    output for state s is mix64(s + i*GAMMA).  The HIP generator implements the
    same definition independently; sampled experts are regenerated here
    bit-identically for checking.
"""
from __future__ import annotations

import numpy as np

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# ---------------------------------------------------------------- host draws

def ternary_symbols(rng: np.random.Generator, rows: int, cols: int, p0: float) -> np.ndarray:
    """uint8 [rows, cols] of symbols {0,1,2}: P(0)=p0, P(1)=P(2)=(1-p0)/2."""
    u = rng.random((rows, cols))
    out = np.zeros((rows, cols), dtype=np.uint8)
    half = p0 + (1.0 - p0) / 2.0
    out[(u >= p0) & (u < half)] = 1
    out[u >= half] = 2
    return out


def row_scales(rng: np.random.Generator, rows: int, lo: float = 0.01, hi: float = 0.05) -> np.ndarray:
    """fp16 per-row scales s_r ~ U(lo, hi), rounded to nearest fp16."""
    return rng.uniform(lo, hi, size=rows).astype(np.float16)


def row_minmax(rng: np.random.Generator, rows: int, lo: float = 0.01, hi: float = 0.05,
               skew: float = 0.4) -> np.ndarray:
    """fp16 [rows, 2] per-row grid values (w_min, w_max): w_max = s*u and
    w_min = -s*v with s ~ U(lo, hi) and u, v ~ U(1 - skew, 1 + skew)."""
    s = rng.uniform(lo, hi, size=rows)
    u = rng.uniform(1 - skew, 1 + skew, size=rows)
    v = rng.uniform(1 - skew, 1 + skew, size=rows)
    return np.stack([-s * v, s * u], axis=1).astype(np.float16)


def activations(rng: np.random.Generator, n_tokens: int, width: int) -> np.ndarray:
    """fp16 [n_tokens, width] ~ N(0,1), rounded to nearest fp16."""
    return rng.standard_normal((n_tokens, width)).astype(np.float16)


def zipf_routing(rng: np.random.Generator, n_tokens: int, n_experts: int, s: float = 1.1) -> np.ndarray:
    """int32 [n_tokens] top-1 expert ids: popularity rank k has probability
    proportional to k^-s (k = 1..E); ranks map to expert ids through a seeded
    permutation; tokens are i.i.d."""
    k = np.arange(1, n_experts + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    perm = rng.permutation(n_experts)
    ranks = rng.choice(n_experts, size=n_tokens, p=p)
    return perm[ranks].astype(np.int32)


def symbols_to_ternary(sym: np.ndarray) -> np.ndarray:
    """int8 view {-1,0,+1} of symbols {0,1,2} (1 -> -1, 2 -> +1)."""
    t = np.zeros(sym.shape, dtype=np.int8)
    t[sym == 1] = -1
    t[sym == 2] = 1
    return t

# ---------------------------------------------------- counter-based (SplitMix64)

def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def splitmix64_at(state: int, idx) -> np.ndarray:
    """Output number idx (idx >= 1) of SplitMix64 started at `state`."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(state & M64) + idx * np.uint64(GAMMA)
    return _mix64(z)


def zero_threshold16(p0: float) -> int:
    """Even 16-bit threshold Z: a 16-bit draw v is a zero symbol iff v < Z.
    Z is even so the 65536-Z nonzero draws split exactly in half by parity."""
    z = 2 * int(round(p0 * 32768.0))
    return max(0, min(65536, z))


def matrix_key(seed: int, layer: int, expert: int, mat: int, n_experts: int) -> int:
    """Per-matrix SplitMix64 state: output number (global matrix index + 1) of
    SplitMix64 started at `seed`.  mat 0 = up projection, 1 = down projection."""
    m = (layer * n_experts + expert) * 2 + mat
    return int(splitmix64_at(seed, m + 1))


def counter_symbols(key: int, rows: int, cols: int, p0: float, row0: int = 0) -> np.ndarray:
    """uint8 [rows, cols] symbols of rows row0..row0+rows-1 of a counter-based
    matrix.  Row r, column j uses 16-bit lane (j % 4) (lane 0 = least
    significant) of output number r*ceil(cols/4) + j//4 + 1 of SplitMix64 at
    `key`.  v < Z -> 0; else odd v -> 2 (positive), even v -> 1 (negative)."""
    w = (cols + 3) // 4
    r = np.arange(row0, row0 + rows, dtype=np.uint64)[:, None]
    j = np.arange(cols, dtype=np.uint64)[None, :]
    idx = r * np.uint64(w) + j // np.uint64(4) + np.uint64(1)
    h = splitmix64_at(key, idx)
    v = (h >> (np.uint64(16) * (j % np.uint64(4)))) & np.uint64(0xFFFF)
    z = zero_threshold16(p0)
    out = np.where(v < z, 0, np.where((v & np.uint64(1)) == 1, 2, 1)).astype(np.uint8)
    return out


SCALE_TABLE_BITS = 12


def scale_table(lo: float = 0.01, hi: float = 0.05) -> np.ndarray:
    """fp16 table of 4096 scales lo + (hi-lo)*(k+0.5)/4096, rounded to fp16.
    Counter-based matrices pick row scales from it (the table is an input)."""
    k = np.arange(1 << SCALE_TABLE_BITS, dtype=np.float64)
    return (lo + (hi - lo) * (k + 0.5) / float(1 << SCALE_TABLE_BITS)).astype(np.float16)


def counter_scale_index(key: int, rows: int, row0: int = 0) -> np.ndarray:
    """uint16 [rows] scale-table indices: top 12 bits of SplitMix64 output
    number (2^40 + r + 1) at `key` (a counter range disjoint from symbols)."""
    r = np.arange(row0, row0 + rows, dtype=np.uint64)
    h = splitmix64_at(key, r + np.uint64((1 << 40) + 1))
    return (h >> np.uint64(64 - SCALE_TABLE_BITS)).astype(np.uint16)
