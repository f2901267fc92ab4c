"""Shared helpers for GPU parity tests: tolerance metrics and stack builders.

Expected values come only from the oracle applied to the seeded inputs; the
library's host encoder output is compared bit-exactly with the oracle's
encoding before any GPU result is checked.
"""
import numpy as np

from oracle import codec as OC
from oracle import matvec as OM
from sub_bit_moe_amd import synth

REL_L2 = 1e-3
MAX_REL = 5e-3


def rel_l2(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(y - ref) / (den if den > 0 else 1.0))


def max_rel(y, ref):
    """max_i |y_i - ref_i| / max(|ref_i|, rms(ref))."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(y - ref) / den)) if ref.size else 0.0


def assert_close(y, ref, rl2=REL_L2, mr=MAX_REL, what=""):
    a, b = rel_l2(y, ref), max_rel(y, ref)
    assert a <= rl2 and b <= mr, f"{what}: rel-L2 {a:.3e} (<= {rl2}), max-rel {b:.3e} (<= {mr})"


def host_experts(E, rows, cols, p0, seed):
    """Seeded symbols and scales for E experts: list of (sym, scales)."""
    rng = np.random.default_rng(seed)
    return [(synth.ternary_symbols(rng, rows, cols, p0), synth.row_scales(rng, rows)) for _ in range(E)]


def encode_all(experts, words, odict=None, check_every=1):
    """Encode with the library; every check_every-th expert is also encoded by
    the oracle and compared bit-exactly."""
    from sub_bit_moe_amd import api
    mats = []
    for i, (sym, sc) in enumerate(experts):
        codes, row_off, bstart = api.encode_matrix(sym, words)
        if odict is not None and i % check_every == 0:
            rc, ro = OC.encode_matrix(sym, odict["child"])
            assert np.array_equal(codes, rc) and np.array_equal(row_off, ro)
            assert np.array_equal(bstart, OC.block_starts(rc, odict["lens"], 1024))
        mats.append((codes, row_off, bstart, sc))
    return mats


def oracle_matvec_from_symbols(sym, scales, x):
    """fp64 y = W_hat x via the oracle's dequantisation of the symbols."""
    W = OC.dequantize(sym, scales)
    return np.asarray(x, np.float64).reshape(-1, sym.shape[1]) @ W.T


def oracle_matvec_from_codes(odict, sym, scales, x):
    """fp64 y through the oracle's own encode + reference decode."""
    codes, row_off = OC.encode_matrix(sym, odict["child"])
    return OM.matvec(codes, row_off, scales, odict["sym28"], odict["lens"], sym.shape[1], x)


def oracle_matvec_minmax_from_codes(odict, sym, minmax, x):
    """fp64 y on the per-row grid (w_min, w_max) through the oracle's own
    encode + reference decode."""
    codes, row_off = OC.encode_matrix(sym, odict["child"])
    return OM.matvec_minmax(codes, row_off, minmax, odict["sym28"], odict["lens"], sym.shape[1], x)


def oracle_matvec_minmax_from_symbols(sym, minmax, x):
    """fp64 y = W_hat x on the per-row grid (w_min, w_max) via the oracle's
    dequantisation of the symbols."""
    W = OC.dequantize_minmax(sym, minmax)
    return np.asarray(x, np.float64).reshape(-1, sym.shape[1]) @ W.T
