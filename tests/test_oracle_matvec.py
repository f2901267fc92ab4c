"""Pins of oracle/matvec.py against codec-free brute force and closed forms."""
from itertools import product

import numpy as np

from oracle import codec as C
from oracle import matvec as M
from sub_bit_moe_amd import synth


def test_all_2x4_ternary_matrices(odict):
    mats = np.array(list(product(range(3), repeat=8)), dtype=np.uint8).reshape(-1, 2, 4)
    sym = mats.reshape(-1, 4)                       # 2*6561 rows, 4 cols
    codes, row_off = C.encode_matrix(sym, odict["child"])
    rng = np.random.default_rng(7)
    scales = synth.row_scales(rng, sym.shape[0])
    x = synth.activations(rng, 1, 4)
    y = M.matvec(codes, row_off, scales, odict["sym28"], odict["lens"], 4, x)
    ref = M.dense_ternary_matvec(synth.symbols_to_ternary(sym), scales, x)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=0)


def _enc(odict, sym):
    return C.encode_matrix(sym, odict["child"])


def test_unit_vector_ones_zero_and_linearity(odict):
    rng = np.random.default_rng(9)
    rows, cols = 37, 210
    sym = synth.ternary_symbols(rng, rows, cols, 0.886)
    tern = synth.symbols_to_ternary(sym).astype(np.float64)
    s = synth.row_scales(rng, rows)
    codes, row_off = _enc(odict, sym)
    args = (codes, row_off, s, odict["sym28"], odict["lens"], cols)
    for j in (0, 1, 101, cols - 1):
        e = np.zeros((1, cols))
        e[0, j] = 1.0
        assert np.array_equal(M.matvec(*args, e)[0], s.astype(np.float64) * tern[:, j])
    ones = np.ones((1, cols))
    npos = (sym == 2).sum(1)
    nneg = (sym == 1).sum(1)
    assert np.array_equal(M.matvec(*args, ones)[0], s.astype(np.float64) * (npos - nneg))
    zc, zo = _enc(odict, np.zeros((rows, cols), np.uint8))
    assert not M.matvec(zc, zo, s, odict["sym28"], odict["lens"], cols, ones).any()
    a = synth.activations(rng, 1, cols).astype(np.float64)
    b = synth.activations(rng, 1, cols).astype(np.float64)
    np.testing.assert_allclose(M.matvec(*args, 2 * a - b),
                               2 * M.matvec(*args, a) - M.matvec(*args, b), rtol=1e-12, atol=1e-12)


def test_rows_subset_matches_full(odict):
    rng = np.random.default_rng(10)
    sym = synth.ternary_symbols(rng, 20, 64, 0.886)
    s = synth.row_scales(rng, 20)
    x = synth.activations(rng, 3, 64)
    codes, row_off = _enc(odict, sym)
    full = M.matvec(codes, row_off, s, odict["sym28"], odict["lens"], 64, x)
    sub = M.matvec_rows(codes, row_off, s, odict["sym28"], odict["lens"], 64, x, [0, 5, 19])
    np.testing.assert_allclose(sub, full[:, [0, 5, 19]], rtol=1e-13)


def test_minmax_all_2x4_ternary_matrices(odict):
    """The page's grid by brute force: every 2x4 ternary matrix, weights looked
    up symbol by symbol from (0, w_min, w_max) of the row, summed by loops."""
    mats = np.array(list(product(range(3), repeat=8)), dtype=np.uint8).reshape(-1, 2, 4)
    sym = mats.reshape(-1, 4)
    codes, row_off = C.encode_matrix(sym, odict["child"])
    rng = np.random.default_rng(8)
    mm = synth.row_minmax(rng, sym.shape[0])
    x = synth.activations(rng, 2, 4).astype(np.float64)
    y = M.matvec_minmax(codes, row_off, mm, odict["sym28"], odict["lens"], 4, x)
    for r in range(0, sym.shape[0], 97):
        vals = {0: 0.0, 1: float(mm[r, 0]), 2: float(mm[r, 1])}
        for t in range(2):
            ref = 0.0
            for j in range(4):
                ref += vals[int(sym[r, j])] * x[t, j]
            assert abs(y[t, r] - ref) <= 1e-12 * (1 + abs(ref))


def test_minmax_special_cases(odict):
    """w_min = -w_max reduces to the symmetric grid; x = e_j picks column j;
    x = 1 gives w_min * #1 + w_max * #2 per row."""
    rng = np.random.default_rng(12)
    rows, cols = 29, 130
    sym = synth.ternary_symbols(rng, rows, cols, 0.886)
    codes, row_off = _enc(odict, sym)
    s = synth.row_scales(rng, rows)
    sym_mm = np.stack([-s, s], axis=1)
    x = synth.activations(rng, 2, cols)
    args = (odict["sym28"], odict["lens"], cols)
    np.testing.assert_array_equal(M.matvec_minmax(codes, row_off, sym_mm, *args, x),
                                  M.matvec(codes, row_off, s, *args, x))
    mm = synth.row_minmax(rng, rows).astype(np.float64)
    for j in (0, 77, cols - 1):
        e = np.zeros((1, cols))
        e[0, j] = 1.0
        col = np.where(sym[:, j] == 1, mm[:, 0], np.where(sym[:, j] == 2, mm[:, 1], 0.0))
        assert np.array_equal(M.matvec_minmax(codes, row_off, mm, *args, e)[0], col)
    ones = M.matvec_minmax(codes, row_off, mm, *args, np.ones((1, cols)))[0]
    np.testing.assert_allclose(ones, mm[:, 0] * (sym == 1).sum(1) + mm[:, 1] * (sym == 2).sum(1), rtol=1e-13)


def test_dequantize_symbol_map():
    sym = np.array([[0, 1, 2]], np.uint8)
    w = C.dequantize(sym, np.array([0.5], np.float16))
    assert w.tolist() == [[0.0, -0.5, 0.5]]
    w2 = C.dequantize_minmax(sym, np.array([[-0.25, 0.75]], np.float16))
    assert w2.tolist() == [[0.0, -0.25, 0.75]]


def test_rms_glue_properties():
    """The stack glue pinned by what it must satisfy rather than by its
    formula: every nonzero output row has unit RMS (up to fp16 rounding) and is
    a positive multiple of its input row; a zero row stays zero."""
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((6, 300)) * rng.uniform(1e-3, 1e3, (6, 1))).astype(np.float16)
    y[2] = 0
    x = M.rms_glue(y).astype(np.float64)
    for t in range(6):
        if t == 2:
            assert not np.any(x[t])
            continue
        assert abs(np.sqrt(np.mean(x[t] ** 2)) - 1.0) < 2e-3
        yt = y[t].astype(np.float64)
        k = np.dot(x[t], yt) / np.dot(yt, yt)
        assert k > 0 and np.allclose(x[t], k * yt, rtol=2e-3, atol=2e-3)
