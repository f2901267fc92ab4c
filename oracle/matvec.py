"""fp64 products with decoded ternary weights ([QMoE] "The GPU Decoding
Kernel": y = W_hat x per row with the ternary grid {w_min, 0, w_max}; the MoE
expert is a ReLU feed-forward pair, up then down).

Two grids: the symmetric reading (-s_r, 0, +s_r) of the benchmark stacks and
the page's per-row (w_min, 0, w_max).

Pins (tests/test_oracle_matvec.py): brute force over all 3^8 ternary 2x4
matrices (both grids), x = e_j, x = 1, W = 0, linearity, the symmetric grid as
the special case w_min = -w_max.
"""
from __future__ import annotations

import numpy as np

from .codec import decode_symbols_with_table, dequantize, dequantize_minmax


def matvec(codes, row_off, scales, sym28, lens, cols, x) -> np.ndarray:
    """y[t, r] = sum_j W_hat[r, j] * x[t, j] in fp64.  x: [T, cols]."""
    sym = decode_symbols_with_table(codes, row_off, sym28, lens, cols)
    W = dequantize(sym, scales)
    X = np.asarray(x, dtype=np.float64).reshape(-1, cols)
    return X @ W.T


def matvec_minmax(codes, row_off, minmax, sym28, lens, cols, x) -> np.ndarray:
    """y[t, r] = sum_j W_hat[r, j] * x[t, j] in fp64 on the per-row grid
    {w_min, 0, w_max}; minmax: [rows, 2].  x: [T, cols]."""
    sym = decode_symbols_with_table(codes, row_off, sym28, lens, cols)
    W = dequantize_minmax(sym, minmax)
    X = np.asarray(x, dtype=np.float64).reshape(-1, cols)
    return X @ W.T


def matvec_rows(codes, row_off, scales, sym28, lens, cols, x, rows_sel) -> np.ndarray:
    """Same as matvec for the selected rows only (sampled checks).  [T, len(rows_sel)]."""
    rows_sel = np.asarray(rows_sel, dtype=np.int64)
    codes = np.asarray(codes)
    row_off = np.asarray(row_off, dtype=np.int64)
    X = np.asarray(x, dtype=np.float64).reshape(-1, cols)
    out = np.zeros((X.shape[0], rows_sel.size))
    for i, r in enumerate(rows_sel):
        sub_codes = codes[row_off[r]:row_off[r + 1]]
        sym = decode_symbols_with_table(sub_codes, np.array([0, sub_codes.size]), sym28, lens, cols)
        w = dequantize(sym, np.asarray(scales)[r:r + 1])[0]
        out[:, i] = X @ w
    return out


def dense_ternary_matvec(tern, scales, x) -> np.ndarray:
    """Brute-force reference without any codec: tern int8 {-1,0,1} [rows, cols]."""
    W = np.asarray(tern, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, None]
    return np.asarray(x, dtype=np.float64).reshape(-1, W.shape[1]) @ W.T


def relu(v):
    return np.maximum(v, 0.0)


def rms_glue(y) -> np.ndarray:
    """Harness glue between stacked layers (not part of the method): x_next =
    y / sqrt(mean(y^2)) per token, fp64, then fp16.  Pinned by its defining
    properties (unit RMS, a positive multiple of the input, zero rows stay zero)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.sqrt(np.mean(y * y, axis=-1, keepdims=True))
    r = np.where(r > 0, r, 1.0)
    return (y / r).astype(np.float16)
