"""Decompress-then-GEMM for experts with many tokens ([QMoE] "Limitations and
Trade-offs": with many tokens per expert, decompressing and multiplying on the
matrix cores is the suggested alternative to the fused kernel).

One expert's up and down matrices are decoded by libsbm's sbm_decode_dense to
dense fp16 {-1, 0, +1} (exact), multiplied by library fp16 GEMMs with fp32
accumulation (torch.nn.functional.linear), and the per-row scales and the ReLU
are applied to the GEMM outputs.  The decode is the library's kernel; the GEMMs
are the platform's (hipBLASLt / rocBLAS), as the two-launch comparison needs.
"""
from __future__ import annotations

from . import api


def expert_ffn(up: "api.ExpertStack", down: "api.ExpertStack", e: int, image_t, x, wu=None, wd=None, bad=None,
               stream=None):
    """y = s_down * (W_down @ relu(s_up * (W_up @ x))) for the tokens x [T, d]
    of expert e, through dense fp16 copies of its matrices.  wu [f, d], wd
    [d, f]: optional preallocated fp16 buffers; bad: optional device uint32
    that sbm_decode_dense sets on a damaged image (1) or a dictionary mismatch
    (2).  Returns (y fp16 [T, d], h fp16 [T, f])."""
    import torch
    import torch.nn.functional as F
    du, dd = up.host_desc[e], down.host_desc[e]
    wu, bad = api.decode_dense(up, e, image_t, out=wu, bad=bad, stream=stream)
    wd, bad = api.decode_dense(down, e, image_t, out=wd, bad=bad, stream=stream)
    su = up.scales[du.scale_base:du.scale_base + up.rows]
    sd = down.scales[dd.scale_base:dd.scale_base + down.rows]
    h = torch.relu(F.linear(x, wu) * su)
    y = F.linear(h, wd) * sd
    return y, h
