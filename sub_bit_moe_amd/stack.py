"""HBM-resident c2048-shaped MoE stack: generation on the GPU and one pass.

Shapes follow the QMoE page's c2048 model (section "Experimental setup" and
Figure 5's matrix shapes 2080x6144 / 6144x2080): every layer has E experts,
each an up projection W_up (f x d, d -> f, ReLU) and a down projection
W_down (d x f).  Weights are ternary with P(0) = 0.886 ("Natural sparsity",
Table 4) and per-row fp16 scales; they are generated and encoded on the GPU
from a counter-based generator, so nothing is ever materialised densely.

A pass sends T tokens through all layers: per layer each token's top-1 expert
(Zipf popularity, the cache-amplification page's routing statistics) applies
up + ReLU + down through the fused decode + matvec; between layers the token
is RMS-normalised (benchmark glue standing in for the absent transformer
block), inside the next up projection's activation staging, and once more
after the last layer.  Every step runs in libsbm's HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import api, synth


@dataclass
class StackConfig:
    n_layers: int = 30
    n_experts: int = 2048
    d_model: int = 2080
    d_ff: int = 6144
    p0: float = 0.886
    dict_p0: float = 0.885
    image_slots: int = 3         # 4: the 4-slot decode image (tables built for P(0) < 0.885)
    seed: int = 41
    n_tokens: int = 64
    zipf_s: float = 1.1


@dataclass
class Stack:
    cfg: StackConfig
    image: object
    up: list = field(default_factory=list)
    down: list = field(default_factory=list)
    routes: object = None        # torch int32 [L, T]
    routes_host: object = None   # numpy int32 [L, T]
    x0: object = None            # torch fp16 [T, d]

    def stored_bytes(self) -> int:
        """Every byte of the artefact on the device: codes (with alignment
        padding), row offsets, block starts, scales, descriptors."""
        tot = 0
        for s in self.up + self.down:
            tot += s.codes.numel() * 2 + s.row_off.numel() * 4 + s.bstart.numel() * 4
            tot += s.scales.numel() * 2 + s.desc.numel()
        return tot

    def n_params(self) -> int:
        c = self.cfg
        return c.n_layers * c.n_experts * 2 * c.d_model * c.d_ff

    def touched(self, layer: int):
        """Experts that receive tokens in this layer."""
        return np.unique(self.routes_host[layer])

    def pass_bytes(self):
        """(compressed bytes read by one pass, bf16-equivalent bytes) over the
        touched (expert, matrix) pairs of all layers."""
        comp = 0
        bf16 = 0
        c = self.cfg
        for l in range(c.n_layers):
            for e in self.touched(l):
                comp += self.up[l].matrix_bytes(int(e)) + self.down[l].matrix_bytes(int(e))
                bf16 += 2 * 2 * c.d_model * c.d_ff
        return comp, bf16


def build(cfg: StackConfig, device="cuda", log=None) -> Stack:
    import torch
    words, checksum = api.build_dictionary(cfg.dict_p0)
    st = Stack(cfg, api.device_image(words, device, cfg.image_slots))
    trie = torch.from_numpy(api.build_trie(words)).to(device)
    table = torch.from_numpy(synth.scale_table().view(np.int16)).to(device)
    for l in range(cfg.n_layers):
        st.up.append(api.generate_stack(cfg.seed, l, cfg.n_experts, 0, cfg.d_ff, cfg.d_model, cfg.p0, trie, table,
                                           dict_checksum=checksum))
        st.down.append(api.generate_stack(cfg.seed, l, cfg.n_experts, 1, cfg.d_model, cfg.d_ff, cfg.p0, trie, table,
                                             dict_checksum=checksum))
        if log:
            log(f"layer {l + 1}/{cfg.n_layers} generated")
    routes = np.stack([synth.zipf_routing(np.random.default_rng(cfg.seed * 1000 + l), cfg.n_tokens,
                                          cfg.n_experts, cfg.zipf_s) for l in range(cfg.n_layers)])
    st.routes_host = routes.astype(np.int32)
    st.routes = torch.from_numpy(st.routes_host).to(device)
    st.x0 = torch.from_numpy(synth.activations(np.random.default_rng(cfg.seed + 1), cfg.n_tokens,
                                               cfg.d_model)).to(device)
    torch.cuda.synchronize()
    return st


def with_minmax(st: Stack, seed: int = 7) -> Stack:
    """The same code streams on the page's per-row grid {w_min, 0, w_max}:
    (w_min, w_max) = (-s v, s u) per row, s the row's symmetric scale and u, v
    ~ U(0.6, 1.4) from a seeded device generator; descriptors with doubled
    scale bases (two fp16 per row)."""
    import dataclasses
    import ctypes
    import torch
    g = torch.Generator(device=st.x0.device)
    g.manual_seed(seed)

    def conv(es):
        s = es.scales.float()
        u = torch.empty_like(s).uniform_(0.6, 1.4, generator=g)
        v = torch.empty_like(s).uniform_(0.6, 1.4, generator=g)
        mm = torch.stack([-s * v, s * u], dim=1).half().contiguous()
        d = es.desc.view(torch.int64).view(es.n_experts, 6).clone()   # field 2: scale_base
        d[:, 2] *= 2
        hd = []
        for x in es.host_desc:
            y = type(x).from_buffer_copy(bytes(x))
            y.scale_base = 2 * x.scale_base
            hd.append(y)
        return dataclasses.replace(es, scales=mm, desc=d.view(torch.uint8).reshape(-1), host_desc=hd)

    out = Stack(st.cfg, st.image, [conv(e) for e in st.up], [conv(e) for e in st.down], st.routes,
                st.routes_host, st.x0)
    torch.cuda.synchronize()
    return out


class Runner:
    """Preallocated buffers for repeated passes (minmax: the stack's scales
    are (w_min, w_max) pairs; deterministic: fixed-point row accumulators)."""

    def __init__(self, st: Stack, minmax: bool = False, layer: bool = False, deterministic: bool = False,
                 layers: bool = False):
        import torch
        c = st.cfg
        dev = st.x0.device
        self.st = st
        self.minmax = minmax
        self.det = deterministic
        self.layer = layer and not minmax and not deterministic   # one launch per layer (sbm_moe_fused_ffn)
        # one launch for all layers (sbm_moe_fused_layers, up to 32 layers per launch)
        self.layers = layers and not minmax and not deterministic and not self.layer
        self.ws_layers = (api.alloc_layers_workspace(min(c.n_layers, 32), c.n_experts, c.n_tokens, dev)
                          if self.layers else None)
        if self.layers:     # every layer's h and output
            self.h_all = torch.empty(c.n_layers, c.n_tokens, c.d_ff, dtype=torch.float16, device=dev)
            self.y_all = torch.empty(c.n_layers, c.n_tokens, c.d_model, dtype=torch.float16, device=dev)
        self.ws_ffn = api.alloc_ffn_workspace(c.n_experts, c.n_tokens, dev) if self.layer else None
        # a layer call reads x while other workgroups already write y: consecutive layers alternate buffers
        self.y2 = [torch.empty(c.n_tokens, c.d_model, dtype=torch.float16, device=dev) for _ in range(2)]
        self.ws_up = api.alloc_workspace(c.n_experts, c.n_tokens, dev)
        self.ws_down = api.alloc_workspace(c.n_experts, c.n_tokens, dev)
        self.h = torch.empty(c.n_tokens, c.d_ff, dtype=torch.float16, device=dev)
        self.y = torch.empty(c.n_tokens, c.d_model, dtype=torch.float16, device=dev)
        self.x = [torch.empty(c.n_tokens, c.d_model, dtype=torch.float16, device=dev) for _ in range(2)]

    def run(self, keep=None):
        """One pass over all layers, then the glue on the last output.  keep:
        optional dict filled with the per-layer (input, h, y) device tensors
        for checking; from layer 1 on the input is the previous y, which the up
        projection scales to unit RMS itself (the glue fused into its
        activation staging)."""
        y = self.run_layers(keep)
        return api.rms_glue(y, out=self.x[0])

    def run_layers(self, keep=None):
        """The fused launches of one pass (1 per layer with layer=True, else 2),
        nothing else."""
        st = self.st
        x = st.x0
        if self.layers:
            # up to 32 layers per launch; every layer's h and y are kept
            L = st.cfg.n_layers
            for l0 in range(0, L, 32):
                l1 = min(L, l0 + 32)
                api.moe_fused_layers(st.up[l0:l1], st.down[l0:l1], st.image, x, st.routes[l0:l1],
                                     h=self.h_all[l0:l1], y=self.y_all[l0:l1], workspace=self.ws_layers,
                                     in_rms=l0 > 0)
                x = self.y_all[l1 - 1]
            if keep is not None:
                for l in range(L):
                    keep[l] = ((st.x0 if l == 0 else self.y_all[l - 1]).clone(), self.h_all[l].clone(),
                               self.y_all[l].clone())
            return x
        for l in range(st.cfg.n_layers):
            ids = st.routes[l]
            if self.layer:
                y = self.y2[l & 1]
                api.moe_fused_ffn(st.up[l], st.down[l], st.image, x, ids, h=self.h, y=y, workspace=self.ws_ffn,
                                  in_rms=l > 0)
                if keep is not None:
                    keep[l] = (x.clone(), self.h.clone(), y.clone())
                x = y
                continue
            api.moe_fused_decode_matvec(st.up[l], st.image, x, ids, relu=True, workspace=self.ws_up, y=self.h,
                                        in_rms=l > 0, minmax=self.minmax, deterministic=self.det)
            if keep is not None:
                keep[l] = (x.clone(), self.h.clone())
            api.moe_fused_decode_matvec(st.down[l], st.image, self.h, ids, workspace=self.ws_down, y=self.y,
                                        minmax=self.minmax, deterministic=self.det)
            if keep is not None:
                keep[l] = keep[l] + (self.y.clone(),)
            x = self.y
        return x
