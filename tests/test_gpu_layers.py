"""The multi-layer call (sbm_moe_fused_layers: n_layers MoE layers of up,
ReLU and down in one launch, each layer's up projection reading the previous
layer's output scaled to unit RMS): every layer's h and y against the oracle
on the GPU's own inputs to that layer, on all grouping paths (one wave, the
workgroup, the grouping launch), over repeated calls on one workspace, graph
replays, a c2048-width stack pass, and its error paths."""
import numpy as np
import pytest

from oracle import matvec as OM
from sub_bit_moe_amd import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _host_layers(odict, dev, L, E, d, f, seed):
    """L layers of E host-encoded experts: up f x d, down d x f (P(0) = 0.886)."""
    from sub_bit_moe_amd import api
    words = odict["words"]
    tag = api.dict_tag(words)
    ups, downs, su, sd = [], [], [], []
    for l in range(L):
        u = P.host_experts(E, f, d, 0.886, seed + 100 * l)
        w = P.host_experts(E, d, f, 0.886, seed + 100 * l + 50)
        ups.append(u)
        downs.append(w)
        su.append(api.ExpertStack.from_host(P.encode_all(u, words, odict if l == 0 else None), f, d, dev,
                                            dict_tag=tag))
        sd.append(api.ExpertStack.from_host(P.encode_all(w, words), d, f, dev, dict_tag=tag))
    return ups, downs, su, sd, api.device_image(words, dev)


def _check_layers(ups, downs, x, ids_h, h, y, in_rms, what, skip_y=()):
    """Every layer's h and y against the oracle on the GPU's own inputs;
    skip_y: (layer, expert) pairs whose y is not checked here."""
    L = len(ups)
    hn = h.float().cpu().numpy().astype(np.float64)
    yn = y.float().cpu().numpy().astype(np.float64)
    for l in range(L):
        if l == 0:
            xin = x.astype(np.float64)
            if in_rms:
                xin = OM.rms_glue(xin).astype(np.float16).astype(np.float64)
        else:
            xin = OM.rms_glue(yn[l - 1]).astype(np.float16).astype(np.float64)
        for e in np.unique(ids_h[l]):
            if e < 0 or e >= len(ups[l]):
                continue
            sel = np.flatnonzero(ids_h[l] == e)
            P.assert_close(hn[l][sel], np.maximum(P.oracle_matvec_from_symbols(*ups[l][e], xin[sel]), 0),
                           what=f"{what}: layer {l} h, expert {e}")
            if (l, e) in skip_y:
                continue
            P.assert_close(yn[l][sel], P.oracle_matvec_from_symbols(*downs[l][e], hn[l][sel].astype(np.float16)),
                           what=f"{what}: layer {l} y, expert {e}")


@pytest.mark.parametrize("L,T,in_rms", [(1, 1, False), (3, 12, False), (3, 64, True), (2, 100, False),
                                        (2, 150, True)])
def test_layers_against_oracle(dev, odict, L, T, in_rms):
    """T = 1 .. 64: in-wave grouping; 100: workgroup grouping; 150: one
    grouping launch per phase.  The workspace is reused over three calls and
    left ready by each."""
    from sub_bit_moe_amd import api
    E, d, f = 6, 512, 768
    print(f"layers L={L} T={T} in_rms={in_rms}", flush=True)
    ups, downs, su, sd, image = _host_layers(odict, dev, L, E, d, f, 900 + T)
    rng = np.random.default_rng(T + L)
    x = synth.activations(rng, T, d) * np.float16(2)
    ids_h = np.stack([synth.zipf_routing(rng, T, E) for _ in range(L)]).astype(np.int32)
    xt, ids = torch.from_numpy(x).to(dev), torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_layers_workspace(L, E, T, dev)
    for rep in range(3):
        y, h = api.moe_fused_layers(su, sd, image, xt, ids, workspace=ws, in_rms=in_rms)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        n_sync = 16 + 2 * L * T
        assert bool((ws[4:4 * n_sync] == 0).all()), "the sync area is left zeroed"
        _check_layers(ups, downs, x, ids_h, h, y, in_rms, f"rep {rep}")


def test_layers_graph_replays(dev, odict):
    """Graph replays of a 4-layer call, with eager work between them, against
    the eager call at the parity bound."""
    from sub_bit_moe_amd import api
    L, E, d, f, T = 4, 5, 512, 1024, 24
    ups, downs, su, sd, image = _host_layers(odict, dev, L, E, d, f, 77)
    rng = np.random.default_rng(3)
    x = torch.from_numpy(synth.activations(rng, T, d)).to(dev)
    ids_h = np.stack([synth.zipf_routing(rng, T, E) for _ in range(L)]).astype(np.int32)
    ids = torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_layers_workspace(L, E, T, dev)
    h = torch.empty((L, T, f), dtype=torch.float16, device=dev)
    y = torch.empty((L, T, d), dtype=torch.float16, device=dev)
    api.moe_fused_layers(su, sd, image, x, ids, h=h, y=y, workspace=ws)
    torch.cuda.synchronize()
    y_eager = y.float().clone()
    _check_layers(ups, downs, x.cpu().numpy(), ids_h, h, y, False, "eager")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_fused_layers(su, sd, image, x, ids, h=h, y=y, workspace=ws)
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        P.assert_close(y.float().cpu().numpy(), y_eager.cpu().numpy(), what=f"replay {rep}")
        _ = api.moe_fused_decode_matvec(su[0], image, x, ids[0], relu=True)     # other work in between
        torch.cuda.synchronize()


def test_layers_stack_pass_c2048(dev):
    """A 4-layer stack of 48 experts with c2048 widths (up 6144 x 2080, down
    2080 x 6144), 64 Zipf tokens, one launch: sampled tokens and rows of every
    layer's h and y against the oracle on the GPU's own inputs to that layer,
    and the whole output against the two-launch pass."""
    from sub_bit_moe_amd import api, stack as S
    cfg = S.StackConfig(n_layers=4, n_experts=48, seed=45)
    st = S.build(cfg, dev)
    run = S.Runner(st, layers=True)
    keep = {}
    yl = run.run_layers(keep).float().clone()
    torch.cuda.synchronize()
    assert api.workspace_error(run.ws_layers) == 0
    y2 = S.Runner(st).run_layers().float()
    torch.cuda.synchronize()
    # the layers compound fp16 roundings of differently ordered sums: a looser bound for the pass
    P.assert_close(yl.cpu().numpy(), y2.cpu().numpy(), rl2=4e-3, mr=4e-2, what="layers vs two launches")
    rng = np.random.default_rng(9)
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        ids = st.routes_host[l]
        xin = OM.rms_glue(xraw).astype(np.float16).astype(np.float64) if l else xraw.astype(np.float64)
        for t in rng.choice(cfg.n_tokens, 5, replace=False):
            e = int(ids[t])
            rs = np.sort(rng.choice(cfg.d_ff, 40, replace=False))
            ref = np.maximum(_oracle_rows(cfg, l, e, 0, rs, xin[t]), 0)
            P.assert_close(h[t][rs], ref, what=f"layer {l} h {t}")
            rs = np.sort(rng.choice(cfg.d_model, 40, replace=False))
            P.assert_close(y[t][rs], _oracle_rows(cfg, l, e, 1, rs, h[t]), what=f"layer {l} y {t}")


def _oracle_rows(cfg, layer, e, mat, rsel, inp):
    rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
    key = synth.matrix_key(cfg.seed, layer, e, mat, cfg.n_experts)
    sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
    sc = synth.scale_table()[synth.counter_scale_index(key, rows)][rsel]
    return P.oracle_matvec_from_symbols(sym, sc, np.asarray(inp, np.float16)[None, :])[0]


@pytest.mark.parametrize("T", [20, 100, 150])
def test_layers_error_paths(dev, odict, T):
    """Out-of-range ids (counted once per layer, no rows); a damaged image
    (nothing computed, bit 31); the workspace is left ready either way.  T =
    20 and 100: the planning launch's one-wave and workgroup grouping; 150:
    the grouping kernel."""
    from sub_bit_moe_amd import api
    L, E, d, f = 2, 4, 512, 768
    ups, downs, su, sd, image = _host_layers(odict, dev, L, E, d, f, 31)
    rng = np.random.default_rng(T)
    x = torch.from_numpy(synth.activations(rng, T, d)).to(dev)
    ids_h = np.stack([synth.zipf_routing(rng, T, E) for _ in range(L)]).astype(np.int32)
    ids_h[0, :2] = [-1, E]
    ids_h[1, 3] = E + 7
    ids = torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_layers_workspace(L, E, T, dev)
    y, h = api.moe_fused_layers(su, sd, image, x, ids, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 3
    bad = torch.zeros_like(image)
    api.moe_fused_layers(su, sd, bad, x, ids, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == (0x80000000 | 3)
    api.moe_fused_layers(su, sd, image, x, ids, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 3


def test_layers_argument_errors(dev, odict):
    """Calls refused before any launch."""
    from sub_bit_moe_amd import api
    from sub_bit_moe_amd import _native as N
    ups, downs, su, sd, image = _host_layers(odict, dev, 2, 3, 512, 768, 5)
    x = torch.zeros((4, 512), dtype=torch.float16, device=dev)
    ids = torch.zeros((2, 4), dtype=torch.int32, device=dev)
    with pytest.raises(N.SbmError):          # a layer with another shape
        api.moe_fused_layers([su[0], sd[0]], [sd[0], sd[1]], image, x, ids)
    with pytest.raises(N.SbmError):          # 33 layers
        api.moe_fused_layers([su[0]] * 33, [sd[0]] * 33, image, x, torch.zeros((33, 4), dtype=torch.int32,
                                                                              device=dev))


def test_layers_refused_expert_in_one_layer(dev, odict):
    """One expert of layer 1's down projection labelled as encoded under
    another dictionary: bit 29 and no rows for its tokens in that layer (they
    stay zero, so the next layer reads zero rows), no wait hangs on them, and
    every other row of every layer matches the oracle; with the label put
    back, the next call on the same workspace is clean."""
    from sub_bit_moe_amd import api
    from sub_bit_moe_amd import _native as N
    L, E, d, f, T = 3, 4, 512, 768, 40
    ups, downs, su, sd, image = _host_layers(odict, dev, L, E, d, f, 123)
    rng = np.random.default_rng(41)
    x = synth.activations(rng, T, d)
    ids_h = np.stack([synth.zipf_routing(rng, T, E) for _ in range(L)]).astype(np.int32)
    e_bad = int(np.bincount(ids_h[1], minlength=E).argmax())
    print(f"layers refused expert {e_bad} of layer 1", flush=True)
    xt, ids = torch.from_numpy(x).to(dev), torch.from_numpy(ids_h).to(dev)
    good = bytes((N.MatrixDesc * E)(*sd[1].host_desc))
    descs = list(sd[1].host_desc)
    descs[e_bad].dict_tag ^= 1
    sd[1].desc.copy_(torch.from_numpy(np.frombuffer(bytes((N.MatrixDesc * E)(*descs)), np.uint8).copy()))
    ws = api.alloc_layers_workspace(L, E, T, dev)
    h = torch.zeros((L, T, f), dtype=torch.float16, device=dev)
    y = torch.zeros((L, T, d), dtype=torch.float16, device=dev)
    api.moe_fused_layers(su, sd, image, xt, ids, h=h, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0x20000000
    bad_tok = ids_h[1] == e_bad
    assert bool((y[1][torch.from_numpy(bad_tok).to(dev)] == 0).all())
    _check_layers(ups, downs, x, ids_h, h, y, False, "refused", skip_y={(1, e_bad)})
    sd[1].desc.copy_(torch.from_numpy(np.frombuffer(good, np.uint8).copy()))
    descs[e_bad].dict_tag ^= 1
    y2, h2 = api.moe_fused_layers(su, sd, image, xt, ids, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    _check_layers(ups, downs, x, ids_h, h2, y2, False, "restored")


def test_layers_32_layers_128_bf16_tokens(dev, odict):
    """The longest call (32 layers) at the in-LDS grouping's largest token
    count (128), with bf16 activations into layer 0: every layer's h and y
    against the oracle on the GPU's own inputs to that layer."""
    from sub_bit_moe_amd import api
    L, E, d, f, T = 32, 3, 512, 512, 128
    print(f"layers L={L} T={T} bf16", flush=True)
    ups, downs, su, sd, image = _host_layers(odict, dev, L, E, d, f, 555)
    rng = np.random.default_rng(77)
    xb = torch.from_numpy(synth.activations(rng, T, d)).float().to(torch.bfloat16)
    ids_h = np.stack([rng.integers(0, E, T) for _ in range(L)]).astype(np.int32)
    ids = torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_layers_workspace(L, E, T, dev)
    y, h = api.moe_fused_layers(su, sd, image, xb.to(dev), ids, workspace=ws)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    _check_layers(ups, downs, xb.float().numpy(), ids_h, h, y, False, "32 layers")
