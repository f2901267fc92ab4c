"""The layer call (sbm_moe_fused_ffn: up, ReLU and down of the routed tokens
in one launch) against two single-projection calls on the same inputs and
against the oracle on the GPU's own inputs, on all grouping paths, over
repeated calls on one workspace, a stack pass, and its error paths."""
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


@pytest.fixture(scope="module")
def c2048(dev):
    """One generated c2048-width layer of 24 experts (up 6144x2080, down 2080x6144)."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=1, n_experts=24, seed=47, n_tokens=64)
    return S.build(cfg, dev)


def _oracle_rows(cfg, layer, e, mat, rsel, inp):
    rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
    key = synth.matrix_key(cfg.seed, layer, e, mat, cfg.n_experts)
    sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
    sc = synth.scale_table()[synth.counter_scale_index(key, rows)][rsel]
    return P.oracle_matvec_from_symbols(sym, sc, np.asarray(inp, np.float16)[None, :])[0]


@pytest.mark.parametrize("T,in_rms,out_f32", [(64, False, False), (100, True, True), (200, False, True)])
def test_layer_call_matches_two_calls_and_oracle(dev, c2048, T, in_rms, out_f32):
    from sub_bit_moe_amd import api
    st = c2048
    cfg = st.cfg
    up, down = st.up[0], st.down[0]
    rng = np.random.default_rng(T)
    x = torch.from_numpy(synth.activations(rng, T, cfg.d_model) * 3).to(dev)
    ids_h = synth.zipf_routing(rng, T, cfg.n_experts).astype(np.int32)
    ids = torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_ffn_workspace(cfg.n_experts, T, dev)
    print(f"layer call T={T} in_rms={in_rms} out_f32={out_f32}", flush=True)
    # two single-projection calls on the same inputs
    h2 = api.moe_fused_decode_matvec(up, st.image, x, ids, relu=True, in_rms=in_rms)
    y2 = api.moe_fused_decode_matvec(down, st.image, h2, ids, out_f32=out_f32)
    for rep in range(3):            # the workspace is reused: each call leaves it ready
        y, h = api.moe_fused_ffn(up, down, st.image, x, ids, workspace=ws, in_rms=in_rms, out_f32=out_f32)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        assert bool((ws[64:64 + 4 * T] == 0).all()) and bool((ws[4:12] == 0).all())
        hn, yn = h.float().cpu().numpy(), y.float().cpu().numpy()
        P.assert_close(hn, h2.float().cpu().numpy(), what=f"h vs two calls, rep {rep}")
        P.assert_close(yn, y2.float().cpu().numpy(), what=f"y vs two calls, rep {rep}")
    xin = x.float().cpu().numpy().astype(np.float64)
    if in_rms:
        xin = OM.rms_glue(xin).astype(np.float16).astype(np.float64)
    sel = np.unique(np.concatenate([rng.choice(T, 5, replace=False), np.flatnonzero(ids_h == np.bincount(ids_h).argmax())[:3]]))
    for t in sel:
        e = int(ids_h[t])
        rs = np.sort(rng.choice(cfg.d_ff, 40, replace=False))
        P.assert_close(hn[t][rs], np.maximum(_oracle_rows(cfg, 0, e, 0, rs, xin[t]), 0), what=f"h token {t}")
        rs = np.sort(rng.choice(cfg.d_model, 40, replace=False))
        P.assert_close(yn[t][rs], _oracle_rows(cfg, 0, e, 1, rs, hn[t]), what=f"y token {t}")


def test_layer_stack_pass_against_oracle(dev):
    """A 3-layer stack of 64 experts with c2048 widths, 64 Zipf tokens, one
    launch per layer: sampled tokens and rows of every layer's h and y against
    the oracle on the GPU's own inputs to that layer."""
    from sub_bit_moe_amd import api, stack as S
    cfg = S.StackConfig(n_layers=3, n_experts=64, seed=43)
    st = S.build(cfg, dev)
    run = S.Runner(st, layer=True)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    assert api.workspace_error(run.ws_ffn) == 0
    rng = np.random.default_rng(5)
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        ids = st.routes_host[l]
        xin = OM.rms_glue(keep[l - 1][2].float().cpu().numpy()).astype(np.float64) if l else xraw
        for t in rng.choice(cfg.n_tokens, 6, replace=False):
            e = int(ids[t])
            rs = np.sort(rng.choice(cfg.d_ff, 48, replace=False))
            P.assert_close(h[t][rs], np.maximum(_oracle_rows(cfg, l, e, 0, rs, xin[t]), 0), what=f"layer {l} h {t}")
            rs = np.sort(rng.choice(cfg.d_model, 48, replace=False))
            P.assert_close(y[t][rs], _oracle_rows(cfg, l, e, 1, rs, h[t]), what=f"layer {l} y {t}")


@pytest.mark.parametrize("T", [20, 90, 160])
def test_layer_call_error_paths(dev, c2048, T):
    """Out-of-range ids are counted and get no rows; a damaged image computes
    nothing and sets bit 31; either way the workspace is left ready."""
    from sub_bit_moe_amd import api
    st = c2048
    cfg = st.cfg
    rng = np.random.default_rng(T + 1)
    x = torch.from_numpy(synth.activations(rng, T, cfg.d_model)).to(dev)
    ids_h = synth.zipf_routing(rng, T, cfg.n_experts).astype(np.int32)
    ids_h[:2] = [-3, cfg.n_experts]
    ids = torch.from_numpy(ids_h).to(dev)
    ws = api.alloc_ffn_workspace(cfg.n_experts, T, dev)
    y = torch.full((T, cfg.d_model), float("nan"), dtype=torch.float32, device=dev)
    api.moe_fused_ffn(st.up[0], st.down[0], st.image, x, ids, y=y, workspace=ws, out_f32=True)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 2
    yn = y.cpu().numpy()
    assert np.isnan(yn[:2]).all() and not np.isnan(yn[2:]).any()
    bad = torch.zeros_like(st.image)
    y.fill_(float("nan"))
    api.moe_fused_ffn(st.up[0], st.down[0], bad, x, ids, y=y, workspace=ws, out_f32=True)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == (0x80000000 | 2)
    assert bool(torch.isnan(y).all())
    y2, _ = api.moe_fused_ffn(st.up[0], st.down[0], st.image, x, ids, workspace=ws, out_f32=True)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 2
    assert np.allclose(y2.cpu().numpy()[2:], yn[2:], rtol=2e-3, atol=1e-3)


def test_layer_call_argument_errors(dev, c2048):
    """Shapes the layer call refuses before any launch (every buffer passed is
    the size the call's own shapes imply)."""
    from sub_bit_moe_amd import api
    from sub_bit_moe_amd import _native as N
    st = c2048
    x = torch.zeros((4, st.cfg.d_model), dtype=torch.float16, device=dev)
    ids = torch.zeros(4, dtype=torch.int32, device=dev)
    with pytest.raises(N.SbmError):          # up rows (6144) differ from down cols (2080)
        api.moe_fused_ffn(st.up[0], st.up[0], st.image, x, ids)
    E = st.cfg.n_experts
    small = api.ExpertStack.from_symbols([np.zeros((8, 256), np.uint8)] * E, [np.ones(8, np.float16)] * E,
                                         api.build_dictionary(0.885)[0], dev)
    small_dn = api.ExpertStack.from_symbols([np.zeros((256, 8), np.uint8)] * E, [np.ones(256, np.float16)] * E,
                                            api.build_dictionary(0.885)[0], dev)
    with pytest.raises(N.SbmError):          # rows narrower than 512 columns
        api.moe_fused_ffn(small, small_dn, st.image, torch.zeros((4, 256), dtype=torch.float16, device=dev), ids)


@pytest.mark.parametrize("T", [1, 3, 7])
def test_layer_call_phases_of_different_widths(dev, odict, T):
    """d_model 512, d_ff 2048: the up phase is cut into more workgroup slices
    than the down phase, so workgroups past the down phase's count skip it.
    Both outputs against two single-projection calls and the oracle."""
    from sub_bit_moe_amd import api
    E, d, f = 3, 512, 2048
    words = odict["words"]
    tag = api.dict_tag(words)
    ups = P.host_experts(E, f, d, 0.886, 60 + T)
    downs = P.host_experts(E, d, f, 0.886, 70 + T)
    up = api.ExpertStack.from_host(P.encode_all(ups, words), f, d, dev, dict_tag=tag)
    down = api.ExpertStack.from_host(P.encode_all(downs, words), d, f, dev, dict_tag=tag)
    image = api.device_image(words, dev)
    rng = np.random.default_rng(T)
    x = synth.activations(rng, T, d)
    ids_h = rng.integers(0, E, T).astype(np.int32)
    xt, ids = torch.from_numpy(x).to(dev), torch.from_numpy(ids_h).to(dev)
    print(f"layer call phases T={T}", flush=True)
    ws = api.alloc_ffn_workspace(E, T, dev)
    y, h = api.moe_fused_ffn(up, down, image, xt, ids, workspace=ws, out_f32=True)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    h2 = api.moe_fused_decode_matvec(up, image, xt, ids, relu=True)
    y2 = api.moe_fused_decode_matvec(down, image, h2, ids, out_f32=True)
    torch.cuda.synchronize()
    hn, yn = h.float().cpu().numpy(), y.cpu().numpy().astype(np.float64)
    P.assert_close(hn, h2.float().cpu().numpy(), what="h vs two calls")
    P.assert_close(yn, y2.cpu().numpy().astype(np.float64), what="y vs two calls")
    for t in range(T):
        e = int(ids_h[t])
        P.assert_close(hn[t], np.maximum(P.oracle_matvec_from_symbols(*ups[e], x[t:t + 1])[0], 0), what=f"h {t}")
        P.assert_close(yn[t], P.oracle_matvec_from_symbols(*downs[e], hn[t:t + 1].astype(np.float16))[0],
                       what=f"y {t}")
