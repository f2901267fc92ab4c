"""GPU parity: the HIP path through the C ABI against the oracle."""
import numpy as np
import pytest

from oracle import codec as OC
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def lib_state(dev, odict):
    from sub_bit_moe_amd import api
    words = odict["words"]
    lw, _ = api.build_dictionary(0.885)
    assert np.array_equal(lw, words)
    return {"api": api, "words_t": torch.from_numpy(words.view(np.int32)).to(dev),
            "image_t": api.device_image(words, dev)}


def _to_dev(a, dt, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)


@pytest.mark.parametrize("rows,cols,p0,seed", [(768, 3072, 0.886, 1), (37, 30, 0.886, 2), (5, 2, 0.5, 3),
                                               (129, 2080, 0.857, 4), (3, 6144, 0.0, 5)])
def test_decode_ref_bit_exact(dev, lib_state, odict, rows, cols, p0, seed):
    print(f"decode_ref {rows}x{cols} p0={p0}", flush=True)
    api = lib_state["api"]
    sym = P.host_experts(1, rows, cols, p0, seed)[0][0]
    codes, row_off, _ = P.encode_all([(sym, np.ones(rows, np.float16))], odict["words"], odict)[0][:3]
    out, bad = api.decode_ref(_to_dev(codes, np.int16, dev), _to_dev(row_off, np.int32, dev), rows, cols,
                              lib_state["words_t"])
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert np.array_equal(out.cpu().numpy(), sym)


def test_decode_ref_flags_truncated_rows(dev, lib_state, odict):
    api = lib_state["api"]
    sym = P.host_experts(1, 6, 60, 0.886, 8)[0][0]
    codes, row_off, _ = api.encode_matrix(sym, odict["words"])
    bad_off = row_off.copy()
    bad_off[2] -= 1                     # row 1 loses a codeword, row 2 gains one
    out, bad = api.decode_ref(_to_dev(codes, np.int16, dev), _to_dev(bad_off, np.int32, dev), 6, 60,
                              lib_state["words_t"])
    torch.cuda.synchronize()
    assert int(bad.item()) == 2


def _run(lib_state, experts, rows, cols, x, ids, dev, odict, relu=False, out_f32=False, check_every=1,
         mfma=False):
    api = lib_state["api"]
    mats = P.encode_all(experts, odict["words"], odict, check_every)
    stack = api.ExpertStack.from_host(mats, rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    xt = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    it = torch.from_numpy(np.asarray(ids, np.int32)).to(dev)
    ws = api.alloc_workspace(stack.n_experts, x.shape[0], dev)
    y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=relu, out_f32=out_f32,
                                    workspace=ws, mfma=mfma)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), api.workspace_error(ws)


@pytest.mark.parametrize("rows,cols,p0,T", [(768, 3072, 0.886, 1), (300, 512, 0.886, 3),
                                            (64, 30, 0.886, 2), (200, 2, 0.7, 1), (33, 254, 0.857, 5),
                                            (1000, 256, 0.886, 4), (17, 6144, 0.886, 2)])
def test_fused_single_expert(dev, lib_state, odict, rows, cols, p0, T):
    print(f"fused single {rows}x{cols} T={T}", flush=True)
    ex = P.host_experts(1, rows, cols, p0, rows + cols)
    x = np.random.default_rng(5).standard_normal((T, cols)).astype(np.float16)
    ref = P.oracle_matvec_from_codes(odict, ex[0][0], ex[0][1], x)
    for out_f32 in (False, True):
        y, err = _run(lib_state, ex, rows, cols, x, np.zeros(T, np.int32), dev, odict, out_f32=out_f32)
        assert err == 0
        P.assert_close(y, ref, what=f"{rows}x{cols} T={T} f32={out_f32}")
        if out_f32:
            P.assert_close(y, ref, 2e-6, 2e-5, what="fp32 output")


@pytest.mark.parametrize("rows,cols,T", [(300, 2080, 3), (130, 6144, 2), (64, 98, 5), (40, 512, 9),
                                         (200, 512, 50), (90, 770, 48)])
def test_fused_input_rms(dev, lib_state, odict, rows, cols, T):
    """SBM_F_IN_RMS: each token row is first scaled to unit RMS (the stack
    glue), including a zero row, which stays zero; at T >= 48 every expert
    has at least 16 tokens and the call asks for the dense-tile path."""
    from oracle import matvec as OM
    api = lib_state["api"]
    E = 3
    ex = P.host_experts(E, rows, cols, 0.886, rows + 7)
    stack = api.ExpertStack.from_host(P.encode_all(ex, odict["words"]), rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    rng = np.random.default_rng(cols)
    x = (rng.standard_normal((T, cols)) * rng.uniform(0.01, 40, (T, 1))).astype(np.float16)
    x[1] = 0
    ids = (np.arange(T) % E).astype(np.int32)
    ws = api.alloc_workspace(E, T, dev)
    y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], torch.from_numpy(x).to(dev),
                                    torch.from_numpy(ids).to(dev), out_f32=True, workspace=ws, in_rms=True,
                                    mfma=T >= 48)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    yn = y.cpu().numpy().astype(np.float64)
    xn = OM.rms_glue(x)
    for t in range(T):
        ref = P.oracle_matvec_from_symbols(*ex[ids[t]], xn[t:t + 1])[0]
        if t == 1:
            assert not np.any(yn[t])
        else:
            P.assert_close(yn[t], ref, what=f"in_rms token {t}")


def test_fused_exact_special_inputs(dev, lib_state, odict):
    rows, cols = 257, 2080
    sym, sc = P.host_experts(1, rows, cols, 0.886, 77)[0]
    js = [0, 1, 27, 28, 1039, 2079]
    x = np.zeros((len(js) + 1, cols), np.float16)
    for i, j in enumerate(js):
        x[i, j] = 1.0
    x[-1, :] = 1.0
    y, _ = _run(lib_state, [(sym, sc)], rows, cols, x, np.zeros(len(x), np.int32), dev, odict, out_f32=True)
    tern = (sym == 2).astype(np.float64) - (sym == 1)
    s = sc.astype(np.float64)
    for i, j in enumerate(js):
        assert np.array_equal(y[i], s * tern[:, j])
    assert np.array_equal(y[-1], s * tern.sum(1))
    zero = [(np.zeros((rows, cols), np.uint8), sc)]
    y0, _ = _run(lib_state, zero, rows, cols, x, np.zeros(len(x), np.int32), dev, odict, out_f32=True)
    assert not np.any(y0)


def test_fused_grouped_routing_and_edges(dev, lib_state, odict):
    E, rows, cols = 12, 300, 512
    ex = P.host_experts(E, rows, cols, 0.886, 99)
    rng = np.random.default_rng(3)
    for T in (1, 8, 32, 37, 129):
        x = rng.standard_normal((T, cols)).astype(np.float16)
        ids = rng.integers(0, E, T).astype(np.int32)
        ids[: T // 2] = 4                      # one heavy expert; several experts stay empty
        y, err = _run(lib_state, ex, rows, cols, x, ids, dev, odict, relu=True, check_every=4)
        assert err == 0
        for t in range(T):
            ref = np.maximum(P.oracle_matvec_from_symbols(*ex[ids[t]], x[t:t + 1])[0], 0)
            P.assert_close(y[t], ref, what=f"T={T} token {t}")


@pytest.mark.parametrize("rows,cols,counts", [(300, 512, (16, 3, 40)), (130, 6144, (17, 1)),
                                               (77, 98, (64, 65, 2)), (100, 2080, (100, 16)),
                                               (45, 770, (33,)), (6, 4, (20, 1))])
def test_fused_heavy_experts_dense_tiles(dev, lib_state, odict, rows, cols, counts):
    """With SBM_F_MFMA, experts with 16 or more tokens run on the dense-tile
    path (items of up to 64 tokens, row tiles with a ragged last tile), the
    rest on the sparse path; both, and the sparse path alone, against the
    oracle."""
    E = len(counts)
    ex = P.host_experts(E, rows, cols, 0.886, rows * 7 + cols)
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    ids = ids[np.random.default_rng(cols).permutation(ids.size)]
    T = ids.size
    x = np.random.default_rng(rows).standard_normal((T, cols)).astype(np.float16)
    ref = np.empty((T, rows))
    for e in range(E):
        tok = np.flatnonzero(ids == e)
        ref[tok] = P.oracle_matvec_from_symbols(*ex[e], x[tok])
    for mfma in (True, False):
        print(f"heavy {rows}x{cols} counts={counts} mfma={mfma}", flush=True)
        for out_f32 in (True, False):
            y, err = _run(lib_state, ex, rows, cols, x, ids, dev, odict, out_f32=out_f32, mfma=mfma)
            assert err == 0
            for e in range(E):
                tok = np.flatnonzero(ids == e)
                P.assert_close(y[tok], ref[tok], what=f"expert {e} ({counts[e]} tokens) mfma={mfma} f32={out_f32}")
                if out_f32:
                    P.assert_close(y[tok], ref[tok], 2e-6, 2e-5, what="fp32 output")


@pytest.mark.parametrize("T", [4, 64, 100, 140])
def test_fused_invalid_ids_are_skipped_and_counted(dev, lib_state, odict, T):
    """Up to 128 tokens are grouped inside the fused kernel, more by the
    grouping kernel: both count out-of-range ids and leave their rows alone."""
    api = lib_state["api"]
    E, rows, cols = 3, 64, 256
    ex = P.host_experts(E, rows, cols, 0.886, 5)
    mats = P.encode_all(ex, odict["words"])
    stack = api.ExpertStack.from_host(mats, rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    x = np.random.default_rng(1).standard_normal((T, cols)).astype(np.float16)
    ids = np.random.default_rng(2).integers(0, E, T).astype(np.int32)
    ids[:4] = [0, -1, 7, 2]
    bad = (ids < 0) | (ids >= E)
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(E, T, dev)
    api.moe_fused_decode_matvec(stack, lib_state["image_t"], torch.from_numpy(x).to(dev),
                                torch.from_numpy(ids).to(dev), out_f32=True, workspace=ws, y=y)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == int(bad.sum())
    yn = y.cpu().numpy()
    assert np.isnan(yn[bad]).all()
    for t in np.flatnonzero(~bad)[:12]:
        P.assert_close(yn[t], P.oracle_matvec_from_symbols(*ex[ids[t]], x[t:t + 1])[0])


@pytest.mark.parametrize("T", [5, 90, 150])
def test_fused_bad_descriptor_is_flagged(dev, lib_state, odict, T):
    """An expert whose descriptor disagrees with the call's shape produces no
    rows and sets the descriptor bit of the error word; the others are exact."""
    import ctypes
    from sub_bit_moe_amd import _native as N
    api = lib_state["api"]
    E, rows, cols = 3, 64, 256
    ex = P.host_experts(E, rows, cols, 0.886, 6)
    stack = api.ExpertStack.from_host(P.encode_all(ex, odict["words"]), rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    descs = list(stack.host_desc)
    descs[1].rows = rows + 1
    arr = (N.MatrixDesc * E)(*descs)
    stack.desc.copy_(torch.from_numpy(np.frombuffer(bytes(arr), np.uint8).copy()))
    x = np.random.default_rng(3).standard_normal((T, cols)).astype(np.float16)
    ids = (np.arange(T) % E).astype(np.int32)
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(E, T, dev)
    api.moe_fused_decode_matvec(stack, lib_state["image_t"], torch.from_numpy(x).to(dev),
                                torch.from_numpy(ids).to(dev), out_f32=True, workspace=ws, y=y)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0x40000000
    yn = y.cpu().numpy()
    assert np.isnan(yn[ids == 1]).all()
    for t in np.flatnonzero(ids != 1)[:8]:
        P.assert_close(yn[t], P.oracle_matvec_from_symbols(*ex[ids[t]], x[t:t + 1])[0])


def test_base128_layer_grouped(dev, lib_state, odict):
    """128 experts, up 3072x768 and down 768x3072 at P(0)=0.857, 128 tokens
    top-1 Zipf(1.1); the down projection runs on the GPU's own relu(up)."""
    from sub_bit_moe_amd import synth
    E, T = 128, 128
    rng = np.random.default_rng(11)
    ups = [(synth.ternary_symbols(rng, 3072, 768, 0.857), synth.row_scales(rng, 3072)) for _ in range(E)]
    downs = [(synth.ternary_symbols(rng, 768, 3072, 0.857), synth.row_scales(rng, 768)) for _ in range(E)]
    rng2 = np.random.default_rng(12)
    x = synth.activations(rng2, T, 768)
    ids = synth.zipf_routing(np.random.default_rng(13), T, E)
    h, err = _run(lib_state, ups, 3072, 768, x, ids, dev, odict, relu=True, check_every=16)
    assert err == 0
    h16 = h.astype(np.float16)
    y, err = _run(lib_state, downs, 768, 3072, h16, ids, dev, odict, check_every=16)
    assert err == 0
    sample = np.unique(np.concatenate([np.random.default_rng(14).choice(T, 24, replace=False),
                                       np.flatnonzero(ids == np.bincount(ids).argmax())[:4]]))
    for t in sample:
        e = ids[t]
        ref_h = np.maximum(P.oracle_matvec_from_symbols(*ups[e], x[t:t + 1])[0], 0)
        P.assert_close(h[t], ref_h, what=f"up token {t}")
        ref_y = P.oracle_matvec_from_symbols(*downs[e], h16[t:t + 1])[0]
        P.assert_close(y[t], ref_y, what=f"down token {t}")


@pytest.mark.parametrize("T", [1, 8, 32])
def test_c2048_pair(dev, lib_state, odict, T):
    """One c2048-shaped pair: up 6144x2080, down 2080x6144, P(0)=0.886, all
    T tokens routed to it."""
    from sub_bit_moe_amd import synth
    rng = np.random.default_rng(21)
    up = (synth.ternary_symbols(rng, 6144, 2080, 0.886), synth.row_scales(rng, 6144))
    down = (synth.ternary_symbols(rng, 2080, 6144, 0.886), synth.row_scales(rng, 2080))
    x = synth.activations(np.random.default_rng(22 + T), T, 2080)
    ids = np.zeros(T, np.int32)
    h, err = _run(lib_state, [up], 6144, 2080, x, ids, dev, odict, relu=True)
    assert err == 0
    h16 = h.astype(np.float16)
    y, err = _run(lib_state, [down], 2080, 6144, h16, ids, dev, odict)
    assert err == 0
    ref_h = np.maximum(P.oracle_matvec_from_symbols(*up, x), 0)
    ref_y = P.oracle_matvec_from_symbols(*down, h16)
    for t in range(T):
        P.assert_close(h[t], ref_h[t], what=f"up t={t}")
        P.assert_close(y[t], ref_y[t], what=f"down t={t}")


@pytest.mark.parametrize("T,d", [(64, 2080), (3, 6144), (5, 98)])
def test_rms_glue_kernel(dev, T, d):
    """The stack glue launch (once per pass) against its fp64 form: fp16 of
    y / rms(y) per token, a zero row staying zero; at most one fp16 ulp apart
    (fp32 against fp64 sums of squares)."""
    from oracle import matvec as OM
    from sub_bit_moe_amd import api
    rng = np.random.default_rng(d)
    y = (rng.standard_normal((T, d)) * rng.uniform(0.01, 30, (T, 1))).astype(np.float16)
    y[T // 2] = 0
    out = api.rms_glue(torch.from_numpy(y).to(dev))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = OM.rms_glue(y)
    assert not np.any(got[T // 2])
    ulp = np.abs(got.view(np.int16).astype(np.int32) - ref.view(np.int16).astype(np.int32))
    assert ulp.max() <= 1, f"max {ulp.max()} fp16 ulps"


@pytest.mark.parametrize("rows,cols,T,E", [(300, 2080, 5, 3), (130, 6144, 3, 2), (64, 98, 7, 2),
                                           (45, 770, 9, 3), (200, 512, 1, 1), (40, 2080, 70, 4),
                                           (33, 1024, 140, 5)])
def test_fused_minmax_grid(dev, lib_state, odict, rows, cols, T, E):
    """SBM_F_MINMAX: the page's per-row grid {w_min, 0, w_max} with
    asymmetric values, against the oracle's dequantisation on that grid; the
    three grouping paths (<= 64, <= 128, > 128 tokens), ReLU and fp32 output."""
    from sub_bit_moe_amd import synth
    print(f"fused minmax {rows}x{cols} T={T} E={E}", flush=True)
    api = lib_state["api"]
    rng = np.random.default_rng(rows * 7 + cols)
    syms = [synth.ternary_symbols(rng, rows, cols, 0.886) for _ in range(E)]
    mms = [synth.row_minmax(rng, rows) for _ in range(E)]
    mats = P.encode_all(list(zip(syms, mms)), odict["words"], odict)
    stack = api.ExpertStack.from_host(mats, rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    x = rng.standard_normal((T, cols)).astype(np.float16)
    ids = (np.arange(T) * 7 + T) % E
    ids = ids.astype(np.int32)
    ref = np.zeros((T, rows))
    for e in range(E):
        sel = np.nonzero(ids == e)[0]
        if sel.size:
            ref[sel] = P.oracle_matvec_minmax_from_codes(odict, syms[e], mms[e], x[sel])
    xt = torch.from_numpy(x).to(dev)
    it = torch.from_numpy(ids).to(dev)
    ws = api.alloc_workspace(E, T, dev)
    for relu, out_f32 in ((False, False), (True, True)):
        y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=relu, out_f32=out_f32,
                                        workspace=ws, minmax=True)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        exp = np.maximum(ref, 0) if relu else ref
        P.assert_close(y.float().cpu().numpy().astype(np.float64), exp, what=f"minmax relu={relu} f32={out_f32}")


def test_fused_minmax_input_rms_and_symmetric_case(dev, lib_state, odict):
    """SBM_F_MINMAX with SBM_F_IN_RMS; and w_min = -w_max gives the symmetric
    path's result."""
    from oracle import matvec as OM
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rows, cols, T, E = 150, 2080, 6, 2
    rng = np.random.default_rng(99)
    syms = [synth.ternary_symbols(rng, rows, cols, 0.886) for _ in range(E)]
    mms = [synth.row_minmax(rng, rows) for _ in range(E)]
    x = rng.standard_normal((T, cols)).astype(np.float16)
    x[1] = 0
    ids = (np.arange(T) % E).astype(np.int32)
    xn = OM.rms_glue(x.astype(np.float64))
    ref = np.zeros((T, rows))
    for e in range(E):
        sel = np.nonzero(ids == e)[0]
        ref[sel] = P.oracle_matvec_minmax_from_codes(odict, syms[e], mms[e], xn[sel])
    stack = api.ExpertStack.from_host(P.encode_all(list(zip(syms, mms)), odict["words"]), rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    xt, it = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
    y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, in_rms=True, out_f32=True, minmax=True)
    torch.cuda.synchronize()
    P.assert_close(y.cpu().numpy().astype(np.float64), ref, what="minmax + in_rms")
    # symmetric grid as a special case: (-s, s) pairs against the one-scale path
    ss = [synth.row_scales(rng, rows) for _ in range(E)]
    mats1 = P.encode_all(list(zip(syms, ss)), odict["words"])
    mats2 = [(c, o, b, np.stack([-s, s], axis=1)) for (c, o, b, s) in mats1]
    y1 = api.moe_fused_decode_matvec(api.ExpertStack.from_host(mats1, rows, cols, dev, dict_tag=api.dict_tag(odict["words"])), lib_state["image_t"],
                                     xt, it, out_f32=True)
    y2 = api.moe_fused_decode_matvec(api.ExpertStack.from_host(mats2, rows, cols, dev, dict_tag=api.dict_tag(odict["words"])), lib_state["image_t"],
                                     xt, it, out_f32=True, minmax=True)
    torch.cuda.synchronize()
    P.assert_close(y2.cpu().numpy().astype(np.float64), y1.cpu().numpy().astype(np.float64), 1e-5, 1e-4,
                   what="minmax(-s, s) vs symmetric")


def test_fused_size_limits(dev, lib_state, odict):
    """Widths near the LDS limit (one activation row of 15000 columns plus its
    wrap copy), a width past it (SBM_ERANGE), and a matrix at the 30-bit
    position limit (80000 x 2080) checked on sampled rows against the oracle's
    dense product of the symbols."""
    from sub_bit_moe_amd import _native as N
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rng = np.random.default_rng(2024)
    # near the widest row that fits
    rows, cols, T = 70, 15000, 3
    ex = P.host_experts(1, rows, cols, 0.886, 5)
    x = rng.standard_normal((T, cols)).astype(np.float16)
    y, err = _run(lib_state, ex, rows, cols, x, np.zeros(T, np.int32), dev, odict, out_f32=True)
    assert err == 0
    P.assert_close(y, P.oracle_matvec_from_symbols(ex[0][0], ex[0][1], x), what="cols=15000")
    # too wide for LDS: rejected before any launch
    wide = P.encode_all([(np.zeros((2, 16384), np.uint8), np.ones(2, np.float16))], odict["words"])
    st = api.ExpertStack.from_host(wide, 2, 16384, dev, dict_tag=api.dict_tag(odict["words"]))
    with pytest.raises(N.SbmError) as e:
        api.moe_fused_decode_matvec(st, lib_state["image_t"], torch.zeros((1, 16384), dtype=torch.float16, device=dev),
                                    torch.zeros(1, dtype=torch.int32, device=dev))
    assert e.value.status == -5
    # at the position limit: rows * cols * 6 just under 2^30
    rows, cols, T = 80000, 2080, 2
    assert rows * cols * 6 + 1024 * 28 * 6 < (1 << 30)
    sym = synth.ternary_symbols(rng, rows, cols, 0.886)
    sc = synth.row_scales(rng, rows)
    codes, row_off, bstart = api.encode_matrix(sym, odict["words"])
    st = api.ExpertStack.from_host([(codes, row_off, bstart, sc)], rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    x = rng.standard_normal((T, cols)).astype(np.float16)
    yt = api.moe_fused_decode_matvec(st, lib_state["image_t"], torch.from_numpy(x).to(dev),
                                     torch.zeros(T, dtype=torch.int32, device=dev), out_f32=True)
    torch.cuda.synchronize()
    y = yt.cpu().numpy().astype(np.float64)
    rsel = np.sort(np.concatenate([rng.choice(rows, 60, replace=False), [0, rows - 1]]))
    ref = P.oracle_matvec_from_symbols(sym[rsel], sc[rsel], x)
    P.assert_close(y[:, rsel], ref, what="80000 x 2080 sampled rows")
    assert not np.isnan(y).any()


def test_fused_random_shapes(dev, lib_state, odict):
    """A seeded sweep of valid shapes: even widths 2..3000 (ragged and not
    multiples of 8), 1..700 rows, 1..160 tokens over 1..9 experts (all three
    grouping paths), P(0) in [0.5, 0.95], both grids, ReLU and fp32 output."""
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rng = np.random.default_rng(77)
    for case in range(18):
        cols = int(rng.choice([2, 6, 30, 98, 254, 510, 512, 514, 770, 1026, 2080, 3000]))
        rows = int(rng.integers(1, 700))
        E = int(rng.integers(1, 10))
        T = int(rng.choice([1, 2, 5, 17, 64, 65, 128, 129, 160]))
        p0 = float(rng.uniform(0.5, 0.95))
        minmax = bool(case % 3 == 2)
        relu, out_f32 = bool(case % 2), bool(case % 4 == 1)
        print(f"case {case}: {rows}x{cols} E={E} T={T} p0={p0:.3f} minmax={minmax}", flush=True)
        syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
        scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
        stack = api.ExpertStack.from_host(P.encode_all(list(zip(syms, scs)), odict["words"]), rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
        x = rng.standard_normal((T, cols)).astype(np.float16)
        ids = rng.integers(0, E, T).astype(np.int32)
        y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], torch.from_numpy(x).to(dev),
                                        torch.from_numpy(ids).to(dev), relu=relu, out_f32=out_f32, minmax=minmax)
        torch.cuda.synchronize()
        y = y.float().cpu().numpy().astype(np.float64)
        for e in range(E):
            sel = np.nonzero(ids == e)[0]
            if not sel.size:
                continue
            if minmax:
                ref = P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], x[sel])
            else:
                ref = P.oracle_matvec_from_symbols(syms[e], scs[e], x[sel])
            if relu:
                ref = np.maximum(ref, 0)
            P.assert_close(y[sel], ref, what=f"case {case} expert {e}")


@pytest.mark.parametrize("p0,rows,cols,E,T,minmax,seed", [
    (0.857, 768, 3072, 6, 64, False, 1),     # base128 down shape, table built for its P(0)
    (0.857, 3072, 768, 6, 129, False, 2),    # up shape; > 128 tokens: grouping in its own launch
    (0.864, 300, 514, 3, 17, False, 3),      # large128 sparsity; wrap copy, ragged rows
    (0.857, 70, 98, 4, 100, False, 4),       # narrow rows: a lane spans several rows
    (0.857, 257, 2080, 3, 9, True, 5),       # per-row (w_min, w_max) grid on the 4-slot image
    (0.885, 129, 2080, 5, 33, False, 6),     # the page's static table through the 4-slot instance
    (0.87, 1, 6144, 2, 3, False, 7),         # one 6144-wide row
])
def test_fused_image4_matched_dictionary(dev, lib_state, odict_for, p0, rows, cols, E, T, minmax, seed):
    """A dictionary built for the data's P(0) (entries with 4 nonzeros) through
    the 4-slot decode image: codes bit-exact with the oracle's encoder under
    that table, y against the oracle's decode of those codes."""
    print(f"image4 p0={p0} {rows}x{cols} E={E} T={T} minmax={minmax}", flush=True)
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    od = odict_for(p0)
    rng = np.random.default_rng(100 + seed)
    syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
    scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
    big = rows * cols > 500_000
    mats = P.encode_all(list(zip(syms, scs)), od["words"], od, check_every=E if big else 1)
    stack = api.ExpertStack.from_host(mats, rows, cols, dev, dict_tag=api.dict_tag(od["words"]))
    image4 = api.device_image(od["words"], dev, slots=4)
    x = synth.activations(rng, T, cols)
    ids = synth.zipf_routing(rng, T, E)
    ws = api.alloc_workspace(E, T, dev)
    y = api.moe_fused_decode_matvec(stack, image4, torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev),
                                    relu=bool(seed % 2), workspace=ws, minmax=minmax)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    y = y.float().cpu().numpy().astype(np.float64)
    for e in range(E):
        sel = np.nonzero(ids == e)[0]
        if not sel.size:
            continue
        if not big or e == 0:        # the oracle's own encode + decode under the matched table
            ref = (P.oracle_matvec_minmax_from_codes(od, syms[e], scs[e], x[sel]) if minmax
                   else P.oracle_matvec_from_codes(od, syms[e], scs[e], x[sel]))
        else:                        # codes of expert 0 were checked bit-exact; the rest via the symbols
            ref = (P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], x[sel]) if minmax
                   else P.oracle_matvec_from_symbols(syms[e], scs[e], x[sel]))
        if seed % 2:
            ref = np.maximum(ref, 0)
        P.assert_close(y[sel], ref, what=f"expert {e}")


def test_fused_image_kind_mismatch_is_flagged(dev, lib_state, odict_for):
    """A 3-slot image used as a 4-slot one (padded to the 4-slot size, so the
    table copy stays inside the buffer) and a 4-slot image used as a 3-slot one
    fail the kernel's header check: error bit 31, nothing computed."""
    api = lib_state["api"]
    od = odict_for(0.857)
    sym, sc = P.host_experts(1, 64, 256, 0.857, 9)[0]
    stack = api.ExpertStack.from_host(P.encode_all([(sym, sc)], od["words"]), 64, 256, dev, dict_tag=api.dict_tag(od["words"]))
    from sub_bit_moe_amd import synth
    from sub_bit_moe_amd import _native as N
    x = torch.from_numpy(synth.activations(np.random.default_rng(9), 3, 256)).to(dev)
    ids = torch.zeros(3, dtype=torch.int32, device=dev)
    n4 = int(N.lib().sbm_dict_image4_bytes())
    im3 = api.dict_image(odict_for(0.885)["words"])
    padded = np.zeros(n4, np.uint8)
    padded[:im3.size] = im3
    im4 = api.device_image(od["words"], dev, slots=4)
    for image_t, image4 in ((torch.from_numpy(padded).to(dev), True), (im4, False)):
        ws = api.alloc_workspace(1, 3, dev)
        api.moe_fused_decode_matvec(stack, image_t, x, ids, workspace=ws, image4=image4)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0x80000000


def test_fused_image4_lds_limits(dev, lib_state, odict_for):
    """The 4-slot instance's LDS budget (65.5 KB table): a 14000-column row
    fits, 15000 columns are rejected with SBM_ERANGE, and the per-row min/max
    grid still fits two activation rows at 6144 columns."""
    from sub_bit_moe_amd import _native as N
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    od = odict_for(0.857)
    image4 = api.device_image(od["words"], dev, slots=4)
    rng = np.random.default_rng(77)
    for rows, cols, T, minmax in ((40, 14000, 2, False), (50, 6144, 3, True)):
        print(f"image4 limit {rows}x{cols} minmax={minmax}", flush=True)
        sym = synth.ternary_symbols(rng, rows, cols, 0.857)
        sc = synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows)
        st = api.ExpertStack.from_host(P.encode_all([(sym, sc)], od["words"], od), rows, cols, dev, dict_tag=api.dict_tag(od["words"]))
        x = synth.activations(rng, T, cols)
        ws = api.alloc_workspace(1, T, dev)
        y = api.moe_fused_decode_matvec(st, image4, torch.from_numpy(x).to(dev),
                                        torch.zeros(T, dtype=torch.int32, device=dev), workspace=ws,
                                        out_f32=True, minmax=minmax)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        ref = (P.oracle_matvec_minmax_from_symbols(sym, sc, x) if minmax
               else P.oracle_matvec_from_symbols(sym, sc, x))
        P.assert_close(y.cpu().numpy().astype(np.float64), ref, what=f"{rows}x{cols}")
    wide = P.encode_all([(np.zeros((2, 15000), np.uint8), np.ones(2, np.float16))], od["words"])
    st = api.ExpertStack.from_host(wide, 2, 15000, dev, dict_tag=api.dict_tag(od["words"]))
    with pytest.raises(N.SbmError) as e:
        api.moe_fused_decode_matvec(st, image4, torch.zeros((1, 15000), dtype=torch.float16, device=dev),
                                    torch.zeros(1, dtype=torch.int32, device=dev))
    assert e.value.status == -5


def test_fused_image4_random_shapes(dev, lib_state, odict_for):
    """A seeded sweep through the 4-slot image with the table built for
    P(0) = 0.857: even widths 2..3000, 1..600 rows, 1..160 tokens over 1..7
    experts (all three grouping paths), data at P(0) in [0.6, 0.95], both
    grids, ReLU and fp32 output; every expert's codes bit-exact with the
    oracle's encoder under that table."""
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    od = odict_for(0.857)
    image4 = api.device_image(od["words"], dev, slots=4)
    rng = np.random.default_rng(4242)
    for case in range(12):
        cols = int(rng.choice([2, 6, 30, 98, 254, 510, 512, 514, 770, 1026, 2080, 3000]))
        rows = int(rng.integers(1, 600))
        E = int(rng.integers(1, 8))
        T = int(rng.choice([1, 2, 5, 17, 64, 65, 128, 129, 160]))
        p0 = float(rng.uniform(0.6, 0.95))
        minmax = bool(case % 3 == 2)
        relu, out_f32 = bool(case % 2), bool(case % 4 == 1)
        print(f"image4 case {case}: {rows}x{cols} E={E} T={T} p0={p0:.3f} minmax={minmax}", flush=True)
        syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
        scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
        stack = api.ExpertStack.from_host(P.encode_all(list(zip(syms, scs)), od["words"], od), rows, cols, dev, dict_tag=api.dict_tag(od["words"]))
        x = rng.standard_normal((T, cols)).astype(np.float16)
        ids = rng.integers(0, E, T).astype(np.int32)
        ws = api.alloc_workspace(E, T, dev)
        y = api.moe_fused_decode_matvec(stack, image4, torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev),
                                        relu=relu, out_f32=out_f32, minmax=minmax, workspace=ws)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0
        y = y.float().cpu().numpy().astype(np.float64)
        for e in range(E):
            sel = np.nonzero(ids == e)[0]
            if not sel.size:
                continue
            ref = (P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], x[sel]) if minmax
                   else P.oracle_matvec_from_symbols(syms[e], scs[e], x[sel]))
            if relu:
                ref = np.maximum(ref, 0)
            P.assert_close(y[sel], ref, what=f"case {case} expert {e}")


def test_stack_from_native_encoder_matches(dev, lib_state, odict):
    """A stack built by sbm_encode_experts (one native call for the whole
    projection) gives the same fused outputs, bit for bit, as the stack
    assembled from per-matrix encodes, on both grids, and matches the oracle."""
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rng = np.random.default_rng(515)
    E, rows, cols, T = 6, 200, 770, 40
    syms = [synth.ternary_symbols(rng, rows, cols, 0.886) for _ in range(E)]
    x = torch.from_numpy(synth.activations(rng, T, cols)).to(dev)
    ids_h = synth.zipf_routing(rng, T, E)
    ids = torch.from_numpy(ids_h).to(dev)
    for minmax in (False, True):
        scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
        a = api.ExpertStack.from_symbols(syms, scs, odict["words"], dev)
        b = api.ExpertStack.from_host([api.encode_matrix(s, odict["words"]) + (sc,) for s, sc in zip(syms, scs)],
                                      rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
        ya = api.moe_fused_decode_matvec(a, lib_state["image_t"], x, ids, minmax=minmax)
        yb = api.moe_fused_decode_matvec(b, lib_state["image_t"], x, ids, minmax=minmax)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
        y = ya.float().cpu().numpy().astype(np.float64)
        xh = x.cpu().numpy()
        for e in range(E):
            sel = np.nonzero(ids_h == e)[0]
            if sel.size:
                ref = (P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], xh[sel]) if minmax
                       else P.oracle_matvec_from_symbols(syms[e], scs[e], xh[sel]))
                P.assert_close(y[sel], ref, what=f"minmax={minmax} expert {e}")


def test_decode_dense_bit_exact(dev, lib_state, odict):
    """sbm_decode_dense against the oracle's decode: every element of every
    matrix of a stack (nonzero code bases; ragged, narrow and c2048 shapes)
    is the fp16 of -1, 0 or +1 for codes 1, 0, 2; a damaged image header
    writes nothing and sets the flag."""
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rng = np.random.default_rng(31)
    to_f16 = np.array([0.0, -1.0, 1.0], np.float16)
    for E, rows, cols, p0 in ((3, 37, 30, 0.886), (2, 5, 2, 0.5), (3, 129, 2080, 0.857), (2, 768, 3072, 0.886),
                              (1, 6144, 2080, 0.886)):
        print(f"decode_dense E={E} {rows}x{cols} p0={p0}", flush=True)
        syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
        st = api.ExpertStack.from_symbols(syms, [synth.row_scales(rng, rows) for _ in range(E)], odict["words"], dev)
        for e in range(E):
            out, bad = api.decode_dense(st, e, lib_state["image_t"])
            torch.cuda.synchronize()
            assert int(bad.item()) == 0
            d = st.host_desc[e]
            codes = st.codes[d.code_base:d.code_base + d.n_codes].cpu().numpy().view(np.uint16)
            row_off = st.row_off[d.off_base:d.off_base + rows + 1].cpu().numpy().view(np.uint32)
            ref = OC.decode_symbols_with_table(codes, row_off, odict["sym28"], odict["lens"], cols)
            assert np.array_equal(ref, syms[e])
            assert np.array_equal(out.cpu().numpy().view(np.uint16), to_f16[ref].view(np.uint16)), (rows, cols, e)
    bad_image = torch.zeros_like(lib_state["image_t"])
    sentinel = torch.full((st.rows, st.cols), 7.0, dtype=torch.float16, device=dev)
    out, bad = api.decode_dense(st, 0, bad_image, out=sentinel)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1 and bool((out == 7.0).all())


def test_decode_dense_unaligned_output(dev, lib_state, odict):
    """sbm_decode_dense into outputs that start 4, 8 or 12 bytes past a
    16-byte boundary: every element right, nothing written outside the
    matrix (the zero fill uses 16-byte stores on the aligned part only)."""
    from sub_bit_moe_amd import synth
    api = lib_state["api"]
    rng = np.random.default_rng(37)
    to_f16 = np.array([0.0, -1.0, 1.0], np.float16)
    for rows, cols in ((37, 30), (129, 2080), (3, 2)):
        syms = [synth.ternary_symbols(rng, rows, cols, 0.886)]
        st = api.ExpertStack.from_symbols(syms, [synth.row_scales(rng, rows)], odict["words"], dev)
        for off in (2, 4, 6):
            print(f"decode_dense {rows}x{cols} output offset {2 * off} bytes", flush=True)
            buf = torch.full((rows * cols + 16,), 7.0, dtype=torch.float16, device=dev)
            out = buf[off:off + rows * cols].view(rows, cols)
            _, bad = api.decode_dense(st, 0, lib_state["image_t"], out=out)
            torch.cuda.synchronize()
            assert int(bad.item()) == 0
            b = buf.cpu().numpy()
            assert np.all(b[:off] == 7.0) and np.all(b[off + rows * cols:] == 7.0)
            assert np.array_equal(b[off:off + rows * cols].view(np.uint16),
                                  to_f16[syms[0]].reshape(-1).view(np.uint16))


@pytest.mark.parametrize("T", [5, 90, 150])
def test_fused_dictionary_mismatch_is_flagged(dev, lib_state, odict_for, T):
    """[M8.5] 0x08B: codes are only meaningful with the dictionary they were
    encoded under.  A stack encoded under the table built for P(0) = 0.857,
    run with the page's static table (its 4-slot image, which the kernel can
    otherwise execute, and its 3-slot image), is refused: error bit 29, no
    output rows.  In a mixed stack only the mislabelled expert is refused."""
    import ctypes
    from sub_bit_moe_amd import _native as N
    api = lib_state["api"]
    od, os_ = odict_for(0.857), odict_for(0.885)
    E, rows, cols = 3, 64, 256
    ex = P.host_experts(E, rows, cols, 0.857, 12)
    x = np.random.default_rng(13).standard_normal((T, cols)).astype(np.float16)
    ids = (np.arange(T) % E).astype(np.int32)
    xt, it = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
    st857 = api.ExpertStack.from_host(P.encode_all(ex, od["words"]), rows, cols, dev, dict_tag=api.dict_tag(od["words"]))
    for image_t, image4 in ((api.device_image(os_["words"], dev, slots=4), True), (lib_state["image_t"], False)):
        y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
        ws = api.alloc_workspace(E, T, dev)
        api.moe_fused_decode_matvec(st857, image_t, xt, it, out_f32=True, workspace=ws, y=y, image4=image4)
        torch.cuda.synchronize()
        assert api.workspace_error(ws) == 0x20000000
        assert bool(torch.isnan(y).all())
    # the same table's image computes them exactly
    y = api.moe_fused_decode_matvec(st857, api.device_image(od["words"], dev, slots=4), xt, it, out_f32=True)
    torch.cuda.synchronize()
    for t in range(min(T, 6)):
        P.assert_close(y[t].cpu().numpy(), P.oracle_matvec_from_symbols(*ex[ids[t]], x[t:t + 1])[0])
    # static-table stack with expert 1 labelled as encoded under the 0.857 table
    ex2 = P.host_experts(E, rows, cols, 0.886, 14)
    st = api.ExpertStack.from_host(P.encode_all(ex2, os_["words"]), rows, cols, dev, dict_tag=api.dict_tag(os_["words"]))
    descs = list(st.host_desc)
    descs[1].dict_tag = api.dict_tag(od["words"])
    arr = (N.MatrixDesc * E)(*descs)
    st.desc.copy_(torch.from_numpy(np.frombuffer(bytes(arr), np.uint8).copy()))
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(E, T, dev)
    api.moe_fused_decode_matvec(st, lib_state["image_t"], xt, it, out_f32=True, workspace=ws, y=y)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0x20000000
    yn = y.cpu().numpy()
    assert np.isnan(yn[ids == 1]).all()
    for t in np.flatnonzero(ids != 1)[:8]:
        P.assert_close(yn[t], P.oracle_matvec_from_symbols(*ex2[ids[t]], x[t:t + 1])[0])
    # the dense decoder refuses a matrix of another dictionary and writes nothing
    sentinel = torch.full((rows, cols), 7.0, dtype=torch.float16, device=dev)
    out, bad = api.decode_dense(st857, 0, lib_state["image_t"], out=sentinel)
    torch.cuda.synchronize()
    assert int(bad.item()) == 2 and bool((out == 7.0).all())


@pytest.mark.parametrize("T", [9, 100, 140])
def test_fused_bad_image_keeps_id_count(dev, lib_state, odict, T):
    """A damaged image with out-of-range ids: the error word keeps the id
    count (from whichever grouping path ran) and adds bit 31; no row is written."""
    api = lib_state["api"]
    E, rows, cols = 3, 64, 256
    ex = P.host_experts(E, rows, cols, 0.886, 15)
    st = api.ExpertStack.from_host(P.encode_all(ex, odict["words"]), rows, cols, dev, dict_tag=api.dict_tag(odict["words"]))
    ids = (np.arange(T) % E).astype(np.int32)
    ids[:3] = [-1, E, 1 << 20]
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(E, T, dev)
    bad_image = torch.zeros_like(lib_state["image_t"])
    x = torch.from_numpy(np.random.default_rng(16).standard_normal((T, cols)).astype(np.float16)).to(dev)
    api.moe_fused_decode_matvec(st, bad_image, x, torch.from_numpy(ids).to(dev), out_f32=True, workspace=ws, y=y)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == (0x80000000 | 3)
    assert bool(torch.isnan(y).all())


@pytest.mark.parametrize("T", [16, 44])
def test_decompress_gemm_expert_matches_oracle(dev, lib_state, odict, T):
    """The two-launch path for a heavy expert ([QMoE] "Limitations and
    Trade-offs": decompress, then multiply on the matrix cores): one c2048 pair
    (up 6144x2080, down 2080x6144, P(0)=0.886) decoded by sbm_decode_dense and
    multiplied by library fp16 GEMMs, against the oracle's own encode +
    reference decode + fp64 product; the down projection on the GPU's h."""
    from sub_bit_moe_amd import hybrid, synth
    api = lib_state["api"]
    rng = np.random.default_rng(41 + T)
    up = (synth.ternary_symbols(rng, 6144, 2080, 0.886), synth.row_scales(rng, 6144))
    down = (synth.ternary_symbols(rng, 2080, 6144, 0.886), synth.row_scales(rng, 2080))
    tag = api.dict_tag(odict["words"])
    su = api.ExpertStack.from_symbols([up[0]], [up[1]], odict["words"], dev)
    sd = api.ExpertStack.from_symbols([down[0]], [down[1]], odict["words"], dev)
    assert su.host_desc[0].dict_tag == tag
    x = synth.activations(np.random.default_rng(42 + T), T, 2080)
    bad = torch.zeros(1, dtype=torch.int32, device=dev)
    y, h = hybrid.expert_ffn(su, sd, 0, lib_state["image_t"], torch.from_numpy(x).to(dev), bad=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    hn = h.float().cpu().numpy().astype(np.float64)
    yn = y.float().cpu().numpy().astype(np.float64)
    ref_h = np.maximum(P.oracle_matvec_from_codes(odict, up[0], up[1], x), 0)
    ref_y = P.oracle_matvec_from_codes(odict, down[0], down[1], h.cpu().numpy())
    P.assert_close(hn, ref_h, what="decompress-then-GEMM up")
    P.assert_close(yn, ref_y, what="decompress-then-GEMM down")
    for t in range(T):
        P.assert_close(hn[t], ref_h[t], what=f"up t={t}")
        P.assert_close(yn[t], ref_y[t], what=f"down t={t}")
