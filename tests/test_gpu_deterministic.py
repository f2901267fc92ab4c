"""SBM_F_DETERMINISTIC: fixed-point row accumulators.  Outputs against the
oracle (same bar as the default path) and bit-identical across repeated calls,
interleaved with other launches and inside graph replays."""
import numpy as np
import pytest

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
    return {"api": api, "image_t": api.device_image(odict["words"], dev)}


def _case(api, rng, words, rows, cols, E, T, p0, minmax, dev, zipf=True):
    from sub_bit_moe_amd import synth
    syms = [synth.ternary_symbols(rng, rows, cols, p0) for _ in range(E)]
    scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
    stack = api.ExpertStack.from_host(P.encode_all(list(zip(syms, scs)), words), rows, cols, dev,
                                      dict_tag=api.dict_tag(words))
    x = synth.activations(rng, T, cols)
    ids = synth.zipf_routing(rng, T, E) if zipf else rng.integers(0, E, T).astype(np.int32)
    return syms, scs, stack, x, ids


def _check_oracle(y, syms, scs, x, ids, minmax, relu, what):
    for e in range(len(syms)):
        sel = np.nonzero(ids == e)[0]
        if not sel.size:
            continue
        ref = (P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], x[sel]) if minmax
               else P.oracle_matvec_from_symbols(syms[e], scs[e], x[sel]))
        if relu:
            ref = np.maximum(ref, 0)
        P.assert_close(y[sel], ref, what=f"{what} expert {e}")


# wide rows (one row split per lane at most) and narrow rows (a lane spans
# several rows), 1-, 2- and 4-token items, in-LDS grouping and the grouping
# launch (T > 128), both grids
@pytest.mark.parametrize("rows,cols,E,T,minmax", [
    (768, 3072, 3, 9, False), (130, 6144, 2, 5, False), (300, 512, 4, 17, True), (64, 30, 3, 7, False),
    (1000, 256, 2, 6, True), (257, 2080, 5, 129, False), (33, 254, 2, 3, True)])
def test_deterministic_matches_oracle_and_repeats(dev, lib_state, odict, rows, cols, E, T, minmax):
    print(f"deterministic {rows}x{cols} E={E} T={T} minmax={minmax}", flush=True)
    api = lib_state["api"]
    rng = np.random.default_rng(rows * 7 + cols)
    syms, scs, stack, x, ids = _case(api, rng, odict["words"], rows, cols, E, T, 0.886, minmax, dev)
    xt, it = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
    ws = api.alloc_workspace(E, T, dev)
    for out_f32 in (True, False):
        runs = []
        for rep in range(3):
            y = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=not out_f32,
                                            out_f32=out_f32, workspace=ws, minmax=minmax, deterministic=True)
            torch.cuda.synchronize()
            assert api.workspace_error(ws) == 0
            runs.append(y.clone())
            # other work on the device between the calls
            torch.matmul(torch.randn(512, 512, device=dev), torch.randn(512, 512, device=dev))
        for r in runs[1:]:
            assert torch.equal(r, runs[0]), "deterministic outputs differ between calls"
        _check_oracle(runs[0].float().cpu().numpy().astype(np.float64), syms, scs, x, ids, minmax,
                      not out_f32, f"det f32={out_f32}")
        yd = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=not out_f32, out_f32=out_f32,
                                         workspace=ws, minmax=minmax)
        torch.cuda.synchronize()
        if out_f32:   # the two summation orders agree to fp32 rounding
            P.assert_close(runs[0].double().cpu().numpy(), yd.double().cpu().numpy(), 2e-6, 2e-5,
                           what="det vs default")


def test_deterministic_image4(dev, lib_state, odict_for):
    """The 4-slot instance (a dictionary built for P(0) = 0.857) with
    fixed-point accumulators, both grids."""
    api = lib_state["api"]
    od = odict_for(0.857)
    image4 = api.device_image(od["words"], dev, slots=4)
    for minmax, (rows, cols, E, T) in ((False, (768, 3072, 4, 33)), (True, (257, 2080, 3, 9))):
        print(f"deterministic image4 {rows}x{cols} minmax={minmax}", flush=True)
        rng = np.random.default_rng(900 + rows)
        syms, scs, stack, x, ids = _case(api, rng, od["words"], rows, cols, E, T, 0.857, minmax, dev)
        xt, it = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
        ys = [api.moe_fused_decode_matvec(stack, image4, xt, it, out_f32=True, minmax=minmax, deterministic=True)
              for _ in range(2)]
        torch.cuda.synchronize()
        assert torch.equal(ys[0], ys[1])
        _check_oracle(ys[0].cpu().numpy().astype(np.float64), syms, scs, x, ids, minmax, False, "det image4")


def test_deterministic_graph_replays(dev, lib_state, odict):
    """A c2048-shaped down projection (2080 x 6144) in a graph: every replay,
    with eager launches and synchronisations between them, returns the eager
    call's bits."""
    api = lib_state["api"]
    rng = np.random.default_rng(31)
    rows, cols, E, T = 2080, 6144, 6, 64
    syms, scs, stack, x, ids = _case(api, rng, odict["words"], rows, cols, E, T, 0.886, False, dev)
    xt, it = torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev)
    ws = api.alloc_workspace(E, T, dev)
    y = torch.empty((T, rows), dtype=torch.float16, device=dev)
    eager = api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=True, workspace=ws,
                                        deterministic=True).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, relu=True, workspace=ws, y=y,
                                    deterministic=True)
    for rep in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep} differs from the eager call"
        api.moe_fused_decode_matvec(stack, lib_state["image_t"], xt, it, workspace=ws)   # default path between
        torch.cuda.synchronize()
    _check_oracle(eager.float().cpu().numpy().astype(np.float64), syms, scs, x, ids, False, True, "det graph")
