"""GPU-generated stacks: codes bit-exact against the oracle's encoding of the
host-regenerated matrices, and fused outputs of a stack pass against the
oracle on the GPU's actual per-layer inputs (sampled experts and rows)."""
import numpy as np
import pytest

from oracle import codec as OC
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


def api_error(ws):
    from sub_bit_moe_amd import api
    return api.workspace_error(ws)


@pytest.fixture(scope="module")
def gen_state(dev, odict):
    from sub_bit_moe_amd import api
    trie = torch.from_numpy(api.build_trie(odict["words"])).to(dev)
    table = torch.from_numpy(synth.scale_table().view(np.int16)).to(dev)
    return api, trie, table


def _host_matrix(st_gpu, e):
    d = st_gpu.host_desc[e]
    codes = st_gpu.codes[d.code_base:d.code_base + d.n_codes].cpu().numpy().view(np.uint16)
    row_off = st_gpu.row_off[d.off_base:d.off_base + st_gpu.rows + 1].cpu().numpy().view(np.uint32)
    nblk = (d.n_codes + 1023) // 1024
    bstart = st_gpu.bstart[d.blk_base:d.blk_base + nblk].cpu().numpy().view(np.uint32)
    scales = st_gpu.scales[d.scale_base:d.scale_base + st_gpu.rows].cpu().numpy()
    return codes, row_off, bstart, scales


@pytest.mark.parametrize("E,rows,cols,mat,layer,p0", [(5, 300, 512, 0, 3, 0.886), (4, 130, 98, 1, 0, 0.857),
                                                     (2, 6144, 2080, 0, 7, 0.886), (2, 2080, 6144, 1, 29, 0.886)])
def test_generated_codes_bit_exact(dev, odict, gen_state, E, rows, cols, mat, layer, p0):
    print(f"gen E={E} {rows}x{cols} mat={mat} layer={layer}", flush=True)
    api, trie, table = gen_state
    seed = 41
    stg = api.generate_stack(seed, layer, E, mat, rows, cols, p0, trie, table,
                             dict_checksum=api.dictionary_checksum(odict["words"]))
    torch.cuda.synchronize()
    for e in range(E):
        key = synth.matrix_key(seed, layer, e, mat, E)
        sym = synth.counter_symbols(key, rows, cols, p0)
        codes, row_off, bstart, scales = _host_matrix(stg, e)
        rc, ro = OC.encode_matrix(sym, odict["child"])
        assert np.array_equal(codes, rc), f"expert {e}: codes differ"
        assert np.array_equal(row_off, ro), f"expert {e}: row offsets differ"
        assert np.array_equal(bstart, OC.block_starts(rc, odict["lens"], 1024)), f"expert {e}: block starts"
        exp_sc = synth.scale_table()[synth.counter_scale_index(key, rows)]
        assert np.array_equal(scales.view(np.uint16), exp_sc.view(np.uint16)), f"expert {e}: scales"
        assert stg.host_desc[e].code_base % 8 == 0
        assert stg.host_desc[e].dict_tag == api.dict_tag(odict["words"])


def test_generated_codes_matched_dictionary(dev, odict_for):
    """The GPU generator's trie walk under a table built for P(0) = 0.857
    (entries with 4 nonzeros): codes, offsets and block starts bit-exact with
    the oracle's encoding under the same table."""
    from sub_bit_moe_amd import api
    od = odict_for(0.857)
    trie = torch.from_numpy(api.build_trie(od["words"])).to(dev)
    table = torch.from_numpy(synth.scale_table().view(np.int16)).to(dev)
    E, rows, cols, mat, layer, seed = 3, 96, 3072, 1, 2, 11
    stg = api.generate_stack(seed, layer, E, mat, rows, cols, 0.857, trie, table,
                             dict_checksum=api.dictionary_checksum(od["words"]))
    torch.cuda.synchronize()
    for e in range(E):
        sym = synth.counter_symbols(synth.matrix_key(seed, layer, e, mat, E), rows, cols, 0.857)
        codes, row_off, bstart, _ = _host_matrix(stg, e)
        rc, ro = OC.encode_matrix(sym, od["child"])
        assert np.array_equal(codes, rc) and np.array_equal(row_off, ro), f"expert {e}"
        assert np.array_equal(bstart, OC.block_starts(rc, od["lens"], 1024)), f"expert {e}"


def test_base128_stack_matched_dictionary_pass(dev):
    """A 2-layer base128-shaped stack (128 experts, up 3072x768, down
    768x3072, P(0) = 0.857, 128 Zipf tokens) encoded under the table built for
    its P(0) and run through the 4-slot image: sampled tokens of every layer
    against the oracle on the GPU's own inputs (sampled rows; the codes under
    that table are pinned by the generator test above)."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=2, n_experts=128, d_model=768, d_ff=3072, p0=0.857, dict_p0=0.857,
                        image_slots=4, seed=11, n_tokens=128)
    st = S.build(cfg, dev)
    run = S.Runner(st)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    assert api_error(run.ws_up) == 0 and api_error(run.ws_down) == 0
    rng = np.random.default_rng(6)
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        ids = st.routes_host[l]
        xin = OM.rms_glue(keep[l - 1][2].float().cpu().numpy()).astype(np.float64) if l else xraw
        for t in rng.choice(cfg.n_tokens, 4, replace=False):
            e = int(ids[t])
            for mat, inp, out, relu in ((0, xin[t], h[t], True), (1, h[t], y[t], False)):
                rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
                key = synth.matrix_key(cfg.seed, l, e, mat, cfg.n_experts)
                rsel = np.sort(rng.choice(rows, 48, replace=False))
                sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
                sc = synth.scale_table()[synth.counter_scale_index(key, rows)][rsel]
                ref = P.oracle_matvec_from_symbols(sym, sc, inp.astype(np.float16)[None, :])[0]
                if relu:
                    ref = np.maximum(ref, 0)
                P.assert_close(out[rsel], ref, what=f"layer {l} token {t} mat {mat}")


def test_small_stack_pass_against_oracle(dev, odict):
    """A 3-layer stack of 64 experts with c2048 widths and 64 Zipf tokens: every
    layer's up and down outputs for sampled tokens against the oracle applied
    to the GPU's own inputs to that layer; the glue against its fp64 form."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=3, n_experts=64, seed=43)
    st = S.build(cfg, dev)
    run = S.Runner(st)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        ids = st.routes_host[l]
        if l > 0:
            prev_y = keep[l - 1][2].float().cpu().numpy()
            assert np.array_equal(xraw, prev_y)
            xin = OM.rms_glue(prev_y).astype(np.float64)     # applied inside the up projection
        else:
            xin = xraw
        for t in rng.choice(cfg.n_tokens, 6, replace=False):
            e = int(ids[t])
            for mat, inp, out, relu in ((0, xin[t], h[t], True), (1, h[t], y[t], False)):
                rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
                key = synth.matrix_key(cfg.seed, l, e, mat, cfg.n_experts)
                rsel = np.sort(rng.choice(rows, 48, replace=False))
                sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
                sc = synth.scale_table()[synth.counter_scale_index(key, rows)][rsel]
                ref = P.oracle_matvec_from_symbols(sym, sc, inp.astype(np.float16)[None, :])[0]
                if relu:
                    ref = np.maximum(ref, 0)
                P.assert_close(out[rsel], ref, what=f"layer {l} token {t} mat {mat}")


def test_small_stack_minmax_pass_against_oracle(dev, odict):
    """The bench's pass on the per-row (w_min, w_max) grid: a 2-layer stack of
    64 experts with c2048 widths, sampled tokens and rows of every layer's up
    and down outputs against the oracle on the GPU's own inputs."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=2, n_experts=64, seed=45)
    st = S.with_minmax(S.build(cfg, dev))
    run = S.Runner(st, minmax=True)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        ids = st.routes_host[l]
        xin = OM.rms_glue(keep[l - 1][2].float().cpu().numpy()).astype(np.float64) if l > 0 else xraw
        mms = (st.up[l].scales.float().cpu().numpy(), st.down[l].scales.float().cpu().numpy())
        for t in rng.choice(cfg.n_tokens, 5, replace=False):
            e = int(ids[t])
            for mat, inp, out, relu in ((0, xin[t], h[t], True), (1, h[t], y[t], False)):
                rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
                key = synth.matrix_key(cfg.seed, l, e, mat, cfg.n_experts)
                rsel = np.sort(rng.choice(rows, 40, replace=False))
                sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
                base = (st.up if mat == 0 else st.down)[l].host_desc[e].scale_base // 2
                mm = mms[mat][base + rsel]
                ref = P.oracle_matvec_minmax_from_symbols(sym, mm, inp.astype(np.float16)[None, :])[0]
                if relu:
                    ref = np.maximum(ref, 0)
                P.assert_close(out[rsel], ref, what=f"minmax layer {l} token {t} mat {mat}")


def test_graph_replay_matches_eager(dev):
    """The bench captures a pass in a HIP graph: several replays, with eager
    work between them, must reproduce the eager pass.  Row sums are combined
    with LDS float atomics whose order varies, so equality is up to fp16
    rounding of the final outputs."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=2, n_experts=32, seed=44, n_tokens=24)
    st = S.build(cfg, dev)
    run = S.Runner(st)
    ref = run.run().clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = run.run()
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        P.assert_close(out.float().cpu().numpy(), ref.float().cpu().numpy(), 2e-3, 2e-3, what="replay")
        run.run()              # eager work in between
        torch.cuda.synchronize()


def _check_sampled(cfg, layer, xin, h, y, ids, experts, n_tok, n_rows, rng):
    """Oracle check of sampled rows of the up (ReLU) and down outputs of the
    given experts for up to n_tok of their tokens, on the GPU's own inputs."""
    for e in experts:
        toks = np.flatnonzero(ids == e)
        toks = toks if toks.size <= n_tok else rng.choice(toks, n_tok, replace=False)
        for mat in (0, 1):
            rows, cols = (cfg.d_ff, cfg.d_model) if mat == 0 else (cfg.d_model, cfg.d_ff)
            key = synth.matrix_key(cfg.seed, layer, int(e), mat, cfg.n_experts)
            rsel = np.sort(rng.choice(rows, n_rows, replace=False))
            sym = np.concatenate([synth.counter_symbols(key, 1, cols, cfg.p0, row0=int(r)) for r in rsel])
            sc = synth.scale_table()[synth.counter_scale_index(key, rows)][rsel]
            inp = (xin if mat == 0 else h)[toks].astype(np.float16)
            ref = P.oracle_matvec_from_symbols(sym, sc, inp)
            if mat == 0:
                ref = np.maximum(ref, 0)
            out = (h if mat == 0 else y)[toks][:, rsel]
            for i, t in enumerate(toks):
                P.assert_close(out[i], ref[i], what=f"layer {layer} expert {e} token {t} mat {mat}")


def _sample_experts(ids, k, rng):
    """Seeded sample of touched experts, always with the most loaded one."""
    touched, counts = np.unique(ids, return_counts=True)
    pick = set(rng.choice(touched, min(k, touched.size), replace=False).tolist())
    pick.add(int(touched[np.argmax(counts)]))
    return sorted(pick)


def test_c2048_layer_256_tokens(dev):
    """One c2048-shaped layer at full size: 2048 experts of 6144x2080 and
    2080x6144, 256 Zipf tokens (grouped by the separate grouping launch): 32
    sampled experts plus the most loaded one, 32 rows per matrix, against the
    oracle."""
    from sub_bit_moe_amd import stack as S
    cfg = S.StackConfig(n_layers=1, n_experts=2048, n_tokens=256, seed=31)
    st = S.build(cfg, dev)
    run = S.Runner(st)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    assert api_error(run.ws_up) == 0 and api_error(run.ws_down) == 0
    xin, h, y = (t.float().cpu().numpy() for t in keep[0])
    rng = np.random.default_rng(32)
    _check_sampled(cfg, 0, xin, h, y, st.routes_host[0], _sample_experts(st.routes_host[0], 32, rng), 4, 32, rng)
    del st, run, keep
    torch.cuda.empty_cache()


def test_full_bench_stack_sampled(dev):
    """The benchmark's own workload and launch configuration: 30 layers x 2048
    experts (~148 GB generated on the GPU), 64 tokens through every layer;
    per layer 2 sampled experts (one of them the most loaded), 2 of their
    tokens and 24 rows per matrix against the oracle on the GPU's inputs."""
    from oracle import matvec as OMv
    from sub_bit_moe_amd import stack as S
    torch.cuda.empty_cache()
    cfg = S.StackConfig()
    st = S.build(cfg, dev)
    run = S.Runner(st)
    keep = {}
    run.run(keep)
    torch.cuda.synchronize()
    assert api_error(run.ws_up) == 0 and api_error(run.ws_down) == 0
    rng = np.random.default_rng(41)
    prev_y = None
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        xin = xraw if l == 0 else OMv.rms_glue(prev_y).astype(np.float64)
        ids = st.routes_host[l]
        _check_sampled(cfg, l, xin, h, y, ids, _sample_experts(ids, 1, rng), 2, 24, rng)
        prev_y = y
    del st, run, keep
    torch.cuda.empty_cache()


def test_full_bench_stack_deterministic(dev):
    """The benchmark workload with fixed-point row accumulators: two passes
    return the same bits at every layer, and sampled rows of every layer
    match the oracle on the GPU's own inputs."""
    from oracle import matvec as OMv
    from sub_bit_moe_amd import stack as S
    torch.cuda.empty_cache()
    cfg = S.StackConfig()
    st = S.build(cfg, dev)
    run = S.Runner(st, deterministic=True)
    keep, keep2 = {}, {}
    run.run(keep)
    run.run(keep2)
    torch.cuda.synchronize()
    assert api_error(run.ws_up) == 0 and api_error(run.ws_down) == 0
    for l in range(cfg.n_layers):
        for a, b in zip(keep[l], keep2[l]):
            assert torch.equal(a, b), f"layer {l}: two deterministic passes differ"
    rng = np.random.default_rng(43)
    prev_y = None
    for l in range(cfg.n_layers):
        xraw, h, y = (t.float().cpu().numpy() for t in keep[l])
        xin = xraw if l == 0 else OMv.rms_glue(prev_y).astype(np.float64)
        ids = st.routes_host[l]
        _check_sampled(cfg, l, xin, h, y, ids, _sample_experts(ids, 1, rng), 2, 16, rng)
        prev_y = y
    del st, run, keep, keep2
    torch.cuda.empty_cache()
