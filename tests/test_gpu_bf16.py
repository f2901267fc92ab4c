"""SBM_F_IN_BF16: bf16 activations (the page's kernel reads bf16 x), converted
to fp16 as they are staged.  Outputs against the oracle on the bf16 values,
and bit-identical (fixed-point accumulators) to the fp16 path fed the same
values converted on the host."""
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


def _bf16_acts(rng, T, cols, scale=1.0):
    """N(0, scale^2) rounded to bf16 (torch tensor on the CPU) and its values in fp64."""
    x = torch.from_numpy((rng.standard_normal((T, cols)) * scale).astype(np.float32)).to(torch.bfloat16)
    return x, x.float().numpy().astype(np.float64)


@pytest.mark.parametrize("rows,cols,E,T,minmax,in_rms", [
    (768, 3072, 1, 1, False, False), (300, 512, 2, 3, False, True), (64, 30, 3, 5, False, False),
    (130, 6144, 2, 6, True, False), (257, 2080, 4, 40, False, True), (90, 770, 3, 150, True, False)])
def test_bf16_activations(dev, odict, rows, cols, E, T, minmax, in_rms):
    from oracle import matvec as OM
    from sub_bit_moe_amd import api, synth
    print(f"bf16 {rows}x{cols} E={E} T={T} minmax={minmax} in_rms={in_rms}", flush=True)
    words = odict["words"]
    rng = np.random.default_rng(rows + cols + T)
    syms = [synth.ternary_symbols(rng, rows, cols, 0.886) for _ in range(E)]
    scs = [synth.row_minmax(rng, rows) if minmax else synth.row_scales(rng, rows) for _ in range(E)]
    stack = api.ExpertStack.from_host(P.encode_all(list(zip(syms, scs)), words), rows, cols, dev,
                                      dict_tag=api.dict_tag(words))
    image = api.device_image(words, dev)
    xb, xv = _bf16_acts(rng, T, cols, 3.0)
    ids = rng.integers(0, E, T).astype(np.int32)
    it = torch.from_numpy(ids).to(dev)
    xb_d = xb.to(dev)
    xh_d = xb.to(torch.float16).to(dev)            # the same values in fp16 (all within fp16's range)
    assert torch.equal(xh_d.float(), xb_d.float())
    y = api.moe_fused_decode_matvec(stack, image, xb_d, it, out_f32=True, minmax=minmax, in_rms=in_rms)
    yb_det = api.moe_fused_decode_matvec(stack, image, xb_d, it, out_f32=True, minmax=minmax, in_rms=in_rms,
                                         deterministic=True)
    yh_det = api.moe_fused_decode_matvec(stack, image, xh_d, it, out_f32=True, minmax=minmax, in_rms=in_rms,
                                         deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(yb_det, yh_det), "bf16 activations must stage exactly as their fp16 conversion"
    yn = y.cpu().numpy().astype(np.float64)
    xin = OM.rms_glue(xv) if in_rms else xv
    for e in range(E):
        sel = np.nonzero(ids == e)[0]
        if not sel.size:
            continue
        ref = (P.oracle_matvec_minmax_from_symbols(syms[e], scs[e], xin[sel]) if minmax
               else P.oracle_matvec_from_symbols(syms[e], scs[e], xin[sel]))
        P.assert_close(yn[sel], ref, what=f"bf16 expert {e}")


def test_bf16_layer_call(dev, odict):
    """The layer call with bf16 x: y equals the fp16 layer call on the same
    values up to the order of the fp32 sums, and h and y match the oracle."""
    from sub_bit_moe_amd import api, synth
    words = odict["words"]
    E, d, f, T = 3, 512, 2048, 9
    tag = api.dict_tag(words)
    ups = P.host_experts(E, f, d, 0.886, 81)
    downs = P.host_experts(E, d, f, 0.886, 82)
    up = api.ExpertStack.from_host(P.encode_all(ups, words), f, d, dev, dict_tag=tag)
    down = api.ExpertStack.from_host(P.encode_all(downs, words), d, f, dev, dict_tag=tag)
    image = api.device_image(words, dev)
    rng = np.random.default_rng(83)
    xb, xv = _bf16_acts(rng, T, d)
    ids_h = rng.integers(0, E, T).astype(np.int32)
    ids = torch.from_numpy(ids_h).to(dev)
    y, h = api.moe_fused_ffn(up, down, image, xb.to(dev), ids, out_f32=True)
    y2, h2 = api.moe_fused_ffn(up, down, image, xb.to(torch.float16).to(dev), ids, out_f32=True)
    torch.cuda.synchronize()
    hn, yn = h.float().cpu().numpy(), y.cpu().numpy().astype(np.float64)
    P.assert_close(hn, h2.float().cpu().numpy(), what="h bf16 vs fp16")
    P.assert_close(yn, y2.cpu().numpy().astype(np.float64), 2e-6, 2e-5, what="y bf16 vs fp16")
    for t in range(T):
        e = int(ids_h[t])
        P.assert_close(hn[t], np.maximum(P.oracle_matvec_from_symbols(*ups[e], xv[t:t + 1])[0], 0), what=f"h {t}")
        P.assert_close(yn[t], P.oracle_matvec_from_symbols(*downs[e], hn[t:t + 1].astype(np.float16))[0],
                       what=f"y {t}")
