"""The allocation-free fused call (sbm_moe_fused_decode_matvec_noalloc)
through the C ABI, against the workspace entry point on the same inputs:
two calls in a row, the second smaller, on both grouping paths (more than
128 tokens: the grouping kernel's tables live in the static scratch array;
at most 128: grouped inside the fused kernel), with the error word it
returns; and a call too large for the scratch array is refused."""
import ctypes as C

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


def _noalloc(stack, image_t, x, ids, y, err, flags):
    from sub_bit_moe_amd import _native as N
    s = torch.cuda.current_stream().cuda_stream
    return N.lib().sbm_moe_fused_decode_matvec_noalloc(
        stack.codes.data_ptr(), stack.row_off.data_ptr(), stack.bstart.data_ptr(), stack.scales.data_ptr(),
        stack.desc.data_ptr(), stack.n_experts, stack.rows, stack.cols, image_t.data_ptr(), x.data_ptr(),
        ids.data_ptr(), int(x.shape[0]), y.data_ptr(), flags, err.data_ptr(), s)


def test_noalloc_matches_workspace_entry(dev, odict):
    from sub_bit_moe_amd import _native as N
    from sub_bit_moe_amd import api, synth
    words = odict["words"]
    image_t = api.device_image(words, dev)
    E, rows, cols = 40, 96, 512
    ex = P.host_experts(E, rows, cols, 0.886, 71)
    stack = api.ExpertStack.from_host(P.encode_all(ex, words), rows, cols, dev, dict_tag=api.dict_tag(words))
    flags = N.SBM_F_RELU | N.SBM_F_OUT_F32
    for T, n_bad, seed in ((200, 3, 72), (37, 0, 73)):       # second call smaller, other grouping path
        print(f"noalloc call: E={E} T={T} invalid ids={n_bad}", flush=True)
        rng = np.random.default_rng(seed)
        x = torch.from_numpy(synth.activations(rng, T, cols)).to(dev)
        ids_h = synth.zipf_routing(rng, T, E).astype(np.int32)
        ids_h[:n_bad] = -1
        ids = torch.from_numpy(ids_h).to(dev)
        y0 = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
        ws = api.alloc_workspace(E, T, dev)
        api.moe_fused_decode_matvec(stack, image_t, x, ids, relu=True, out_f32=True, workspace=ws, y=y0)
        y1 = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
        err = torch.full((1,), -1, dtype=torch.int32, device=dev)
        assert _noalloc(stack, image_t, x, ids, y1, err, flags) == 0
        torch.cuda.synchronize()
        assert int(err.item()) == api.workspace_error(ws) == n_bad
        a, b = y0.cpu().numpy(), y1.cpu().numpy()
        ok = ids_h >= 0
        assert np.isnan(b[~ok]).all()
        P.assert_close(b[ok], a[ok], what=f"noalloc vs workspace entry, T={T}")
        xs = x.cpu().numpy()
        for t in np.flatnonzero(ok)[:6]:
            ref = np.maximum(P.oracle_matvec_from_symbols(*ex[ids_h[t]], xs[t:t + 1])[0], 0)
            P.assert_close(b[t], ref, what=f"noalloc vs oracle, token {t}")
    # too large for the static array: refused before any launch
    big_e = 1 << 16
    assert api.workspace_bytes(big_e, 64) > 256 * 1024
    z = C.c_void_p(0)
    st = N.lib().sbm_moe_fused_decode_matvec_noalloc(z, z, z, z, z, big_e, rows, cols, z, z, z, 64, z, 0, z, z)
    assert st == -5 and b"allocation-free" in N.lib().sbm_last_error()


def test_noalloc_deterministic_bf16(dev, odict):
    """The allocation-free call with fixed-point accumulators and bf16
    activations returns the workspace entry point's bits, twice in a row
    (the second call smaller)."""
    from sub_bit_moe_amd import _native as N
    from sub_bit_moe_amd import api
    words = odict["words"]
    image_t = api.device_image(words, dev)
    E, rows, cols = 12, 300, 2080
    ex = P.host_experts(E, rows, cols, 0.886, 91)
    stack = api.ExpertStack.from_host(P.encode_all(ex, words), rows, cols, dev, dict_tag=api.dict_tag(words))
    flags = N.SBM_F_OUT_F32 | N.SBM_F_DETERMINISTIC | N.SBM_F_IN_BF16
    for T, seed in ((150, 92), (9, 93)):
        print(f"noalloc deterministic bf16: T={T}", flush=True)
        rng = np.random.default_rng(seed)
        x = torch.from_numpy(rng.standard_normal((T, cols)).astype(np.float32)).to(torch.bfloat16).to(dev)
        ids = torch.from_numpy(rng.integers(0, E, T).astype(np.int32)).to(dev)
        y0 = api.moe_fused_decode_matvec(stack, image_t, x, ids, out_f32=True, deterministic=True)
        y1 = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
        err = torch.full((1,), -1, dtype=torch.int32, device=dev)
        assert _noalloc(stack, image_t, x, ids, y1, err, flags) == 0
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(y0, y1)
