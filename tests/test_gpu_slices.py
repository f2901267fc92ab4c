"""Workgroup slices numbered per XCD: calls whose grid is not a multiple of the
8 XCDs (13, 37, 41, 42, 100 and 255 workgroups, on the one-wave, workgroup and
launched grouping paths) must still cover every output row exactly once.  The
output starts as NaN, so a slice that no workgroup takes leaves NaN rows; every
row is compared with the oracle."""
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


def _grid(rows, E, T, tcmax):
    """The call's workgroup count: one per 16 rows of an upper bound of its
    items' rows, at most the CU count."""
    max_items = min(E, T) + T // tcmax + 1
    return min(-(-max_items * rows // 16), torch.cuda.get_device_properties(0).multi_processor_count)


# (rows, cols, tokens, experts, items per token group on this width) -> grids 13, 37, 100, 255, 42, 41
@pytest.mark.parametrize("rows,cols,T,E,tcmax", [(104, 512, 1, 2, 4), (296, 768, 1, 2, 4), (800, 512, 1, 1, 4),
                                                 (2040, 512, 1, 1, 4), (24, 1024, 100, 2, 4),
                                                 (16, 512, 150, 3, 4)])
def test_every_row_covered_on_odd_grids(dev, odict, rows, cols, T, E, tcmax):
    from sub_bit_moe_amd import api
    g = _grid(rows, E, T, tcmax)
    print(f"slices rows={rows} cols={cols} T={T} E={E} grid={g}", flush=True)
    ex = P.host_experts(E, rows, cols, 0.886, rows + T)
    words = odict["words"]
    stack = api.ExpertStack.from_host(P.encode_all(ex, words), rows, cols, dev, dict_tag=api.dict_tag(words))
    image = api.device_image(words, dev)
    rng = np.random.default_rng(rows)
    x = rng.standard_normal((T, cols)).astype(np.float16)
    ids = (np.arange(T) % E).astype(np.int32)
    y = torch.full((T, rows), float("nan"), dtype=torch.float32, device=dev)
    ws = api.alloc_workspace(E, T, dev)
    api.moe_fused_decode_matvec(stack, image, torch.from_numpy(x).to(dev), torch.from_numpy(ids).to(dev),
                                out_f32=True, workspace=ws, y=y)
    torch.cuda.synchronize()
    assert api.workspace_error(ws) == 0
    yn = y.cpu().numpy()
    assert not np.isnan(yn).any(), "rows that no workgroup wrote"
    for e in range(E):
        sel = np.flatnonzero(ids == e)
        P.assert_close(yn[sel], P.oracle_matvec_from_symbols(*ex[e], x[sel]), what=f"expert {e}")
