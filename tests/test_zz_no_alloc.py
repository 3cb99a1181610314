"""GPU check of the allocation-free entry point rgt_route_sort_quant_noalloc
(the library's per-GPU scratch array in place of a caller's workspace)
against rgt_route_sort_quant on the same inputs: bit-identical outputs on
two calls in a row, the second with a smaller input, and a shape beyond the
scratch array rejected before any launch."""
import numpy as np
import pytest

from _helpers import CANARY, say, to_dev, to_dev_bf16
from router_gemv_top_amd.inputs import Workload

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def _outputs(R, m, n, kdim, k, block):
    out = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY)
    out["topk_ids"] = torch.empty((m, k), dtype=torch.int32, device="cuda")
    out["topk_w"] = torch.empty((m, k), dtype=torch.float32, device="cuda")
    out["logits"] = torch.empty((m, n), dtype=torch.float32, device="cuda")
    return out


def _compare(a, b, block):
    a = {k: v.cpu().numpy() for k, v in a.items()}
    b = {k: v.cpu().numpy() for k, v in b.items()}
    for key in ("logits", "topk_w"):
        np.testing.assert_array_equal(a[key].view(np.uint32), b[key].view(np.uint32), err_msg=key)
    for key in ("topk_ids", "offsets"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    total = int(a["offsets"][-1])
    np.testing.assert_array_equal(a["sorted_ids"][:total], b["sorted_ids"][:total], err_msg="sorted_ids")
    np.testing.assert_array_equal(a["expert_ids"][:total // block], b["expert_ids"][:total // block],
                                  err_msg="expert_ids")
    valid = a["sorted_ids"][:total] != a["topk_ids"].size
    np.testing.assert_array_equal(a["a_q"][:total][valid], b["a_q"][:total][valid], err_msg="a_q")
    np.testing.assert_array_equal(a["a_scale"][:total][valid], b["a_scale"][:total][valid], err_msg="a_scale")


@pytest.mark.parametrize("first,second", [((16, 128, 6144, 8, 16, False), (4, 128, 6144, 8, 16, False)),
                                          ((32, 896, 3584, 16, 16, True), (1, 896, 3584, 16, 16, True))])
def test_noalloc_matches_workspace_entry_point(R, first, second):
    for (m, n, kdim, k, block, bias) in (first, second):
        say(f"route_sort_quant_noalloc M={m} N={n} K={kdim} k={k} B={block} bias={bias}")
        x, w, b = Workload("noalloc", m, n, kdim, k, block, bias=bias).make()
        xd, wd = to_dev_bf16(x), to_dev_bf16(w)
        bd = None if b is None else to_dev(b)
        ws = R.Workspace(m, n, kdim, k, block)
        ref = R.route_sort_quant(xd, wd, k, block, ws, bias=bd, out=_outputs(R, m, n, kdim, k, block))
        got = R.route_sort_quant_noalloc(xd, wd, k, block, bias=bd, out=_outputs(R, m, n, kdim, k, block))
        launches = R.last_launch_count()
        torch.cuda.synchronize()
        assert launches in (1, 2), "one fused launch (plus the scratch fill on a GPU's first call)"
        assert R.check_workspace(ws) == 0
        _compare(got, ref, block)


def test_noalloc_rejects_shapes_beyond_its_scratch(R):
    say("route_sort_quant_noalloc: a wide batch beyond the scratch array")
    m, n, kdim, k, block = 1024, 1024, 8192, 32, 64
    xd = torch.zeros((m, kdim), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((n, kdim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(R.RgtUnsupported):
        R.route_sort_quant_noalloc(xd, wd, k, block)
    assert R.last_launch_count() == 0
