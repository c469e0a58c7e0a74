"""attn_tree_verify_noalloc (the library's built-in scratch instead of a workspace) against
attn_tree_verify on the same inputs: two calls in a row, the second with a smaller input, so
the second call runs over scratch that still holds the first call's partials.  The split plan
is the same for both entry points, so the outputs match bit for bit."""
import numpy as np
import pytest
import torch

import tree_verify_linear_amd as tvl
from tvutil import attn_to_device
from workloads import gen_attn, trees_for

pytestmark = pytest.mark.gpu


def _both(A):
    d = attn_to_device(A)
    B, N = A.parent.shape
    args = (d["q"], d["k_cache"], d["v_cache"], A.k_type, A.v_type, d["n_past"], d["parent"], d["n_nodes"],
            A.window, A.scale)
    o_ws = torch.full((B, N, A.Hq, A.D), float("nan"), device="cuda")
    l_ws = torch.full((B, N, A.Hq), float("nan"), device="cuda")
    tvl.attn_tree_verify(*args, out=o_ws, lse=l_ws)
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    tvl.attn_tree_verify_noalloc(*args, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    return (o_ws.cpu().numpy(), l_ws.cpu().numpy()), (o_na.cpu().numpy(), l_na.cpu().numpy())


def test_noalloc_matches_workspace_entry_point_twice():
    """First a split-heavy call (one sequence, 4096 slots, window 2048: many KV splits), then a
    smaller one (one sequence, 700 slots, Q4_0 V), both compared bit for bit."""
    big_parents, _ = trees_for(90, 1, "ddtree")
    big = gen_attn(90, big_parents, 24, 4, 256, 4096, "q8_0", "q8_0", 2048)
    small_parents, _ = trees_for(91, 1, "ddtree", budget=8)
    small = gen_attn(91, small_parents, 24, 4, 256, 700, "q8_0", "q4_0", 0)
    need_big = tvl.attn_tree_workspace_bytes(1, big.parent.shape[1], 24, 4, 256, big.Tcap, 2048)
    need_small = tvl.attn_tree_workspace_bytes(1, small.parent.shape[1], 24, 4, 256, small.Tcap, 0)
    assert need_big > need_small > 256, "both calls should use KV splits (scratch partials)"
    for A in (big, small):
        (o1, l1), (o2, l2) = _both(A)
        assert np.array_equal(o1, o2, equal_nan=True), "outputs differ from attn_tree_verify"
        assert np.array_equal(l1, l2, equal_nan=True), "lse differs from attn_tree_verify"
        assert np.isfinite(o2[0, :int(A.n_nodes[0])]).all()
