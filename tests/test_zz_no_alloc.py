"""The allocation-free backward (prism_bsa_bwd_noalloc, workspace in the library's fixed
per-device scratch) against prism_bsa_bwd with a caller workspace, through the C ABI: the same
dQ, dK, dV bit for bit, on two calls in a row, the second on a smaller problem (the scratch
keeps the first call's contents, which must not matter)."""
import pytest
import torch

import synth
from dynamic_block_sparse_var_amd import (PrismLayer, make_problem, prism_bsa_bwd, prism_bsa_bwd_noalloc,
                                          prism_bsa_bwd_noalloc_max_bytes, prism_bsa_bwd_workspace_bytes)
from parity_util import say

pytestmark = pytest.mark.gpu

CASES = [
    synth.Config("noalloc_a", 16, 32, 32, 2, 128, "bf16", blobs=2, k_abs=0, k_frac=0.05, p=0.9, backward=True,
                 seed=2201),
    synth.Config("noalloc_b", 8, 16, 32, 2, 64, "bf16", blobs=1, k_abs=3, k_frac=0.0, p=0.8, backward=True,
                 seed=2202),
]


def _run(cfg):
    inp = synth.make_inputs(cfg, with_dout=True)
    pb = make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, 1, "bf16")
    L = PrismLayer(pb, backward=True)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    a = torch.from_numpy(inp["a"]).cuda()
    L.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), a, cfg.sm_scale, cfg.k_abs, cfg.k_frac, cfg.p)
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(pb, L.shape_idx, 0, [dev(inp["dout"])], [L.dop])
    args = (pb, L.block_start, L.sel_count, L.sel_idx, cfg.sm_scale, L.qp, L.kp, L.vp, L.op, L.op_lo, L.dop, L.lse)
    ref = [torch.full_like(L.dqp, float("nan")) for _ in range(3)]
    prism_bsa_bwd(*args, *ref, L.workspace)
    got = [torch.full_like(L.dqp, float("nan")) for _ in range(3)]
    prism_bsa_bwd_noalloc(*args, *got)
    torch.cuda.synchronize()
    assert prism_bsa_bwd_workspace_bytes(pb) <= prism_bsa_bwd_noalloc_max_bytes()
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert not torch.isnan(y).any(), name
        assert torch.equal(x, y), name
    say(f"  {cfg.name}: allocation-free backward bitwise equal to the workspace call "
        f"({prism_bsa_bwd_workspace_bytes(pb)} of {prism_bsa_bwd_noalloc_max_bytes()} scratch bytes)")


def test_noalloc_backward_equals_workspace_backward_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for cfg in CASES:  # the second call is the smaller problem
        _run(cfg)
