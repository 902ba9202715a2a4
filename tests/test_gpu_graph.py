"""The whole layer (statistics through the attention backward) captured once in a HIP graph and
replayed: the calls make no host synchronisation, allocation or memset, so the captured
kernels replay exactly.  Every replay must reproduce the eager run bit for bit; the outputs
are overwritten with garbage before each replay, and other eager GPU work runs between the
replays."""
import numpy as np
import pytest
import torch

import synth
from dynamic_block_sparse_var_amd import PrismLayer, make_problem
from parity_util import say

pytestmark = pytest.mark.gpu

CASES = {
    # bf16, matrix-core kernels with their launch orders, Top-p extending lists
    "small_bf16": synth.Config("small_bf16", 16, 32, 32, 2, 128, "bf16", blobs=2, k_abs=0, k_frac=0.05, p=0.9,
                               backward=True, seed=2002),
    # fp32 path, head dim 64
    "tiny": synth.CONFIGS["tiny"].replace(backward=True),
}

OUTS = ("g", "rho", "zone_audio", "shape_idx", "zone_block_off", "block_start", "o", "o_lo", "lse", "dq", "dk",
        "dv")
BLOCK_ROWS = ("qbar", "kbar", "sel_count")  # [heads, NBMAX, ...]: compared over the layer's N_b blocks


@pytest.mark.parametrize("name", list(CASES))
def test_layer_replays_bitwise_in_a_graph(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = CASES[name]
    inp = synth.make_inputs(cfg, with_dout=True)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()  # noqa: E731
    q, k, v, do = dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["dout"])
    a = torch.from_numpy(inp["a"]).cuda()
    pb = make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.groups, cfg.dtype)
    L = PrismLayer(pb, backward=True, token_io=True)

    def step():
        L.forward(q, k, v, a, cfg.sm_scale, cfg.k_abs, cfg.k_frac, cfg.p)
        L.backward(do, cfg.sm_scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                          # eager reference, on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    nb = int(L.block_start.cpu().numpy()[0].searchsorted(cfg.N))

    def outputs():
        out = {n: getattr(L, n) for n in OUTS if getattr(L, n) is not None}
        out.update({n: getattr(L, n)[:, :nb] for n in BLOCK_ROWS})
        return out

    ref = {n: t.clone() for n, t in outputs().items()}
    cnt = L.sel_count.cpu().numpy()
    sel_ref = [L.sel_idx[h, i, :cnt[h, i]].clone() for h in range(cfg.heads) for i in range(nb)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()

    x = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        for t in outputs().values():                    # garbage in every output before the replay
            t.fill_(float("nan") if t.is_floating_point() else 123)
        L.sel_idx.fill_(123)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_all = outputs()
        for n, r in ref.items():                        # bit patterns, so NaN or -inf compare too
            got = got_all[n]
            assert torch.equal(got.contiguous().view(torch.uint8), r.contiguous().view(torch.uint8)), \
                f"{name} replay {rep}: {n}"
        j = 0
        for h in range(cfg.heads):
            for i in range(nb):
                assert torch.equal(L.sel_idx[h, i, :cnt[h, i]], sel_ref[j]), f"{name} replay {rep}: sel_idx"
                j += 1
        y = (x @ x).sum()                               # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(y)
    say(f"  {name}: 3 graph replays of the whole layer bitwise equal to the eager run")
