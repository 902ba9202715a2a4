"""The autograd front (PrismAttention / PrismAttentionFunction) against the layer calls it
wraps: the same outputs and gradients bit for bit, buffers allocated once per module, and a
backward after a second forward on the same layer refused."""
import pytest
import torch

import synth
from dynamic_block_sparse_var_amd import PrismAttention, PrismLayer, make_problem
from parity_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.Config("autograd", 8, 16, 32, 2, 128, "bf16", blobs=1, k_abs=0, k_frac=0.1, p=0.9, backward=True,
                       seed=2101)
    inp = synth.make_inputs(cfg, with_dout=True)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    return cfg, inp, dev


def test_autograd_equals_layer_calls(case):
    cfg, inp, dev = case
    pb = make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, 1, "bf16")
    a = torch.from_numpy(inp["a"]).cuda()
    do = dev(inp["dout"])
    ref = PrismLayer(pb, backward=True, token_io=True)
    o_ref = ref.forward(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), a, cfg.sm_scale, cfg.k_abs, cfg.k_frac, cfg.p)
    dq_ref, dk_ref, dv_ref = ref.backward(do, cfg.sm_scale)
    torch.cuda.synchronize()

    mod = PrismAttention(pb, cfg.sm_scale, cfg.k_abs, cfg.k_frac, cfg.p)
    bufs = {name: getattr(mod.layer, name).data_ptr() for name in ("qp", "sel_idx", "o", "dq", "workspace")}
    for it in range(2):  # the second step reuses the module's buffers
        q, k, v = (dev(inp[x]).requires_grad_() for x in ("q", "k", "v"))
        o = mod(q, k, v, a)
        o.backward(do)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        assert torch.equal(q.grad, dq_ref.to(torch.bfloat16))
        assert torch.equal(k.grad, dk_ref.to(torch.bfloat16))
        assert torch.equal(v.grad, dv_ref.to(torch.bfloat16))
        for name, ptr in bufs.items():
            assert getattr(mod.layer, name).data_ptr() == ptr, name
    say("  autograd front: outputs and gradients bitwise equal to the layer calls over two steps")


def test_backward_after_second_forward_is_refused(case):
    cfg, inp, dev = case
    pb = make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, 1, "bf16")
    a = torch.from_numpy(inp["a"]).cuda()
    mod = PrismAttention(pb, cfg.sm_scale, cfg.k_abs, cfg.k_frac, cfg.p)
    q, k, v = (dev(inp[x]).requires_grad_() for x in ("q", "k", "v"))
    o1 = mod(q, k, v, a)
    mod(q, k, v, a)
    with pytest.raises(RuntimeError, match="another forward"):
        o1.backward(dev(inp["dout"]))
