"""GPU audio coupling input (prism_audio_norms, through the C ABI) against the oracle.

RG M1: the zone statistics read, per video token, the L2 norm of the token's audio-to-video
cross-attention output.  The GPU norms (fp32 sums of squares, one wave per row) must match the
oracle's fp64 norms of the same values to 1e-5 relative, exactly 0 for zero rows, and, fed into
the zone statistics, give the same coupling strengths and indicators as the oracle's norms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from dynamic_block_sparse_var_amd import BF16, F32, PrismLayer, make_problem, prism_audio_norms
from parity_util import problem_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


@pytest.mark.parametrize("dtype,C", [("bf16", 8), ("bf16", 64), ("bf16", 512), ("bf16", 1032), ("f32", 128)])
def test_norms_match_oracle(dtype, C):
    T, H, W = 8, 16, 16
    N = T * H * W
    rng = np.random.default_rng(5100 + C)
    x = rng.standard_normal((N, C)) * np.exp(rng.normal(0.0, 2.0, size=(N, 1)))
    x[rng.choice(N, 5, replace=False)] = 0.0
    xt = torch.from_numpy(x.astype(np.float32))
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    pb = make_problem(T, H, W, 2, 64, 1, BF16 if dtype == "bf16" else F32)
    xd = xt.cuda()
    a = torch.empty(N, dtype=torch.float32, device="cuda")
    a2 = torch.empty_like(a)
    prism_audio_norms(pb, xd, a)
    prism_audio_norms(pb, xd, a2, squared=True)
    torch.cuda.synchronize()
    xs = xt.float().numpy()
    ref = oracle.audio_norms(xs)
    ref2 = oracle.audio_norms(xs, squared=True)
    got, got2 = a.cpu().numpy().astype(np.float64), a2.cpu().numpy().astype(np.float64)
    zero = ref == 0.0
    assert (got[zero] == 0.0).all() and (got2[zero] == 0.0).all()
    rel = np.abs(got[~zero] - ref[~zero]) / ref[~zero]
    rel2 = np.abs(got2[~zero] - ref2[~zero]) / ref2[~zero]
    say(f"  {dtype} C={C}: max rel err norm {rel.max():.2e}, sum of squares {rel2.max():.2e}")
    assert rel.max() <= 1e-5 and rel2.max() <= 1e-5


def test_norms_feed_zone_statistics():
    """hhat with the config's audio field as row norms -> GPU norms -> GPU zone statistics, against
    the oracle's norms -> oracle zone statistics."""
    cfg = synth.Config("audio_norms", 16, 32, 32, 2, 128, "bf16", blobs=2, k_abs=0, k_frac=0.05, p=0.9,
                       backward=False, seed=2101)
    inp = synth.make_inputs(cfg, with_dout=False)
    C = cfg.heads * cfg.d
    hhat = synth.make_hhat(cfg, inp["a"], C)
    pb = problem_of(cfg)
    L = PrismLayer(pb)
    a = torch.empty(pb.N, dtype=torch.float32, device="cuda")
    prism_audio_norms(pb, torch.from_numpy(hhat).to(torch.bfloat16).cuda(), a)
    v = torch.from_numpy(inp["v"]).to(torch.bfloat16).cuda()
    L.plan(v, a, cfg.eps, cfg.tau128, cfg.tau256)
    torch.cuda.synchronize()
    a_ref = oracle.audio_norms(hhat)
    assert np.abs(a.cpu().numpy() - a_ref).max() <= 1e-5 * a_ref.max()
    st = oracle.zone_stats(inp["v"], a_ref.astype(np.float32), cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, 1, cfg.eps)
    za = L.zone_audio.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(za[:, 0], st["abar"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(za[:, 1:], st["vhat"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(L.g.cpu().numpy().astype(np.float64), st["g"], rtol=1e-4, atol=1e-6)
    # the rows were built with the blob field as their norms: the producer recovers it up to bf16
    rel = np.abs(a_ref - inp["a"]) / inp["a"]
    say(f"  norms vs the generator's field: max rel {rel.max():.2e} (bf16 rounding of hhat)")
    assert rel.max() < 1e-2
