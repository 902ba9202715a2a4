"""GPU parity at the full configured sizes (720p-, 1080p-, 2K-shaped grids and the 2K stress
case), in the launch configuration the benchmark times.

Zone statistics, shapes and the complete selection are compared against the oracle over
every zone and every query block.  Attention outputs and gradients, given the oracle's
shapes and mask, are compared on sampled blocks the oracle computes one by one: O, LSE and
dQ on random query blocks of every head, dK and dV on random key blocks of every head drawn
from those selected by at most 24 query blocks (the oracle's cost of a key block's gradient
grows with the number of query blocks that attend to it).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (LSE_ABS, Run, assert_close_attn, cap, compare_masks, compare_shapes, f64, say)

pytestmark = pytest.mark.gpu

FULL = ["720p", "1080p", "2k", "2k_stress"]
QB_PER_HEAD = 3
KB_PER_HEAD = 1


@pytest.fixture(scope="module", params=FULL)
def run(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    r = Run(synth.CONFIGS[request.param])
    yield r
    del r
    torch.cuda.empty_cache()


def test_plan_full(run):
    c, o = run.cfg, run.orc
    run.gpu_plan()
    L = run.layer
    np.testing.assert_allclose(f64(L.g), o["stats"]["g"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(f64(L.rho), o["stats"]["rho"], rtol=1e-4, atol=1e-6)
    za = f64(L.zone_audio)
    np.testing.assert_allclose(za[:, 0], o["stats"]["abar"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(za[:, 1:], o["stats"]["vhat"], rtol=1e-4, atol=1e-6)
    hard, soft, n = compare_shapes(L.shape_idx.cpu().numpy(), o["stats"], o["shapes"], c.tau128, c.tau256)
    vols = np.array([64] * 7 + [128] * 6 + [256] * 3)[o["shapes"]["shape_idx"]]
    say(f"  {c.name}: {n} zones, B=64/128/256: {(vols == 64).sum()}/{(vols == 128).sum()}/{(vols == 256).sum()}, "
        f"hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(n)


def test_select_full(run):
    c, o = run.cfg, run.orc
    run.inject_oracle_plan()
    run.gpu_select()
    L = run.layer
    np.testing.assert_allclose(f64(L.qbar), o["qbar"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(f64(L.kbar), o["kbar"], rtol=1e-5, atol=1e-5)
    hard, soft, rows = compare_masks(L.sel_count.cpu().numpy(), L.sel_idx.cpu().numpy(), o["sel_count"],
                                     o["sel_idx"], o["sel_info"], o["nblocks"], c.groups)
    nb = int(o["nblocks"][0])
    frac = (o["sel_count"][:, :nb] / nb).mean()
    say(f"  {c.name}: {rows} rows, mean selected block fraction {frac:.3f}, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(rows)


def test_attention_full_sampled(run):
    c, o = run.cfg, run.orc
    rng = np.random.default_rng(c.seed)
    nb = int(o["nblocks"][0])
    qmask = np.zeros((c.heads, c.nbmax), np.uint8)
    kmask = np.zeros((c.heads, c.nbmax), np.uint8)
    colcount = np.zeros((c.heads, nb), np.int64)
    for h in range(c.heads):
        qmask[h, rng.choice(nb, QB_PER_HEAD, replace=False)] = 1
        for i in range(nb):
            colcount[h, o["sel_idx"][h, i, :o["sel_count"][h, i]]] += 1
        cand = np.flatnonzero((colcount[h] > 0) & (colcount[h] <= 24))
        if len(cand):
            kmask[h, rng.choice(cand, min(KB_PER_HEAD, len(cand)), replace=False)] = 1
    say(f"  {c.name}: oracle attention on {int(qmask.sum())} query blocks, {int(kmask.sum())} key blocks")
    vp = oracle.permute(run.inp["v"], o["pos"], c.heads)
    of, lf = oracle.attn_fwd(o["qp"], o["kp"], vp, o["block_start"], o["nblocks"], c.groups, o["sel_count"],
                             o["sel_idx"], c.sm_scale, qblock_mask=qmask)
    ob = None
    if run.backward:
        dop = oracle.permute(run.inp["dout"], o["pos"], c.heads)
        ob = oracle.attn_bwd(o["qp"], o["kp"], vp, dop, o["block_start"], o["nblocks"], c.groups, o["sel_count"],
                             o["sel_idx"], c.sm_scale, qblock_mask=qmask, kblock_mask=kmask)
    # GPU, given the oracle's plan and mask, in block order
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    run.inject_oracle_mask()
    L.attend(c.sm_scale)
    if run.backward:
        L.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    bs = o["block_start"][0]

    def rows_of(mask):
        out = []
        for h in range(c.heads):
            for j in np.flatnonzero(mask[h, :nb]):
                out.append((h, np.arange(bs[j], bs[j + 1])))
        return out

    qrows = rows_of(qmask)
    pick = lambda arr, rows: np.concatenate([arr[h, r] for h, r in rows])  # noqa: E731
    op = f64(L.op)
    assert_close_attn("O (sampled query blocks)", pick(op, qrows), pick(of, qrows))
    dl = np.abs(pick(L.lse.cpu().numpy().astype(np.float64), qrows) - pick(lf, qrows)).max()
    say(f"  LSE: max_abs={dl:.3e}")
    assert dl <= LSE_ABS
    if run.backward:
        assert_close_attn("dQ (sampled query blocks)", pick(f64(L.dqp), qrows), pick(ob["dq"], qrows))
        krows = rows_of(kmask)
        if krows:
            assert_close_attn("dK (sampled key blocks)", pick(f64(L.dkp), krows), pick(ob["dk"], krows))
            assert_close_attn("dV (sampled key blocks)", pick(f64(L.dvp), krows), pick(ob["dv"], krows))
        # exact identities over all keys of a head, at any size: every softmax row sums to 1,
        # so sum_c dV_c = sum_r dO_r; and every row of dS sums to 0, so sum_c dK_c = 0
        dop = oracle.permute(run.inp["dout"], o["pos"], c.heads).astype(np.float64)
        for h in range(c.heads):
            dv = L.dvp[h].double().sum(0).cpu().numpy()
            ref = dop[h].sum(0)
            rel = np.abs(dv - ref).max() / max(np.abs(ref).max(), 1e-30)
            dk_sum = L.dkp[h].double().sum(0).abs().max().item()
            dk_scale = L.dkp[h].double().abs().sum(0).max().item()
            say(f"  head {h}: |sum dV - sum dO| rel {rel:.2e}; |sum dK| / sum |dK| {dk_sum / dk_scale:.2e}")
            assert rel < 1e-4 and dk_sum <= 1e-4 * dk_scale


def test_token_order_path_full(run):
    """The path the benchmark times (one-pass permute+pool, token-order attention) at full size:
    bitwise equal to the block-order calls plus permutes, whose parity the tests above check,
    given the oracle's plan and mask."""
    from dynamic_block_sparse_var_amd import PrismLayer, prism_permute, prism_permute_pool

    c = run.cfg
    run.inject_oracle_plan()
    L = run.layer
    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    run.inject_oracle_mask()
    L.attend(c.sm_scale)
    if run.backward:
        L.backward(run.dout, c.sm_scale)
    T = PrismLayer(run.pb, backward=run.backward, token_io=True)
    for name in ("shape_idx", "zone_block_off", "block_start", "sel_count", "sel_idx"):
        getattr(T, name).copy_(getattr(L, name))
    prism_permute_pool(run.pb, T.shape_idx, T.zone_block_off, [run.q, run.k, run.v], [T.qp, T.kp, T.vp],
                       [T.qbar, T.kbar, None])
    T.attend(c.sm_scale)
    if run.backward:
        T.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    for name in ("qp", "kp", "vp", "o", "lse") + (("dq", "dk", "dv") if run.backward else ()):
        assert torch.equal(getattr(T, name), getattr(L, name)), name
    say(f"  {c.name}: token-order path bitwise equal to block order + permutes")
    del T
    torch.cuda.empty_cache()
