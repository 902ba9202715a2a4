"""GPU parity of every stage of the HIP path (through the C ABI) against the CPU oracle, on
small seeded configs that still span several zones, tiles and mixed block volumes.

Comparison rules: integer outputs (shape indices, block offsets, permutations, masks) exact,
with near-tie decisions (oracle margin < 1e-5 relative) counted separately and capped at
0.1 % of cases; fp32 statistics to 1e-4 relative; attention outputs and gradients, computed
given the oracle's shapes and mask, within max-abs 2e-2 and mean-relative 5e-3, LSE within
1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from dynamic_block_sparse_var_amd import PrismLayer
from parity_util import (LSE_ABS, Run, assert_close_attn, cap, compare_masks, compare_shapes, f64, report, say)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": synth.CONFIGS["tiny"].replace(backward=True),
    "tiny_bf16": synth.CONFIGS["tiny"].replace(name="tiny_bf16", dtype="bf16", d=128, backward=True, seed=2001),
    "small_bf16": synth.Config("small_bf16", 16, 32, 32, 2, 128, "bf16", blobs=2, k_abs=0, k_frac=0.05, p=0.9,
                               backward=True, seed=2002),
    "d64_groups2": synth.Config("d64_groups2", 8, 16, 32, 4, 64, "bf16", blobs=1, k_abs=3, k_frac=0.0, p=0.8,
                                backward=True, seed=2003, groups=2, gamma=6.0),
    # the 2K stress regime's generator on a grid the oracle covers in full: field amplitude 0.1
    # on V (near-isotropic zones, 256-row blocks), logits x 0.3, k 2 %, p 0.95, so Top-p
    # expands most lists far beyond k (the pages' dispersed-attention case)
    "stress_small": synth.Config("stress_small", 16, 16, 32, 2, 128, "bf16", blobs=2, k_abs=0, k_frac=0.02,
                                 p=0.95, backward=True, seed=2004, amp_v=0.1, gamma=16.0 * 0.3),
    # the smallest grid: one 8x8x8 zone (2 to 8 blocks, 8 atoms and 4 atom pairs per head)
    "one_zone": synth.Config("one_zone", 8, 8, 8, 2, 128, "bf16", blobs=1, k_abs=1, k_frac=0.0, p=0.5,
                             backward=True, seed=2005),
}


@pytest.fixture(scope="module", params=list(SMALL))
def run(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    r = Run(SMALL[request.param])
    yield r
    del r
    torch.cuda.empty_cache()


def test_zone_stats_and_shapes(run):
    c, o = run.cfg, run.orc
    run.gpu_plan()
    L = run.layer
    np.testing.assert_allclose(f64(L.g), o["stats"]["g"], rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(f64(L.rho), o["stats"]["rho"], rtol=1e-4, atol=1e-6)
    za = f64(L.zone_audio)
    np.testing.assert_allclose(za[:, 0], o["stats"]["abar"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(za[:, 1:], o["stats"]["vhat"], rtol=1e-4, atol=1e-6)
    shape = L.shape_idx.cpu().numpy()
    hard, soft, n = compare_shapes(shape, o["stats"], o["shapes"], c.tau128, c.tau256)
    report(f"{c.name} shapes: {n} zones, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(n)
    if soft == 0:
        assert np.array_equal(L.zone_block_off.cpu().numpy(), o["shapes"]["zone_block_off"])
        assert np.array_equal(L.block_start.cpu().numpy(), o["block_start"])


def test_zone_stats_without_audio(run):
    """First layer (no cached audio norms): g = r + eps."""
    c = run.cfg
    st = oracle.zone_stats(run.inp["v"], None, c.T, c.H, c.W, c.heads, c.d, c.groups, c.eps)
    run.gpu_plan(with_audio=False)
    np.testing.assert_allclose(f64(run.layer.g), st["g"], rtol=1e-4, atol=1e-6)


def test_permute_bitwise_and_inverse(run):
    run.inject_oracle_plan()
    L, o, c = run.layer, run.orc, run.cfg
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    back = torch.empty_like(run.q)
    prism_permute(run.pb, L.shape_idx, 1, [L.kp], [back])
    torch.cuda.synchronize()
    assert np.array_equal(L.qp.float().cpu().numpy(), o["qp"])
    assert np.array_equal(L.kp.float().cpu().numpy(), o["kp"])
    assert np.array_equal(L.vp.float().cpu().numpy(), oracle.permute(run.inp["v"], o["pos"], c.heads))
    assert torch.equal(back, run.k)


def test_pool(run):
    run.inject_oracle_plan()
    run.gpu_select()
    o = run.orc
    np.testing.assert_allclose(f64(run.layer.qbar), o["qbar"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(f64(run.layer.kbar), o["kbar"], rtol=1e-5, atol=1e-5)


def test_select(run):
    run.inject_oracle_plan()
    run.gpu_select()
    L, o, c = run.layer, run.orc, run.cfg
    hard, soft, rows = compare_masks(L.sel_count.cpu().numpy(), L.sel_idx.cpu().numpy(), o["sel_count"],
                                     o["sel_idx"], o["sel_info"], o["nblocks"], c.groups, qbar=o["qbar"],
                                     kbar=o["kbar"], sm_scale=c.sm_scale)
    report(f"{c.name} masks: {rows} rows, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(rows)
    nb = o["nblocks"]
    hpg = c.heads // c.groups
    for h in range(c.heads):
        assert (L.sel_count.cpu().numpy()[h, nb[h // hpg]:] == 0).all()


def _oracle_attention(run):
    if getattr(run, "_oatt", None) is None:
        o, c = run.orc, run.cfg
        vp = oracle.permute(run.inp["v"], o["pos"], c.heads)
        of, lf = oracle.attn_fwd(o["qp"], o["kp"], vp, o["block_start"], o["nblocks"], c.groups, o["sel_count"],
                                 o["sel_idx"], c.sm_scale)
        ob = None
        if run.backward:
            dop = oracle.permute(run.inp["dout"], o["pos"], c.heads)
            ob = oracle.attn_bwd(o["qp"], o["kp"], vp, dop, o["block_start"], o["nblocks"], c.groups,
                                 o["sel_count"], o["sel_idx"], c.sm_scale)
        run._oatt = (of, lf, ob)
    return run._oatt


def _gpu_attention(run):
    c = run.cfg
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    run.inject_oracle_mask()
    L.attend(c.sm_scale)
    if run.backward:
        L.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()


def test_attention_forward(run):
    o = run.orc
    of, lf, _ = _oracle_attention(run)
    _gpu_attention(run)
    L = run.layer
    assert_close_attn("O", f64(L.o), oracle.unpermute(of, o["pos"], run.cfg.heads))
    lse = L.lse.cpu().numpy().astype(np.float64)
    dl = np.abs(lse - lf).max()
    say(f"  LSE: max_abs={dl:.3e}")
    assert dl <= LSE_ABS


def test_attention_backward(run):
    if not run.backward:
        pytest.skip("forward-only config")
    o, c = run.orc, run.cfg
    _, _, ob = _oracle_attention(run)
    _gpu_attention(run)
    L = run.layer
    for name, mine, ref in (("dQ", L.dq, ob["dq"]), ("dK", L.dk, ob["dk"]), ("dV", L.dv, ob["dv"])):
        assert_close_attn(name, f64(mine), oracle.unpermute(ref, o["pos"], c.heads))


def test_empty_lists(run):
    """Query blocks with an empty list (possible through the C ABI with a caller's selection):
    their rows get O = 0 and LSE = -inf, zero dQ and no share in dK, dV; every other row is
    unchanged.  Blocks i with i % 5 in {1, 2} are emptied, which leaves atom pairs of the
    forward with one empty and one non-empty list as well as pairs with both lists empty."""
    c, o = run.cfg, run.orc
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    cnt = o["sel_count"].copy()
    blk = np.arange(cnt.shape[1])
    cnt[:, (blk % 5 == 1) | (blk % 5 == 2)] = 0
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.sel_idx.copy_(torch.from_numpy(o["sel_idx"]))
    L.attend(c.sm_scale)
    if run.backward:
        L.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    vp = oracle.permute(run.inp["v"], o["pos"], c.heads)
    of, lf = oracle.attn_fwd(o["qp"], o["kp"], vp, o["block_start"], o["nblocks"], c.groups, cnt, o["sel_idx"],
                             c.sm_scale)
    assert_close_attn("O (empty lists)", f64(L.o), oracle.unpermute(of, o["pos"], c.heads))
    lse = L.lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lf)
    assert (~fin).any(), "no row had an empty list"
    assert np.isneginf(lse[~fin]).all()
    assert np.abs(lse[fin] - lf[fin]).max() <= LSE_ABS
    if run.backward:
        dop = oracle.permute(run.inp["dout"], o["pos"], c.heads)
        ob = oracle.attn_bwd(o["qp"], o["kp"], vp, dop, o["block_start"], o["nblocks"], c.groups, cnt,
                             o["sel_idx"], c.sm_scale)
        for name, mine, ref in (("dQ", L.dq, ob["dq"]), ("dK", L.dk, ob["dk"]), ("dV", L.dv, ob["dv"])):
            assert_close_attn(name + " (empty lists)", f64(mine), oracle.unpermute(ref, o["pos"], c.heads))


def test_forward_launch_order_bitwise(run):
    """The launch orders (heaviest units first, built on the device in the workspaces) only
    change which workgroup runs when: O, LSE and the gradients are bitwise those of the plain
    launch order (prism_set_launch_order(0)); outputs are pre-filled with NaN so a unit that
    never ran would show."""
    c = run.cfg
    if c.dtype != "bf16":
        pytest.skip("fp32 problems run the plain kernels, without a launch order")
    from dynamic_block_sparse_var_amd import prism_permute, prism_set_launch_order

    run.inject_oracle_plan()
    L = run.layer
    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    run.inject_oracle_mask()
    outs = []
    try:
        for heavy in (True, False):
            prism_set_launch_order(heavy)
            for t in [L.o, L.lse] + ([L.dq, L.dk, L.dv] if run.backward else []):
                t.fill_(float("nan"))
            L.attend(c.sm_scale)
            if run.backward:
                L.backward(run.dout, c.sm_scale)
            torch.cuda.synchronize()
            outs.append([t.clone() for t in [L.o, L.lse] + ([L.dq, L.dk, L.dv] if run.backward else [])])
    finally:
        prism_set_launch_order(True)
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert not torch.isnan(outs[0][0].float()).any()


def test_deterministic(run):
    _gpu_attention(run)
    L = run.layer
    first = [t.clone() for t in ([L.o, L.lse] + ([L.dq, L.dk, L.dv] if run.backward else []))]
    _gpu_attention(run)
    second = [L.o, L.lse] + ([L.dq, L.dk, L.dv] if run.backward else [])
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_all_blocks_is_dense_attention(run):
    """Every key block selected: the sparse kernel must equal dense attention (torch SDPA in
    fp32 on the CPU, on the same bf16/fp32 inputs)."""
    c, o = run.cfg, run.orc
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    nb = o["nblocks"]
    hpg = c.heads // c.groups
    cnt = np.zeros_like(o["sel_count"])
    idx = np.zeros_like(o["sel_idx"])
    for h in range(c.heads):
        n = nb[h // hpg]
        cnt[h, :n] = n
        idx[h, :n, :n] = np.arange(n)
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.sel_idx.copy_(torch.from_numpy(idx))
    L.attend(c.sm_scale)
    torch.cuda.synchronize()
    q = torch.from_numpy(run.inp["q"]).permute(1, 0, 2)
    k = torch.from_numpy(run.inp["k"]).permute(1, 0, 2)
    v = torch.from_numpy(run.inp["v"]).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], scale=c.sm_scale)[0]
    assert_close_attn("dense O", f64(L.o), ref.permute(1, 0, 2).double().numpy())


def test_all_blocks_dense_backward(run):
    """Every key block selected (the dense baseline's selection): the sparse backward must equal
    the gradient of dense softmax attention, taken by torch autograd in fp64 on the CPU from the
    same inputs (per head: O = softmax(sm_scale Q K^T) V, loss = sum O * dO)."""
    if not run.backward:
        pytest.skip("forward-only config")
    c, o = run.cfg, run.orc
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    nb = o["nblocks"]
    hpg = c.heads // c.groups
    cnt = np.zeros_like(o["sel_count"])
    idx = np.zeros_like(o["sel_idx"])
    for h in range(c.heads):
        n = nb[h // hpg]
        cnt[h, :n] = n
        idx[h, :n, :n] = np.arange(n)
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.sel_idx.copy_(torch.from_numpy(idx))
    L.attend(c.sm_scale)
    L.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    ref = {name: np.zeros((c.N, c.heads, c.d)) for name in ("dq", "dk", "dv")}
    for h in range(c.heads):
        q, k, v = (torch.from_numpy(run.inp[x][:, h, :]).double().requires_grad_() for x in ("q", "k", "v"))
        out = torch.softmax((q @ k.T) * c.sm_scale, dim=-1) @ v
        out.backward(torch.from_numpy(run.inp["dout"][:, h, :]).double())
        for name, t in (("dq", q), ("dk", k), ("dv", v)):
            ref[name][:, h, :] = t.grad.numpy()
        del q, k, v, out
    for name in ("dq", "dk", "dv"):
        assert_close_attn(f"dense {name}", f64(getattr(L, name)), ref[name])


def test_fixed_shapes_path(run):
    """Fixed 4x4x4 blocks for every zone (the pages' fixed-block ablation): layout exact against
    the oracle's block order for the same shape map, then permute, pool, selection and the
    forward on that layout against the oracle."""
    from dynamic_block_sparse_var_amd import fixed_shape_index, prism_permute

    c, L = run.cfg, run.layer
    fs = fixed_shape_index((4, 4, 4))
    run.layer.plan(run.v, run.a, c.eps, c.tau128, c.tau256, fixed_shape=fs)
    torch.cuda.synchronize()
    shp = np.full((c.groups, c.Z), fs, np.uint8)
    pos, bs, nb = oracle.block_layout(c.T, c.H, c.W, shp)
    assert (L.shape_idx.cpu().numpy() == fs).all()
    np.testing.assert_array_equal(L.block_start.cpu().numpy(), bs)
    zbo = L.zone_block_off.cpu().numpy()
    np.testing.assert_array_equal(zbo[:, -1], nb)
    np.testing.assert_array_equal(zbo[:, :-1], np.broadcast_to(np.arange(c.Z) * 8, (c.groups, c.Z)))
    # the rest of the path on this layout
    run.gpu_select()
    qp = oracle.permute(run.inp["q"], pos, c.heads)
    kp = oracle.permute(run.inp["k"], pos, c.heads)
    np.testing.assert_array_equal(f64(L.qp), qp)
    qbar = oracle.pool(qp, bs, nb, c.groups)
    kbar = oracle.pool(kp, bs, nb, c.groups)
    np.testing.assert_allclose(f64(L.qbar), qbar, rtol=1e-5, atol=1e-5)
    cnt, idx, info = oracle.select(qbar, kbar, nb, c.groups, c.sm_scale, c.k_abs, c.k_frac, c.p)
    hard, soft, rows = compare_masks(L.sel_count.cpu().numpy(), L.sel_idx.cpu().numpy(), cnt, idx, info, nb,
                                     c.groups, qbar=qbar, kbar=kbar, sm_scale=c.sm_scale)
    report(f"{c.name} fixed 4x4x4 masks: {int(nb[0])} blocks, {rows} rows, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(rows)
    L.sel_count.copy_(torch.from_numpy(cnt))
    L.sel_idx.copy_(torch.from_numpy(idx))
    L.attend(c.sm_scale)
    torch.cuda.synchronize()
    vp = oracle.permute(run.inp["v"], pos, c.heads)
    of, lf = oracle.attn_fwd(qp, kp, vp, bs, nb, c.groups, cnt, idx, c.sm_scale)
    assert_close_attn("O (fixed shapes)", f64(L.o), oracle.unpermute(of, pos, c.heads))
    assert np.abs(L.lse.cpu().numpy().astype(np.float64) - lf).max() <= LSE_ABS


def test_dense_selection_through_select(run):
    """k = N_b through the selection kernel itself selects every block, in order (the dense
    baseline runs the same kernels with this selection)."""
    c, o, L = run.cfg, run.orc, run.layer
    run.inject_oracle_plan()
    L.select(run.q, run.k, run.v, c.sm_scale, c.nbmax, 0.0, c.p)
    torch.cuda.synchronize()
    nb = o["nblocks"]
    hpg = c.heads // c.groups
    cnt, idx = L.sel_count.cpu().numpy(), L.sel_idx.cpu().numpy()
    for h in range(c.heads):
        n = int(nb[h // hpg])
        assert (cnt[h, :n] == n).all() and (cnt[h, n:] == 0).all()
        np.testing.assert_array_equal(idx[h, :n, :n], np.broadcast_to(np.arange(n), (n, n)))


def test_token_order_attention_bitwise(run):
    """prism_bsa_fwd_tok / prism_bsa_bwd_tok write O, its residual and the gradients straight
    to token order: they must equal the block-order calls followed by the inverse permute, bit
    for bit (same arithmetic, different output rows), given the oracle's plan and mask."""
    c = run.cfg
    _gpu_attention(run)
    L = run.layer
    ref = {"o": L.o.clone(), "lse": L.lse.clone()}
    if run.backward:
        ref.update(dq=L.dq.clone(), dk=L.dk.clone(), dv=L.dv.clone())
        if L.op_lo is not None:
            from dynamic_block_sparse_var_amd import prism_permute

            lo = torch.empty_like(L.o)
            prism_permute(run.pb, L.shape_idx, 1, [L.op_lo], [lo])
            ref["o_lo"] = lo
    T = PrismLayer(run.pb, backward=run.backward, token_io=True)
    for name in ("shape_idx", "zone_block_off", "block_start", "qp", "kp", "vp", "sel_count", "sel_idx"):
        getattr(T, name).copy_(getattr(L, name))
    T.attend(c.sm_scale)
    if run.backward:
        T.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(T.o, ref["o"])
    assert torch.equal(T.lse, ref["lse"])
    if run.backward:
        for name in ("dq", "dk", "dv"):
            assert torch.equal(getattr(T, name), ref[name]), name
        if "o_lo" in ref:
            assert torch.equal(T.o_lo, ref["o_lo"])
    say(f"  token-order outputs bitwise equal to block order + inverse permute ({c.name})")


def test_permute_pool_bitwise(run):
    """prism_permute_pool = prism_permute + prism_pool_blocks, bit for bit, with pooled rows past
    N_b zero (the outputs are pre-filled with NaN) and no pooling for a tensor whose xbar is
    None."""
    from dynamic_block_sparse_var_amd import prism_permute, prism_permute_pool, prism_pool_blocks

    run.inject_oracle_plan()
    L = run.layer
    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    prism_pool_blocks(run.pb, L.block_start, [L.qp, L.kp], [L.qbar, L.kbar])
    outs = [torch.full_like(t, float("nan")) for t in (L.qp, L.kp, L.vp, L.qbar, L.kbar)]
    prism_permute_pool(run.pb, L.shape_idx, L.zone_block_off, [run.q, run.k, run.v], outs[:3], outs[3:] + [None])
    torch.cuda.synchronize()
    for mine, ref in zip(outs, (L.qp, L.kp, L.vp, L.qbar, L.kbar)):
        assert torch.equal(mine, ref)
