"""GPU parity at the full configured sizes (720p-, 1080p-, 2K-shaped grids, the 2K stress case,
the largest grid, 64x128x128 = 1,048,576 tokens in 2048 zones, and the 720p grid with head dim
64 and a backward), in the launch configuration the benchmark times.

Zone statistics, shapes and the complete selection are compared against the oracle over
every zone and every query block.  Attention outputs and gradients, given the oracle's
shapes and mask, are compared on sampled blocks the oracle computes one by one: O, LSE and
dQ on random query blocks of every head (the C oracle), dK and dV on chosen key blocks of
every head (the fp64 matrix-product oracle, oracle/attn_rows.py, whose cost grows with the
number of query blocks that selected the key block):

* 1080p, 720p at head dim 64, 2K and the 1,048,576-token grid: one rarely selected key block (at most 24 selecting
  query blocks), the key block at the median selector count (the largest grid: first head
  only), and one of the heavy key blocks that the backward's launch order moves to the front
  (selected by more than 2.5 times the mean; the least selected of them, 2K every head, 1080p
  and the largest grid the first head);
* 2K stress: the least selected key block of every head (every key block there is chosen by
  hundreds of query blocks of 256 rows, which is the dispersed regime Top-p expands).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import attn_rows
from parity_util import (LSE_ABS, Run, assert_close_attn, cap, compare_masks, compare_shapes, f64, report, say)

pytestmark = pytest.mark.gpu

FULL = ["720p", "1080p", "2k", "2k_stress", "1m", "720p_d64"]
QB_PER_HEAD = 3
HEAVY = 2.5  # the backward launch order's threshold for dK/dV work (times the mean per atom)


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
    report(f"{c.name} shapes: {n} zones, B=64/128/256: {(vols == 64).sum()}/{(vols == 128).sum()}/"
           f"{(vols == 256).sum()}, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(n)


def test_select_full(run):
    c, o = run.cfg, run.orc
    run.inject_oracle_plan()
    run.gpu_select()
    L = run.layer
    np.testing.assert_allclose(f64(L.qbar), o["qbar"], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(f64(L.kbar), o["kbar"], rtol=1e-5, atol=1e-5)
    hard, soft, rows = compare_masks(L.sel_count.cpu().numpy(), L.sel_idx.cpu().numpy(), o["sel_count"],
                                     o["sel_idx"], o["sel_info"], o["nblocks"], c.groups, qbar=o["qbar"],
                                     kbar=o["kbar"], sm_scale=c.sm_scale)
    nb = int(o["nblocks"][0])
    frac = (o["sel_count"][:, :nb] / nb).mean()
    report(f"{c.name} masks: {rows} rows, mean selected block fraction {frac:.3f}, hard {hard}, near-tie {soft}")
    assert hard == 0 and soft <= cap(rows)


def key_block_picks(c, o, rng):
    """{head: [(label, key block)]} for the dK/dV checks (see the module docstring)."""
    nb = int(o["nblocks"][0])
    bs = o["block_start"][0]
    atoms = np.diff(bs)[:nb] // 64
    picks = {}
    for h in range(c.heads):
        col = attn_rows.selector_counts(o["sel_count"], o["sel_idx"], nb, h)
        used = np.flatnonzero(col > 0)
        order = used[np.argsort(col[used], kind="stable")]
        if c.name == "2k_stress":
            picks[h] = [("least selected", int(order[0]))]
            continue
        out = []
        rare = np.flatnonzero((col > 0) & (col <= 24))
        if len(rare):
            out.append(("rare", int(rng.choice(rare))))
        if h == 0 or c.name != "1m":
            out.append(("median", int(order[len(order) // 2])))
        if h == 0 or c.name == "2k":
            mean_atom = (col * atoms).sum() / atoms.sum()
            heavy = order[col[order] > HEAVY * mean_atom]
            out.append(("heavy", int(heavy[0]) if len(heavy) else int(order[-1])))
        picks[h] = out
    return picks, col


@pytest.mark.timeout(1500)
def test_attention_full_sampled(run):
    c, o = run.cfg, run.orc
    rng = np.random.default_rng(c.seed)
    nb = int(o["nblocks"][0])
    qmask = np.zeros((c.heads, c.nbmax), np.uint8)
    for h in range(c.heads):
        qmask[h, rng.choice(nb, QB_PER_HEAD, replace=False)] = 1
    say(f"  {c.name}: oracle attention on {int(qmask.sum())} query blocks")
    vp = oracle.permute(run.inp["v"], o["pos"], c.heads)
    of, lf = oracle.attn_fwd(o["qp"], o["kp"], vp, o["block_start"], o["nblocks"], c.groups, o["sel_count"],
                             o["sel_idx"], c.sm_scale, qblock_mask=qmask)
    ob = dop = None
    if run.backward:
        dop = oracle.permute(run.inp["dout"], o["pos"], c.heads)
        ob = oracle.attn_bwd(o["qp"], o["kp"], vp, dop, o["block_start"], o["nblocks"], c.groups, o["sel_count"],
                             o["sel_idx"], c.sm_scale, qblock_mask=qmask, kblock_mask=np.zeros_like(qmask))
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
    if not run.backward:
        return
    assert_close_attn("dQ (sampled query blocks)", pick(f64(L.dqp), qrows), pick(ob["dq"], qrows))
    # dK, dV of the chosen key blocks, element by element
    picks, _ = key_block_picks(c, o, rng)
    assert sum(len(v) for v in picks.values()) >= c.heads, "no key block sampled"
    dkp, dvp = L.dkp.cpu().numpy(), L.dvp.cpu().numpy()
    for h, lst in picks.items():
        head = attn_rows.Head(o["qp"], o["kp"], vp, dop, bs, nb, o["sel_count"], o["sel_idx"], h, c.sm_scale)
        for label, j in lst:
            sel = head.selectors(j)
            say(f"  head {h} key block {j} ({label}, {bs[j + 1] - bs[j]} rows, {len(sel)} selecting query "
                f"blocks): oracle ...")
            rows, dk, dv = head.dkdv(j, sel)
            assert_close_attn(f"dK h{h} kb{j} ({label})", dkp[h, rows].astype(np.float64), dk)
            assert_close_attn(f"dV h{h} kb{j} ({label})", dvp[h, rows].astype(np.float64), dv)
        del head
    # exact identities over all keys of a head, at any size: every softmax row sums to 1,
    # so sum_c dV_c = sum_r dO_r; and every row of dS sums to 0, so sum_c dK_c = 0
    for h in range(c.heads):
        dv = L.dvp[h].double().sum(0).cpu().numpy()
        ref = dop[h].astype(np.float64).sum(0)
        rel = np.abs(dv - ref).max() / max(np.abs(ref).max(), 1e-30)
        dk_sum = L.dkp[h].double().sum(0).abs().max().item()
        dk_scale = L.dkp[h].double().abs().sum(0).max().item()
        say(f"  head {h}: |sum dV - sum dO| rel {rel:.2e}; |sum dK| / sum |dK| {dk_sum / dk_scale:.2e}")
        assert rel < 1e-4 and dk_sum <= 1e-4 * dk_scale


def _expected_order(work, heads, units, f):
    """The documented launch order: units of each head in XCD-contiguous order, those whose work
    exceeds f/10 times the mean first, both parts keeping that order."""
    def xcd(x, n):
        return (x & 7) * (n >> 3) + (x >> 3) if n % 8 == 0 else x
    plain = [(t // units) * units + xcd(t % units, units) for t in range(heads * units)]
    n, total = heads * units, int(work.sum())
    heavy = [it for it in plain if 10 * int(work[it]) * n > f * total]
    light = [it for it in plain if not 10 * int(work[it]) * n > f * total]
    return np.array(heavy + light, np.int64), len(heavy)


def test_launch_orders_read_back(run):
    """The launch orders the attention builds in its workspaces, read back at full size (where a
    thread of the order kernel partitions many units): each is the documented partition of the
    plain XCD-contiguous order -- units with more than 1.5x (forward pairs, dQ atoms) or 2.5x
    (dK/dV atoms) the mean work first -- built from work estimates that match the selection."""
    c, o = run.cfg, run.orc
    if not run.backward:
        pytest.skip("forward-only config")
    run.inject_oracle_plan()
    L = run.layer
    from dynamic_block_sparse_var_amd import prism_permute

    prism_permute(run.pb, L.shape_idx, 0, [run.q, run.k, run.v], [L.qp, L.kp, L.vp])
    run.inject_oracle_mask()
    L.attend(c.sm_scale)
    L.backward(run.dout, c.sm_scale)
    torch.cuda.synchronize()
    A = lambda x: (x + 255) // 256 * 256  # noqa: E731
    heads, N = c.heads, c.N
    nb = int(o["nblocks"][0])
    bs = o["block_start"][0].astype(np.int64)
    cnt = o["sel_count"][:, :nb].astype(np.int64)
    col = np.stack([attn_rows.selector_counts(o["sel_count"], o["sel_idx"], nb, h) for h in range(heads)])
    # backward: per atom, its block's list length (dQ) and selector count (dK/dV)
    items = heads * (N // 64)
    ws = L.workspace.cpu().numpy()
    nw = (c.nbmax + 31) // 32
    off = 2 * A(4 * heads * N) + A(4 * heads * c.nbmax * nw)
    order = ws[off:off + 8 * items].view(np.int32).reshape(2, items)
    work = ws[off + A(8 * items):off + A(8 * items) + 8 * items].view(np.int32).reshape(2, items)
    blk = np.searchsorted(bs[:nb + 1], np.arange(0, N, 64), side="right") - 1
    np.testing.assert_array_equal(work[0].reshape(heads, -1), cnt[:, blk])
    np.testing.assert_array_equal(work[1].reshape(heads, -1), col[:, blk])
    for side, f in ((0, 15), (1, 25)):
        want, nheavy = _expected_order(work[side].astype(np.int64), heads, N // 64, f)
        np.testing.assert_array_equal(order[side], want)
        assert np.array_equal(np.sort(order[side]), np.arange(items))
        say(f"  {c.name}: {'dQ' if side == 0 else 'dK/dV'} launch order: {nheavy} of {items} atoms first")
    # forward: pairs of atoms, work twice the zone's longest list (zones of 64-row blocks) or twice
    # the pair's block list
    pairs = heads * (N // 128)
    fw = L.fwd_workspace.cpu().numpy()
    forder = fw[:4 * pairs].view(np.int32)
    fwork = fw[A(4 * pairs):A(4 * pairs) + 4 * pairs].view(np.int32).reshape(heads, -1)
    j0 = np.searchsorted(bs[:nb + 1], np.arange(0, N, 512), side="right") - 1
    small = (bs[j0 + 1] - bs[j0]) == 64
    for h in range(heads):
        zw = np.where(small, np.max(np.stack([cnt[h, np.minimum(j0 + q, nb - 1)] for q in range(8)]), 0), 0)
        for s_ in range(4):
            big = cnt[h, np.minimum(j0 + (128 * s_) // np.maximum(bs[j0 + 1] - bs[j0], 1), nb - 1)]
            np.testing.assert_array_equal(fwork[h, s_::4], 2 * np.where(small, zw, big))
    want, nheavy = _expected_order(fwork.reshape(-1).astype(np.int64), heads, N // 128, 15)
    np.testing.assert_array_equal(forder, want)
    say(f"  {c.name}: forward launch order: {nheavy} of {pairs} pairs first")


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
