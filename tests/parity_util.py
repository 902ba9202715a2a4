"""Helpers for the GPU-vs-oracle parity tests: running the HIP path through the C ABI on
seeded inputs, and the comparison rules (exact for integers, near-tie accounting for
discrete decisions, max-abs / mean-relative tolerances for attention)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import synth
from dynamic_block_sparse_var_amd import PrismLayer, make_problem

# tolerances of the attention outputs and gradients (bf16 in, fp32 accumulate)
MAX_ABS = 2e-2
MEAN_REL = 5e-3
LSE_ABS = 1e-3
NEAR_TIE = 1e-5       # relative margin under which a discrete decision is a near tie
NEAR_TIE_CAP = 1e-3   # near-tie mismatches allowed, as a fraction of cases (rounded up)


def say(*a):
    """Progress and result lines of the parity checks, shown as they happen (also under -q)."""
    line = " ".join(str(x) for x in a)
    conftest = sys.modules.get("conftest")
    if conftest is not None and hasattr(conftest, "progress"):
        conftest.progress(line)
    else:
        print(line, flush=True)


def problem_of(cfg: synth.Config):
    return make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.groups, cfg.dtype)


def to_dev(x, cfg, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype or (torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)).cuda()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_stats(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(x - ref)
    return float(d.max()) if d.size else 0.0, float(d.sum() / max(np.abs(ref).sum(), 1e-30))


def assert_close_attn(name, x, ref):
    ma, mr = err_stats(x, ref)
    say(f"  {name}: max_abs={ma:.3e} mean_rel={mr:.3e}")
    assert ma <= MAX_ABS and mr <= MEAN_REL, f"{name}: max_abs {ma:.3e}, mean_rel {mr:.3e}"


def cap(n):
    return math.ceil(NEAR_TIE_CAP * n)


def shape_near_ties(orc_stats, orc_shapes, tau128, tau256):
    rho = orc_stats["rho"]
    near_vol = np.minimum(np.abs(rho - tau128) / tau128, np.abs(rho - tau256) / max(tau256, 1e-30)) < NEAR_TIE
    dist = np.sort(orc_shapes["dist"], axis=-1)
    d1, d2 = dist[..., 0], dist[..., 1]
    near_shape = (d2 - d1) / np.maximum(d2, 1e-12) < NEAR_TIE
    return near_vol | near_shape


def compare_shapes(gpu_shape, orc_stats, orc_shapes, tau128, tau256):
    mism = gpu_shape != orc_shapes["shape_idx"]
    near = shape_near_ties(orc_stats, orc_shapes, tau128, tau256)
    hard = int((mism & ~near).sum())
    soft = int((mism & near).sum())
    return hard, soft, mism.size


REPORT: list[str] = []   # near-tie counts per check, printed in pytest's terminal summary


def report(line):
    say(line)
    REPORT.append(line)


def oracle_scores(qbar, kbar, sm_scale, h, i, nb):
    """The oracle's fp64 block scores of query block i of head h against the nb key blocks."""
    return sm_scale * (kbar[h, :nb] @ qbar[h, i])


def at_the_cut(sym, s, n_sel):
    """True when every block of the symmetric difference sym sits at the oracle's cut: its
    fp64 score within NEAR_TIE (relative) of the cut score s_(n_sel), or its rank in the
    oracle's order (score descending, index ascending) next to the cut."""
    order = np.lexsort((np.arange(len(s)), -s))
    rank = np.empty(len(s), np.int64)
    rank[order] = np.arange(len(s))
    s_cut = s[order[n_sel - 1]] if n_sel > 0 else s[order[0]]
    for b in sym:
        near_score = abs(s[b] - s_cut) <= NEAR_TIE * abs(s_cut)
        near_rank = n_sel - 1 <= rank[b] <= n_sel
        if not (near_score or near_rank):
            return False
    return True


def compare_masks(gcnt, gidx, ocnt, oidx, oinfo, nblocks, groups, rows_mask=None, qbar=None, kbar=None,
                  sm_scale=None):
    """Row-by-row set comparison of the selection; returns (hard, soft, rows).

    A differing row counts as a near tie (soft) only if the oracle's margin at one of its cuts
    is below NEAR_TIE and, when the oracle's pooled blocks are given, every block in which the
    two sets differ lies at that cut (at_the_cut); every other difference is hard."""
    heads, nbmax = ocnt.shape
    hpg = heads // groups
    hard = soft = rows = 0
    for h in range(heads):
        nb = int(nblocks[h // hpg])
        for i in range(nb):
            if rows_mask is not None and not rows_mask[h, i]:
                continue
            rows += 1
            a = gidx[h, i, : gcnt[h, i]]
            b = oidx[h, i, : ocnt[h, i]]
            if gcnt[h, i] == ocnt[h, i] and np.array_equal(a, b):
                continue
            inf = oinfo[h, i]
            ok = min(inf[3], inf[4]) < NEAR_TIE
            if ok and qbar is not None:
                sym = np.setxor1d(a, b)
                ok = at_the_cut(sym, oracle_scores(qbar, kbar, sm_scale, h, i, nb), int(ocnt[h, i]))
            if ok:
                soft += 1
                if soft <= 5:
                    say(f"  near-tie mismatch h={h} i={i}: gpu n={gcnt[h, i]} oracle n={ocnt[h, i]} "
                        f"margins score {inf[3]:.3e} cdf {inf[4]:.3e}")
            else:
                hard += 1
                if hard <= 5:
                    say(f"  mask mismatch h={h} i={i}: gpu n={gcnt[h, i]} oracle n={ocnt[h, i]} info={inf}")
    return hard, soft, rows


class Run:
    """One config: seeded inputs, the oracle's plan, and the GPU layer."""

    def __init__(self, cfg: synth.Config, backward=None, oracle_rows=None, nthreads=None):
        self.cfg = cfg
        self.backward = cfg.backward if backward is None else backward
        say(f"[{cfg.name}] grid {cfg.T}x{cfg.H}x{cfg.W} heads {cfg.heads} d {cfg.d} {cfg.dtype} seed {cfg.seed}")
        self.inp = synth.make_inputs(cfg, with_dout=self.backward)
        self.orc = oracle.forward_path(self.inp, groups=cfg.groups, row_mask=oracle_rows, nthreads=nthreads)
        self.pb = problem_of(cfg)
        self.layer = PrismLayer(self.pb, backward=self.backward)
        self.q = to_dev(self.inp["q"], cfg)
        self.k = to_dev(self.inp["k"], cfg)
        self.v = to_dev(self.inp["v"], cfg)
        self.a = torch.from_numpy(self.inp["a"]).cuda()
        self.dout = to_dev(self.inp["dout"], cfg) if self.backward else None

    def gpu_plan(self, with_audio=True):
        c = self.cfg
        self.layer.plan(self.v, self.a if with_audio else None, c.eps, c.tau128, c.tau256)
        torch.cuda.synchronize()

    def inject_oracle_plan(self):
        """Feed the oracle's shapes and block layout to the GPU layer (isolates later stages)."""
        L, o = self.layer, self.orc
        L.shape_idx.copy_(torch.from_numpy(o["shapes"]["shape_idx"]))
        L.zone_block_off.copy_(torch.from_numpy(o["shapes"]["zone_block_off"]))
        L.block_start.copy_(torch.from_numpy(o["block_start"]))

    def gpu_select(self):
        c = self.cfg
        self.layer.select(self.q, self.k, self.v, c.sm_scale, c.k_abs, c.k_frac, c.p)
        torch.cuda.synchronize()

    def inject_oracle_mask(self):
        L, o = self.layer, self.orc
        L.sel_count.copy_(torch.from_numpy(o["sel_count"]))
        L.sel_idx.copy_(torch.from_numpy(o["sel_idx"]))
