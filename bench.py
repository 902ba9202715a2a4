#!/usr/bin/env python
"""Benchmark of the Prism hot path on one MI355X.

One step = one layer's whole path, forward and backward, on the 2K-shaped token grid
32 x 96 x 160 (491,520 tokens, 960 zones), 4 heads, head_dim 128, bf16, k = 5 % of key
blocks, p = 0.9 (seeded synthetic inputs of that shape; see synth/):

  zone statistics -> volume/shape assignment -> permute Q,K,V -> pool Q,K -> select ->
  sparse attention forward (O written in token order) -> sparse attention backward (dO
  permuted into block order inside; dQ, dK, dV written in token order)

``--block-io`` runs the block-order calls instead, with separate unpermute O / permute dO /
unpermute gradient passes.

Printed: one JSON line.  ``value`` is ms per layer (whole step, lower is better).  Extra
fields give per-stage times, attention TFLOP/s on executed (selected-block, algorithmic)
FLOPs, the roofline of the dominant kernel (timed with HIP events recorded by the library
around that kernel's launches), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config 2k] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak (published)
MFMA_KERNELS = ("k_fwd", "k_dq", "k_dkdv")
HBM_KERNELS = ("k_zone_stats", "k_pool", "k_permute_pool")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "dynamic_block_sparse_var_amd", "csrc"))):
        with open(os.path.join(ROOT, "dynamic_block_sparse_var_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def selection_stats(layer, pb):
    """Executed query-key pairs from the GPU's own selection: sum over heads and query blocks
    of |B_i| * sum_{j in S_i} |B_j|; also the mean key-token fraction and the B histogram."""
    import torch

    N, nbmax = pb.N, pb.nbmax
    hpg = pb.heads // pb.groups
    pairs = 0
    frac = []
    for h in range(pb.heads):
        bs = layer.block_start[h // hpg].long()
        sizes = (bs[1:] - bs[:-1]).clamp(min=0)
        nb = int((bs[:-1] < N).sum())
        ext = torch.cat([sizes, sizes.new_zeros(1)])
        cnt = layer.sel_count[h, :nb].long()
        keytok = torch.zeros(nb, dtype=torch.int64, device=bs.device)
        for r0 in range(0, nb, 1024):
            r1 = min(nb, r0 + 1024)
            idx = layer.sel_idx[h, r0:r1, :].long()
            col = torch.arange(nbmax, device=bs.device)[None, :]
            idx = torch.where(col < cnt[r0:r1, None], idx, torch.full_like(idx, nbmax))
            keytok[r0:r1] = ext[idx].sum(1)
        pairs += int((sizes[:nb] * keytok).sum())
        frac.append(float((keytok.double() / N).mean()))
    vols = [64, 64, 64, 64, 64, 64, 64, 128, 128, 128, 128, 128, 128, 256, 256, 256]
    sh = layer.shape_idx.cpu().numpy().reshape(-1)
    hist = {64: 0, 128: 0, 256: 0}
    for s in sh:
        hist[vols[int(s)]] += 1
    nblocks = int((layer.block_start[0, :-1] < N).sum())
    return pairs, sum(frac) / len(frac), hist, nblocks


def forward_pair_tiles(layer, pb):
    """(pair, union tile) units of the forward, which runs one workgroup per pair of atoms of a
    zone and loads each tile of the union of the two lists once.  Pairs as the kernel forms them:
    in a zone of 128- or 256-row blocks, neighbouring atoms of one block (one shared list); in a
    zone of eight 64-row blocks, greedy matching by the number of blocks two lists share (largest
    first, the lexicographically first pair among equal counts).  Also returns the per-atom count
    (every atom loading its own tiles) for comparison."""
    import numpy as np
    import torch

    N = pb.N
    hpg = pb.heads // pb.groups
    union_units = 0
    atom_units = 0
    for h in range(pb.heads):
        bs = layer.block_start[h // hpg].long()
        nb = int((bs[:-1] < N).sum())
        sizes = bs[1:nb + 1] - bs[:nb]
        tiles = (sizes // 64).float()
        cnt = layer.sel_count[h, :nb].long()
        M = torch.zeros(nb, nb, dtype=torch.float32, device=bs.device)
        for r0 in range(0, nb, 1024):
            r1 = min(nb, r0 + 1024)
            idx = layer.sel_idx[h, r0:r1, :nb].long()
            valid = torch.arange(nb, device=bs.device)[None, :] < cnt[r0:r1, None]
            rows = torch.arange(r0, r1, device=bs.device)[:, None].expand_as(idx)
            M[rows[valid], idx[valid]] = 1.0
        ltiles = (M @ tiles).double()          # tiles in each query block's list
        atom_units += int(((sizes // 64).double() * ltiles).sum())
        j0 = torch.searchsorted(bs[:nb].contiguous(), torch.arange(0, N, 512, device=bs.device))
        small = sizes[j0] == 64
        # zones of 128/256-row blocks: B/128 pairs per block, each loading the block's list once
        big = sizes >= 128
        union_units += int(((sizes[big] // 128).double() * ltiles[big]).sum())
        zs = j0[small]
        if zs.numel() == 0:
            continue
        ids = zs[:, None] + torch.arange(8, device=bs.device)[None, :]
        M8 = M[ids]                                                   # [zones, 8, nb]
        M8t = M8.transpose(1, 2).contiguous()
        shared = torch.bmm(M8, M8t).cpu().numpy()                     # blocks both lists hold
        shared_t = torch.bmm(M8 * tiles[None, None, :], M8t).cpu().numpy()  # tiles both lists hold
        lt = ltiles[ids].cpu().numpy()
        for z in range(ids.shape[0]):
            used = 0
            for _ in range(4):
                best, ba, bc = -1.0, 0, 1
                for a in range(8):
                    for c in range(a + 1, 8):
                        if not (used >> a) & 1 and not (used >> c) & 1 and shared[z, a, c] > best:
                            best, ba, bc = shared[z, a, c], a, c
                used |= (1 << ba) | (1 << bc)
                union_units += int(round(lt[z, ba] + lt[z, bc] - shared_t[z, ba, bc]))
    return union_units, atom_units


def host_record():
    """nproc, the threads this process may use, and the CPU model name."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable_threads": usable, "cpu_model": model}


def cpu_baseline(inp, budget_s=20.0):
    """The oracle as it stands, on the same inputs: the planning half (stats, shapes, block
    layout, permute + pool of Q and K, full selection) timed in full; the attention's three
    passes timed on samples and extrapolated by the query-key pairs each pass visits:
    the forward on sampled query blocks, the backward's row statistics + dQ on the same
    blocks, and its row statistics + dK/dV on sampled key blocks (chosen among those few query
    blocks select, so that their row statistics stay cheap).  The oracle reports the wall time
    of each of its backward passes, so every pass is timed on its own."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    nth = oracle.default_threads()
    cfg = inp["cfg"]
    t0 = time.perf_counter()
    orc = oracle.forward_path(inp, nthreads=nth)
    t_plan = time.perf_counter() - t0
    vp = oracle.permute(inp["v"], orc["pos"], cfg.heads)
    dop = oracle.permute(inp["dout"], orc["pos"], cfg.heads)
    bs, nb = orc["block_start"][0], int(orc["nblocks"][0])
    sizes = np.diff(bs)[:nb].astype(np.int64)
    rowpairs = np.zeros((cfg.heads, nb), np.int64)
    colpairs = np.zeros((cfg.heads, nb), np.int64)      # pairs the dK/dV pass visits per key block
    selectors = [[[] for _ in range(nb)] for _ in range(cfg.heads)]
    for h in range(cfg.heads):
        for i in range(nb):
            lst = orc["sel_idx"][h, i, :orc["sel_count"][h, i]]
            rowpairs[h, i] = sizes[i] * sizes[lst].sum()
            colpairs[h, lst] += sizes[i] * sizes[lst]
            for j in lst:
                selectors[h][j].append(i)
    total = int(rowpairs.sum())
    rng = np.random.default_rng(0)
    nq = max(1, nth // cfg.heads)
    args = (orc["qp"], orc["kp"], vp, dop, orc["block_start"], orc["nblocks"], 1, orc["sel_count"], orc["sel_idx"],
            cfg.sm_scale)
    zero = np.zeros((cfg.heads, cfg.nbmax), np.uint8)
    t_fwd = t_rs = t_dq = t_dkdv = 0.0
    pq = pk = prs = 0
    rq = rk = 0
    spent = 0.0
    # query blocks: forward, then row statistics + dQ
    while spent < 0.6 * budget_s and rq < 64:
        mask = zero.copy()
        for h in range(cfg.heads):
            mask[h, rng.choice(nb, size=min(nq, nb), replace=False)] = 1
        pq += int(rowpairs[mask[:, :nb].astype(bool)].sum())
        a = time.perf_counter()
        oracle.attn_fwd(*args[:3], *args[4:], qblock_mask=mask, nthreads=nth)
        b = time.perf_counter()
        oracle.attn_bwd(*args, qblock_mask=mask, kblock_mask=zero, nthreads=nth)
        c = time.perf_counter()
        ph = oracle.last_bwd_phase_seconds()
        t_fwd += b - a
        t_rs += ph[0]
        t_dq += ph[1]
        spent += c - a
        rq += 1
    # key blocks: row statistics of their selectors + dK/dV
    few = [np.flatnonzero((np.array([len(x) for x in selectors[h]]) > 0)
                          & (np.array([len(x) for x in selectors[h]]) <= 24)) for h in range(cfg.heads)]
    while spent < budget_s and rk < 64:
        kmask = zero.copy()
        need = np.zeros((cfg.heads, nb), bool)
        for h in range(cfg.heads):
            pool = few[h] if len(few[h]) else np.flatnonzero(colpairs[h] > 0)
            for j in rng.choice(pool, size=min(nq, len(pool)), replace=False):
                kmask[h, j] = 1
                pk += int(colpairs[h, j])
                need[h, selectors[h][j]] = True
        prs += int(rowpairs[need].sum())
        a = time.perf_counter()
        oracle.attn_bwd(*args, qblock_mask=zero, kblock_mask=kmask, nthreads=nth)
        ph = oracle.last_bwd_phase_seconds()
        t_rs += ph[0]
        t_dkdv += ph[2]
        spent += time.perf_counter() - a
        rk += 1
    fwd_pp = t_fwd / max(pq, 1)
    rs_pp = t_rs / max(pq + prs, 1)
    dq_pp = t_dq / max(pq, 1)
    dkdv_pp = t_dkdv / max(pk, 1)
    # forward + backward (row statistics, dQ, dK/dV) over every pair
    est_ms = (t_plan + total * (fwd_pp + rs_pp + dq_pp + dkdv_pp)) * 1e3
    sample = (f"planning (stats, shapes, layout, permute+pool Q/K, full selection) timed in full "
              f"({t_plan:.1f} s); forward and row-stat+dQ passes timed on {rq} x {nq} query blocks per head "
              f"({pq:,} pairs), row-stat+dK/dV pass on {rk} x {nq} key blocks per head ({pk:,} dK/dV pairs, "
              f"{prs:,} row-stat pairs), {spent:.1f} s in all; per-pair rates (ns): forward {fwd_pp * 1e9:.2f}, "
              f"row statistics {rs_pp * 1e9:.2f}, dQ {dq_pp * 1e9:.2f}, dK/dV {dkdv_pp * 1e9:.2f}; extrapolated to all {total:,} pairs")
    return {"value": round(est_ms, 1), "unit": "ms/layer", "cores": nth, "kind": "oracle", "sample": sample,
            **host_record()}


def write_traffic(d, probe_mb, config, out_path=None):
    """HBM bytes per dispatch from two rocprofv3 --pmc runs.  The counters are scaled by what
    they read for the known-size device copy (probe_mb MiB read and written) in the same run.
    Written to out_path (default profiles/traffic.json)."""
    import csv
    import glob

    def load(cnt):
        fs = glob.glob(os.path.join(d, cnt, "**", "*counter_collection.csv"), recursive=True)
        if len(fs) != 1:
            raise SystemExit(f"expected one counter CSV under {d}/{cnt}, found {fs}")
        out = []
        with open(fs[0]) as f:
            for r in csv.DictReader(f):
                out.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]) * 1024.0))
        return out

    fetch, write = load("FETCH_SIZE"), load("WRITE_SIZE")
    probe = probe_mb << 20

    def scale(rows):
        big = max((b for n, _, b in rows if "copyBuffer" in n), default=0.0)
        if big <= 0:
            raise SystemExit("no device-copy dispatch found to calibrate the counter")
        return probe / big

    fs, ws = scale(fetch), scale(write)
    res = {}
    for (nf, gf, bf), (nw, gw, bw) in zip(fetch, write):
        if nf != nw or gf != gw:
            raise SystemExit("FETCH_SIZE and WRITE_SIZE runs dispatched different kernels")
        if "copyBuffer" in nf:
            continue
        m = re.search(r"::(k_\w+)", nf)
        base = m.group(1) if m else nf
        e = res.setdefault(base, {"per_dispatch": []})
        e["per_dispatch"].append({"grid": gf, "read": round(bf * fs), "write": round(bw * ws)})
    for e in res.values():
        pdl = e["per_dispatch"]
        e["bytes_per_launch"] = round(sum(x["read"] + x["write"] for x in pdl) / len(pdl))
        e["source_sha"] = kernel_source_sha()
        e["config"] = config
    meta = {"fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "probe_bytes": probe,
            "note": "bytes = counter KiB x 1024 x scale; scale = probe bytes / counter bytes of the probe copy"}
    out = {"_calibration": meta, **res}
    with open(out_path or os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps({k: v.get("bytes_per_launch") for k, v in res.items()}))


# Matrix-core FLOPs each attention kernel issues per query-key pair, in units of d: the
# forward's S and its split PV (3 products of 2d FLOP), the dQ kernel's recomputed S and dP
# plus its split dQ (4), the dK/dV kernel's S, dP, split dV and split dK (6).
ISSUED_PER_PAIR = {"k_fwd": 6.0, "k_dq": 8.0, "k_dkdv": 12.0}
# Algorithmic FLOPs per pair (the convention F_fwd = 4d per pair, F_bwd = 2.5 F_fwd with the
# recomputed S among the five backward products): the forward's QK^T and PV; the dK/dV kernel's
# S, dP, dV and dK; the dQ kernel's dQ product (its S and dP repeat the dK/dV kernel's).
ALG_PER_PAIR = {"k_fwd": 4.0, "k_dq": 2.0, "k_dkdv": 8.0}


def make_step(P, pb, L, cfg, q, k, v, a, do, block_io, fixed, k_abs, k_frac):
    """One layer, forward + backward, as a function of an optional list of events to mark the
    stage boundaries with; returns the stage names."""
    sm = cfg.sm_scale
    pb32 = P.Problem(pb.T, pb.H, pb.W, pb.heads, pb.head_dim, pb.groups, P.F32)
    if block_io:
        stages = ["zone_stats", "assign_shapes", "permute_qkv", "pool", "select", "bsa_fwd", "unpermute_o",
                  "permute_do", "bsa_bwd", "unpermute_grads"]
    else:
        stages = ["zone_stats", "assign_shapes", "permute_pool", "select", "bsa_fwd", "bsa_bwd"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        if fixed is None:
            P.prism_zone_stats(pb, v, a, cfg.eps, L.g, L.rho, L.zone_audio)
            mark(1)
            P.prism_assign_shapes(pb, L.g, L.rho, cfg.tau128, cfg.tau256, L.shape_idx, L.zone_block_off,
                                  L.block_start)
        else:  # fixed-block ablation: a1 and a2 replaced by one shape for every zone
            mark(1)
            P.prism_fixed_shapes(pb, fixed, L.shape_idx, L.zone_block_off, L.block_start)
        mark(2)
        if not block_io:
            # permute Q, K, V and pool Q, K in one pass; attention outputs straight to token order
            P.prism_permute_pool(pb, L.shape_idx, L.zone_block_off, [q, k, v], [L.qp, L.kp, L.vp],
                                 [L.qbar, L.kbar, None])
            mark(3)
            P.prism_select_blocks(pb, L.block_start, L.qbar, L.kbar, sm, k_abs, k_frac, cfg.p, L.sel_count,
                                  L.sel_idx)
            mark(4)
            P.prism_bsa_fwd_tok(pb, L.shape_idx, L.block_start, L.sel_count, L.sel_idx, sm, L.qp, L.kp, L.vp, L.o,
                                L.o_lo, L.lse, L.fwd_workspace)
            mark(5)
            P.prism_bsa_bwd_tok(pb, L.shape_idx, L.block_start, L.sel_count, L.sel_idx, sm, L.qp, L.kp, L.vp, L.o,
                                L.o_lo, do, L.lse, L.dq, L.dk, L.dv, L.workspace)
            mark(6)
            return
        P.prism_permute(pb, L.shape_idx, 0, [q, k, v], [L.qp, L.kp, L.vp])
        mark(3)
        P.prism_pool_blocks(pb, L.block_start, [L.qp, L.kp], [L.qbar, L.kbar])
        mark(4)
        P.prism_select_blocks(pb, L.block_start, L.qbar, L.kbar, sm, k_abs, k_frac, cfg.p, L.sel_count,
                              L.sel_idx)
        mark(5)
        P.prism_bsa_fwd(pb, L.block_start, L.sel_count, L.sel_idx, sm, L.qp, L.kp, L.vp, L.op, L.op_lo, L.lse,
                        L.fwd_workspace)
        mark(6)
        P.prism_permute(pb, L.shape_idx, 1, [L.op], [L.o])
        mark(7)
        P.prism_permute(pb, L.shape_idx, 0, [do], [L.dop])
        mark(8)
        P.prism_bsa_bwd(pb, L.block_start, L.sel_count, L.sel_idx, sm, L.qp, L.kp, L.vp, L.op, L.op_lo, L.dop, L.lse,
                        L.dqp, L.dkp, L.dvp, L.workspace)
        mark(9)
        P.prism_permute(pb32, L.shape_idx, 1, [L.dqp, L.dkp, L.dvp], [L.dq, L.dk, L.dv])
        mark(10)

    return step, stages


def measure(cfg, steps, warmup, block_io=False, dense=False, fixed_shape=False, detail=True, inp=None,
            copy_probe_mb=0):
    """Time `steps` whole layers (after `warmup`) of one configuration.  Returns a dict of the
    measurements and, for the caller's CPU baseline, the inputs."""
    import torch

    import dynamic_block_sparse_var_amd as P
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if inp is None:
        log(f"bench: config {cfg.name} grid {cfg.T}x{cfg.H}x{cfg.W} heads {cfg.heads} d {cfg.d}; generating inputs")
        inp = synth.make_inputs(cfg, with_dout=True)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(inp["q"]).to(dt).to(dev)
    k = torch.from_numpy(inp["k"]).to(dt).to(dev)
    v = torch.from_numpy(inp["v"]).to(dt).to(dev)
    do = torch.from_numpy(inp["dout"]).to(dt).to(dev)
    a = torch.from_numpy(inp["a"]).to(dev)
    pb = P.make_problem(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d, cfg.groups, cfg.dtype)
    L = P.PrismLayer(pb, device=dev, backward=True, token_io=not block_io)
    fixed = P.fixed_shape_index((4, 4, 4)) if fixed_shape else None
    # dense baseline: every key block selected (k = N_b), the same kernels otherwise
    k_abs, k_frac = (pb.nbmax, 0.0) if dense else (cfg.k_abs, cfg.k_frac)
    step, stages = make_step(P, pb, L, cfg, q, k, v, a, do, block_io, fixed, k_abs, k_frac)

    if copy_probe_mb > 0:
        src = torch.ones(copy_probe_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"bench: {cfg.name}: warmup")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # per-kernel events recorded by the library around its own launches
    kev = {kn: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)] for kn in MFMA_KERNELS + HBM_KERNELS}
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for st in range(steps):  # make every event a live HIP event before timing
        for kn in kev:
            for e in kev[kn][st]:
                e.record()
        for e in sev[st]:
            e.record()
    torch.cuda.synchronize()
    log(f"bench: {cfg.name}: timing {steps} steps")
    t_wall = time.perf_counter()
    t_start.record()
    for st in range(steps):
        for kn in kev:
            P.prism_trace_kernel(kn, *kev[kn][st])
        step(sev[st])
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    P.prism_trace_kernel(None)
    ms_step = t_start.elapsed_time(t_stop) / steps

    stage_ms = {s_: sum(sev[st][i].elapsed_time(sev[st][i + 1]) for st in range(steps)) / steps
                for i, s_ in enumerate(stages)}
    kern_ms = {kn: sum(a_.elapsed_time(b_) for a_, b_ in kev[kn]) / steps for kn in kev}

    pairs, key_frac, hist, nblocks = selection_stats(L, pb)
    d = cfg.d
    attn_ms = stage_ms["bsa_fwd"] + stage_ms["bsa_bwd"]
    f_attn = 14.0 * d * pairs          # F_fwd + F_bwd = 4d + 10d per pair
    res = {"cfg": cfg, "inp": inp, "L": L, "pb": pb, "dev_tensors": (q, k, v, a), "ms_step": ms_step,
           "wall": wall, "stage_ms": stage_ms, "kern_ms": kern_ms, "pairs": pairs, "key_frac": key_frac, "hist": hist, "nblocks": nblocks,
           "attn_ms": attn_ms, "attn_tflops": f_attn / (attn_ms * 1e-3) / 1e12}
    if detail and cfg.dtype == "bf16":
        res["fwd_units"], res["atom_units"] = forward_pair_tiles(L, pb)
    return res


def summary(res):
    """The compact per-configuration record of the `configs` object."""
    cfg, km = res["cfg"], res["kern_ms"]
    d, pairs = cfg.d, res["pairs"]
    out = {"workload": f"{cfg.T}x{cfg.H}x{cfg.W} tokens, {cfg.heads} heads, d {cfg.d}, {cfg.dtype}",
           "ms_per_layer": round(res["ms_step"], 3),
           "attn_fwd_bwd_ms": round(res["attn_ms"], 3),
           "attn_tflops": round(res["attn_tflops"], 1),
           "attn_mfma_frac": round(res["attn_tflops"] / PEAK_BF16_TFLOPS, 4),
           "stage_ms": {s_: round(x, 4) for s_, x in res["stage_ms"].items()},
           "selection": {"executed_pairs": pairs, "mean_key_fraction": round(res["key_frac"], 4),
                         "n_blocks": res["nblocks"]}}
    if cfg.dtype == "bf16":
        out["kernel_ms"] = {kn: round(km[kn], 3) for kn in MFMA_KERNELS}
        dom = max(MFMA_KERNELS, key=lambda kn: km[kn])
        tf = ALG_PER_PAIR[dom] * d * pairs / (km[dom] * 1e-3) / 1e12
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="2k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the named configuration (no `configs` object of the other workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a known-size reference "
                         "for hardware byte counters)")
    ap.add_argument("--block-io", action="store_true",
                    help="block-order attention calls with separate permutes of O, dO and the gradients")
    ap.add_argument("--dense", action="store_true",
                    help="dense baseline: every key block selected (k = N_b) on the same kernels")
    ap.add_argument("--fixed-shape", action="store_true",
                    help="fixed-block ablation: 4x4x4 blocks in every zone, zone statistics and shape "
                         "assignment skipped")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="no GPU work: read rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs under DIR/FETCH_SIZE and "
                         "DIR/WRITE_SIZE (taken with --copy-probe-mb on this source tree) and write "
                         "profiles/traffic.json")
    args = ap.parse_args()
    if args.dense and args.fixed_shape:
        ap.error("--dense and --fixed-shape are separate variants")
    if args.traffic_from:
        write_traffic(args.traffic_from, args.copy_probe_mb or 4096, args.config)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is built and measured on one "
              f"GPU; sharding it by head group over several GPUs is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_block_sparse_var_amd as P
    import synth

    cfg = synth.CONFIGS[args.config]
    res = measure(cfg, args.steps, args.warmup, block_io=args.block_io, dense=args.dense,
                  fixed_shape=args.fixed_shape, copy_probe_mb=args.copy_probe_mb)
    L, pb, inp = res["L"], res["pb"], res["inp"]
    q_dev, k_dev, v_dev, a_dev = res.pop("dev_tensors")
    stage_ms, kern_ms, pairs = res["stage_ms"], res["kern_ms"], res["pairs"]
    dev = torch.device("cuda:0")
    d = cfg.d
    attn_ms = res["attn_ms"]
    attn_tflops = res["attn_tflops"]
    attn_issued_tflops = sum(ISSUED_PER_PAIR.values()) * d * pairs / (attn_ms * 1e-3) / 1e12
    N, H_ = cfg.N, cfg.heads
    ebytes = 2 if cfg.dtype == "bf16" else 4
    kbytes = {
        "k_zone_stats": N * H_ * d * ebytes + 4 * N,
        "k_pool": 2 * N * H_ * d * ebytes + 2 * H_ * pb.nbmax * d * 4,
    }
    # Memory side of the attention kernels (a property of this dataflow, not of the method):
    # the selected-tile stream.  For every (64-row atom, 64-row tile of a block the atom attends
    # to) unit a kernel reads the two bf16 tiles of the other side (K and V; for dK/dV: Q and dO
    # plus their lse2/delta rows); the forward runs per pair of atoms and loads each tile of the
    # union of the pair's lists once.  unique_io is what each kernel must read and write at
    # least once: its input tensors and its outputs.
    units = pairs // 4096
    atoms = H_ * (N // 64)
    tile = 2 * 64 * d * ebytes
    fwd_units, atom_units = res.get("fwd_units", units), res.get("atom_units", units)
    kalg = {
        "k_fwd": fwd_units * tile + atoms * (3 * 64 * d * ebytes + 64 * 4),
        "k_dq": units * tile + atoms * (2 * 64 * d * ebytes + 64 * d * 4 + 2 * 64 * 4),
        "k_dkdv": units * (tile + 2 * 64 * 4) + atoms * (2 * 64 * d * ebytes + 2 * 64 * d * 4),
    }
    row = N * H_ * d
    unique_io = {
        "k_fwd": 3 * row * ebytes + 2 * row * ebytes + 4 * N * H_,           # Q, K, V; O and its residual; LSE
        "k_dq": 4 * row * ebytes + 2 * 4 * N * H_ + 4 * row,                 # Q, K, V, dO; lse2, delta; dQ fp32
        "k_dkdv": 4 * row * ebytes + 2 * 4 * N * H_ + 2 * 4 * row,           # ...; dK, dV fp32
    }
    traffic = {}
    tr_path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tr_path):
        with open(tr_path) as f:
            tr = json.load(f)
        sha = kernel_source_sha()
        for kn, ent in tr.items():
            if (isinstance(ent, dict) and ent.get("source_sha") == sha and ent.get("config") == cfg.name
                    and not (args.dense or args.fixed_shape)):
                traffic[kn] = ent["bytes_per_launch"]
    attn_k = {}
    for kn in MFMA_KERNELS:
        sec = kern_ms[kn] * 1e-3
        fl = ALG_PER_PAIR[kn] * d * pairs
        attn_k[kn] = {"ms": round(kern_ms[kn], 3),
                      "TFLOP/s": round(fl / sec / 1e12, 1),
                      "mfma_frac": round(fl / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "issued_TFLOP/s": round(ISSUED_PER_PAIR[kn] * d * pairs / sec / 1e12, 1),
                      "unique_io_GB": round(unique_io[kn] / 1e9, 3),
                      "tile_stream_GB": round(kalg[kn] / 1e9, 2),
                      "tile_stream_GB/s": round(kalg[kn] / sec / 1e9, 1),
                      "tile_stream_over_unique_io": round(kalg[kn] / unique_io[kn], 1),
                      "measured_traffic_GB": round(traffic[kn] / 1e9, 2) if kn in traffic else None,
                      "measured_traffic_over_unique_io": (round(traffic[kn] / unique_io[kn], 1)
                                                          if kn in traffic else None)}
    # the forward's stream if every atom loaded its own tiles (the dQ walk), for comparison
    attn_k["k_fwd"]["per_atom_stream_GB"] = round((atom_units * tile + (kalg["k_fwd"] - fwd_units * tile)) / 1e9, 2)
    # Roofline: the attention kernels are matrix-core work; achieved = the dominant kernel's
    # algorithmic FLOPs per launch (its share of F_fwd + F_bwd) over its mean launch time
    dom = max(MFMA_KERNELS, key=lambda kn: kern_ms[kn])
    roof = {"kernel": dom, "bound": "mfma", "achieved": attn_k[dom]["TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": attn_k[dom]["mfma_frac"], "traffic": traffic.get(dom),
            "flop_per_launch": ALG_PER_PAIR[dom] * d * pairs,
            "attention": {"ms": round(attn_ms, 3), "flop": 14.0 * d * pairs, "TFLOP/s": round(attn_tflops, 1),
                          "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4)}}
    if args.block_io:
        # permute of Q, K, V is one launch of k_permute: time it with the stage events around it
        kbytes["k_permute"] = 3 * 2 * N * H_ * d * ebytes
        kern_ms["k_permute"] = stage_ms["permute_qkv"]
        hbm_names = ("k_zone_stats", "k_permute", "k_pool")
    else:
        # Q, K, V read and written once, pooled Q and K written
        kbytes["k_permute_pool"] = 3 * 2 * N * H_ * d * ebytes + 2 * H_ * pb.nbmax * d * 4
        hbm_names = ("k_zone_stats", "k_permute_pool")
    hbm = {kn: {"ms": round(kern_ms[kn], 4), "GB/s": round(kbytes[kn] / (kern_ms[kn] * 1e-3) / 1e9, 1),
                "frac": round(kbytes[kn] / (kern_ms[kn] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
           for kn in hbm_names}
    # the whole statistics stage (every launch of prism_zone_stats) against its bytes
    hbm["zone_stats_stage"] = {"ms": round(stage_ms["zone_stats"], 4),
                               "GB/s": round(kbytes["k_zone_stats"] / (stage_ms["zone_stats"] * 1e-3) / 1e9, 1),
                               "frac": round(kbytes["k_zone_stats"] / (stage_ms["zone_stats"] * 1e-3) / 1e9
                                             / PEAK_HBM_GBS, 4)}

    out = {
        "metric": "2K-shaped sparse-attn fwd+bwd ms/layer, TFLOP/s and % bf16 MFMA peak",
        "value": round(res["ms_step"], 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_step"], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded generator; 2K-shaped token grid)",
        "config": {"workload": f"{cfg.name}: {cfg.T}x{cfg.H}x{cfg.W} tokens, {cfg.heads} heads, d {cfg.d}, "
                               + ("dense (every key block), " if args.dense else
                                  f"k {cfg.k_frac:.0%} p {cfg.p}, ")
                               + ("fixed 4x4x4 blocks, " if args.fixed_shape else "")
                               + "forward + backward",
                   "io": "block order + permutes" if args.block_io else "token order",
                   "parallelism": "none (1 GPU)"},
        "attn_fwd_bwd_ms": round(attn_ms, 3),
        "attn_tflops": round(attn_tflops, 1),
        "attn_mfma_frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "attn_issued_mfma": ({"TFLOP/s": round(attn_issued_tflops, 1),
                              "frac": round(attn_issued_tflops / PEAK_BF16_TFLOPS, 4),
                              "issued_over_algorithmic": round(sum(ISSUED_PER_PAIR.values()) / 14.0, 3),
                              "note": "matrix-core FLOPs issued (split P / dS products and the dQ kernel's "
                                      "recomputed S and dP included); not the algorithmic rate"}
                             if cfg.dtype == "bf16" else None),
        "stage_ms": {s_: round(x, 4) for s_, x in stage_ms.items()},
        "kernel_ms": {kn: round(kern_ms[kn], 4) for kn in MFMA_KERNELS},
        "attn_kernels": attn_k,
        "hbm_stages": hbm,
        "selection": {"executed_pairs": pairs, "mean_key_fraction": round(res["key_frac"], 4),
                      "n_blocks": res["nblocks"], "zones_by_volume": {str(kk): vv for kk, vv in res["hist"].items()}},
        "wall_s_timed": round(res["wall"], 3),
        "roofline": roof,
        "cpu_baseline": None,
    }
    # the HBM-bound stages again with the 256 MB Infinity Cache evicted before every repetition,
    # each timed alone: kernel (library events) and stage (call).  The eviction reads 1 GiB (a
    # write would leave the cache full of dirty lines, whose write-back the timed kernel pays for)
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    calls = {"zone_stats": ("k_zone_stats", lambda: P.prism_zone_stats(pb, v_dev, a_dev, cfg.eps, L.g, L.rho,
                                                                       L.zone_audio))}
    if args.block_io:
        calls["permute_qkv"] = ("k_permute", lambda: P.prism_permute(pb, L.shape_idx, 0, [q_dev, k_dev, v_dev],
                                                                     [L.qp, L.kp, L.vp]))
        calls["pool"] = ("k_pool", lambda: P.prism_pool_blocks(pb, L.block_start, [L.qp, L.kp],
                                                               [L.qbar, L.kbar]))
    else:
        calls["permute_pool"] = ("k_permute_pool", lambda: P.prism_permute_pool(
            pb, L.shape_idx, L.zone_block_off, [q_dev, k_dev, v_dev], [L.qp, L.kp, L.vp],
            [L.qbar, L.kbar, None]))
    cold = {}
    for st_name, (kn, fn) in calls.items():
        ks, ss = [], []
        for r in range(7):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            for e in evs:
                e.record()
            flush.sum()
            P.prism_trace_kernel(kn, evs[2], evs[3])
            evs[0].record()
            fn()
            evs[1].record()
            torch.cuda.synchronize()
            P.prism_trace_kernel(None)
            ss.append(evs[0].elapsed_time(evs[1]))
            ks.append(evs[2].elapsed_time(evs[3]))
        km_, sm_ = sorted(ks)[len(ks) // 2], sorted(ss)[len(ss) // 2]
        nbytes = kbytes[kn]
        cold[st_name] = {"kernel_ms": round(km_, 4), "stage_ms": round(sm_, 4),
                         "kernel_frac": round(nbytes / (km_ * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         "stage_frac": round(nbytes / (sm_ * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del flush
    out["hbm_stages_cold"] = {"note": "median of 7 repetitions, a 1 GiB read before each (evicts the "
                                      "256 MB Infinity Cache)", **cold}
    # auxiliary, not part of the step: the audio-norm producer (the next layer's coupling input)
    # on a cross-attention output of this GPU's heads x d channels, device-generated
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    hh = torch.randn(N, H_ * d, dtype=dt, device=dev, generator=gen)
    an = torch.empty(N, dtype=torch.float32, device=dev)
    for _ in range(2):
        P.prism_audio_norms(pb, hh, an)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        P.prism_audio_norms(pb, hh, an)
    e1.record()
    torch.cuda.synchronize()
    an_ms = e0.elapsed_time(e1) / 10
    an_bytes = N * H_ * d * ebytes + 4 * N
    out["aux_stages"] = {"audio_norms": {"ms": round(an_ms, 4), "channels": H_ * d,
                                         "GB/s": round(an_bytes / (an_ms * 1e-3) / 1e9, 1),
                                         "frac": round(an_bytes / (an_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del hh, an, L, q_dev, k_dev, v_dev, a_dev
    res.pop("L")
    torch.cuda.empty_cache()
    # the other workloads, each timed the same way with fewer steps (one line, one run)
    if not args.no_configs and args.config == "2k" and not (args.dense or args.fixed_shape or args.block_io):
        cfgs = {}
        for name, steps, warm, kw, reuse in (("720p", 3, 1, {}, False), ("1080p", 3, 1, {}, False),
                                             ("2k_stress", 2, 1, {}, False),
                                             ("2k_dense", 1, 1, {"dense": True}, True),
                                             ("2k_fixed_shape", 3, 1, {"fixed_shape": True}, True),
                                             ("1m", 1, 1, {}, False), ("tiny", 3, 1, {}, False)):
            c2 = cfg if reuse else synth.CONFIGS[name]
            r2 = measure(c2, steps, warm, detail=False, inp=inp if reuse else None, **kw)
            r2.pop("L")
            r2.pop("dev_tensors")
            sm2 = summary(r2)
            sm2["steps"] = steps
            if name == "tiny":
                sm2["note"] = "fp32 correctness path (one thread per row), not tuned"
            cfgs[name] = sm2
            del r2
            torch.cuda.empty_cache()
        out["configs"] = cfgs
    if not args.no_cpu_baseline and not (args.dense or args.fixed_shape):
        log("bench: CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(inp, budget_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
