"""Host logic of bench.py (no GPU): the one-GPU guard, the counter-to-bytes conversion behind
roofline.traffic, the FLOP conventions, the per-configuration roofline arithmetic and the
executed query-key pair count every FLOP figure is built on."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_flop_conventions():
    # algorithmic: F_fwd = 4d per executed pair, F_bwd = 2.5 F_fwd (five products counted once)
    assert bench.ALG_PER_PAIR["k_fwd"] == 4.0
    assert bench.ALG_PER_PAIR["k_dq"] + bench.ALG_PER_PAIR["k_dkdv"] == 2.5 * 4.0
    # issued: forward S + split PV (3 x 2d), dQ recomputed S, dP + split dQ (4 x 2d), dK/dV S, dP,
    # split dV, split dK (6 x 2d)
    assert sum(bench.ISSUED_PER_PAIR.values()) == 2.0 * (3 + 4 + 6)


def _write_counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, grid, cnt, kib in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": cnt, "Counter_Value": kib})


def test_traffic_conversion(tmp_path):
    probe_mb = 4
    probe = probe_mb << 20
    copy = "__amd_rocclr_copyBuffer"
    fwd = "void prism::(anonymous namespace)::k_fwd<128>(unsigned short const*)"
    dq = "void prism::(anonymous namespace)::k_dq<128>(unsigned short const*)"
    # FETCH_SIZE reads the copy as half its bytes (64 B counted per 128 B request): scale 2;
    # WRITE_SIZE reads it whole: scale 1.  Values are KiB per dispatch.
    fetch = [(copy, 1024, "FETCH_SIZE", probe / 2 / 1024), (fwd, 64, "FETCH_SIZE", 100.0),
             (fwd, 64, "FETCH_SIZE", 300.0), (dq, 32, "FETCH_SIZE", 50.0)]
    write = [(copy, 1024, "WRITE_SIZE", probe / 1024), (fwd, 64, "WRITE_SIZE", 10.0),
             (fwd, 64, "WRITE_SIZE", 30.0), (dq, 32, "WRITE_SIZE", 5.0)]
    _write_counter_csv(str(tmp_path / "FETCH_SIZE" / "r" / "t_counter_collection.csv"), fetch)
    _write_counter_csv(str(tmp_path / "WRITE_SIZE" / "r" / "t_counter_collection.csv"), write)
    out = tmp_path / "traffic.json"
    bench.write_traffic(str(tmp_path), probe_mb, "2k", out_path=str(out))
    t = json.loads(out.read_text())
    assert t["_calibration"]["fetch_scale"] == 2.0 and t["_calibration"]["write_scale"] == 1.0
    assert "__amd_rocclr_copyBuffer" not in t
    # k_fwd: mean over its two dispatches of (2 x fetch + write) KiB
    assert t["k_fwd"]["bytes_per_launch"] == round(((2 * 100 + 10) + (2 * 300 + 30)) * 1024 / 2)
    assert len(t["k_fwd"]["per_dispatch"]) == 2
    assert t["k_dq"]["bytes_per_launch"] == (2 * 50 + 5) * 1024
    assert t["k_dq"]["source_sha"] == bench.kernel_source_sha() and t["k_dq"]["config"] == "2k"


def test_traffic_conversion_needs_the_copy(tmp_path):
    fwd = "void prism::(anonymous namespace)::k_fwd<128>(unsigned short const*)"
    _write_counter_csv(str(tmp_path / "FETCH_SIZE" / "t_counter_collection.csv"), [(fwd, 64, "FETCH_SIZE", 1.0)])
    _write_counter_csv(str(tmp_path / "WRITE_SIZE" / "t_counter_collection.csv"), [(fwd, 64, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic(str(tmp_path), 4, "2k", out_path=str(tmp_path / "t.json"))


def test_summary_roofline_arithmetic():
    cfg = synth.CONFIGS["2k"]
    pairs = 58_322_317_312
    res = {"cfg": cfg, "kern_ms": {"k_fwd": 46.0, "k_dq": 56.0, "k_dkdv": 76.0}, "pairs": pairs,
           "ms_step": 181.0, "attn_ms": 178.0, "attn_tflops": 14.0 * 128 * pairs / 0.178 / 1e12,
           "stage_ms": {"bsa_fwd": 46.0, "bsa_bwd": 132.0}, "key_frac": 0.0607, "nblocks": 7124}
    s = bench.summary(res)
    assert s["roofline"]["kernel"] == "k_dkdv"
    want = 8.0 * 128 * pairs / 0.076 / 1e12
    assert s["roofline"]["achieved"] == round(want, 1)
    assert s["roofline"]["frac"] == round(want / bench.PEAK_BF16_TFLOPS, 4)
    assert s["attn_mfma_frac"] == round(res["attn_tflops"] / bench.PEAK_BF16_TFLOPS, 4)


def test_executed_pairs_by_brute_force():
    """selection_stats against a direct count over token pairs on a hand-built two-zone layout:
    every (query token, key token) pair whose key block is in the query block's list."""
    import types

    import numpy as np
    import torch

    N = 1024
    sizes = [64] * 8 + [256, 256]          # zone 0: eight 64-row blocks; zone 1: two 256-row blocks
    nb, nbmax = len(sizes), 8 * (N // 512)
    bs = torch.full((1, nbmax + 1), N, dtype=torch.int32)
    bs[0, 0] = 0
    bs[0, 1:nb + 1] = torch.tensor(sizes, dtype=torch.int32).cumsum(0)
    rng = np.random.default_rng(3)
    heads = 2
    cnt = torch.zeros(heads, nbmax, dtype=torch.int32)
    idx = torch.zeros(heads, nbmax, nbmax, dtype=torch.int32)
    lists = {}
    for h in range(heads):
        for i in range(nb):
            l = sorted(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False).tolist())
            lists[h, i] = l
            cnt[h, i] = len(l)
            idx[h, i, :len(l)] = torch.tensor(l, dtype=torch.int32)
            idx[h, i, len(l):] = 5                # stale entries past the count must be ignored
    shape_idx = torch.tensor([[3, 13]], dtype=torch.uint8)  # a 64-row shape and a 256-row shape
    layer = types.SimpleNamespace(block_start=bs, sel_count=cnt, sel_idx=idx, shape_idx=shape_idx)
    pb = types.SimpleNamespace(N=N, heads=heads, groups=1, nbmax=nbmax)
    pairs, key_frac, hist, nblocks = bench.selection_stats(layer, pb)

    block_of = np.repeat(np.arange(nb), sizes)
    want, fr = 0, []
    for h in range(heads):
        keyset = [set(lists[h, i]) for i in range(nb)]
        allowed = np.array([[block_of[c] in keyset[block_of[r]] for c in range(N)] for r in range(0, N, 64)])
        want += int(allowed.sum()) * 64    # rows come in 64-row groups of one block each
        fr.append(np.mean([sum(sizes[j] for j in lists[h, i]) / N for i in range(nb)]))
    assert pairs == want
    assert abs(key_frac - float(np.mean(fr))) < 1e-12
    assert hist == {64: 1, 128: 0, 256: 1} and nblocks == nb
