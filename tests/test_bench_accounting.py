"""Host-side accounting of the benchmark: the forward's (pair, union tile) units, on small
hand-built block layouts and selections where the answer is known without the matching."""
import types

import torch

import bench


def _layer(block_sizes, lists, N):
    """A stand-in for PrismLayer's selection outputs: one head, one group."""
    nb = len(block_sizes)
    nbmax = 8 * (N // 512)
    bs = torch.full((1, nbmax + 1), N, dtype=torch.int32)
    bs[0, 0] = 0
    bs[0, 1:nb + 1] = torch.tensor(block_sizes, dtype=torch.int32).cumsum(0)
    cnt = torch.zeros(1, nbmax, dtype=torch.int32)
    idx = torch.zeros(1, nbmax, nbmax, dtype=torch.int32)
    for i, l in enumerate(lists):
        cnt[0, i] = len(l)
        idx[0, i, :len(l)] = torch.tensor(sorted(l), dtype=torch.int32)
    layer = types.SimpleNamespace(block_start=bs, sel_count=cnt, sel_idx=idx)
    pb = types.SimpleNamespace(N=N, heads=1, groups=1, nbmax=nbmax)
    return layer, pb


def test_identical_lists_halve_the_stream():
    # two zones: eight 64-row blocks, then four 128-row blocks; every list is the same
    sizes = [64] * 8 + [128] * 4
    lists = [[0, 3, 8, 11]] * 12
    layer, pb = _layer(sizes, lists, 1024)
    union, atom = bench.forward_pair_tiles(layer, pb)
    per_list = 1 + 1 + 2 + 2  # tiles of blocks 0, 3 (64 rows) and 8, 11 (128 rows)
    assert atom == 16 * per_list  # 16 atoms
    assert union == 8 * per_list  # 8 pairs, one shared list each


def test_disjoint_lists_are_not_shared():
    # one zone of eight 64-row blocks, every list a different single block
    sizes = [64] * 8
    lists = [[i] for i in range(8)]
    layer, pb = _layer(sizes, lists, 512)
    union, atom = bench.forward_pair_tiles(layer, pb)
    assert atom == 8 and union == 8


def test_matching_pairs_the_overlapping_lists():
    # blocks 0 and 5, 1 and 6, 2 and 7, 3 and 4 hold identical lists; neighbours share nothing,
    # so only a matching by overlap halves the stream
    sizes = [64] * 8
    groups = {0: [0, 1], 5: [0, 1], 1: [2, 3], 6: [2, 3], 2: [4, 5], 7: [4, 5], 3: [6, 7], 4: [6, 7]}
    lists = [groups[i] for i in range(8)]
    layer, pb = _layer(sizes, lists, 512)
    union, atom = bench.forward_pair_tiles(layer, pb)
    assert atom == 16 and union == 8
