"""The C ABI on the host (no GPU): the library loads, exports every function include/prism.h
declares, reports the candidate table the oracle enumerates independently, and rejects bad
arguments with the documented status before any HIP call."""
import ctypes

import numpy as np
import pytest

import dynamic_block_sparse_var_amd as P
import oracle


@pytest.fixture(scope="module")
def L():
    return P.lib()


def test_exports_every_header_function(L):
    names = P.header_functions()
    assert len(names) == 23
    for n in names:
        assert hasattr(L, n), n
    assert P.prism_abi_version() == 3


def test_shape_table_matches_oracle_enumeration():
    edges, _ = oracle.candidates()
    assert P.prism_shape_table() == [tuple(e) for e in edges.tolist()]


def test_status_strings(L):
    for s in range(8):
        assert L.prism_status_string(s)


def _pb(**kw):
    base = dict(T=8, H=16, W=16, heads=2, head_dim=64, groups=1, dtype=P.BF16)
    base.update(kw)
    return P.Problem(**base)


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), 2), (dict(T=12), 2), (dict(W=4), 2), (dict(heads=0), 2), (dict(head_dim=96), 2),
    (dict(groups=3), 2), (dict(dtype=7), 4), (dict(T=8, H=8 * 64, W=8 * 33), 2),
])
def test_bad_problem_rejected(L, kw, status):
    pb = _pb(**kw)
    rc = L.prism_zone_stats(ctypes.byref(pb), FAKE, None, 1e-6, FAKE, FAKE, None, None)
    assert rc == status, L.prism_last_error()
    assert L.prism_last_error()


def test_null_and_alignment_rejected(L):
    pb = _pb()
    assert L.prism_zone_stats(None, FAKE, None, 1e-6, FAKE, FAKE, None, None) == 1
    assert L.prism_zone_stats(ctypes.byref(pb), None, None, 1e-6, FAKE, FAKE, None, None) == 1
    assert L.prism_zone_stats(ctypes.byref(pb), MISALIGNED, None, 1e-6, FAKE, FAKE, None, None) == 5
    # audio given but no zone_audio output
    assert L.prism_zone_stats(ctypes.byref(pb), FAKE, FAKE, 1e-6, FAKE, FAKE, None, None) == 1
    assert L.prism_bsa_fwd(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.125, FAKE, FAKE, None, FAKE, None, FAKE, None, 0,
                           None) == 1
    assert L.prism_bsa_fwd(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.125, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE,
                           None, 0, None) == 5


def test_forward_workspace(L):
    """The forward's workspace is optional (NULL: plain launch order); when given it must be
    256-byte aligned and at least prism_bsa_fwd_workspace_bytes large (launch order and work
    estimates, one int32 each per pair of 64-row atoms and head)."""
    pb = _pb()
    need = P.prism_bsa_fwd_workspace_bytes(pb)
    N, heads = 8 * 16 * 16, 2
    assert need >= 2 * heads * (N // 128) * 4
    args = [ctypes.byref(pb)] + [FAKE] * 3 + [0.125] + [FAKE] * 4 + [None, FAKE]
    assert L.prism_bsa_fwd(*args, FAKE, need - 1, None) == 6
    assert L.prism_bsa_fwd(*args, MISALIGNED, need, None) == 5
    tok = [ctypes.byref(pb)] + [FAKE] * 4 + [0.125] + [FAKE] * 4 + [None, FAKE]
    assert L.prism_bsa_fwd_tok(*tok, FAKE, need - 1, None) == 6
    assert P.prism_bsa_fwd_workspace_bytes(_pb(T=3)) == 0
    # fp32 problems run the plain kernels and need none
    assert P.prism_bsa_fwd_workspace_bytes(_pb(dtype=P.F32)) == 0


def test_noalloc_backward_refuses_beyond_its_scratch(L):
    """prism_bsa_bwd_noalloc: the 2K-shaped problem fits its fixed 64 MiB scratch, the largest
    grid does not and is refused with PRISM_E_WORKSPACE before any launch."""
    assert P.prism_bsa_bwd_noalloc_max_bytes() == 64 << 20
    assert P.prism_bsa_bwd_workspace_bytes(_pb(T=32, H=96, W=160, heads=4, head_dim=128)) <= 64 << 20
    big = _pb(T=64, H=128, W=128, heads=4, head_dim=128)
    assert P.prism_bsa_bwd_workspace_bytes(big) > 64 << 20
    args = [ctypes.byref(big)] + [FAKE] * 3 + [0.125] + [FAKE] * 10 + [None]
    assert L.prism_bsa_bwd_noalloc(*args) == 6
    assert "scratch" in L.prism_last_error().decode()
    small = _pb()
    args = [ctypes.byref(small)] + [FAKE] * 3 + [0.125] + [FAKE] * 4 + [MISALIGNED] + [FAKE] * 5 + [None]
    assert L.prism_bsa_bwd_noalloc(*args) == 5


def test_launch_order_switch(L):
    assert L.prism_set_launch_order(2) == 3
    assert L.prism_set_launch_order(0) == 0
    assert L.prism_set_launch_order(1) == 0


def test_scalar_ranges_rejected(L):
    pb = _pb()
    assert L.prism_zone_stats(ctypes.byref(pb), FAKE, None, 0.0, FAKE, FAKE, None, None) == 3
    assert L.prism_assign_shapes(ctypes.byref(pb), FAKE, FAKE, 0.2, 0.3, FAKE, FAKE, FAKE, None) == 3
    assert L.prism_assign_shapes(ctypes.byref(pb), FAKE, FAKE, 0.5, -0.1, FAKE, FAKE, FAKE, None) == 3
    sel = L.prism_select_blocks
    assert sel(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.1, -1, 0.0, 0.5, FAKE, FAKE, None) == 3
    assert sel(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.1, 0, 1.5, 0.5, FAKE, FAKE, None) == 3
    assert sel(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.1, 0, 0.05, 1.01, FAKE, FAKE, None) == 3
    assert sel(ctypes.byref(pb), FAKE, FAKE, FAKE, 0.0, 0, 0.05, 0.5, FAKE, FAKE, None) == 3
    assert sel(ctypes.byref(pb), FAKE, FAKE, FAKE, float("nan"), 2, 0.0, 0.5, FAKE, FAKE, None) == 3
    arr = (ctypes.c_void_p * 5)(*([0x10000] * 5))
    assert L.prism_permute(ctypes.byref(pb), FAKE, 2, 1, arr, arr, None) == 3
    assert L.prism_permute(ctypes.byref(pb), FAKE, 0, 5, arr, arr, None) == 3
    assert L.prism_pool_blocks(ctypes.byref(pb), FAKE, 0, arr, arr, None) == 3
    assert L.prism_permute_pool(ctypes.byref(pb), FAKE, FAKE, 0, arr, arr, None, None) == 3
    assert L.prism_permute_pool(ctypes.byref(pb), FAKE, FAKE, 5, arr, arr, arr, None) == 3
    bad = (ctypes.c_void_p * 2)(0x10000, 0x10008)
    assert L.prism_permute_pool(ctypes.byref(pb), FAKE, FAKE, 2, arr, arr, bad, None) == 5
    assert L.prism_permute_pool(ctypes.byref(pb), None, FAKE, 1, arr, arr, None, None) == 1
    assert L.prism_fixed_shapes(ctypes.byref(pb), 16, FAKE, FAKE, FAKE, None) == 3
    assert L.prism_fixed_shapes(ctypes.byref(pb), -1, FAKE, FAKE, FAKE, None) == 3


def test_fixed_shape_index():
    # the pages' fixed-block ablation uses 4x4x4 blocks
    assert P.fixed_shape_index((4, 4, 4)) == 3
    assert P.prism_shape_table()[P.fixed_shape_index((2, 4, 8))] == (2, 4, 8)


def test_backward_workspace(L):
    pb = _pb()
    need = P.prism_bsa_bwd_workspace_bytes(pb)
    N, nb = 8 * 16 * 16, 8 * 4
    # delta and lse2, the transposed selection bitmap, two launch orders and their work estimates
    assert need >= 2 * N * 4 + 2 * nb * ((nb + 31) // 32) * 4 + 4 * (N // 64) * 4
    args = [ctypes.byref(pb)] + [FAKE] * 3 + [0.125] + [FAKE] * 10
    assert L.prism_bsa_bwd(*args, FAKE, need - 1, None) == 6
    assert L.prism_bsa_bwd(*args, MISALIGNED, need, None) == 5
    assert P.prism_bsa_bwd_workspace_bytes(_pb(T=3)) == 0


def test_audio_norms_validation(L):
    pb = _pb()
    assert L.prism_audio_norms(ctypes.byref(pb), FAKE, 0, 0, FAKE, None) == 3
    assert L.prism_audio_norms(ctypes.byref(pb), FAKE, 12, 0, FAKE, None) == 3
    assert L.prism_audio_norms(ctypes.byref(pb), FAKE, 64, 2, FAKE, None) == 3
    assert L.prism_audio_norms(ctypes.byref(pb), None, 64, 0, FAKE, None) == 1
    assert L.prism_audio_norms(ctypes.byref(pb), FAKE, 64, 0, MISALIGNED, None) == 5
    assert L.prism_audio_norms(ctypes.byref(_pb(T=3)), FAKE, 64, 0, FAKE, None) == 2


def test_token_order_attention_validation(L):
    pb = _pb()
    fwd = L.prism_bsa_fwd_tok
    # shape_idx is required: the output rows' tokens come from it
    assert fwd(ctypes.byref(pb), None, FAKE, FAKE, FAKE, 0.125, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == 1
    assert fwd(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0, None) == 3
    assert fwd(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, 0.125, FAKE, FAKE, FAKE, MISALIGNED, None, FAKE, None, 0,
               None) == 5
    need = P.prism_bsa_bwd_tok_workspace_bytes(pb)
    N, d = 8 * 16 * 16, 64
    # the block-order workspace plus a bf16 block-order copy of dO
    assert need >= P.prism_bsa_bwd_workspace_bytes(pb) + 2 * N * d * 2
    args = [ctypes.byref(pb)] + [FAKE] * 4 + [0.125] + [FAKE] * 10
    assert L.prism_bsa_bwd_tok(*args, FAKE, need - 1, None) == 6
    assert L.prism_bsa_bwd_tok(*args, MISALIGNED, need, None) == 5
    assert L.prism_bsa_bwd_tok(ctypes.byref(pb), None, *([FAKE] * 3), 0.125, *([FAKE] * 10), FAKE, need,
                               None) == 1
    assert P.prism_bsa_bwd_tok_workspace_bytes(_pb(T=3)) == 0


def test_selection_capacity_limit(L):
    # 2048 zones (1,048,576 tokens) is the largest grid; 2049+ must be refused up front
    pb = _pb(T=8, H=8 * 32, W=8 * 65)
    assert L.prism_zone_stats(ctypes.byref(pb), FAKE, None, 1e-6, FAKE, FAKE, None, None) == 2
    assert np.isfinite(0.0)
