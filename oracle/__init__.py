"""Python front of the plain CPU oracle (``liboracle.so``, built from ``prism_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with the
HIP library or its binding, and it imports neither.

Every function is a thin ctypes call into the C oracle, except :func:`permute` /
:func:`unpermute`, which move rows with a numpy gather using the C oracle's per-token
positions.  Citations (RG M1/M2/M3, RG KI) are explained in ``prism_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prism_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (portable -O2: no host-specific ISA, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


_c_int, _c_dbl = ctypes.c_int, ctypes.c_double


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


# ------------------------------------------------------------------------------------- #

def candidates():
    """Candidate shapes (RG KI / RG M2, reading: edges in {2,4,8}) -> (edges[16,3], volume[16])."""
    lib = _load()
    edges = np.zeros((16, 3), np.int32)
    vol = np.zeros(16, np.int32)
    n = lib.orc_candidates(_p(edges), _p(vol))
    return edges[:n].copy(), vol[:n].copy()


def audio_norms(hhat, squared=False):
    """RG M1 audio coupling input: per-token L2 norm of hhat [N, C] (sum of squares if squared)."""
    lib = _load()
    x = _f32(hhat)
    N, C = x.shape
    a = np.zeros(N)
    rc = lib.orc_audio_norms(ctypes.c_int64(N), _c_int(C), _p(x), _c_int(1 if squared else 0), _p(a))
    _check(rc, "audio_norms")
    return a


def zone_stats(v, a, T, H, W, heads, d, groups, eps, nthreads=None):
    """RG M1: zone statistics and the composite indicator g (see prism_oracle.h)."""
    lib = _load()
    v = _f32(v)
    a = None if a is None else _f32(a)
    Z = (T // 8) * (H // 8) * (W // 8)
    out = dict(sig2=np.zeros((groups, Z, 4)), r=np.zeros((groups, Z, 3)), rho=np.zeros((groups, Z)),
               abar=np.zeros(Z), vhat=np.zeros((Z, 3)), g=np.zeros((groups, Z, 3)))
    rc = lib.orc_zone_stats(_c_int(T), _c_int(H), _c_int(W), _c_int(heads), _c_int(d), _c_int(groups),
                            _p(v), _p(a), _c_dbl(eps), _p(out["sig2"]), _p(out["r"]), _p(out["rho"]),
                            _p(out["abar"]), _p(out["vhat"]), _p(out["g"]),
                            _c_int(nthreads or default_threads()))
    _check(rc, "zone_stats")
    return out


def assign_shapes(g, rho, tau128, tau256):
    """RG M2: volume, l*, distances to candidates, shape index and per-zone block offsets."""
    lib = _load()
    g = np.ascontiguousarray(g, np.float64)
    rho = np.ascontiguousarray(rho, np.float64)
    G, Z = rho.shape
    out = dict(volume=np.zeros((G, Z), np.int32), lstar=np.zeros((G, Z, 3)), dist=np.zeros((G, Z, 16)),
               shape_idx=np.zeros((G, Z), np.uint8), zone_block_off=np.zeros((G, Z + 1), np.int32))
    rc = lib.orc_assign_shapes(_c_int(G), _c_int(Z), _p(g), _p(rho), _c_dbl(tau128), _c_dbl(tau256),
                               _p(out["volume"]), _p(out["lstar"]), _p(out["dist"]),
                               _p(out["shape_idx"]), _p(out["zone_block_off"]))
    _check(rc, "assign_shapes")
    return out


def block_layout(T, H, W, shape_idx):
    """Block-order geometry -> (pos[G,N] int64, block_start[G,8Z+1] int32, nblocks[G] int32)."""
    lib = _load()
    shape_idx = np.ascontiguousarray(shape_idx, np.uint8)
    G, Z = shape_idx.shape
    N = T * H * W
    pos = np.zeros((G, N), np.int64)
    bs = np.zeros((G, 8 * Z + 1), np.int32)
    nb = np.zeros(G, np.int32)
    rc = lib.orc_block_layout(_c_int(T), _c_int(H), _c_int(W), _c_int(G), _p(shape_idx), _p(pos), _p(bs),
                              _p(nb))
    _check(rc, "block_layout")
    return pos, bs, nb


def permute(x, pos, heads):
    """Token order [N,heads,d] -> block order [heads,N,d]: y[h, pos[g(h), n]] = x[n, h]."""
    G, N = pos.shape
    hpg = heads // G
    y = np.empty((heads, N, x.shape[2]), dtype=x.dtype)
    for h in range(heads):
        y[h, pos[h // hpg]] = x[:, h, :]
    return y


def unpermute(y, pos, heads):
    """Block order [heads,N,...] -> token order [N,heads,...] (inverse of :func:`permute`)."""
    G, N = pos.shape
    hpg = heads // G
    x = np.empty((N, heads) + y.shape[2:], dtype=y.dtype)
    for h in range(heads):
        x[:, h] = y[h, pos[h // hpg]]
    return x


def pool(xperm, block_start, nblocks, groups, nthreads=None):
    """RG M3: block means of a block-order tensor [heads,N,d] -> [heads,8Z,d] fp64."""
    lib = _load()
    xperm = _f32(xperm)
    heads, N, d = xperm.shape
    nbmax = block_start.shape[1] - 1
    xbar = np.zeros((heads, nbmax, d))
    rc = lib.orc_pool(_c_int(heads), _c_int(groups), _c_int(N), _c_int(d), _c_int(nbmax),
                      _p(np.ascontiguousarray(block_start, np.int32)), _p(np.ascontiguousarray(nblocks, np.int32)),
                      _p(xperm), _p(xbar), _c_int(nthreads or default_threads()))
    _check(rc, "pool")
    return xbar


def select(qbar, kbar, nblocks, groups, sm_scale, k_abs, k_frac, p, row_mask=None, nthreads=None):
    """RG M3 attended-set equation -> (sel_count[heads,NB], sel_idx[heads,NB,NB], info[heads,NB,5])."""
    lib = _load()
    qbar = np.ascontiguousarray(qbar, np.float64)
    kbar = np.ascontiguousarray(kbar, np.float64)
    heads, nbmax, d = qbar.shape
    cnt = np.zeros((heads, nbmax), np.int32)
    idx = np.zeros((heads, nbmax, nbmax), np.int32)
    info = np.full((heads, nbmax, 5), np.nan)
    rm = None if row_mask is None else np.ascontiguousarray(row_mask, np.uint8)
    rc = lib.orc_select(_c_int(heads), _c_int(groups), _c_int(d), _c_int(nbmax),
                        _p(np.ascontiguousarray(nblocks, np.int32)), _p(qbar), _p(kbar), _c_dbl(sm_scale),
                        ctypes.c_int32(int(k_abs)), _c_dbl(k_frac), _c_dbl(p), _p(rm), _p(cnt), _p(idx),
                        _p(info), _c_int(nthreads or default_threads()))
    _check(rc, "select")
    return cnt, idx, info


def attn_fwd(q, k, v, block_start, nblocks, groups, sel_count, sel_idx, sm_scale, qblock_mask=None,
             nthreads=None):
    """RG M3 attention over S_i, block order -> (o[heads,N,d] fp64, lse[heads,N] fp64)."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    heads, N, d = q.shape
    nbmax = block_start.shape[1] - 1
    o = np.zeros((heads, N, d))
    lse = np.full((heads, N), np.nan)
    m = None if qblock_mask is None else np.ascontiguousarray(qblock_mask, np.uint8)
    rc = lib.orc_attn_fwd(_c_int(heads), _c_int(groups), _c_int(N), _c_int(d), _c_int(nbmax),
                          _p(np.ascontiguousarray(block_start, np.int32)), _p(np.ascontiguousarray(nblocks, np.int32)),
                          _p(np.ascontiguousarray(sel_count, np.int32)), _p(np.ascontiguousarray(sel_idx, np.int32)),
                          _c_dbl(sm_scale), _p(q), _p(k), _p(v), _p(m), _p(o), _p(lse),
                          _c_int(nthreads or default_threads()))
    _check(rc, "attn_fwd")
    return o, lse


def attn_bwd(q, k, v, dout, block_start, nblocks, groups, sel_count, sel_idx, sm_scale,
             qblock_mask=None, kblock_mask=None, nthreads=None):
    """Gradient of :func:`attn_fwd` (selection constant) -> dict(dq, dk, dv, lse, delta)."""
    lib = _load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    heads, N, d = q.shape
    nbmax = block_start.shape[1] - 1
    out = dict(dq=np.zeros((heads, N, d)), dk=np.zeros((heads, N, d)), dv=np.zeros((heads, N, d)),
               lse=np.full((heads, N), np.nan), delta=np.full((heads, N), np.nan))
    qm = None if qblock_mask is None else np.ascontiguousarray(qblock_mask, np.uint8)
    km = None if kblock_mask is None else np.ascontiguousarray(kblock_mask, np.uint8)
    rc = lib.orc_attn_bwd(_c_int(heads), _c_int(groups), _c_int(N), _c_int(d), _c_int(nbmax),
                          _p(np.ascontiguousarray(block_start, np.int32)), _p(np.ascontiguousarray(nblocks, np.int32)),
                          _p(np.ascontiguousarray(sel_count, np.int32)), _p(np.ascontiguousarray(sel_idx, np.int32)),
                          _c_dbl(sm_scale), _p(q), _p(k), _p(v), _p(dout), _p(qm), _p(km),
                          _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["lse"]), _p(out["delta"]),
                          _c_int(nthreads or default_threads()))
    _check(rc, "attn_bwd")
    return out


def last_bwd_phase_seconds():
    """Wall seconds of the last attn_bwd call's passes: (row statistics, dQ, dK/dV)."""
    out = np.zeros(3)
    _load().orc_last_bwd_phase_seconds(_p(out))
    return tuple(out)


def forward_path(inp, groups=1, row_mask=None, nthreads=None):
    """Whole oracle pipeline for one layer on a dict from ``synth.make_inputs``:
    stats -> shapes -> block order -> pooled Q/K -> selection.  Attention is left to the
    caller (it is the expensive part).  Returns a dict of every intermediate."""
    cfg = inp["cfg"]
    T, H, W, heads, d = cfg.T, cfg.H, cfg.W, cfg.heads, cfg.d
    st = zone_stats(inp["v"], inp["a"], T, H, W, heads, d, groups, inp["eps"], nthreads)
    sh = assign_shapes(st["g"], st["rho"], inp["tau128"], inp["tau256"])
    pos, bs, nb = block_layout(T, H, W, sh["shape_idx"])
    qp = permute(inp["q"], pos, heads)
    kp = permute(inp["k"], pos, heads)
    qbar = pool(qp, bs, nb, groups, nthreads)
    kbar = pool(kp, bs, nb, groups, nthreads)
    cnt, idx, info = select(qbar, kbar, nb, groups, inp["sm_scale"], inp["k_abs"], inp["k_frac"], inp["p"],
                            row_mask=row_mask, nthreads=nthreads)
    return dict(stats=st, shapes=sh, pos=pos, block_start=bs, nblocks=nb, qp=qp, kp=kp, qbar=qbar,
                kbar=kbar, sel_count=cnt, sel_idx=idx, sel_info=info)
