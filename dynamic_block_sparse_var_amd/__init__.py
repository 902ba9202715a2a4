"""Python binding of libprism, the MI355X (gfx950) HIP implementation of Prism's dynamic
block-sparse video self-attention hot path.

The functions named ``prism_*`` mirror the C ABI in ``include/prism.h`` one to one: they take
a :class:`Problem` and torch tensors (device memory), pass raw pointers and the current HIP
stream, and raise :class:`PrismError` on a non-zero status.  Every step of the computation
runs in the library's kernels; torch only provides memory and streams.  There is no
fallback: if ``libprism.so`` has not been built, loading raises.

:class:`PrismLayer` strings the calls together for one layer (allocating the outputs with
torch, once), :class:`PrismAttentionFunction` wraps forward and backward for autograd and
:class:`PrismAttention` is a module that owns one layer's buffers.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprism.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "prism.h")

F32, BF16 = 0, 1
_STATUS = {0: "PRISM_OK", 1: "PRISM_E_NULL", 2: "PRISM_E_SHAPE", 3: "PRISM_E_RANGE", 4: "PRISM_E_DTYPE",
           5: "PRISM_E_ALIGN", 6: "PRISM_E_WORKSPACE", 7: "PRISM_E_HIP"}


class PrismError(RuntimeError):
    def __init__(self, name, status, detail):
        super().__init__(f"{name} failed: {_STATUS.get(status, status)}: {detail}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]

    @property
    def N(self):
        return self.T * self.H * self.W

    @property
    def Z(self):
        return self.N // 512

    @property
    def nbmax(self):
        return 8 * self.Z

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == BF16 else torch.float32


def make_problem(T, H, W, heads, head_dim, groups=1, dtype=BF16) -> Problem:
    if isinstance(dtype, str):
        dtype = {"bf16": BF16, "f32": F32}[dtype]
    return Problem(T, H, W, heads, head_dim, groups, dtype)


_lib = None
_vp, _i32, _f32, _f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double
_PB = ctypes.POINTER(Problem)


def lib():
    """Load libprism.so (raises if it was not built: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m dynamic_block_sparse_var_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "prism_abi_version": (_i32, []),
        "prism_status_string": (ctypes.c_char_p, [_i32]),
        "prism_last_error": (ctypes.c_char_p, []),
        "prism_shape_table": (_i32, [_vp]),
        "prism_zone_stats": (_i32, [_PB, _vp, _vp, _f32, _vp, _vp, _vp, _vp]),
        "prism_assign_shapes": (_i32, [_PB, _vp, _vp, _f32, _f32, _vp, _vp, _vp, _vp]),
        "prism_fixed_shapes": (_i32, [_PB, _i32, _vp, _vp, _vp, _vp]),
        "prism_permute": (_i32, [_PB, _vp, _i32, _i32, _vp, _vp, _vp]),
        "prism_pool_blocks": (_i32, [_PB, _vp, _i32, _vp, _vp, _vp]),
        "prism_select_blocks": (_i32, [_PB, _vp, _vp, _vp, _f32, _i32, _f64, _f64, _vp, _vp, _vp]),
        "prism_bsa_fwd_workspace_bytes": (ctypes.c_size_t, [_PB]),
        "prism_bsa_fwd": (_i32, [_PB, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                 _vp]),
        "prism_bsa_bwd_workspace_bytes": (ctypes.c_size_t, [_PB]),
        "prism_trace_kernel": (_i32, [ctypes.c_char_p, _vp, _vp]),
        "prism_set_launch_order": (_i32, [_i32]),
        "prism_bsa_bwd_noalloc_max_bytes": (ctypes.c_size_t, []),
        "prism_bsa_bwd_noalloc": (_i32, [_PB, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp]),
        "prism_bsa_bwd": (_i32, [_PB, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.c_size_t, _vp]),
        "prism_audio_norms": (_i32, [_PB, _vp, _i32, _i32, _vp, _vp]),
        "prism_permute_pool": (_i32, [_PB, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
        "prism_bsa_fwd_tok": (_i32, [_PB, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]),
        "prism_bsa_bwd_tok_workspace_bytes": (ctypes.c_size_t, [_PB]),
        "prism_bsa_bwd_tok": (_i32, [_PB, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, ctypes.c_size_t, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions declared in include/prism.h."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z0-9_]+)\s*\(", text)))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, name):
    if status != 0:
        raise PrismError(name, status, lib().prism_last_error().decode())


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    return arr


# ---- one-to-one ABI wrappers ------------------------------------------------------------

def prism_abi_version() -> int:
    return lib().prism_abi_version()


def prism_shape_table() -> list[tuple[int, int, int]]:
    buf = (ctypes.c_int32 * 48)()
    n = lib().prism_shape_table(buf)
    return [tuple(buf[3 * i:3 * i + 3]) for i in range(n)]


def prism_audio_norms(pb, hhat, a, squared=False, stream=None):
    """Per-token L2 norm (or sum of squares) of hhat [N, C] -> a [N] fp32."""
    _check(lib().prism_audio_norms(ctypes.byref(pb), _p(hhat), int(hhat.shape[-1]), 1 if squared else 0, _p(a),
                                   _stream(stream)), "prism_audio_norms")


def prism_zone_stats(pb, v, a, eps, g, rho, zone_audio, stream=None):
    _check(lib().prism_zone_stats(ctypes.byref(pb), _p(v), _p(a), eps, _p(g), _p(rho), _p(zone_audio),
                                  _stream(stream)), "prism_zone_stats")


def prism_assign_shapes(pb, g, rho, tau128, tau256, shape_idx, zone_block_off, block_start, stream=None):
    _check(lib().prism_assign_shapes(ctypes.byref(pb), _p(g), _p(rho), tau128, tau256, _p(shape_idx),
                                     _p(zone_block_off), _p(block_start), _stream(stream)), "prism_assign_shapes")


def prism_fixed_shapes(pb, shape_index, shape_idx, zone_block_off, block_start, stream=None):
    _check(lib().prism_fixed_shapes(ctypes.byref(pb), int(shape_index), _p(shape_idx), _p(zone_block_off),
                                    _p(block_start), _stream(stream)), "prism_fixed_shapes")


def fixed_shape_index(edges=(4, 4, 4)) -> int:
    """Index of a candidate shape (bT, bH, bW) in prism_shape_table (4x4x4 -> 3)."""
    return prism_shape_table().index(tuple(edges))


def prism_permute(pb, shape_idx, inverse, src, dst, stream=None):
    src, dst = list(src), list(dst)
    _check(lib().prism_permute(ctypes.byref(pb), _p(shape_idx), int(inverse), len(src), _ptr_array(src),
                               _ptr_array(dst), _stream(stream)), "prism_permute")


def prism_permute_pool(pb, shape_idx, zone_block_off, src, dst, xbar=None, stream=None):
    """Token -> block order for the tensors in src (into dst) and, where xbar[i] is a tensor,
    their pooled block means (prism_permute + prism_pool_blocks in one pass)."""
    n = len(src)
    pooled = None
    if xbar is not None:
        pooled = (ctypes.c_void_p * n)(*[None if x is None else x.data_ptr() for x in xbar])
    _check(lib().prism_permute_pool(ctypes.byref(pb), _p(shape_idx), _p(zone_block_off), n, _ptr_array(src),
                                    _ptr_array(dst), pooled, _stream(stream)), "prism_permute_pool")


def prism_pool_blocks(pb, block_start, x_perm, xbar, stream=None):
    x_perm, xbar = list(x_perm), list(xbar)
    _check(lib().prism_pool_blocks(ctypes.byref(pb), _p(block_start), len(x_perm), _ptr_array(x_perm),
                                   _ptr_array(xbar), _stream(stream)), "prism_pool_blocks")


def prism_select_blocks(pb, block_start, qbar, kbar, sm_scale, k_abs, k_frac, p, sel_count, sel_idx, stream=None):
    _check(lib().prism_select_blocks(ctypes.byref(pb), _p(block_start), _p(qbar), _p(kbar), sm_scale, int(k_abs),
                                     float(k_frac), float(p), _p(sel_count), _p(sel_idx), _stream(stream)),
           "prism_select_blocks")


def prism_bsa_fwd_workspace_bytes(pb) -> int:
    return int(lib().prism_bsa_fwd_workspace_bytes(ctypes.byref(pb)))


def _ws(workspace):
    """(pointer, bytes) of an optional workspace tensor."""
    if workspace is None:
        return None, 0
    return _p(workspace), workspace.numel() * workspace.element_size()


def prism_bsa_fwd(pb, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, o_lo, lse, workspace=None, stream=None):
    wp, wn = _ws(workspace)
    _check(lib().prism_bsa_fwd(ctypes.byref(pb), _p(block_start), _p(sel_count), _p(sel_idx), sm_scale, _p(q), _p(k),
                               _p(v), _p(o), _p(o_lo), _p(lse), wp, wn, _stream(stream)), "prism_bsa_fwd")


def prism_bsa_bwd_workspace_bytes(pb) -> int:
    return int(lib().prism_bsa_bwd_workspace_bytes(ctypes.byref(pb)))


def prism_bsa_bwd(pb, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, o_lo, dout, lse, dq, dk, dv, workspace,
                  stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().prism_bsa_bwd(ctypes.byref(pb), _p(block_start), _p(sel_count), _p(sel_idx), sm_scale, _p(q), _p(k),
                               _p(v), _p(o), _p(o_lo), _p(dout), _p(lse), _p(dq), _p(dk), _p(dv), _p(workspace),
                               nbytes, _stream(stream)), "prism_bsa_bwd")


def prism_bsa_bwd_noalloc_max_bytes() -> int:
    return int(lib().prism_bsa_bwd_noalloc_max_bytes())


def prism_bsa_bwd_noalloc(pb, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, o_lo, dout, lse, dq, dk, dv,
                          stream=None):
    """prism_bsa_bwd without a workspace argument: the library's fixed per-device scratch."""
    _check(lib().prism_bsa_bwd_noalloc(ctypes.byref(pb), _p(block_start), _p(sel_count), _p(sel_idx), sm_scale,
                                       _p(q), _p(k), _p(v), _p(o), _p(o_lo), _p(dout), _p(lse), _p(dq), _p(dk),
                                       _p(dv), _stream(stream)), "prism_bsa_bwd_noalloc")


def prism_bsa_fwd_tok(pb, shape_idx, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, o_lo, lse, workspace=None,
                      stream=None):
    wp, wn = _ws(workspace)
    _check(lib().prism_bsa_fwd_tok(ctypes.byref(pb), _p(shape_idx), _p(block_start), _p(sel_count), _p(sel_idx),
                                   sm_scale, _p(q), _p(k), _p(v), _p(o), _p(o_lo), _p(lse), wp, wn,
                                   _stream(stream)), "prism_bsa_fwd_tok")


def prism_bsa_bwd_tok_workspace_bytes(pb) -> int:
    return int(lib().prism_bsa_bwd_tok_workspace_bytes(ctypes.byref(pb)))


def prism_bsa_bwd_tok(pb, shape_idx, block_start, sel_count, sel_idx, sm_scale, q, k, v, o, o_lo, dout, lse, dq, dk,
                      dv, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().prism_bsa_bwd_tok(ctypes.byref(pb), _p(shape_idx), _p(block_start), _p(sel_count), _p(sel_idx),
                                   sm_scale, _p(q), _p(k), _p(v), _p(o), _p(o_lo), _p(dout), _p(lse), _p(dq), _p(dk),
                                   _p(dv), _p(workspace), nbytes, _stream(stream)), "prism_bsa_bwd_tok")


def prism_set_launch_order(heavy_first: bool):
    """Heavy units first (True, the default) or the plain launch order (False); process-wide."""
    _check(lib().prism_set_launch_order(1 if heavy_first else 0), "prism_set_launch_order")


def prism_trace_kernel(kernel, start_event=None, stop_event=None):
    """Time one library kernel with two torch.cuda.Event(enable_timing=True) objects
    (kernel=None clears all hooks).  The events must already exist as HIP events, so they
    are recorded once here before their handles are handed over."""
    if kernel is None:
        _check(lib().prism_trace_kernel(None, None, None), "prism_trace_kernel")
        return
    for ev in (start_event, stop_event):
        ev.record()
    _check(lib().prism_trace_kernel(kernel.encode(), ctypes.c_void_p(start_event.cuda_event),
                                    ctypes.c_void_p(stop_event.cuda_event)), "prism_trace_kernel")


# ---- one layer -------------------------------------------------------------------------

class PrismLayer:
    """Buffers and call sequence for one layer's Prism attention on one device.

    The outputs of every stage are kept as attributes (g, rho, zone_audio, shape_idx,
    zone_block_off, block_start, qp/kp/vp, qbar/kbar, sel_count/sel_idx, op, lse, o, ...),
    which is what the tests inspect.  Allocation happens once, in the constructor."""

    def __init__(self, pb: Problem, device="cuda", backward=False, token_io=False):
        """token_io: the attention writes O and the gradients straight to token order
        (prism_bsa_fwd_tok / prism_bsa_bwd_tok), with no block-order O, dO or gradient buffers."""
        self.pb = pb
        self.token_io = token_io
        self.generation = 0  # forwards run through PrismAttentionFunction
        dt = pb.torch_dtype
        N, H_, d, G, Z, NB = pb.N, pb.heads, pb.head_dim, pb.groups, pb.Z, pb.nbmax
        e = dict(device=device)
        self.g = torch.empty(G, Z, 3, dtype=torch.float32, **e)
        self.rho = torch.empty(G, Z, dtype=torch.float32, **e)
        self.zone_audio = torch.empty(Z, 4, dtype=torch.float32, **e)
        self.shape_idx = torch.empty(G, Z, dtype=torch.uint8, **e)
        self.zone_block_off = torch.empty(G, Z + 1, dtype=torch.int32, **e)
        self.block_start = torch.empty(G, NB + 1, dtype=torch.int32, **e)
        self.qp = torch.empty(H_, N, d, dtype=dt, **e)
        self.kp = torch.empty_like(self.qp)
        self.vp = torch.empty_like(self.qp)
        self.qbar = torch.empty(H_, NB, d, dtype=torch.float32, **e)
        self.kbar = torch.empty_like(self.qbar)
        self.sel_count = torch.empty(H_, NB, dtype=torch.int32, **e)
        self.sel_idx = torch.empty(H_, NB, NB, dtype=torch.int32, **e)
        self.lse = torch.empty(H_, N, dtype=torch.float32, **e)
        self.o = torch.empty(N, H_, d, dtype=dt, **e)
        # the forward's launch order (heaviest pairs of atoms first); none for fp32 problems
        fbytes = prism_bsa_fwd_workspace_bytes(pb)
        self.fwd_workspace = torch.empty(fbytes, dtype=torch.uint8, **e) if fbytes > 0 else None
        # rounding residual of O (bf16 only), kept for an accurate backward
        keep_lo = backward and pb.dtype == BF16
        if token_io:
            self.op = None
            self.o_lo = torch.empty_like(self.o) if keep_lo else None
        else:
            self.op = torch.empty_like(self.qp)
            self.op_lo = torch.empty_like(self.qp) if keep_lo else None
        if backward:
            if not token_io:
                self.dop = torch.empty_like(self.qp)
                self.dqp = torch.empty(H_, N, d, dtype=torch.float32, **e)
                self.dkp = torch.empty_like(self.dqp)
                self.dvp = torch.empty_like(self.dqp)
            self.dq = torch.empty(N, H_, d, dtype=torch.float32, **e)
            self.dk = torch.empty_like(self.dq)
            self.dv = torch.empty_like(self.dq)
            nbytes = prism_bsa_bwd_tok_workspace_bytes(pb) if token_io else prism_bsa_bwd_workspace_bytes(pb)
            self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, **e)

    # a1..a5
    def plan(self, v, a, eps=1e-6, tau128=0.5, tau256=0.25, stream=None, fixed_shape=None):
        """a1 + a2; with fixed_shape (a candidate index) both are replaced by one shape for
        every zone (the pages' fixed-block ablation)."""
        pb = self.pb
        if fixed_shape is not None:
            prism_fixed_shapes(pb, fixed_shape, self.shape_idx, self.zone_block_off, self.block_start, stream)
            return
        prism_zone_stats(pb, v, a, eps, self.g, self.rho, self.zone_audio if a is not None else None, stream)
        prism_assign_shapes(pb, self.g, self.rho, tau128, tau256, self.shape_idx, self.zone_block_off,
                            self.block_start, stream)

    def select(self, q, k, v, sm_scale, k_abs, k_frac, p, stream=None):
        pb = self.pb
        if self.token_io:
            prism_permute_pool(pb, self.shape_idx, self.zone_block_off, [q, k, v], [self.qp, self.kp, self.vp],
                               [self.qbar, self.kbar, None], stream)
        else:
            prism_permute(pb, self.shape_idx, 0, [q, k, v], [self.qp, self.kp, self.vp], stream)
            prism_pool_blocks(pb, self.block_start, [self.qp, self.kp], [self.qbar, self.kbar], stream)
        prism_select_blocks(pb, self.block_start, self.qbar, self.kbar, sm_scale, k_abs, k_frac, p, self.sel_count,
                            self.sel_idx, stream)

    # a6
    def attend(self, sm_scale, stream=None):
        pb = self.pb
        if self.token_io:
            prism_bsa_fwd_tok(pb, self.shape_idx, self.block_start, self.sel_count, self.sel_idx, sm_scale, self.qp,
                              self.kp, self.vp, self.o, self.o_lo, self.lse, self.fwd_workspace, stream)
            return self.o
        prism_bsa_fwd(pb, self.block_start, self.sel_count, self.sel_idx, sm_scale, self.qp, self.kp, self.vp,
                      self.op, self.op_lo, self.lse, self.fwd_workspace, stream)
        prism_permute(pb, self.shape_idx, 1, [self.op], [self.o], stream)
        return self.o

    def forward(self, q, k, v, a, sm_scale, k_abs, k_frac, p, eps=1e-6, tau128=0.5, tau256=0.25, stream=None,
                fixed_shape=None):
        self.plan(v, a, eps, tau128, tau256, stream, fixed_shape)
        self.select(q, k, v, sm_scale, k_abs, k_frac, p, stream)
        return self.attend(sm_scale, stream)

    # a7
    def backward(self, dout, sm_scale, stream=None):
        pb = self.pb
        if self.token_io:
            prism_bsa_bwd_tok(pb, self.shape_idx, self.block_start, self.sel_count, self.sel_idx, sm_scale, self.qp,
                              self.kp, self.vp, self.o, self.o_lo, dout, self.lse, self.dq, self.dk, self.dv,
                              self.workspace, stream)
            return self.dq, self.dk, self.dv
        prism_permute(pb, self.shape_idx, 0, [dout], [self.dop], stream)
        prism_bsa_bwd(pb, self.block_start, self.sel_count, self.sel_idx, sm_scale, self.qp, self.kp, self.vp,
                      self.op, self.op_lo, self.dop, self.lse, self.dqp, self.dkp, self.dvp, self.workspace, stream)
        # gradients are fp32: move them with an fp32 view of the same geometry
        pb32 = Problem(pb.T, pb.H, pb.W, pb.heads, pb.head_dim, pb.groups, F32)
        prism_permute(pb32, self.shape_idx, 1, [self.dqp, self.dkp, self.dvp], [self.dq, self.dk, self.dv], stream)
        return self.dq, self.dk, self.dv


class PrismAttentionFunction(torch.autograd.Function):
    """Autograd wrapper: (q, k, v) token order [N, heads, d] -> o, computed by a caller-owned
    :class:`PrismLayer` (built with backward=True, token_io=True), whose buffers are reused from
    call to call.  The selection is a constant of the backward (no gradient to statistics,
    shapes, pooling or selection).  One forward per backward: the layer keeps the state of its
    last forward, so a second forward on the same layer before the first one's backward makes
    that backward raise."""

    @staticmethod
    def forward(ctx, q, k, v, a, layer, sm_scale, k_abs, k_frac, p):
        o = layer.forward(q.contiguous(), k.contiguous(), v.contiguous(), a, sm_scale, k_abs, k_frac, p)
        layer.generation += 1
        ctx.layer, ctx.generation, ctx.sm_scale = layer, layer.generation, sm_scale
        return o.clone()

    @staticmethod
    def backward(ctx, do):
        if ctx.layer.generation != ctx.generation:
            raise RuntimeError("PrismAttentionFunction: the layer ran another forward before this backward")
        dq, dk, dv = ctx.layer.backward(do.contiguous(), ctx.sm_scale)
        return dq.clone(), dk.clone(), dv.clone(), None, None, None, None, None, None


class PrismAttention(torch.nn.Module):
    """One attention layer for autograd: owns its PrismLayer (allocated once, here) and calls
    PrismAttentionFunction with the layer's knobs (bsa_sparsity s maps to k_frac = 1 - s,
    bsa_cdf_threshold to p)."""

    def __init__(self, pb: Problem, sm_scale: float, k_abs: int = 0, k_frac: float = 0.05, p: float = 0.9,
                 device="cuda"):
        super().__init__()
        self.layer = PrismLayer(pb, device=device, backward=True, token_io=True)
        self.sm_scale, self.k_abs, self.k_frac, self.p = float(sm_scale), int(k_abs), float(k_frac), float(p)

    def forward(self, q, k, v, a=None):
        return PrismAttentionFunction.apply(q, k, v, a, self.layer, self.sm_scale, self.k_abs, self.k_frac,
                                            self.p)


def default_sm_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
