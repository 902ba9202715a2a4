"""Block-sparse attention and its gradient for chosen query and key blocks, in fp64 (plain
PyTorch CPU ops).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this module.  It shares no code with the HIP library or its
binding and imports neither.

This is the same definition as the C oracle's ``orc_attn_fwd`` / ``orc_attn_bwd``, written a
second way: each query block's attention is formed with whole-matrix products (a CPU matmul as
the one library step) instead of per-row loops, so that the gradient of a key block chosen by
a thousand query blocks can be checked at the full 2K sizes in seconds.  It is pinned against
the C oracle and against torch autograd in ``tests/test_oracle_pins.py``.

What it computes (reading guide of "Prism: Dynamic Sparse Attention for Native 2K Joint
Video-Audio Generation Model Training", Method part 3, "Hybrid Top-k / Top-p Attention": the
softmax attention of a query block runs solely over the key blocks of its attended set S_i;
the gradient holds the selection constant):

* forward, per query row r of block i:  z_c = sm_scale * q_r . k_c over every key row c of the
  blocks in S_i;  LSE_r = ln sum_c exp(z_c);  O_r = sum_c exp(z_c - LSE_r) v_c;
* backward:  delta_r = dO_r . O_r;  P_rc = exp(z_rc - LSE_r);  dP_rc = dO_r . v_c;
  dS_rc = P_rc (dP_rc - delta_r);  dQ_r = sm_scale sum_c dS_rc k_c;  dV_c = sum_r P_rc dO_r;
  dK_c = sm_scale sum_r dS_rc q_r, the sums over r running over the rows of every query block
  whose attended set holds the key's block.

Tensors come in block order [heads, N, d] (fp32 numpy arrays holding the exact input values);
every product is taken in fp64.  Results are numpy fp64 arrays.
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64)


class Head:
    """One head: its block-order tensors in fp64, its block layout and its selection."""

    def __init__(self, q, k, v, dout, block_start, nblocks, sel_count, sel_idx, h, sm_scale):
        self.q, self.k, self.v = _f64(q[h]), _f64(k[h]), _f64(v[h])
        self.do = None if dout is None else _f64(dout[h])
        self.bs = np.asarray(block_start, np.int64)
        self.nb = int(nblocks)
        self.cnt = np.asarray(sel_count[h, : self.nb], np.int64)
        self.idx = sel_idx[h]
        self.sm = float(sm_scale)
        self.d = self.q.shape[1]
        self._bufs = {}

    def rows(self, j):
        return torch.arange(int(self.bs[j]), int(self.bs[j + 1]), dtype=torch.int64)

    def key_rows(self, i):
        """Block-order rows of the key blocks in query block i's attended set, ascending."""
        lst = self.idx[i, : self.cnt[i]]
        if len(lst) == 0:
            return torch.zeros(0, dtype=torch.int64)
        return torch.from_numpy(np.concatenate([np.arange(self.bs[j], self.bs[j + 1]) for j in lst]))

    def _buf(self, name, shape):
        """A reused scratch tensor (large per-block buffers are not re-allocated per block)."""
        b = self._bufs.get(name)
        n = int(np.prod(shape))
        if b is None or b.numel() < n:
            b = torch.empty(n, dtype=torch.float64)
            self._bufs[name] = b
        return b[:n].view(*shape)

    def query_block(self, i, want_p=True):
        """Forward of query block i: (rows, keys, P [rows, keys] or None, O, LSE, delta or
        None).  The probabilities are only kept when want_p is set (P is then a fresh tensor)."""
        rows, keys = self.rows(i), self.key_rows(i)
        qi = self.q.index_select(0, rows)
        if len(keys) == 0:
            p = torch.zeros(len(rows), 0, dtype=torch.float64)
            o = torch.zeros(len(rows), self.d, dtype=torch.float64)
            lse = torch.full((len(rows),), -torch.inf, dtype=torch.float64)
            return rows, keys, p, o, lse, None if self.do is None else torch.zeros(len(rows), dtype=torch.float64)
        ks = torch.index_select(self.k, 0, keys, out=self._buf("ks", (len(keys), self.d)))
        e = torch.matmul(qi, ks.T, out=self._buf("e", (len(rows), len(keys))))
        e.mul_(self.sm)
        m = e.amax(dim=1)
        e.sub_(m[:, None]).exp_()          # exp(z - max) in place
        s = e.sum(dim=1)
        lse = m + torch.log(s)
        vs = torch.index_select(self.v, 0, keys, out=self._buf("ks", (len(keys), self.d)))
        o = (e @ vs).div_(s[:, None])
        p = e.div(s[:, None]) if want_p else None
        delta = None
        if self.do is not None:
            delta = (self.do.index_select(0, rows) * o).sum(dim=1)
        return rows, keys, p, o, lse, delta

    def fwd(self, i):
        """(rows, O, LSE) of query block i as numpy arrays."""
        rows, _, _, o, lse, _ = self.query_block(i, want_p=False)
        return rows.numpy(), o.numpy(), lse.numpy()

    def dq(self, i):
        """(rows, dQ) of query block i."""
        rows, keys, p, o, lse, delta = self.query_block(i)
        if len(keys) == 0:
            return rows.numpy(), np.zeros((len(rows), self.d))
        dp = self.do.index_select(0, rows) @ self.v.index_select(0, keys).T
        ds = p * (dp - delta[:, None])
        return rows.numpy(), (self.sm * (ds @ self.k.index_select(0, keys))).numpy()

    def selectors(self, j):
        """Query blocks whose attended sets hold key block j, ascending."""
        lists = self.idx[: self.nb]
        held = (lists == j) & (np.arange(lists.shape[1])[None, :] < self.cnt[:, None])
        return np.flatnonzero(held.any(axis=1)).tolist()

    def dkdv(self, j, selectors=None):
        """(rows, dK, dV) of key block j: sums over the rows of every query block that
        selected it."""
        krows = self.rows(j)
        kj, vj = self.k.index_select(0, krows), self.v.index_select(0, krows)
        dk = torch.zeros(len(krows), self.d, dtype=torch.float64)
        dv = torch.zeros_like(dk)
        for i in (self.selectors(j) if selectors is None else selectors):
            rows, _, _, _, lse, delta = self.query_block(i, want_p=False)
            qi, doi = self.q.index_select(0, rows), self.do.index_select(0, rows)
            pj = torch.exp((qi @ kj.T) * self.sm - lse[:, None])
            dsj = pj * (doi @ vj.T - delta[:, None])
            dv += pj.T @ doi
            dk += (dsj.T @ qi) * self.sm
        return krows.numpy(), dk.numpy(), dv.numpy()


def selector_counts(sel_count, sel_idx, nblocks, h):
    """For head h: how many query blocks selected each key block."""
    nb = int(nblocks)
    col = np.zeros(nb, np.int64)
    for i in range(nb):
        np.add.at(col, sel_idx[h, i, : sel_count[h, i]], 1)
    return col
