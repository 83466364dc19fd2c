"""Plain float64 definition of exact attention and its gradient (oracle).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Nothing in the
product path may import this module.

What is computed (per batch index b and head h, with N queries = N keys):

  S = scale * Q K^T                       [lynx] "El algoritmo naive de
                                          attention" (step 1; scale 1/sqrt(d)
                                          as in [mm] "O algoritmo de atencao do
                                          Flash"); [tonho] "como funciona"
                                          writes the same factor as tau.
  S_ij = -inf where key j is not visible  [mm] "O mascaramento causal ..."
         to query i                       (causal: keys in the future of the
                                          query are excluded); [agi] block-sparse
                                          paragraph (whole blocks dropped).
  LSE_i = log sum_j exp(S_ij)             natural log; the pages keep the row
                                          max m and row sum l, and
                                          LSE = m + log(l) carries both.
  P = exp(S - LSE)                        [lynx] "El algoritmo naive" step 2
  O = P V                                 [lynx] "El algoritmo naive" step 3

Backward (the pages give no gradient formulas except the D identity; this is
the analytic gradient of the definition above, pinned by finite differences
in the tests):

  dV = P^T dO
  dP = dO V^T
  D_i = sum_j P_ij dP_ij                  [tonho] "como funciona" states that
                                          this equals the d-length dot
                                          dO_i . O_i; both are returned.
  dS = P o (dP - D)
  dQ = scale * dS K
  dK = scale * dS^T Q

Visibility of key j to query i (mask_block = side of a mask block):
  [not causal or j <= i] and [block_mask is None or
                              block_mask[i // mask_block, j // mask_block] != 0]
  and [window == 0 or |i - j| < window]
The window term is the sliding-window rule of [lynx] "Problemas de
practica" (a window of W keys around each query).  The page poses it without
fixing the boundary; the reading taken is |i - j| < W, which together with
the causal rule keeps the W most recent keys i-W+1 .. i.

Grouped heads (GQA/MQA, [ldl] sections 4-6): K and V may carry H_kv heads
with H_kv dividing the H query heads; query head h reads K/V head
h // (H / H_kv).  dK and dV of a K/V head are the sums of the contributions of
the H / H_kv query heads that read it.

Dropout ([tonho] "como funciona"; [agi] algorithm paragraph: the mask is
applied inside the fused kernel and regenerated in the backward pass from
the saved generator state): with keep mask Z01 from ``oracle.philox`` and
Z = Z01 / (1 - p'),
  O = (P o Z) V,  LSE unchanged (it is the normaliser of P, not of P o Z),
  dV = (P o Z)^T dO,  dP = Z o (dO V^T),  D_i = sum_j P_ij dP_ij = dO_i . O_i,
  dS = P o (dP - D).

Fully masked rows (possible only with a general block mask): O_i = 0,
LSE_i = -inf, and the row contributes nothing to any gradient.

Queries at an offset (the decode shape: a few queries against a long key
sequence, as in incremental decoding after the
[ldl] sections 4-6 discussion of grouped heads): query row r sits at position
q_offset + r of the key sequence, and every visibility rule above uses that
position (causal: key j <= q_offset + r; window: |q_offset + r - j| < W).
q_offset = 0 with as many queries as keys is the square case; decoding the
last n_q positions of N keys is q_offset = N - n_q.

Memory: rows are processed in chunks, and each chunk only touches the key
columns that can be visible to some row of the chunk (a causal prefix, or the
kept key blocks of the chunk's query blocks).  Columns left out are exactly
those whose probability is 0 for every row of the chunk, so the result is the
same as the dense masked evaluation; a test checks this on small shapes.
Each row's softmax is always evaluated over all of its candidate columns at
once -- no online recurrence is used here.
"""

from __future__ import annotations

import numpy as np

from .philox import dropout_keep

__all__ = [
    "visibility",
    "attention_probs",
    "attention_forward",
    "attention_backward",
]

_CHUNK_ELEMS = 1 << 22  # rows * candidate columns per chunk (32 MiB of f64)


def visibility(rows, cols, causal=False, block_mask=None, mask_block=128, window=0):
    """Boolean matrix vis[r, c]: is key ``cols[c]`` visible to query ``rows[r]``."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    vis = np.ones((rows.size, cols.size), dtype=bool)
    if causal:
        vis &= cols[None, :] <= rows[:, None]
    if window:
        vis &= np.abs(cols[None, :] - rows[:, None]) < window
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        vis &= bm[(rows // mask_block)[:, None], (cols // mask_block)[None, :]]
    return vis


def _candidate_columns(r0, r1, n, causal, block_mask, mask_block, window=0):
    """Key columns that may be visible to some query row in [r0, r1)."""
    cols = np.arange(n, dtype=np.int64)
    if causal:
        cols = cols[cols < r1]
    if window:
        cols = cols[(cols > r0 - window) & (cols < r1 - 1 + window)]
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        qblocks = np.unique(np.arange(r0, r1) // mask_block)
        kept_kblocks = bm[qblocks].any(axis=0)
        cols = cols[kept_kblocks[cols // mask_block]]
    return cols


def _row_chunks(n, causal, block_mask, mask_block, row_chunk):
    if row_chunk is None:
        if block_mask is not None:
            row_chunk = mask_block
        else:
            row_chunk = max(1, min(n, _CHUNK_ELEMS // max(n, 1)))
    r0 = 0
    while r0 < n:
        r1 = min(n, r0 + row_chunk)
        yield r0, r1
        r0 = r1


def _softmax_rows(s):
    """Natural-log LSE and probabilities of each row of s (entries may be -inf).

    A row whose entries are all -inf gets LSE = -inf and probabilities 0.
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(live, m_safe + np.log(np.where(live, l, 1.0)), -np.inf)
    p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
    return lse, p


def attention_probs(q, k, scale, causal=False, block_mask=None, mask_block=128, window=0):
    """Dense P (N x N) and LSE (N) for ONE head; small shapes only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n = q.shape[0]
    s = scale * (q @ k.T)
    vis = visibility(np.arange(n), np.arange(k.shape[0]), causal, block_mask, mask_block,
                     window)
    s = np.where(vis, s, -np.inf)
    lse, p = _softmax_rows(s)
    return p, lse


class _Spec:
    """Mask and dropout settings shared by the per-head routines."""

    def __init__(self, scale, causal, block_mask, mask_block, window, dropout_p, seed,
                 offset, row_chunk, q_offset=0):
        if window < 0:
            raise ValueError("window must be >= 0")
        if q_offset < 0:
            raise ValueError("q_offset must be >= 0")
        self.q_offset = q_offset
        if not 0.0 <= dropout_p < 1.0:
            raise ValueError("dropout_p must be in [0, 1)")
        self.scale, self.causal = scale, causal
        self.block_mask, self.mask_block = block_mask, mask_block
        self.window, self.row_chunk = window, row_chunk
        self.dropout_p, self.seed, self.offset = dropout_p, seed, offset

    def chunks(self, n):
        return _row_chunks(n, self.causal, self.block_mask, self.mask_block, self.row_chunk)

    def columns(self, r0, r1, n):
        """Candidate key columns of query rows [r0, r1) (positions shifted by q_offset)."""
        return _candidate_columns(r0 + self.q_offset, r1 + self.q_offset, n, self.causal,
                                  self.block_mask, self.mask_block, self.window)

    def scores(self, q, k, rows, cols):
        s = self.scale * (q[rows] @ k[cols].T)
        vis = visibility(rows + self.q_offset, cols, self.causal, self.block_mask,
                         self.mask_block, self.window)
        return np.where(vis, s, -np.inf)

    def drop(self, rows, cols, head):
        """Dropout multiplier Z for the (rows x cols) block, or None if p = 0."""
        if self.dropout_p == 0.0:
            return None
        keep, mult = dropout_keep(rows + self.q_offset, cols, head, self.seed, self.offset,
                                  self.dropout_p)
        return keep * mult


def _forward_head(q, k, v, spec, head):
    n, d = q.shape
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    for r0, r1 in spec.chunks(n):
        cols = spec.columns(r0, r1, k.shape[0])
        rows = np.arange(r0, r1)
        if cols.size == 0:
            continue
        lse_c, p = _softmax_rows(spec.scores(q, k, rows, cols))
        z = spec.drop(rows, cols, head)
        if z is not None:
            p = p * z
        lse[r0:r1] = lse_c
        o[r0:r1] = p @ v[cols]
    return o, lse


def _backward_head(q, k, v, do, spec, head):
    n, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    d_vec = np.zeros(n)
    d_dot = np.zeros(n)
    for r0, r1 in spec.chunks(n):
        cols = spec.columns(r0, r1, k.shape[0])
        rows = np.arange(r0, r1)
        if cols.size == 0:
            continue
        _, p = _softmax_rows(spec.scores(q, k, rows, cols))
        z = spec.drop(rows, cols, head)
        pz = p if z is None else p * z
        o_c = pz @ v[cols]
        dv[cols] += pz.T @ do[r0:r1]
        dp = do[r0:r1] @ v[cols].T
        if z is not None:
            dp = dp * z
        dd = (p * dp).sum(axis=1)
        ds = p * (dp - dd[:, None])
        dq[r0:r1] = spec.scale * (ds @ k[cols])
        dk[cols] += spec.scale * (ds.T @ q[r0:r1])
        d_vec[r0:r1] = dd
        d_dot[r0:r1] = (do[r0:r1] * o_c).sum(axis=1)
    return dq, dk, dv, d_vec, d_dot


def _as_bhnd(x):
    """View as (B, H, N, d); the float64 upcast happens per head (``_f64``)."""
    x = np.asarray(x)
    if x.ndim == 2:
        x = x[None, None]
    if x.ndim != 4:
        raise ValueError("expected (B, H, N, d) or (N, d)")
    if not np.issubdtype(x.dtype, np.floating):
        raise ValueError("expected a float array")
    return x


def _f64(x):
    """Exact upcast of one head's (N, d) slice to float64."""
    return np.asarray(x, dtype=np.float64)


def _select(x, heads):
    if heads is None:
        return [(b, h) for b in range(x.shape[0]) for h in range(x.shape[1])]
    return [tuple(bh) for bh in heads]


def _group(q, k, v):
    """Query heads per K/V head; checks the grouped-head shapes."""
    hq, hkv = q.shape[1], k.shape[1]
    if k.shape[:2] != v.shape[:2] or k.shape[0] != q.shape[0] or hkv == 0 or hq % hkv:
        raise ValueError("K/V heads must divide the query heads")
    return hq // hkv


def attention_forward(q, k, v, scale, causal=False, block_mask=None, mask_block=128,
                      heads=None, row_chunk=None, window=0, dropout_p=0.0, seed=0,
                      offset=0, q_offset=0):
    """O (float64) and natural-log LSE (float64) of the definition above.

    q: (B, H, N, d); k, v: (B, H_kv, N, d) with H_kv dividing H; or all (N, d).
    Any float dtype (upcast exactly).
    heads: optional list of (b, h) query heads; then the results are stacked
           in that order with shapes (len(heads), N, d) and (len(heads), N).
    window: 0 (none) or W > 0, keys with |i - j| >= W hidden.
    dropout_p, seed, offset: dropout of P as in ``oracle.philox.dropout_keep``
           with head index b * H + h.
    q_offset: position of query row 0 in the key sequence (decode: N_k - N_q);
           q may then have fewer rows than k and v.
    """
    q, k, v = _as_bhnd(q), _as_bhnd(k), _as_bhnd(v)
    g = _group(q, k, v)
    spec = _Spec(scale, causal, block_mask, mask_block, window, dropout_p, seed, offset,
                 row_chunk, q_offset)
    outs, lses = [], []
    for b, h in _select(q, heads):
        o, lse = _forward_head(_f64(q[b, h]), _f64(k[b, h // g]), _f64(v[b, h // g]), spec,
                               b * q.shape[1] + h)
        outs.append(o)
        lses.append(lse)
    o = np.stack(outs)
    lse = np.stack(lses)
    if heads is None:
        o = o.reshape(q.shape[0], q.shape[1], *o.shape[1:])
        lse = lse.reshape(q.shape[0], q.shape[1], -1)
    return o, lse


def attention_backward(q, k, v, do, scale, causal=False, block_mask=None, mask_block=128,
                       heads=None, row_chunk=None, return_d=False, window=0, dropout_p=0.0,
                       seed=0, offset=0):
    """dQ, dK, dV (float64) of f = <O(Q, K, V), dO>; P is rebuilt from Q and K.

    Shapes as in ``attention_forward``; dK, dV have the shape of K, V, each
    K/V head summing the contributions of its group of query heads.  With
    ``heads`` given, the results are stacked per selected query head and
    dK, dV hold that head's own contribution (not summed over the group).
    With return_d=True also returns (D, D_dot): D_i = sum_j P_ij dP_ij and the
    d-length dot dO_i . O_i, which the pages state are equal.
    """
    q, k, v, do = _as_bhnd(q), _as_bhnd(k), _as_bhnd(v), _as_bhnd(do)
    g = _group(q, k, v)
    spec = _Spec(scale, causal, block_mask, mask_block, window, dropout_p, seed, offset,
                 row_chunk)
    sel = _select(q, heads)
    res = [_backward_head(_f64(q[b, h]), _f64(k[b, h // g]), _f64(v[b, h // g]),
                          _f64(do[b, h]), spec, b * q.shape[1] + h) for b, h in sel]
    dq, dk, dv, dd, ddot = (np.stack([r[i] for r in res]) for i in range(5))
    if heads is None:
        shp = (q.shape[0], q.shape[1])
        dq = dq.reshape(*shp, *dq.shape[1:])
        dk, dv = (x.reshape(q.shape[0], k.shape[1], g, *x.shape[1:]).sum(axis=2)
                  for x in (dk, dv))
        dd, ddot = (x.reshape(*shp, -1) for x in (dd, ddot))
    if return_d:
        return dq, dk, dv, dd, ddot
    return dq, dk, dv
