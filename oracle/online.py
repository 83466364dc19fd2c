"""Block-by-block online-softmax forward, in the two loop orders the pages give.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Used solely by the
CPU tests to check ``oracle.attention`` (the one-shot definition) against an
independent formulation of the method; the GPU path does not use it.

The recurrence ([tonho] "como funciona"; [mm] "A recorrencia do softmax
online"; [agi] algorithm paragraph; [ldl] section 8): for each query row keep
a running maximum m and a running sum l of exponentials taken relative to m.
When a new block of scores arrives with block maximum m~, the new maximum is
m' = max(m, m~); everything accumulated so far is multiplied by exp(m - m'),
and the block's exponentials (taken relative to m~, or directly to m') are
added.  In exact arithmetic the final O / l equals the one-shot softmax.

* ``tiled_forward_kv_outer``: key/value blocks in the outer loop, query
  blocks inner, and the output kept normalised after every step (the order of
  [tonho] "como funciona" and of [agi]'s algorithm paragraph).
* ``tiled_forward_q_outer``: query blocks outer, key/value blocks inner,
  the division by l deferred to the end of the row block (the order of
  [lynx] "El algoritmo Flash (forward)" and [mm] "O algoritmo de atencao do
  Flash"; [lynx] "Una nota sobre Flash 1 vs Flash 2" states that the two
  orders compute the same thing).

Masked scores are -inf.  Reading for the case the pages leave open: while a
row has seen only masked scores its maximum is -inf, and exp(-inf - (-inf))
is taken as 0 by using 0 as the reference instead of -inf.

Both functions take ONE head: q (N, d), k (N, d), v (N, dv), float64.
They return (O, LSE) with LSE = m + log(l) (natural log).
"""

from __future__ import annotations

import numpy as np

from .attention import visibility

__all__ = ["tiled_forward_kv_outer", "tiled_forward_q_outer"]


def _ref(m):
    """Reference point for exponentials: m itself, or 0 where m is -inf."""
    return np.where(np.isfinite(m), m, 0.0)


def _block_scores(q, k, scale, i0, i1, j0, j1, causal, block_mask, mask_block, window):
    s = scale * (q[i0:i1] @ k[j0:j1].T)
    vis = visibility(np.arange(i0, i1), np.arange(j0, j1), causal, block_mask, mask_block,
                     window)
    return np.where(vis, s, -np.inf)


def tiled_forward_kv_outer(q, k, v, scale, br, bc, causal=False, block_mask=None,
                           mask_block=128, window=0):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    nk = k.shape[0]
    o = np.zeros((n, v.shape[1]))
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    for j0 in range(0, nk, bc):
        j1 = min(nk, j0 + bc)
        vj = v[j0:j1]  # one block of values (keys are sliced in _block_scores)
        for i0 in range(0, n, br):
            i1 = min(n, i0 + br)
            s = _block_scores(q, k, scale, i0, i1, j0, j1, causal, block_mask, mask_block,
                              window)
            m_blk = s.max(axis=1)
            p_blk = np.exp(s - _ref(m_blk)[:, None])
            l_blk = p_blk.sum(axis=1)
            m_old, l_old = m[i0:i1], l[i0:i1]
            m_new = np.maximum(m_old, m_blk)
            a_old = np.exp(m_old - _ref(m_new))  # weight of what was accumulated
            a_blk = np.exp(m_blk - _ref(m_new))  # weight of the new block
            l_new = a_old * l_old + a_blk * l_blk
            num = (l_old * a_old)[:, None] * o[i0:i1] + a_blk[:, None] * (p_blk @ vj)
            safe = np.where(l_new > 0, l_new, 1.0)
            o[i0:i1] = np.where((l_new > 0)[:, None], num / safe[:, None], 0.0)
            m[i0:i1], l[i0:i1] = m_new, l_new
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


def tiled_forward_q_outer(q, k, v, scale, br, bc, causal=False, block_mask=None,
                          mask_block=128, window=0):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    nk = k.shape[0]
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        acc = np.zeros((i1 - i0, v.shape[1]))  # un-normalised output rows
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        for j0 in range(0, nk, bc):
            j1 = min(nk, j0 + bc)
            s = _block_scores(q, k, scale, i0, i1, j0, j1, causal, block_mask, mask_block,
                              window)
            m_new = np.maximum(m, s.max(axis=1))
            alpha = np.exp(m - _ref(m_new))
            p = np.exp(s - _ref(m_new)[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j1]
            m = m_new
        live = l > 0
        o[i0:i1] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            lse[i0:i1] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse
