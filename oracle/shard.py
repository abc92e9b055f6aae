"""CPU oracle for one vocabulary shard of the loss (a tensor-parallel output head).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test suite and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path.

The released code takes a tensor-parallel rank and size (codewithpapers.app
record: ``tensor_parallel_rank``, ``tensor_parallel_size``): each of G ranks
holds a contiguous block of rows ``[v0, v0 + Vs)`` of the output projection W,
so the logits of a token are split across ranks by vocabulary entry.  The
definitions below restrict the dense loss of ``oracle.forward_backward`` to one
such block, written out in float64 with numpy:

* ``shard_stats``: per token, the shard's logit maximum ``m``, its sum
  ``s = sum_{v in shard} exp(z_v - m)`` and ``pz = sum_k p_k z_{idx_k}`` over the
  teacher entries whose index lies in the shard;
* ``combine``: the statistics of shards that tile the vocabulary give the
  global ``lse = log sum_g s_g exp(m_g)`` and the per-token loss
  ``l = sum_k p_k log p_k - sum_g pz_g + M lse`` (``M = sum_k p_k``), the same
  ``l = sum_k p_k (log p_k - log q_{idx_k})`` as the dense definition because
  every teacher index lies in exactly one shard;
* ``shard_backward``: given the global lse, the shard's columns of the
  closed-form gradient (legiblepapers.com summary, Q5: a dense M * softmax term
  minus the sparse teacher correction at the support positions), restricted to
  the shard's entries: ``dz = g (mask/count) (M exp(z - lse) - sum of p at
  in-shard indices)``; the shard's partial ``dh_g = dz @ W_shard`` (the ranks'
  partials sum to dh) and its rows ``dW_shard = dz^T @ h``.

Rows are independent, so tokens are taken in row blocks only to bound host
memory.
"""
from __future__ import annotations

import numpy as np

__all__ = ["shard_stats", "combine", "shard_backward"]


def _in_shard(idx, v0, Vs):
    return (idx >= v0) & (idx < v0 + Vs)


def shard_stats(h, W_shard, v0: int, idx, p, block_rows: int = 256):
    """Per-token statistics of the vocabulary rows ``[v0, v0 + Vs)``.

    Args: h [N, d]; W_shard [Vs, d] (rows v0..v0+Vs-1 of W); idx [N, K] global teacher
    indices; p [N, K] teacher probabilities.
    Returns (m, s, pz), each [N] float64: the shard's max logit, sum of exp(z - m) over
    the shard, and sum of p_k * z_{idx_k} over the entries whose index is in the shard.
    """
    h = np.asarray(h, dtype=np.float64)
    W_shard = np.asarray(W_shard, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    p = np.asarray(p, dtype=np.float64)
    N, Vs = h.shape[0], W_shard.shape[0]
    m, s, pz = np.zeros(N), np.zeros(N), np.zeros(N)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        Z = h[r0:r1] @ W_shard.T                       # the shard's logits [b, Vs]
        m[r0:r1] = Z.max(axis=1)
        s[r0:r1] = np.exp(Z - m[r0:r1, None]).sum(axis=1)
        ib = idx[r0:r1]
        inside = _in_shard(ib, v0, Vs)
        z_at = np.take_along_axis(Z, np.where(inside, ib - v0, 0), axis=1)
        pz[r0:r1] = np.where(inside, p[r0:r1] * z_at, 0.0).sum(axis=1)
    return m, s, pz


def combine(ms, ss, pzs, p, mask=None):
    """Global logsumexp and loss from the statistics of G shards that tile the vocabulary.

    Args: ms, ss, pzs [G, N] (``shard_stats`` of each shard); p [N, K]; mask [N] or None.
    Returns a dict with ``loss`` (mean over counted tokens), ``row_lse`` [N], ``row_loss``
    [N] (``l_n`` where the mask is set, else 0) and ``count``.
    """
    ms = np.asarray(ms, dtype=np.float64)
    ss = np.asarray(ss, dtype=np.float64)
    pzs = np.asarray(pzs, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    N = p.shape[0]
    mask = np.ones(N, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    count = int(mask.sum())
    top = ms.max(axis=0)
    lse = top + np.log((ss * np.exp(ms - top[None, :])).sum(axis=0))
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)   # 0 log 0 = 0
    ell = plogp.sum(axis=1) - pzs.sum(axis=0) + p.sum(axis=1) * lse
    row_loss = np.where(mask, ell, 0.0)
    loss = float(row_loss.sum() / count) if count else 0.0
    return dict(loss=loss, row_lse=lse, row_loss=row_loss, count=count)


def shard_backward(h, W_shard, v0: int, idx, p, lse, mask=None, count=None, g: float = 1.0,
                   block_rows: int = 256, rows=None):
    """The shard's share of the gradients for an upstream gradient g of the mean loss.

    Args: h [N, d]; W_shard [Vs, d]; idx, p [N, K]; lse [N] the global logsumexp; mask [N]
    or None; count: counted tokens of the whole batch (default: from mask); rows: optional
    token indices whose dh partial rows are returned (all rows when None).
    Returns (dh_partial [N or len(rows), d], dW_shard [Vs, d]).
    """
    h = np.asarray(h, dtype=np.float64)
    W_shard = np.asarray(W_shard, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    p = np.asarray(p, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    N, d, Vs = h.shape[0], h.shape[1], W_shard.shape[0]
    mask = np.ones(N, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    count = int(mask.sum()) if count is None else int(count)
    scale = g * mask / count if count else np.zeros(N)
    keep = None if rows is None else np.zeros(N, dtype=bool)
    if keep is not None:
        keep[np.asarray(rows)] = True
    dh = np.zeros((N, d)) if rows is None else {}
    dW = np.zeros((Vs, d))
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        Z = h[r0:r1] @ W_shard.T
        ib, pb = idx[r0:r1], p[r0:r1]
        dZ = (scale[r0:r1] * pb.sum(axis=1))[:, None] * np.exp(Z - lse[r0:r1, None])
        inside = _in_shard(ib, v0, Vs)
        rr = np.broadcast_to(np.arange(r1 - r0)[:, None], ib.shape)
        np.add.at(dZ, (rr[inside], ib[inside] - v0), -(scale[r0:r1, None] * pb)[inside])
        dW += dZ.T @ h[r0:r1]
        if rows is None:
            dh[r0:r1] = dZ @ W_shard
        else:
            for j in np.nonzero(keep[r0:r1])[0]:
                dh[r0 + j] = dZ[j] @ W_shard
    if rows is not None:
        dh = np.array([dh[r] for r in np.asarray(rows)]).reshape(len(rows), d)
    return dh, dW

