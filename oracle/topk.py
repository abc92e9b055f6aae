"""CPU oracle for the teacher top-K cache producer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the test suite and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path.

The offline step runs the teacher once and keeps, for every position, its most
likely tokens with their scores; the pages keep the top 100 (thorstenmeyerai.com
article, TL;DR and infographic "Select top 100", "Write cache").  The student's
loss reads that cache as probabilities (aimodeling.com article, "First cut":
the teacher's top-100 probabilities for every token).  Written out in float64:

* ``lse_n = log sum_v exp(t[n, v])`` over the full vocabulary;
* the K positions with the largest logits, in decreasing order of logit, equal
  logits ordered by increasing token index (the pages do not say how ties are
  broken; this is the reading taken).  +0.0 and -0.0 are equal logits;
* ``p[n, k] = exp(t[n, idx[n, k]] - lse_n)``, the teacher's probability under its
  full softmax (no renormalisation over the K kept tokens, so ``sum_k p <= 1``,
  which is the mass M the loss uses).

A logit that is NaN or +inf, or a row with no finite logit, is an error.
"""
from __future__ import annotations

import numpy as np

__all__ = ["topk_probs"]


def topk_probs(logits, K: int):
    """Returns ``(idx [N, K] int32, p [N, K] float64, lse [N] float64)``."""
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("logits must be [N, V]")
    N, V = x.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    if np.isnan(x).any() or np.isposinf(x).any():
        raise ValueError("logit NaN or +inf")
    m = x.max(axis=1) if N else np.zeros(0)
    if N and not np.all(np.isfinite(m)):
        raise ValueError("row without a finite logit")
    # two-pass logsumexp per row
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1)) if N else np.zeros(0)
    # decreasing logit, ties by increasing index: a stable sort of -x keeps index order
    order = np.argsort(-x, axis=1, kind="stable")[:, :K]
    p = np.exp(np.take_along_axis(x, order, axis=1) - lse[:, None])
    return order.astype(np.int32), p, lse
