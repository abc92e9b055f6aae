"""CPU oracle for the fused chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
package: only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP path.

It is the plain dense definition of the loss, written out in float64 with
numpy, so that a reader can check it against the pages by eye:

* The student's logits are the output projection of its last hidden states,
  ``Z = h @ W.T`` (the fused loss "joins the student model's output projection
  to the loss calculation": thorstenmeyerai.com article, TL;DR; aimodeling.com
  article, "Second cut": "output projection, normalization, and sparse teacher
  terms").
* The teacher is a cache of its top-K tokens and their probabilities per
  position (aimodeling.com article, "First cut": top-100 probabilities per
  token; thorstenmeyerai.com infographic, "Select top 100").
* The per-token loss is the KL term over the teacher's K support positions,
  ``l_n = sum_k p_k (log p_k - log q_{idx_k})`` with ``q = softmax(Z_n)``.
  The pages name the loss a KL over the cached top-K and give its gradient in
  words only (legiblepapers.com summary, Cross-Examination Q5); this is the
  forward-KL form whose gradient is that one.  No renormalisation of p, no
  tail term for the missing mass ``1 - M``, temperature 1, ``0 log 0 = 0``.
* The reduction is the mean over tokens whose loss mask is nonzero; with no
  such token the loss and both gradients are zero.
* The gradient with respect to the logits is the closed form the pages
  describe: a dense ``M * softmax`` term minus the sparse teacher correction at
  the top-K support positions (legiblepapers.com summary, Q5), where
  ``M_n = sum_k p_k``; repeated indices in a row add up (scatter-add).
  ``dh = dZ @ W`` and ``dW = dZ.T @ h``.
* The fused, chunked and dense implementations compute the same thing
  (thorstenmeyerai.com article, "Quality and Generality Need Testing": the
  three loss implementations are mathematically equivalent), so the dense
  definition is the reference for the chunked GPU path.

Rows are independent, so the sum over tokens is split into row blocks only to
bound host memory; ``block_rows`` changes nothing but rounding order.
"""
from __future__ import annotations

import numpy as np

__all__ = ["check_inputs", "forward_backward", "rows_forward_backward", "loss_only"]


def check_inputs(idx: np.ndarray, p: np.ndarray, V: int) -> None:
    """Reject indices outside ``[0, V)`` and probabilities that are negative or not finite."""
    idx = np.asarray(idx)
    p = np.asarray(p, dtype=np.float64)
    if idx.size and (idx.min() < 0 or idx.max() >= V):
        raise ValueError("teacher index out of range")
    if not np.all(np.isfinite(p)):
        raise ValueError("teacher probability not finite")
    if p.size and p.min() < 0:
        raise ValueError("teacher probability negative")


def _block(Hb, W, idx_b, p_b, scale_b):
    """All per-token quantities of one row block (float64).

    ``scale_b[n] = mask_n / count`` is the token's weight in the mean.
    Returns (row_loss, row_lse, zg, dZ) where row_loss is the unweighted l_n.
    """
    Z = Hb @ W.T                                           # [b, V] student logits
    m = Z.max(axis=1)
    lse = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))  # log sum_v exp Z[n, v]
    logq = Z - lse[:, None]                                # log softmax
    logq_at = np.take_along_axis(logq, idx_b, axis=1)      # log q at the teacher's tokens
    safe_p = np.where(p_b > 0, p_b, 1.0)
    plogp = np.where(p_b > 0, p_b * np.log(safe_p), 0.0)   # 0 log 0 = 0
    ell = (plogp - p_b * logq_at).sum(axis=1)              # sum_k p_k (log p_k - log q_idx_k)
    zg = np.take_along_axis(Z, idx_b, axis=1)              # logits at the teacher's tokens

    # dL/dZ = scale * (M * softmax(Z) - scatter_add(p at idx))
    M = p_b.sum(axis=1)
    dZ = (scale_b * M)[:, None] * np.exp(logq)
    rows = np.broadcast_to(np.arange(Hb.shape[0])[:, None], idx_b.shape)
    np.add.at(dZ, (rows, idx_b), -(scale_b[:, None] * p_b))
    return ell, lse, zg, dZ


def forward_backward(h, W, idx, p, mask=None, block_rows: int = 256):
    """Loss, gradients and per-row outputs for the whole batch.

    Args:
      h: [N, d] hidden states; W: [V, d] output projection (any float type, used as float64).
      idx: [N, K] teacher token indices; p: [N, K] teacher probabilities.
      mask: [N] loss mask (nonzero = counts), or None for all ones.
    Returns a dict with ``loss`` (float), ``dh`` [N,d], ``dW`` [V,d], ``row_loss`` [N]
    (``l_n`` where the mask is set, else 0), ``row_lse`` [N], ``zg`` [N,K], ``count``.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    p = np.asarray(p, dtype=np.float64)
    N, d = h.shape
    V = W.shape[0]
    check_inputs(idx, p, V)
    mask = np.ones(N, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    count = int(mask.sum())
    out = dict(loss=0.0, dh=np.zeros((N, d)), dW=np.zeros((V, d)), row_loss=np.zeros(N),
               row_lse=np.zeros(N), zg=np.zeros(idx.shape), count=count)
    scale = mask / count if count else np.zeros(N)
    total = 0.0
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        ell, lse, zg, dZ = _block(h[r0:r1], W, idx[r0:r1], p[r0:r1], scale[r0:r1])
        out["row_lse"][r0:r1] = lse
        out["zg"][r0:r1] = zg
        out["row_loss"][r0:r1] = np.where(mask[r0:r1], ell, 0.0)
        if count:
            total += float(np.sum(np.where(mask[r0:r1], ell, 0.0)))
            out["dh"][r0:r1] = dZ @ W
            out["dW"] += dZ.T @ h[r0:r1]
    out["loss"] = total / count if count else 0.0
    return out


def rows_forward_backward(h_rows, W, idx_rows, p_rows, mask_rows, count: int,
                          block_rows: int = 128):
    """Per-row outputs for selected token rows of a larger batch.

    ``count`` is the number of unmasked tokens in the whole batch (it sets each
    row's weight ``mask/count``).  Returns ``row_loss``, ``row_lse``, ``zg`` and
    the rows of ``dh``; ``dW`` needs every row and is not returned.
    """
    h_rows = np.asarray(h_rows, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    idx_rows = np.asarray(idx_rows, dtype=np.int64)
    p_rows = np.asarray(p_rows, dtype=np.float64)
    check_inputs(idx_rows, p_rows, W.shape[0])
    mask_rows = np.asarray(mask_rows) != 0
    n = h_rows.shape[0]
    scale = mask_rows / count if count else np.zeros(n)
    res = dict(row_loss=np.zeros(n), row_lse=np.zeros(n), zg=np.zeros(idx_rows.shape),
               dh=np.zeros(h_rows.shape))
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        ell, lse, zg, dZ = _block(h_rows[r0:r1], W, idx_rows[r0:r1], p_rows[r0:r1],
                                  scale[r0:r1])
        res["row_loss"][r0:r1] = np.where(mask_rows[r0:r1], ell, 0.0)
        res["row_lse"][r0:r1] = lse
        res["zg"][r0:r1] = zg
        res["dh"][r0:r1] = dZ @ W
    return res


def loss_only(h, W, idx, p, mask=None) -> float:
    """The mean loss alone (used by finite-difference checks)."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    p = np.asarray(p, dtype=np.float64)
    N = h.shape[0]
    mask = np.ones(N, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    count = int(mask.sum())
    if count == 0:
        return 0.0
    ell, _, _, _ = _block(h, W, idx, p, mask / count)
    return float(np.sum(np.where(mask, ell, 0.0)) / count)
