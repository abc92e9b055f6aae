"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``output_head_kl_amd/``).  It draws inputs and nothing else: it holds none
of the loss arithmetic (no log-softmax, no KL term, no gradient).

The workloads stand in for the ones the pages measure (no dataset or model
weights are used):

* the output-head-only toy benchmark swept from 4K to 256K tokens
  ("Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
  Chunked KL Loss", abstract; aimodeling.com article, section "Second cut");
* the 32,768-token single-GPU context (same article, "Second cut");
* the 201,088-entry gpt-oss vocabulary (thorstenmeyerai.com article, TL;DR);
* a teacher cache holding the top 100 tokens and their probabilities per
  position (aimodeling.com article, "First cut").

Recipe (one independent PCG64 stream per component, so that any component can
be drawn alone and in row blocks):

* ``h[N,d] ~ N(0,1)``;  ``W[V,d] = 2 * N(0, 1/d)`` (std ``2/sqrt(d)``);
* teacher indices: per row, K distinct tokens from Zipf(s) over ``[0,V)``,
  ``P(v) ∝ (v+1)^-s``, drawn one after another with repeats rejected; draw
  order is kept;
* teacher probabilities: K scores ``~ N(0, 2)`` (variance 2) sorted
  descending, soft-maxed, then scaled to a mass ``M ~ U(lo, hi)``; the k-th
  drawn index gets the k-th largest probability;
* loss mask: all ones, or packed sequences of length ``U{512..8192}`` whose
  first token is masked, optionally with the last ``round(0.1*len)`` positions
  of each sequence masked as right padding (~10% of positions).

bf16 inputs are rounded once, here, with round-to-nearest-even; both the GPU
path (which reads the 16-bit patterns) and the oracle (which reads their exact
float64 values) see the same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20260804

# Component ids for the per-component streams.
_H, _W, _IDX, _SCORES, _MASS, _LENGTHS, _SUBSET, _TEACHER = range(8)


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    N: int
    d: int
    V: int
    K: int
    chunk: int
    dtype: str          # "f32" or "bf16"
    zipf_s: float
    mass_lo: float
    mass_hi: float
    mask: str           # "ones" | "packed" | "packed_pad"


CONFIGS = {
    0: Config(0, "tiny_f32", 512, 256, 8192, 16, 128, "f32", 1.1, 0.8, 0.99, "ones"),
    1: Config(1, "bf16_4k", 4096, 3072, 128256, 100, 1024, "bf16", 1.1, 0.8, 0.99, "ones"),
    2: Config(2, "bf16_32k_packed", 32768, 3072, 128256, 100, 2048, "bf16", 1.1, 0.8, 0.99,
              "packed"),
    3: Config(3, "bf16_32k_vocab201k", 32768, 2880, 201088, 100, 2048, "bf16", 1.05, 0.85,
              0.995, "ones"),
    4: Config(4, "bf16_256k_packed_pad", 262144, 3072, 128256, 100, 4096, "bf16", 1.1, 0.8,
              0.99, "packed_pad"),
}


def config(cid: int, **overrides) -> Config:
    """Return config ``cid``, optionally with fields replaced (e.g. ``N=...``)."""
    return dataclasses.replace(CONFIGS[cid], **overrides)


def _rng(seed: int, component: int) -> np.random.Generator:
    return np.random.default_rng([seed, component])


# --------------------------------------------------------------------------
# bf16 representation (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


# --------------------------------------------------------------------------
# Dense inputs
# --------------------------------------------------------------------------
def _normal_rows(seed: int, component: int, rows: int, cols: int, scale: float,
                 row_lo: int = 0, row_hi: Optional[int] = None,
                 block: int = 8192) -> np.ndarray:
    """Rows ``[row_lo,row_hi)`` of a ``rows x cols`` matrix of ``scale*N(0,1)``.

    The matrix is drawn in fixed blocks of ``block`` rows, each block from its own
    stream, so any row range reproduces exactly the same values.
    """
    row_hi = rows if row_hi is None else row_hi
    out = np.empty((row_hi - row_lo, cols), dtype=np.float32)
    b0 = row_lo // block
    b1 = (row_hi + block - 1) // block
    for b in range(b0, b1):
        lo, hi = b * block, min(rows, (b + 1) * block)
        g = np.random.default_rng([seed, component, b])
        blk = g.standard_normal((hi - lo, cols), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        s0, s1 = max(lo, row_lo), min(hi, row_hi)
        out[s0 - row_lo:s1 - row_lo] = blk[s0 - lo:s1 - lo]
    return out


def make_h(cfg: Config, seed: int, row_lo: int = 0, row_hi: Optional[int] = None) -> np.ndarray:
    """Student hidden states ``h ~ N(0,1)``; float32, or uint16 bf16 bits for bf16 configs."""
    x = _normal_rows(seed, _H, cfg.N, cfg.d, 1.0, row_lo, row_hi)
    return f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x


def make_W(cfg: Config, seed: int) -> np.ndarray:
    """Output-projection weights ``W = 2*N(0,1/d)``; float32 or bf16 bits."""
    x = _normal_rows(seed, _W, cfg.V, cfg.d, 2.0 / np.sqrt(cfg.d))
    return f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x


# --------------------------------------------------------------------------
# Teacher top-K cache
# --------------------------------------------------------------------------
def _zipf_cdf(V: int, s: float) -> np.ndarray:
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def _distinct_in_order(cand: np.ndarray, K: int):
    """For each row of ``cand`` keep the first K distinct values, in draw order.

    Returns (out[B,K], ok[B]) where ok marks rows that had at least K distinct values.
    """
    B, m = cand.shape
    order = np.argsort(cand, axis=1, kind="stable")
    srt = np.take_along_axis(cand, order, axis=1)
    first_sorted = np.ones_like(srt, dtype=bool)
    first_sorted[:, 1:] = srt[:, 1:] != srt[:, :-1]
    first = np.empty_like(first_sorted)
    np.put_along_axis(first, order, first_sorted, axis=1)
    cnt = np.cumsum(first, axis=1)
    ok = cnt[:, -1] >= K
    keep = first & (cnt <= K)
    out = np.zeros((B, K), dtype=np.int64)
    if ok.any():
        out[ok] = cand[ok][keep[ok]].reshape(-1, K)
    return out, ok


def make_topk_idx(cfg: Config, seed: int, row_lo: int = 0,
                  row_hi: Optional[int] = None, block: int = 8192) -> np.ndarray:
    """Teacher indices ``[rows, K]`` int32: K distinct Zipf(s) draws per row."""
    row_hi = cfg.N if row_hi is None else row_hi
    cdf = _zipf_cdf(cfg.V, cfg.zipf_s)
    m = 8 * cfg.K if cfg.V > 8 * cfg.K else 4 * cfg.V
    out = np.empty((row_hi - row_lo, cfg.K), dtype=np.int32)
    for b in range(row_lo // block, (row_hi + block - 1) // block):
        lo, hi = b * block, min(cfg.N, (b + 1) * block)
        g = np.random.default_rng([seed, _IDX, b])
        u = g.random((hi - lo, m))
        cand = np.minimum(np.searchsorted(cdf, u, side="right"), cfg.V - 1)
        rows, ok = _distinct_in_order(cand, cfg.K)
        # Rows that did not reach K distinct draws keep drawing, one at a time.
        for r in np.nonzero(~ok)[0]:
            seen, seq = set(), []
            for v in cand[r]:
                if v not in seen:
                    seen.add(int(v)); seq.append(int(v))
            while len(seq) < cfg.K:
                v = int(min(np.searchsorted(cdf, g.random(), side="right"), cfg.V - 1))
                if v not in seen:
                    seen.add(v); seq.append(v)
            rows[r] = seq[:cfg.K]
        s0, s1 = max(lo, row_lo), min(hi, row_hi)
        out[s0 - row_lo:s1 - row_lo] = rows[s0 - lo:s1 - lo]
    return out


def make_topk_p(cfg: Config, seed: int, row_lo: int = 0,
                row_hi: Optional[int] = None, block: int = 8192) -> np.ndarray:
    """Teacher probabilities ``[rows, K]`` float32, descending, summing to M < 1."""
    row_hi = cfg.N if row_hi is None else row_hi
    out = np.empty((row_hi - row_lo, cfg.K), dtype=np.float32)
    for b in range(row_lo // block, (row_hi + block - 1) // block):
        lo, hi = b * block, min(cfg.N, (b + 1) * block)
        g = np.random.default_rng([seed, _SCORES, b])
        sc = -np.sort(-(np.sqrt(2.0) * g.standard_normal((hi - lo, cfg.K))), axis=1)
        e = np.exp(sc - sc[:, :1])
        q = e / e.sum(axis=1, keepdims=True)
        gm = np.random.default_rng([seed, _MASS, b])
        mass = gm.uniform(cfg.mass_lo, cfg.mass_hi, size=(hi - lo, 1))
        s0, s1 = max(lo, row_lo), min(hi, row_hi)
        out[s0 - row_lo:s1 - row_lo] = (q * mass)[s0 - lo:s1 - lo].astype(np.float32)
    return out


# --------------------------------------------------------------------------
# Loss mask
# --------------------------------------------------------------------------
def packed_lengths(cfg: Config, seed: int) -> np.ndarray:
    """Lengths of the packed sequences covering N tokens (last one truncated)."""
    g = _rng(seed, _LENGTHS)
    lens = []
    total = 0
    while total < cfg.N:
        n = int(g.integers(512, 8193))
        n = min(n, cfg.N - total)
        lens.append(n)
        total += n
    return np.asarray(lens, dtype=np.int64)


def make_mask(cfg: Config, seed: int) -> np.ndarray:
    """uint8 loss mask ``[N]`` (1 = token counts in the loss)."""
    mask = np.ones(cfg.N, dtype=np.uint8)
    if cfg.mask == "ones":
        return mask
    lens = packed_lengths(cfg, seed)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    mask[starts] = 0
    if cfg.mask == "packed_pad":
        for st, n in zip(starts, lens):
            pad = int(round(0.1 * n))
            if pad:
                mask[st + n - pad: st + n] = 0
    return mask


def subset_rows(cfg: Config, seed: int, count: int = 512) -> np.ndarray:
    """Sorted, distinct token rows sampled for full-size comparisons."""
    g = _rng(seed, _SUBSET)
    return np.sort(g.choice(cfg.N, size=min(count, cfg.N), replace=False)).astype(np.int64)


# --------------------------------------------------------------------------
# Whole workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Inputs:
    cfg: Config
    seed: int
    h: np.ndarray        # [N,d] float32, or uint16 bf16 bits
    W: np.ndarray        # [V,d] float32, or uint16 bf16 bits
    idx: np.ndarray      # [N,K] int32
    p: np.ndarray        # [N,K] float32
    mask: np.ndarray     # [N]   uint8

    def h64(self, rows=None) -> np.ndarray:
        h = self.h if rows is None else self.h[rows]
        return widen(h, self.cfg.dtype)

    def W64(self) -> np.ndarray:
        return widen(self.W, self.cfg.dtype)


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def make(cid: int, seed: Optional[int] = None, **overrides) -> Inputs:
    """Draw the full workload of config ``cid`` (fields may be overridden, e.g. N)."""
    cfg = config(cid, **overrides)
    seed = BASE_SEED + cid if seed is None else seed
    return Inputs(cfg, seed, make_h(cfg, seed), make_W(cfg, seed), make_topk_idx(cfg, seed),
                  make_topk_p(cfg, seed), make_mask(cfg, seed))


def take_rows(inp: Inputs, rows: np.ndarray) -> Inputs:
    """A sub-batch made of the given token rows (same W)."""
    cfg = dataclasses.replace(inp.cfg, N=len(rows))
    return Inputs(cfg, inp.seed, np.ascontiguousarray(inp.h[rows]), inp.W,
                  np.ascontiguousarray(inp.idx[rows]), np.ascontiguousarray(inp.p[rows]),
                  np.ascontiguousarray(inp.mask[rows]))


# --------------------------------------------------------------------------
# Teacher logits (input of the top-K cache producer)
# --------------------------------------------------------------------------
def make_teacher_logits(N: int, V: int, seed: int, dtype: str = "bf16", row_lo: int = 0,
                        row_hi: Optional[int] = None, sigma: float = 2.0,
                        alpha: float = 1.0, threads: int = 8) -> np.ndarray:
    """Rows ``[row_lo, row_hi)`` of synthetic teacher logits
    ``t[n, v] = sigma * N(0, 1) - alpha * log(v + 1)``.

    The ``-alpha log(v+1)`` term is a token-frequency prior (low token ids are the
    frequent ones, as with the Zipf-drawn cache indices), so each row's top tokens
    concentrate at low ids while the rest of the vocabulary is a Gaussian tail.
    Every row is drawn from its own stream, so any row subset is reproducible
    cheaply.  bf16 logits are returned as uint16 bits (rounded once, RNE), whose
    many exactly equal values exercise the tie rule of the top-K selection.
    """
    row_hi = N if row_hi is None else row_hi
    prior = (-alpha * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
    out = np.empty((row_hi - row_lo, V), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(r0, r1):
        for r in range(r0, r1):
            g = np.random.default_rng([seed, _TEACHER, r])
            x = g.standard_normal(V, dtype=np.float32)
            x *= np.float32(sigma)
            x += prior
            out[r - row_lo] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    n = row_hi - row_lo
    if n <= 64 or threads <= 1:
        fill(row_lo, row_hi)
    else:
        from concurrent.futures import ThreadPoolExecutor
        step = (n + threads - 1) // threads
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda i: fill(row_lo + i * step, min(row_hi, row_lo + (i + 1) * step)),
                        range(threads)))
    return out
