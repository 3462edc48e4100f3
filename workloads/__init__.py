"""Seeded synthetic inputs for the chunked LM-head + loss path.

This module only draws numbers. It holds none of the method's arithmetic
(no logits, no softmax, no loss): the fp64 oracle and the HIP library both
receive the exact bytes produced here, so it is the one piece of code the two
sides share.

Recipe (every draw comes from ``numpy.random.default_rng(seed)``, in this
order):

1. ``H``: fp32 standard normals, ``n * hidden`` of them, drawn in row blocks,
   rounded to bf16 with round-to-nearest-even.
2. ``W``: fp32 normals with standard deviation ``w_std`` (0.02), ``vocab *
   hidden`` of them, drawn in row blocks, rounded to bf16 the same way.
3. Labels:
   * ``uniform``: integers uniform in ``[0, vocab)``;
   * ``zipf``: ``P(v) proportional to (v + 1) ** -s`` over ids ``0..vocab-1``,
     sampled by inverse CDF from uniform floats.
4. Ignored rows: a seeded permutation of the rows; its first
   ``floor(ignore_frac * n)`` rows get ``ignore_index`` (-100).
5. Candidate ids (support entry): ``k`` distinct ids per row, uniform without
   replacement over ``[0, vocab)``; reference log-probabilities over those
   ``k`` candidates are the log-softmax of fp32 standard normals.
6. Upstream gradients: fp32 standard normals of the entry's output shape.

The configurations mirror the post-training workloads of the pages: a
Qwen-style 151,936-id vocabulary, a Llama-3-style 128,256-id vocabulary,
hidden sizes 2048 and 4096 and 4k to 16k tokens per call. The pages name no
public dataset, so these synthetic inputs stand in for real hidden states.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

IGNORE_INDEX = -100

# entry kinds (mirrored by the C ABI's entry enumeration)
ENTRY_CE_MEAN = 0
ENTRY_CE_SUM = 1
ENTRY_LOGPROB = 2
ENTRY_SUPPORT = 3
ENTRY_SUPPORT_KL = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    hidden: int
    vocab: int
    chunk: int
    seed: int
    entry: int = ENTRY_CE_MEAN
    labels: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 1.1
    ignore_frac: float = 0.0
    k: int = 1                        # candidates per row (support entry)
    w_std: float = 0.02
    pad_frac: float = 0.0             # padded candidate lists: mean fraction of padding slots

    @property
    def flops_fwd_bwd(self) -> float:
        """Dense MFMA work of one forward + backward: four n*vocab*hidden GEMMs."""
        return 8.0 * self.n * self.vocab * self.hidden


WORKLOADS = {
    "tiny": Workload("tiny", n=64, hidden=256, vocab=1024, chunk=256, seed=1001,
                     ignore_frac=0.10),
    "mid": Workload("mid", n=4096, hidden=2048, vocab=151936, chunk=8192, seed=1002,
                    labels="zipf", ignore_frac=0.05),
    "headline": Workload("headline", n=8192, hidden=4096, vocab=151936, chunk=8192,
                         seed=1003),
    "logprob": Workload("logprob", n=16384, hidden=4096, vocab=128256, chunk=8192,
                        seed=1004, entry=ENTRY_LOGPROB),
    "support": Workload("support", n=8192, hidden=4096, vocab=151936, chunk=8192,
                        seed=1005, entry=ENTRY_SUPPORT, k=64),
    # the headline's H, W and chunk at a small batch (256 rows: one row tile),
    # where the backward's dH contraction takes the K-split
    "small": Workload("small", n=256, hidden=4096, vocab=151936, chunk=8192, seed=1006),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite normals, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, rows: int, cols: int, std: float,
                 block_rows: int = 4096) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.uint16)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def _labels(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    if wl.labels == "uniform":
        t = rng.integers(0, wl.vocab, size=wl.n, dtype=np.int64)
    elif wl.labels == "zipf":
        w = np.arange(1, wl.vocab + 1, dtype=np.float64) ** (-wl.zipf_s)
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(wl.n)
        t = np.minimum(np.searchsorted(cdf, u, side="right"), wl.vocab - 1)
    else:
        raise ValueError(f"unknown label distribution {wl.labels!r}")
    t = t.astype(np.int32)
    n_ignore = int(math.floor(wl.ignore_frac * wl.n))
    perm = rng.permutation(wl.n)
    if n_ignore:
        t[perm[:n_ignore]] = IGNORE_INDEX
    return t


@dataclasses.dataclass
class Inputs:
    wl: Workload
    H: np.ndarray                      # uint16 bf16 bits [n, hidden]
    W: np.ndarray                      # uint16 bf16 bits [vocab, hidden]
    targets: Optional[np.ndarray]      # int32 [n] (CE / logprob)
    ids: Optional[np.ndarray]          # int32 [n, k] (support)
    ref_logq: Optional[np.ndarray]     # fp32 [n, k] (support)
    grad: np.ndarray                   # fp32: [1] CE, [n] logprob, [n, k] support
    grad_kl: Optional[np.ndarray]      # fp32 [n] (support)


def make_inputs(wl: Workload, *, with_W: bool = True) -> Inputs:
    """Draw one workload's inputs in the documented order."""
    rng = np.random.default_rng(wl.seed)
    H = _normal_bf16(rng, wl.n, wl.hidden, 1.0)
    if with_W:
        W = _normal_bf16(rng, wl.vocab, wl.hidden, wl.w_std)
    else:  # caller substitutes W; keep the stream position identical
        _ = _normal_bf16(rng, wl.vocab, wl.hidden, wl.w_std)
        W = None
    targets = ids = ref_logq = grad_kl = None
    if wl.entry in (ENTRY_CE_MEAN, ENTRY_CE_SUM, ENTRY_LOGPROB):
        targets = _labels(rng, wl)
    if wl.entry in (ENTRY_CE_MEAN, ENTRY_CE_SUM):
        grad = np.ones(1, dtype=np.float32)
    elif wl.entry == ENTRY_LOGPROB:
        grad = rng.standard_normal(wl.n, dtype=np.float32)
    else:
        ids = np.empty((wl.n, wl.k), dtype=np.int32)
        for i in range(wl.n):
            ids[i] = rng.choice(wl.vocab, size=wl.k, replace=False)
        g = rng.standard_normal((wl.n, wl.k)).astype(np.float64)
        g -= g.max(axis=1, keepdims=True)
        ref_logq = (g - np.log(np.exp(g).sum(axis=1, keepdims=True))).astype(np.float32)
        grad = rng.standard_normal((wl.n, wl.k), dtype=np.float32)
        grad_kl = rng.standard_normal(wl.n, dtype=np.float32)
        if wl.pad_frac > 0.0:
            # right-padded lists: row i keeps its first k - p_i ids, p_i ~ Binomial(k, pad_frac)
            pads = rng.binomial(wl.k, wl.pad_frac, size=wl.n)
            for i in range(wl.n):
                if pads[i]:
                    ids[i, wl.k - pads[i]:] = -1
    return Inputs(wl, H, W, targets, ids, ref_logq, grad, grad_kl)


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with explicit sizes (parity cases, edge cases)."""
    base = dict(n=64, hidden=256, vocab=1024, chunk=256, seed=7)
    base.update(kw)
    return Workload(name, **base)
