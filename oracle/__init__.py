"""Plain, slow fp64 CPU oracle for the chunked LM-head + loss path.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. It shares no
code with the HIP library (``chunked_lm_head_amd``) and imports nothing from
it; the two meet only through the seeded inputs of ``workloads``.

What it computes is the plain, unchunked definition, in fp64, from the same
bf16 bytes the GPU receives (bf16 widens to fp64 exactly):

* logits ``z = H W^T`` (C loops in ``lmhead_oracle.c``);
* ``lse[n] = m + log sum_v exp(z[n, v] - m)``, ``m = max_v z[n, v]``;
* cross-entropy per row ``lse - z[n, t_n]``, mean over valid rows;
* per-token log-probability ``z[n, t_n] - lse``;
* support-set log-probabilities ``z[n, id_nk] - lse`` and
  ``KL(q_ref || p_hat)`` with ``p_hat`` the model renormalised over the K
  listed candidates, also as a KL-only entry and over padded candidate lists
  (a negative id is a padding slot that takes no part);
* backward: ``dZ = dL/dz`` from the textbook derivative of each entry, then
  ``dH = dZ W`` and ``dW = dZ^T H`` (C loops).

Sources: FlashInfer PR #8059 "det names for the chunked LM-head + loss
backend" (PR description: the backend covers CE and policy losses, the
log-probability entry and the support-set log-probability and KL entries;
CodeRabbit summary: candidate-restricted log-probabilities and forward KL);
miles-ext-kernels PR #14, the commit that declares the lm_head op (every
negative label marks an ignored row; a label >= V is an error; dW is the BF16
cast of an FP32 accumulator) and the commit that adds tests/cake/lm_head/
(given counts, zero-gradient rows, frozen inputs).

Readings where the pages are silent (each is listed in the design notes):
an empty valid set gives loss 0 and zero gradients; a given valid count is
used verbatim as the mean's denominator; the support entry has no ignored
rows; KL terms with q = 0 are 0; duplicate candidate ids count separately.

Parity pins: every function here is checked in ``tests/test_oracle.py``
against closed forms (W = 0), torch fp64 library routines, brute-force
pure-Python loops, finite differences and invariants.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build as _build

ENTRY_CE_MEAN = 0
ENTRY_CE_SUM = 1
ENTRY_LOGPROB = 2
ENTRY_SUPPORT = 3
ENTRY_SUPPORT_KL = 4

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        i64, vp, dp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        lib.oracle_logits.argtypes = [vp, ip, i64, i64, vp, i64, vp, ip, i64, dp, ip]
        lib.oracle_dh.argtypes = [dp, i64, vp, ip, i64, i64, dp, ip]
        lib.oracle_dw.argtypes = [dp, i64, vp, ip, i64, i64, vp, i64, dp, ip]
        for f in (lib.oracle_logits, lib.oracle_dh, lib.oracle_dw):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _operand(x: np.ndarray):
    """(array, is_f64) for a bf16-bits (uint16) or fp64 operand."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), 1
    raise TypeError(f"operand must be uint16 bf16 bits or float64, got {x.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- contractions

def logits(H: np.ndarray, W: np.ndarray, rows=None, threads: int = 0) -> np.ndarray:
    """z[i, v] = sum_h H[rows[i], h] W[v, h] in fp64 (all rows if rows is None)."""
    Hc, hf = _operand(H)
    Wc, wf = _operand(W)
    n, hd = Hc.shape
    V, hd2 = Wc.shape
    assert hd == hd2
    rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    z = np.empty((rows.size, V), dtype=np.float64)
    rc = _load().oracle_logits(_ptr(Hc), hf, n, hd, _ptr(rows), rows.size, _ptr(Wc), wf, V, _ptr(z), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_logits failed ({rc})")
    return z


def grad_hidden(dz: np.ndarray, W: np.ndarray, threads: int = 0) -> np.ndarray:
    """dH[i, h] = sum_v dz[i, v] W[v, h] in fp64."""
    Wc, wf = _operand(W)
    dz = np.ascontiguousarray(dz, dtype=np.float64)
    nr, V = dz.shape
    hd = Wc.shape[1]
    out = np.empty((nr, hd), dtype=np.float64)
    rc = _load().oracle_dh(_ptr(dz), nr, _ptr(Wc), wf, V, hd, _ptr(out), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_dh failed ({rc})")
    return out


def grad_weight(dz_cols: np.ndarray, H: np.ndarray, rows, threads: int = 0) -> np.ndarray:
    """dW[j, h] = sum_i dz_cols[i, j] H[rows[i], h] in fp64, rows ascending.

    ``dz_cols`` holds dL/dz for the selected vocabulary columns only
    ([len(rows), nv]); rows that do not appear contribute nothing.
    """
    Hc, hf = _operand(H)
    n, hd = Hc.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert np.all(np.diff(rows) > 0), "rows must be strictly ascending"
    dzt = np.ascontiguousarray(np.asarray(dz_cols, dtype=np.float64).T)
    nv = dzt.shape[0]
    out = np.empty((nv, hd), dtype=np.float64)
    rc = _load().oracle_dw(_ptr(dzt), nv, _ptr(Hc), hf, n, hd, _ptr(rows), rows.size, _ptr(out), threads)
    if rc != 0:
        raise RuntimeError(f"oracle_dw failed ({rc})")
    return out


# ------------------------------------------------------------ per-row definitions

def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """lse[i] = m + log(sum_v exp(z[i, v] - m)), m = max_v z[i, v]."""
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def check_targets(t: np.ndarray, vocab: int) -> np.ndarray:
    """valid[n] = 0 <= t[n] < V; any negative label is ignored; t >= V is an error."""
    t = np.asarray(t, dtype=np.int64)
    bad = np.nonzero(t >= vocab)[0]
    if bad.size:
        raise ValueError(f"label {int(t[bad[0]])} >= vocab {vocab} at row {int(bad[0])}")
    return t >= 0


def check_ids(ids: np.ndarray, vocab: int, padded: bool = False) -> np.ndarray:
    """Validates candidate ids; returns the mask of real (non-padding) slots.
    With padded lists a negative id is a padding slot; otherwise every id must
    lie in [0, vocab)."""
    bad = np.argwhere((ids >= vocab) | ((ids < 0) & (not padded)))
    if bad.size:
        r, k = bad[0]
        raise ValueError(f"candidate id {int(ids[r, k])} outside [0, {vocab}) at row {int(r)}")
    return ids >= 0


def _gather(z: np.ndarray, t: np.ndarray, valid: np.ndarray) -> np.ndarray:
    out = np.zeros(z.shape[0], dtype=np.float64)
    idx = np.nonzero(valid)[0]
    out[idx] = z[idx, t[idx]]
    return out


def ce_forward(z: np.ndarray, t: np.ndarray, num_valid: int = -1, reduction: str = "mean"):
    """Cross-entropy over all rows of z. Returns dict(loss, loss_rows, lse, count)."""
    vocab = z.shape[1]
    valid = check_targets(t, vocab)
    lse = logsumexp_rows(z)
    zt = _gather(z, np.asarray(t, dtype=np.int64), valid)
    loss_rows = np.where(valid, lse - zt, 0.0)
    count = int(valid.sum()) if num_valid < 0 else int(num_valid)
    total = float(loss_rows.sum())
    if reduction == "sum":
        loss = total
    else:
        loss = total / count if count > 0 else 0.0
    return dict(loss=loss, loss_rows=loss_rows, lse=lse, count=count, valid=valid)


def logprob_forward(z: np.ndarray, t: np.ndarray):
    """Per-token log-probability: logp[n] = z[n, t_n] - lse[n] (0 on ignored rows)."""
    vocab = z.shape[1]
    valid = check_targets(t, vocab)
    lse = logsumexp_rows(z)
    zt = _gather(z, np.asarray(t, dtype=np.int64), valid)
    return dict(logp=np.where(valid, zt - lse, 0.0), lse=lse, valid=valid)


def support_forward(z: np.ndarray, ids: np.ndarray, ref_logq: Optional[np.ndarray],
                    padded: bool = False):
    """Support-set log-probabilities and KL(q_ref || p_hat) over the K candidates.

    lp[n, k]      = z[n, id_nk] - lse[n]                  (full-vocabulary log-prob)
    log p_hat     = z[n, id_nk] - log sum_j exp z[n, id_nj] (renormalised over the K ids)
    KL[n]         = sum_k q_nk (ref_logq_nk - log p_hat_nk), q = exp(ref_logq), 0 where q = 0

    Padded lists (negative id = padding slot): a padding slot has lp = 0 and
    log p_hat = 0, and takes no part in the renormalisation or the KL sum; a
    row with no real candidate has KL = 0.
    """
    vocab = z.shape[1]
    ids = np.asarray(ids, dtype=np.int64)
    real = check_ids(ids, vocab, padded)
    lse = logsumexp_rows(z)
    zc = np.take_along_axis(z, np.where(real, ids, 0), axis=1)
    lp = np.where(real, zc - lse[:, None], 0.0)
    out = dict(lp=lp, lse=lse)
    if ref_logq is not None:
        r = np.asarray(ref_logq, dtype=np.float64)
        log_phat = np.zeros_like(zc)
        for n in range(zc.shape[0]):
            sel = real[n]
            if sel.any():
                v = zc[n, sel]
                m = v.max()
                log_phat[n, sel] = v - (m + np.log(np.exp(v - m).sum()))
        q = np.exp(r)
        terms = np.where(real & (q > 0.0), q * (r - log_phat), 0.0)
        out["kl"] = terms.sum(axis=1)
        out["log_phat"] = log_phat
    return out


def support_kl_forward(z: np.ndarray, ids: np.ndarray, ref_logq: np.ndarray,
                       padded: bool = False):
    """KL-only support entry: KL(q_ref || p_hat) and log p_hat; neither depends
    on logits outside the listed candidates."""
    f = support_forward(z, ids, ref_logq, padded)
    return dict(kl=f["kl"], log_phat=f["log_phat"])


# ----------------------------------------------------------------- derivatives

def softmax_rows(z: np.ndarray, lse: np.ndarray) -> np.ndarray:
    return np.exp(z - lse[:, None])


def ce_dz(z: np.ndarray, t: np.ndarray, grad: float, num_valid: int = -1,
          reduction: str = "mean") -> np.ndarray:
    """d(loss)/dz scaled by the upstream grad: (valid * g / count) (p - onehot(t))."""
    f = ce_forward(z, t, num_valid, reduction)
    valid, count = f["valid"], f["count"]
    if reduction == "sum":
        scale = np.where(valid, grad, 0.0)
    else:
        scale = np.where(valid, grad / count, 0.0) if count > 0 else np.zeros(z.shape[0])
    dz = scale[:, None] * softmax_rows(z, f["lse"])
    idx = np.nonzero(valid)[0]
    tt = np.asarray(t, dtype=np.int64)
    dz[idx, tt[idx]] -= scale[idx]
    return dz


def logprob_dz(z: np.ndarray, t: np.ndarray, grad: np.ndarray) -> np.ndarray:
    """d(sum_n grad_n logp_n)/dz = valid * grad_n (onehot(t) - p)."""
    f = logprob_forward(z, t)
    valid = f["valid"]
    g = np.where(valid, np.asarray(grad, dtype=np.float64), 0.0)
    dz = -g[:, None] * softmax_rows(z, f["lse"])
    idx = np.nonzero(valid)[0]
    tt = np.asarray(t, dtype=np.int64)
    dz[idx, tt[idx]] += g[idx]
    return dz


def support_dz(z: np.ndarray, ids: np.ndarray, ref_logq: Optional[np.ndarray],
               grad: Optional[np.ndarray], grad_kl: Optional[np.ndarray],
               padded: bool = False) -> np.ndarray:
    """d(sum grad * lp + sum grad_kl * KL)/dz.

    lp part:  sum_k g_nk ([v = id_nk] - p_nv)
    KL part:  b_n sum_k [v = id_nk] (Q_n p_hat_nk - q_nk),  Q_n = sum_k q_nk
    Padding slots (padded lists) contribute nothing and are not in Q_n.
    """
    n, vocab = z.shape
    ids = np.asarray(ids, dtype=np.int64)
    f = support_forward(z, ids, ref_logq, padded)
    real = ids >= 0
    safe = np.where(real, ids, 0)
    dz = np.zeros_like(z)
    rows = np.arange(n)
    if grad is not None:
        g = np.where(real, np.asarray(grad, dtype=np.float64), 0.0)
        dz -= g.sum(axis=1)[:, None] * softmax_rows(z, f["lse"])
        for k in range(ids.shape[1]):
            np.add.at(dz, (rows, safe[:, k]), g[:, k])
    if grad_kl is not None and ref_logq is not None:
        b = np.asarray(grad_kl, dtype=np.float64)
        q = np.where(real, np.exp(np.asarray(ref_logq, dtype=np.float64)), 0.0)
        Q = q.sum(axis=1)
        phat = np.where(real, np.exp(f["log_phat"]), 0.0)
        coef = b[:, None] * (Q[:, None] * phat - q)
        for k in range(ids.shape[1]):
            np.add.at(dz, (rows, safe[:, k]), coef[:, k])
    return dz


# ------------------------------------------------------------- whole-problem API

def temperature_scale(n: int, temperature: float = 0.0, row_temperature=None) -> np.ndarray:
    """Per-row temperature tau_n = t * r_n, with t = 1 when temperature is 0 (off) and
    r_n = 1 without a per-row array (miles-ext-kernels PR #14, tests/cake/lm_head/ commit:
    routes with the temperature off, scalar, per-row and 1.0). The method then works on
    the logits z / tau_n."""
    t = 1.0 if temperature == 0.0 else float(temperature)
    tau = np.full(n, t, dtype=np.float64)
    if row_temperature is not None:
        tau = tau * np.asarray(row_temperature, dtype=np.float64)
    if np.any(~(tau > 0)) or not np.all(np.isfinite(tau)):
        raise ValueError("temperature must be positive and finite")
    return tau


def run(entry: int, H: np.ndarray, W: np.ndarray, *, targets=None, ids=None, ref_logq=None,
        grad=None, grad_kl=None, num_valid: int = -1, backward: bool = True,
        temperature: float = 0.0, row_temperature=None, padded: bool = False,
        threads: int = 0) -> dict:
    """Full forward (+ backward) of one entry over every row. For small problems.

    With a temperature, every definition applies to z / tau_n, and the backward
    multiplies dL/d(z / tau) by 1 / tau_n (chain rule) before the contractions."""
    tau = temperature_scale(H.shape[0], temperature, row_temperature)
    z = logits(H, W, threads=threads) / tau[:, None]
    out: dict = {}
    if entry in (ENTRY_CE_MEAN, ENTRY_CE_SUM):
        red = "mean" if entry == ENTRY_CE_MEAN else "sum"
        f = ce_forward(z, targets, num_valid, red)
        out.update(loss=f["loss"], loss_rows=f["loss_rows"], lse=f["lse"], count=f["count"])
        if backward:
            g = 1.0 if grad is None else float(np.asarray(grad).reshape(-1)[0])
            dz = ce_dz(z, targets, g, num_valid, red)
    elif entry == ENTRY_LOGPROB:
        f = logprob_forward(z, targets)
        out.update(logp=f["logp"], lse=f["lse"])
        if backward:
            dz = logprob_dz(z, targets, grad)
    elif entry == ENTRY_SUPPORT:
        f = support_forward(z, ids, ref_logq, padded)
        out.update(lp=f["lp"], lse=f["lse"])
        if "kl" in f:
            out["kl"] = f["kl"]
            out["log_phat"] = f["log_phat"]
        if backward:
            dz = support_dz(z, ids, ref_logq, grad, grad_kl, padded)
    elif entry == ENTRY_SUPPORT_KL:
        f = support_kl_forward(z, ids, ref_logq, padded)
        out.update(kl=f["kl"], log_phat=f["log_phat"])
        if backward:
            dz = support_dz(z, ids, ref_logq, None, grad_kl, padded)
    else:
        raise ValueError(f"unknown entry {entry}")
    if backward:
        dz = dz / tau[:, None]
        out["dz"] = dz
        out["dH"] = grad_hidden(dz, W, threads=threads)
        out["dW"] = grad_weight(dz, H, np.arange(H.shape[0]), threads=threads)
    return out


def rows_forward_backward(entry: int, H: np.ndarray, W: np.ndarray, rows, *, targets=None,
                          ids=None, ref_logq=None, grad=None, grad_kl=None,
                          count: Optional[int] = None, temperature: float = 0.0,
                          row_temperature=None, padded: bool = False, threads: int = 0) -> dict:
    """Forward values and dH for a sample of rows, each computed over the whole vocabulary.

    Rows are independent except through the CE mean's denominator, which the
    caller passes as ``count`` (the number of valid rows of the full problem).
    """
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    tau = temperature_scale(H.shape[0], temperature, row_temperature)[rows]
    z = logits(H, W, rows, threads=threads) / tau[:, None]
    out: dict = {"rows": rows}
    if entry in (ENTRY_CE_MEAN, ENTRY_CE_SUM):
        t = np.asarray(targets)[rows]
        red = "mean" if entry == ENTRY_CE_MEAN else "sum"
        f = ce_forward(z, t, -1, red)
        out.update(lse=f["lse"], loss_rows=f["loss_rows"])
        g = 1.0 if grad is None else float(np.asarray(grad).reshape(-1)[0])
        if red == "mean":
            assert count is not None, "the CE mean needs the full problem's valid count"
            dz = ce_dz(z, t, g, int(count), "mean")
        else:
            dz = ce_dz(z, t, g, -1, "sum")
    elif entry == ENTRY_LOGPROB:
        t = np.asarray(targets)[rows]
        f = logprob_forward(z, t)
        out.update(lse=f["lse"], logp=f["logp"])
        dz = logprob_dz(z, t, np.asarray(grad)[rows])
    else:
        kl_only = entry == ENTRY_SUPPORT_KL
        ids_r = np.asarray(ids)[rows]
        ref_r = None if ref_logq is None else ref_logq[rows]
        f = support_forward(z, ids_r, ref_r, padded)
        if not kl_only:
            out.update(lse=f["lse"], lp=f["lp"])
        if "kl" in f:
            out.update(kl=f["kl"], log_phat=f["log_phat"])
        dz = support_dz(z, ids_r, ref_r,
                        None if (kl_only or grad is None) else np.asarray(grad)[rows],
                        None if grad_kl is None else np.asarray(grad_kl)[rows], padded)
    dz = dz / tau[:, None]
    out["dz"] = dz
    out["dH"] = grad_hidden(dz, W, threads=threads)
    return out

