"""Helpers for the GPU tests: move seeded inputs to the device, run an entry
through the C ABI, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import chunked_lm_head_amd as lm

# Tolerances: loss, lse and log-probabilities within 2e-3 relative (absolute
# floor 1e-5 for values near 0: KL near its minimum, logp near 0); dH and dW
# within 2e-2 of the reference's largest magnitude, plus a relative-RMS gate
# of 1e-2 that a 2 % scale error fails (checked by a mutation test).
REL_TOL = 2e-3
ABS_FLOOR = 1e-5
GRAD_MAXABS_TOL = 2e-2
GRAD_RELRMS_TOL = 1e-2


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_i32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def dev_f32(a, device="cuda"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def to_np(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.float64)


def rel_check(name, got, ref, rel=REL_TOL, floor=ABS_FLOOR):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    bound = np.maximum(rel * np.abs(ref), floor)
    worst = np.argmax(err / bound) if err.size else 0
    assert np.all(err <= bound), (
        f"{name}: worst at {np.unravel_index(worst, err.shape)} got {got.flat[worst]!r} "
        f"ref {ref.flat[worst]!r} (|err| {err.flat[worst]:.3e} > {bound.flat[worst]:.3e})")
    return float((err / np.maximum(np.abs(ref), floor)).max()) if err.size else 0.0


def grad_check(name, got, ref, maxabs=GRAD_MAXABS_TOL, relrms=GRAD_RELRMS_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    if scale == 0.0:
        assert np.all(got == 0.0), f"{name}: expected exact zeros"
        return 0.0, 0.0
    e_max = np.abs(got - ref).max() / scale
    e_rms = np.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum())
    assert e_max <= maxabs, f"{name}: max-abs error {e_max:.3e} of max|ref| > {maxabs}"
    assert e_rms <= relrms, f"{name}: relative RMS error {e_rms:.3e} > {relrms}"
    return float(e_max), float(e_rms)


class Dev:
    """Seeded inputs of one workload on the GPU."""

    def __init__(self, inp, device="cuda"):
        self.inp = inp
        self.H = dev_bf16(inp.H, device)
        self.W = dev_bf16(inp.W, device)
        self.t = dev_i32(inp.targets, device) if inp.targets is not None else None
        self.ids = dev_i32(inp.ids, device) if inp.ids is not None else None
        self.ref_logq = dev_f32(inp.ref_logq, device)
        self.grad = dev_f32(inp.grad, device)
        self.grad_kl = dev_f32(inp.grad_kl, device)


def run_entry(d: Dev, entry: int, chunk: int, *, num_valid=-1, need_dH=True, need_dW=True,
              with_kl=True, stream=None, temperature=0.0, row_temperature=None):
    """Forward + backward of one entry through the C ABI. Returns torch outputs."""
    out = {}
    tk = dict(temperature=temperature, row_temperature=row_temperature)
    if entry in (lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM):
        red = "mean" if entry == lm.ENTRY_CE_MEAN else "sum"
        loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, chunk, red, num_valid, **tk)
        out.update(loss=loss, lse=lse)
        grad = d.grad
        idx, saved_lp, ref, gkl = d.t, None, None, None
    elif entry == lm.ENTRY_LOGPROB:
        logp, lse, _ = lm.logprob_forward(d.H, d.W, d.t, chunk, **tk)
        out.update(logp=logp, lse=lse)
        grad = d.grad
        idx, saved_lp, ref, gkl = d.t, None, None, None
    else:
        ref = d.ref_logq if with_kl else None
        lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, ref, chunk, **tk)
        out.update(lp=lp, kl=kl, lse=lse)
        grad = d.grad
        idx, saved_lp, gkl = d.ids, (lp if with_kl else None), (d.grad_kl if with_kl else None)
    if need_dH or need_dW:
        dH, dW = lm.backward(entry, d.H, d.W, idx, out["lse"], grad, chunk, ref_logq=ref,
                             saved_lp=saved_lp, grad_kl=gkl, num_valid=num_valid,
                             need_dH=need_dH, need_dW=need_dW, **tk)
        out.update(dH=dH, dW=dW)
    return out
