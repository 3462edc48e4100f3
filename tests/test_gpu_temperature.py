"""GPU parity of the temperature-scaled path: every entry with a scalar
temperature, a per-row temperature and both together, against the fp64 oracle
at the same tolerances as the untempered path; tau = 1 reproduces the
untempered result bit for bit; a per-row temperature that is not positive and
finite is flagged on the device and gives that row NaN outputs and no gradient.
"""
import math

import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, dev_f32, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu


def _inputs(entry, **kw):
    d = dict(n=300, hidden=512, vocab=1000, chunk=512, seed=400 + entry, ignore_frac=0.1,
             entry=entry)
    if entry == wlmod.ENTRY_SUPPORT:
        d.update(k=16, ignore_frac=0.0)
    d.update(kw)
    return wlmod.make_inputs(wlmod.custom(**d))


def _row_temperature(n, seed):
    return np.random.default_rng(seed).uniform(0.5, 2.0, size=n).astype(np.float32)


def _check(entry, got, ref, label):
    print(f"[{label}]", flush=True)
    rel_check(f"{label} lse", to_np(got["lse"]), ref["lse"])
    if entry in (lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM):
        rel_check(f"{label} loss", [got["loss"].item()], [ref["loss"]])
    elif entry == lm.ENTRY_LOGPROB:
        rel_check(f"{label} logp", to_np(got["logp"]), ref["logp"])
    else:
        rel_check(f"{label} lp", to_np(got["lp"]), ref["lp"])
        rel_check(f"{label} kl", to_np(got["kl"]), ref["kl"])
    grad_check(f"{label} dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check(f"{label} dW", bf16_to_np(got["dW"]), ref["dW"])


@pytest.mark.parametrize("entry", [0, 1, 2, 3])
@pytest.mark.parametrize("mode", ["scalar", "per_row", "both"])
def test_temperature_against_oracle(entry, mode):
    inp = _inputs(entry)
    d = Dev(inp)
    t = {"scalar": 0.7, "per_row": 0.0, "both": 1.3}[mode]
    r = None if mode == "scalar" else _row_temperature(inp.wl.n, 77 + entry)
    got = run_entry(d, entry, inp.wl.chunk, temperature=t, row_temperature=dev_f32(r))
    ref = oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids,
                     ref_logq=inp.ref_logq, grad=inp.grad, grad_kl=inp.grad_kl,
                     temperature=t, row_temperature=r)
    _check(entry, got, ref, f"entry {entry} {mode}")


@pytest.mark.parametrize("entry", [0, 3])
def test_temperature_one_is_bitwise_untempered(entry):
    inp = _inputs(entry)
    d = Dev(inp)
    off = run_entry(d, entry, inp.wl.chunk)
    one = run_entry(d, entry, inp.wl.chunk, temperature=1.0)
    ones = run_entry(d, entry, inp.wl.chunk,
                     row_temperature=torch.ones(inp.wl.n, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    for k, v in off.items():
        if v is None:
            continue
        assert torch.equal(v, one[k]), f"temperature=1: {k} differs"
        assert torch.equal(v, ones[k]), f"row_temperature=1: {k} differs"


def test_temperature_changes_the_result():
    """A planted mistake that ignored the temperature would pass tau = 1 tests;
    this one sees it: the tempered loss must match the oracle's tempered loss and
    differ from the untempered one."""
    inp = _inputs(0)
    d = Dev(inp)
    a = run_entry(d, 0, 512, need_dH=False, need_dW=False)["loss"].item()
    b = run_entry(d, 0, 512, temperature=0.5, need_dH=False, need_dW=False)["loss"].item()
    ref = oracle.run(0, inp.H, inp.W, targets=inp.targets, temperature=0.5, backward=False)
    assert abs(a - b) > 1e-3 * abs(a)
    rel_check("tempered loss", [b], [ref["loss"]])


@pytest.mark.parametrize("bad", [0.0, -1.0, math.inf, math.nan])
def test_bad_row_temperature_is_flagged(bad):
    inp = _inputs(2)
    d = Dev(inp)
    r = _row_temperature(inp.wl.n, 5)
    r[41] = bad
    r[250] = bad
    rt = dev_f32(r)
    logp, lse, ws = lm.logprob_forward(d.H, d.W, d.t, 512, row_temperature=rt)
    code, row = lm.lmhead_read_device_error(ws)
    assert code == lm.DEVERR_TEMPERATURE and row == 41
    lp = logp.cpu().numpy()
    good = np.ones(inp.wl.n, dtype=bool)
    good[[41, 250]] = False
    assert np.all(np.isnan(lp[~good]))
    valid = good & (inp.targets >= 0)
    assert np.all(np.isfinite(lp[valid]))
    dH, dW = lm.backward(lm.ENTRY_LOGPROB, d.H, d.W, d.t, lse, d.grad, 512, row_temperature=rt)
    dHn = bf16_to_np(dH)
    assert np.all(dHn[~good] == 0.0) and np.all(np.isfinite(dHn))
    assert torch.all(torch.isfinite(dW.float()))
    # the other rows are those of the oracle with the bad rows carrying no gradient
    g = inp.grad.copy()
    g[~good] = 0.0
    r_ok = r.copy()
    r_ok[~good] = 1.0
    ref = oracle.run(2, inp.H, inp.W, targets=inp.targets, grad=g, row_temperature=r_ok)
    rel_check("logp good rows", lp[valid], ref["logp"][valid])
    grad_check("dH good rows", dHn[good], ref["dH"][good])
    grad_check("dW", bf16_to_np(dW), ref["dW"])


def test_bad_scalar_temperature_is_rejected_on_the_host():
    inp = _inputs(0)
    d = Dev(inp)
    ws = lm.workspace(lm.problem(inp.wl.n, inp.wl.hidden, inp.wl.vocab, 512), 0, False, "cuda")
    for t in (-0.5, math.inf, math.nan):
        with pytest.raises(lm.LMHeadError) as e:
            lm.ce_loss_forward(d.H, d.W, d.t, 512, ws=ws, temperature=t)
        assert e.value.status == lm.LMHEAD_ERR_ARG


def test_autograd_with_temperature():
    inp = _inputs(2, n=130, vocab=700)
    d = Dev(inp)
    r = _row_temperature(inp.wl.n, 9)
    H = d.H.clone().requires_grad_(True)
    W = d.W.clone().requires_grad_(True)
    logp = lm.logprob(H, W, d.t, 512, temperature=0.9, row_temperature=dev_f32(r))
    logp.backward(d.grad)
    ref = oracle.run(2, inp.H, inp.W, targets=inp.targets, grad=inp.grad, temperature=0.9,
                     row_temperature=r)
    rel_check("logp", to_np(logp), ref["logp"])
    grad_check("dH", bf16_to_np(H.grad), ref["dH"])
    grad_check("dW", bf16_to_np(W.grad), ref["dW"])
