"""GPU parity of the backward into caller-owned fp32 accumulators
(lmhead_loss_bwd_accumulate): gradients of several calls sum in fp32, the
bf16 outputs are the casts of the accumulators, zero-initialised
accumulators reproduce the plain backward bit for bit, and micro-batches with
the global valid count reproduce the whole batch's gradient."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, dev_f32, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu


def _inputs(entry, **kw):
    d = dict(n=300, hidden=512, vocab=1000, chunk=512, seed=600 + entry, ignore_frac=0.1,
             entry=entry)
    if entry == wlmod.ENTRY_SUPPORT:
        d.update(k=16, ignore_frac=0.0)
    d.update(kw)
    return wlmod.make_inputs(wlmod.custom(**d))


def _forward(d, entry, chunk, num_valid=-1, rows=slice(None)):
    H = d.H[rows]
    if entry in (lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM):
        red = "mean" if entry == lm.ENTRY_CE_MEAN else "sum"
        loss, lse, _ = lm.ce_loss_forward(H, d.W, d.t[rows], chunk, red, num_valid)
        return dict(loss=loss, lse=lse, idx=d.t[rows], saved_lp=None)
    if entry == lm.ENTRY_LOGPROB:
        logp, lse, _ = lm.logprob_forward(H, d.W, d.t[rows], chunk)
        return dict(logp=logp, lse=lse, idx=d.t[rows], saved_lp=None)
    lp, kl, lse, _ = lm.support_forward(H, d.W, d.ids[rows], d.ref_logq[rows], chunk)
    return dict(lp=lp, kl=kl, lse=lse, idx=d.ids[rows], saved_lp=lp)


def _acc(d, entry, chunk, f, dH_acc, dW_acc, rows=slice(None), grad=None, num_valid=-1,
         out_bf16=True):
    g = d.grad if entry in (lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM) else d.grad[rows]
    if grad is not None:
        g = grad
    sup = entry == lm.ENTRY_SUPPORT
    return lm.backward_accumulate(entry, d.H[rows], d.W, f["idx"], f["lse"], g, chunk,
                                  dH_acc=dH_acc, dW_acc=dW_acc,
                                  ref_logq=d.ref_logq[rows] if sup else None,
                                  saved_lp=f["saved_lp"], grad_kl=d.grad_kl[rows] if sup else None,
                                  num_valid=num_valid, out_bf16=out_bf16)


@pytest.mark.parametrize("entry", [0, 2, 3])
def test_zero_accumulators_match_plain_bitwise(entry):
    inp = _inputs(entry)
    d = Dev(inp)
    plain = run_entry(d, entry, 512)
    f = _forward(d, entry, 512)
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    dH, dW = _acc(d, entry, 512, f, dH_acc, dW_acc)
    torch.cuda.synchronize()
    assert torch.equal(dH, plain["dH"]) and torch.equal(dW, plain["dW"])
    assert torch.equal(dH, dH_acc.to(torch.bfloat16)) and torch.equal(dW, dW_acc.to(torch.bfloat16))
    ref = oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad=inp.grad, grad_kl=inp.grad_kl)
    grad_check("dH_acc", to_np(dH_acc), ref["dH"])
    grad_check("dW_acc", to_np(dW_acc), ref["dW"])


def test_micro_batches_with_global_count_equal_the_whole_batch():
    """CE mean over two micro-batches, each given the global valid count: the
    losses add up to the whole batch's loss and dW_acc to its dW."""
    inp = _inputs(0)
    d = Dev(inp)
    count = int((inp.targets >= 0).sum())
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    loss = 0.0
    for rows in (slice(0, 160), slice(160, 300)):
        f = _forward(d, 0, 512, num_valid=count, rows=rows)
        loss += f["loss"].item()
        _acc(d, 0, 512, f, dH_acc[rows], dW_acc, rows=rows, num_valid=count, out_bf16=False)
    torch.cuda.synchronize()
    ref = oracle.run(0, inp.H, inp.W, targets=inp.targets, grad=inp.grad)
    rel_check("summed micro-batch loss", [loss], [ref["loss"]])
    grad_check("dH_acc", to_np(dH_acc), ref["dH"])
    grad_check("dW_acc", to_np(dW_acc), ref["dW"])


@pytest.mark.parametrize("entry", [1, 3])
def test_nonzero_initial_accumulators(entry):
    inp = _inputs(entry)
    d = Dev(inp)
    rng = np.random.default_rng(71 + entry)
    h0 = rng.normal(0, 1e-3, size=d.H.shape).astype(np.float32)
    w0 = rng.normal(0, 1e-3, size=d.W.shape).astype(np.float32)
    dH_acc, dW_acc = dev_f32(h0), dev_f32(w0)
    f = _forward(d, entry, 512)
    dH, dW = _acc(d, entry, 512, f, dH_acc, dW_acc)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH_acc.to(torch.bfloat16)) and torch.equal(dW, dW_acc.to(torch.bfloat16))
    ref = oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad=inp.grad, grad_kl=inp.grad_kl)
    grad_check("dH_acc - initial", to_np(dH_acc) - h0, ref["dH"])
    grad_check("dW_acc - initial", to_np(dW_acc) - w0, ref["dW"])


def test_two_losses_on_the_same_rows_add():
    """Gradient accumulation of two log-probability losses on one batch equals
    the gradient of their sum (the map grad -> dZ is linear)."""
    inp = _inputs(2)
    d = Dev(inp)
    rng = np.random.default_rng(5)
    g2 = rng.normal(0, 1, size=inp.wl.n).astype(np.float32)
    f = _forward(d, 2, 512)
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    _acc(d, 2, 512, f, dH_acc, dW_acc, out_bf16=False)
    _acc(d, 2, 512, f, dH_acc, dW_acc, grad=dev_f32(g2), out_bf16=False)
    torch.cuda.synchronize()
    ref = oracle.run(2, inp.H, inp.W, targets=inp.targets, grad=inp.grad + g2)
    grad_check("dH_acc", to_np(dH_acc), ref["dH"])
    grad_check("dW_acc", to_np(dW_acc), ref["dW"])


def test_frozen_side_and_empty_batch():
    inp = _inputs(0)
    d = Dev(inp)
    f = _forward(d, 0, 512)
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dH, dW = _acc(d, 0, 512, f, dH_acc, None)
    assert dW is None and torch.equal(dH, run_entry(d, 0, 512, need_dW=False)["dH"])
    # n = 0: the accumulator is unchanged and the bf16 output is its cast
    w0 = dev_f32(np.random.default_rng(3).normal(0, 1, size=d.W.shape).astype(np.float32))
    keep = w0.clone()
    H0 = d.H[:0]
    t0 = d.t[:0]
    lse0 = torch.empty(0, dtype=torch.float32, device="cuda")
    _, dW0 = lm.backward_accumulate(0, H0, d.W, t0, lse0, d.grad, 512, dW_acc=w0, out_bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(w0, keep) and torch.equal(dW0, keep.to(torch.bfloat16))


def test_accumulate_is_deterministic():
    inp = _inputs(3)
    d = Dev(inp)
    f = _forward(d, 3, 512)
    outs = []
    for _ in range(2):
        dH_acc = torch.full(d.H.shape, 0.5, dtype=torch.float32, device="cuda")
        dW_acc = torch.full(d.W.shape, -0.25, dtype=torch.float32, device="cuda")
        _acc(d, 3, 512, f, dH_acc, dW_acc, out_bf16=False)
        outs.append((dH_acc, dW_acc))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
