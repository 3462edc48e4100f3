"""More edge cases of the method against the fp64 oracle: a single support
candidate per row, a vocabulary below one tile with padded candidate lists, a
one-column last chunk, the widest accepted chunk, every row sharing one
label, and the caller accumulators with a temperature."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, dev_f32, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu


def _ref(entry, inp, **kw):
    return oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids,
                      ref_logq=inp.ref_logq, grad=inp.grad, grad_kl=inp.grad_kl, **kw)


def _check(entry, got, ref):
    rel_check("lse", to_np(got["lse"]), ref["lse"])
    if entry == lm.ENTRY_SUPPORT:
        rel_check("lp", to_np(got["lp"]), ref["lp"])
        rel_check("kl", to_np(got["kl"]), ref["kl"])
    elif entry == lm.ENTRY_LOGPROB:
        rel_check("logp", to_np(got["logp"]), ref["logp"])
    else:
        rel_check("loss", [got["loss"].item()], [ref["loss"]])
    grad_check("dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("dW", bf16_to_np(got["dW"]), ref["dW"])


def test_single_candidate_per_row():
    """k = 1: p_hat = 1 for every row, so KL = q log q and its gradient
    reaches z only through the lp term."""
    inp = wlmod.make_inputs(wlmod.custom(n=200, hidden=256, vocab=900, chunk=512, seed=1600,
                                         entry=wlmod.ENTRY_SUPPORT, k=1))
    got = run_entry(Dev(inp), lm.ENTRY_SUPPORT, 512)
    torch.cuda.synchronize()
    _check(lm.ENTRY_SUPPORT, got, _ref(lm.ENTRY_SUPPORT, inp))


def test_vocab_below_one_tile_with_padded_lists():
    """V = 100 (one masked tile) and k = 32 padded lists, one row all padding."""
    inp = wlmod.make_inputs(wlmod.custom(n=90, hidden=192, vocab=100, chunk=256, seed=1601,
                                         entry=wlmod.ENTRY_SUPPORT, k=32, pad_frac=0.25))
    inp.ids[7, :] = -1
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 256, padded=True)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 256, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl, padded=True)
    torch.cuda.synchronize()
    ref = _ref(lm.ENTRY_SUPPORT, inp, padded=True)
    _check(lm.ENTRY_SUPPORT, dict(lse=lse, lp=lp, kl=kl, dH=dH, dW=dW), ref)


@pytest.mark.parametrize("entry", [0, 2])
def test_one_column_last_chunk(entry):
    """V = 513 with chunk 256: three chunks, the last one column wide."""
    inp = wlmod.make_inputs(wlmod.custom(n=260, hidden=320, vocab=513, chunk=256, seed=1602 + entry,
                                         entry=entry, ignore_frac=0.05))
    got = run_entry(Dev(inp), entry, 256)
    torch.cuda.synchronize()
    _check(entry, got, _ref(entry, inp))


def test_widest_chunk():
    """The widest chunk the shape check accepts, round_up(min(chunk, V), 256) =
    2^22 - 256 = 4,194,048 columns (V 300 columns wider: a second, 300-wide
    chunk follows). dL/dz is read with that row pitch, and a 256-row tile of
    it spans 2,147,352,576 bytes, just under the 2^31-byte buffer range the
    bound protects. n = 16: the bound depends on the pitch and the 256-row
    tile only."""
    cap = (1 << 22) - 256
    inp = wlmod.make_inputs(wlmod.custom(n=16, hidden=64, vocab=cap + 300, chunk=cap, seed=1606,
                                         ignore_frac=0.1))
    got = run_entry(Dev(inp), lm.ENTRY_CE_MEAN, cap)
    torch.cuda.synchronize()
    _check(lm.ENTRY_CE_MEAN, got, _ref(lm.ENTRY_CE_MEAN, inp))


def test_every_row_has_the_same_label():
    """All labels equal: one dW row collects every row's -1 term."""
    inp = wlmod.make_inputs(wlmod.custom(n=300, hidden=256, vocab=700, chunk=512, seed=1604,
                                         entry=wlmod.ENTRY_LOGPROB))
    inp.targets[:] = 417
    got = run_entry(Dev(inp), lm.ENTRY_LOGPROB, 512)
    torch.cuda.synchronize()
    _check(lm.ENTRY_LOGPROB, got, _ref(lm.ENTRY_LOGPROB, inp))


def test_accumulators_with_temperature():
    """Caller fp32 accumulators under a per-row temperature: the accumulated
    gradients equal the oracle's tempered gradients plus the initial values."""
    inp = wlmod.make_inputs(wlmod.custom(n=270, hidden=256, vocab=800, chunk=512, seed=1605,
                                         entry=wlmod.ENTRY_CE_SUM, ignore_frac=0.1))
    d = Dev(inp)
    rng = np.random.default_rng(1606)
    rt = rng.uniform(0.5, 2.0, size=270).astype(np.float32)
    rt_d = dev_f32(rt)
    loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, 512, "sum", temperature=1.3, row_temperature=rt_d)
    h0 = rng.standard_normal((270, 256)).astype(np.float32)
    w0 = rng.standard_normal((800, 256)).astype(np.float32)
    dH_acc, dW_acc = dev_f32(h0), dev_f32(w0)
    lm.backward_accumulate(lm.ENTRY_CE_SUM, d.H, d.W, d.t, lse, d.grad, 512, dH_acc=dH_acc,
                           dW_acc=dW_acc, temperature=1.3, row_temperature=rt_d)
    torch.cuda.synchronize()
    ref = oracle.run(lm.ENTRY_CE_SUM, inp.H, inp.W, targets=inp.targets, grad=inp.grad,
                     temperature=1.3, row_temperature=rt)
    rel_check("loss", [loss.item()], [ref["loss"]])
    rel_check("lse", to_np(lse), ref["lse"])
    grad_check("dH_acc - initial", to_np(dH_acc) - h0.astype(np.float64), ref["dH"])
    grad_check("dW_acc - initial", to_np(dW_acc) - w0.astype(np.float64), ref["dW"])
