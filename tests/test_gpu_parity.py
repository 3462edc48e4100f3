"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element, on seeded inputs small enough for the full oracle but
spanning several 256 x 256 tiles, several vocabulary chunks and ragged tails;
plus bitwise determinism and the edge cases of the method."""
import math

import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import (Dev, bf16_to_np, grad_check, rel_check, run_entry, to_np)

pytestmark = pytest.mark.gpu


def _oracle(entry, inp, num_valid=-1, with_kl=True):
    return oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids,
                      ref_logq=inp.ref_logq if with_kl else None, grad=inp.grad,
                      grad_kl=inp.grad_kl if with_kl else None, num_valid=num_valid)


def _compare(entry, got, ref, label, inp=None):
    """Compare one entry's outputs with the oracle. With the inputs given, dW
    is checked a second time on the vocabulary rows that are no row's label or
    candidate, against their own largest magnitude: the label rows dominate
    max|ref|, so the first check alone would be loose for the others."""
    print(f"[{label}]", flush=True)
    rel_check(f"{label} lse", to_np(got["lse"]), ref["lse"])
    if entry in (lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM):
        rel_check(f"{label} loss", [got["loss"].item()], [ref["loss"]])
    elif entry == lm.ENTRY_LOGPROB:
        rel_check(f"{label} logp", to_np(got["logp"]), ref["logp"])
    else:
        rel_check(f"{label} lp", to_np(got["lp"]), ref["lp"])
        if "kl" in ref:
            rel_check(f"{label} kl", to_np(got["kl"]), ref["kl"])
    if got.get("dH") is not None:
        grad_check(f"{label} dH", bf16_to_np(got["dH"]), ref["dH"])
    if got.get("dW") is not None:
        gw = bf16_to_np(got["dW"])
        grad_check(f"{label} dW", gw, ref["dW"])
        if inp is not None:
            idx = inp.ids if entry == lm.ENTRY_SUPPORT else inp.targets
            other = np.ones(gw.shape[0], dtype=bool)
            other[idx[idx >= 0]] = False
            if other.any():
                grad_check(f"{label} dW (non-label rows)", gw[other], ref["dW"][other])


def _ragged(entry, **kw):
    d = dict(n=300, hidden=512, vocab=1000, chunk=512, seed=200 + entry, ignore_frac=0.1,
             entry=entry)
    if entry == wlmod.ENTRY_SUPPORT:
        d.update(k=16, ignore_frac=0.0)
    d.update(kw)
    return wlmod.make_inputs(wlmod.custom(**d))


# ------------------------------------------------------------------ parity

def test_tiny_config_ce_mean():
    wl = wlmod.WORKLOADS["tiny"]
    inp = wlmod.make_inputs(wl)
    got = run_entry(Dev(inp), lm.ENTRY_CE_MEAN, wl.chunk)
    _compare(lm.ENTRY_CE_MEAN, got, _oracle(lm.ENTRY_CE_MEAN, inp), "tiny", inp)


@pytest.mark.parametrize("entry", [0, 1, 2, 3])
def test_ragged_all_entries(entry):
    """n = 300 (two row tiles, ragged), V = 1000 (ragged last tile), chunk 512
    (two chunks, the second 488 wide), 10 % ignored rows."""
    inp = _ragged(entry)
    got = run_entry(Dev(inp), entry, 512)
    _compare(entry, got, _oracle(entry, inp), f"ragged entry {entry}", inp)


@pytest.mark.parametrize("shape", [
    dict(n=1, hidden=64, vocab=1, chunk=256),           # one logit: lse = z, loss 0
    dict(n=5, hidden=128, vocab=100, chunk=256),        # vocab below one tile
    dict(n=257, hidden=320, vocab=777, chunk=256),      # hidden not a multiple of 256
    dict(n=64, hidden=256, vocab=2048, chunk=4096),     # chunk larger than vocab
    dict(n=130, hidden=192, vocab=1537, chunk=768),     # three-tile chunks, 1-wide tail tile
    dict(n=70, hidden=65536, vocab=300, chunk=256),     # the largest hidden size accepted
])
def test_shapes_ce(shape):
    inp = wlmod.make_inputs(wlmod.custom(seed=300, ignore_frac=0.1, **shape))
    got = run_entry(Dev(inp), lm.ENTRY_CE_MEAN, shape["chunk"])
    _compare(0, got, _oracle(0, inp), f"shape {shape}", inp)


def test_support_without_kl():
    inp = _ragged(3)
    got = run_entry(Dev(inp), 3, 512, with_kl=False)
    ref = _oracle(3, inp, with_kl=False)
    assert got["kl"] is None
    _compare(3, got, ref, "support no KL", inp)


def test_given_count_and_sum():
    inp = _ragged(0)
    got = run_entry(Dev(inp), 0, 512, num_valid=1000)
    _compare(0, got, _oracle(0, inp, num_valid=1000), "given count 1000", inp)


# ----------------------------------------------------------- closed forms

def test_w_zero_closed_form_on_gpu():
    """W = 0: lse = ln V for every row, mean CE = ln V, dH = 0 exactly."""
    inp = wlmod.make_inputs(wlmod.custom(n=300, hidden=256, vocab=1000, chunk=512, seed=5,
                                         ignore_frac=0.1))
    inp.W[:] = 0
    d = Dev(inp)
    got = run_entry(d, 0, 512)
    lnV = math.log(1000)
    assert np.all(np.abs(to_np(got["lse"]) - lnV) <= 2e-6 * lnV)
    assert abs(got["loss"].item() - lnV) <= 2e-6 * lnV
    assert torch.all(got["dH"] == 0)
    ref = _oracle(0, inp)
    grad_check("W=0 dW", bf16_to_np(got["dW"]), ref["dW"])


def test_support_lp_equals_logprob_bitwise():
    """lp[n, k] and the logprob entry with t = id[n, k] come from the same
    tile partials and the same logit: bit-identical."""
    inp = _ragged(3)
    d = Dev(inp)
    lp, _, lse_s, _ = lm.support_forward(d.H, d.W, d.ids, None, 512)
    for k in (0, 7, 15):
        logp, lse_l, _ = lm.logprob_forward(d.H, d.W, d.ids[:, k].contiguous(), 512)
        assert torch.equal(lp[:, k], logp)
        assert torch.equal(lse_s, lse_l)


def test_logprobs_sum_to_one_on_gpu():
    """K = V candidates listing the whole vocabulary: sum_k exp(lp) = 1."""
    inp = wlmod.make_inputs(wlmod.custom(n=8, hidden=128, vocab=512, chunk=256, seed=9))
    d = Dev(inp)
    ids = torch.arange(512, dtype=torch.int32, device="cuda").repeat(8, 1).contiguous()
    lp, _, _, _ = lm.support_forward(d.H, d.W, ids, None, 256)
    s = torch.exp(lp.double()).sum(1)
    assert torch.all((s - 1).abs() < 1e-4), s


# ------------------------------------------------------------ determinism

def _digest(out):
    return {k: v.detach().cpu().clone() for k, v in out.items() if isinstance(v, torch.Tensor)}


@pytest.mark.parametrize("entry", [0, 2, 3])
def test_bitwise_repeat_and_side_stream(entry):
    inp = _ragged(entry)
    d = Dev(inp)
    a = _digest(run_entry(d, entry, 512))
    b = _digest(run_entry(d, entry, 512))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        c = _digest(run_entry(d, entry, 512))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), f"{k} differs between two runs"
        assert torch.equal(a[k], c[k]), f"{k} differs on a side stream"


# ------------------------------------------------------------ edge cases

def test_empty_call():
    inp = wlmod.make_inputs(wlmod.custom(n=0, hidden=128, vocab=300, chunk=256, seed=1))
    d = Dev(inp)
    loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, 256)
    assert loss.item() == 0.0 and lse.numel() == 0
    dH, dW = lm.backward(0, d.H, d.W, d.t, lse, d.grad, 256)
    torch.cuda.synchronize()
    assert dH.numel() == 0 and torch.all(dW == 0)


def test_all_rows_ignored():
    inp = wlmod.make_inputs(wlmod.custom(n=40, hidden=128, vocab=300, chunk=256, seed=2))
    inp.targets[:] = -100
    inp.targets[::3] = -7       # any negative label is ignored
    got = run_entry(Dev(inp), 0, 256)
    assert got["loss"].item() == 0.0
    assert torch.all(got["dH"] == 0) and torch.all(got["dW"] == 0)


def test_ignored_and_zero_grad_rows_get_exact_zero():
    inp = _ragged(2)
    inp.grad[::4] = 0.0
    got = run_entry(Dev(inp), 2, 512)
    dH = got["dH"].float().cpu().numpy()
    zero_rows = (inp.targets < 0) | (np.arange(300) % 4 == 0)
    assert np.all(dH[zero_rows] == 0.0)
    assert np.all(to_np(got["logp"])[inp.targets < 0] == 0.0)


def test_frozen_inputs():
    inp = _ragged(0)
    d = Dev(inp)
    full = run_entry(d, 0, 512)
    only_h = run_entry(d, 0, 512, need_dW=False)
    only_w = run_entry(d, 0, 512, need_dH=False)
    assert only_h["dW"] is None and only_w["dH"] is None
    assert torch.equal(full["dH"], only_h["dH"])
    assert torch.equal(full["dW"], only_w["dW"])


def test_label_out_of_range_is_flagged():
    inp = _ragged(0)
    inp.targets[17] = 1000
    inp.targets[230] = 5000
    d = Dev(inp)
    loss, lse, ws = lm.ce_loss_forward(d.H, d.W, d.t, 512)
    assert math.isnan(loss.item())
    code, row = lm.lmhead_read_device_error(ws)
    assert code == lm.DEVERR_LABEL and row == 17
    logp, _, ws2 = lm.logprob_forward(d.H, d.W, d.t, 512)
    lp = logp.cpu().numpy()
    assert np.isnan(lp[17]) and np.isnan(lp[230]) and np.all(np.isfinite(np.delete(lp, [17, 230])))
    dH, dW = lm.backward(lm.ENTRY_CE_MEAN, d.H, d.W, d.t, lse, d.grad, 512)  # grad: [1]
    dHn = dH.float().cpu().numpy()
    assert np.all(dHn[[17, 230]] == 0) and np.all(np.isfinite(dHn))
    assert torch.all(torch.isfinite(dW.float()))


def test_candidate_out_of_range_is_flagged():
    inp = _ragged(3)
    inp.ids[9, 3] = -1
    d = Dev(inp)
    lp, kl, lse, ws = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512)
    code, row = lm.lmhead_read_device_error(ws)
    assert code == lm.DEVERR_CANDIDATE and row == 9
    assert torch.all(torch.isnan(lp[9])) and torch.isnan(kl[9])
    assert torch.all(torch.isfinite(lp[10:]))


def test_mutation_gate_catches_two_percent():
    """The gradient gate rejects a 2 % scale error of a correct result."""
    inp = _ragged(0)
    got = run_entry(Dev(inp), 0, 512)
    ref = _oracle(0, inp)
    dW = bf16_to_np(got["dW"])
    grad_check("dW", dW, ref["dW"])
    with pytest.raises(AssertionError):
        grad_check("dW x1.02", dW * 1.02, ref["dW"])
    with pytest.raises(AssertionError):
        rel_check("loss x1.02", [got["loss"].item() * 1.02], [ref["loss"]])


def test_planned_chunk_against_oracle():
    """The smallest workspace as the budget (that of chunk 256): the planned
    chunk runs, fits, and matches the oracle (the result does not depend on
    the plan beyond rounding of the bf16 dL/dz operand). n = 300, V = 40000:
    that workspace already holds 256 tiles of dL/dz (32768 columns at two row
    tiles), so the planner takes the fewest passes within it, two chunks of
    20224 and 19776 columns."""
    inp = _ragged(0, hidden=256, vocab=40000)
    d = Dev(inp)
    p = lm.problem(inp.wl.n, inp.wl.hidden, inp.wl.vocab, 256)
    budget = lm.lmhead_workspace_size(p, 0, 1) + 1000
    chunk = lm.plan_chunk(inp.wl.n, inp.wl.hidden, inp.wl.vocab, budget)
    r = lm.memory_report(inp.wl.n, inp.wl.hidden, inp.wl.vocab, chunk, 0, True, 1)
    assert r["workspace_bytes"] <= budget
    assert (chunk, r["chunks"], r["dz_group"]) == (20224, 2, 1)
    H = d.H.clone().requires_grad_(True)
    W = d.W.clone().requires_grad_(True)
    loss = lm.ce_loss(H, W, d.t, memory_budget=budget)
    loss.backward()
    ref = _oracle(0, inp)
    rel_check("loss", [loss.item()], [ref["loss"]])
    grad_check("dH", bf16_to_np(H.grad), ref["dH"])
    grad_check("dW", bf16_to_np(W.grad), ref["dW"])


def test_binding_rejects_mismatched_shapes():
    """The torch helpers refuse targets / ids whose rows do not match H and
    side inputs of the wrong shape, before anything is launched."""
    inp = _ragged(0)
    d = Dev(inp)
    n = d.H.shape[0]
    with pytest.raises(ValueError, match="targets"):
        lm.ce_loss_forward(d.H, d.W, d.t[: n - 1], 512)
    with pytest.raises(ValueError, match="candidate ids"):
        lm.support_forward(d.H, d.W, d.t, None, 512)
    loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, 512)
    with pytest.raises(ValueError, match="grad"):
        lm.backward(lm.ENTRY_CE_MEAN, d.H, d.W, d.t, lse, torch.ones(2, device=d.H.device), 512)
    with pytest.raises(ValueError, match="lse"):
        lm.backward(lm.ENTRY_CE_MEAN, d.H, d.W, d.t, lse.double(), torch.ones(1, device=d.H.device),
                    512)
    torch.cuda.synchronize()


@pytest.mark.parametrize("entry", [0, 3])
def test_joint_dw_dh_launch_matches_separate_launches_bitwise(entry):
    """Small problems run a chunk's dW and dH tiles in one launch (the units
    one kind leaves idle take tiles of the other); a backward that wants only
    dH or only dW runs that kind's own kernel. Each tile is the same
    computation either way, so the results agree bit for bit."""
    inp = _ragged(entry)
    d = Dev(inp)
    both = run_entry(d, entry, 512)
    only_dh = run_entry(d, entry, 512, need_dW=False)
    only_dw = run_entry(d, entry, 512, need_dH=False)
    torch.cuda.synchronize()
    assert only_dh["dW"] is None and only_dw["dH"] is None
    assert torch.equal(both["dH"], only_dh["dH"])
    assert torch.equal(both["dW"], only_dw["dW"])
