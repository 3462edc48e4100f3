"""GPU parity of the split support entries and padded candidate lists:
lmhead_support_logprob (lp without KL), lmhead_support_kl (the KL-only entry,
computed from candidate gathers without a vocabulary-wide pass) and
LMHEAD_FLAG_PADDED_IDS, against the fp64 oracle; plus their edge cases and
bitwise determinism (the KL-only dW orders its sums by a counting sort)."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, dev_f32, dev_i32, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu


def _inputs(**kw):
    d = dict(n=300, hidden=512, vocab=1000, chunk=512, seed=700, entry=wlmod.ENTRY_SUPPORT, k=16)
    d.update(kw)
    return wlmod.make_inputs(wlmod.custom(**d))


def _kl_only(d, padded=False, temperature=0.0, row_temperature=None, acc=None):
    kl, lph, ws = lm.support_kl_forward(d.H, d.W, d.ids, d.ref_logq, padded=padded,
                                        temperature=temperature, row_temperature=row_temperature)
    if acc is None:
        dH, dW = lm.backward(lm.ENTRY_SUPPORT_KL, d.H, d.W, d.ids, None, None, 256,
                             ref_logq=d.ref_logq, saved_lp=lph, grad_kl=d.grad_kl, padded=padded,
                             temperature=temperature, row_temperature=row_temperature)
    else:
        dH, dW = lm.backward_accumulate(lm.ENTRY_SUPPORT_KL, d.H, d.W, d.ids, None, None, 256,
                                        dH_acc=acc[0], dW_acc=acc[1], ref_logq=d.ref_logq,
                                        saved_lp=lph, grad_kl=d.grad_kl, padded=padded,
                                        out_bf16=True)
    return dict(kl=kl, log_phat=lph, dH=dH, dW=dW, ws=ws)


def test_support_logprob_entry_equals_lp_of_the_combined_entry():
    inp = _inputs()
    d = Dev(inp)
    lp, lse, _ = lm.support_logprob_forward(d.H, d.W, d.ids, 512)
    lp2, kl2, lse2, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp2) and torch.equal(lse, lse2)
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, grad=inp.grad)
    rel_check("lp", to_np(lp), ref["lp"])
    # autograd through the lp-only function
    H = d.H.clone().requires_grad_(True)
    W = d.W.clone().requires_grad_(True)
    lm.support_logprob(H, W, d.ids, 512).backward(d.grad)
    grad_check("dH", bf16_to_np(H.grad), ref["dH"])
    grad_check("dW", bf16_to_np(W.grad), ref["dW"])


# 1024 and 3072 take the forward path that keeps the row of H in registers
# (hidden a multiple of 1024, at most 4096); the others stream H with W
@pytest.mark.parametrize("hidden", [512, 192, 1088, 1024, 3072])
def test_kl_only_against_oracle(hidden):
    inp = _inputs(hidden=hidden, seed=710 + hidden)
    inp.ids[7, 3] = inp.ids[7, 0]          # a duplicate id: two entries in one dW bucket
    d = Dev(inp)
    got = _kl_only(d)
    torch.cuda.synchronize()
    ref = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl)
    rel_check("kl", to_np(got["kl"]), ref["kl"])
    rel_check("log p_hat", to_np(got["log_phat"]), ref["log_phat"])
    grad_check("dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("dW", bf16_to_np(got["dW"]), ref["dW"])
    # vocabulary rows no candidate names get exactly zero
    named = np.zeros(inp.wl.vocab, dtype=bool)
    named[inp.ids.ravel()] = True
    assert torch.all(got["dW"][torch.from_numpy(~named).cuda()] == 0)


def test_kl_only_matches_the_dense_entry():
    """The gather path and the dense path compute the same KL (two summation
    orders of the same products): agreement far inside the oracle tolerance."""
    inp = _inputs(seed=720)
    d = Dev(inp)
    got = _kl_only(d)
    _, kl, _, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512)
    torch.cuda.synchronize()
    rel_check("kl gather vs dense", to_np(got["kl"]), to_np(kl), rel=2e-4, floor=1e-6)


@pytest.mark.parametrize("hidden", [512, 2048])
def test_kl_only_with_temperature_and_autograd(hidden):
    inp = _inputs(hidden=hidden, seed=730)
    d = Dev(inp)
    r = np.random.default_rng(4).uniform(0.5, 2.0, size=inp.wl.n).astype(np.float32)
    rt = dev_f32(r)
    H = d.H.clone().requires_grad_(True)
    W = d.W.clone().requires_grad_(True)
    kl = lm.support_kl(H, W, d.ids, d.ref_logq, temperature=0.8, row_temperature=rt)
    kl.backward(d.grad_kl)
    ref = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl, temperature=0.8, row_temperature=r)
    rel_check("kl", to_np(kl), ref["kl"])
    grad_check("dH", bf16_to_np(H.grad), ref["dH"])
    grad_check("dW", bf16_to_np(W.grad), ref["dW"])


@pytest.mark.parametrize("hidden", [512, 2048])
def test_padded_lists_dense_and_kl_only(hidden):
    inp = _inputs(hidden=hidden, seed=740, pad_frac=0.3)
    inp.ids[11, :] = -1                    # a row with no real candidate
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512, padded=True)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 512, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl, padded=True)
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq, grad=inp.grad,
                     grad_kl=inp.grad_kl, padded=True)
    rel_check("padded lp", to_np(lp), ref["lp"])
    rel_check("padded kl", to_np(kl), ref["kl"])
    assert torch.all(lp[d.ids < 0] == 0) and kl[11].item() == 0.0
    grad_check("padded dH", bf16_to_np(dH), ref["dH"])
    grad_check("padded dW", bf16_to_np(dW), ref["dW"])
    got = _kl_only(d, padded=True)
    refk = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                      grad_kl=inp.grad_kl, padded=True)
    rel_check("padded KL-only kl", to_np(got["kl"]), refk["kl"])
    rel_check("padded log p_hat", to_np(got["log_phat"]), refk["log_phat"])
    grad_check("padded KL-only dH", bf16_to_np(got["dH"]), refk["dH"])
    grad_check("padded KL-only dW", bf16_to_np(got["dW"]), refk["dW"])
    assert torch.all(got["dH"][11] == 0)


def test_id_errors_with_and_without_padding():
    inp = _inputs(seed=750)
    inp.ids[20, 5] = -1
    inp.ids[40, 2] = inp.wl.vocab
    d = Dev(inp)
    # unpadded: both rows are errors, the lowest is reported
    lp, kl, _, ws = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512)
    code, row = lm.lmhead_read_device_error(ws)
    assert code == lm.DEVERR_CANDIDATE and row == 20
    assert torch.isnan(kl[20]) and torch.isnan(kl[40]) and torch.isfinite(kl[21])
    # padded: -1 is padding, the id >= V is still an error
    lp, kl, _, ws = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512, padded=True)
    code, row = lm.lmhead_read_device_error(ws)
    assert code == lm.DEVERR_CANDIDATE and row == 40
    assert torch.isfinite(kl[20]) and torch.isnan(kl[40])
    kl2, lph, ws2 = lm.support_kl_forward(d.H, d.W, d.ids, d.ref_logq, padded=True)
    code, row = lm.lmhead_read_device_error(ws2)
    assert code == lm.DEVERR_CANDIDATE and row == 40
    assert torch.isnan(kl2[40]) and torch.all(torch.isnan(lph[40]))
    dH, dW = lm.backward(lm.ENTRY_SUPPORT_KL, d.H, d.W, d.ids, None, None, 256, ref_logq=d.ref_logq,
                         saved_lp=lph, grad_kl=d.grad_kl, padded=True)
    assert torch.all(dH[40] == 0) and torch.all(torch.isfinite(dW.float()))


def test_kl_only_bitwise_repeat_and_accumulate():
    inp = _inputs(seed=760, n=513, k=64, vocab=700)   # many entries per dW bucket
    d = Dev(inp)
    a = _kl_only(d)
    b = _kl_only(d)
    torch.cuda.synchronize()
    for key in ("kl", "log_phat", "dH", "dW"):
        assert torch.equal(a[key], b[key]), key
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    c = _kl_only(d, acc=(dH_acc, dW_acc))
    torch.cuda.synchronize()
    assert torch.equal(c["dH"], a["dH"]) and torch.equal(c["dW"], a["dW"])
    ref = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl)
    grad_check("dW_acc", to_np(dW_acc), ref["dW"])


def test_kl_only_empty_call():
    inp = _inputs(seed=770)
    d = Dev(inp)
    kl, lph, _ = lm.support_kl_forward(d.H[:0], d.W, d.ids[:0], d.ref_logq[:0])
    assert kl.numel() == 0
    dW = torch.full_like(d.W, 7.0)
    lm.backward(lm.ENTRY_SUPPORT_KL, d.H[:0], d.W, d.ids[:0], None, None, 256,
                ref_logq=d.ref_logq[:0], saved_lp=lph, grad_kl=d.grad_kl[:0], need_dH=False,
                dW=dW)
    torch.cuda.synchronize()
    assert torch.all(dW == 0)


def test_kl_only_full_size_sampled():
    """The support workload's sizes (N = 8192, K = 64, V = 151936): KL and dH
    on sampled rows, dW on sampled vocabulary rows (each from the rows that
    list it), against the oracle."""
    wl = wlmod.WORKLOADS["support"]
    inp = wlmod.make_inputs(wl)
    d = Dev(inp)
    got = _kl_only(d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed + 31)
    rows = np.sort(rng.choice(wl.n, size=6, replace=False))
    ref = oracle.rows_forward_backward(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, rows, ids=inp.ids,
                                       ref_logq=inp.ref_logq, grad_kl=inp.grad_kl, threads=16)
    rel_check("kl rows", to_np(got["kl"])[rows], ref["kl"])
    grad_check("dH rows", bf16_to_np(got["dH"][torch.from_numpy(rows).cuda()]), ref["dH"])
    vs = np.unique(inp.ids[rows[:3], :2].ravel())          # vocabulary rows some sampled row lists
    for v in vs:
        listing = np.nonzero((inp.ids == v).any(axis=1))[0]
        rv = oracle.rows_forward_backward(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, listing,
                                          ids=inp.ids, ref_logq=inp.ref_logq, grad_kl=inp.grad_kl,
                                          threads=16)
        dw_ref = oracle.grad_weight(rv["dz"][:, [v]], inp.H, listing, threads=16)
        grad_check(f"dW row {v}", bf16_to_np(got["dW"][int(v)][None]), dw_ref)


@pytest.mark.parametrize("k, pad", [(100, 0.0), (130, 0.3)])
def test_more_candidates_than_wave_lanes(k, pad):
    """k above 64: the tile epilogues scan a row's ids in several 64-slot
    batches (the last one ragged), one wave over its 64 rows (the last wave
    partly past n); with duplicate ids within and across batches and, for
    padded lists, padding slots and a row with no real candidate."""
    padded = pad > 0.0
    inp = _inputs(n=150, vocab=1500, k=k, seed=760 + k, pad_frac=pad)
    inp.ids[5, 1] = inp.ids[5, 0]           # duplicate within a batch
    if padded:
        inp.ids[140, :] = -1
    else:
        inp.ids[9, 70] = inp.ids[9, 3]      # duplicates across batches
        inp.ids[149, k - 1] = inp.ids[149, 0]
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512, padded=padded)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 512, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl, padded=padded)
    torch.cuda.synchronize()
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq, grad=inp.grad,
                     grad_kl=inp.grad_kl, padded=padded)
    rel_check("lp", to_np(lp), ref["lp"])
    rel_check("kl", to_np(kl), ref["kl"])
    rel_check("lse", to_np(lse), ref["lse"])
    grad_check("dH", bf16_to_np(dH), ref["dH"])
    grad_check("dW", bf16_to_np(dW), ref["dW"])
    # repeat: bitwise
    lp2, kl2, lse2, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512, padded=padded)
    dH2, dW2 = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse2, d.grad, 512,
                           ref_logq=d.ref_logq, saved_lp=lp2, grad_kl=d.grad_kl, padded=padded)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp2) and torch.equal(kl, kl2) and torch.equal(dH, dH2) and torch.equal(dW, dW2)


@pytest.mark.parametrize("k, pad", [(67, 0.25), (1024, 0.0)])
def test_kl_only_register_path_candidate_counts(k, pad):
    """The KL-only forward's path that keeps the row of H in registers
    (hidden 1024) with a candidate count whose last group of four is ragged
    (67) and with the largest count (1024); padding slots, a row with no real
    candidate, and a last workgroup holding only two rows (n = 130)."""
    padded = pad > 0.0
    inp = _inputs(n=130, hidden=1024, vocab=3000, k=k, seed=870 + k, pad_frac=pad)
    if padded:
        inp.ids[129, :] = -1
    d = Dev(inp)
    got = _kl_only(d, padded=padded)
    torch.cuda.synchronize()
    ref = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl, padded=padded)
    rel_check("kl", to_np(got["kl"]), ref["kl"])
    rel_check("log p_hat", to_np(got["log_phat"]), ref["log_phat"])
    grad_check("dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("dW", bf16_to_np(got["dW"]), ref["dW"])
    if padded:
        assert got["kl"][129].item() == 0.0 and torch.all(got["dH"][129] == 0)
    again = _kl_only(d, padded=padded)
    torch.cuda.synchronize()
    for key in ("kl", "log_phat", "dH", "dW"):
        assert torch.equal(got[key], again[key]), key


@pytest.mark.parametrize("pad", [0.0, 0.2])
def test_maximum_candidate_count(pad):
    """k = 1024, the largest count the library accepts: sixteen 64-id batches
    per row in the tile epilogues, the per-row coefficient pass and the
    KL-only entry's gathers and counting sort, for both the dense support
    entry and the KL-only one (n = 70: two waves, the second ragged)."""
    padded = pad > 0.0
    k = 1024
    inp = _inputs(n=70, hidden=128, vocab=2500, k=k, seed=790, pad_frac=pad)
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512, padded=padded)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 512, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl, padded=padded)
    ko = _kl_only(d, padded=padded)
    torch.cuda.synchronize()
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq, grad=inp.grad,
                     grad_kl=inp.grad_kl, padded=padded)
    rel_check("lp", to_np(lp), ref["lp"])
    rel_check("kl", to_np(kl), ref["kl"])
    rel_check("lse", to_np(lse), ref["lse"])
    grad_check("dH", bf16_to_np(dH), ref["dH"])
    grad_check("dW", bf16_to_np(dW), ref["dW"])
    ref_kl = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                        grad_kl=inp.grad_kl, padded=padded)
    rel_check("kl-only kl", to_np(ko["kl"]), ref_kl["kl"])
    grad_check("kl-only dH", bf16_to_np(ko["dH"]), ref_kl["dH"])
    grad_check("kl-only dW", bf16_to_np(ko["dW"]), ref_kl["dW"])


def test_skewed_candidate_lists():
    """Candidate ids drawn from a Zipf law (every row lists the most common
    ids): vocabulary buckets of the KL-only entry with hundreds of entries and
    per-tile hit buckets with thousands, sorted by the workgroup sort, for the
    dense support entry and the KL-only one, against the oracle, plus a
    bitwise repeat."""
    inp = _inputs(n=600, vocab=3000, k=64, seed=800)
    rng = np.random.default_rng(801)
    w = np.arange(1, 3001, dtype=np.float64) ** -1.1
    w /= w.sum()
    for i in range(inp.ids.shape[0]):
        inp.ids[i] = rng.choice(3000, size=64, replace=False, p=w)
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 512)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 512, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl)
    ko = _kl_only(d)
    torch.cuda.synchronize()
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq, grad=inp.grad,
                     grad_kl=inp.grad_kl)
    rel_check("lp", to_np(lp), ref["lp"])
    rel_check("kl", to_np(kl), ref["kl"])
    grad_check("dH", bf16_to_np(dH), ref["dH"])
    grad_check("dW", bf16_to_np(dW), ref["dW"])
    ref_kl = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                        grad_kl=inp.grad_kl)
    rel_check("kl-only kl", to_np(ko["kl"]), ref_kl["kl"])
    grad_check("kl-only dH", bf16_to_np(ko["dH"]), ref_kl["dH"])
    grad_check("kl-only dW", bf16_to_np(ko["dW"]), ref_kl["dW"])
    ko2 = _kl_only(d)
    dH2, dW2 = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 512, ref_logq=d.ref_logq,
                           saved_lp=lp, grad_kl=d.grad_kl)
    torch.cuda.synchronize()
    assert torch.equal(ko["dW"], ko2["dW"]) and torch.equal(ko["dH"], ko2["dH"])
    assert torch.equal(dW, dW2) and torch.equal(dH, dH2)


def test_bucket_beyond_one_lds_sort_kl_only():
    """A vocabulary bucket of the KL-only dW with more entries than one
    workgroup sorts in LDS (32768): n = 33000 rows all list id 5 (and one
    other id), so bucket 5 holds 33000 entries, sorted as two LDS runs and one
    merge pass. dW row 5 sums them in ascending (row, slot) order: against the
    oracle, plus a bitwise repeat."""
    inp = _inputs(n=33000, hidden=64, vocab=300, k=2, seed=820)
    rng = np.random.default_rng(821)
    inp.ids[:, 0] = 5
    inp.ids[:, 1] = rng.integers(6, 300, size=inp.ids.shape[0])
    d = Dev(inp)
    ko = _kl_only(d)
    torch.cuda.synchronize()
    ref = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl)
    rel_check("kl-only kl", to_np(ko["kl"]), ref["kl"])
    grad_check("kl-only dH", bf16_to_np(ko["dH"]), ref["dH"])
    grad_check("kl-only dW", bf16_to_np(ko["dW"]), ref["dW"])
    ko2 = _kl_only(d)
    torch.cuda.synchronize()
    assert torch.equal(ko["dW"], ko2["dW"]) and torch.equal(ko["dH"], ko2["dH"])


def test_hit_bucket_beyond_one_lds_sort():
    """A per-tile hit bucket of the dense support entry with more entries
    than one workgroup sorts in LDS: V = 256 (one vocabulary tile) and
    k = 160 distinct candidates per row, so the first row tile's bucket holds
    256 x 160 = 40960 (row, column, slot) hits, sorted as two LDS runs and one
    merge pass: forward and backward against the oracle, plus a bitwise
    repeat."""
    inp = _inputs(n=300, hidden=128, vocab=256, k=160, seed=830)
    rng = np.random.default_rng(831)
    for i in range(inp.ids.shape[0]):
        inp.ids[i] = rng.permutation(256)[:160]
    d = Dev(inp)
    lp, kl, lse, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 256)
    dH, dW = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse, d.grad, 256, ref_logq=d.ref_logq,
                         saved_lp=lp, grad_kl=d.grad_kl)
    torch.cuda.synchronize()
    ref = oracle.run(3, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq, grad=inp.grad,
                     grad_kl=inp.grad_kl)
    rel_check("lp", to_np(lp), ref["lp"])
    rel_check("kl", to_np(kl), ref["kl"])
    grad_check("dH", bf16_to_np(dH), ref["dH"])
    grad_check("dW", bf16_to_np(dW), ref["dW"])
    lp2, kl2, lse2, _ = lm.support_forward(d.H, d.W, d.ids, d.ref_logq, 256)
    dH2, dW2 = lm.backward(lm.ENTRY_SUPPORT, d.H, d.W, d.ids, lse2, d.grad, 256, ref_logq=d.ref_logq,
                           saved_lp=lp2, grad_kl=d.grad_kl)
    torch.cuda.synchronize()
    assert torch.equal(lp, lp2) and torch.equal(dW, dW2) and torch.equal(dH, dH2)
