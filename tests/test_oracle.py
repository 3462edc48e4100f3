"""Pins for the fp64 oracle, against what the mathematics fixes.

Each check is independent of the oracle's own code: hand-derived closed forms
(tests/golden), the W = 0 closed form, torch fp64 library routines
(cross_entropy, log_softmax, kl_div, autograd), brute-force pure-Python loops,
central finite differences and invariants. A mutation section plants
plausible mistakes in the oracle (on the CPU only) and shows a pin catches
each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wlmod
from workloads import IGNORE_INDEX, bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _tiny_inputs(**kw):
    wl = wlmod.custom(**kw)
    return wl, wlmod.make_inputs(wl)


# --------------------------------------------------------------- hand-derived

def _cases():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


def test_golden_identity_case():
    c = _cases()["identity_3vocab"]
    H, W = np.array(c["H"]), np.array(c["W"])
    z = oracle.logits(H, W)
    f = oracle.ce_forward(z, np.array(c["targets"]))
    np.testing.assert_allclose(f["lse"], c["lse"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(f["loss_rows"], c["loss_rows"], rtol=0, atol=1e-15)
    assert abs(f["loss"] - c["loss_mean"]) < 1e-15
    lp = oracle.logprob_forward(z, np.array(c["targets"]))
    np.testing.assert_allclose(lp["logp"], c["logp"], atol=1e-15)
    dz = oracle.ce_dz(z, np.array(c["targets"]), 1.0)
    np.testing.assert_allclose(dz, c["dz_mean"], atol=1e-15)


def test_golden_negative_labels():
    c = _cases()["negative_labels_ignored"]
    z = oracle.logits(np.array(c["H"]), np.array(c["W"]))
    f = oracle.ce_forward(z, np.array(c["targets"]))
    np.testing.assert_allclose(f["lse"], c["lse"], atol=1e-15)
    np.testing.assert_allclose(f["loss_rows"], c["loss_rows"], atol=1e-15)
    assert f["count"] == 1
    assert abs(f["loss"] - c["loss_mean"]) < 1e-15
    lp = oracle.logprob_forward(z, np.array(c["targets"]))
    np.testing.assert_allclose(lp["logp"], c["logp"], atol=1e-15)


def test_golden_support_case():
    c = _cases()["support_two_candidates"]
    z = oracle.logits(np.array(c["H"]), np.array(c["W"]))
    f = oracle.support_forward(z, np.array(c["ids"]), np.array(c["ref_logq"]))
    np.testing.assert_allclose(f["lp"], c["lp"], atol=1e-15)
    np.testing.assert_allclose(f["kl"], c["kl"], atol=1e-15)


# ------------------------------------------------------------------ W = 0 form

@pytest.mark.parametrize("vocab", [1024, 1000, 4099])
def test_w_zero_closed_form(vocab):
    """W = 0: every logit is 0, softmax is uniform, lse = ln V, mean CE = ln V."""
    wl, inp = _tiny_inputs(n=48, hidden=64, vocab=vocab, ignore_frac=0.25, seed=11)
    W = np.zeros((vocab, 64), dtype=np.uint16)
    t = inp.targets
    out = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, W, targets=t)
    lnV = math.log(vocab)
    assert np.all(out["lse"] == lnV)
    assert abs(out["loss"] - lnV) < 1e-12
    assert np.all(out["dH"] == 0.0)
    # dW[v] = (1/count) sum_{valid n} (1/V - [t_n = v]) H[n]
    Hf = _f64(inp.H)
    valid = t >= 0
    count = valid.sum()
    onehot = np.zeros((48, vocab))
    onehot[np.nonzero(valid)[0], t[valid]] = 1.0
    expect = ((valid[:, None] / count) * (1.0 / vocab - onehot)).T @ Hf
    np.testing.assert_allclose(out["dW"], expect, rtol=1e-12, atol=1e-14)
    lp = oracle.run(oracle.ENTRY_LOGPROB, inp.H, W, targets=t, grad=inp.grad[:1].repeat(48),
                    backward=False)
    assert np.all(lp["logp"][valid] == -lnV) and np.all(lp["logp"][~valid] == 0.0)


def test_w_zero_support_kl_closed_form():
    """W = 0: p_hat = 1/K, so KL = sum q log q + Q log K and lp = -ln V."""
    wl = wlmod.custom(n=16, hidden=32, vocab=512, entry=wlmod.ENTRY_SUPPORT, k=8, seed=5)
    inp = wlmod.make_inputs(wl)
    W = np.zeros((512, 32), dtype=np.uint16)
    f = oracle.support_forward(oracle.logits(inp.H, W), inp.ids, inp.ref_logq)
    q = np.exp(inp.ref_logq.astype(np.float64))
    expect = (q * inp.ref_logq.astype(np.float64)).sum(1) + q.sum(1) * math.log(8)
    np.testing.assert_allclose(f["kl"], expect, rtol=1e-12, atol=1e-14)
    assert np.all(f["lp"] == -math.log(512))


# ------------------------------------------------------------- torch fp64 pins

def _torch_problem(inp):
    H = torch.tensor(_f64(inp.H), requires_grad=True)
    W = torch.tensor(_f64(inp.W), requires_grad=True)
    return H, W


def test_ce_vs_torch_tiny():
    """Tiny config: torch fp64 cross_entropy (ignore_index=-100, mean) and autograd."""
    inp = wlmod.make_inputs(wlmod.WORKLOADS["tiny"])
    out = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    H, W = _torch_problem(inp)
    z = H @ W.T
    t = torch.tensor(inp.targets, dtype=torch.long)
    loss = F.cross_entropy(z, t, ignore_index=IGNORE_INDEX, reduction="mean")
    loss.backward()
    assert abs(out["loss"] - loss.item()) < 1e-12
    np.testing.assert_allclose(out["lse"], torch.logsumexp(z, 1).detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-14)
    assert out["count"] == int((inp.targets >= 0).sum()) == 64 - 6


def test_ce_sum_vs_torch():
    wl, inp = _tiny_inputs(n=40, hidden=64, vocab=300, ignore_frac=0.2, seed=21)
    out = oracle.run(oracle.ENTRY_CE_SUM, inp.H, inp.W, targets=inp.targets, grad=np.array([0.75]))
    H, W = _torch_problem(inp)
    loss = F.cross_entropy(H @ W.T, torch.tensor(inp.targets, dtype=torch.long),
                           ignore_index=IGNORE_INDEX, reduction="sum")
    (0.75 * loss).backward()
    assert abs(out["loss"] - loss.item()) < 1e-11
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_logprob_vs_torch():
    wl = wlmod.custom(n=50, hidden=128, vocab=700, entry=wlmod.ENTRY_LOGPROB, seed=31,
                      ignore_frac=0.1)
    inp = wlmod.make_inputs(wl)
    out = oracle.run(oracle.ENTRY_LOGPROB, inp.H, inp.W, targets=inp.targets, grad=inp.grad)
    H, W = _torch_problem(inp)
    logsm = F.log_softmax(H @ W.T, dim=1)
    t = torch.tensor(inp.targets, dtype=torch.long)
    valid = t >= 0
    lp = torch.where(valid, logsm.gather(1, t.clamp(min=0)[:, None])[:, 0], torch.zeros(()))
    np.testing.assert_allclose(out["logp"], lp.detach().numpy(), rtol=1e-12, atol=1e-13)
    (lp * torch.tensor(inp.grad, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_support_vs_torch():
    wl = wlmod.custom(n=24, hidden=64, vocab=400, entry=wlmod.ENTRY_SUPPORT, k=16, seed=41)
    inp = wlmod.make_inputs(wl)
    out = oracle.run(oracle.ENTRY_SUPPORT, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad=inp.grad, grad_kl=inp.grad_kl)
    H, W = _torch_problem(inp)
    z = H @ W.T
    ids = torch.tensor(inp.ids, dtype=torch.long)
    lp = F.log_softmax(z, 1).gather(1, ids)
    zc = z.gather(1, ids)
    log_phat = F.log_softmax(zc, 1)
    r = torch.tensor(inp.ref_logq, dtype=torch.float64)
    kl = F.kl_div(log_phat, r, log_target=True, reduction="none").sum(1)
    np.testing.assert_allclose(out["lp"], lp.detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out["kl"], kl.detach().numpy(), rtol=1e-10, atol=1e-14)
    obj = (lp * torch.tensor(inp.grad, dtype=torch.float64)).sum() + \
        (kl * torch.tensor(inp.grad_kl, dtype=torch.float64)).sum()
    obj.backward()
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-9, atol=1e-13)


# ---------------------------------------------------------------- brute force

def _brute_logits(H, W):
    return [[math.fsum(H[n][h] * W[v][h] for h in range(len(H[0]))) for v in range(len(W))]
            for n in range(len(H))]


def _brute_lse(row):
    m = max(row)
    return m + math.log(math.fsum(math.exp(x - m) for x in row))


def test_bruteforce_all_entries():
    rng = np.random.default_rng(3)
    Hb = f32_to_bf16_bits(rng.standard_normal((3, 4)).astype(np.float32))
    Wb = f32_to_bf16_bits(rng.standard_normal((5, 4)).astype(np.float32))
    H, W = _f64(Hb).tolist(), _f64(Wb).tolist()
    z = _brute_logits(H, W)
    t = [4, -100, 0]
    zo = oracle.logits(Hb, Wb)
    np.testing.assert_allclose(zo, z, rtol=1e-15, atol=1e-15)
    lse = [_brute_lse(r) for r in z]
    rows = [lse[n] - z[n][t[n]] for n in (0, 2)]
    f = oracle.ce_forward(zo, np.array(t))
    assert abs(f["loss"] - math.fsum(rows) / 2) < 1e-14
    lp = oracle.logprob_forward(zo, np.array(t))["logp"]
    assert abs(lp[0] - (z[0][4] - lse[0])) < 1e-14 and lp[1] == 0.0
    ids = np.array([[1, 3], [0, 4], [2, 2]])
    rq = np.log(np.array([[0.3, 0.7], [0.5, 0.5], [0.9, 0.1]]))
    s = oracle.support_forward(zo, ids, rq)
    for n in range(3):
        zc = [z[n][int(i)] for i in ids[n]]
        lc = _brute_lse(zc)
        kl = math.fsum(math.exp(rq[n, k]) * (rq[n, k] - (zc[k] - lc)) for k in range(2))
        assert abs(s["kl"][n] - kl) < 1e-14
        for k in range(2):
            assert abs(s["lp"][n, k] - (zc[k] - lse[n])) < 1e-14


# --------------------------------------------------------- finite differences

def _objective(entry, H, W, t, ids, rq, g, gkl, num_valid=-1):
    z = oracle.logits(H, W)
    if entry == oracle.ENTRY_CE_MEAN:
        return g * oracle.ce_forward(z, t, num_valid, "mean")["loss"]
    if entry == oracle.ENTRY_CE_SUM:
        return g * oracle.ce_forward(z, t, -1, "sum")["loss"]
    if entry == oracle.ENTRY_LOGPROB:
        return float((oracle.logprob_forward(z, t)["logp"] * g).sum())
    f = oracle.support_forward(z, ids, rq)
    return float((f["lp"] * g).sum() + (f["kl"] * gkl).sum())


@pytest.mark.parametrize("entry", [0, 1, 2, 3])
def test_finite_differences(entry):
    """Central differences (h = 1e-6, fp64) on every element of H and W."""
    rng = np.random.default_rng(100 + entry)
    N, Hd, V, K = 4, 8, 16, 4
    H = rng.standard_normal((N, Hd))
    W = rng.standard_normal((V, Hd)) * 0.5
    t = np.array([3, -100, 15, 0])
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    ids[1, 2] = ids[1, 0]  # a duplicate id counts twice
    q = rng.random((N, K)) + 0.1
    rq = np.log(q / q.sum(1, keepdims=True))
    if entry in (0, 1):
        g, gkl = 1.3, None
    elif entry == 2:
        g, gkl = rng.standard_normal(N), None
    else:
        g, gkl = rng.standard_normal((N, K)), rng.standard_normal(N)
    out = oracle.run(entry, H, W, targets=t if entry < 3 else None, ids=ids if entry == 3 else None,
                     ref_logq=rq if entry == 3 else None,
                     grad=np.array([g]) if entry < 2 else g, grad_kl=gkl)
    h = 1e-6
    for name, X, G in (("H", H, out["dH"]), ("W", W, out["dW"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = (Xp, W) if name == "H" else (H, Xp)
            argm = (Xm, W) if name == "H" else (H, Xm)
            fp = _objective(entry, *args, t, ids, rq, g, gkl)
            fm = _objective(entry, *argm, t, ids, rq, g, gkl)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8, err_msg=f"d{name} entry {entry}")


# ------------------------------------------------------------------ invariants

@pytest.mark.parametrize("shift", [0.0, 10.0, 1000.0])
def test_shift_invariance(shift):
    """Appending column c to H and 1 to W adds c to every logit: loss and logp are unchanged.
    c = 1000 overflows exp() unless the max is subtracted first."""
    wl, inp = _tiny_inputs(n=32, hidden=64, vocab=500, ignore_frac=0.1, seed=51)
    H0, W0 = _f64(inp.H), _f64(inp.W)
    Hs = np.concatenate([H0, np.full((32, 1), shift)], 1)
    Ws = np.concatenate([W0, np.ones((500, 1))], 1)
    a = oracle.ce_forward(oracle.logits(H0, W0), inp.targets)
    b = oracle.ce_forward(oracle.logits(Hs, Ws), inp.targets)
    assert np.isfinite(b["loss"])
    assert abs(a["loss"] - b["loss"]) < 1e-12 * max(1.0, shift)
    np.testing.assert_allclose(b["lse"] - shift, a["lse"], rtol=0, atol=1e-12 * max(1.0, shift))


def test_logprobs_sum_to_one():
    """Each tiny row replicated with every label 0..V-1: sum_v exp(logp_v) = 1."""
    inp = wlmod.make_inputs(wlmod.WORKLOADS["tiny"])
    V = 1024
    z = oracle.logits(inp.H[:4], inp.W)
    for r in range(4):
        zr = np.repeat(z[r:r + 1], V, axis=0)
        lp = oracle.logprob_forward(zr, np.arange(V))["logp"]
        assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-13
        # logp = -(per-row CE)
        ce = oracle.ce_forward(zr, np.arange(V), reduction="sum")["loss_rows"]
        np.testing.assert_allclose(lp, -ce, rtol=0, atol=1e-14)


def test_support_full_vocab_lists_sum_to_one():
    """K = V listing every id: sum_k exp(lp) = 1 and lp equals the logprob entry."""
    wl, inp = _tiny_inputs(n=8, hidden=32, vocab=64, seed=61)
    z = oracle.logits(inp.H, inp.W)
    ids = np.tile(np.arange(64), (8, 1))
    f = oracle.support_forward(z, ids, None)
    np.testing.assert_allclose(np.exp(f["lp"]).sum(1), 1.0, rtol=0, atol=1e-13)
    for k in (0, 17, 63):
        lp = oracle.logprob_forward(z, np.full(8, k))["logp"]
        np.testing.assert_array_equal(f["lp"][:, k], lp)


def test_kl_zero_for_identical_and_nonnegative():
    wl = wlmod.custom(n=16, hidden=64, vocab=300, entry=wlmod.ENTRY_SUPPORT, k=12, seed=71)
    inp = wlmod.make_inputs(wl)
    z = oracle.logits(inp.H, inp.W)
    f = oracle.support_forward(z, inp.ids, inp.ref_logq)
    assert np.all(f["kl"] >= -1e-15)
    same = oracle.support_forward(z, inp.ids, f["log_phat"])
    assert np.all(np.abs(same["kl"]) < 1e-14)
    dz = oracle.support_dz(z, inp.ids, f["log_phat"], None, np.ones(16))
    assert np.all(np.abs(dz) < 1e-15)  # KL minimum: zero gradient


def test_ignored_and_zero_grad_rows():
    wl, inp = _tiny_inputs(n=32, hidden=64, vocab=256, ignore_frac=0.25, seed=81)
    out = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    ign = inp.targets < 0
    assert np.all(out["loss_rows"][ign] == 0.0)
    assert np.all(out["dz"][ign] == 0.0) and np.all(out["dH"][ign] == 0.0)
    # CE: each valid row of dz sums to zero over the vocabulary
    assert np.all(np.abs(out["dz"].sum(1)) < 1e-16 + 1e-15 * np.abs(out["dz"]).sum(1))
    g = np.ones(32)
    g[::3] = 0.0
    lp = oracle.run(oracle.ENTRY_LOGPROB, inp.H, inp.W, targets=inp.targets, grad=g)
    assert np.all(lp["dH"][::3] == 0.0)


def test_empty_valid_set_and_given_count():
    wl, inp = _tiny_inputs(n=16, hidden=32, vocab=128, seed=91)
    t = np.full(16, -100, dtype=np.int32)
    out = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=t)
    assert out["loss"] == 0.0 and out["count"] == 0
    assert np.all(out["dH"] == 0.0) and np.all(out["dW"] == 0.0)
    a = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    b = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets, num_valid=64)
    assert abs(b["loss"] * 64 - a["loss"] * 16) < 1e-12
    np.testing.assert_allclose(b["dW"] * 64, a["dW"] * 16, rtol=1e-12, atol=1e-15)


def test_errors():
    wl, inp = _tiny_inputs(n=8, hidden=32, vocab=64, seed=1)
    z = oracle.logits(inp.H, inp.W)
    t = np.zeros(8, dtype=np.int32)
    t[5] = 64
    with pytest.raises(ValueError, match="row 5"):
        oracle.ce_forward(z, t)
    ids = np.zeros((8, 2), dtype=np.int32)
    ids[3, 1] = -1
    with pytest.raises(ValueError, match="row 3"):
        oracle.support_forward(z, ids, None)


def test_row_sample_matches_full():
    """The sampled-row path (used at full sizes) equals the full path on those rows."""
    wl, inp = _tiny_inputs(n=40, hidden=64, vocab=333, ignore_frac=0.1, seed=13)
    full = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    rows = np.array([0, 7, 39])
    s = oracle.rows_forward_backward(oracle.ENTRY_CE_MEAN, inp.H, inp.W, rows,
                                     targets=inp.targets, count=full["count"])
    np.testing.assert_array_equal(s["lse"], full["lse"][rows])
    np.testing.assert_allclose(s["dH"], full["dH"][rows], rtol=1e-14, atol=1e-18)
    # dW over a subset of vocabulary columns from all rows equals the full dW rows
    cols = np.array([3, 100, 332])
    dw = oracle.grad_weight(full["dz"][:, cols], inp.H, np.arange(40))
    np.testing.assert_array_equal(dw, full["dW"][cols])


_ROW_CASES = [
    # (entry, padded, with KL grads, temperature, per-row temperature)
    (oracle.ENTRY_CE_MEAN, False, False, 0.0, True),
    (oracle.ENTRY_CE_SUM, False, False, 1.3, False),
    (oracle.ENTRY_LOGPROB, False, False, 0.0, False),
    (oracle.ENTRY_LOGPROB, False, False, 1.3, True),
    (oracle.ENTRY_SUPPORT, False, True, 0.0, True),
    (oracle.ENTRY_SUPPORT, False, False, 0.7, True),
    (oracle.ENTRY_SUPPORT, True, True, 0.0, True),
    (oracle.ENTRY_SUPPORT, True, False, 0.0, False),
    (oracle.ENTRY_SUPPORT_KL, False, True, 0.0, True),
    (oracle.ENTRY_SUPPORT_KL, True, True, 1.3, True),
]


@pytest.mark.parametrize("entry,padded,with_kl,temp,per_row", _ROW_CASES)
def test_row_sample_matches_full_every_entry(entry, padded, with_kl, temp, per_row):
    """The sampled-row path that the full-size GPU parity tests use equals the
    pinned full path (oracle.run) on the same rows for every entry: CE mean and
    sum, log-prob, support with and without the KL term, KL-only, padded
    candidate lists, scalar and per-row temperatures. The rows are not a prefix
    and every row has its own upstream gradient and temperature, so a per-row
    input not indexed by the sampled rows changes the result."""
    support = entry in (oracle.ENTRY_SUPPORT, oracle.ENTRY_SUPPORT_KL)
    kw = dict(n=40, hidden=64, vocab=333, ignore_frac=0.1 if not support else 0.0, seed=31 + entry,
              entry=entry if entry != oracle.ENTRY_SUPPORT_KL else oracle.ENTRY_SUPPORT,
              k=6 if support else 1, pad_frac=0.3 if padded else 0.0)
    wl, inp = _tiny_inputs(**kw)
    rng = np.random.default_rng(5 + entry)
    rt = rng.uniform(0.5, 2.0, size=40) if per_row else None
    grad = inp.grad
    if entry in (oracle.ENTRY_CE_MEAN, oracle.ENTRY_CE_SUM):
        grad = np.array([0.75])
    grad_kl = inp.grad_kl if with_kl else None
    common = dict(targets=inp.targets, ids=inp.ids, ref_logq=inp.ref_logq,
                  grad=None if entry == oracle.ENTRY_SUPPORT_KL else grad, grad_kl=grad_kl,
                  temperature=temp, row_temperature=rt, padded=padded)
    if entry == oracle.ENTRY_SUPPORT_KL:
        common["grad_kl"] = inp.grad_kl
    full = oracle.run(entry, inp.H, inp.W, **common)
    rows = np.array([1, 7, 22, 39])
    count = full.get("count")
    s = oracle.rows_forward_backward(entry, inp.H, inp.W, rows, count=count, **common)
    for key in ("lse", "loss_rows", "logp", "lp", "kl", "log_phat"):
        if key in full and key in s:
            np.testing.assert_allclose(s[key], full[key][rows], rtol=1e-13, atol=1e-15, err_msg=key)
    expect = {oracle.ENTRY_CE_MEAN: ("lse", "loss_rows"), oracle.ENTRY_CE_SUM: ("lse", "loss_rows"),
              oracle.ENTRY_LOGPROB: ("lse", "logp"), oracle.ENTRY_SUPPORT: ("lse", "lp"),
              oracle.ENTRY_SUPPORT_KL: ("kl", "log_phat")}[entry]
    for key in expect:
        assert key in s, key
    if entry == oracle.ENTRY_SUPPORT and inp.ref_logq is not None:
        assert "kl" in s
    np.testing.assert_allclose(s["dz"], full["dz"][rows], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(s["dH"], full["dH"][rows], rtol=1e-12, atol=1e-16)
    # the sampled rows' gradient is not trivially zero
    assert np.abs(s["dH"]).max() > 0


# ------------------------------------------------------------------ mutations

def test_mutations_are_caught(monkeypatch):
    """Plant plausible mistakes in the oracle and show a pin fails for each."""
    inp = wlmod.make_inputs(wlmod.WORKLOADS["tiny"])
    H, W = _torch_problem(inp)
    t = torch.tensor(inp.targets, dtype=torch.long)
    ref = F.cross_entropy(H @ W.T, t, ignore_index=IGNORE_INDEX).item()

    def loss_now():
        return oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets,
                          backward=False)["loss"]

    # 1. dropped max add-back in logsumexp
    orig = oracle.logsumexp_rows
    monkeypatch.setattr(oracle, "logsumexp_rows",
                        lambda z: np.log(np.exp(z - z.max(1)[:, None]).sum(1)))
    assert abs(loss_now() - ref) > 1e-3
    monkeypatch.setattr(oracle, "logsumexp_rows", orig)
    # 2. transposed operand: the logits of W H^T-like misuse (rows of W as hidden)
    z_bad = oracle.logits(inp.H, inp.W)[:, ::-1]
    assert abs(oracle.ce_forward(z_bad, inp.targets)["loss"] - ref) > 1e-3
    # 3. wrong sign of the softmax term in the CE gradient: the autograd pin fails
    z = oracle.logits(inp.H, inp.W)
    F.cross_entropy(H @ W.T, t, ignore_index=IGNORE_INDEX).backward()
    orig_sm = oracle.softmax_rows
    monkeypatch.setattr(oracle, "softmax_rows", lambda z, l: -orig_sm(z, l))
    bad = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    assert not np.allclose(bad["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-14)
    assert not np.allclose(bad["dH"], H.grad.numpy(), rtol=1e-10, atol=1e-14)
    monkeypatch.setattr(oracle, "softmax_rows", orig_sm)
    good = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    np.testing.assert_allclose(good["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-14)
    # 4. mean over all rows instead of valid rows
    f = oracle.ce_forward(z, inp.targets)
    assert abs(f["loss_rows"].sum() / 64 - ref) > 1e-3
    assert abs(f["loss"] - ref) < 1e-12


# ----------------------------------------------------------------- temperature

def test_temperature_routes():
    """tau = 1.0 equals no temperature exactly; a scalar tau equals logits / tau in
    torch fp64 cross_entropy and autograd; a per-row tau scales each row."""
    wl, inp = _tiny_inputs(n=24, hidden=64, vocab=300, ignore_frac=0.1, seed=17)
    off = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    one = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets, temperature=1.0)
    assert off["loss"] == one["loss"]
    np.testing.assert_array_equal(off["dW"], one["dW"])
    tau = np.linspace(0.5, 2.0, 24)
    for temp, rowt in ((0.7, None), (0.0, tau), (1.3, tau)):
        got = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets,
                         temperature=temp, row_temperature=rowt)
        H, W = _torch_problem(inp)
        t_eff = torch.tensor((temp if temp else 1.0) * (rowt if rowt is not None else np.ones(24)))
        z = (H @ W.T) / t_eff[:, None]
        loss = F.cross_entropy(z, torch.tensor(inp.targets, dtype=torch.long), ignore_index=IGNORE_INDEX)
        loss.backward()
        assert abs(got["loss"] - loss.item()) < 1e-12
        np.testing.assert_allclose(got["dH"], H.grad.numpy(), rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(got["dW"], W.grad.numpy(), rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("entry", [0, 2, 3])
def test_temperature_finite_differences(entry):
    rng = np.random.default_rng(300 + entry)
    N, Hd, V, K = 3, 6, 12, 3
    H = rng.standard_normal((N, Hd))
    W = rng.standard_normal((V, Hd)) * 0.5
    t = np.array([2, -100, 11])
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    q = rng.random((N, K)) + 0.1
    rq = np.log(q / q.sum(1, keepdims=True))
    rowt = np.array([0.6, 1.7, 1.1])
    g = np.array([0.9]) if entry == 0 else rng.standard_normal(N if entry == 2 else (N, K))
    gkl = rng.standard_normal(N) if entry == 3 else None
    kw = dict(targets=t if entry < 3 else None, ids=ids if entry == 3 else None,
              ref_logq=rq if entry == 3 else None, grad=g, grad_kl=gkl,
              temperature=0.8, row_temperature=rowt)
    out = oracle.run(entry, H, W, **kw)

    def obj(Hx, Wx):
        f = oracle.run(entry, Hx, Wx, backward=False, **kw)
        if entry == 0:
            return float(g[0] * f["loss"])
        if entry == 2:
            return float((f["logp"] * g).sum())
        return float((f["lp"] * g).sum() + (f["kl"] * gkl).sum())

    h = 1e-6
    for name, X, G in (("H", H, out["dH"]), ("W", W, out["dW"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            num[idx] = ((obj(Xp, W) - obj(Xm, W)) if name == "H" else (obj(H, Xp) - obj(H, Xm))) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8, err_msg=f"d{name} entry {entry}")


def test_temperature_rejects_nonpositive():
    with pytest.raises(ValueError):
        oracle.temperature_scale(3, -1.0)
    with pytest.raises(ValueError):
        oracle.temperature_scale(3, 0.0, np.array([1.0, 0.0, 2.0]))


# ------------------------------------------- padded lists and the KL-only entry

def _padded_case(seed=61):
    wl = wlmod.custom(n=12, hidden=64, vocab=300, entry=wlmod.ENTRY_SUPPORT, k=8, seed=seed,
                      pad_frac=0.3)
    inp = wlmod.make_inputs(wl)
    inp.ids[3, :] = -1            # a row with no real candidate
    inp.ids[5, 2] = -7            # any negative id is padding, also mid-list
    return inp


def test_padded_support_vs_torch_on_compacted_lists():
    """A padded list equals the list with its padding slots removed: torch fp64
    log_softmax / kl_div / autograd on each row's real candidates only."""
    inp = _padded_case()
    out = oracle.run(oracle.ENTRY_SUPPORT, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad=inp.grad, grad_kl=inp.grad_kl, padded=True)
    H, W = _torch_problem(inp)
    z = H @ W.T
    lsm = F.log_softmax(z, 1)
    obj = torch.zeros((), dtype=torch.float64)
    for n in range(inp.ids.shape[0]):
        real = np.nonzero(inp.ids[n] >= 0)[0]
        pad = np.nonzero(inp.ids[n] < 0)[0]
        assert np.all(out["lp"][n, pad] == 0.0)
        if real.size == 0:
            assert out["kl"][n] == 0.0
            continue
        idx = torch.tensor(inp.ids[n, real], dtype=torch.long)
        lp = lsm[n, idx]
        r = torch.tensor(inp.ref_logq[n, real], dtype=torch.float64)
        kl = F.kl_div(F.log_softmax(z[n, idx], 0), r, log_target=True, reduction="sum")
        np.testing.assert_allclose(out["lp"][n, real], lp.detach().numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(out["kl"][n], kl.item(), rtol=1e-10, atol=1e-14)
        g = torch.tensor(inp.grad[n, real], dtype=torch.float64)
        obj = obj + (lp * g).sum() + kl * float(inp.grad_kl[n])
    obj.backward()
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-9, atol=1e-13)


def test_kl_only_entry_vs_torch():
    """KL-only entry: KL(q || softmax over the candidates) and its gradient,
    torch fp64 autograd; log p_hat is torch's log_softmax over the candidates."""
    wl = wlmod.custom(n=10, hidden=64, vocab=350, entry=wlmod.ENTRY_SUPPORT, k=12, seed=62)
    inp = wlmod.make_inputs(wl)
    out = oracle.run(oracle.ENTRY_SUPPORT_KL, inp.H, inp.W, ids=inp.ids, ref_logq=inp.ref_logq,
                     grad_kl=inp.grad_kl)
    assert "lp" not in out and "lse" not in out
    H, W = _torch_problem(inp)
    zc = (H @ W.T).gather(1, torch.tensor(inp.ids, dtype=torch.long))
    log_phat = F.log_softmax(zc, 1)
    r = torch.tensor(inp.ref_logq, dtype=torch.float64)
    kl = F.kl_div(log_phat, r, log_target=True, reduction="none").sum(1)
    np.testing.assert_allclose(out["kl"], kl.detach().numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(out["log_phat"], log_phat.detach().numpy(), rtol=1e-12, atol=1e-13)
    (kl * torch.tensor(inp.grad_kl, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(out["dH"], H.grad.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(out["dW"], W.grad.numpy(), rtol=1e-9, atol=1e-13)


@pytest.mark.parametrize("entry", [3, 4])
def test_padded_finite_differences(entry):
    """Central differences on every element of H and W with padded lists (and
    a duplicate id) for the support and KL-only entries."""
    rng = np.random.default_rng(120 + entry)
    N, Hd, V, K = 4, 6, 12, 5
    H = rng.standard_normal((N, Hd))
    W = rng.standard_normal((V, Hd)) * 0.5
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    ids[0, 3:] = -1
    ids[2, 1] = -1
    ids[3, 4] = ids[3, 0]
    q = rng.random((N, K)) + 0.1
    rq = np.log(q / q.sum(1, keepdims=True))
    g = rng.standard_normal((N, K)) if entry == 3 else None
    gkl = rng.standard_normal(N)
    out = oracle.run(entry, H, W, ids=ids, ref_logq=rq, grad=g, grad_kl=gkl, padded=True)

    def obj(Hx, Wx):
        z = oracle.logits(Hx, Wx)
        f = oracle.support_forward(z, ids, rq, padded=True)
        v = float((f["kl"] * gkl).sum())
        if entry == 3:
            v += float((f["lp"] * g).sum())
        return v

    h = 1e-6
    for name, X, G in (("H", H, out["dH"]), ("W", W, out["dW"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            num[idx] = ((obj(Xp, W) - obj(Xm, W)) if name == "H" else (obj(H, Xp) - obj(H, Xm))) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=1e-6, atol=1e-8, err_msg=f"d{name} entry {entry}")


def test_padding_rules():
    z = np.zeros((2, 10))
    ids = np.array([[1, -1], [3, 4]])
    with pytest.raises(ValueError):
        oracle.support_forward(z, ids, None)               # negative id without padding
    with pytest.raises(ValueError):
        oracle.support_forward(z, np.array([[1, 10], [0, 2]]), None, padded=True)   # >= V
    f = oracle.support_forward(z, ids, np.log(np.full((2, 2), 0.5)), padded=True)
    # row 0 has one real candidate: p_hat = 1 there, KL = q (log q - 0) with q = 0.5
    assert f["log_phat"][0, 0] == 0.0 and abs(f["kl"][0] - 0.5 * math.log(0.5)) < 1e-15
    assert f["lp"][0, 1] == 0.0
