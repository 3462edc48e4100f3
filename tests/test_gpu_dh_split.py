"""GPU parity of the K-split dH contraction: with fewer dH tiles (row tiles x
hidden tiles) than half the compute units and a chunk of at least 16 K steps
(1024 columns), each chunk's dH tiles are cut along the chunk's columns into
slices whose fp32 partials are added in slice order. These shapes take that
route (n = 200 and hidden = 512: two dH tiles; chunk 2048: four slices, the
last chunk 1024 wide: two). Checked against the oracle, with caller-owned
accumulators, and for a dH-only backward."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu

CHUNK = 2048


def _inputs(entry, **kw):
    d = dict(n=200, hidden=512, vocab=5000, chunk=CHUNK, seed=900 + entry, ignore_frac=0.1,
             entry=entry)
    if entry == wlmod.ENTRY_SUPPORT:
        d.update(k=16, ignore_frac=0.0)
    d.update(kw)
    return wlmod.make_inputs(wlmod.custom(**d))


def _ref(entry, inp):
    return oracle.run(entry, inp.H, inp.W, targets=inp.targets, ids=inp.ids, ref_logq=inp.ref_logq,
                      grad=inp.grad, grad_kl=inp.grad_kl)


@pytest.mark.parametrize("entry", [0, 2, 3])
def test_split_dh_against_oracle(entry):
    inp = _inputs(entry)
    got = run_entry(Dev(inp), entry, CHUNK)
    ref = _ref(entry, inp)
    rel_check("lse", to_np(got["lse"]), ref["lse"])
    grad_check("dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("dW", bf16_to_np(got["dW"]), ref["dW"])


@pytest.mark.parametrize("shape", [
    dict(n=1, hidden=64, vocab=3000, chunk=4096),       # one row, one dH tile, 48 K steps: 4 slices
    dict(n=33, hidden=320, vocab=4100, chunk=1024),     # ragged hidden tile; 4-wide tail chunk: no split
    dict(n=513, hidden=256, vocab=2600, chunk=2560),    # three row tiles, 40 K steps: 4 slices
])
def test_split_dh_shapes(shape):
    inp = wlmod.make_inputs(wlmod.custom(seed=910, ignore_frac=0.1, **shape))
    got = run_entry(Dev(inp), 0, shape["chunk"])
    ref = _ref(0, inp)
    rel_check("loss", [got["loss"].item()], [ref["loss"]])
    grad_check("dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("dW", bf16_to_np(got["dW"]), ref["dW"])


def test_split_dh_only_matches_both_bitwise():
    """The slice count depends on the shape alone, so a dH-only backward sums
    in the same order as one that also wants dW."""
    inp = _inputs(0)
    d = Dev(inp)
    both = run_entry(d, 0, CHUNK)
    only_dh = run_entry(d, 0, CHUNK, need_dW=False)
    torch.cuda.synchronize()
    assert only_dh["dW"] is None
    assert torch.equal(both["dH"], only_dh["dH"])


def test_split_dh_into_accumulator():
    """A caller accumulator holding X ends at X + dH: the running sum is read
    from the first chunk on and stored after the last."""
    inp = _inputs(0)
    d = Dev(inp)
    plain = run_entry(d, 0, CHUNK)
    loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, CHUNK)
    torch.manual_seed(0)
    x = torch.randn(d.H.shape, dtype=torch.float32, device="cuda") * 1e-3
    dH_acc = x.clone()
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    dH, _ = lm.backward_accumulate(0, d.H, d.W, d.t, lse, d.grad, CHUNK, dH_acc=dH_acc,
                                   dW_acc=dW_acc, out_bf16=True)
    torch.cuda.synchronize()
    assert torch.equal(dH, dH_acc.to(torch.bfloat16))
    ref = _ref(0, inp)
    grad_check("dH_acc - X", to_np(dH_acc - x), ref["dH"])
    grad_check("dW_acc", to_np(dW_acc), ref["dW"])
    assert torch.equal(dW_acc.to(torch.bfloat16), plain["dW"])
