"""GPU parity of the shared dH pass: when a problem has at least 256 dH tiles
of 256 x 256, four consecutive vocabulary chunks share one dH contraction
over all of their columns (one fp32 running-sum update per pass). The
smallest shapes where that happens with the full oracle still in reach:
65,536 rows of hidden 256 (256 row tiles x 1 hidden tile) and 256-wide
chunks, so that each chunk fills the 256 compute units with its own
recompute tiles. Vocabularies of 5 chunks (a full pass, then the ragged last
chunk alone), 7 chunks (a full pass, then a pass of three ending in the
ragged chunk, as at V = 151,936 with 8192-wide chunks) and 4 chunks (one
pass ending in the ragged chunk)."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu

N, HID, CHUNK = 65536, 256, 256


@pytest.mark.parametrize("vocab", [1124, 1636, 868])
def test_shared_dh_pass_against_oracle(vocab):
    chunks = -(-vocab // CHUNK)
    # the dL/dz region holds four chunks: the shared passes are on for this shape
    r = lm.memory_report(N, HID, vocab, CHUNK, lm.ENTRY_CE_MEAN, True, 1)
    assert r["dz_group"] == 1 and r["dz_chunk_bytes"] == 2 * N * 4 * CHUNK
    print(f"[dH passes] n={N} hidden={HID} vocab={vocab} chunk={CHUNK} ({chunks} chunks)", flush=True)
    inp = wlmod.make_inputs(wlmod.custom(n=N, hidden=HID, vocab=vocab, chunk=CHUNK, seed=910,
                                         ignore_frac=0.05))
    d = Dev(inp)
    got = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK)
    again = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK)
    torch.cuda.synchronize()
    assert torch.equal(got["dH"], again["dH"]) and torch.equal(got["dW"], again["dW"])
    assert torch.equal(got["loss"], again["loss"])
    ref = oracle.run(lm.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets, grad=inp.grad)
    rel_check("passes lse", to_np(got["lse"]), ref["lse"])
    rel_check("passes loss", [got["loss"].item()], [ref["loss"]])
    grad_check("passes dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("passes dW", bf16_to_np(got["dW"]), ref["dW"])


def test_shared_dh_pass_accumulate_and_frozen_sides_bitwise():
    """At a shape with shared dH passes (a full pass, then a pass of three
    ending in the ragged chunk): zero-initialised caller accumulators give the
    plain backward's bits, and a dH-only or dW-only backward (W or H frozen)
    gives the same dH or dW as the backward of both."""
    vocab = 1636
    inp = wlmod.make_inputs(wlmod.custom(n=N, hidden=HID, vocab=vocab, chunk=CHUNK, seed=911,
                                         ignore_frac=0.05))
    print(f"[dH passes, accumulate / frozen] n={N} hidden={HID} vocab={vocab} chunk={CHUNK}", flush=True)
    d = Dev(inp)
    plain = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK)
    dh_only = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK, need_dW=False)
    dw_only = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK, need_dH=False)
    dH_acc = torch.zeros(d.H.shape, dtype=torch.float32, device="cuda")
    dW_acc = torch.zeros(d.W.shape, dtype=torch.float32, device="cuda")
    dH, dW = lm.backward_accumulate(lm.ENTRY_CE_MEAN, d.H, d.W, d.t, plain["lse"], d.grad, CHUNK,
                                    dH_acc=dH_acc, dW_acc=dW_acc, out_bf16=True)
    torch.cuda.synchronize()
    assert dh_only["dW"] is None and dw_only["dH"] is None
    assert torch.equal(dh_only["dH"], plain["dH"]) and torch.equal(dw_only["dW"], plain["dW"])
    assert torch.equal(dH, plain["dH"]) and torch.equal(dW, plain["dW"])
    assert torch.equal(dH, dH_acc.to(torch.bfloat16)) and torch.equal(dW, dW_acc.to(torch.bfloat16))
