"""GPU parity of the paired dH pass: when a problem has at least 256 dH tiles
of 256 x 256, two consecutive vocabulary chunks share one dH contraction over
both chunks' columns (one fp32 running-sum update per pair). The smallest
shapes where that happens with the full oracle still in reach: 65,536 rows of
hidden 256 (256 row tiles x 1 hidden tile) and 256-wide chunks, so that each
chunk fills the 256 compute units with its own recompute tiles. Vocabularies
of 5 chunks (two pairs and an odd, ragged last chunk) and 4 chunks (the
second pair ends in the ragged chunk)."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import Dev, bf16_to_np, grad_check, rel_check, run_entry, to_np

pytestmark = pytest.mark.gpu

N, HID, CHUNK = 65536, 256, 256


@pytest.mark.parametrize("vocab", [1124, 868])
def test_paired_dh_pass_against_oracle(vocab):
    chunks = -(-vocab // CHUNK)
    # the dL/dz region holds two chunks: the pairing is on for this shape
    r = lm.memory_report(N, HID, vocab, CHUNK, lm.ENTRY_CE_MEAN, True, 1)
    assert r["dz_group"] == 1 and r["dz_chunk_bytes"] == 2 * N * 2 * CHUNK
    print(f"[pairs] n={N} hidden={HID} vocab={vocab} chunk={CHUNK} ({chunks} chunks)", flush=True)
    inp = wlmod.make_inputs(wlmod.custom(n=N, hidden=HID, vocab=vocab, chunk=CHUNK, seed=910,
                                         ignore_frac=0.05))
    d = Dev(inp)
    got = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK)
    again = run_entry(d, lm.ENTRY_CE_MEAN, CHUNK)
    torch.cuda.synchronize()
    assert torch.equal(got["dH"], again["dH"]) and torch.equal(got["dW"], again["dW"])
    assert torch.equal(got["loss"], again["loss"])
    ref = oracle.run(lm.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets, grad=inp.grad)
    rel_check("pairs lse", to_np(got["lse"]), ref["lse"])
    rel_check("pairs loss", [got["loss"].item()], [ref["loss"]])
    grad_check("pairs dH", bf16_to_np(got["dH"]), ref["dH"])
    grad_check("pairs dW", bf16_to_np(got["dW"]), ref["dW"])
