"""The allocation-free forward (lmhead_loss_fwd_noalloc) against the
workspace form (lmhead_loss_fwd) through the C ABI: same results bit for bit,
on two calls in a row, the second with a smaller problem (the static buffer
keeps the first call's contents), for CE mean and sum; both also against the
oracle; a problem past the buffer's size is refused before any launch."""
import numpy as np
import pytest
import torch

import chunked_lm_head_amd as lm
import oracle
import workloads as wlmod
from gpu_util import rel_check

pytestmark = pytest.mark.gpu

SHAPES = [  # (n, hidden, vocab, chunk, ignore fraction, seed): the second is smaller
    (300, 256, 5000, 1024, 0.1, 71),
    (100, 128, 3000, 512, 0.2, 72),
]


def _dev(inp):
    H = torch.from_numpy(inp.H.view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(inp.targets).cuda()
    return H, W, t


@pytest.mark.parametrize("entry", [lm.ENTRY_CE_MEAN, lm.ENTRY_CE_SUM])
def test_noalloc_forward_matches_workspace_form(entry):
    for n, hidden, vocab, chunk, ign, seed in SHAPES:
        print(f"[noalloc] entry {entry} n={n} hidden={hidden} vocab={vocab}", flush=True)
        wl = wlmod.custom(n=n, hidden=hidden, vocab=vocab, chunk=chunk, ignore_frac=ign, seed=seed)
        inp = wlmod.make_inputs(wl)
        H, W, t = _dev(inp)
        p = lm.problem(n, hidden, vocab, chunk, -1, 1)
        ws_bytes = lm.lmhead_workspace_size(p, entry, 0)
        assert 0 < ws_bytes <= lm.STATIC_SCRATCH_BYTES
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        loss_a = torch.empty(1, dtype=torch.float32, device="cuda")
        lse_a = torch.empty(n, dtype=torch.float32, device="cuda")
        loss_b = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        lse_b = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        assert lm.lmhead_loss_fwd(p, entry, H, W, t, loss_a, lse_a, ws, ws_bytes) == lm.LMHEAD_OK
        assert lm.lmhead_loss_fwd_noalloc(p, entry, H, W, t, loss_b, lse_b) == lm.LMHEAD_OK
        torch.cuda.synchronize()
        assert torch.equal(loss_a, loss_b), (loss_a.item(), loss_b.item())
        assert torch.equal(lse_a, lse_b)
        ref = oracle.run(entry, inp.H, inp.W, targets=inp.targets, backward=False)
        rel_check("noalloc loss", loss_b.cpu().numpy().astype(np.float64), np.array([ref["loss"]]))
        rel_check("noalloc lse", lse_b.cpu().numpy().astype(np.float64), ref["lse"])


def test_noalloc_refuses_problems_past_the_buffer():
    # forward workspace = header + lse + (max, sum) per 256-column tile and row + ...
    p = lm.problem(1 << 16, 256, 1 << 17, 1024, -1, 1)
    assert lm.lmhead_workspace_size(p, lm.ENTRY_CE_MEAN, 0) > lm.STATIC_SCRATCH_BYTES
    fake = 1 << 20
    assert lm.lmhead_loss_fwd_noalloc(p, lm.ENTRY_CE_MEAN, fake, fake, fake, fake, fake) \
        == lm.LMHEAD_ERR_SCRATCH
    assert lm.lmhead_loss_fwd_noalloc(p, lm.ENTRY_LOGPROB, fake, fake, fake, fake, fake) \
        == lm.LMHEAD_ERR_ARG
