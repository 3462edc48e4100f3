"""A whole forward + backward captured into a HIP graph replays to the eager
bits. The entry points allocate nothing, never synchronise and clear memory
with kernels (no memset nodes), so a captured step is an ordinary graph of
kernel launches. Every replay is checked against the eager result, with eager
work on the same buffers and device synchronisations between the replays;
the workspace and the outputs are scribbled over before each replay, so a
replay that skipped a write would be seen."""
import pytest
import torch

import chunked_lm_head_amd as lm
import workloads as wlmod
from gpu_util import Dev

pytestmark = pytest.mark.gpu

CHUNK = 512


def _inputs(entry, **shape):
    d = dict(n=300, hidden=512, vocab=1000, chunk=CHUNK, seed=900 + entry, ignore_frac=0.1,
             entry=entry)
    d.update(shape)
    if entry in (wlmod.ENTRY_SUPPORT, wlmod.ENTRY_SUPPORT_KL):
        d.update(k=16, ignore_frac=0.0)
    return Dev(wlmod.make_inputs(wlmod.custom(**d)))


def _step_fn(d, entry, chunk=CHUNK):
    n, hidden = d.H.shape
    vocab = d.W.shape[0]
    k = d.ids.shape[1] if entry in (lm.ENTRY_SUPPORT, lm.ENTRY_SUPPORT_KL) else 1
    p = lm.problem(n, hidden, vocab, chunk, -1, k)
    ws = lm.workspace(p, entry, True, d.H.device)
    out = dict(dH=torch.empty_like(d.H), dW=torch.empty_like(d.W))
    if entry != lm.ENTRY_SUPPORT_KL:
        out["lse"] = torch.empty(n, dtype=torch.float32, device="cuda")
    if entry == lm.ENTRY_SUPPORT_KL:
        # the KL-only entry: candidate gathers, integer counting sort in the backward
        out["kl"] = torch.empty(n, dtype=torch.float32, device="cuda")
        out["log_phat"] = torch.empty(n, k, dtype=torch.float32, device="cuda")
    elif entry == lm.ENTRY_CE_MEAN:
        out["loss"] = torch.empty(1, dtype=torch.float32, device="cuda")
    elif entry == lm.ENTRY_LOGPROB:
        out["logp"] = torch.empty(n, dtype=torch.float32, device="cuda")
    else:
        out["lp"] = torch.empty(n, k, dtype=torch.float32, device="cuda")
        out["kl"] = torch.empty(n, dtype=torch.float32, device="cuda")

    def step():
        if entry == lm.ENTRY_SUPPORT_KL:
            st = lm.lmhead_support_kl(p, d.H, d.W, d.ids, d.ref_logq, out["kl"], out["log_phat"], ws,
                                      ws.numel())
            assert st == lm.LMHEAD_OK, lm.lmhead_status_string(st)
            st = lm.lmhead_loss_bwd(p, entry, d.H, d.W, d.ids, d.ref_logq, None, out["log_phat"],
                                    None, d.grad_kl, out["dH"], out["dW"], ws, ws.numel())
            assert st == lm.LMHEAD_OK, lm.lmhead_status_string(st)
            return
        if entry == lm.ENTRY_CE_MEAN:
            st = lm.lmhead_loss_fwd(p, entry, d.H, d.W, d.t, out["loss"], out["lse"], ws, ws.numel())
            idx, ref, saved, gkl = d.t, None, None, None
        elif entry == lm.ENTRY_LOGPROB:
            st = lm.lmhead_logprob(p, d.H, d.W, d.t, out["logp"], out["lse"], ws, ws.numel())
            idx, ref, saved, gkl = d.t, None, None, None
        else:
            st = lm.lmhead_support_logprob_kl(p, d.H, d.W, d.ids, d.ref_logq, out["lp"], out["kl"],
                                              out["lse"], ws, ws.numel())
            idx, ref, saved, gkl = d.ids, d.ref_logq, out["lp"], d.grad_kl
        assert st == lm.LMHEAD_OK, lm.lmhead_status_string(st)
        st = lm.lmhead_loss_bwd(p, entry, d.H, d.W, idx, ref, out["lse"], saved, d.grad, gkl,
                                out["dH"], out["dW"], ws, ws.numel())
        assert st == lm.LMHEAD_OK, lm.lmhead_status_string(st)

    return step, out, ws


# the last two: n = 200 rows with chunk 2048 split each chunk's dH contraction
# into K slices (partials, then an ordered join kernel)
@pytest.mark.parametrize("entry,shape", [
    (lm.ENTRY_CE_MEAN, {}), (lm.ENTRY_LOGPROB, {}), (lm.ENTRY_SUPPORT, {}), (lm.ENTRY_SUPPORT_KL, {}),
    (lm.ENTRY_CE_MEAN, dict(n=200, vocab=5000, chunk=2048)),
    (lm.ENTRY_SUPPORT, dict(n=200, vocab=5000, chunk=2048)),
])
def test_graph_replays_match_eager(entry, shape):
    d = _inputs(entry, **shape)
    step, out, ws = _step_fn(d, entry, shape.get("chunk", CHUNK))
    step()
    torch.cuda.synchronize()
    ref = {name: t.clone() for name, t in out.items()}

    # warm up on a side stream, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work on the same memory between replays
        ws.fill_(0x7F)
        for t in out.values():
            t.fill_(float("nan")) if t.dtype == torch.float32 else t.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from the eager result"
        # an eager step between replays leaves the same bits too
        step()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, ref[name]), f"eager step after replay {rep}: {name} differs"
