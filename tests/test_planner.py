"""Memory report and memory-budgeted chunk planner (pure host functions of the
C ABI; no GPU needed)."""
import math

import pytest

import chunked_lm_head_amd as lm

HEAD = dict(n=8192, hidden=4096, vocab=151936)


def _ws(chunk, entry=0, k=1, **shape):
    s = dict(HEAD)
    s.update(shape)
    return lm.lmhead_workspace_size(lm.problem(s["n"], s["hidden"], s["vocab"], chunk, -1, k),
                                    entry, 1)


def test_report_matches_workspace_and_layout():
    for entry, k in ((0, 1), (2, 1), (3, 64)):
        r = lm.memory_report(8192, 4096, 151936, 8192, entry, True, k)
        assert r["workspace_bytes"] == _ws(8192, entry, k)
        assert r["chunk"] == 8192 and r["chunks"] == 19
        assert r["dz_chunk_bytes"] == 2 * 8192 * 8192              # one chunk of G, bf16
        assert r["dh_acc_bytes"] == 4 * 8192 * 4096
        assert r["partials_bytes"] == 8 * 594 * 8192
        parts = r["dz_chunk_bytes"] + r["dh_acc_bytes"]
        assert parts <= r["workspace_bytes"] <= parts + (1 << 20) + 4 * 8192 * (k + 2) * 2
        f = lm.memory_report(8192, 4096, 151936, 8192, entry, False, k)
        assert f["workspace_bytes"] == f["forward_bytes"] == r["forward_bytes"]
        assert f["dz_chunk_bytes"] == f["dh_acc_bytes"] == 0
        assert f["partials_bytes"] <= f["forward_bytes"]
    # caller outputs: CE: loss + lse; backward adds bf16 dH and dW
    r = lm.memory_report(8192, 4096, 151936, 8192, 0, True, 1)
    assert r["caller_output_bytes"] == 4 + 4 * 8192 + 2 * 8192 * 4096 + 2 * 151936 * 4096
    s = lm.memory_report(100, 256, 1000, 512, 3, False, 16)
    assert s["caller_output_bytes"] == 4 * 100 + 4 * 100 * 16 + 4 * 100


@pytest.mark.parametrize("budget_mib", [300, 420, 600, 1024, 4096])
def test_plan_fits_and_uses_fewest_passes(budget_mib):
    budget = budget_mib << 20
    c = lm.plan_chunk(8192, 4096, 151936, budget)
    assert c % 256 == 0 and c >= 256
    assert _ws(c) <= budget
    passes = math.ceil(151936 / c)
    # no chunk with fewer passes fits, and the chunk is the smallest for its pass count
    if passes > 1:
        fewer = 256 * math.ceil(math.ceil(151936 / (passes - 1)) / 256)
        assert _ws(fewer) > budget
    assert c == 256 * math.ceil(math.ceil(151936 / passes) / 256)


def test_plan_examples_and_errors():
    # a budget of exactly the 8192 workspace plans 8192 (19 passes either way)
    assert lm.plan_chunk(8192, 4096, 151936, _ws(8192)) == 8192
    # unlimited budget: one pass over the whole (256-padded) vocabulary
    assert lm.plan_chunk(64, 256, 1000, 1 << 40) == 1024
    # too small for a 256 chunk
    with pytest.raises(lm.LMHeadError) as e:
        lm.plan_chunk(8192, 4096, 151936, 1 << 20)
    assert e.value.status == lm.LMHEAD_ERR_WORKSPACE
    with pytest.raises(lm.LMHeadError) as e:
        lm.plan_chunk(8192, 100, 151936, 1 << 30)
    assert e.value.status == lm.LMHEAD_ERR_SHAPE
    # the support entry's candidates add to the workspace, never to fewer bytes
    assert lm.plan_chunk(8192, 4096, 151936, 600 << 20, entry=3, k=64) <= \
        lm.plan_chunk(8192, 4096, 151936, 600 << 20)


@pytest.mark.parametrize("shape", [dict(n=256, hidden=4096, vocab=151936),
                                   dict(n=200, hidden=512, vocab=5000),
                                   dict(n=1024, hidden=2048, vocab=151936)])
def test_plan_always_fits_with_dh_split_partials(shape):
    """Small batches hold the dH K-split's fp32 partials, whose slice count
    follows the chunk's K steps and can fall as the chunk widens, so the
    workspace is not monotone in the chunk there. Whatever the budget, the
    planned chunk's workspace fits it."""
    ws = [_ws(c, **shape) for c in range(256, 256 * math.ceil(shape["vocab"] / 256) + 1, 256)]
    assert all(w > 0 for w in ws)
    lo, hi = min(ws), max(ws)
    for i in range(41):
        budget = lo + (hi - lo) * i // 40
        c = lm.plan_chunk(shape["n"], shape["hidden"], shape["vocab"], budget)
        assert c % 256 == 0 and _ws(c, **shape) <= budget, (budget, c)


def test_report_lists_dh_split_partials():
    """Small batches: the fp32 partials of the dH K-split are listed, S slices
    of [n, hidden] (n = 256, Hd = 4096, chunk 8192: 16 slices; the 4480-wide
    tail chunk takes fewer); none at the headline or without the backward."""
    r = lm.memory_report(256, 4096, 151936, 8192, 0, True, 1)
    assert r["dh_split_bytes"] == 16 * 4 * 256 * 4096
    parts = r["dz_chunk_bytes"] + r["dh_acc_bytes"] + r["dh_split_bytes"]
    assert parts <= r["workspace_bytes"] <= parts + (1 << 20)
    assert lm.memory_report(256, 4096, 151936, 8192, 0, False, 1)["dh_split_bytes"] == 0
    assert lm.memory_report(8192, 4096, 151936, 8192, 0, True, 1)["dh_split_bytes"] == 0
    # chunk 512 has 8 K steps: too few to split
    assert lm.memory_report(256, 4096, 151936, 512, 0, True, 1)["dh_split_bytes"] == 0
