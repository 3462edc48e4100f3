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
        assert r["dz_chunk_bytes"] == 2 * 8192 * 32768             # four chunks of G (one dH pass), bf16
        assert r["dh_acc_bytes"] == 4 * 8192 * 4096
        assert r["partials_bytes"] == 8 * 594 * 8192
        # H in fragment order, and in the backward H^T too
        assert r["operand_copy_bytes"] == 2 * (2 * 8192 * 4096)
        parts = r["dz_chunk_bytes"] + r["dh_acc_bytes"] + r["operand_copy_bytes"]
        # the rest: header, per-row coefficients and, with candidates, the
        # per-tile hit list and its merge-sort buffer (4 N k bytes each)
        assert parts <= r["workspace_bytes"] <= parts + (1 << 20) + 4 * 8192 * (k + 2) * 3
        f = lm.memory_report(8192, 4096, 151936, 8192, entry, False, k)
        assert f["workspace_bytes"] == f["forward_bytes"] == r["forward_bytes"]
        assert f["dz_chunk_bytes"] == f["dh_acc_bytes"] == 0
        assert f["operand_copy_bytes"] == 2 * 8192 * 4096
        assert f["partials_bytes"] + f["operand_copy_bytes"] <= f["forward_bytes"]
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
    """Small batches hold the dH K-split's fp32 partials (sized by the shape)
    and the dL/dz of several chunks (sized to grow with the chunk), so the
    workspace never shrinks as the chunk widens. Whatever the budget, the
    planned chunk's workspace fits it."""
    ws = [_ws(c, **shape) for c in range(256, 256 * math.ceil(shape["vocab"] / 256) + 1, 256)]
    assert all(w > 0 for w in ws)
    assert all(a <= b for a, b in zip(ws, ws[1:]))
    lo, hi = min(ws), max(ws)
    for i in range(41):
        budget = lo + (hi - lo) * i // 40
        c = lm.plan_chunk(shape["n"], shape["hidden"], shape["vocab"], budget)
        assert c % 256 == 0 and _ws(c, **shape) <= budget, (budget, c)


def test_report_lists_dh_split_partials():
    """Small batches: the fp32 partials of the dH K-split are listed, one
    [n, hidden] plane per (chunk, slice) unit of a launch, at most 16 and at
    most 256 dH tiles' worth (n = 256, Hd = 4096: 16 dH tiles, so 16 planes,
    whatever the chunk); none at the headline (512 dH tiles) or without the
    backward."""
    r = lm.memory_report(256, 4096, 151936, 8192, 0, True, 1)
    assert r["dh_split_bytes"] == 16 * 4 * 256 * 4096
    parts = r["dz_chunk_bytes"] + r["dh_acc_bytes"] + r["dh_split_bytes"] + r["operand_copy_bytes"]
    assert parts <= r["workspace_bytes"] <= parts + (1 << 20)
    assert lm.memory_report(256, 4096, 151936, 8192, 0, False, 1)["dh_split_bytes"] == 0
    assert lm.memory_report(8192, 4096, 151936, 8192, 0, True, 1)["dh_split_bytes"] == 0
    for chunk in (256, 512, 4096, 65536):
        assert lm.memory_report(256, 4096, 151936, chunk, 0, True, 1)["dh_split_bytes"] == 16 * 4 * 256 * 4096
    # 64 dH tiles (n = 1024): 4 planes; 128 (n = 2048): 2; 129 .. : none
    assert lm.memory_report(1024, 4096, 151936, 8192, 0, True, 1)["dh_split_bytes"] == 4 * 4 * 1024 * 4096
    assert lm.memory_report(2048, 4096, 151936, 8192, 0, True, 1)["dh_split_bytes"] == 2 * 4 * 2048 * 4096
    assert lm.memory_report(2048, 4352, 151936, 8192, 0, True, 1)["dh_split_bytes"] == 0
    # the planes never exceed 256 fp32 tiles of 256 x 256 (64 MiB)
    for n in (1, 200, 256, 513, 1024, 2048, 4000):
        for hidden in (64, 256, 512, 4096, 8192):
            b = lm.memory_report(n, hidden, 151936, 8192, 0, True, 1)["dh_split_bytes"]
            assert b <= 64 << 20, (n, hidden, b)


def test_dh_split_slices_are_capped():
    """The dH K-split takes at most 16 slices, so its fp32 partials stay within
    16 x [n, hidden] even where the chunk has many more K steps (n = 256,
    hidden = 256, chunk 32768: 512 K steps, one dH tile)."""
    for chunk in (8192, 32768, 65536):
        r = lm.memory_report(256, 256, 151936, chunk, 0, True, 1)
        assert 0 < r["dh_split_bytes"] <= 16 * 4 * 256 * 256, (chunk, r["dh_split_bytes"])
    assert lm.memory_report(256, 256, 151936, 32768, 0, True, 1)["dh_split_bytes"] == 16 * 4 * 256 * 256


def test_chunks_share_a_dh_pass_region():
    """With at least 256 dH tiles (the headline's 512) four consecutive chunks
    share one dH pass, so the dL/dz region holds min(4 padded chunks, V)
    columns; with fewer dH tiles (n = 2048, hidden 4096: 128) it holds one
    chunk's; the region, and the workspace, never shrink as the chunk widens
    (also past the pairs)."""
    vpad = 152064   # V rounded up to 256
    assert lm.memory_report(8192, 4096, 151936, 8192, 0, True, 1)["dz_chunk_bytes"] == 2 * 8192 * 32768
    assert lm.memory_report(8192, 4096, 151936, 32768, 0, True, 1)["dz_chunk_bytes"] == 2 * 8192 * 131072
    assert lm.memory_report(8192, 4096, 151936, 40960, 0, True, 1)["dz_chunk_bytes"] == 2 * 8192 * vpad
    assert lm.memory_report(8192, 4096, 151936, 100096, 0, True, 1)["dz_chunk_bytes"] == 2 * 8192 * vpad
    assert lm.memory_report(8192, 4096, 151936, 152064, 0, True, 1)["dz_chunk_bytes"] == 2 * 8192 * vpad
    assert lm.memory_report(4096, 4096, 151936, 8192, 0, True, 1)["dz_chunk_bytes"] == 2 * 4096 * 32768
    assert lm.memory_report(2048, 4096, 151936, 8192, 0, True, 1)["dz_chunk_bytes"] == 2 * 2048 * 8192
    prev = 0
    for chunk in sorted(set(list(range(256, 151936 + 256, 256 * 13)) + [8192, 75776, 76032, 152064])):
        w = _ws(chunk)
        assert w >= prev, chunk
        prev = w


def test_small_batch_groups_chunks_per_recompute():
    """A chunk of fewer than 256 tiles of 256 x 256 shares its recompute launch
    with the chunks after it, up to 256 tiles, each in a dL/dz slot of its
    own: n = 256, chunk 8192 has 32 tiles, so 8 chunks (4 MiB of bf16 dL/dz
    each) go together; the headline's 1024 tiles stay one per launch; the
    group never exceeds the chunk count. The region holding the slots is
    sized so that the smallest chunk still needs the least workspace."""
    r = lm.memory_report(256, 4096, 151936, 8192, 0, True, 1)
    assert r["dz_group"] == 8
    assert r["dz_chunk_bytes"] == 8 * 2 * 256 * 8192
    h = lm.memory_report(8192, 4096, 151936, 8192, 0, True, 1)
    assert h["dz_group"] == 1 and h["dz_chunk_bytes"] == 2 * 8192 * 32768
    # 3 tiles per chunk (n = 256, chunk 768): 85 chunks, 255 tiles
    assert lm.memory_report(256, 4096, 151936, 768, 0, True, 1)["dz_group"] == 85
    # 1000 columns: 4 chunks of 256 in all
    t = lm.memory_report(64, 256, 1000, 256, 0, True, 1)
    assert t["dz_group"] == 4 and t["dz_chunk_bytes"] == 4 * 2 * 256 * 256
    # 129 .. 255 tiles: alone (no two fit in 256)
    assert lm.memory_report(2048, 4096, 151936, 4352, 0, True, 1)["dz_group"] == 1    # 136 tiles
    assert lm.memory_report(2048, 4096, 151936, 4096, 0, True, 1)["dz_group"] == 2    # 128 tiles
    # the slots together stay within 256 tiles of bf16 (32 MiB) at any chunk
    for chunk in range(256, 151936 + 256, 256 * 37):
        g = lm.memory_report(256, 4096, 151936, chunk, 0, True, 1)
        tiles = math.ceil(chunk / 256)
        assert 1 <= g["dz_group"] <= g["chunks"]
        assert g["dz_group"] == 1 or g["dz_group"] * tiles <= 256
        slots = g["dz_group"] * 2 * 256 * 256 * tiles
        assert slots <= g["dz_chunk_bytes"] <= max(slots, 32 << 20)
    # the floor: the chunk-256 workspace is the smallest of any chunk; a budget
    # of it plans a chunk, and that chunk fits
    floor = _ws(256, n=256)
    assert all(_ws(c, n=256) >= floor for c in range(256, 151936 + 256, 256 * 7))
    c = lm.plan_chunk(256, 4096, 151936, floor)
    assert c >= 256 and _ws(c, n=256) <= floor
    with pytest.raises(lm.LMHeadError):
        lm.plan_chunk(256, 4096, 151936, floor - 1)


@pytest.mark.parametrize("shape", [dict(n=256, hidden=4096, vocab=151936),
                                   dict(n=200, hidden=512, vocab=5000),
                                   dict(n=2048, hidden=4352, vocab=151936)])
def test_plan_takes_fewest_passes_at_small_batches(shape):
    """The workspace never shrinks as the chunk widens, so the planner's
    bisection finds the fewest vocabulary passes that fit: no chunk with
    fewer passes fits the budget, and the planned chunk fits it."""
    v = shape["vocab"]
    ws = {c: _ws(c, **shape) for c in range(256, 256 * math.ceil(v / 256) + 1, 256)}
    lo, hi = min(ws.values()), max(ws.values())
    for i in range(0, 41, 4):
        budget = lo + (hi - lo) * i // 40
        c = lm.plan_chunk(shape["n"], shape["hidden"], v, budget)
        assert ws[c] <= budget
        passes = math.ceil(v / c)
        assert all(w > budget for cc, w in ws.items() if math.ceil(v / cc) < passes), (budget, c)
