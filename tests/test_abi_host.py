"""Host-side checks of the C ABI (no GPU needed).

The library loads and exports every function include/lmhead.h declares;
lmhead_workspace_size is a pure host function; every host-checkable error is
returned before anything touches a device. Calls here use fake addresses
and always fail validation first, so nothing is ever launched.
"""
import ctypes
import math
import os
import re

import pytest
import torch

import chunked_lm_head_amd as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")

FAKE = 1 << 20          # a 256-aligned fake address; never dereferenced
BIG = 1 << 40


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == sorted([
        "lmhead_loss_bwd", "lmhead_loss_bwd_accumulate", "lmhead_loss_fwd", "lmhead_loss_fwd_noalloc",
        "lmhead_logprob",
        "lmhead_memory_report", "lmhead_plan_chunk", "lmhead_read_device_error",
        "lmhead_support_kl", "lmhead_support_logprob",
        "lmhead_status_string", "lmhead_support_logprob_kl", "lmhead_workspace_size"])
    L = ctypes.CDLL(lm.LIB_PATH)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    for st in range(8):
        assert lm.lmhead_status_string(st)
    assert lm.lmhead_status_string(99) == "unknown status"


def _p(**kw):
    d = dict(n=64, hidden=256, vocab=1024, chunk=256, num_valid=-1, k=1, flags=0)
    d.update(kw)
    return lm.problem(**d)


def test_workspace_size_rules():
    ws = lm.lmhead_workspace_size
    assert ws(_p(), lm.ENTRY_CE_MEAN, 0) > 0
    assert ws(_p(), lm.ENTRY_CE_MEAN, 1) >= ws(_p(), lm.ENTRY_CE_MEAN, 0)
    # invalid problems report 0
    for bad in (dict(hidden=100), dict(hidden=0), dict(vocab=0), dict(chunk=100), dict(chunk=0),
                dict(n=-1), dict(num_valid=-2), dict(flags=1), dict(n=1 << 31),
                dict(temperature=-1.0), dict(temperature=float("inf")),
                dict(temperature=float("nan"))):
        assert ws(_p(**bad), lm.ENTRY_CE_MEAN, 0) == 0, bad
    assert ws(_p(), 7, 0) == 0
    assert ws(_p(k=0), lm.ENTRY_SUPPORT, 0) == 0
    assert ws(_p(k=1025), lm.ENTRY_SUPPORT, 0) == 0
    # grows with n, vocab and k; the forward does not depend on the chunk
    assert ws(_p(n=128), 0, 0) > ws(_p(n=64), 0, 0)
    assert ws(_p(vocab=4096), 0, 0) > ws(_p(vocab=1024), 0, 0)
    assert ws(_p(k=64), lm.ENTRY_SUPPORT, 0) > ws(_p(k=8), lm.ENTRY_SUPPORT, 0)
    assert ws(_p(chunk=512), 0, 0) == ws(_p(chunk=256), 0, 0)
    # the backward's dL/dz grows with the chunk once a chunk fills the chip
    # (256 row tiles here, whose dL/dz region holds a dH pass of four chunks:
    # 1024 and 2048 of the 4096 columns); below that, consecutive chunks share
    # a recompute launch up to 256 tiles, whose dL/dz then takes the same bytes
    assert ws(_p(n=65536, vocab=4096, chunk=512), 0, 1) > ws(_p(n=65536, vocab=4096, chunk=256), 0, 1)
    assert ws(_p(chunk=512), 0, 1) == ws(_p(chunk=256), 0, 1)
    # headline: 64-bit arithmetic (the dL/dz chunk alone is 2 x 134 MB)
    head = lm.problem(8192, 4096, 151936, 8192, -1, 1, 0)
    b = ws(head, 0, 1)
    assert b > 2 * 2 * 8192 * 8192 and b < 1 << 31
    # the largest vocabulary whose forward grid fits one launch at 2^20 rows
    big = lm.problem(1 << 20, 8192, 4095 * 256, 1 << 20, -1, 1, 0)
    assert ws(big, 0, 1) > 1 << 40    # no 32-bit wrap
    assert ws(_p(n=0), 0, 0) > 0 and ws(_p(n=0), 0, 1) > 0


def test_host_errors_precede_device_use():
    p = _p()
    WSZ = lm.lmhead_workspace_size(p, 0, 1)
    f = lm.lmhead_loss_fwd
    assert f(p, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_ARG
    assert f(p, 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_ARG
    assert f(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, WSZ, 0) == lm.LMHEAD_ERR_ARG
    assert f(p, lm.ENTRY_LOGPROB, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_ARG
    assert f(_p(hidden=96), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_SHAPE
    assert f(p, 0, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_ALIGN
    assert f(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, WSZ, 0) == lm.LMHEAD_ERR_ALIGN
    assert f(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, 0) == lm.LMHEAD_ERR_WORKSPACE
    g = lm.lmhead_logprob
    assert g(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, WSZ, 0) == lm.LMHEAD_ERR_ARG
    s = lm.lmhead_support_logprob_kl
    ps = _p(k=4)
    # kl requested without ref_logq
    assert s(ps, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG
    assert s(_p(k=0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_SHAPE
    b = lm.lmhead_loss_bwd
    assert b(p, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, None, FAKE, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG          # lse missing
    assert b(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG          # CE grad missing
    assert b(ps, 3, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG          # KL grad without ref_logq / saved lp
    assert b(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE + 8, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ALIGN
    assert b(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, 4096, 0) \
        == lm.LMHEAD_ERR_WORKSPACE
    assert b(p, 9, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG


def test_accumulate_host_checks():
    p = _p()
    a = lm.lmhead_loss_bwd_accumulate
    # a bf16 output needs its accumulator
    assert a(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, None, FAKE, FAKE, None, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG
    assert a(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None, None, FAKE, FAKE, BIG, 0) \
        == lm.LMHEAD_ERR_ARG
    assert a(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE + 8, FAKE, None, None, FAKE,
             BIG, 0) == lm.LMHEAD_ERR_ALIGN
    assert a(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, None, None, FAKE,
             4096, 0) == lm.LMHEAD_ERR_WORKSPACE
    assert a(p, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, None, FAKE, FAKE, None, None, FAKE,
             BIG, 0) == lm.LMHEAD_ERR_ARG   # lse missing


def test_temperature_host_checks():
    """The scalar temperature is 0 (off) or positive and finite; the reserved
    word is 0; a per-row temperature array is 4-byte aligned."""
    ws = lm.lmhead_workspace_size
    assert ws(_p(temperature=0.7), 0, 1) == ws(_p(), 0, 1)
    assert ws(_p(temperature=0.7, row_temperature=FAKE), 0, 1) == ws(_p(), 0, 1)
    f = lm.lmhead_loss_fwd
    W = ws(_p(), 0, 1)
    for t in (-0.5, float("inf"), float("nan")):
        assert f(_p(temperature=t), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W, 0) == lm.LMHEAD_ERR_ARG
    q = _p()
    q.reserved = 1
    assert f(q, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W, 0) == lm.LMHEAD_ERR_ARG
    assert f(_p(row_temperature=FAKE + 2), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W, 0) \
        == lm.LMHEAD_ERR_ALIGN
    b = lm.lmhead_loss_bwd
    assert b(_p(row_temperature=FAKE + 1), 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE,
             FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ALIGN
    assert b(_p(temperature=-2.0), 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE,
             FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_status():
    p = _p()
    WSZ = lm.lmhead_workspace_size(p, 0, 1)
    st = lm.lmhead_loss_fwd(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WSZ, 0)
    assert st == lm.LMHEAD_ERR_DEVICE


def test_python_layer_rejects_cpu_tensors():
    H = torch.zeros(4, 64, dtype=torch.bfloat16)
    W = torch.zeros(8, 64, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        lm.ce_loss(H, W, t, chunk=256)


def test_support_split_and_padding_host_checks():
    ws = lm.lmhead_workspace_size
    # the padding flag belongs to the support entries only
    assert ws(_p(flags=lm.FLAG_PADDED_IDS), lm.ENTRY_CE_MEAN, 0) == 0
    assert ws(_p(flags=lm.FLAG_PADDED_IDS, k=8), lm.ENTRY_SUPPORT, 1) > 0
    assert ws(_p(flags=2, k=8), lm.ENTRY_SUPPORT, 0) == 0
    # KL-only: a small forward workspace, no chunk-sized backward buffers
    kl_f = ws(_p(k=8), lm.ENTRY_SUPPORT_KL, 0)
    kl_b = ws(_p(k=8), lm.ENTRY_SUPPORT_KL, 1)
    assert 0 < kl_f <= 256 < kl_b < ws(_p(k=8), lm.ENTRY_SUPPORT, 1)
    assert ws(_p(k=8, chunk=512), lm.ENTRY_SUPPORT_KL, 1) == kl_b
    assert ws(_p(k=0), lm.ENTRY_SUPPORT_KL, 0) == 0
    assert ws(_p(n=1 << 22, k=1024), lm.ENTRY_SUPPORT_KL, 0) == 0      # n * k >= 2^31
    assert ws(_p(n=1 << 22, k=1024), lm.ENTRY_SUPPORT, 0) == 0         # int32 buckets too
    pk = _p(k=8)
    f = lm.lmhead_support_kl
    assert f(pk, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG   # ref_logq
    assert f(pk, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG   # kl
    assert f(pk, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ALIGN
    assert f(pk, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0) == lm.LMHEAD_ERR_WORKSPACE
    g = lm.lmhead_support_logprob
    assert g(pk, FAKE, FAKE, FAKE, None, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG          # lp
    b = lm.lmhead_loss_bwd
    # the KL-only backward takes no lp gradient and needs the saved log p_hat
    assert b(pk, lm.ENTRY_SUPPORT_KL, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
             FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG
    assert b(pk, lm.ENTRY_SUPPORT_KL, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE, FAKE,
             FAKE, BIG, 0) == lm.LMHEAD_ERR_ARG
    r = lm.memory_report(64, 256, 1024, 256, lm.ENTRY_SUPPORT_KL, True, 8)
    assert r["partials_bytes"] == r["dz_chunk_bytes"] == 0
    assert r["caller_output_bytes"] == 4 * 64 * 8 + 4 * 64 + 2 * 64 * 256 + 2 * 1024 * 256


def test_support_entries_reject_int32_entry_counts():
    """Both support entries index their (row, candidate) entries with int32
    (the dense entry's per-tile buckets and offset scans, the KL-only entry's
    inverse index), so n * k above 2^31 - 1 is a shape error before anything
    is enqueued; n * k = 2^31 - 1024 is accepted."""
    over = dict(n=1 << 21, k=1024, hidden=64, vocab=4096, chunk=4096)   # n k = 2^31
    under = dict(over, n=(1 << 21) - 1)
    ws = lm.lmhead_workspace_size
    for entry in (lm.ENTRY_SUPPORT, lm.ENTRY_SUPPORT_KL):
        for bwd in (0, 1):
            assert ws(_p(**over), entry, bwd) == 0, (entry, bwd)
            assert ws(_p(**under), entry, bwd) > 0, (entry, bwd)
    # the single-id entries ignore k
    assert ws(_p(**over), lm.ENTRY_CE_MEAN, 1) > 0
    p = _p(**over)
    S = lm.LMHEAD_ERR_SHAPE
    assert lm.lmhead_support_logprob_kl(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == S
    assert lm.lmhead_support_logprob(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == S
    assert lm.lmhead_support_kl(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == S
    for entry in (lm.ENTRY_SUPPORT, lm.ENTRY_SUPPORT_KL):
        grad = FAKE if entry == lm.ENTRY_SUPPORT else None
        assert lm.lmhead_loss_bwd(p, entry, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, grad, FAKE, FAKE, FAKE,
                                  FAKE, BIG, 0) == S
        assert lm.lmhead_loss_bwd_accumulate(p, entry, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, grad, FAKE,
                                             FAKE, FAKE, None, None, FAKE, BIG, 0) == S
    with pytest.raises(lm.LMHeadError) as e:
        lm.memory_report(over["n"], 64, 4096, 4096, lm.ENTRY_SUPPORT, True, 1024)
    assert e.value.status == S


def test_launch_sizes_are_bounded():
    """One launch holds at most 2^32 - 1 work-items: the per-row kernels (8
    threads per padded row, 64 for the support entries), the tile kernels (one
    256-thread workgroup per 256 x 256 tile of rows x vocabulary or rows x
    hidden) and the KL-only entry's per-id dW pass (64 threads per id) must
    each fit, or the call is a shape error before any launch. Each rule is
    checked on both sides of its boundary."""
    ws = lm.lmhead_workspace_size
    top = (1 << 32) - 1
    S = lm.LMHEAD_ERR_SHAPE
    # 8 threads per padded row
    n8 = top // 8 // 256 * 256
    assert ws(_p(n=n8, hidden=64, vocab=256), lm.ENTRY_CE_MEAN, 1) > 0
    assert ws(_p(n=n8 + 1, hidden=64, vocab=256), lm.ENTRY_CE_MEAN, 1) == 0
    assert ws(_p(n=n8 + 1, hidden=64, vocab=256), lm.ENTRY_LOGPROB, 0) == 0
    # 64 threads per padded row for the support entries
    n64 = top // 64 // 256 * 256
    for e in (lm.ENTRY_SUPPORT, lm.ENTRY_SUPPORT_KL):
        assert ws(_p(n=n64, hidden=64, vocab=256, k=1), e, 1) > 0
        assert ws(_p(n=n64 + 1, hidden=64, vocab=256, k=1), e, 1) == 0
    # one workgroup per tile: rows x vocabulary at the 151,936-id vocabulary
    tv = -(-151936 // 256)
    nt = (top // 256) // tv * 256
    assert nt == 7230464
    assert ws(_p(n=nt, hidden=4096, vocab=151936, chunk=8192), lm.ENTRY_CE_MEAN, 1) > 0
    assert ws(_p(n=nt + 1, hidden=4096, vocab=151936, chunk=8192), lm.ENTRY_CE_MEAN, 1) == 0
    assert ws(_p(n=nt + 1, hidden=4096, vocab=151936, chunk=8192), lm.ENTRY_CE_MEAN, 0) == 0
    # ... and rows x hidden, when the hidden size has more tiles than the vocabulary
    nh = (top // 256) // 256 * 256
    assert ws(_p(n=nh, hidden=65536, vocab=256), lm.ENTRY_LOGPROB, 1) > 0
    assert ws(_p(n=nh + 1, hidden=65536, vocab=256), lm.ENTRY_LOGPROB, 1) == 0
    # the KL-only entry has no tile pass (the rows x vocabulary rule does not
    # apply) but 64 threads per vocabulary id
    assert ws(_p(n=nt + 1, hidden=4096, vocab=151936, chunk=8192, k=4), lm.ENTRY_SUPPORT_KL, 1) > 0
    vk = top // 64 // 4 * 4
    assert ws(_p(n=256, hidden=64, vocab=vk, chunk=256, k=4), lm.ENTRY_SUPPORT_KL, 1) > 0
    assert ws(_p(n=256, hidden=64, vocab=vk + 1, chunk=256, k=4), lm.ENTRY_SUPPORT_KL, 1) == 0
    # the entry points return the same shape error before touching a device
    p = _p(n=nt + 1, hidden=4096, vocab=151936, chunk=8192)
    assert lm.lmhead_loss_fwd(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == S
    assert lm.lmhead_loss_bwd(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                              BIG, 0) == S


def test_chunk_width_is_capped():
    """dL/dz of one chunk is read with a row pitch of the padded chunk width,
    256 rows per buffer range below 2^31 bytes: round_up(min(chunk, vocab),
    256) above 2^22 - 256 is a shape error for every entry with a
    vocabulary-wide pass (the KL-only entry has none and ignores the chunk)."""
    cap = (1 << 22) - 256
    ws = lm.lmhead_workspace_size
    big_v = 1 << 23
    assert ws(_p(hidden=64, vocab=big_v, chunk=cap), lm.ENTRY_CE_MEAN, 1) > 0
    assert ws(_p(hidden=64, vocab=big_v, chunk=cap + 256), lm.ENTRY_CE_MEAN, 1) == 0
    assert ws(_p(hidden=64, vocab=big_v, chunk=cap + 256), lm.ENTRY_CE_MEAN, 0) == 0
    # a chunk wider than the vocabulary counts as the vocabulary's width
    assert ws(_p(hidden=64, vocab=cap, chunk=1 << 30), lm.ENTRY_LOGPROB, 1) > 0
    assert ws(_p(hidden=64, vocab=cap + 1, chunk=1 << 30), lm.ENTRY_LOGPROB, 1) == 0
    assert ws(_p(hidden=64, vocab=big_v, chunk=1 << 23, k=4), lm.ENTRY_SUPPORT, 1) == 0
    assert ws(_p(hidden=64, vocab=big_v, chunk=1 << 23, k=4), lm.ENTRY_SUPPORT_KL, 1) > 0
    p = _p(hidden=64, vocab=big_v, chunk=1 << 23)
    assert lm.lmhead_loss_fwd(p, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, BIG, 0) == lm.LMHEAD_ERR_SHAPE
    assert lm.lmhead_loss_bwd(p, 0, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                              BIG, 0) == lm.LMHEAD_ERR_SHAPE
    # the planner never goes past the cap, whatever the budget
    c = lm.plan_chunk(64, 64, big_v, 1 << 45)
    assert c <= cap and c % 256 == 0 and ws(_p(hidden=64, vocab=big_v, chunk=c), 0, 1) > 0
    assert c == 256 * -(-big_v // 3 // 256) + (256 if big_v % 3 else 0) or math.ceil(big_v / c) == 3


def test_noalloc_forward_host_checks():
    """The allocation-free forward refuses, before touching a device, a problem
    whose forward workspace exceeds its static buffer, and a non-CE entry."""
    big = lm.problem(1 << 16, 256, 1 << 17, 1024, -1, 1)
    assert lm.lmhead_workspace_size(big, 0, 0) > lm.STATIC_SCRATCH_BYTES
    f = lm.lmhead_loss_fwd_noalloc
    assert f(big, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == lm.LMHEAD_ERR_SCRATCH
    assert f(_p(), lm.ENTRY_LOGPROB, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == lm.LMHEAD_ERR_ARG
    assert f(_p(hidden=96), 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == lm.LMHEAD_ERR_SHAPE
    assert "static scratch" in lm.lmhead_status_string(lm.LMHEAD_ERR_SCRATCH)
