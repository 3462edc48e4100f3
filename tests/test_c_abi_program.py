"""The C ABI used from plain host C++ (tests/c_abi/ce_roundtrip.cpp, built by
the package build with g++ against liblmhead.so and the HIP runtime, no
Python or torch in between). CPU: the program links against the in-tree
library and rejects bad arguments. GPU: a ragged CE problem through the
program gives the same bits as the same calls through the Python binding,
and matches the oracle."""
import os
import struct
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "c_abi", "ce_roundtrip")


def _need_prog():
    if not os.path.exists(PROG):
        pytest.fail(f"{PROG} is missing: run __graft_entry__.build()")


def test_program_links_the_in_tree_library():
    _need_prog()
    out = subprocess.run(["ldd", PROG], capture_output=True, text=True, timeout=60).stdout
    line = [ln for ln in out.splitlines() if "liblmhead.so" in ln]
    assert line and os.path.realpath(line[0].split("=>")[1].split("(")[0].strip()) == \
        os.path.realpath(os.path.join(ROOT, "chunked_lm_head_amd", "liblmhead.so")), out


def test_program_rejects_bad_arguments(tmp_path):
    _need_prog()
    r = subprocess.run([PROG], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    short = tmp_path / "short.bin"
    short.write_bytes(struct.pack("<2q", 1, 64))
    r = subprocess.run([PROG, str(short), str(tmp_path / "out.bin")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "short input" in r.stderr


def write_problem(path, inp, chunk):
    wl = inp.wl
    with open(path, "wb") as f:
        f.write(struct.pack("<4q", wl.n, wl.hidden, wl.vocab, chunk))
        f.write(np.ascontiguousarray(inp.H, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(inp.W, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(inp.targets, dtype=np.int32).tobytes())


def read_result(path, n, hidden, vocab):
    b = open(path, "rb").read()
    o = 0
    loss = np.frombuffer(b, np.float32, 1, o)[0]
    o += 4
    lse = np.frombuffer(b, np.float32, n, o)
    o += 4 * n
    dH = np.frombuffer(b, np.uint16, n * hidden, o).reshape(n, hidden)
    o += 2 * n * hidden
    dW = np.frombuffer(b, np.uint16, vocab * hidden, o).reshape(vocab, hidden)
    o += 2 * vocab * hidden
    code = int(np.frombuffer(b, np.int32, 1, o)[0])
    row = int(np.frombuffer(b, np.int64, 1, o + 4)[0])
    return dict(loss=loss, lse=lse, dH=dH, dW=dW, code=code, row=row)


@pytest.mark.gpu
def test_program_matches_binding_bitwise_and_the_oracle(tmp_path):
    import torch

    import chunked_lm_head_amd as lm
    import oracle
    import workloads as wlmod
    from gpu_util import Dev, grad_check, rel_check

    _need_prog()
    chunk = 512
    inp = wlmod.make_inputs(wlmod.custom(n=300, hidden=512, vocab=1000, chunk=chunk, seed=1500,
                                         ignore_frac=0.1))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    write_problem(src, inp, chunk)
    print(f"running {PROG} on n=300 hidden=512 vocab=1000 chunk=512", flush=True)
    r = subprocess.run([PROG, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = read_result(dst, 300, 512, 1000)
    assert got["code"] == 0 and got["row"] == -1

    d = Dev(inp)
    loss, lse, _ = lm.ce_loss_forward(d.H, d.W, d.t, chunk)
    dH, dW = lm.backward(lm.ENTRY_CE_MEAN, d.H, d.W, d.t, lse, torch.ones(1, device="cuda"), chunk)
    torch.cuda.synchronize()
    assert np.float32(loss.item()).tobytes() == got["loss"].tobytes()
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), got["lse"].view(np.uint32))
    assert np.array_equal(dH.view(torch.int16).cpu().numpy().view(np.uint16), got["dH"])
    assert np.array_equal(dW.view(torch.int16).cpu().numpy().view(np.uint16), got["dW"])

    ref = oracle.run(oracle.ENTRY_CE_MEAN, inp.H, inp.W, targets=inp.targets)
    bf = lambda bits: (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel_check("loss", np.float64(got["loss"]), ref["loss"])
    rel_check("lse", got["lse"].astype(np.float64), ref["lse"])
    grad_check("dH", bf(got["dH"]), ref["dH"])
    grad_check("dW", bf(got["dW"]), ref["dW"])
