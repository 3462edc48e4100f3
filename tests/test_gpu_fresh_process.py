"""Bitwise determinism across processes: a forward + backward computed in a
child Python process gives the same bytes (SHA-256 over every output) as the
same call in this process, for the CE mean, log-prob and support entries."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Runs in both processes: seeded inputs, one entry through the C ABI, the
# digest of every output (device tensors copied to the host as raw bytes).
_DIGEST = r'''
import hashlib, sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import torch
import workloads as wlmod
from gpu_util import Dev, run_entry

def digest(entry):
    d = dict(n=300, hidden=512, vocab=1000, chunk=512, seed=1200 + entry, ignore_frac=0.1,
             entry=entry)
    if entry == wlmod.ENTRY_SUPPORT:
        d.update(k=16, ignore_frac=0.0)
    out = run_entry(Dev(wlmod.make_inputs(wlmod.custom(**d))), entry, 512)
    torch.cuda.synchronize()
    h = hashlib.sha256()
    for name in sorted(out):
        h.update(name.encode())
        h.update(out[name].contiguous().reshape(-1).view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()
'''


def _source():
    return _DIGEST.format(root=ROOT, tests=os.path.join(ROOT, "tests"))


@pytest.mark.parametrize("entry", [0, 2, 3])
def test_child_process_gives_the_same_bits(entry):
    ns = {}
    exec(_source(), ns)
    here = ns["digest"](entry)
    code = _source() + f"\nprint(digest({entry}))\n"
    child = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert child.returncode == 0, child.stderr[-2000:]
    there = child.stdout.strip().splitlines()[-1]
    assert there == here, f"entry {entry}: digest {there} in a fresh process, {here} here"
