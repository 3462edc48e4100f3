#!/usr/bin/env python3
"""Benchmark of the chunked LM-head + loss path on one MI355X.

One step = the whole hot path over one batch: forward (label scan, logits
tiles with the online max / sum-exp epilogue, per-row logsumexp merge, loss
reduction) and backward (row coefficients, per-chunk logits recompute with
the dL/dz epilogue, dW and dH contractions). Inputs are resident in HBM
before the timed region; outputs and workspace are allocated once.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0
METRIC = "fused LM-head+CE fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak) at V=151936"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "mid", "logprob", "support", "tiny", "small"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--kl-only", action="store_true",
                    help="with --workload support: time the KL-only support entry "
                         "(lmhead_support_kl + its backward) instead of the dense one")
    ap.add_argument("--vendor-line", action="store_true",
                    help="also time the vendor library's plain bf16 GEMMs (torch.matmul) at the "
                         "path's shapes, outside the timed region, and report them under vendor_gemm")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (counter calibration)")
    ap.add_argument("--other-steps", type=int, default=5,
                    help="timed steps of each other workload (log-prob, dense support, KL-only "
                         "support) reported under other_workloads; 0 skips them")
    return ap.parse_args()


KERNEL_SOURCES = ["chunked_lm_head_amd/csrc/gemm_core.h", "chunked_lm_head_amd/csrc/lmhead_kernels.hip",
                  "chunked_lm_head_amd/csrc/lmhead_kernels.h", "chunked_lm_head_amd/build.py"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_tiles_headline_traffic.json")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch of the forward tiles kernel, from the committed
    FETCH_SIZE / WRITE_SIZE counter runs, if they were taken on the current
    kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import __graft_entry__

    __graft_entry__.ensure_built()   # builds only in a fresh checkout

    import torch

    import chunked_lm_head_amd as lm
    import workloads

    if args.copy_probe:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE readings
        # calibrate the counters to bytes
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": src.numel() * 4}), flush=True)
        return

    wl = workloads.WORKLOADS[args.workload]
    if args.kl_only and wl.entry != workloads.ENTRY_SUPPORT:
        print("--kl-only needs a support workload (--workload support)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = workloads.make_inputs(wl)
    log(f"inputs for {wl.name} drawn in {time.time() - t0:.1f}s")

    entry = workloads.ENTRY_SUPPORT_KL if args.kl_only else wl.entry
    run = Runner(torch, lm, workloads, wl, inp, entry, dev)
    t = time_steps(torch, run, args.steps, args.warmup)
    K = args.steps
    wall, ms_per_step = t["wall_s"], t["ms_per_step"]
    fwd_ms, bwd_ms, step_ms = t["fwd_ms"], t["bwd_ms"], t["step_ms"]
    deterministic = t["deterministic"]
    k = run.k
    H, W, stream = run.H, run.W, run.stream

    flops = wl.flops_fwd_bwd
    tokens_per_s = wl.n * K / wall
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    fwd_flops = 2.0 * wl.n * wl.vocab * wl.hidden
    fwd_avg_ms = float(np.mean(fwd_ms))
    achieved = fwd_flops / (fwd_avg_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normals, no checkpoint or dataset)",
        "config": {
            "workload": f"{wl.name}: N={wl.n} tokens, Hd={wl.hidden}, V={wl.vocab}, "
                        f"chunk {wl.chunk}, entry {['ce_mean', 'ce_sum', 'logprob', 'support', 'support_kl'][entry]}"
                        + (f", K={wl.k}" if k > 1 else "") + ", forward + backward (dH, dW)",
            "n": wl.n, "hidden": wl.hidden, "vocab": wl.vocab, "chunk": wl.chunk,
            "seed": wl.seed,
        },
        "tflops_8nvh": round(tflops, 2),
        "tflops_6nvh_model": round(tflops * 6 / 8, 2),
        "pct_bf16_peak": round(100 * tflops / BF16_PEAK_TFLOPS, 2),
        "fwd_ms": round(fwd_avg_ms, 4),
        "bwd_ms": round(float(np.mean(bwd_ms)), 4),
        "step_ms_events": {"median": round(float(np.median(step_ms)), 4),
                           "min": round(float(np.min(step_ms)), 4),
                           "max": round(float(np.max(step_ms)), 4)},
        "deterministic_repeat": deterministic,
        "roofline": {
            "kernel": "fwd_tiles_kernel (logits GEMM + online max/sum-exp epilogue, one launch over all of V)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": recorded_traffic(wl.name),
            "timing": "HIP events around lmhead_loss_fwd on its stream (label scan, row merge "
                      "and loss reduction add <1% next to the tiles kernel)",
        },
    }
    # the backward's three contractions per chunk (recompute, dW, dH: 3 x 2NVHd
    # flops) as one figure over the whole lmhead_loss_bwd call, which also
    # holds the row-coefficient pass and every chunk's epilogues
    bwd_avg_ms = float(np.mean(bwd_ms))
    bwd_achieved = 3.0 * fwd_flops / (bwd_avg_ms * 1e-3) / 1e12
    out["roofline_backward"] = {
        "kernels": "per vocabulary chunk bwd_logit_grad_kernel and its dW tiles; dH once per pass of up to "
                   "four chunks, with the pass's last dW tiles (bwd_dw_kernel, bwd_dwdh_kernel; small batches "
                   "split dH), with the coefficient pass",
        "bound": "mfma",
        "achieved": round(bwd_achieved, 2),
        "peak": BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(bwd_achieved / BF16_PEAK_TFLOPS, 4),
        "timing": "HIP events around lmhead_loss_bwd on its stream",
    }
    if entry == workloads.ENTRY_SUPPORT_KL:
        out.pop("roofline_backward")
        # the KL-only entry gathers rows instead of contracting over V: its
        # forward kernel reads one W row per (row, candidate) and H once
        gather_bytes = 2.0 * wl.n * k * wl.hidden + 2.0 * wl.n * wl.hidden + 12.0 * wl.n * k + 4.0 * wl.n
        gbs = gather_bytes / (fwd_avg_ms * 1e-3) / 1e9
        for key in ("tflops_8nvh", "tflops_6nvh_model", "pct_bf16_peak"):
            out.pop(key)
        out["metric"] = "KL-only support entry fwd+bwd tokens/s at V=151936, K=64"
        out["config"]["workload"] = (f"{wl.name}: N={wl.n} tokens, Hd={wl.hidden}, V={wl.vocab}, "
                                     f"K={k}, entry support_kl (KL(q_ref || p_hat) over the candidates, "
                                     "no vocabulary-wide pass), forward + backward (dH, dW)")
        out["roofline"] = {
            "kernel": "cand_kl_fwd_kernel (one wave per row gathers its K rows of W)",
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": int(gather_bytes),
            "timing": "HIP events around lmhead_support_kl on its stream (the id scan adds <2%); "
                      "W rows repeat across rows, so part of the gathered bytes come from the caches",
        }
    if args.vendor_line and entry != workloads.ENTRY_SUPPORT_KL:
        out["vendor_gemm"] = vendor_gemm(torch, H, W, wl, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds, entry)
    if args.other_steps > 0 and args.workload == "headline" and not args.kl_only:
        del run, H, W, inp
        torch.cuda.empty_cache()
        out["other_workloads"] = other_workloads(torch, lm, workloads, dev, args.other_steps)
    print(json.dumps(out), flush=True)


class Runner:
    """One entry's inputs on the device, its outputs and workspace allocated
    once, and its forward / backward through the C ABI on the current stream."""

    def __init__(self, torch, lm, workloads, wl, inp, entry, dev):
        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.torch, self.lm, self.entry = torch, lm, entry
        E = workloads
        self.E = E
        self.H, self.W = bf16(inp.H), bf16(inp.W)
        k = wl.k if entry in (E.ENTRY_SUPPORT, E.ENTRY_SUPPORT_KL) else 1
        self.k = k
        self.idx = torch.from_numpy(inp.targets if inp.targets is not None else inp.ids).to(dev)
        self.grad = torch.from_numpy(inp.grad).to(dev)
        self.ref_logq = torch.from_numpy(inp.ref_logq).to(dev) if inp.ref_logq is not None else None
        self.grad_kl = torch.from_numpy(inp.grad_kl).to(dev) if inp.grad_kl is not None else None
        self.p = lm.problem(wl.n, wl.hidden, wl.vocab, wl.chunk, -1, k)
        self.ws_bytes = lm.lmhead_workspace_size(self.p, entry, 1)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.lse = torch.empty(wl.n, dtype=torch.float32, device=dev)
        self.row_out = torch.empty((wl.n, k) if k > 1 else (wl.n,), dtype=torch.float32, device=dev)
        self.kl = torch.empty(wl.n, dtype=torch.float32, device=dev)
        self.dH = torch.empty_like(self.H)
        self.dW = torch.empty_like(self.W)
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream
        log(f"{wl.name}: workspace {self.ws_bytes / 2**20:.1f} MiB; dtype bf16; chunk {wl.chunk}")

    def fwd(self):
        lm, E, e = self.lm, self.E, self.entry
        if e in (E.ENTRY_CE_MEAN, E.ENTRY_CE_SUM):
            st = lm.lmhead_loss_fwd(self.p, e, self.H, self.W, self.idx, self.loss, self.lse, self.ws,
                                    self.ws_bytes, self.sp)
        elif e == E.ENTRY_LOGPROB:
            st = lm.lmhead_logprob(self.p, self.H, self.W, self.idx, self.row_out, self.lse, self.ws,
                                   self.ws_bytes, self.sp)
        elif e == E.ENTRY_SUPPORT:
            st = lm.lmhead_support_logprob_kl(self.p, self.H, self.W, self.idx, self.ref_logq, self.row_out,
                                              self.kl, self.lse, self.ws, self.ws_bytes, self.sp)
        else:   # KL-only: row_out holds log p_hat
            st = lm.lmhead_support_kl(self.p, self.H, self.W, self.idx, self.ref_logq, self.kl, self.row_out,
                                      self.ws, self.ws_bytes, self.sp)
        if st:
            raise lm.LMHeadError(st, "forward")

    def bwd(self):
        lm, E, e = self.lm, self.E, self.entry
        if e == E.ENTRY_SUPPORT_KL:
            st = lm.lmhead_loss_bwd(self.p, e, self.H, self.W, self.idx, self.ref_logq, None, self.row_out,
                                    None, self.grad_kl, self.dH, self.dW, self.ws, self.ws_bytes, self.sp)
        else:
            saved = self.row_out if e == E.ENTRY_SUPPORT else None
            st = lm.lmhead_loss_bwd(self.p, e, self.H, self.W, self.idx, self.ref_logq, self.lse, saved,
                                    self.grad, self.grad_kl, self.dH, self.dW, self.ws, self.ws_bytes, self.sp)
        if st:
            raise lm.LMHeadError(st, "backward")

    def outputs(self):
        return (self.loss, self.lse, self.row_out, self.kl, self.dH, self.dW)

    def snapshot(self):
        """Device copies of the outputs, enqueued on the calls' stream (no host
        round trip, so the next step starts right behind them)."""
        with self.torch.cuda.stream(self.stream):
            return tuple(t.clone() for t in self.outputs())

    def digest(self, tensors=None):
        self.torch.cuda.synchronize()
        h = hashlib.sha256()
        for t in tensors if tensors is not None else self.outputs():
            h.update(t.view(self.torch.uint8).cpu().numpy().tobytes())
        return h.hexdigest()


def time_steps(torch, run, steps, warmup):
    """`warmup` untimed steps, then `steps` timed ones (HIP events on the calls'
    stream, wall clock between device synchronisations); then one more step
    must reproduce the last timed step's outputs bit for bit. The last timed
    step's outputs are copied on the device and the extra step follows at once,
    so it runs as warm as the timed ones; both are hashed afterwards."""
    for _ in range(warmup):
        run.fwd()
        run.bwd()
    torch.cuda.synchronize()
    log(f"{warmup} warmup steps done")
    stream = run.stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        run.fwd()
        ev[i][1].record(stream)
        run.bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    fwd_ms = [a.elapsed_time(b) for a, b, _ in ev]
    bwd_ms = [b.elapsed_time(c) for _, b, c in ev]
    step_ms = [a.elapsed_time(c) for a, _, c in ev]
    ms_per_step = wall * 1e3 / steps
    log(f"timed {steps} steps: wall {ms_per_step:.3f} ms/step; events fwd {np.mean(fwd_ms):.3f} "
        f"bwd {np.mean(bwd_ms):.3f} step {np.mean(step_ms):.3f} ms")
    snap = run.snapshot()
    run.fwd()
    run.bwd()
    d2 = run.digest()
    d1 = run.digest(snap)
    del snap
    log(f"bitwise repeat: {d1 == d2} ({d1[:16]})")
    return {"wall_s": wall, "ms_per_step": ms_per_step, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
            "step_ms": step_ms, "deterministic": d1 == d2}


def other_workloads(torch, lm, workloads, dev, steps):
    """The other workloads of the path, timed the same way with a few steps
    each (inputs drawn by the same seeded recipe): the per-token log-prob
    entry, the dense support entry (log-probs + KL over K = 64 candidates) and
    the KL-only support entry on the same inputs."""
    E = workloads
    res = {}
    support_inp = None
    for key, name, entry in (("logprob", "logprob", E.ENTRY_LOGPROB),
                             ("support", "support", E.ENTRY_SUPPORT),
                             ("support_kl_only", "support", E.ENTRY_SUPPORT_KL)):
        wl = E.WORKLOADS[name]
        t0 = time.time()
        if name == "support" and support_inp is not None:
            inp = support_inp
        else:
            inp = E.make_inputs(wl)
            log(f"inputs for {name} drawn in {time.time() - t0:.1f}s")
        if name == "support":
            support_inp = inp
        run = Runner(torch, lm, workloads, wl, inp, entry, dev)
        t = time_steps(torch, run, steps, 2)
        ms = t["ms_per_step"]
        rec = {
            "workload": f"{name}: N={wl.n}, Hd={wl.hidden}, V={wl.vocab}, chunk {wl.chunk}"
                        + (f", K={wl.k}" if run.k > 1 else "") + f", entry "
                        + {E.ENTRY_LOGPROB: "logprob", E.ENTRY_SUPPORT: "support (lp + KL)",
                           E.ENTRY_SUPPORT_KL: "support_kl (KL only)"}[entry]
                        + ", forward + backward (dH, dW)",
            "tokens_per_s": round(wl.n * steps / t["wall_s"], 1),
            "ms_per_step": round(ms, 4),
            "fwd_ms": round(float(np.mean(t["fwd_ms"])), 4),
            "bwd_ms": round(float(np.mean(t["bwd_ms"])), 4),
            "steps": steps,
            "deterministic_repeat": t["deterministic"],
        }
        if entry != E.ENTRY_SUPPORT_KL:
            tf = wl.flops_fwd_bwd / (ms * 1e-3) / 1e12
            rec["tflops_8nvh"] = round(tf, 2)
            rec["pct_bf16_peak"] = round(100 * tf / BF16_PEAK_TFLOPS, 2)
        res[key] = rec
        del run
        torch.cuda.empty_cache()
    return res


def vendor_gemm(torch, H, W, wl, stream, reps=5):
    """The vendor library's plain bf16 GEMMs (torch.matmul, i.e. hipBLASLt) at
    the shapes of the path, for comparison only: the full logits H W^T (bf16
    output, no epilogue), and per vocabulary chunk the logits, G^T H and G W_c
    with a random bf16 G. An unfused step built from these GEMMs alone would
    take at least full + chunks x (chunk logits + dW + dH)."""
    n, C = wl.n, min(wl.chunk, wl.vocab)
    g = torch.Generator(device=H.device)
    g.manual_seed(wl.seed + 5)
    G = (torch.randn(n, C, device=H.device, generator=g) * 0.01).to(torch.bfloat16)
    Wc = W[:C]

    def timed(f):
        with torch.cuda.stream(stream):
            for _ in range(2):
                f()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                f()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    full = timed(lambda: torch.matmul(H, W.t()))
    cl = timed(lambda: torch.matmul(H, Wc.t()))
    dw = timed(lambda: torch.matmul(G.t(), H))
    dh = timed(lambda: torch.matmul(G, Wc))
    chunks = -(-wl.vocab // C)
    gf = lambda ms, flop: round(flop / (ms * 1e-3) / 1e12, 1)
    fl_full = 2.0 * n * wl.vocab * wl.hidden
    fl_c = 2.0 * n * C * wl.hidden
    rec = {
        "library": "torch.matmul (hipBLASLt) bf16, plain GEMMs without the path's epilogues",
        "logits_full_ms": round(full, 4), "logits_full_tflops": gf(full, fl_full),
        "chunk_logits_us": round(cl * 1e3, 1), "chunk_logits_tflops": gf(cl, fl_c),
        "dw_chunk_us": round(dw * 1e3, 1), "dw_chunk_tflops": gf(dw, fl_c),
        "dh_chunk_us": round(dh * 1e3, 1), "dh_chunk_tflops": gf(dh, fl_c),
        "unfused_step_lower_bound_ms": round(full + chunks * (cl + dw + dh), 3),
    }
    log(f"vendor GEMMs: full logits {full:.3f} ms; per chunk logits {cl * 1e3:.1f} us, "
        f"dW {dw * 1e3:.1f} us, dH {dh * 1e3:.1f} us")
    return rec


def host_cpus():
    """The host cores this process may run on: its CPU affinity set, bounded by
    a cgroup CPU quota if one is set; and the CPU model."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = int(q) / int(period)
    except (OSError, ValueError):
        pass
    threads = avail if quota is None else max(1, min(avail, int(quota)))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"threads": threads, "available": avail, "quota": quota, "model": model}


def cpu_baseline(wl, inp, target_s, entry=None):
    """The fp64 oracle, as it stands, on a bounded sample of rows of the same
    workload: for each sampled row the full forward (logits over the whole
    vocabulary, lse, loss) and backward (dL/dz, its dH row and its share of
    every dW row). Throughput is scaled to tokens/s."""
    import oracle

    entry = wl.entry if entry is None else entry
    host = host_cpus()
    threads = host["threads"]
    rng = np.random.default_rng(wl.seed + 77)

    def one(rows):
        rows = np.sort(rows)
        t0 = time.perf_counter()
        z = oracle.logits(inp.H, inp.W, rows, threads=threads)
        if entry == oracle.ENTRY_SUPPORT_KL:
            oracle.support_kl_forward(z, inp.ids[rows], inp.ref_logq[rows])
            dz = oracle.support_dz(z, inp.ids[rows], inp.ref_logq[rows], None, inp.grad_kl[rows])
        elif entry in (0, 1):
            t = inp.targets[rows]
            f = oracle.ce_forward(z, t, -1, "mean")
            dz = oracle.ce_dz(z, t, 1.0, max(f["count"], 1), "mean")
        elif entry == 2:
            t = inp.targets[rows]
            oracle.logprob_forward(z, t)
            dz = oracle.logprob_dz(z, t, inp.grad[rows])
        else:
            oracle.support_forward(z, inp.ids[rows], inp.ref_logq[rows])
            dz = oracle.support_dz(z, inp.ids[rows], inp.ref_logq[rows], inp.grad[rows],
                                   inp.grad_kl[rows])
        oracle.grad_hidden(dz, inp.W, threads=threads)
        for v0 in range(0, wl.vocab, 8192):   # dW in vocabulary blocks (bounded memory)
            oracle.grad_weight(dz[:, v0:v0 + 8192], inp.H, rows, threads=threads)
        return time.perf_counter() - t0

    # two probes: the slope between them is the cost of a row without the
    # call's fixed part, so the timed sample lands near target_s
    t4 = one(rng.choice(wl.n, size=4, replace=False))
    t16 = one(rng.choice(wl.n, size=16, replace=False))
    per_row = (t16 - t4) / 12 if t16 > t4 else t16 / 16
    fixed = max(0.0, t16 - 16 * per_row)
    n_rows = int(max(4, min(1024, (target_s - fixed) / max(per_row, 1e-6))))
    n_rows = (n_rows // 4) * 4
    rows = rng.choice(wl.n, size=n_rows, replace=False)
    log(f"cpu baseline: probes {t4:.2f}s for 4 rows, {t16:.2f}s for 16; "
        f"timing {n_rows} rows on {threads} threads")
    dt = one(rows)
    return {
        "value": round(n_rows / dt, 4),
        "unit": "tokens/s",
        "cores": threads,
        "cores_available": host["available"],
        "cgroup_cpu_quota": host["quota"],
        "cpu_model": host["model"],
        "kind": "oracle",
        "sample": f"{n_rows} rows of the {wl.name} workload (fp64 C oracle, entry {entry}: logits "
                  f"over all {wl.vocab} ids, the entry's outputs, dL/dz, the rows' dH and their dW "
                  f"contribution over all vocabulary rows), {dt:.1f}s wall",
        "seconds": round(dt, 2),
    }


if __name__ == "__main__":
    main()
