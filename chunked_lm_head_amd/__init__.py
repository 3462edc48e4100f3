"""Python binding of liblmhead.so, the deterministic chunked LM-head + loss
library for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/lmhead.h). PyTorch supplies device memory
and the current stream. There is no CPU fallback: if the library is missing,
every entry raises.

Two layers:

* ``lmhead_workspace_size``, ``lmhead_loss_fwd``, ``lmhead_loss_fwd_noalloc``, ``lmhead_logprob``,
  ``lmhead_support_logprob_kl``, ``lmhead_support_logprob``,
  ``lmhead_support_kl``, ``lmhead_loss_bwd``,
  ``lmhead_loss_bwd_accumulate``, ``lmhead_memory_report``,
  ``lmhead_plan_chunk``, ``lmhead_status_string``,
  ``lmhead_read_device_error``: the C entry points
  under the same names. Pointer arguments accept a torch tensor, an integer
  address or None; the return value is the C status code.
* ``ce_loss``, ``logprob``, ``support_logprob_kl`` (and their autograd
  functions): allocate outputs and workspace with torch, call the entry
  points and raise ``LMHeadError`` on a nonzero status.
"""

from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblmhead.so")

LMHEAD_OK = 0
LMHEAD_ERR_ARG = 1
LMHEAD_ERR_SHAPE = 2
LMHEAD_ERR_ALIGN = 3
LMHEAD_ERR_WORKSPACE = 4
LMHEAD_ERR_DEVICE = 5
LMHEAD_ERR_HIP = 6
LMHEAD_ERR_SCRATCH = 7
STATIC_SCRATCH_BYTES = 64 << 20

ENTRY_CE_MEAN = 0
ENTRY_CE_SUM = 1
ENTRY_LOGPROB = 2
ENTRY_SUPPORT = 3
ENTRY_SUPPORT_KL = 4

FLAG_PADDED_IDS = 1

DEVERR_LABEL = 1
DEVERR_CANDIDATE = 2
DEVERR_TEMPERATURE = 4

IGNORE_INDEX = -100


class lmhead_problem(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("num_valid", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("temperature", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("row_temperature", ctypes.c_void_p),
    ]


def problem(n: int, hidden: int, vocab: int, chunk: int, num_valid: int = -1, k: int = 1,
            flags: int = 0, temperature: float = 0.0, row_temperature=None) -> lmhead_problem:
    """row_temperature: a device fp32 [n] tensor (kept alive by the caller) or an address."""
    return lmhead_problem(n, hidden, vocab, chunk, num_valid, k, flags, float(temperature), 0,
                          _p(row_temperature))


class lmhead_memory_figures(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int64),
        ("chunks", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("forward_bytes", ctypes.c_size_t),
        ("partials_bytes", ctypes.c_size_t),
        ("dz_chunk_bytes", ctypes.c_size_t),
        ("dh_acc_bytes", ctypes.c_size_t),
        ("caller_output_bytes", ctypes.c_size_t),
        ("dh_split_bytes", ctypes.c_size_t),
        ("operand_copy_bytes", ctypes.c_size_t),
        ("dz_group", ctypes.c_int64),
    ]


class LMHeadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lmhead_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblmhead.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m chunked_lm_head_amd.build` "
                "(or __graft_entry__.build()); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(lmhead_problem)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.lmhead_workspace_size.argtypes = [P, i32, i32]
        L.lmhead_workspace_size.restype = sz
        L.lmhead_loss_fwd.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_loss_fwd_noalloc.argtypes = [P, i32, vp, vp, vp, vp, vp, vp]
        L.lmhead_logprob.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_support_logprob_kl.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_support_logprob.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_support_kl.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_loss_bwd.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.lmhead_loss_bwd_accumulate.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 vp, vp, sz, vp]
        L.lmhead_memory_report.argtypes = [P, i32, i32, ctypes.POINTER(lmhead_memory_figures)]
        L.lmhead_plan_chunk.argtypes = [P, i32, sz, ctypes.POINTER(ctypes.c_int64)]
        L.lmhead_status_string.argtypes = [i32]
        L.lmhead_status_string.restype = ctypes.c_char_p
        L.lmhead_read_device_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int64)]
        for f in (L.lmhead_loss_fwd, L.lmhead_loss_fwd_noalloc, L.lmhead_logprob, L.lmhead_support_logprob_kl,
                  L.lmhead_support_logprob, L.lmhead_support_kl,
                  L.lmhead_loss_bwd, L.lmhead_loss_bwd_accumulate, L.lmhead_read_device_error,
                  L.lmhead_memory_report, L.lmhead_plan_chunk):
            f.restype = i32
        _lib = L
    return _lib


def _p(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ----------------------------------------------------------- C entry points

def lmhead_workspace_size(p: lmhead_problem, entry: int, with_backward: int) -> int:
    return int(lib().lmhead_workspace_size(ctypes.byref(p), entry, int(with_backward)))


def lmhead_memory_report(p: lmhead_problem, entry: int, with_backward: int, out) -> int:
    return lib().lmhead_memory_report(ctypes.byref(p), entry, int(with_backward), ctypes.byref(out))


def lmhead_plan_chunk(p: lmhead_problem, entry: int, budget_bytes: int, chunk) -> int:
    return lib().lmhead_plan_chunk(ctypes.byref(p), entry, int(budget_bytes), ctypes.byref(chunk))


def memory_report(n: int, hidden: int, vocab: int, chunk: int, entry: int = ENTRY_CE_MEAN,
                  with_backward: bool = True, k: int = 1) -> dict:
    """Byte counts of one call: workspace and its parts, and the outputs the
    caller allocates (lmhead_memory_report)."""
    r = lmhead_memory_figures()
    _ok(lmhead_memory_report(problem(n, hidden, vocab, chunk, -1, k), entry, with_backward, r),
        "lmhead_memory_report")
    return {name: int(getattr(r, name)) for name, _ in r._fields_}


def plan_chunk(n: int, hidden: int, vocab: int, budget_bytes: int, entry: int = ENTRY_CE_MEAN,
               k: int = 1) -> int:
    """The backward chunk whose workspace fits the byte budget with the fewest
    vocabulary passes (lmhead_plan_chunk)."""
    c = ctypes.c_int64(0)
    _ok(lmhead_plan_chunk(problem(n, hidden, vocab, 256, -1, k), entry, budget_bytes, c),
        "lmhead_plan_chunk")
    return int(c.value)


def lmhead_loss_fwd(p, entry, H, W, targets, loss, lse, workspace, workspace_bytes, stream=None) -> int:
    return lib().lmhead_loss_fwd(ctypes.byref(p), entry, _p(H), _p(W), _p(targets), _p(loss),
                                 _p(lse), _p(workspace), workspace_bytes, _stream(stream))


def lmhead_loss_fwd_noalloc(p, entry, H, W, targets, loss, lse, stream=None) -> int:
    return lib().lmhead_loss_fwd_noalloc(ctypes.byref(p), entry, _p(H), _p(W), _p(targets), _p(loss),
                                         _p(lse), _stream(stream))


def lmhead_logprob(p, H, W, targets, logp, lse, workspace, workspace_bytes, stream=None) -> int:
    return lib().lmhead_logprob(ctypes.byref(p), _p(H), _p(W), _p(targets), _p(logp), _p(lse),
                                _p(workspace), workspace_bytes, _stream(stream))


def lmhead_support_logprob_kl(p, H, W, ids, ref_logq, lp, kl, lse, workspace, workspace_bytes,
                              stream=None) -> int:
    return lib().lmhead_support_logprob_kl(ctypes.byref(p), _p(H), _p(W), _p(ids), _p(ref_logq),
                                           _p(lp), _p(kl), _p(lse), _p(workspace), workspace_bytes,
                                           _stream(stream))


def lmhead_support_logprob(p, H, W, ids, lp, lse, workspace, workspace_bytes, stream=None) -> int:
    return lib().lmhead_support_logprob(ctypes.byref(p), _p(H), _p(W), _p(ids), _p(lp), _p(lse),
                                        _p(workspace), workspace_bytes, _stream(stream))


def lmhead_support_kl(p, H, W, ids, ref_logq, kl, logp_hat, workspace, workspace_bytes,
                      stream=None) -> int:
    return lib().lmhead_support_kl(ctypes.byref(p), _p(H), _p(W), _p(ids), _p(ref_logq), _p(kl),
                                   _p(logp_hat), _p(workspace), workspace_bytes, _stream(stream))


def lmhead_loss_bwd(p, entry, H, W, targets_or_ids, ref_logq, lse, saved_lp, grad, grad_kl, dH, dW,
                    workspace, workspace_bytes, stream=None) -> int:
    return lib().lmhead_loss_bwd(ctypes.byref(p), entry, _p(H), _p(W), _p(targets_or_ids),
                                 _p(ref_logq), _p(lse), _p(saved_lp), _p(grad), _p(grad_kl), _p(dH),
                                 _p(dW), _p(workspace), workspace_bytes, _stream(stream))


def lmhead_loss_bwd_accumulate(p, entry, H, W, targets_or_ids, ref_logq, lse, saved_lp, grad,
                               grad_kl, dH_acc, dW_acc, dH, dW, workspace, workspace_bytes,
                               stream=None) -> int:
    return lib().lmhead_loss_bwd_accumulate(ctypes.byref(p), entry, _p(H), _p(W), _p(targets_or_ids),
                                            _p(ref_logq), _p(lse), _p(saved_lp), _p(grad),
                                            _p(grad_kl), _p(dH_acc), _p(dW_acc), _p(dH), _p(dW),
                                            _p(workspace), workspace_bytes, _stream(stream))


def lmhead_status_string(status: int) -> str:
    return lib().lmhead_status_string(int(status)).decode()


def lmhead_read_device_error(workspace, stream=None):
    code = ctypes.c_int32(0)
    row = ctypes.c_int64(0)
    st = lib().lmhead_read_device_error(_p(workspace), _stream(stream), ctypes.byref(code),
                                        ctypes.byref(row))
    if st != LMHEAD_OK:
        raise LMHeadError(st, "lmhead_read_device_error")
    return int(code.value), int(row.value)


# ------------------------------------------------------------- torch helpers

def _check_inputs(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor, support: bool = False):
    """H bf16 [n, hidden], W bf16 [vocab, hidden], targets int32 [n] (support:
    ids int32 [n, k]), contiguous, all on one GPU."""
    for name, t in (("H", H), ("W", W), ("targets/ids", idx)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a tensor on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if W.device != H.device or idx.device != H.device:
        raise ValueError("H, W and the targets / ids must be on the same device")
    if H.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise ValueError("H and W must be bfloat16")
    if idx.dtype != torch.int32:
        raise ValueError("targets / candidate ids must be int32")
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("expected H [n, hidden] and W [vocab, hidden]")
    if support:
        if idx.dim() != 2 or idx.shape[0] != H.shape[0]:
            raise ValueError("candidate ids must be int32 [n, k] with n = H.shape[0]")
    elif idx.dim() != 1 or idx.shape[0] != H.shape[0]:
        raise ValueError("targets must be int32 [n] with n = H.shape[0]")


def _check_f32(name, t, shape, device, required: bool = False):
    """An fp32 side input (lse, upstream gradients, reference log-probs)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError(f"{name} must be a tensor on the inputs' device")
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")


def _check_side(entry: int, H, idx, lse, grad, ref_logq, saved_lp, grad_kl):
    """Shapes of the backward's fp32 side inputs for one entry."""
    n = H.shape[0]
    dev = H.device
    if entry in (ENTRY_CE_MEAN, ENTRY_CE_SUM, ENTRY_LOGPROB):
        _check_f32("lse", lse, (n,), dev, required=n > 0)
        _check_f32("grad", grad, (1,) if entry != ENTRY_LOGPROB else (n,), dev, required=n > 0)
        return
    k = idx.shape[1]
    if entry == ENTRY_SUPPORT:
        _check_f32("lse", lse, (n,), dev, required=n > 0)
        _check_f32("grad", grad, (n, k), dev)
    _check_f32("ref_logq", ref_logq, (n, k), dev)
    _check_f32("saved_lp", saved_lp, (n, k), dev)
    _check_f32("grad_kl", grad_kl, (n,), dev)


def _check_row_temperature(rt, n: int):
    if rt is None:
        return
    if not isinstance(rt, torch.Tensor) or rt.device.type != "cuda":
        raise ValueError("row_temperature must be a tensor on a GPU device")
    if rt.dtype != torch.float32 or not rt.is_contiguous() or tuple(rt.shape) != (n,):
        raise ValueError("row_temperature must be a contiguous float32 tensor of shape [n]")


def _on_device_of(arg: int):
    """Run a helper with the device of its positional argument `arg` (H)
    current, so that the library's device check, its launches and the
    current-stream lookup all refer to the tensors' GPU."""
    def wrap(fn):
        @functools.wraps(fn)
        def call(*args, **kwargs):
            t = args[arg] if len(args) > arg else None
            if isinstance(t, torch.Tensor) and t.device.type == "cuda":
                with torch.cuda.device(t.device):
                    return fn(*args, **kwargs)
            return fn(*args, **kwargs)
        return call
    return wrap


def workspace(p: lmhead_problem, entry: int, with_backward: bool, device) -> torch.Tensor:
    nbytes = lmhead_workspace_size(p, entry, int(with_backward))
    if nbytes == 0:
        raise LMHeadError(LMHEAD_ERR_SHAPE, "lmhead_workspace_size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _ok(status: int, where: str):
    if status != LMHEAD_OK:
        raise LMHeadError(status, where)


@_on_device_of(0)
def ce_loss_forward(H, W, targets, chunk: int, reduction: str = "mean", num_valid: int = -1,
                    ws: Optional[torch.Tensor] = None, temperature: float = 0.0,
                    row_temperature=None):
    """Returns (loss fp32 [], lse fp32 [n], workspace). temperature 0 = off;
    row_temperature: optional fp32 [n] factors (tau_n = t * r_n)."""
    _check_inputs(H, W, targets)
    _check_row_temperature(row_temperature, H.shape[0])
    entry = ENTRY_CE_MEAN if reduction == "mean" else ENTRY_CE_SUM
    p = problem(H.shape[0], H.shape[1], W.shape[0], chunk, num_valid,
                temperature=temperature, row_temperature=row_temperature)
    if ws is None:
        ws = workspace(p, entry, False, H.device)
    loss = torch.empty(1, dtype=torch.float32, device=H.device)
    lse = torch.empty(H.shape[0], dtype=torch.float32, device=H.device)
    _ok(lmhead_loss_fwd(p, entry, H, W, targets, loss, lse, ws, ws.numel()), "lmhead_loss_fwd")
    return loss[0], lse, ws


@_on_device_of(0)
def logprob_forward(H, W, targets, chunk: int, ws: Optional[torch.Tensor] = None,
                    temperature: float = 0.0, row_temperature=None):
    """Returns (logp fp32 [n], lse fp32 [n], workspace); lse is of the tempered logits."""
    _check_inputs(H, W, targets)
    _check_row_temperature(row_temperature, H.shape[0])
    p = problem(H.shape[0], H.shape[1], W.shape[0], chunk, temperature=temperature,
                row_temperature=row_temperature)
    if ws is None:
        ws = workspace(p, ENTRY_LOGPROB, False, H.device)
    logp = torch.empty(H.shape[0], dtype=torch.float32, device=H.device)
    lse = torch.empty(H.shape[0], dtype=torch.float32, device=H.device)
    _ok(lmhead_logprob(p, H, W, targets, logp, lse, ws, ws.numel()), "lmhead_logprob")
    return logp, lse, ws


@_on_device_of(0)
def support_forward(H, W, ids, ref_logq, chunk: int, ws: Optional[torch.Tensor] = None,
                    temperature: float = 0.0, row_temperature=None, padded: bool = False):
    """Returns (lp fp32 [n, k], kl fp32 [n] or None, lse fp32 [n], workspace).
    padded: a negative id is a padding slot (LMHEAD_FLAG_PADDED_IDS)."""
    _check_inputs(H, W, ids, support=True)
    n, k = ids.shape
    _check_row_temperature(row_temperature, n)
    p = problem(n, H.shape[1], W.shape[0], chunk, -1, k, FLAG_PADDED_IDS if padded else 0,
                temperature=temperature, row_temperature=row_temperature)
    _check_f32("ref_logq", ref_logq, (n, k), H.device)
    if ws is None:
        ws = workspace(p, ENTRY_SUPPORT, False, H.device)
    lp = torch.empty(n, k, dtype=torch.float32, device=H.device)
    kl = torch.empty(n, dtype=torch.float32, device=H.device) if ref_logq is not None else None
    lse = torch.empty(n, dtype=torch.float32, device=H.device)
    _ok(lmhead_support_logprob_kl(p, H, W, ids, ref_logq, lp, kl, lse, ws, ws.numel()),
        "lmhead_support_logprob_kl")
    return lp, kl, lse, ws


@_on_device_of(0)
def support_logprob_forward(H, W, ids, chunk: int, ws: Optional[torch.Tensor] = None,
                            temperature: float = 0.0, row_temperature=None, padded: bool = False):
    """Support-set log-probabilities only. Returns (lp fp32 [n, k], lse fp32 [n], workspace)."""
    _check_inputs(H, W, ids, support=True)
    n, k = ids.shape
    _check_row_temperature(row_temperature, n)
    p = problem(n, H.shape[1], W.shape[0], chunk, -1, k, FLAG_PADDED_IDS if padded else 0,
                temperature=temperature, row_temperature=row_temperature)
    if ws is None:
        ws = workspace(p, ENTRY_SUPPORT, False, H.device)
    lp = torch.empty(n, k, dtype=torch.float32, device=H.device)
    lse = torch.empty(n, dtype=torch.float32, device=H.device)
    _ok(lmhead_support_logprob(p, H, W, ids, lp, lse, ws, ws.numel()), "lmhead_support_logprob")
    return lp, lse, ws


@_on_device_of(0)
def support_kl_forward(H, W, ids, ref_logq, ws: Optional[torch.Tensor] = None,
                       temperature: float = 0.0, row_temperature=None, padded: bool = False):
    """KL-only support entry (no vocabulary-wide pass). Returns (kl fp32 [n],
    log p_hat fp32 [n, k], workspace)."""
    _check_inputs(H, W, ids, support=True)
    n, k = ids.shape
    _check_row_temperature(row_temperature, n)
    p = problem(n, H.shape[1], W.shape[0], 256, -1, k, FLAG_PADDED_IDS if padded else 0,
                temperature=temperature, row_temperature=row_temperature)
    _check_f32("ref_logq", ref_logq, (n, k), H.device, required=n > 0)
    if ws is None:
        ws = workspace(p, ENTRY_SUPPORT_KL, False, H.device)
    kl = torch.empty(n, dtype=torch.float32, device=H.device)
    logp_hat = torch.empty(n, k, dtype=torch.float32, device=H.device)
    _ok(lmhead_support_kl(p, H, W, ids, ref_logq, kl, logp_hat, ws, ws.numel()), "lmhead_support_kl")
    return kl, logp_hat, ws


@_on_device_of(1)
def backward(entry: int, H, W, idx, lse, grad, chunk: int, *, ref_logq=None, saved_lp=None,
             grad_kl=None, num_valid: int = -1, need_dH: bool = True, need_dW: bool = True,
             ws: Optional[torch.Tensor] = None, dH=None, dW=None, temperature: float = 0.0,
             row_temperature=None, padded: bool = False):
    """Returns (dH bf16 [n, hidden] or None, dW bf16 [vocab, hidden] or None).
    temperature / row_temperature must be those of the forward that produced lse.
    ENTRY_SUPPORT_KL: saved_lp is the forward's log p_hat; lse and grad are unused."""
    support = entry in (ENTRY_SUPPORT, ENTRY_SUPPORT_KL)
    _check_inputs(H, W, idx, support=support)
    _check_row_temperature(row_temperature, H.shape[0])
    _check_side(entry, H, idx, lse, grad, ref_logq, saved_lp, grad_kl)
    k = idx.shape[1] if support else 1
    p = problem(H.shape[0], H.shape[1], W.shape[0], chunk, num_valid, k,
                FLAG_PADDED_IDS if padded else 0, temperature=temperature,
                row_temperature=row_temperature)
    if ws is None:
        ws = workspace(p, entry, True, H.device)
    if need_dH and dH is None:
        dH = torch.empty_like(H)
    if need_dW and dW is None:
        dW = torch.empty_like(W)
    _ok(lmhead_loss_bwd(p, entry, H, W, idx, ref_logq, lse, saved_lp, grad, grad_kl,
                        dH if need_dH else None, dW if need_dW else None, ws, ws.numel()),
        "lmhead_loss_bwd")
    return (dH if need_dH else None), (dW if need_dW else None)


def _check_acc(name, t, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device != device:
        raise ValueError(f"{name} must be a tensor on the inputs' device")
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")


@_on_device_of(1)
def backward_accumulate(entry: int, H, W, idx, lse, grad, chunk: int, *, dH_acc=None, dW_acc=None,
                        ref_logq=None, saved_lp=None, grad_kl=None, num_valid: int = -1,
                        out_bf16: bool = False, ws: Optional[torch.Tensor] = None,
                        temperature: float = 0.0, row_temperature=None, padded: bool = False):
    """dH_acc += dL/dH and dW_acc += dL/dW in fp32 (either may be None).
    Returns (dH, dW): the bf16 casts of the updated accumulators when out_bf16,
    else (None, None)."""
    support = entry in (ENTRY_SUPPORT, ENTRY_SUPPORT_KL)
    _check_inputs(H, W, idx, support=support)
    _check_row_temperature(row_temperature, H.shape[0])
    _check_side(entry, H, idx, lse, grad, ref_logq, saved_lp, grad_kl)
    _check_acc("dH_acc", dH_acc, H.shape, H.device)
    _check_acc("dW_acc", dW_acc, W.shape, H.device)
    k = idx.shape[1] if support else 1
    p = problem(H.shape[0], H.shape[1], W.shape[0], chunk, num_valid, k,
                FLAG_PADDED_IDS if padded else 0, temperature=temperature,
                row_temperature=row_temperature)
    if ws is None:
        ws = workspace(p, entry, True, H.device)
    dH = torch.empty_like(H) if (out_bf16 and dH_acc is not None) else None
    dW = torch.empty_like(W) if (out_bf16 and dW_acc is not None) else None
    _ok(lmhead_loss_bwd_accumulate(p, entry, H, W, idx, ref_logq, lse, saved_lp, grad, grad_kl,
                                   dH_acc, dW_acc, dH, dW, ws, ws.numel()),
        "lmhead_loss_bwd_accumulate")
    return dH, dW


# --------------------------------------------------------------- autograd

class ChunkedLMHeadCE(torch.autograd.Function):
    """Cross-entropy of softmax(H W^T) against targets, mean or sum over valid rows."""

    @staticmethod
    def forward(ctx, H, W, targets, chunk, reduction="mean", num_valid=-1, temperature=0.0,
                row_temperature=None):
        loss, lse, _ = ce_loss_forward(H, W, targets, chunk, reduction, num_valid,
                                       temperature=temperature, row_temperature=row_temperature)
        ctx.save_for_backward(H, W, targets, lse, row_temperature)
        ctx.cfg = (chunk, reduction, num_valid, temperature)
        return loss

    @staticmethod
    def backward(ctx, g):
        H, W, targets, lse, rt = ctx.saved_tensors
        chunk, reduction, num_valid, temperature = ctx.cfg
        entry = ENTRY_CE_MEAN if reduction == "mean" else ENTRY_CE_SUM
        grad = g.reshape(1).to(torch.float32).contiguous()
        dH, dW = backward(entry, H, W, targets, lse, grad, chunk, num_valid=num_valid,
                          need_dH=ctx.needs_input_grad[0], need_dW=ctx.needs_input_grad[1],
                          temperature=temperature, row_temperature=rt)
        return dH, dW, None, None, None, None, None, None


class ChunkedLMHeadLogprob(torch.autograd.Function):
    """Per-token log-probability of the target under softmax(H W^T)."""

    @staticmethod
    def forward(ctx, H, W, targets, chunk, temperature=0.0, row_temperature=None):
        logp, lse, _ = logprob_forward(H, W, targets, chunk, temperature=temperature,
                                       row_temperature=row_temperature)
        ctx.save_for_backward(H, W, targets, lse, row_temperature)
        ctx.cfg = (chunk, temperature)
        return logp

    @staticmethod
    def backward(ctx, g):
        H, W, targets, lse, rt = ctx.saved_tensors
        chunk, temperature = ctx.cfg
        dH, dW = backward(ENTRY_LOGPROB, H, W, targets, lse, g.to(torch.float32).contiguous(),
                          chunk, need_dH=ctx.needs_input_grad[0],
                          need_dW=ctx.needs_input_grad[1], temperature=temperature,
                          row_temperature=rt)
        return dH, dW, None, None, None, None


class ChunkedLMHeadSupport(torch.autograd.Function):
    """Full-vocabulary log-probabilities of K candidates per row and KL(q || p_hat)."""

    @staticmethod
    def forward(ctx, H, W, ids, ref_logq, chunk, temperature=0.0, row_temperature=None,
                padded=False):
        lp, kl, lse, _ = support_forward(H, W, ids, ref_logq, chunk, temperature=temperature,
                                         row_temperature=row_temperature, padded=padded)
        ctx.save_for_backward(H, W, ids, ref_logq, lse, lp, row_temperature)
        ctx.cfg = (chunk, temperature, padded)
        ctx.has_kl = kl is not None
        if kl is None:
            kl = torch.zeros(H.shape[0], dtype=torch.float32, device=H.device)
        return lp, kl

    @staticmethod
    def backward(ctx, g_lp, g_kl):
        H, W, ids, ref_logq, lse, lp, rt = ctx.saved_tensors
        chunk, temperature, padded = ctx.cfg
        gl = g_lp.to(torch.float32).contiguous() if g_lp is not None else None
        gk = g_kl.to(torch.float32).contiguous() if (g_kl is not None and ctx.has_kl) else None
        dH, dW = backward(ENTRY_SUPPORT, H, W, ids, lse, gl, chunk,
                          ref_logq=ref_logq if ctx.has_kl else None,
                          saved_lp=lp if ctx.has_kl else None, grad_kl=gk,
                          need_dH=ctx.needs_input_grad[0], need_dW=ctx.needs_input_grad[1],
                          temperature=temperature, row_temperature=rt, padded=padded)
        return dH, dW, None, None, None, None, None, None


class ChunkedLMHeadSupportKL(torch.autograd.Function):
    """KL(q || p_hat) over each row's candidates, without a vocabulary-wide pass."""

    @staticmethod
    def forward(ctx, H, W, ids, ref_logq, temperature=0.0, row_temperature=None, padded=False):
        kl, logp_hat, _ = support_kl_forward(H, W, ids, ref_logq, temperature=temperature,
                                             row_temperature=row_temperature, padded=padded)
        ctx.save_for_backward(H, W, ids, ref_logq, logp_hat, row_temperature)
        ctx.cfg = (temperature, padded)
        return kl

    @staticmethod
    def backward(ctx, g_kl):
        H, W, ids, ref_logq, logp_hat, rt = ctx.saved_tensors
        temperature, padded = ctx.cfg
        dH, dW = backward(ENTRY_SUPPORT_KL, H, W, ids, None, None, 256, ref_logq=ref_logq,
                          saved_lp=logp_hat, grad_kl=g_kl.to(torch.float32).contiguous(),
                          need_dH=ctx.needs_input_grad[0], need_dW=ctx.needs_input_grad[1],
                          temperature=temperature, row_temperature=rt, padded=padded)
        return dH, dW, None, None, None, None, None


def _chunk(chunk, memory_budget, H, W, entry, k=1):
    """The given chunk, or the planned one when a workspace byte budget is given."""
    if memory_budget is None:
        return chunk
    return plan_chunk(H.shape[0], H.shape[1], W.shape[0], memory_budget, entry, k)


def ce_loss(H, W, targets, chunk: int = 8192, reduction: str = "mean", num_valid: int = -1,
            temperature: float = 0.0, row_temperature=None, memory_budget: Optional[int] = None):
    chunk = _chunk(chunk, memory_budget, H, W, ENTRY_CE_MEAN)
    return ChunkedLMHeadCE.apply(H, W, targets, chunk, reduction, num_valid, temperature,
                                 row_temperature)


def logprob(H, W, targets, chunk: int = 8192, temperature: float = 0.0, row_temperature=None,
            memory_budget: Optional[int] = None):
    chunk = _chunk(chunk, memory_budget, H, W, ENTRY_LOGPROB)
    return ChunkedLMHeadLogprob.apply(H, W, targets, chunk, temperature, row_temperature)


def support_logprob_kl(H, W, ids, ref_logq, chunk: int = 8192, temperature: float = 0.0,
                       row_temperature=None, memory_budget: Optional[int] = None,
                       padded: bool = False):
    chunk = _chunk(chunk, memory_budget, H, W, ENTRY_SUPPORT, ids.shape[1])
    return ChunkedLMHeadSupport.apply(H, W, ids, ref_logq, chunk, temperature, row_temperature,
                                      padded)


def support_logprob(H, W, ids, chunk: int = 8192, temperature: float = 0.0, row_temperature=None,
                    memory_budget: Optional[int] = None, padded: bool = False):
    """Full-vocabulary log-probabilities of the candidates (no KL)."""
    lp, _ = support_logprob_kl(H, W, ids, None, chunk, temperature, row_temperature,
                               memory_budget, padded)
    return lp


def support_kl(H, W, ids, ref_logq, temperature: float = 0.0, row_temperature=None,
               padded: bool = False):
    """KL(q || p_hat) per row over the candidates (KL-only entry)."""
    return ChunkedLMHeadSupportKL.apply(H, W, ids, ref_logq, temperature, row_temperature, padded)
