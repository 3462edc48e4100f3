"""Host-side argument checks of the Python binding's torch helpers: the fp32
side inputs of the backward (lse, upstream gradients, reference log-probs,
saved log-probs) are checked for dtype, shape, contiguity and device before
anything reaches the library. CPU tensors stand in for device tensors here:
the checks only compare devices."""
import pytest
import torch

import chunked_lm_head_amd as lm


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_f32_side_input_checks():
    dev = torch.device("cpu")
    lm._check_f32("x", f32(4), (4,), dev)
    lm._check_f32("x", None, (4,), dev)
    with pytest.raises(ValueError, match="required"):
        lm._check_f32("x", None, (4,), dev, required=True)
    with pytest.raises(ValueError, match="float32"):
        lm._check_f32("x", torch.zeros(4, dtype=torch.float64), (4,), dev)
    with pytest.raises(ValueError, match="shape"):
        lm._check_f32("x", f32(5), (4,), dev)
    with pytest.raises(ValueError, match="float32"):
        lm._check_f32("x", f32(4, 2).t(), (2, 4), dev)       # not contiguous
    with pytest.raises(ValueError, match="device"):
        lm._check_f32("x", f32(4), (4,), torch.device("meta"))


def test_backward_side_inputs_per_entry():
    n, k = 6, 3
    H = torch.zeros(n, 8, dtype=torch.bfloat16)
    t = torch.zeros(n, dtype=torch.int32)
    ids = torch.zeros(n, k, dtype=torch.int32)
    # CE: lse [n], grad [1]
    lm._check_side(lm.ENTRY_CE_MEAN, H, t, f32(n), f32(1), None, None, None)
    with pytest.raises(ValueError):
        lm._check_side(lm.ENTRY_CE_MEAN, H, t, f32(n), f32(n), None, None, None)
    with pytest.raises(ValueError, match="lse"):
        lm._check_side(lm.ENTRY_CE_SUM, H, t, None, f32(1), None, None, None)
    # log-prob: grad [n]
    lm._check_side(lm.ENTRY_LOGPROB, H, t, f32(n), f32(n), None, None, None)
    with pytest.raises(ValueError):
        lm._check_side(lm.ENTRY_LOGPROB, H, t, f32(n), f32(1), None, None, None)
    # support: grad [n, k] or None, ref_logq / saved_lp [n, k], grad_kl [n]
    lm._check_side(lm.ENTRY_SUPPORT, H, ids, f32(n), f32(n, k), f32(n, k), f32(n, k), f32(n))
    lm._check_side(lm.ENTRY_SUPPORT, H, ids, f32(n), None, None, None, None)
    with pytest.raises(ValueError, match="ref_logq"):
        lm._check_side(lm.ENTRY_SUPPORT, H, ids, f32(n), None, f32(n, k + 1), f32(n, k), f32(n))
    with pytest.raises(ValueError, match="grad_kl"):
        lm._check_side(lm.ENTRY_SUPPORT, H, ids, f32(n), None, f32(n, k), f32(n, k), f32(n, 1))
    # KL-only: no lse, no lp gradient
    lm._check_side(lm.ENTRY_SUPPORT_KL, H, ids, None, None, f32(n, k), f32(n, k), f32(n))
    # an empty batch needs no lse or gradient
    H0 = torch.zeros(0, 8, dtype=torch.bfloat16)
    lm._check_side(lm.ENTRY_CE_MEAN, H0, torch.zeros(0, dtype=torch.int32), None, None, None, None,
                   None)


def test_inputs_must_be_gpu_tensors():
    H = torch.zeros(4, 64, dtype=torch.bfloat16)
    W = torch.zeros(10, 64, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        lm._check_inputs(H, W, t)
