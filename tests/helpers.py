"""Shared test helpers: device copies of the seeded inputs and the error
metrics used by the parity tests."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case on stdout before a GPU step, flushed."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(a, device="cuda"):
    """numpy uint16 (BF16 bits) -> torch.bfloat16, float32/uint8 -> same dtype."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def to_f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return num / den if den > 0 else num


def bf16_round_f64(a):
    """Round FP64 values to BF16 (via torch, nearest-even) and back to FP64."""
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.bfloat16).double().numpy()


def bf16_floor(ref):
    """rel-L2 that BF16 rounding of the exact result alone costs."""
    return rel_l2(bf16_round_f64(ref), ref)
