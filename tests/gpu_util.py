"""Helpers for the GPU parity tests: host <-> device conversion and tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    """Progress line that names the case before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array (uint16 bf16 bits or float32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def tdtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def round_storage(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """Oracle float64 values rounded to the storage type, on the device (oracle -> GPU input)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64))
    return t.to(tdtype(dtype)).cuda()


def check_rel(got: np.ndarray, ref: np.ndarray, rel_l2: float, rel_max: float, what: str):
    """||got-ref||/||ref|| <= rel_l2 and max|got-ref| <= rel_max * max(1, |ref|)."""
    d = got - ref
    nr = np.linalg.norm(ref)
    l2 = np.linalg.norm(d) / (nr if nr > 0 else 1.0)
    lim = rel_max * np.maximum(1.0, np.abs(ref))
    bad = np.abs(d) > lim
    assert l2 <= rel_l2, "%s: relative L2 error %.3e > %.1e" % (what, l2, rel_l2)
    assert not bad.any(), "%s: %d elements beyond %.1e*max(1,|ref|); worst |d| %.3e at ref %.3e" % (
        what, int(bad.sum()), rel_max, float(np.abs(d)[bad].max()), float(ref[bad][np.argmax(np.abs(d)[bad])]))


def check_hidden(got: np.ndarray, ref: np.ndarray, rel_l2: float, what: str, k_out: float = 7.0, rel_max: float = 2e-2):
    """Tolerance for rows that went through bf16 intermediates (activations, q/k/v, P, o, FFN activation).

    The error is the sum of many independent rounding errors, so it is close to
    Gaussian: require relative L2 <= rel_l2, and per element
    |d| <= max(k_out * rms(d), rel_max * max(1, |ref|)), i.e. no outliers beyond
    7 standard deviations (a Gaussian over 4M elements peaks near 5.3)."""
    d = got - ref
    nr = np.linalg.norm(ref)
    l2 = np.linalg.norm(d) / (nr if nr > 0 else 1.0)
    rms = float(np.sqrt(np.mean(d * d))) if d.size else 0.0
    lim = np.maximum(k_out * rms, rel_max * np.maximum(1.0, np.abs(ref)))
    bad = np.abs(d) > lim
    assert l2 <= rel_l2, "%s: relative L2 error %.3e > %.1e" % (what, l2, rel_l2)
    assert not bad.any(), "%s: %d outliers; worst |d| %.3e with rms %.3e" % (what, int(bad.sum()), float(np.abs(d).max()), rms)
    return l2, rms, float(np.abs(d).max()) if d.size else 0.0
