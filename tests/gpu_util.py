"""Helpers for the GPU parity tests: host <-> device conversion and tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.surelock_oracle as O


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


# Lock decisions may differ from the oracle's only where the oracle's KL lies within KL_BAND of eps
# (the band the lock criterion allows), or, with the gate on, where the oracle's u lies within
# GATE_BAND of the oracle's gate threshold.  GATE_BAND is twice the asserted bound on the fp32 u
# against the float64 u of the same logits (2e-6): inside it two rows can be ordered differently.
KL_BAND = 1e-3
U_TOL = 2e-6
GATE_BAND = 2 * U_TOL


def bf16_out_err(got, ref, acc: float = 2e-3):
    """Largest excess of |got - ref| over the bound for a bf16-stored result of an fp32 computation:
    2e-2 absolute, or, where larger, half a bf16 ulp (at most 2^-8 |ref|) plus `acc` of fp32
    accumulation."""
    return float(np.max(np.abs(got - ref) - np.maximum(2e-2, 2.0 ** -8 * np.abs(ref) + acc)))


def compare_lock(g, st, lr, locked0, act_idx, act_off, B, N, eps, gate_q, have_prev, stats_exact=True):
    """GPU statistics, lock mask and new active list against the oracle's on identical logits.

    g: dict of the GPU's kl, u, lse (and optionally conf, argmax, gate_thr) per active row, and its
    locked mask, act_idx, act_off and M after the update.  st, lr: O.posterior_stats and
    O.lock_update on the same inputs.  Returns the number of (exempt) differing lock decisions."""
    M = len(act_idx)
    if M and stats_exact:
        if have_prev:
            assert np.max(np.abs(g["kl"][:M] - st.kl)) <= 2e-5   # fp32 accumulation; the lock band is 1e-3
        else:
            assert np.all(np.isinf(g["kl"][:M]))
        np.testing.assert_allclose(g["lse"][:M], st.lse, rtol=2e-6, atol=2e-5)
        np.testing.assert_allclose(g["u"][:M], st.u, rtol=0, atol=U_TOL)
        if g.get("conf") is not None:
            np.testing.assert_allclose(g["conf"][:M], st.conf, rtol=1e-5, atol=1e-7)
        if g.get("argmax") is not None:
            np.testing.assert_array_equal(g["argmax"][:M], st.argmax)   # comparisons of identical inputs
    if gate_q >= 0 and g.get("gate_thr") is not None:
        np.testing.assert_allclose(g["gate_thr"], lr.gate_thr, rtol=0, atol=U_TOL)
    rows_seq = O.seq_of_rows(act_off)
    glob = rows_seq * N + np.asarray(act_idx, np.int64)
    row_of = {int(gp): i for i, gp in enumerate(glob)}
    diff = np.flatnonzero(g["locked"] != lr.locked)
    for gp in diff:
        i = row_of.get(int(gp))
        assert i is not None, "a position outside A_t changed its lock state"
        near_kl = abs(st.kl[i] - eps) <= KL_BAND
        near_gate = gate_q >= 0 and abs(st.u[i] - lr.gate_thr[rows_seq[i]]) <= GATE_BAND
        assert near_kl or near_gate, "lock mismatch at %d (kl %.6g u %.9g thr %.9g)" % (
            gp, st.kl[i], st.u[i], lr.gate_thr[rows_seq[i]])
    assert np.all(g["locked"] >= locked0)                               # monotone
    ri, ro = O.active_set(g["locked"], B, N)                            # compaction of the GPU's mask
    assert g["M"] == int(ro[-1])
    np.testing.assert_array_equal(g["act_off"], ro)
    np.testing.assert_array_equal(g["act_idx"][:g["M"]], ri)
    if len(diff) == 0:                                                  # and the oracle's list
        np.testing.assert_array_equal(g["act_off"], lr.act_off)
        np.testing.assert_array_equal(g["act_idx"][:g["M"]], lr.act_idx)
    return len(diff)
