"""sl_kl_lock_noalloc (the allocation-free variant of sl_kl_lock) against sl_kl_lock itself.

Both run the same kernels on the same inputs, so every output must be identical: statistics,
gate thresholds, lock mask, new active list and count.  Two calls in a row on the library's
scratch array, the second one smaller, show that the array's leftover contents from the first
call do not leak into the second.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import dev, say, tdtype

pytestmark = pytest.mark.gpu


def _inputs(case):
    B, N, V = case.B, case.N, case.V
    dt = tdtype(case.dtype)
    glob = np.concatenate([b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]] for b in range(B)]).astype(np.int64)
    cur = torch.zeros((B * N, V), dtype=dt, device="cuda")
    prev = torch.zeros((B * N, V), dtype=dt, device="cuda")
    gi = torch.from_numpy(glob).cuda()
    cur.index_copy_(0, gi, dev(case.cur, case.dtype))
    prev.index_copy_(0, gi, dev(case.prev, case.dtype))
    return cur, prev


def _call(sl, fn, case, cur, prev, eps, gate_q, ws=None):
    B, N, M = case.B, case.N, case.M_tot
    o = dict(kl=torch.full((max(M, 1),), -1.0, device="cuda"), u=torch.full((max(M, 1),), -1.0, device="cuda"),
             lse=torch.full((max(M, 1),), -1.0, device="cuda"), conf=torch.full((max(M, 1),), -1.0, device="cuda"),
             argmax=torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda"),
             gate_thr=torch.full((B,), -1.0, device="cuda"),
             act_idx=torch.full((B * N,), -7, dtype=torch.int32, device="cuda"),
             act_off=torch.full((B + 1,), -7, dtype=torch.int32, device="cuda"),
             locked=torch.from_numpy(case.locked.copy()).cuda())
    cand = None if case.cand is None else torch.from_numpy(case.cand).cuda()
    m = sl.PinnedInt()
    args = (cur, prev, case.V, torch.from_numpy(case.act_idx).cuda(), torch.from_numpy(case.act_off).cuda(), B, N, M,
            cand, eps, gate_q, -1, True, o["locked"], o["kl"], o["u"], o["lse"], o["argmax"], o["conf"],
            o["gate_thr"], o["act_idx"], o["act_off"])
    if ws is None:
        o["M"] = fn(*args, m_tot_host=m)
    else:
        o["M"] = fn(*args, ws, m_tot_host=m)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in o.items()}


def test_kl_lock_noalloc_matches_kl_lock_on_two_calls():
    import token_locking_sparse_amd as sl
    cases = [  # the KL-lock workload at full vocabulary, then a smaller one on the same scratch array
        (W.kl_lock_case(N=2048, V=126464, B=2, locked_frac=0.6, dtype="bf16", key=2048), 0.01, 0.5),
        (W.kl_lock_case(N=300, V=4096, B=3, locked_frac=0.3, dtype="bf16", cand_frac=0.7, key=300), 0.05, 0.3),
    ]
    for case, eps, gate_q in cases:
        say("noalloc kl_lock", case.B, case.N, case.V, case.M_tot)
        cur, prev = _inputs(case)
        ws = torch.empty(sl.sl_kl_lock_workspace_size(case.B, case.N, case.M_tot, case.V), dtype=torch.uint8,
                         device="cuda")
        ref = _call(sl, sl.sl_kl_lock, case, cur, prev, eps, gate_q, ws)
        got = _call(sl, sl.sl_kl_lock_noalloc, case, cur, prev, eps, gate_q)
        assert got["M"] == ref["M"]
        for k in ("kl", "u", "lse", "conf", "argmax", "gate_thr", "act_off", "locked"):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        np.testing.assert_array_equal(got["act_idx"][:got["M"]], ref["act_idx"][:ref["M"]])
        assert np.all(got["act_idx"][got["M"]:] == -7)
        assert int(got["locked"].sum()) > int(case.locked.sum())      # the call did lock something
