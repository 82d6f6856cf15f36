"""GPU parity of the kernel-level entry points against the CPU oracle.

sl_compact and the lock/compaction decisions of sl_kl_lock are integer work:
bit-exact, except (for sl_kl_lock) positions whose oracle KL lies within 1e-3
of eps (the tolerance band the lock rule allows) or whose oracle u lies within
GATE_BAND = 4e-6 of the oracle gate threshold (twice the asserted 2e-6 bound on
the fp32 u: an fp32 u and the fp64 u can order values that close differently).
Floating-point outputs: KL within 2e-5 (the lock rule's band is 1e-3); LSE, u,
conf within the fp32 accumulation error of a V-term sum; bf16 GEMM outputs within
half a bf16 ulp plus fp32 accumulation; bf16 attention outputs within the margin
over the bf16-storage emulation (tests/bf16_emulation.py) of the same inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle.surelock_oracle as O
import workloads as W
from tests import bf16_emulation as E
from tests.gpu_util import bf16_out_err, compare_lock, dev, host64, say, tdtype

pytestmark = pytest.mark.gpu


def _sl():
    import token_locking_sparse_amd as sl
    return sl


# ------------------------------------------------------------------ compaction
@pytest.mark.parametrize("B,N,p", [(1, 1, 0.5), (1, 4096, 0.6), (3, 1000, 0.3), (8, 2048, 0.5),
                                   (2, 64, 0.0), (2, 64, 1.0), (5, 3001, 0.97), (1, 65536, 0.5),
                                   (2, 3000, 0.5), (7, 9999, 0.4)])
def test_compact_bit_exact(B, N, p):
    sl = _sl()
    say("compact", B, N, p)
    locked = W.random_mask(B * N, p, seed=11, key=B * N + int(p * 100))
    ai = torch.full((B * N,), -7, dtype=torch.int32, device="cuda")
    ao = torch.full((B + 1,), -7, dtype=torch.int32, device="cuda")
    m = sl.PinnedInt()
    M = sl.sl_compact(torch.from_numpy(locked).cuda(), B, N, ai, ao, m)
    ref_idx, ref_off = O.active_set(locked, B, N)
    assert M == int(ref_off[-1])
    np.testing.assert_array_equal(ao.cpu().numpy(), ref_off)
    np.testing.assert_array_equal(ai[:M].cpu().numpy(), ref_idx)
    assert np.all(ai[M:].cpu().numpy() == -7)          # nothing written past M_tot


def test_compact_rejects_bad_args():
    sl = _sl()
    t = torch.zeros(8, dtype=torch.uint8, device="cuda")
    ai = torch.empty(8, dtype=torch.int32, device="cuda")
    ao = torch.empty(3, dtype=torch.int32, device="cuda")
    with pytest.raises(sl.SureLockError):
        sl.sl_compact(t, 0, 4, ai, ao)
    with pytest.raises(sl.SureLockError):
        sl.sl_compact(t, 2, -1, ai, ao)


# ------------------------------------------------------------------ KL-lock pass
def _run_kl(case, eps, gate_q, mask_id, have_prev, unlock_rows_nan=True, cached_lse=False):
    """cached_lse: the previous posterior's LSE comes from the per-position store that a pass over
    the previous logits (as that step's current ones) wrote, as in the sampler loop; the store this
    pass writes is checked against its per-row lse output."""
    sl = _sl()
    B, N, V, M = case.B, case.N, case.V, case.M_tot
    dt = tdtype(case.dtype)
    glob = np.concatenate([b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]] for b in range(B)]).astype(np.int64)
    fill = float("nan") if unlock_rows_nan else 0.0
    cur = torch.full((B * N, V), fill, dtype=dt, device="cuda")
    prev = torch.full((B * N, V), fill, dtype=dt, device="cuda")
    gi = torch.from_numpy(glob).cuda()
    cur.index_copy_(0, gi, dev(case.cur, case.dtype))
    prev.index_copy_(0, gi, dev(case.prev, case.dtype))
    locked = torch.from_numpy(case.locked.copy()).cuda()
    ai = torch.from_numpy(case.act_idx).cuda()
    ao = torch.from_numpy(case.act_off).cuda()
    out = dict(kl=torch.empty(max(M, 1), device="cuda"), u=torch.empty(max(M, 1), device="cuda"),
               lse=torch.empty(max(M, 1), device="cuda"), conf=torch.empty(max(M, 1), device="cuda"),
               argmax=torch.empty(max(M, 1), dtype=torch.int32, device="cuda"),
               gate_thr=torch.empty(B, device="cuda"))
    nai = torch.full((B * N,), -7, dtype=torch.int32, device="cuda")
    nao = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    ws = torch.full((sl.sl_kl_lock_workspace_size(B, N, M, V),), 0xA5, dtype=torch.uint8, device="cuda")
    cand = None if case.cand is None else torch.from_numpy(case.cand).cuda()
    m = sl.PinnedInt()
    lse_prev = lse_pos = None
    if cached_lse:
        # the previous step's pass: prev as its current logits (nothing locks, only the store matters)
        lse_prev = torch.full((B * N,), float("nan"), device="cuda")
        lse_pos = torch.full((B * N,), float("nan"), device="cuda")
        scratch = {k: torch.empty_like(v) for k, v in out.items()}
        sl.sl_kl_lock(prev, None, V, ai, ao, B, N, M, None, 0.0, -1.0, mask_id, False, locked.clone(),
                      scratch["kl"], scratch["u"], scratch["lse"], scratch["argmax"], scratch["conf"],
                      scratch["gate_thr"], torch.empty_like(nai), torch.empty_like(nao), ws, lse_pos=lse_prev)
    Mn = sl.sl_kl_lock(cur, prev, V, ai, ao, B, N, M, cand, eps, gate_q, mask_id, have_prev, locked,
                       out["kl"], out["u"], out["lse"], out["argmax"], out["conf"], out["gate_thr"], nai, nao,
                       ws, m, lse_prev=lse_prev, lse_pos=lse_pos)
    res = {k: v.cpu().numpy() for k, v in out.items()}
    if cached_lse:
        lp, lc = lse_prev.cpu().numpy(), lse_pos.cpu().numpy()
        inactive = np.ones(B * N, bool)
        inactive[glob] = False
        # this pass's store holds exactly its per-row LSE at the active positions, nothing elsewhere
        np.testing.assert_array_equal(lc[glob], res["lse"][:M])
        assert np.all(np.isnan(lc[inactive])) and np.all(np.isnan(lp[inactive]))
        res["lse_prev_store"] = lp[glob]
    res["locked"] = locked.cpu().numpy()
    res["act_idx"] = nai.cpu().numpy()
    res["act_off"] = nao.cpu().numpy()
    res["M"] = Mn
    return res


def _oracle_kl(case, eps, gate_q, mask_id, have_prev):
    z = O.widen(case.cur, case.dtype)
    y = O.widen(case.prev, case.dtype) if have_prev else None
    st = O.posterior_stats(z, y, mask_id)
    lr = O.lock_update(case.locked, case.act_idx, case.act_off, case.B, case.N, st.kl, st.u, case.cand,
                       eps, gate_q, have_prev)
    return st, lr


def _compare_kl(case, g, st, lr, eps, gate_q, have_prev):
    return compare_lock(g, st, lr, case.locked, case.act_idx, case.act_off, case.B, case.N, eps, gate_q,
                        have_prev)


KL_CASES = [
    # N, V, B, locked_frac, dtype, eps, gate_q, mask_id, have_prev, cand_frac
    (64, 5000, 1, 0.6, "bf16", 0.01, 0.5, -1, True, None),
    (300, 4096, 2, 0.3, "bf16", 0.002, -1.0, -1, True, 0.7),
    (257, 12288, 3, 0.5, "bf16", 0.05, 0.3, 12287, True, 0.8),
    (128, 2048, 2, 0.0, "f32", 0.01, 0.9, 2047, True, None),
    (64, 512, 1, 0.25, "f32", 0.05, -1.0, 511, False, 0.5),
    (64, 1000, 2, 1.0, "bf16", 0.05, 0.5, -1, True, None),            # every row locked: M = 0
    (100, 126464, 1, 0.9, "bf16", 0.01, 0.5, 126463, True, None),     # full vocabulary, ragged chunks
    (4096, 256, 1, 0.2, "bf16", 0.0, 0.5, -1, True, None),            # eps = 0: nothing locks
    (5000, 256, 1, 0.1, "f32", 0.05, 0.5, 255, True, None),           # tail in LDS, 4500 rows: select over LDS
    (10000, 256, 2, 0.7, "bf16", 0.05, 0.5, -1, True, 0.8),           # B*N above the tail's LDS copies
    (20000, 256, 1, 0.3, "bf16", 0.05, 0.5, -1, True, None),          # 14000 rows: tail reads global memory
    (512, 4096, 2, 0.4, "bf16", math.inf, 0.5, -1, True, 0.8),        # eps = +inf: confidence gate only
    (256, 1024, 12, 0.5, "bf16", 0.05, 0.5, -1, True, 0.8),           # 12 sequences: two rounds of grouped selects
    (3276, 512, 5, (0.02, 0.9, 0.9, 0.9, 0.9), "bf16", 0.05, 0.5, 511, True, None),   # one sequence beyond
                                                                      # its group's registers: one at a time
]


@pytest.mark.parametrize("N,V,B,lf,dtype,eps,gq,mask,hp,cf", KL_CASES)
def test_kl_lock_parity(N, V, B, lf, dtype, eps, gq, mask, hp, cf):
    say("kl_lock", N, V, B, lf, dtype, eps, gq, mask, hp, cf)
    case = W.kl_lock_case(N=N, V=V, B=B, locked_frac=lf, dtype=dtype, cand_frac=cf, key=N + V)
    g = _run_kl(case, eps, gq, mask, hp)
    st, lr = _oracle_kl(case, eps, gq, mask, hp)
    _compare_kl(case, g, st, lr, eps, gq, hp)
    if eps <= 0 or not hp:
        np.testing.assert_array_equal(g["locked"], case.locked)


@pytest.mark.parametrize("N,V,B,lf,dtype,eps,gq,mask,hp,cf", [c for c in KL_CASES if c[8]])
def test_kl_lock_parity_cached_prev_lse(N, V, B, lf, dtype, eps, gq, mask, hp, cf):
    """The same cases with the previous posterior's LSE taken from the per-position store of the
    pass that produced it (the previous logits are then read only for sum p (a - b))."""
    say("kl_lock cached lse", N, V, B, lf, dtype, eps, gq, mask, hp, cf)
    case = W.kl_lock_case(N=N, V=V, B=B, locked_frac=lf, dtype=dtype, cand_frac=cf, key=N + V)
    g = _run_kl(case, eps, gq, mask, hp, cached_lse=True)
    st, lr = _oracle_kl(case, eps, gq, mask, hp)
    _compare_kl(case, g, st, lr, eps, gq, hp)
    if case.M_tot > 0:
        # the stored previous LSE is the oracle's LSE of the previous logits
        ref = O.posterior_stats(O.widen(case.prev, case.dtype), None, mask).lse
        np.testing.assert_allclose(g["lse_prev_store"], ref, rtol=2e-6, atol=2e-5)


def test_kl_lock_repeat_reuses_workspace():
    """Two calls in a row on one (garbage-filled) workspace give the same, correct result."""
    say("kl_lock repeat")
    case = W.kl_lock_case(N=200, V=4096, B=2, locked_frac=0.5, dtype="bf16", key=77)
    for _ in range(2):
        g = _run_kl(case, 0.01, 0.5, -1, True)
        st, lr = _oracle_kl(case, 0.01, 0.5, -1, True)
        _compare_kl(case, g, st, lr, 0.01, 0.5, True)


@pytest.mark.slow
def test_kl_lock_full_size():
    """The KL-lock workload at full size: N=4096, V=126464, 60 % locked (M=1639), eps=0.01, gate 0.5."""
    say("kl_lock full size")
    case = W.kl_lock_case()
    assert case.M_tot == 1639
    g = _run_kl(case, 0.01, 0.5, -1, True)
    st, lr = _oracle_kl(case, 0.01, 0.5, -1, True)
    nd = _compare_kl(case, g, st, lr, 0.01, 0.5, True)
    say("full-size KL-lock: new locks gpu %d oracle %d, exempt mismatches %d" % (
        int(g["locked"].sum() - case.locked.sum()), int(lr.locked.sum() - case.locked.sum()), nd))
    assert nd == 0


@pytest.mark.slow
def test_kl_lock_full_size_cached_prev_lse():
    """The full-size KL-lock workload in the loop's steady state: the previous posterior's LSE from the
    store of the pass that produced it (the configuration the benchmark times)."""
    say("kl_lock full size, cached previous LSE")
    case = W.kl_lock_case()
    g = _run_kl(case, 0.01, 0.5, -1, True, cached_lse=True)
    st, lr = _oracle_kl(case, 0.01, 0.5, -1, True)
    nd = _compare_kl(case, g, st, lr, 0.01, 0.5, True)
    say("full-size KL-lock, cached LSE: exempt mismatches %d" % nd)
    assert nd == 0


@pytest.mark.slow
def test_kl_lock_batched_full_size():
    """The KL-lock pass at the batched ragged shape: 8 sequences x N=2048, V=126464, active fraction
    per sequence uniform on [0.05, 0.8], eps=0.05, gate 0.5 per sequence."""
    say("kl_lock batched full size")
    B, N = 8, 2048
    lf = 1.0 - W.ragged_fracs(B, key=B * N)
    case = W.kl_lock_case(N=N, V=126464, B=B, locked_frac=lf, key=B * N)
    g = _run_kl(case, 0.05, 0.5, -1, True)
    st, lr = _oracle_kl(case, 0.05, 0.5, -1, True)
    nd = _compare_kl(case, g, st, lr, 0.05, 0.5, True)
    say("batched KL-lock: M=%d, new locks gpu %d oracle %d, exempt mismatches %d" % (
        case.M_tot, int(g["locked"].sum() - case.locked.sum()), int(lr.locked.sum() - case.locked.sum()), nd))
    assert nd == 0


# ------------------------------------------------------------------ LM head at full vocabulary
@pytest.mark.slow
def test_lm_head_full_vocabulary():
    """Logits of the active rows at d=4096, V=126464, written at rows b*N+pos of the posterior buffer;
    every other row stays untouched.  Max-abs 2e-2 against the float64 product."""
    sl = _sl()
    say("lm head full vocabulary")
    dm = W.LLADA_LAYER
    B, N, Ms = 2, 512, [300, 77]
    g = W.rng(W.SEED_SETS, 4242)
    acts = [np.sort(g.permutation(N)[:M]).astype(np.int32) for M in Ms]
    off = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int32)
    act_idx = np.concatenate(acts)
    M = int(off[-1])
    x = W.to_storage(W.normal(W.rng(W.SEED_ACT, 4242), (M, dm.d), 1.0), "bf16")
    head = W.lm_head_weights(dm)
    out = torch.full((B * N, dm.vocab), 7.0, dtype=torch.bfloat16, device="cuda")
    sl.sl_gemm(sl.SL_EPI_LOGITS, dev(x, "bf16"), M, dm.d, dm.vocab, dev(head, "bf16"), out0=out,
               act_idx=torch.from_numpy(act_idx).cuda(), act_off=torch.from_numpy(off).cuda(), B=B, N=N)
    torch.cuda.synchronize()
    glob = O.seq_of_rows(off) * N + act_idx.astype(np.int64)
    ref = O.widen(x, "bf16") @ O.widen(head, "bf16").T
    got = host64(out)
    err = np.max(np.abs(got[glob] - ref))
    say("lm head max |err| %.3e" % err)
    assert err <= 2e-2
    others = np.setdiff1d(np.arange(B * N), glob)
    assert np.all(got[others] == 7.0)


# ------------------------------------------------------------------ gathered-row GEMM, every tile shape
# (epilogue, M, K, n_out): shapes on which the launcher's cost model picks each of its tile
# shapes (and split-K for the residual); the union is checked to cover every tile.
GEMM_CASES = [
    ("resid", 16, 512, 768), ("resid", 16, 1024, 768), ("swiglu", 130, 512, 12288),
    ("resid", 16, 1024, 12288), ("resid", 16, 2048, 12288), ("swiglu", 300, 512, 12288),
    ("resid", 130, 4096, 6144), ("swiglu", 700, 512, 12288), ("swiglu", 128, 512, 36864),
    ("swiglu", 640, 512, 18432), ("swiglu", 768, 512, 18432), ("qkv", 300, 512, 1536),
    ("qkv", 700, 1024, 3072), ("logits", 130, 512, 6144), ("logits", 600, 1024, 12288),
    ("swiglu", 16, 512, 24576), ("swiglu", 16, 512, 768), ("resid", 1, 2048, 6144),
    ("logits", 5, 1024, 24576), ("qkv", 16, 8192, 24576),
    ("qkv", 250, 512, 12288), ("swiglu", 450, 512, 6144), ("resid", 200, 512, 12288), ("logits", 770, 512, 3072),
    ("qkv", 390, 512, 12288), ("swiglu", 200, 512, 18432), ("resid", 700, 512, 6144), ("logits", 450, 512, 12288),
    ("qkv", 520, 512, 6144), ("resid", 900, 512, 8192),
    # more than 8 row tiles: the tile order walks groups of 8 row tiles, the last group partial
    ("logits", 2400, 512, 2048), ("swiglu", 2300, 512, 4096), ("resid", 2200, 512, 2048), ("qkv", 2400, 512, 1536),
]
# (tile rows, tile columns, weights through registers instead of direct-to-LDS loads)
ALL_TILES = {(256, 256, 0), (256, 128, 0), (128, 256, 0), (128, 128, 0), (128, 64, 0), (256, 192, 0), (128, 384, 0),
             (64, 128, 0), (64, 64, 0), (64, 128, 1), (128, 96, 0), (128, 192, 0)}


def tile_of(sl, epi, M, K, n):
    bm, bn, _, vb = sl.sl_gemm_plan(torch.bfloat16, epi, M, K, n, with_path=True)
    return bm, bn, vb


def test_gemm_cases_cover_every_tile():
    sl = _sl()
    epi = {"resid": sl.SL_EPI_RESIDUAL, "swiglu": sl.SL_EPI_SWIGLU, "qkv": sl.SL_EPI_QKV_ROPE,
           "logits": sl.SL_EPI_LOGITS}
    tiles = {tile_of(sl, epi[e], M, K, n) for e, M, K, n in GEMM_CASES}
    assert tiles == ALL_TILES


@pytest.mark.parametrize("kind,M,K,n_out", GEMM_CASES)
def test_gemm_parity(kind, M, K, n_out):
    """sl_gemm against the float64 product of the same bf16 inputs, per epilogue."""
    sl = _sl()
    say("gemm", kind, M, K, n_out, sl.sl_gemm_plan(torch.bfloat16, {"resid": 1, "swiglu": 2, "qkv": 0, "logits": 3}[kind],
                                                   M, K, n_out, with_path=True))
    g = W.rng(W.SEED_ACT, 9000 + M + K + n_out)
    A = W.to_storage(W.normal(g, (M, K), 1.0), "bf16")
    A64 = O.widen(A, "bf16")
    if kind == "swiglu":
        F = n_out // 2
        w0 = W.to_storage(W.normal(g, (F, K), 0.02), "bf16")
        w1 = W.to_storage(W.normal(g, (F, K), 0.02), "bf16")
        out = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
        sl.sl_gemm(sl.SL_EPI_SWIGLU, dev(A, "bf16"), M, K, n_out, dev(w0, "bf16"), dev(w1, "bf16"), out0=out)
        ref = O.silu(A64 @ O.widen(w0, "bf16").T) * (A64 @ O.widen(w1, "bf16").T)
        got = host64(out)
        # half a bf16 ulp of the stored product, plus the fp32 accumulation of g = a.w_g and u = a.w_u
        # over K (|dg| <= K 2^-24 sum_k |a_k w_k|, likewise du) carried through SiLU(g) u:
        # |d(SiLU(g) u)| <= max|SiLU'| |u| |dg| + |SiLU(g)| |du|, with max|SiLU'| < 1.1; 2e-6 relative
        # covers the fp32 evaluation of SiLU (exp and reciprocal) and of the product
        wg64, wu64 = O.widen(w0, "bf16"), O.widen(w1, "bf16")
        gg, uu = A64 @ wg64.T, A64 @ wu64.T
        dg = K * 2.0 ** -24 * (np.abs(A64) @ np.abs(wg64).T)
        du = K * 2.0 ** -24 * (np.abs(A64) @ np.abs(wu64).T)
        acc = 1.1 * np.abs(uu) * dg + np.abs(O.silu(gg)) * du
        bound = (2.0 ** -8 + 2e-6) * np.abs(ref) + (1 + 2.0 ** -8) * acc
        excess = np.abs(got - ref) - bound
        say("swiglu max |d| %.3e, max excess over the bound %.3e" % (np.abs(got - ref).max(), excess.max()))
        assert excess.max() <= 0, "swiglu mismatch"
        return
    if kind == "resid":
        w0 = W.to_storage(W.normal(g, (n_out, K), 0.02), "bf16")
        h0 = W.normal(g, (M, n_out), 1.0).astype(np.float32)
        out = torch.from_numpy(h0.copy()).cuda()
        sl.sl_gemm(sl.SL_EPI_RESIDUAL, dev(A, "bf16"), M, K, n_out, dev(w0, "bf16"), out0=out)
        ref = h0.astype(np.float64) + A64 @ O.widen(w0, "bf16").T
        np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-4, atol=2e-3)
        return
    # row-to-position maps over two ragged sequences
    B, N = 2, max(512, M)
    m0 = M // 3
    acts = [np.sort(g.permutation(N)[:m0]), np.sort(g.permutation(N)[:M - m0])]
    off = np.array([0, m0, M], dtype=np.int32)
    act_idx = np.concatenate(acts).astype(np.int32)
    glob = O.seq_of_rows(off) * N + act_idx.astype(np.int64)
    ai, ao = torch.from_numpy(act_idx).cuda(), torch.from_numpy(off).cuda()
    if kind == "logits":
        w0 = W.to_storage(W.normal(g, (n_out, K), 0.02), "bf16")
        out = torch.full((B * N, n_out), 3.0, dtype=torch.bfloat16, device="cuda")
        sl.sl_gemm(sl.SL_EPI_LOGITS, dev(A, "bf16"), M, K, n_out, dev(w0, "bf16"), out0=out, act_idx=ai,
                   act_off=ao, B=B, N=N)
        got = host64(out)
        assert bf16_out_err(got[glob], A64 @ O.widen(w0, "bf16").T) <= 0
        assert np.all(np.delete(got, glob, axis=0) == 3.0)
        return
    # QKV + RoPE + cache scatter
    d, Dh = K, 64
    H = d // Dh
    ws = [W.to_storage(W.normal(g, (d, d), 0.02), "bf16") for _ in range(3)]
    rope = torch.empty(N, Dh // 2, 2, dtype=torch.float32, device="cuda")
    sl.sl_rope_table(N, Dh, 1e4, rope)
    q = torch.empty(M, d, dtype=torch.bfloat16, device="cuda")
    kc = torch.full((B, N, d), 5.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, N, d), 5.0, dtype=torch.bfloat16, device="cuda")
    sl.sl_gemm(sl.SL_EPI_QKV_ROPE, dev(A, "bf16"), M, d, 3 * d, *[dev(w, "bf16") for w in ws], out0=q, out1=kc,
               out2=vc, rope=rope, d=d, head_dim=Dh, act_idx=ai, act_off=ao, B=B, N=N)
    W64 = [O.widen(w, "bf16") for w in ws]
    rq = O.rope((A64 @ W64[0].T).reshape(M, H, Dh), act_idx, 1e4).reshape(M, d)
    rk = O.rope((A64 @ W64[1].T).reshape(M, H, Dh), act_idx, 1e4).reshape(M, d)
    rv = A64 @ W64[2].T
    assert bf16_out_err(host64(q), rq) <= 0
    gk, gv = host64(kc).reshape(B * N, d), host64(vc).reshape(B * N, d)
    assert bf16_out_err(gk[glob], rk) <= 0
    assert bf16_out_err(gv[glob], rv) <= 0
    assert np.all(np.delete(gk, glob, axis=0) == 5.0) and np.all(np.delete(gv, glob, axis=0) == 5.0)


# ------------------------------------------------------------------ measurement variants
@pytest.mark.parametrize("kind,M,K,n_out", [("swiglu", 300, 512, 12288), ("swiglu", 1024, 1024, 6144),
                                             ("logits", 130, 512, 6144), ("logits", 700, 1024, 3072)])
def test_gemm_clocked_matches_gemm(kind, M, K, n_out):
    """The clock-recording GEMM variant stores exactly what sl_gemm stores (the same launch plan and
    arithmetic), and fills one plausible record per workgroup: a clock between 0.3 and 4 GHz, a k-tile
    loop shorter than the workgroup, K elements multiplied."""
    sl = _sl()
    epi = sl.SL_EPI_SWIGLU if kind == "swiglu" else sl.SL_EPI_LOGITS
    bm, bn, split = sl.sl_gemm_plan(torch.bfloat16, epi, M, K, n_out)
    nwg = -(-M // bm) * (n_out // bn) * split
    say("gemm_clocked", kind, M, K, n_out, (bm, bn, split), nwg)
    g = W.rng(W.SEED_ACT, 9100 + M + K + n_out)
    A = dev(W.to_storage(W.normal(g, (M, K), 1.0), "bf16"), "bf16")
    clocks = torch.full((4 * nwg + 4,), -1, dtype=torch.int64, device="cuda")
    clocks[: 4 * nwg].zero_()
    if kind == "swiglu":
        F = n_out // 2
        w0 = dev(W.to_storage(W.normal(g, (F, K), 0.02), "bf16"), "bf16")
        w1 = dev(W.to_storage(W.normal(g, (F, K), 0.02), "bf16"), "bf16")
        ref = torch.empty(M, F, dtype=torch.bfloat16, device="cuda")
        got = torch.empty_like(ref)
        sl.sl_gemm(epi, A, M, K, n_out, w0, w1, out0=ref)
        sl.sl_gemm_clocked(epi, A, M, K, n_out, w0, w1, out0=got, clocks=clocks[: 4 * nwg])
    else:
        B, N = 2, max(512, M)
        m0 = M // 3
        acts = [np.sort(g.permutation(N)[:m0]), np.sort(g.permutation(N)[:M - m0])]
        ai = torch.from_numpy(np.concatenate(acts).astype(np.int32)).cuda()
        ao = torch.tensor([0, m0, M], dtype=torch.int32, device="cuda")
        w0 = dev(W.to_storage(W.normal(g, (n_out, K), 0.02), "bf16"), "bf16")
        ref = torch.full((B * N, n_out), 3.0, dtype=torch.bfloat16, device="cuda")
        got = ref.clone()
        sl.sl_gemm(epi, A, M, K, n_out, w0, out0=ref, act_idx=ai, act_off=ao, B=B, N=N)
        sl.sl_gemm_clocked(epi, A, M, K, n_out, w0, out0=got, act_idx=ai, act_off=ao, B=B, N=N,
                           clocks=clocks[: 4 * nwg])
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    c = clocks.cpu().numpy()
    assert np.all(c[4 * nwg:] == -1)   # nothing past the record
    c = c[: 4 * nwg].reshape(nwg, 4).astype(np.float64)
    ghz = c[:, 0] / c[:, 1] / 10.0
    say("clock GHz min %.2f median %.2f max %.2f" % (ghz.min(), np.median(ghz), ghz.max()))
    assert np.all(c[:, 1] > 0) and np.all((ghz > 0.3) & (ghz < 4.0))
    assert np.all((c[:, 2] > 0) & (c[:, 2] < c[:, 0]))
    assert np.all(c[:, 3] * split == K)


def test_peak_mfma_operands_clocks():
    """The operand-dependent MFMA loop fills one clock record per workgroup and nothing beyond."""
    sl = _sl()
    wg, iters = 64, 256
    ops = torch.randn(16 * 256 * 8, device="cuda").to(torch.bfloat16)
    sink = torch.zeros(256, device="cuda")
    clocks = torch.full((2 * wg + 2,), -1, dtype=torch.int64, device="cuda")
    flops = sl.sl_peak_mfma_operands(wg, iters, ops, sink, clocks[: 2 * wg])
    torch.cuda.synchronize()
    assert flops == wg * 4 * iters * 4 * 2.0 * 32 * 32 * 16
    c = clocks.cpu().numpy()
    assert np.all(c[2 * wg:] == -1)
    c = c[: 2 * wg].reshape(wg, 2).astype(np.float64)
    assert np.all(c[:, 1] > 0)
    ghz = c[:, 0] / c[:, 1] / 10.0
    assert np.all((ghz > 0.3) & (ghz < 4.0))
    with pytest.raises(Exception):
        sl.sl_peak_mfma_operands(wg, iters + 3, ops, sink)   # not a multiple of the 8 operand sets


# ------------------------------------------------------------------ attention
ATTN_CASES = [
    # dtype, Dh, H, N, Ms
    ("bf16", 128, 2, 256, [256, 37]),
    ("bf16", 128, 3, 1024, [5]),          # few query tiles: split over keys + merge
    ("bf16", 128, 32, 1024, [40]),        # split four ways (128 keys per key group)
    ("bf16", 128, 32, 1024, [768]),       # 128-query workgroups: 64-query ones would not fit one wave
    ("bf16", 128, 32, 512, [9]),          # short sequence, few queries: four key groups, no split
    ("bf16", 128, 4, 256, [3, 60]),       # the same with two sequences
    ("bf16", 128, 2, 64, [7]),            # four key groups over two 32-key tiles: two groups idle
    ("bf16", 128, 8, 512, [300, 1, 77]),  # heads a multiple of 8 (XCD placement), ragged
    ("bf16", 128, 16, 1024, [640]),       # several query tiles per head, no split
    ("bf16", 128, 32, 1024, [1024]),      # 128-query workgroups (two key groups)
    ("bf16", 128, 32, 1024, [256]),       # 64-query workgroups, four key groups of 256 keys, half the chip
    ("bf16", 128, 32, 1024, [100, 28]),   # the same with two sequences and ragged tiles
    ("bf16", 128, 32, 1024, [600, 500]),  # same, ragged tails in both sequences
    ("bf16", 128, 32, 576, [560]),        # nine key tiles: one key group has none in the last round
    ("bf16", 64, 2, 128, [1, 128, 70]),
    ("bf16", 32, 4, 64, [64]),
    ("f32", 32, 4, 64, [64, 3]),
    ("f32", 128, 2, 192, [150]),
    ("f32", 64, 1, 512, [9, 300]),
]


def _attn_abs_weighted(q, K, V, scale):
    """(P |V|) per output element, P = softmax(q K^T scale) in float64: the sum that bounds what
    rounding the probabilities can move an output by."""
    qh, kh, vh = np.transpose(q, (1, 0, 2)), np.transpose(K, (1, 2, 0)), np.transpose(np.abs(V), (1, 0, 2))
    s_ = (qh @ kh) * scale
    s_ -= s_.max(axis=-1, keepdims=True)
    p_ = np.exp(s_)
    p_ /= p_.sum(axis=-1, keepdims=True)
    return np.transpose(p_ @ vh, (1, 0, 2))


def _check_attention(got, q64, K64, V64, off, keys, Dh, dtype):
    """Per sequence against the float64 oracle over the attended keys (all N, or `keys`).  fp32:
    2e-5 absolute.  bf16: relative L2 within the margin over the bf16-storage emulation (P rounded
    before P.V, output rounded) of the same inputs.  Per element, the worst case of those roundings:
    o = sum_j P_j v_j / l with every P_j rounded to bf16 (|dP_j| <= 2^-8 P_j) moves o by at most
    2^-8 sum_j p_j |v_j|; 1e-4 of that and of |o| covers the fp32 scores, exponentials and row sum;
    the stored output adds half an ulp (at most 2^-8 |o|)."""
    for b in range(len(off) - 1):
        s_ = slice(off[b], off[b + 1])
        Kb, Vb = (K64[b], V64[b]) if keys[b] is None else (K64[b][keys[b]], V64[b][keys[b]])
        ref = O.attention(q64[s_], Kb, Vb, 1.0 / math.sqrt(Dh))
        if dtype == "f32":
            np.testing.assert_allclose(got[s_], ref, atol=2e-5, rtol=0)
            continue
        emu = E.err_stats(E.attention(q64[s_], Kb, Vb, 1.0 / math.sqrt(Dh)), ref)
        g = E.err_stats(got[s_], ref)
        l2_b = E.bounds(emu)[0]
        assert g.rel_l2 <= l2_b, "attention, sequence %d: relative L2 %.3e > %.3e (emulated %.3e)" % (
            b, g.rel_l2, l2_b, emu.rel_l2)
        pv = _attn_abs_weighted(q64[s_], Kb, Vb, 1.0 / math.sqrt(Dh))
        lim = 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * ((2.0 ** -8 + 1e-4) * pv + 1e-4 * np.abs(ref))
        excess = float(np.max(np.abs(got[s_] - ref) - lim)) if g.n else 0.0
        say("attention seq %d: rel L2 %.3e (emulated %.3e), max %.3e (emulated %.3e), max |d| / bound %.3f" % (
            b, g.rel_l2, emu.rel_l2, g.max, emu.max, float(np.max(np.abs(got[s_] - ref) / lim)) if g.n else 0.0))
        assert excess <= 0, "attention, sequence %d: an element exceeds its rounding bound by %.3e" % (b, excess)


@pytest.mark.parametrize("dtype,Dh,H,N,Ms", ATTN_CASES)
def test_attention_parity(dtype, Dh, H, N, Ms):
    sl = _sl()
    say("attn", dtype, Dh, H, N, Ms)
    B = len(Ms)
    g = W.rng(123, Dh, N, len(Ms))
    acts = [np.sort(g.permutation(N)[:M]).astype(np.int32) for M in Ms]
    off = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int32)
    M_tot = int(off[-1])
    q = W.to_storage(W.normal(g, (M_tot, H, Dh), 1.0), dtype)
    Kc = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
    Vc = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
    out = torch.empty(M_tot, H * Dh, dtype=tdtype(dtype), device="cuda")
    ws = torch.empty(max(1, sl.sl_attn_workspace_size(B, N, M_tot, H, Dh)), dtype=torch.uint8, device="cuda")
    sl.sl_attn_active(dev(q, dtype), dev(Kc, dtype), dev(Vc, dtype), torch.from_numpy(off).cuda(), B, N, M_tot,
                      H, Dh, 1.0 / math.sqrt(Dh), out, ws)
    got = host64(out).reshape(M_tot, H, Dh)
    q64, K64, V64 = O.widen(q, dtype), O.widen(Kc, dtype), O.widen(Vc, dtype)
    _check_attention(got, q64, K64, V64, off, [None] * B, Dh, dtype)


# The no-KV-cache ablation: every query attends over its sequence's active positions only
# (the other positions' flags are set).  Key patterns: "random" = active set uniform;
# "ends" = active positions in the first and last eighth (whole key tiles excluded in
# between); "first" = active positions inside the first 64 keys (with a key split, every
# other split sees no key at all).
ATTN_EXCL_CASES = [
    ("bf16", 128, 3, 1024, [5], "first"),
    ("bf16", 128, 32, 512, [9], "random"),
    ("bf16", 128, 8, 512, [300, 1, 77], "random"),
    ("bf16", 128, 32, 1024, [200, 180], "ends"),
    ("bf16", 128, 16, 1024, [200], "ends"),
    ("bf16", 128, 32, 1024, [1024], "random"),
    ("bf16", 128, 32, 576, [560], "ends"),
    ("bf16", 64, 2, 128, [1, 128, 70], "random"),
    ("f32", 128, 2, 192, [150], "random"),
    ("f32", 32, 4, 128, [3, 64], "first"),
    ("f32", 64, 1, 512, [9, 120], "ends"),
]


def _active_keys(g, N, M, pattern):
    if pattern == "random":
        return np.sort(g.permutation(N)[:M]).astype(np.int32)
    if pattern == "first":
        return np.sort(g.permutation(64)[:M]).astype(np.int32)
    pool = np.concatenate([np.arange(N // 8), np.arange(N - N // 8, N)])
    return np.sort(g.permutation(pool)[:M]).astype(np.int32)


@pytest.mark.parametrize("dtype,Dh,H,N,Ms,pattern", ATTN_EXCL_CASES)
def test_attention_excluded_keys_parity(dtype, Dh, H, N, Ms, pattern):
    sl = _sl()
    say("attn excl", dtype, Dh, H, N, Ms, pattern)
    B = len(Ms)
    g = W.rng(124, Dh, N, len(Ms))
    acts = [_active_keys(g, N, M, pattern) for M in Ms]
    off = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int32)
    M_tot = int(off[-1])
    excl = np.ones(B * N, np.uint8)
    for b in range(B):
        excl[b * N + acts[b]] = 0
    q = W.to_storage(W.normal(g, (M_tot, H, Dh), 1.0), dtype)
    Kc = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
    Vc = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
    out = torch.empty(M_tot, H * Dh, dtype=tdtype(dtype), device="cuda")
    ws = torch.empty(max(1, sl.sl_attn_workspace_size(B, N, M_tot, H, Dh)), dtype=torch.uint8, device="cuda")
    sl.sl_attn_active(dev(q, dtype), dev(Kc, dtype), dev(Vc, dtype), torch.from_numpy(off).cuda(), B, N, M_tot,
                      H, Dh, 1.0 / math.sqrt(Dh), out, ws, key_excl=torch.from_numpy(excl).cuda())
    got = host64(out).reshape(M_tot, H, Dh)
    assert np.isfinite(got).all()
    q64, K64, V64 = O.widen(q, dtype), O.widen(Kc, dtype), O.widen(Vc, dtype)
    _check_attention(got, q64, K64, V64, off, acts, Dh, dtype)


# ------------------------------------------------------------------ cache scatter
def test_cache_scatter_bit_exact():
    sl = _sl()
    say("scatter")
    B, N, H, Dh = 3, 128, 2, 64
    for dtype in ("bf16", "f32"):
        g = W.rng(5, 5)
        Ms = [0, 77, 128]
        acts = [np.sort(g.permutation(N)[:M]).astype(np.int32) for M in Ms]
        ai = np.concatenate(acts).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(Ms)]).astype(np.int32)
        M = int(off[-1])
        kc0 = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
        vc0 = W.to_storage(W.normal(g, (B, N, H, Dh), 1.0), dtype)
        kn = W.to_storage(W.normal(g, (M, H, Dh), 1.0), dtype)
        vn = W.to_storage(W.normal(g, (M, H, Dh), 1.0), dtype)
        kc, vc = dev(kc0, dtype), dev(vc0, dtype)
        sl.sl_cache_scatter(kc, vc, dev(kn, dtype), dev(vn, dtype), torch.from_numpy(ai).cuda(),
                            torch.from_numpy(off).cuda(), B, N, M, H, Dh)
        ek, ev = kc0.copy(), vc0.copy()
        for b in range(B):
            ek[b, acts[b]] = kn[off[b]:off[b + 1]]
            ev[b, acts[b]] = vn[off[b]:off[b + 1]]
        view = (lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)) if dtype == "bf16" else (lambda t: t.cpu().numpy())
        np.testing.assert_array_equal(view(kc), ek)
        np.testing.assert_array_equal(view(vc), ev)
