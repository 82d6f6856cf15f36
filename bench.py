#!/usr/bin/env python3
"""SureLock step benchmark on one MI355X.

One timed step = the hot path over one batch of synthetic input:
  * the SureLock layer step at the LLaDA-8B layer shape (d=4096, 32 heads x 128,
    SwiGLU 12288, bf16, N=1024, batch 1) for each active-set size
    M in {1024, 512, 256, 64} (gather, RMSNorm, QKV + RoPE + K/V scatter,
    attention of M queries over all N cached keys, O projection, SwiGLU FFN);
  * the KL-lock pass (N=4096, V=126464, 60 % already locked -> M=1639,
    eps=0.01, gate at the 0.5 quantile): vocabulary pass, gate, lock update,
    compaction.
Also reported, outside `value`: the batched ragged step (8 x N=2048, one layer +
LM head + KL-lock + compaction) and the 32-layer sampler loop.
value = algorithmic TFLOP/s of the layer sweep (FLOPs of the four layer steps
over their summed time).  Inputs are resident in HBM; weights rotate over 3
copies and logits over 2 copies (each larger than the 256 MB Infinity Cache).
Synthetic data: random N(0, 0.02) weights and N(0,1) hidden rows / caches;
logits N(0, 2^2) with +8 spikes in 70 % of rows and N(0, 0.05^2) drift.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SureLock step ms & TFLOP/s vs M/N at LLaDA-8B layer shape; KL-lock HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
D, H, DH, F, N_LAYER = 4096, 32, 128, 12288, 1024
MS = (1024, 512, 256, 64)
N_KL, V_KL, EPS_KL, GATE_KL = 4096, 126464, 0.01, 0.5


def layer_flops(M, N=N_LAYER, d=D, f=F):
    return float(M) * (8.0 * d * d + 6.0 * d * f + 4.0 * N * d)


def layer_bytes(M, N=N_LAYER, d=D, f=F):
    weights = 2.0 * (4 * d * d + 3 * d * f)
    return weights + 2.0 * N * d * 2 + M * d * 2.0 * 4


def kl_bytes(M, N=N_KL, V=V_KL):
    # both logit rows of every active row, mask read and write, per-row outputs, new list
    return 2.0 * M * V * 2 + 2.0 * N + 16.0 * M + 4.0 * (N + 2)


# HBM traffic of the two roofline kernels from rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) of `python3 bench.py --profile-kernels`, each scaled by
# what the counter reads for a plain device copy of known size in the same run.  Valid
# only for the kernel sources they were taken on (sha256 of the listed files); otherwise
# the report says null.
TRAFFIC = {
    "gemm": {"files": ["token_locking_sparse_amd/csrc/gemm.hip"],
             "sha256": "e5f1e7f1fcf5263ed631bb9c27a288938a92aee728f89564972e677793a4b23a", "bytes": 427913169},
    "kl": {"files": ["token_locking_sparse_amd/csrc/kl_lock.hip"],
           "sha256": "a6a4e62877720e68390bd3e5422ba13a6e5dc9e146d828b897213f02f43c1d32", "bytes": 829654277},
}


def _sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(key):
    t = TRAFFIC[key]
    if t["bytes"] is None or t["sha256"] != _sources_sha(t["files"]):
        return None
    return t["bytes"]


def gpu_part(args):
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import token_locking_sparse_amd.surelock as S
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16

    def randn(shape, std=1.0):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

    # ---------------- layer-step inputs (3 weight copies)
    shapes = {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    wsets = [{k: randn(s, 0.02) for k, s in shapes.items()} for _ in range(3)]
    models = [sl.DeviceModel(dtype=bf, n_layers=1, d=D, n_heads=H, head_dim=DH, ffn=F, vocab=126464, rms_eps=1e-5,
                             rope_theta=1e4, layers=[w], rope_n=N_LAYER) for w in wsets]
    h_in = randn((N_LAYER, D))
    kc = randn((1, 1, N_LAYER, H, DH))
    vc = randn((1, 1, N_LAYER, H, DH))
    states = {}
    for M in MS:
        act = W.choose_active(N_LAYER, M, W.SEED_SETS, M)
        locked = torch.from_numpy(W.locked_from_active(N_LAYER, act)).to(dev)
        st = sl.DeviceState(models[0], 1, N_LAYER, locked=locked, h_in=h_in, k_cache=kc, v_cache=vc,
                            with_h_out=True)
        assert st.M_tot == M
        states[M] = (st, st.struct())
    p_layer = S.sl_step_params(0.0, -1.0, -1, 0, 0)

    # ---------------- KL-lock inputs (2 logits copies)
    locked_np, act_idx_np, act_off_np = W.kl_lock_mask(N_KL, 1, 0.6, 0)
    M_kl = int(act_off_np[-1])
    kl_sets = []
    for sidx in range(2):
        cur = torch.randn((N_KL, V_KL), generator=g, device=dev, dtype=torch.float32).mul_(2.0)
        rows = torch.randperm(N_KL, generator=g, device=dev)[: int(round(0.7 * N_KL))]
        toks = torch.randint(0, V_KL, (rows.numel(),), generator=g, device=dev)
        cur[rows, toks] += 8.0
        prev = (cur + 0.05 * torch.randn((N_KL, V_KL), generator=g, device=dev, dtype=torch.float32)).to(bf)
        kl_sets.append((cur.to(bf), prev))
        del cur
        torch.cuda.empty_cache()
    kl_locked0 = torch.from_numpy(locked_np).to(dev)
    kl_locked = kl_locked0.clone()
    kl_ai = torch.from_numpy(act_idx_np).to(dev)
    kl_ao = torch.from_numpy(act_off_np).to(dev)
    kl_out = {k: torch.empty(M_kl, device=dev) for k in ("kl", "u", "lse", "conf")}
    kl_am = torch.empty(M_kl, dtype=torch.int32, device=dev)
    kl_thr = torch.empty(1, device=dev)
    kl_nai = torch.empty(N_KL, dtype=torch.int32, device=dev)
    kl_nao = torch.empty(2, dtype=torch.int32, device=dev)
    kl_ws = torch.empty(sl.sl_kl_lock_workspace_size(1, N_KL, M_kl, V_KL), dtype=torch.uint8, device=dev)

    def kl_call(i):
        cur, prev = kl_sets[i % 2]
        sl.sl_kl_lock(cur, prev, V_KL, kl_ai, kl_ao, 1, N_KL, M_kl, None, EPS_KL, GATE_KL, -1, True, kl_locked,
                      kl_out["kl"], kl_out["u"], kl_out["lse"], kl_am, kl_out["conf"], kl_thr, kl_nai, kl_nao, kl_ws)

    def layer_call(i, M):
        st, sst = states[M]
        S.sl_step(models[i % 3].s, sst, p_layer, st.ws)

    # ---------------- timed steps
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_it = args.warmup + args.steps
    evs = [{M: (ev(), ev()) for M in MS} for _ in range(n_it)]
    evk = [(ev(), ev()) for _ in range(n_it)]
    torch.cuda.synchronize()
    t0 = None
    for i in range(n_it):
        if i == args.warmup:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        for M in MS:
            evs[i][M][0].record()
            layer_call(i, M)
            evs[i][M][1].record()
        evk[i][0].record()
        kl_call(i)
        evk[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_M = {M: float(np.mean([evs[i][M][0].elapsed_time(evs[i][M][1]) for i in range(args.warmup, n_it)])) for M in MS}
    ms_kl = float(np.mean([evk[i][0].elapsed_time(evk[i][1]) for i in range(args.warmup, n_it)]))
    M_after = int(kl_nao[1].item())

    # ---------------- the no-KV-cache ablation on the same active sets: attention over the M
    # active positions instead of all N (outside `value`)
    p_abl = S.sl_step_params(0.0, -1.0, -1, 0, 0, 1)
    ms_abl = {}
    for M in MS:
        st, sst = states[M]
        es = []
        for i in range(args.warmup + args.steps):
            e0, e1 = ev(), ev()
            e0.record()
            S.sl_step(models[i % 3].s, sst, p_abl, st.ws)
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        ms_abl[M] = float(np.mean([a.elapsed_time(b) for a, b in es[args.warmup:]]))

    # ---------------- dominant kernel alone: the FFN gate/up GEMM + SwiGLU at M = 1024
    Mg = 1024
    xa = randn((Mg, D))
    act = torch.empty(Mg, F, dtype=bf, device=dev)
    kg = []
    for i in range(args.warmup + args.steps):
        w = wsets[i % 3]
        e0, e1 = ev(), ev()
        e0.record()
        sl.sl_gemm(sl.SL_EPI_SWIGLU, xa, Mg, D, 2 * F, w["wg"], w["wu"], out0=act)
        e1.record()
        kg.append((e0, e1))
    torch.cuda.synchronize()
    ms_gu = float(np.mean([a.elapsed_time(b) for a, b in kg[args.warmup:]]))

    # breakdown of the M=1024 layer step by GEMM (same kernels sl_step launches)
    h32 = torch.zeros(Mg, D, dtype=torch.float32, device=dev)
    actx = randn((Mg, F))
    qb = torch.empty(Mg, D, dtype=bf, device=dev)
    st1024 = states[1024][0]
    br = {}
    for name, fn in (
        ("qkv_rope_scatter", lambda w: sl.sl_gemm(sl.SL_EPI_QKV_ROPE, xa, Mg, D, 3 * D, w["wq"], w["wk"], w["wv"],
                                                   out0=qb, out1=kc, out2=vc, rope=models[0].rope, d=D, head_dim=DH,
                                                   act_idx=st1024.act_idx, act_off=st1024.act_off, B=1, N=N_LAYER)),
        ("o_proj_residual", lambda w: sl.sl_gemm(sl.SL_EPI_RESIDUAL, xa, Mg, D, D, w["wo"], out0=h32)),
        ("down_residual", lambda w: sl.sl_gemm(sl.SL_EPI_RESIDUAL, actx, Mg, F, D, w["wd"], out0=h32)),
    ):
        es = []
        for i in range(args.warmup + args.steps):
            e0, e1 = ev(), ev()
            e0.record()
            fn(wsets[i % 3])
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        br[name] = float(np.mean([a.elapsed_time(b) for a, b in es[args.warmup:]]))
    br["gate_up_swiglu"] = ms_gu

    per_M = []
    for M in MS:
        fl, by = layer_flops(M), layer_bytes(M)
        t = ms_M[M] * 1e-3
        floor = max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
        per_M.append({"M": M, "M_over_N": M / N_LAYER, "ms": round(ms_M[M], 4), "tflops": round(fl / t / 1e12, 2),
                      "gbs": round(by / t / 1e9, 1), "frac_mfma_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "frac_roofline": round(floor / t, 4)})
    tot_fl = sum(layer_flops(M) for M in MS)
    tot_ms = sum(ms_M.values())
    kb = kl_bytes(M_kl)
    fl_gu = 4.0 * Mg * D * F
    gu_plan = sl.sl_gemm_plan(bf, sl.SL_EPI_SWIGLU, Mg, D, 2 * F)
    out = {
        "value": round(tot_fl / (tot_ms * 1e-3) / 1e12, 3),
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "per_M": per_M,
        "kl_lock": {"ms": round(ms_kl, 4), "gbs": round(kb / (ms_kl * 1e-3) / 1e9, 1), "bytes": kb, "M": M_kl,
                    "M_after": M_after, "frac_hbm_peak": round(kb / (ms_kl * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "kernels_ms_M1024": {k: round(v, 4) for k, v in br.items()},
        "ablation_no_kv_cache_ms": {str(M): round(v, 4) for M, v in ms_abl.items()},
        "roofline": {"kernel": "gemm_kernel<bf16,%dx%d,split %d,EPI_SWIGLU> (FFN gate/up + SwiGLU, M=1024)" % gu_plan,
                     "bound": "mfma",
                     "achieved": round(fl_gu / (ms_gu * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fl_gu / (ms_gu * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "traffic": traffic_for("gemm"),
                     "flops_per_launch": fl_gu, "avg_launch_ms": round(ms_gu, 4)},
        "roofline_kl": {"kernel": "kl_rows_kernel + kl_tail_kernel <bf16> (KL-lock pass, M=1639, V=126464)", "bound": "hbm",
                        "achieved": round(kb / (ms_kl * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(kb / (ms_kl * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": traffic_for("kl"),
                        "bytes_per_launch": kb, "avg_launch_ms": round(ms_kl, 4)},
    }
    return out


SURELOCK_RUNS = (("eps=0", 0.0, -1.0, False), ("eps=0.01", 0.01, -1.0, False), ("eps=0.05", 0.05, -1.0, False))
# the notes page's ablations: confidence gate only (eps = +inf, gate at the median u), and
# no KV cache (positions locked before a step are not attended)
ABLATION_RUNS = (("gate_only m=0.5", math.inf, 0.5, False), ("no_kv_cache eps=0.05", 0.05, -1.0, True))


def e2e_loop(runs=SURELOCK_RUNS, steps=128, N=512, n_prompt=128, unmask=3, B=1):
    """The whole sampler loop on a 32-layer LLaDA-8B-shaped model with random-init weights (d=4096,
    32 heads x 128, SwiGLU 12288, vocab 126464, bf16), B sequences of N=512 = 128 seeded prompt ids +
    384 [MASK]; 128 steps, 3 unmasks per sequence per step by confidence.  Each run is (name, eps,
    gate quantile or -1 for off, no-KV-cache ablation); eps = 0 is the dense reference (nothing
    locks).  Reports per-step time against the active count M_t (summed over the batch)."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import workloads as W

    dm = W.LLADA_8B
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    bf = torch.bfloat16

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

    shapes = {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    layers = [{k: randn(sh, 0.02) for k, sh in shapes.items()} for _ in range(dm.n_layers)]
    embed = randn((dm.vocab, D), 0.02)
    head = randn((dm.vocab, D), 0.02)
    model = sl.DeviceModel(dtype=bf, n_layers=dm.n_layers, d=D, n_heads=H, head_dim=DH, ffn=F, vocab=dm.vocab,
                           rms_eps=1e-5, rope_theta=1e4, layers=layers, embed=embed, lm_head=head, rope_n=N)
    tok0 = W.prompt_tokens(dm, B, N, n_prompt).reshape(-1)
    out = {}
    for name, eps, gate, no_kv in runs:
        st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).to(dev),
                            cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).to(dev))
        Ms, ms = [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            Ms.append(st.M_tot)
            e0.record()
            st.step(eps, gate, dm.mask_id, True, unmask, no_kv_cache=no_kv)
            e1.record()
            ms.append((e0, e1))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in ms]
        # per row: the layers' projections and FFN, attention over N keys (over the M_t / B active
        # positions of its sequence when locked positions are not attended), and the LM head
        per_row = dm.n_layers * (8.0 * D * D + 6.0 * D * F) + 2.0 * D * dm.vocab
        fl = sum(M_t * (per_row + dm.n_layers * 4.0 * (M_t / B if no_kv else N) * D) for M_t in Ms)
        by_M = {}
        for M_t, t_ms in zip(Ms, ms):
            by_M.setdefault(M_t, []).append(t_ms)
        curve = [[M_t, round(float(np.median(v)), 3)] for M_t, v in sorted(by_M.items(), reverse=True)]
        if len(curve) > 12:
            curve = [curve[i] for i in np.linspace(0, len(curve) - 1, 12).round().astype(int)]
        out[name] = {"ms_total": round(wall * 1e3, 2), "ms_per_step_mean": round(wall * 1e3 / steps, 3),
                               "tokens_per_s": round(B * (N - n_prompt) / wall, 1),
                               "tflops": round(fl / wall / 1e12, 2), "M_first": Ms[0], "M_last": st.M_tot,
                               "rows_computed": int(sum(Ms)), "flops": fl, "ms_vs_M": curve}
        del st
    dense = out.get("eps=0")
    for k, v in out.items():
        if dense:
            v["rows_frac_vs_dense"] = round(v["rows_computed"] / dense["rows_computed"], 4)
            v["flops_frac_vs_dense"] = round(v["flops"] / dense["flops"], 4)
            v["time_frac_vs_dense"] = round(v["ms_total"] / dense["ms_total"], 4)
    del layers, embed, head, model
    torch.cuda.empty_cache()
    return out


def batched_step(steps=5, warmup=2, B=8, N=2048, eps=0.05, gate=0.5):
    """The batched ragged workload: 8 sequences x N=2048, active fraction per sequence uniform on
    [0.05, 0.8] (seeded), one LLaDA-8B-shaped layer + final norm + LM head (V=126464) + KL-lock
    (eps 0.05, gate at each sequence's median u) + compaction, all in one sl_step at t = 1.  The
    previous posterior is this step's own logits plus N(0, 0.05^2) drift, so the KL test passes
    almost everywhere and the gate decides.  Also times, on the same active rows, the layer alone, the
    LM head GEMM alone and the KL-lock pass alone.  Lock state is restored between timed steps
    (outside the timed region)."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import token_locking_sparse_amd.surelock as S
    import workloads as W

    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    bf = torch.bfloat16
    V = V_KL

    def randn(shape, std):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

    Ms = W.ragged_ms(B, N, key=B * N)
    acts = [W.choose_active(N, M, W.SEED_SETS, B * N * 64 + b) for b, M in enumerate(Ms)]
    locked_np = np.concatenate([W.locked_from_active(N, a) for a in acts])
    M_tot = int(sum(Ms))
    shapes = {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    layer = {k: randn(sh, 0.02) for k, sh in shapes.items()}
    head = randn((V, D), 0.02)
    common = dict(dtype=bf, n_layers=1, d=D, n_heads=H, head_dim=DH, ffn=F, vocab=V, rms_eps=1e-5, rope_theta=1e4,
                  layers=[layer], rope_n=N)
    model = sl.DeviceModel(lm_head=head, **common)
    model_l = sl.DeviceModel(**common)
    h_in = randn((B * N, D), 1.0)
    kc = randn((1, B, N, H, DH), 1.0)
    vc = randn((1, B, N, H, DH), 1.0)
    locked0 = torch.from_numpy(locked_np).to(dev)
    st = sl.DeviceState(model, B, N, locked=locked0.clone(), h_in=h_in, k_cache=kc, v_cache=vc,
                        cand=torch.ones(B * N, dtype=torch.uint8, device=dev))
    st_l = sl.DeviceState(model_l, B, N, locked=locked0.clone(), h_in=h_in, k_cache=kc, v_cache=vc)
    assert st.M_tot == M_tot and st_l.M_tot == M_tot
    ai0, ao0 = st.act_idx.clone(), st.act_off.clone()
    # previous posterior: this step's logits (t = 0, no lock) plus drift, in buffer 0
    st.step(0.0, do_lock=False)
    for r0 in range(0, B * N, 1024):
        blk = st.logits[0][r0:r0 + 1024]
        blk.copy_((blk.float() + 0.05 * torch.randn(blk.shape, generator=g, device=dev)).to(bf))
    st.t = 1
    sst = st.struct()
    sst.m_tot_host = None                     # no host copy of M: nothing to wait for inside the timing
    p_full = S.sl_step_params(eps, gate, -1, 1, 0)
    sst_l = st_l.struct()
    p_layer = S.sl_step_params(0.0, -1.0, -1, 0, 0)
    x = randn((M_tot, D), 1.0)
    kl_o = {k: torch.empty(M_tot, device=dev) for k in ("kl", "u", "lse", "conf")}
    kl_am = torch.empty(M_tot, dtype=torch.int32, device=dev)
    kl_thr = torch.empty(B, device=dev)
    kl_nai = torch.empty(B * N, dtype=torch.int32, device=dev)
    kl_nao = torch.empty(B + 1, dtype=torch.int32, device=dev)
    kl_lk = locked0.clone()
    kl_ws = torch.empty(sl.sl_kl_lock_workspace_size(B, N, M_tot, V), dtype=torch.uint8, device=dev)

    def restore():
        st.locked.copy_(locked0)
        st.act_idx.copy_(ai0)
        st.act_off.copy_(ao0)
        kl_lk.copy_(locked0)

    calls = {
        "step": lambda: S.sl_step(model.s, sst, p_full, st.ws),
        "layer": lambda: S.sl_step(model_l.s, sst_l, p_layer, st_l.ws),
        "lm_head": lambda: sl.sl_gemm(sl.SL_EPI_LOGITS, x, M_tot, D, V, head, out0=st.logits[1], act_idx=ai0,
                                      act_off=ao0, B=B, N=N),
        "kl_lock": lambda: sl.sl_kl_lock(st.logits[1], st.logits[0], V, ai0, ao0, B, N, M_tot, None, eps, gate, -1,
                                         True, kl_lk, kl_o["kl"], kl_o["u"], kl_o["lse"], kl_am, kl_o["conf"],
                                         kl_thr, kl_nai, kl_nao, kl_ws),
    }
    ms = {}
    for name, fn in calls.items():
        es = []
        for i in range(warmup + steps):
            restore()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        ms[name] = float(np.mean([a.elapsed_time(b) for a, b in es[warmup:]]))
    restore()
    calls["step"]()
    torch.cuda.synchronize()
    M_after = int(st.act_off[B].item())
    fl_layer = layer_flops(M_tot, N=N)
    fl_head = 2.0 * M_tot * D * V
    kb = kl_bytes(M_tot, N=B * N, V=V)
    head_plan = sl.sl_gemm_plan(bf, sl.SL_EPI_LOGITS, M_tot, D, V)
    out = {"B": B, "N": N, "M_b": Ms, "M_tot": M_tot, "M_after": M_after, "eps": eps, "gate": gate,
           "ms_step": round(ms["step"], 4), "ms_layer": round(ms["layer"], 4), "ms_lm_head": round(ms["lm_head"], 4),
           "ms_kl_lock": round(ms["kl_lock"], 4),
           "step_tflops": round((fl_layer + fl_head) / (ms["step"] * 1e-3) / 1e12, 2),
           "layer_tflops": round(fl_layer / (ms["layer"] * 1e-3) / 1e12, 2),
           "lm_head": {"kernel": "gemm_kernel<bf16,%dx%d,split %d,EPI_LOGITS>" % head_plan, "bound": "mfma",
                       "tflops": round(fl_head / (ms["lm_head"] * 1e-3) / 1e12, 2),
                       "frac_mfma_peak": round(fl_head / (ms["lm_head"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
           "kl": {"bound": "hbm", "bytes": kb, "gbs": round(kb / (ms["kl_lock"] * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(kb / (ms["kl_lock"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del st, st_l, model, model_l, layer, head, h_in, kc, vc, x
    torch.cuda.empty_cache()
    return out


def profile_kernels():
    """Launch only the two roofline kernels and a plain copy of known size, 3 times each
    (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE; the copy calibrates the counters)."""
    import torch

    import token_locking_sparse_amd as sl
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16
    Mg = 1024
    x = (torch.randn((Mg, D), generator=g, device=dev) * 1.0).to(bf)
    wg = (torch.randn((F, D), generator=g, device=dev) * 0.02).to(bf)
    wu = (torch.randn((F, D), generator=g, device=dev) * 0.02).to(bf)
    act = torch.empty(Mg, F, dtype=bf, device=dev)
    locked_np, act_idx_np, act_off_np = W.kl_lock_mask(N_KL, 1, 0.6, 0)
    M_kl = int(act_off_np[-1])
    cur = (torch.randn((N_KL, V_KL), generator=g, device=dev) * 2.0).to(bf)
    prev = (cur.float() + 0.05 * torch.randn((N_KL, V_KL), generator=g, device=dev)).to(bf)
    locked = torch.from_numpy(locked_np).to(dev)
    ai = torch.from_numpy(act_idx_np).to(dev)
    ao = torch.from_numpy(act_off_np).to(dev)
    o = {k: torch.empty(M_kl, device=dev) for k in ("kl", "u", "lse", "conf")}
    am = torch.empty(M_kl, dtype=torch.int32, device=dev)
    thr = torch.empty(1, device=dev)
    nai = torch.empty(N_KL, dtype=torch.int32, device=dev)
    nao = torch.empty(2, dtype=torch.int32, device=dev)
    ws = torch.empty(sl.sl_kl_lock_workspace_size(1, N_KL, M_kl, V_KL), dtype=torch.uint8, device=dev)
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        sl.sl_gemm(sl.SL_EPI_SWIGLU, x, Mg, D, 2 * F, wg, wu, out0=act)
        sl.sl_kl_lock(cur, prev, V_KL, ai, ao, 1, N_KL, M_kl, None, EPS_KL, GATE_KL, -1, True, locked, o["kl"],
                      o["u"], o["lse"], am, o["conf"], thr, nai, nao, ws)
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profiled: gate/up GEMM M=%d plan %s, KL-lock pass M=%d, copy of %d bytes" %
          (Mg, sl.sl_gemm_plan(bf, sl.SL_EPI_SWIGLU, Mg, D, 2 * F), M_kl, src.numel()), flush=True)


def cpu_part(seconds: float):
    """The oracle as it stands, on a bounded sample of the same workload, on the host cores."""
    import numpy as np

    import oracle.surelock_oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info() if i.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover
        cores, blas = os.cpu_count(), "?"
    dm = W.LLADA_LAYER
    od = O.OracleDims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.vocab, dm.rms_eps, dm.rope_theta)
    Wl = {k: O.widen(v, "bf16") for k, v in W.layer_weights(dm, 0).items()}
    M = 64
    case = W.layer_case(dm, N_LAYER, [M], key=M)
    h = O.widen(case.h_in, "bf16")[case.act_idx]
    K = O.widen(case.k_cache, "bf16")[0]
    V = O.widen(case.v_cache, "bf16")[0]
    reps, t = 0, 0.0
    while t < seconds:
        t0 = time.perf_counter()
        O.layer_forward(h, case.act_idx, Wl, K.copy(), V.copy(), od)
        t += time.perf_counter() - t0
        reps += 1
    fl = layer_flops(M) * reps
    return {"value": round(fl / t / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "float64 NumPy oracle layer step at the LLaDA-8B layer shape, N=1024, M=%d, %d reps in %.1f s "
                      "(BLAS %s, host %s, os.cpu_count %d)" % (M, reps, t, blas, platform.processor() or
                                                                   platform.machine(), os.cpu_count())}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline leg")
    ap.add_argument("--no-e2e", action="store_true", help="skip the 32-layer sampler loop")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched ragged step")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="only launch the roofline kernels and a calibration copy (for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.profile_kernels:
        profile_kernels()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SureLock path here is built and measured on a single MI355X "
              "(sequences are independent, so data parallelism needs no collective). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    res = gpu_part(args)
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "LLaDA-8B layer step (d=4096, 32x128 heads, SwiGLU 12288, N=1024, batch 1) at "
                               "M in {1024,512,256,64} + KL-lock pass (N=4096, V=126464, M=1639, eps=0.01, gate 0.5)",
                   "N": N_LAYER, "M": list(MS), "d": D, "heads": H, "head_dim": DH, "ffn": F,
                   "kl_N": N_KL, "kl_V": V_KL, "kl_M": res["kl_lock"]["M"]},
        "per_M": res["per_M"],
        "kl_lock": res["kl_lock"],
        "kernels_ms_M1024": res["kernels_ms_M1024"],
        "ablation_no_kv_cache_ms": res["ablation_no_kv_cache_ms"],
        "roofline": res["roofline"],
        "roofline_kl": res["roofline_kl"],
        "batched_step": None if args.no_batched else batched_step(),
        "e2e_loop": None if args.no_e2e else e2e_loop(runs=SURELOCK_RUNS + ABLATION_RUNS),
        "e2e_loop_b8": None if args.no_e2e else e2e_loop(runs=(SURELOCK_RUNS[0], SURELOCK_RUNS[2]), B=8),
        "cpu_baseline": None if args.no_cpu else cpu_part(args.cpu_seconds),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
