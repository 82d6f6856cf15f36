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
# dense bf16 MFMA FLOPs per GHz of shader clock: 256 CUs x 4 matrix cores x 1024 FLOP per cycle
# (one v_mfma_f32_32x32x16_bf16, 32768 FLOP, every 32 cycles); 2.5 PFLOP/s is this at 2.4 GHz
MFMA_TFLOPS_PER_GHZ = 256 * 4096 * 1e9 / 1e12
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
             "sha256": "00b9cdb5bc034fbda4bc5f9d2755e0462b3222fae296ee047fbf9e7f2d4f46a4", "bytes": 427952890},
    "kl": {"files": ["token_locking_sparse_amd/csrc/kl_lock.hip"],
           "sha256": "b9af60198ebd6cc2e4792e38638b94e920b6336b8ab86b23673e02d410df6fab", "bytes": 832050488},
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

    # ---------------- KL-lock inputs: the two posterior buffers of the sampler loop (X1 = X0 plus a
    # small drift) and their per-position LSE stores.  Pass i reads X[i%2] as the current posterior
    # and X[(i+1)%2] as the previous one, whose LSE the pass before stored in L[(i+1)%2], and stores
    # its own in L[i%2]: the loop's steady state, in which each posterior's LSE is computed once, by
    # the pass that first sees it.  An untimed pass over X1 first stands for the step before.
    locked_np, act_idx_np, act_off_np = W.kl_lock_mask(N_KL, 1, 0.6, 0)
    M_kl = int(act_off_np[-1])
    x0 = torch.randn((N_KL, V_KL), generator=g, device=dev, dtype=torch.float32).mul_(2.0)
    rows = torch.randperm(N_KL, generator=g, device=dev)[: int(round(0.7 * N_KL))]
    toks = torch.randint(0, V_KL, (rows.numel(),), generator=g, device=dev)
    x0[rows, toks] += 8.0
    x1 = (x0 + 0.05 * torch.randn((N_KL, V_KL), generator=g, device=dev, dtype=torch.float32)).to(bf)
    kl_x = [x0.to(bf), x1]
    del x0
    torch.cuda.empty_cache()
    kl_lse = [torch.zeros(N_KL, device=dev) for _ in range(2)]
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

    def kl_call(i, cached=True):
        c, p = i % 2, (i + 1) % 2
        sl.sl_kl_lock(kl_x[c], kl_x[p], V_KL, kl_ai, kl_ao, 1, N_KL, M_kl, None, EPS_KL, GATE_KL, -1, True, kl_locked,
                      kl_out["kl"], kl_out["u"], kl_out["lse"], kl_am, kl_out["conf"], kl_thr, kl_nai, kl_nao, kl_ws,
                      lse_prev=kl_lse[p] if cached else None, lse_pos=kl_lse[c])

    # the step before the first timed one: the pass over X1 (no previous posterior) stores its LSE
    sl.sl_kl_lock(kl_x[1], None, V_KL, kl_ai, kl_ao, 1, N_KL, M_kl, None, 0.0, -1.0, -1, False, kl_locked.clone(),
                  kl_out["kl"], kl_out["u"], kl_out["lse"], kl_am, kl_out["conf"], kl_thr, kl_nai, kl_nao, kl_ws,
                  lse_pos=kl_lse[1])

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
    ms_M = {M: float(np.median([evs[i][M][0].elapsed_time(evs[i][M][1]) for i in range(args.warmup, n_it)])) for M in MS}
    ms_kl = float(np.median([evk[i][0].elapsed_time(evk[i][1]) for i in range(args.warmup, n_it)]))
    M_after = int(kl_nao[1].item())
    # the same pass recomputing the previous posterior's LSE from its logits (no store)
    ekr = []
    for i in range(args.warmup + args.steps):
        e0, e1 = ev(), ev()
        e0.record()
        kl_call(i, cached=False)
        e1.record()
        ekr.append((e0, e1))
    torch.cuda.synchronize()
    ms_kl_recompute = float(np.median([a.elapsed_time(b) for a, b in ekr[args.warmup:]]))

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
        ms_abl[M] = float(np.median([a.elapsed_time(b) for a, b in es[args.warmup:]]))

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
    ms_gu = float(np.median([a.elapsed_time(b) for a, b in kg[args.warmup:]]))

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
        br[name] = float(np.median([a.elapsed_time(b) for a, b in es[args.warmup:]]))
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
                    "M_after": M_after, "frac_hbm_peak": round(kb / (ms_kl * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "previous_lse": "from the store of the pass that produced the previous posterior",
                    "ms_recomputing_previous_lse": round(ms_kl_recompute, 4)},
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


def e2e_loop(runs=SURELOCK_RUNS, steps=128, N=512, n_prompt=128, unmask=3, B=1, captured=False):
    """The whole sampler loop on a 32-layer LLaDA-8B-shaped model with random-init weights (d=4096,
    32 heads x 128, SwiGLU 12288, vocab 126464, bf16), B sequences of N=512 = 128 seeded prompt ids +
    384 [MASK]; 128 steps, 3 unmasks per sequence per step by confidence.  Each run is (name, eps,
    gate quantile or -1 for off, no-KV-cache ablation); eps = 0 is the dense reference (nothing
    locks).  Reports per-step time against the active count M_t (summed over the batch).
    captured: the device-resident loop (the first step eager, then one HIP graph replay per step,
    the active count never read back inside the loop) instead of the host-driven one."""
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
                            cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).to(dev), cached_lse=True)
        Ms, ms = [], []
        loop, n_graphs = None, 0
        if captured:
            # the graphs of every capacity (multiples of 64 up to B*N) and both step parities are
            # captured before the timed loop: capture is host work paid once per shape
            loop = sl.CapturedLoop(st, eps, gate, dm.mask_id, unmask, no_kv, bucket=max(64, 16 * B))
            loop.precapture()
            m_hist = torch.full((steps,), -1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if not captured:
                Ms.append(st.M_tot)
            e0.record()
            if captured and t > 0:
                loop.step(m_hist)
            else:
                if captured:
                    m_hist[0:1].copy_(st.act_off[B:B + 1])
                st.step(eps, gate, dm.mask_id, True, unmask, no_kv_cache=no_kv)
                if captured:
                    loop.known_m = st.M_tot
            e1.record()
            ms.append((e0, e1))
        if captured:
            loop.finish()
            n_graphs = len(loop.graphs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if captured:
            Ms = m_hist.cpu().tolist()
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
        if captured:
            out[name]["graphs_captured"] = n_graphs
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


def cache_layout_study(steps=50, warmup=10, Ms=(1024, 256, 64)):
    """The K/V cache laid out token-major ([B][N][H][Dh], a position's K row is one 8 KB run: the
    scatter writes whole rows, attention reads 256-byte slices 8 KB apart) against head-major
    ([B][H][N][Dh], a head's keys are one contiguous run: attention streams it, the scatter writes
    256-byte slices).  Only the fused QKV scatter and attention see the layout, so the layer step's
    time difference is theirs.  LLaDA-8B layer shape, N = 1024, weights rotated over 3 copies;
    medians of `steps` steps."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import token_locking_sparse_amd.surelock as S
    import workloads as W

    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    bf = torch.bfloat16

    def randn(shape, std=1.0):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

    shapes = {"wq": (D, D), "wk": (D, D), "wv": (D, D), "wo": (D, D), "wg": (F, D), "wu": (F, D), "wd": (D, F)}
    wsets = [{k: randn(sh, 0.02) for k, sh in shapes.items()} for _ in range(3)]
    models = [sl.DeviceModel(dtype=bf, n_layers=1, d=D, n_heads=H, head_dim=DH, ffn=F, vocab=126464, rms_eps=1e-5,
                             rope_theta=1e4, layers=[w], rope_n=N_LAYER) for w in wsets]
    h_in = randn((N_LAYER, D))
    kc_t = randn((1, 1, N_LAYER, H, DH))
    vc_t = randn((1, 1, N_LAYER, H, DH))
    caches = {False: (kc_t, vc_t),
              True: (kc_t.permute(0, 1, 3, 2, 4).contiguous(), vc_t.permute(0, 1, 3, 2, 4).contiguous())}
    p = S.sl_step_params(0.0, -1.0, -1, 0, 0)
    out = {}
    for M in Ms:
        act = W.choose_active(N_LAYER, M, W.SEED_SETS, M)
        locked = torch.from_numpy(W.locked_from_active(N_LAYER, act)).to(dev)
        row = {}
        for hm in (False, True):
            kc, vc = caches[hm]
            st = sl.DeviceState(models[0], 1, N_LAYER, locked=locked, h_in=h_in, k_cache=kc, v_cache=vc,
                                with_h_out=True, kv_head_major=hm)
            sst = st.struct()
            es = []
            for i in range(warmup + steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                S.sl_step(models[i % 3].s, sst, p, st.ws)
                e1.record()
                es.append((e0, e1))
            torch.cuda.synchronize()
            row["head_major" if hm else "token_major"] = round(float(np.median([a.elapsed_time(b) for a, b in es[warmup:]])), 4)
            del st
        out[str(M)] = row
    del wsets, models, caches, kc_t, vc_t
    torch.cuda.empty_cache()
    return {"layer_step_ms": out, "config": "LLaDA-8B layer, N=1024, M in %s; medians of %d steps" % (list(Ms), steps)}


def measured_peaks(reps=7):
    """What this chip sustains: a register-only bf16 MFMA loop on every CU, and 16-byte non-temporal
    streaming of 1 GiB (read only, and copy).  Medians of `reps` launches timed with HIP events."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl

    dev = "cuda"
    sink = torch.zeros(256, device=dev)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def timed(fn):
        fn()
        es = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    wg, iters = 2048, 2048
    flops = sl.sl_peak_mfma(wg, iters, sink)
    ms_mfma = timed(lambda: sl.sl_peak_mfma(wg, iters, sink))
    ms_read = timed(lambda: sl.sl_peak_stream(src, None, 2048, sink))
    ms_copy = timed(lambda: sl.sl_peak_stream(src, dst, 2048, sink))
    # the 256 x 256 GEMM tile's LDS-to-MFMA loop alone, one workgroup per CU, then with the k-tile
    # loop's direct loads (from an L2-resident 1 MiB), waits and barrier
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = 2048
    l2src = torch.zeros(1 << 20, dtype=torch.uint8, device=dev)
    fl_loop = sl.sl_peak_gemm_loop(cus, tiles, False, l2src, sink)
    ms_loop = timed(lambda: sl.sl_peak_gemm_loop(cus, tiles, False, l2src, sink))
    ms_loop_ld = timed(lambda: sl.sl_peak_gemm_loop(cus, tiles, True, l2src, sink))
    nb = src.numel()
    # the same MFMA loop on operands read from memory (eight sets per lane, rotated): random bf16 values,
    # as the step's weights and activations are, then all ones and all zeros.  The matrix cores' power
    # depends on the operand bits, and the clock the chip holds with it; each launch also reports its
    # workgroups' shader-clock cycles against 100 MHz real-time ticks.
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    n_ops = 16 * 256 * 8
    operand_sets = {"random": torch.randn(n_ops, generator=gen, device=dev).to(torch.bfloat16),
                    "ones": torch.ones(n_ops, device=dev, dtype=torch.bfloat16),
                    "zeros": torch.zeros(n_ops, device=dev, dtype=torch.bfloat16)}
    clocks = torch.zeros(2 * wg, dtype=torch.int64, device=dev)
    by_operands = {}
    for name, ops in operand_sets.items():
        ms_op = timed(lambda: sl.sl_peak_mfma_operands(wg, iters, ops, sink))
        clocks.zero_()
        sl.sl_peak_mfma_operands(wg, iters, ops, sink, clocks)
        torch.cuda.synchronize()
        c = clocks.view(wg, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(c[:, 0] / c[:, 1] / 10.0))
        tf = flops / (ms_op * 1e-3) / 1e12
        by_operands[name] = {"tflops": round(tf, 1), "ghz": round(ghz, 3),
                             "frac_at_clock": round(tf / (MFMA_TFLOPS_PER_GHZ * ghz), 3)}
    out = {"mfma_bf16_tflops": round(flops / (ms_mfma * 1e-3) / 1e12, 1),
           "mfma_bf16_by_operands": by_operands,
           "hbm_read_gbs": round(nb / (ms_read * 1e-3) / 1e9, 1),
           "hbm_copy_gbs": round(2 * nb / (ms_copy * 1e-3) / 1e9, 1),
           "gemm_loop_tflops": round(fl_loop / (ms_loop * 1e-3) / 1e12, 1),
           "gemm_loop_with_l2_loads_tflops": round(fl_loop / (ms_loop_ld * 1e-3) / 1e12, 1),
           "how": "register-only v_mfma_f32_32x32x16_bf16 loop, %d workgroups x 4 waves x %d x 4 MFMAs; "
                  "1 GiB streamed with 16-byte non-temporal loads (read) and loads + stores (copy, bytes "
                  "read + written), each workgroup on a contiguous range; the 256 x 256 GEMM tile's "
                  "LDS-to-MFMA loop on %d workgroups x %d k-tiles of 32, alone and with its direct loads "
                  "from L2, waits and barrier; medians of %d launches; mfma_bf16_by_operands: the MFMA loop "
                  "on operands from memory (random N(0,1) bf16, ones, zeros), clock = median over workgroups "
                  "of s_memtime cycles / s_memrealtime ticks, frac_at_clock = TFLOP/s over 256 CUs x 4096 "
                  "FLOP per cycle at that clock" % (wg, iters, cus, tiles, reps)}
    del src, dst, l2src, operand_sets, clocks
    torch.cuda.empty_cache()
    return out


def gemm_clock_study(reps=20, warmup=5):
    """The dominant kernel (FFN gate/up + SwiGLU at M = 1024) on random operands, as in the step, and on
    all-zero operands: its rate (product kernel, HIP events), then one launch of its clock-recording
    variant, which gives the clock the chip held (shader-clock cycles over 100 MHz ticks, median over
    workgroups) and the k-tile loop's MFMA utilisation at that clock (the workgroup's FLOPs over the
    loop's cycles x 4096 FLOP per CU-cycle)."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl

    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    M, K, n_out = 1024, D, 2 * F
    bm, bn, split = sl.sl_gemm_plan(bf, sl.SL_EPI_SWIGLU, M, K, n_out)
    nwg = -(-M // bm) * (n_out // bn) * split
    clocks = torch.zeros(4 * nwg, dtype=torch.int64, device=dev)
    out = torch.empty(M, F, dtype=bf, device=dev)
    res = {"tile": [bm, bn], "split_k": split, "workgroups": nwg}
    for name in ("random", "zeros"):
        if name == "random":
            A = torch.randn(M, K, generator=g, device=dev).to(bf)
            wg_ = (torch.randn(F, K, generator=g, device=dev) * 0.02).to(bf)
            wu_ = (torch.randn(F, K, generator=g, device=dev) * 0.02).to(bf)
        else:
            A = torch.zeros(M, K, device=dev, dtype=bf)
            wg_ = torch.zeros(F, K, device=dev, dtype=bf)
            wu_ = torch.zeros(F, K, device=dev, dtype=bf)
        call = lambda: sl.sl_gemm(sl.SL_EPI_SWIGLU, A, M, K, n_out, wg_, wu_, out0=out)
        for _ in range(warmup):
            call()
        es = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in es]))
        clocks.zero_()
        sl.sl_gemm_clocked(sl.SL_EPI_SWIGLU, A, M, K, n_out, wg_, wu_, out0=out, clocks=clocks)
        torch.cuda.synchronize()
        c = clocks.view(nwg, 4).cpu().numpy().astype(np.float64)
        c = c[c[:, 1] > 0]
        ghz = float(np.median(c[:, 0] / c[:, 1] / 10.0))
        util = float(np.median(bm * bn * c[:, 3] * 2.0 / 4096.0 / c[:, 2]))
        tf = 2.0 * M * K * n_out / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "ghz": round(ghz, 3),
                     "frac_at_clock": round(tf / (MFMA_TFLOPS_PER_GHZ * ghz), 3),
                     "kloop_mfma_util_at_clock": round(util, 3)}
        del A, wg_, wu_
    del clocks, out
    torch.cuda.empty_cache()
    return res


def gemm_study(reps=20, warmup=5):
    """The library's GEMM (with its epilogue) against torch.matmul (the vendor library, plain
    bf16 output) on the step's shapes and two large ones, weights resident; TFLOP/s of each."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl

    dev, bf = "cuda", torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(3)

    def timed(fn):
        for _ in range(warmup):
            fn()
        es = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            es.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in es]))

    rows = []
    for M, K, Nn, epi in [(1024, 4096, 24576, "swiglu"), (1024, 4096, 12288, "residual"),
                          (1024, 12288, 4096, "residual"), (4873, 4096, 126464, "logits"),
                          (8192, 8192, 8192, "logits")]:
        A = (torch.randn(M, K, generator=g, device=dev) * 0.5).to(bf)
        Wt = (torch.randn(Nn, K, generator=g, device=dev) * 0.02).to(bf)
        if epi == "swiglu":
            w0, w1 = Wt[: Nn // 2].contiguous(), Wt[Nn // 2:].contiguous()
            out = torch.empty(M, Nn // 2, dtype=bf, device=dev)
            fn = lambda: sl.sl_gemm(sl.SL_EPI_SWIGLU, A, M, K, Nn, w0, w1, out0=out)
        elif epi == "residual":
            out = torch.zeros(M, Nn, dtype=torch.float32, device=dev)
            fn = lambda: sl.sl_gemm(sl.SL_EPI_RESIDUAL, A, M, K, Nn, Wt, out0=out)
        else:
            out = torch.empty(M, Nn, dtype=bf, device=dev)
            ai = torch.arange(M, dtype=torch.int32, device=dev)
            ao = torch.tensor([0, M], dtype=torch.int32, device=dev)
            fn = lambda: sl.sl_gemm(sl.SL_EPI_LOGITS, A, M, K, Nn, Wt, out0=out, act_idx=ai, act_off=ao, B=1, N=M)
        fl = 2.0 * M * K * Nn
        ms = timed(fn)
        ms_t = timed(lambda: torch.matmul(A, Wt.t()))
        rows.append({"M": M, "K": K, "N": Nn, "epilogue": epi, "tile": list(sl.sl_gemm_plan(bf, {"swiglu": 2, "residual": 1, "logits": 3}[epi], M, K, Nn)),
                     "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                     "torch_matmul_ms": round(ms_t, 4), "torch_matmul_tflops": round(fl / ms_t / 1e9, 1)})
        del A, Wt, out
        torch.cuda.empty_cache()
    return rows


def tiny_loop(steps=16, B=1, N=64, n_prompt=16, unmask=3, eps=0.05, reps=5):
    """The tiny fp32 sampler loop (2 layers, d=128, 4 heads x 32, SwiGLU 384, vocab 512, N=64 = 16
    prompt ids + 48 [MASK], 16 steps, 3 unmasks per step, eps 0.05, gate off): ms per step (median
    over `reps` loops) and the active count M_t per step, host-driven and device-resident."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import workloads as W

    dm = W.TINY
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    layers = [W.layer_weights(dm, l) for l in range(dm.n_layers)]
    model = sl.DeviceModel(dtype=torch.float32, n_layers=dm.n_layers, d=dm.d, n_heads=dm.n_heads,
                           head_dim=dm.head_dim, ffn=dm.ffn, vocab=dm.vocab, rms_eps=dm.rms_eps,
                           rope_theta=dm.rope_theta, layers=[{k: to_dev(v) for k, v in L.items()} for L in layers],
                           embed=to_dev(W.embed_weights(dm)), lm_head=to_dev(W.lm_head_weights(dm)), rope_n=N)
    tok0 = W.prompt_tokens(dm, B, N, n_prompt)
    res = {}
    for mode in ("host", "captured"):
        walls, Ms = [], None
        for r in range(reps + 1):
            st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                                cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda())
            loop = None
            if mode == "captured":
                loop = sl.CapturedLoop(st, eps, -1.0, dm.mask_id, unmask, bucket=16)
                loop.precapture()
                m_hist = torch.full((steps,), -1, dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if mode == "host":
                ms_t = [st.M_tot]
                for t in range(steps):
                    st.step(eps, -1.0, dm.mask_id, True, unmask)
                    ms_t.append(st.M_tot)
                ms_t = ms_t[:steps]
            else:
                m_hist[0:1].copy_(st.act_off[B:B + 1])
                st.step(eps, -1.0, dm.mask_id, True, unmask)
                loop.known_m = st.M_tot
                for t in range(1, steps):
                    loop.step(m_hist)
                loop.finish()
            torch.cuda.synchronize()
            if r > 0:                               # the first loop warms up
                walls.append(time.perf_counter() - t0)
            Ms = ms_t if mode == "host" else m_hist.cpu().tolist()
        res[mode] = {"ms_per_step": round(float(np.median(walls)) * 1e3 / steps, 4), "M_t": Ms}
    res["config"] = "tiny fp32 model (2 layers, d=128, 4x32 heads, FFN 384, V=512), B=%d, N=%d (%d prompt + %d [MASK]), " \
                    "%d steps, %d unmasks per step, eps=%g, gate off" % (B, N, n_prompt, N - n_prompt, steps, unmask, eps)
    return res


def batched_step(steps=50, warmup=10, B=8, N=2048, eps=0.05, gate=0.5):
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
                        cand=torch.ones(B * N, dtype=torch.uint8, device=dev), cached_lse=True)
    st_l = sl.DeviceState(model_l, B, N, locked=locked0.clone(), h_in=h_in, k_cache=kc, v_cache=vc)
    st_hm = sl.DeviceState(model_l, B, N, locked=locked0.clone(), h_in=h_in, kv_head_major=True,
                           k_cache=kc.permute(0, 1, 3, 2, 4).contiguous(), v_cache=vc.permute(0, 1, 3, 2, 4).contiguous())
    assert st.M_tot == M_tot and st_l.M_tot == M_tot and st_hm.M_tot == M_tot
    ai0, ao0 = st.act_idx.clone(), st.act_off.clone()
    kl_o = {k: torch.empty(M_tot, device=dev) for k in ("kl", "u", "lse", "conf")}
    kl_am = torch.empty(M_tot, dtype=torch.int32, device=dev)
    kl_thr = torch.empty(B, device=dev)
    kl_nai = torch.empty(B * N, dtype=torch.int32, device=dev)
    kl_nao = torch.empty(B + 1, dtype=torch.int32, device=dev)
    kl_lk = locked0.clone()
    kl_ws = torch.empty(sl.sl_kl_lock_workspace_size(B, N, M_tot, V), dtype=torch.uint8, device=dev)
    kl_lse = torch.empty(B * N, device=dev)
    # previous posterior: this step's logits (t = 0, eps = 0: nothing locks) plus drift, in buffer 0,
    # and its LSE in the store beside it, as the pass of the step that produced it leaves it
    st.step(0.0)
    for r0 in range(0, B * N, 1024):
        blk = st.logits[0][r0:r0 + 1024]
        blk.copy_((blk.float() + 0.05 * torch.randn(blk.shape, generator=g, device=dev)).to(bf))
    sl.sl_kl_lock(st.logits[0], None, V, ai0, ao0, B, N, M_tot, None, 0.0, -1.0, -1, False, kl_lk.clone(),
                  kl_o["kl"], kl_o["u"], kl_o["lse"], kl_am, kl_o["conf"], kl_thr, kl_nai, kl_nao, kl_ws,
                  lse_pos=st.lse_pos[0])
    st.t = 1
    sst = st.struct()
    sst.m_tot_host = None                     # no host copy of M: nothing to wait for inside the timing
    sst_c = st.struct()                       # takes the previous posterior's LSE from the store
    sst_c.m_tot_host = None
    sst.lse_pos[0] = sst.lse_pos[1] = None    # recomputes it from the previous logits
    p_full = S.sl_step_params(eps, gate, -1, 1, 0)
    p_fused = S.sl_step_params(eps, gate, -1, 1, 0, 0, 0, 1)   # LM head computes the vocabulary statistics
    sst_l = st_l.struct()
    sst_hm = st_hm.struct()
    p_layer = S.sl_step_params(0.0, -1.0, -1, 0, 0)
    x = randn((M_tot, D), 1.0)

    def restore():
        st.locked.copy_(locked0)
        st.act_idx.copy_(ai0)
        st.act_off.copy_(ao0)
        kl_lk.copy_(locked0)

    calls = {
        "step": lambda: S.sl_step(model.s, sst, p_full, st.ws),
        "step_cached_lse": lambda: S.sl_step(model.s, sst_c, p_full, st.ws),
        "step_fused": lambda: S.sl_step(model.s, sst, p_fused, st.ws),
        "layer": lambda: S.sl_step(model_l.s, sst_l, p_layer, st_l.ws),
        "layer_head_major": lambda: S.sl_step(model_l.s, sst_hm, p_layer, st_hm.ws),
        "lm_head": lambda: sl.sl_gemm(sl.SL_EPI_LOGITS, x, M_tot, D, V, head, out0=st.logits[1], act_idx=ai0,
                                      act_off=ao0, B=B, N=N),
        "kl_lock": lambda: sl.sl_kl_lock(st.logits[1], st.logits[0], V, ai0, ao0, B, N, M_tot, None, eps, gate, -1,
                                         True, kl_lk, kl_o["kl"], kl_o["u"], kl_o["lse"], kl_am, kl_o["conf"],
                                         kl_thr, kl_nai, kl_nao, kl_ws),
        "kl_lock_cached_lse": lambda: sl.sl_kl_lock(st.logits[1], st.logits[0], V, ai0, ao0, B, N, M_tot, None, eps,
                                                    gate, -1, True, kl_lk, kl_o["kl"], kl_o["u"], kl_o["lse"], kl_am,
                                                    kl_o["conf"], kl_thr, kl_nai, kl_nao, kl_ws,
                                                    lse_prev=st.lse_pos[0], lse_pos=kl_lse),
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
        ms[name] = float(np.median([a.elapsed_time(b) for a, b in es[warmup:]]))
    restore()
    calls["step"]()
    torch.cuda.synchronize()
    M_after = int(st.act_off[B].item())
    fl_layer = layer_flops(M_tot, N=N)
    fl_head = 2.0 * M_tot * D * V
    kb = kl_bytes(M_tot, N=B * N, V=V)
    head_plan = sl.sl_gemm_plan(bf, sl.SL_EPI_LOGITS, M_tot, D, V)
    out = {"B": B, "N": N, "M_b": Ms, "M_tot": M_tot, "M_after": M_after, "eps": eps, "gate": gate,
           "ms_step": round(ms["step"], 4), "ms_step_fused_head_kl": round(ms["step_fused"], 4),
           "ms_layer": round(ms["layer"], 4), "ms_layer_head_major_cache": round(ms["layer_head_major"], 4),
           "ms_lm_head": round(ms["lm_head"], 4),
           "ms_kl_lock": round(ms["kl_lock"], 4),
           "ms_step_cached_lse": round(ms["step_cached_lse"], 4),
           "ms_kl_lock_cached_lse": round(ms["kl_lock_cached_lse"], 4),
           "step_tflops": round((fl_layer + fl_head) / (ms["step"] * 1e-3) / 1e12, 2),
           "layer_tflops": round(fl_layer / (ms["layer"] * 1e-3) / 1e12, 2),
           "lm_head": {"kernel": "gemm_kernel<bf16,%dx%d,split %d,EPI_LOGITS>" % head_plan, "bound": "mfma",
                       "tflops": round(fl_head / (ms["lm_head"] * 1e-3) / 1e12, 2),
                       "frac_mfma_peak": round(fl_head / (ms["lm_head"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
           "kl": {"bound": "hbm", "bytes": kb, "gbs": round(kb / (ms["kl_lock"] * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(kb / (ms["kl_lock"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del st, st_l, st_hm, model, model_l, layer, head, h_in, kc, vc, x
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
    # the previous posterior's LSE, as the pass that produced it stores it (the configuration bench.py times)
    lse_p, lse_c = torch.zeros(N_KL, device=dev), torch.zeros(N_KL, device=dev)
    sl.sl_kl_lock(prev, None, V_KL, ai, ao, 1, N_KL, M_kl, None, 0.0, -1.0, -1, False, locked.clone(), o["kl"],
                  o["u"], o["lse"], am, o["conf"], thr, nai, nao, ws, lse_pos=lse_p)
    for _ in range(3):
        sl.sl_gemm(sl.SL_EPI_SWIGLU, x, Mg, D, 2 * F, wg, wu, out0=act)
        sl.sl_kl_lock(cur, prev, V_KL, ai, ao, 1, N_KL, M_kl, None, EPS_KL, GATE_KL, -1, True, locked, o["kl"],
                      o["u"], o["lse"], am, o["conf"], thr, nai, nao, ws, lse_prev=lse_p, lse_pos=lse_c)
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profiled: gate/up GEMM M=%d plan %s, KL-lock pass M=%d, copy of %d bytes" %
          (Mg, sl.sl_gemm_plan(bf, sl.SL_EPI_SWIGLU, Mg, D, 2 * F), M_kl, src.numel()), flush=True)


def profile_attention():
    """Launch only the active-query attention at the LLaDA-8B layer shape (32 heads x 128, N=1024),
    M = 1024 and M = 256 (bf16, each 3 times), for rocprofv3 --pmc counter runs."""
    import numpy as np
    import torch

    import token_locking_sparse_amd as sl
    import workloads as W

    dev = "cuda"
    torch.cuda.set_device(0)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16
    kc = torch.randn((1, N_LAYER, H, DH), generator=g, device=dev).to(bf)
    vc = torch.randn((1, N_LAYER, H, DH), generator=g, device=dev).to(bf)
    for M in (1024, 256):
        q = torch.randn((M, H, DH), generator=g, device=dev).to(bf)
        out = torch.empty(M, H * DH, dtype=bf, device=dev)
        off = torch.tensor([0, M], dtype=torch.int32, device=dev)
        ws = torch.empty(max(1, sl.sl_attn_workspace_size(1, N_LAYER, M, H, DH)), dtype=torch.uint8, device=dev)
        for _ in range(3):
            sl.sl_attn_active(q, kc, vc, off, 1, N_LAYER, M, H, DH, 1.0 / math.sqrt(DH), out, ws)
    torch.cuda.synchronize()
    print("profiled: attention at M = 1024 and 256, N = %d, %d heads x %d" % (N_LAYER, H, DH), flush=True)


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


def _host_info():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
    except Exception:  # pragma: no cover
        cores, blas = os.cpu_count(), "?"
    return int(cores), blas


def cpu_configs():
    """The oracle as it stands on bounded samples of the other workloads, on the host cores; each
    figure is scaled from its sample to the whole workload by rows (the oracle's cost is linear in
    the active rows)."""
    import numpy as np

    import oracle.surelock_oracle as O
    import workloads as W
    cores, blas = _host_info()
    out = {"cores": cores, "blas": blas, "host": platform.processor() or platform.machine(),
           "os_cpu_count": os.cpu_count()}
    # KL-lock pass: posterior statistics and lock update of 256 active rows at V = 126464
    case = W.kl_lock_case(N=640, V=V_KL, B=1, locked_frac=0.6, key=640)
    z, y = O.widen(case.cur, "bf16"), O.widen(case.prev, "bf16")
    t0 = time.perf_counter()
    st = O.posterior_stats(z, y)
    O.lock_update(case.locked, case.act_idx, case.act_off, 1, case.N, st.kl, st.u, None, EPS_KL, GATE_KL, True)
    t = (time.perf_counter() - t0) * 1639 / case.M_tot
    out["kl_lock_pass"] = {"value": round(kl_bytes(1639) / t / 1e9, 3), "unit": "GB/s", "ms": round(t * 1e3, 1),
                           "sample": "float64 posterior statistics + lock update of %d rows x V=%d (scaled to "
                                     "M=1639)" % (case.M_tot, V_KL)}
    del z, y, case
    # batched ragged step: one layer + final norm + LM head + statistics of the smallest sequence
    dm = W.LLADA_LAYER
    Ms = W.ragged_ms(8, 2048, key=8 * 2048)
    b = int(np.argmin(Ms))
    od = O.OracleDims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.vocab, dm.rms_eps, dm.rope_theta)
    Wl = {k: O.widen(v, "bf16") for k, v in W.layer_weights(dm, 0).items()}
    head = O.widen(W.lm_head_weights(dm), "bf16")
    lc = W.layer_case(dm, 2048, [Ms[b]], key=5)
    h = O.widen(lc.h_in, "bf16")[lc.act_idx]
    K, V = O.widen(lc.k_cache, "bf16")[0], O.widen(lc.v_cache, "bf16")[0]
    t0 = time.perf_counter()
    hh = O.layer_forward(h, lc.act_idx, Wl, K, V, od)
    zz = O.rmsnorm(hh, dm.rms_eps) @ head.T
    O.posterior_stats(zz, zz)
    t = (time.perf_counter() - t0) * sum(Ms) / Ms[b]
    fl = layer_flops(sum(Ms), N=2048) + 2.0 * sum(Ms) * D * V_KL
    out["batched_step"] = {"value": round(fl / t / 1e12, 4), "unit": "TFLOP/s", "ms": round(t * 1e3, 1),
                           "sample": "float64 layer + LM head + statistics of one sequence (M_b=%d of 2048), scaled "
                                     "to the 8-sequence step (sum M_b=%d)" % (Ms[b], sum(Ms))}
    del Wl, head, hh, zz
    # tiny sampler loop, whole
    tdm = W.TINY
    tod = O.OracleDims(tdm.d, tdm.n_heads, tdm.head_dim, tdm.ffn, tdm.vocab, tdm.rms_eps, tdm.rope_theta)
    L64 = [{k: O.widen(v, "f32") for k, v in W.layer_weights(tdm, l).items()} for l in range(tdm.n_layers)]
    om = O.OracleModel(tod, tdm.n_layers, lambda l: L64[l], O.widen(W.embed_weights(tdm), "f32"),
                       O.widen(W.lm_head_weights(tdm), "f32"))
    tok0 = W.prompt_tokens(tdm, 1, 64, 16)
    t0 = time.perf_counter()
    recs = O.run_loop(om, tok0, 1, 64, 16, 0.05, -1.0, 3)
    t = time.perf_counter() - t0
    out["tiny_loop"] = {"value": round(t * 1e3 / 16, 3), "unit": "ms/step", "M_t": [r.M for r in recs],
                        "sample": "the whole 16-step loop of the tiny model in float64 (the oracle evaluates in "
                                  "float64 only)"}
    return out


def leg(name, fn):
    """Run one leg of the bench and note its end on stderr (the JSON line stays alone on stdout)."""
    import time
    t0 = time.time()
    r = fn()
    print("bench: %s done in %.1f s" % (name, time.time() - t0), file=sys.stderr, flush=True)
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline leg")
    ap.add_argument("--no-e2e", action="store_true", help="skip the 32-layer sampler loop")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched ragged step")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="only launch the roofline kernels and a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--profile-attention", action="store_true",
                    help="only launch the attention at M = 1024 and 256 (for rocprofv3 --pmc)")
    ap.add_argument("--gemm-study", action="store_true",
                    help="only time the library's GEMM against torch.matmul on the step's shapes and two "
                         "large ones (one JSON line)")
    ap.add_argument("--clock-study", action="store_true",
                    help="only measure the MFMA loop on random / constant operands and the dominant GEMM's "
                         "clock and k-loop MFMA utilisation (one JSON line)")
    args = ap.parse_args()
    if args.clock_study:
        print(json.dumps({"measured_peaks": measured_peaks(), "gemm_clock": gemm_clock_study()}), flush=True)
        return
    if args.gemm_study:
        print(json.dumps({"gemm_study": gemm_study()}), flush=True)
        return
    if args.profile_kernels:
        profile_kernels()
        return
    if args.profile_attention:
        profile_attention()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SureLock path here is built and measured on a single MI355X "
              "(sequences are independent, so data parallelism needs no collective). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    res = leg("layer sweep and KL-lock pass", lambda: gpu_part(args))
    peaks = leg("measured peaks", measured_peaks)
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
        "measured_peaks": peaks,
        "gemm_clock": leg("GEMM clock", gemm_clock_study),
        "cache_layout": leg("cache layout", cache_layout_study),
        "batched_step": None if args.no_batched else leg("batched step", batched_step),
        "tiny_loop": leg("tiny loop", tiny_loop),
        "e2e_loop": None if args.no_e2e else leg("sampler loop", lambda: e2e_loop(runs=SURELOCK_RUNS + ABLATION_RUNS)),
        "e2e_loop_b8": None if args.no_e2e else leg("sampler loop B=8", lambda: e2e_loop(runs=(SURELOCK_RUNS[0], SURELOCK_RUNS[2]), B=8)),
        "e2e_loop_captured": None if args.no_e2e else leg("captured loop", lambda: e2e_loop(runs=(SURELOCK_RUNS[2],), captured=True)),
        "e2e_loop_b8_captured": None if args.no_e2e else leg("captured loop B=8", lambda: e2e_loop(runs=(SURELOCK_RUNS[2],), B=8, captured=True)),
        "cpu_baseline": None,
    }
    # fractions of the measured ceilings, beside the vendor ones
    line["roofline"]["frac_of_measured_peak"] = round(line["roofline"]["achieved"] / peaks["mfma_bf16_tflops"], 4)
    line["roofline"]["measured_peak"] = peaks["mfma_bf16_tflops"]
    rnd = peaks["mfma_bf16_by_operands"]["random"]["tflops"]
    line["roofline"]["frac_of_random_operand_mfma_peak"] = round(line["roofline"]["achieved"] / rnd, 4)
    line["roofline"]["random_operand_mfma_peak"] = rnd
    line["roofline_kl"]["frac_of_measured_peak"] = round(line["roofline_kl"]["achieved"] / peaks["hbm_read_gbs"], 4)
    line["roofline_kl"]["measured_peak"] = peaks["hbm_read_gbs"]
    for r in line["per_M"]:
        r["frac_measured_mfma_peak"] = round(r["tflops"] / peaks["mfma_bf16_tflops"], 4)
    if not args.no_cpu:
        cb = leg("oracle baseline", lambda: cpu_part(args.cpu_seconds))
        cb["per_config"] = leg("oracle per configuration", cpu_configs)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
