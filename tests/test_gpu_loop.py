"""The device-resident sampler loop: the active count stays on the GPU and every step after the
first is one replay of a captured HIP graph (token_locking_sparse_amd.CapturedLoop).

The loop must take exactly the decisions of the host-driven loop (which reads the count back
after every step): same tokens, lock masks, lock steps, active lists, posterior buffers and
counts, bit for bit.  The kernels of both loops are the same; only the grids differ (a capacity
instead of the exact count), and no reduction here depends on the grid.
"""
import numpy as np
import pytest
import torch

import oracle.surelock_oracle as O
import workloads as W
from tests import bf16_emulation as E
from tests.gpu_util import dev, say, tdtype

pytestmark = pytest.mark.gpu


def _model(sl, dm, N, seed_key=0):
    layers = [W.layer_weights(dm, l) for l in range(dm.n_layers)]
    emb, head = W.embed_weights(dm), W.lm_head_weights(dm)
    return sl.DeviceModel(dtype=tdtype(dm.dtype), n_layers=dm.n_layers, d=dm.d, n_heads=dm.n_heads,
                          head_dim=dm.head_dim, ffn=dm.ffn, vocab=dm.vocab, rms_eps=dm.rms_eps,
                          rope_theta=dm.rope_theta,
                          layers=[{k: dev(v, dm.dtype) for k, v in L.items()} for L in layers],
                          embed=dev(emb, dm.dtype), lm_head=dev(head, dm.dtype), rope_n=N)


def _state(sl, model, dm, B, N, tok0, cached_lse=False):
    return sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                          cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda(), cached_lse=cached_lse)


def _snapshot(st):
    torch.cuda.synchronize()
    M = int(st.act_off[st.B].item())
    return dict(tok=st.tok.cpu().numpy(), locked=st.locked.cpu().numpy(), lock_step=st.lock_step.cpu().numpy(),
                act_off=st.act_off.cpu().numpy(), act_idx=st.act_idx[:M].cpu().numpy(), M=M,
                l0=st.logits[0].cpu(), l1=st.logits[1].cpu())


LOOPS = [
    # dims, B, N, steps, eps, gate, unmask per step
    (W.TINY, 2, 64, 16, 0.05, -1.0, 3),
    (W.TINY, 2, 64, 16, 0.05, 0.5, 3),
    (W.Dims(n_layers=2, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16"), 3, 128, 12, 0.05, -1.0, 6),
]


@pytest.mark.parametrize("dm,B,N,T,eps,gate,k,cached", [c + (False,) for c in LOOPS] + [LOOPS[2] + (True,)])
def test_captured_loop_matches_host_loop(dm, B, N, T, eps, gate, k, cached):
    """cached: both loops keep the per-position LSE store (the previous posterior's LSE from the step
    that produced it), so the graphs also alternate between the two stores."""
    import token_locking_sparse_amd as sl
    say("captured loop", dm.d, dm.dtype, B, N, T, eps, gate, k, cached)
    model = _model(sl, dm, N)
    tok0 = W.prompt_tokens(dm, B, N, 16)
    # host-driven: every step reads the count back
    ref = _state(sl, model, dm, B, N, tok0, cached)
    ms_ref = []
    for t in range(T):
        ms_ref.append(ref.M_tot)
        ref.step(eps, gate, dm.mask_id, True, k)
    r = _snapshot(ref)
    # device-resident: the first step eager, then graph replays; a small bucket so that the
    # capacity shrinks (and new graphs are captured) as the loop goes on
    st = _state(sl, model, dm, B, N, tok0, cached)
    st.step(eps, gate, dm.mask_id, True, k)
    loop = sl.CapturedLoop(st, eps, gate, dm.mask_id, k, bucket=16)
    m_hist = torch.full((T,), -1, dtype=torch.int32, device="cuda")
    for t in range(1, T):
        loop.step(m_hist)
    M_end = loop.finish()
    g = _snapshot(st)
    ms = [ms_ref[0]] + m_hist[1:].cpu().tolist()
    say("counts host %s, device %s; graphs captured %d" % (ms_ref, ms, len(loop.graphs)))
    assert ms == ms_ref
    assert M_end == r["M"] and st.t == T
    for key in ("tok", "locked", "lock_step", "act_off", "act_idx"):
        np.testing.assert_array_equal(g[key], r[key], err_msg=key)
    assert torch.equal(g["l0"], r["l0"]) and torch.equal(g["l1"], r["l1"])
    if cached:
        assert torch.equal(st.lse_pos[0], ref.lse_pos[0]) and torch.equal(st.lse_pos[1], ref.lse_pos[1])
    assert int((g["lock_step"] > 0).sum()) > 0          # positions locked at steps the graphs ran
    assert len(loop.graphs) >= 2


def test_device_count_step_equals_host_count_step():
    """One layer step with the count left on the device (device_m) against the same step with the
    exact count, at the LLaDA-8B layer width, M = 40 of N = 1024 (split-K residual projections and
    key-split attention): with the exact count as the capacity the outputs are identical; with a
    capacity of 200 the launch plan changes but the rows computed do not."""
    import token_locking_sparse_amd as sl
    dm = W.Dims(n_layers=1, d=4096, n_heads=32, head_dim=128, ffn=12288, vocab=1024, dtype="bf16")
    N, M = 1024, 40
    say("device-count layer step", M)
    case = W.layer_case(dm, N, [M], key=77)
    Wl = W.layer_weights(dm, 0)
    model = sl.DeviceModel(dtype=torch.bfloat16, n_layers=1, d=dm.d, n_heads=dm.n_heads, head_dim=dm.head_dim,
                           ffn=dm.ffn, vocab=dm.vocab, rms_eps=dm.rms_eps, rope_theta=dm.rope_theta,
                           layers=[{k: dev(v, "bf16") for k, v in Wl.items()}], rope_n=N)
    locked = np.ones(N, np.uint8)
    locked[case.act_idx] = 0
    outs = []
    for device_m, cap in ((False, M), (True, M), (True, 200)):
        kc = dev(case.k_cache, "bf16").reshape(1, 1, N, dm.n_heads, dm.head_dim)
        vc = dev(case.v_cache, "bf16").reshape(1, 1, N, dm.n_heads, dm.head_dim)
        st = sl.DeviceState(model, 1, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, "bf16"),
                            k_cache=kc, v_cache=vc, with_h_out=True)
        assert st.M_tot == M
        st.M_tot = cap
        st.step(0.0, do_lock=False, device_m=device_m)
        torch.cuda.synchronize()
        outs.append((st.h_out[:M].clone(), kc.clone(), vc.clone(), st.h_out[M:cap].clone()))
    # same capacity: the same launches, bit-identical
    assert all(torch.equal(a, b) for a, b in zip(outs[0][:3], outs[1][:3]))
    # a larger capacity may change the launch plan (tiles, key and K splits) but not the rows computed:
    # rows past the live count are never written, and the QKV projection (no K split) gives
    # bit-identical fresh K/V rows.  Attention rounds its probabilities to bf16 against a running
    # maximum that depends on how the keys are split, so the hidden rows are another realisation of
    # the bf16 roundings: both steps are held to the bf16-storage emulation against the oracle.
    assert torch.all(outs[2][3] == 0)
    assert torch.equal(outs[0][1], outs[2][1]) and torch.equal(outs[0][2], outs[2][2])
    od = O.OracleDims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.vocab, dm.rms_eps, dm.rope_theta)
    W64 = {k: O.widen(v, "bf16") for k, v in Wl.items()}
    h = O.widen(case.h_in, "bf16")[case.act_idx]
    K64, V64 = O.widen(case.k_cache, "bf16")[0], O.widen(case.v_cache, "bf16")[0]
    ref = O.layer_forward(h, case.act_idx, W64, K64.copy(), V64.copy(), od)
    emu = E.err_stats(E.layer(h, case.act_idx, W64, K64.copy(), V64.copy(),
                              E.Dims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.rms_eps, dm.rope_theta)), ref)
    for name, o in (("exact count", outs[0]), ("capacity 200", outs[2])):
        g = E.check(o[0].cpu().numpy().astype(np.float64), ref, emu, "hidden rows, " + name)
        say("%s: hidden rows rel L2 %.3e (emulated %.3e)" % (name, g.rel_l2, emu.rel_l2))


# ------------------------------------------------------------------ cache layout
def _to_head_major(c):
    """[L][B][N][H][Dh] -> [L][B][H][N][Dh] (contiguous)."""
    return c.permute(0, 1, 3, 2, 4).contiguous()


@pytest.mark.parametrize("dm,N,Ms,no_kv", [
    (W.LLADA_LAYER, 1024, [1024], False),
    (W.LLADA_LAYER, 1024, [64], False),     # key-split attention and merge
    (W.LLADA_LAYER, 1024, [300], True),     # the no-KV-cache ablation's excluded keys
    (W.Dims(n_layers=1, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16"), 128, [128, 3, 77], False),
    (W.Dims(n_layers=1, d=128, n_heads=4, head_dim=32, ffn=384, vocab=512, dtype="f32"), 64, [20, 64], False),
])
def test_head_major_cache_matches_token_major(dm, N, Ms, no_kv):
    """The same layer step with the K/V cache head-major ([B][H][N][Dh]) and token-major
    ([B][N][H][Dh]): the kernels visit the same keys in the same order, only the addresses differ,
    so hidden rows and caches (transposed) are bit-identical."""
    import token_locking_sparse_amd as sl
    say("head-major cache", dm.d, dm.dtype, N, Ms, no_kv)
    case = W.layer_case(dm, N, Ms, key=N + sum(Ms) + 9)
    B, M = case.B, case.M_tot
    model = sl.DeviceModel(dtype=tdtype(dm.dtype), n_layers=1, d=dm.d, n_heads=dm.n_heads, head_dim=dm.head_dim,
                           ffn=dm.ffn, vocab=dm.vocab, rms_eps=dm.rms_eps, rope_theta=dm.rope_theta,
                           layers=[{k: dev(v, dm.dtype) for k, v in W.layer_weights(dm, 0).items()}], rope_n=N)
    locked = np.ones(B * N, np.uint8)
    for b in range(B):
        locked[b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]]] = 0
    out = []
    for hm in (False, True):
        kc = dev(case.k_cache, dm.dtype).reshape(1, B, N, dm.n_heads, dm.head_dim)
        vc = dev(case.v_cache, dm.dtype).reshape(1, B, N, dm.n_heads, dm.head_dim)
        if hm:
            kc, vc = _to_head_major(kc), _to_head_major(vc)
        st = sl.DeviceState(model, B, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, dm.dtype),
                            k_cache=kc, v_cache=vc, with_h_out=True, kv_head_major=hm)
        st.step(0.0, do_lock=False, no_kv_cache=no_kv)
        torch.cuda.synchronize()
        if hm:
            kc, vc = kc.permute(0, 1, 3, 2, 4), vc.permute(0, 1, 3, 2, 4)
        out.append((st.h_out[:M].clone(), kc.contiguous(), vc.contiguous()))
    assert all(torch.equal(a, b) for a, b in zip(out[0], out[1]))


def test_head_major_cache_loop_matches_token_major():
    """The tiny fp32 sampler loop (2 sequences, 16 steps) with both cache layouts: identical tokens,
    lock masks and posteriors at every step."""
    import token_locking_sparse_amd as sl
    dm, B, N = W.TINY, 2, 64
    model = _model(sl, dm, N)
    tok0 = W.prompt_tokens(dm, B, N, 16)
    sts = [sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                          cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda(), kv_head_major=hm)
           for hm in (False, True)]
    for t in range(16):
        say("head-major loop step", t)
        for st in sts:
            st.step(0.05, -1.0, dm.mask_id, True, 3)
        a, b = _snapshot(sts[0]), _snapshot(sts[1])
        for key in ("tok", "locked", "lock_step", "act_off", "act_idx"):
            np.testing.assert_array_equal(a[key], b[key], err_msg=key)
        assert torch.equal(a["l0"], b["l0"]) and torch.equal(a["l1"], b["l1"])
