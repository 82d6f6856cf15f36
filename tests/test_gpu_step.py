"""GPU parity of sl_step (whole SureLock iterations) against the CPU oracle.

Hidden rows and K/V (bf16 storage): relative L2 <= 1e-2 and no element beyond
max(7 rms(d), 2e-2 max(1,|ref|)) -- the bf16 rounding of intermediates gives a
near-Gaussian error whose maximum over millions of elements exceeds a fixed
2e-2 at full width; fp32 storage is held to 1e-4.  Logits: max-abs 2e-2.  KL: 1e-3
absolute.  Lock masks and active lists: bit-exact except near-threshold
positions (|KL-eps| <= 1e-3, or |u - q| <= 1e-5 when the gate is on).
Locked positions' cache rows and posterior rows: bitwise unchanged.
Multi-step loops are checked teacher-forced: every GPU step starts from the
oracle's state (rounded to the storage type).
"""
import math

import numpy as np
import pytest
import torch

import oracle.surelock_oracle as O
import workloads as W
from tests.gpu_util import check_hidden, check_rel, dev, host64, round_storage, say, tdtype

pytestmark = pytest.mark.gpu

KL_BAND, GATE_BAND = 1e-3, 1e-5


def _sl():
    import token_locking_sparse_amd as sl
    return sl


def _odims(dm):
    return O.OracleDims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.vocab, dm.rms_eps, dm.rope_theta)


def _dev_model(dm, layers_np, embed=None, head=None, rope_n=None):
    sl = _sl()
    layers = [{k: dev(v, dm.dtype) for k, v in L.items()} for L in layers_np]
    return sl.DeviceModel(dtype=tdtype(dm.dtype), n_layers=dm.n_layers, d=dm.d, n_heads=dm.n_heads,
                          head_dim=dm.head_dim, ffn=dm.ffn, vocab=dm.vocab, rms_eps=dm.rms_eps,
                          rope_theta=dm.rope_theta, layers=layers,
                          embed=None if embed is None else dev(embed, dm.dtype),
                          lm_head=None if head is None else dev(head, dm.dtype), rope_n=rope_n)


# ------------------------------------------------------------------ one layer, hidden rows in
def _layer_case_run(dm, N, Ms, key, tol, no_kv_cache=False, minimal_ws=False, ws_rows=None):
    sl = _sl()
    case = W.layer_case(dm, N, Ms, key=key)
    B, M = case.B, case.M_tot
    Wnp = W.layer_weights(dm, 0)
    model = _dev_model(dm, [Wnp], rope_n=N)
    locked = np.ones(B * N, np.uint8)
    for b in range(B):
        locked[b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]]] = 0
    kc = dev(case.k_cache, dm.dtype).reshape(1, B, N, dm.n_heads, dm.head_dim)
    vc = dev(case.v_cache, dm.dtype).reshape(1, B, N, dm.n_heads, dm.head_dim)
    kc0, vc0 = kc.clone(), vc.clone()
    st = sl.DeviceState(model, B, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, dm.dtype),
                        k_cache=kc, v_cache=vc, with_h_out=True, minimal_workspace=minimal_ws)
    assert st.M_tot == M
    np.testing.assert_array_equal(st.act_idx[:M].cpu().numpy(), case.act_idx)
    if ws_rows is not None:   # the workspace a first step with ws_rows active rows would have been given
        st.ws = torch.empty(model.workspace_size(B, N, ws_rows, minimal_ws), dtype=torch.uint8, device="cuda")
    st.step(eps=0.0, do_lock=False, no_kv_cache=no_kv_cache)
    torch.cuda.synchronize()
    got_h = st.h_out[:M].cpu().numpy().astype(np.float64)
    # oracle
    od = _odims(dm)
    W64 = {k: O.widen(v, dm.dtype) for k, v in Wnp.items()}
    h_in = O.widen(case.h_in, dm.dtype)
    K64 = O.widen(case.k_cache, dm.dtype)
    V64 = O.widen(case.v_cache, dm.dtype)
    ostate = O.OracleState(B=B, N=N, t=0, locked=locked, kc=[K64], vc=[V64], h_in=h_in)
    om = O.OracleModel(od, 1, lambda l: W64)
    out = O.step(om, ostate, 0.0, -1.0, do_lock=False, attend_locked=not no_kv_cache)
    if dm.dtype == "bf16":
        l2, rms, mx = check_hidden(got_h, out.h, tol[0], "hidden rows")
        say("hidden rows: rel L2 %.3e rms %.3e max %.3e" % (l2, rms, mx))
    else:
        check_rel(got_h, out.h, tol[0], tol[1], "hidden rows")
    gk = host64(kc).reshape(B * N, -1)
    gv = host64(vc).reshape(B * N, -1)
    rk = ostate.kc[0].reshape(B * N, -1)
    rv = ostate.vc[0].reshape(B * N, -1)
    act_g = np.flatnonzero(locked == 0)
    chk = (lambda a, b, w: check_hidden(a, b, tol[0], w)) if dm.dtype == "bf16" else (lambda a, b, w: check_rel(a, b, tol[0], tol[1], w))
    chk(gk[act_g], rk[act_g], "fresh K rows")
    chk(gv[act_g], rv[act_g], "fresh V rows")
    lk = np.flatnonzero(locked != 0)
    assert torch.equal(kc.reshape(B * N, -1)[torch.from_numpy(lk).cuda()], kc0.reshape(B * N, -1)[torch.from_numpy(lk).cuda()])
    assert torch.equal(vc.reshape(B * N, -1)[torch.from_numpy(lk).cuda()], vc0.reshape(B * N, -1)[torch.from_numpy(lk).cuda()])


SMALL_BF16 = W.Dims(n_layers=1, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16")
SMALL_F32 = W.Dims(n_layers=1, d=128, n_heads=4, head_dim=32, ffn=384, vocab=512, dtype="f32")
TOL = {"bf16": (1e-2, 2e-2), "f32": (1e-4, 1e-4)}


@pytest.mark.parametrize("dm,N,Ms", [
    (SMALL_BF16, 256, [256]), (SMALL_BF16, 256, [100]), (SMALL_BF16, 256, [1]),
    (SMALL_BF16, 128, [128, 3, 77]), (SMALL_F32, 64, [64]), (SMALL_F32, 64, [20, 64]),
    (W.Dims(n_layers=1, d=512, n_heads=8, head_dim=64, ffn=1024, vocab=1024, dtype="bf16"), 320, [300, 17]),
    (SMALL_BF16, 1024, [700]),   # enough rows for the largest GEMM tile
])
def test_layer_step_parity(dm, N, Ms):
    say("layer step", dm.d, dm.dtype, N, Ms)
    _layer_case_run(dm, N, Ms, key=N + sum(Ms), tol=TOL[dm.dtype])


@pytest.mark.slow
@pytest.mark.parametrize("M", [1024, 512, 256, 64])
def test_layer_step_full_llada_shape(M):
    """One LLaDA-8B-shaped layer (d=4096, 32x128, FFN 12288), N=1024, M active rows."""
    say("full layer step M=%d" % M)
    _layer_case_run(W.LLADA_LAYER, 1024, [M], key=M, tol=TOL["bf16"])


@pytest.mark.slow
@pytest.mark.parametrize("dm,N,Ms", [
    (SMALL_BF16, 256, [100]), (SMALL_BF16, 128, [128, 3, 77]), (SMALL_F32, 64, [20, 64]),
    (W.Dims(n_layers=1, d=512, n_heads=8, head_dim=64, ffn=1024, vocab=1024, dtype="bf16"), 320, [300, 17]),
    (W.LLADA_LAYER, 1024, [256]),
])
def test_layer_step_no_kv_cache_ablation(dm, N, Ms):
    """The no-KV-cache ablation (positions locked before the step are not attended) against the
    oracle's step with attend_locked=False."""
    say("layer step no kv cache", dm.d, dm.dtype, N, Ms)
    _layer_case_run(dm, N, Ms, key=N + sum(Ms) + 1, tol=TOL[dm.dtype], no_kv_cache=True)


@pytest.mark.parametrize("M", [512, 64])
def test_layer_step_minimal_workspace(M):
    """The smallest workspace sl_step accepts: the split-K residual projections (down at M = 512, O and
    down at M = 64) accumulate with fp32 atomics instead of partial-sum planes; same bar against the
    oracle."""
    say("layer step minimal workspace", M)
    _layer_case_run(W.LLADA_LAYER, 1024, [M], key=M + 3, tol=TOL["bf16"], minimal_ws=True)


def test_layer_step_in_workspace_sized_for_more_rows():
    """A step at M = 128 in exactly the workspace sized for 129 rows (a later, smaller step of the same
    loop).  At 128 rows the attention splits its keys and stores per-split partials, so the step needs
    more than 129 rows' own layout; the size covers every M up to the one it is asked for."""
    say("layer step M=128 in the workspace for 129 rows")
    _layer_case_run(W.LLADA_LAYER, 1024, [128], key=128 + 5, tol=TOL["bf16"], ws_rows=129)


@pytest.mark.parametrize("M", [256, 64])
def test_layer_step_is_deterministic(M):
    """Two runs of the same step give bit-identical hidden rows and caches: split-K partial sums are
    added in a fixed order (no atomics) and every other reduction has a fixed shape."""
    sl = _sl()
    say("layer step determinism", M)
    dm, N = W.LLADA_LAYER, 1024
    case = W.layer_case(dm, N, [M], key=M + 5)
    model = _dev_model(dm, [W.layer_weights(dm, 0)], rope_n=N)
    locked = np.ones(N, np.uint8)
    locked[case.act_idx] = 0
    outs = []
    for _ in range(2):
        kc = dev(case.k_cache, "bf16").reshape(1, 1, N, dm.n_heads, dm.head_dim)
        vc = dev(case.v_cache, "bf16").reshape(1, 1, N, dm.n_heads, dm.head_dim)
        st = sl.DeviceState(model, 1, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, "bf16"),
                            k_cache=kc, v_cache=vc, with_h_out=True)
        st.step(eps=0.0, do_lock=False)
        torch.cuda.synchronize()
        outs.append((st.h_out[:M].clone(), kc.clone(), vc.clone()))
    assert all(torch.equal(a, b) for a, b in zip(outs[0], outs[1]))


def test_layer_step_batched_full_shape():
    """The LLaDA-8B-shaped layer on 8 sequences x N=2048 with ragged active sets (fraction per
    sequence uniform on [0.05, 0.8]): attention within each sequence only."""
    Ms = W.ragged_ms(8, 2048, key=8 * 2048)
    say("batched full layer step", Ms)
    _layer_case_run(W.LLADA_LAYER, 2048, Ms, key=8 * 2048, tol=TOL["bf16"])


_LLADA8B = {}


def _llada8b_weights():
    """Storage weights of the 32-layer LLaDA-8B-shaped model (generated once per test session)."""
    if not _LLADA8B:
        from concurrent.futures import ThreadPoolExecutor
        dm = W.LLADA_8B
        say("32-layer model: generating weights")
        with ThreadPoolExecutor(16) as ex:
            layers = list(ex.map(lambda l: W.layer_weights(dm, l), range(dm.n_layers)))
            emb_f, head_f = ex.submit(W.embed_weights, dm), ex.submit(W.lm_head_weights, dm)
            _LLADA8B["w"] = (layers, emb_f.result(), head_f.result())
    return _LLADA8B["w"]


@pytest.mark.slow
def test_full_model_step_32_layers():
    """One step (t = 0, all 512 positions active) of the 32-layer LLaDA-8B-shaped model: embedding of
    128 prompt ids + 384 [MASK], 32 layers, LM head over V = 126464, sampler unmasking 3 positions.

    After 32 layers the bf16 storage of the intermediates leaves a logits error of relative L2
    1.20e-2 (rms 0.0154, max 0.095): a CPU emulation that rounds exactly where the kernels store
    bf16 gives those figures against the float64 oracle.  The test holds the GPU to relative L2
    <= 1.5e-2 with no element beyond 7 rms; argmax and sampler choices may differ only at near-ties
    within that error."""
    sl = _sl()
    dm = W.LLADA_8B
    B, N, n_prompt, k_unmask = 1, 512, 128, 3
    layers, emb, head = _llada8b_weights()
    tok0 = W.prompt_tokens(dm, B, N, n_prompt)
    cand0 = (tok0 != dm.mask_id).astype(np.uint8)
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                        cand=torch.from_numpy(cand0.copy()).cuda())
    st.step(0.05, -1.0, dm.mask_id, True, k_unmask)
    torch.cuda.synchronize()
    gz = host64(st.logits[0])[:N]
    gtok = st.tok.cpu().numpy()
    assert st.M_tot == N and int(st.locked.sum()) == 0            # t = 0: no previous posterior, no lock
    say("32-layer step: oracle")
    od = _odims(dm)
    om = O.OracleModel(od, dm.n_layers, lambda l: {k: O.widen(v, dm.dtype) for k, v in layers[l].items()},
                       O.widen(emb, dm.dtype), O.widen(head, dm.dtype))
    ost = O.OracleState(B=B, N=N, t=0, locked=np.zeros(B * N, np.uint8),
                        kc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(dm.n_layers)],
                        vc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(dm.n_layers)],
                        tok=tok0.copy(), cand=cand0.copy())
    out = O.step(om, ost, 0.05, -1.0, True, dm.mask_id)
    z = out.logits
    d = gz - z
    rms = float(np.sqrt(np.mean(d * d)))
    rel = float(np.linalg.norm(d) / np.linalg.norm(z))
    say("32-layer logits: rel L2 %.3e rms %.3e max %.3e" % (rel, rms, np.abs(d).max()))
    assert rel <= 1.5e-2
    assert np.abs(d).max() <= max(7 * rms, 2e-2)
    # argmax over ids other than [MASK]: a mismatch only where the oracle's top two are within the error
    keep = np.ones(dm.vocab, bool)
    keep[dm.mask_id] = False
    zk, gk = z[:, keep], gz[:, keep]
    ia, ga = np.argmax(zk, 1), np.argmax(gk, 1)
    top2 = np.sort(zk, 1)[:, -2:]
    for i in np.flatnonzero(ia != ga):
        assert top2[i, 1] - top2[i, 0] <= 2 * 7 * rms, "argmax mismatch at %d with margin %.3g" % (i, top2[i, 1] - top2[i, 0])
    # sampler: the k most confident [MASK] positions; differing picks only at near-ties of confidence
    picked = O.sampler_unmask(ost.tok, ost.cand, out.act_idx, out.act_off, N, out.stats.argmax, out.stats.conf,
                              dm.mask_id, k_unmask)
    gpu_picked = np.flatnonzero(gtok != tok0)
    assert len(gpu_picked) == k_unmask
    conf = out.stats.conf
    kth = np.sort(conf[tok0 == dm.mask_id])[-k_unmask]
    for gp in set(picked) ^ set(gpu_picked.tolist()):
        assert abs(conf[gp] - kth) <= 0.1 * kth, "sampler pick %d not a near-tie" % gp
    for gp in set(picked) & set(gpu_picked.tolist()):
        i = int(gp)
        assert gtok[gp] == ost.tok[gp] or top2[i, 1] - top2[i, 0] <= 2 * 7 * rms


@pytest.mark.slow
def test_full_model_late_step_32_layers():
    """A late step of the 32-layer LLaDA-8B-shaped model, teacher-forced from a seeded mid-loop state:
    N = 512 with 128 prompt ids and 200 positions already unmasked to random ids; 260 of those 328
    positions locked (their cached K/V in every layer random N(0,1)), 252 active; t = 40 with the
    previous posterior equal to the oracle's logits of this step plus N(0, 0.05^2) drift; eps = 0.05,
    gate at the median, 3 unmasks.

    Attending to random unit-variance caches grows the residual stream faster than at t = 0 (hidden
    rms 13.4 after layer 31 against the oracle), and the bf16 roundings compound with it: a CPU
    emulation that rounds to bf16 exactly where the kernels store bf16 gives logits relative L2
    2.23e-2, rms 0.0286, max 0.181 (6.3 rms) on this state.  The test holds the GPU to relative L2
    <= 2.8e-2 (the t = 0 test's 1.25x margin over its emulation) with no element beyond 7 rms; an
    argmax may differ only at a top-two margin within 2 * 7 rms.  KL within 1e-3; gate, lock,
    compaction and sampler exact against the GPU's own statistics, and against the oracle except where
    the measured u error or a confidence near-tie can move a decision."""
    sl = _sl()
    dm = W.LLADA_8B
    B, N, t, eps, gate, k_unmask = 1, 512, 40, 0.05, 0.5, 3
    layers, emb, head = _llada8b_weights()
    g = W.rng(W.SEED_SETS, 7777)
    tok0 = W.prompt_tokens(dm, B, N, 128)
    done = 128 + g.permutation(N - 128)[:200]
    tok0[done] = g.integers(0, dm.vocab - 1, size=200)
    unmasked = np.flatnonzero(tok0 != dm.mask_id)
    locked = np.zeros(N, np.uint8)
    locked[g.permutation(unmasked)[:260]] = 1
    cand0 = (tok0 != dm.mask_id).astype(np.uint8)
    act = np.flatnonzero(locked == 0).astype(np.int32)
    M = len(act)
    kc_st = [W.to_storage(W.normal(W.rng(W.SEED_CACHE, 7777, l, 0), (B, N, dm.n_heads, dm.head_dim), 1.0), "bf16")
             for l in range(dm.n_layers)]
    vc_st = [W.to_storage(W.normal(W.rng(W.SEED_CACHE, 7777, l, 1), (B, N, dm.n_heads, dm.head_dim), 1.0), "bf16")
             for l in range(dm.n_layers)]
    # oracle: this step's logits (the layers and LM head over the active rows), then the statistics
    say("32-layer late step: oracle, M = %d" % M)
    od = _odims(dm)
    om = O.OracleModel(od, dm.n_layers, lambda l: {k: O.widen(v, dm.dtype) for k, v in layers[l].items()},
                       O.widen(emb, dm.dtype), O.widen(head, dm.dtype))
    ost = O.OracleState(B=B, N=N, t=0, locked=locked.copy(), kc=[O.widen(k, "bf16") for k in kc_st],
                        vc=[O.widen(v, "bf16") for v in vc_st], tok=tok0.copy(), cand=cand0.copy())
    z = O.step(om, ost, 0.0, -1.0, do_lock=False, mask_id=dm.mask_id).logits
    prev_st = W.to_storage(z.astype(np.float32) + W.normal(W.rng(W.SEED_DRIFT, 7777), z.shape, 0.05), "bf16")
    ref = O.posterior_stats(z, O.widen(prev_st, "bf16"), dm.mask_id)
    off = np.array([0, M], np.int32)
    lr = O.lock_update(locked, act, off, B, N, ref.kl, ref.u, cand0, eps, gate, True)
    # GPU: the same state at step t
    say("32-layer late step: GPU")
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    kc = torch.stack([dev(k, "bf16") for k in kc_st])
    vc = torch.stack([dev(v, "bf16") for v in vc_st])
    lk = torch.from_numpy(np.flatnonzero(locked)).cuda()
    kc_lock0, vc_lock0 = kc[:, 0, lk].clone(), vc[:, 0, lk].clone()
    st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(), cand=torch.from_numpy(cand0.copy()).cuda(),
                        locked=torch.from_numpy(locked.copy()).cuda(), k_cache=kc, v_cache=vc)
    assert st.M_tot == M
    gi = torch.from_numpy(act.astype(np.int64)).cuda()
    st.logits[(t + 1) & 1].index_copy_(0, gi, dev(prev_st, "bf16"))
    st.t = t
    st.step(eps, gate, dm.mask_id, True, k_unmask)
    torch.cuda.synchronize()
    gz = host64(st.logits[t & 1].index_select(0, gi))
    d = gz - z
    rms = float(np.sqrt(np.mean(d * d)))
    rel = float(np.linalg.norm(d) / np.linalg.norm(z))
    say("32-layer late-step logits: rel L2 %.3e rms %.3e max %.3e" % (rel, rms, np.abs(d).max()))
    assert rel <= 2.8e-2
    assert np.abs(d).max() <= max(7 * rms, 2e-2)
    keep = np.ones(dm.vocab, bool)
    keep[dm.mask_id] = False
    zk, gk = z[:, keep], gz[:, keep]
    ia, ga = np.argmax(zk, 1), np.argmax(gk, 1)
    top2 = np.sort(zk, 1)[:, -2:]
    say("late-step argmax agreement %.4f" % float(np.mean(ia == ga)))
    for i in np.flatnonzero(ia != ga):
        assert top2[i, 1] - top2[i, 0] <= 2 * 7 * rms, "argmax mismatch at %d with margin %.3g" % (i, top2[i, 1] - top2[i, 0])
    del zk, gk
    # locked rows' caches untouched in every layer
    assert torch.equal(kc[:, 0, lk], kc_lock0) and torch.equal(vc[:, 0, lk], vc_lock0)
    kl, u = st.kl[:M].cpu().numpy(), st.u[:M].cpu().numpy()
    assert np.max(np.abs(kl - ref.kl)) <= KL_BAND
    du = float(np.max(np.abs(u - ref.u)))
    # exact against the GPU's own statistics: gate threshold, lock update, compaction
    thr = float(st.gate_thr[0].item())
    assert thr == np.sort(u)[int(np.floor(np.float32(gate) * (M - 1)))]
    new = (cand0[act] != 0) & (kl <= np.float32(eps)) & (u <= thr)
    want = locked.copy()
    want[act[new]] = 1
    g_locked = st.locked.cpu().numpy()
    np.testing.assert_array_equal(g_locked, want)
    ri, ro = O.active_set(g_locked, B, N)
    np.testing.assert_array_equal(st.act_off.cpu().numpy(), ro)
    np.testing.assert_array_equal(st.act_idx[:int(ro[-1])].cpu().numpy(), ri)
    # against the oracle: differing decisions only inside the band the u error allows
    band = 2 * du + abs(thr - lr.gate_thr[0])
    diff = np.flatnonzero(new != lr.new_lock)
    say("late-step locks: gpu %d oracle %d differing %d (u error %.2e)" % (int(new.sum()), int(lr.new_lock.sum()),
                                                                        len(diff), du))
    assert np.all(np.abs(ref.u[diff] - lr.gate_thr[0]) <= band)
    # sampler: the GPU's picks follow its own confidences; against the oracle only near-ties differ
    gtok = st.tok.cpu().numpy()
    gpu_picked = np.flatnonzero(gtok != tok0)
    assert len(gpu_picked) == k_unmask and np.all(tok0[gpu_picked] == dm.mask_id)
    conf_g = st.conf[:M].cpu().numpy()
    masked_rows = np.flatnonzero(tok0[act] == dm.mask_id)
    order = masked_rows[np.lexsort((act[masked_rows], -conf_g[masked_rows]))][:k_unmask]
    np.testing.assert_array_equal(np.sort(act[order]), np.sort(gpu_picked))
    g_am = st.argmax[:M].cpu().numpy()
    np.testing.assert_array_equal(gtok[act[order]], g_am[order])
    picked = O.sampler_unmask(tok0.copy(), cand0.copy(), act, off, N, ref.argmax, ref.conf, dm.mask_id, k_unmask)
    kth = np.sort(ref.conf[masked_rows])[-k_unmask]
    rowof = {int(p): i for i, p in enumerate(act)}
    for gp in set(picked) ^ set(gpu_picked.tolist()):
        assert abs(ref.conf[rowof[gp]] - kth) <= 0.1 * kth, "sampler pick %d not a near-tie" % gp


# ------------------------------------------------------------------ tiny fp32 sampler loop (teacher-forced)
def _tiny_setup(dm, B, N, n_prompt):
    layers = [W.layer_weights(dm, l) for l in range(dm.n_layers)]
    emb = W.embed_weights(dm)
    head = W.lm_head_weights(dm)
    od = _odims(dm)
    L64 = [{k: O.widen(v, dm.dtype) for k, v in L.items()} for L in layers]
    om = O.OracleModel(od, dm.n_layers, lambda l: L64[l], O.widen(emb, dm.dtype), O.widen(head, dm.dtype))
    tok0 = W.prompt_tokens(dm, B, N, n_prompt)
    return layers, emb, head, om, tok0


def _load_state(st, ost, dm, B, N, t):
    """GPU state <- oracle state before step t (oracle -> GPU inputs, rounded to storage)."""
    sl = _sl()
    st.tok.copy_(torch.from_numpy(ost.tok).cuda())
    st.cand.copy_(torch.from_numpy(ost.cand).cuda())
    st.locked.copy_(torch.from_numpy(ost.locked).cuda())
    for l in range(dm.n_layers):
        st.k_cache[l].copy_(round_storage(ost.kc[l], dm.dtype))
        st.v_cache[l].copy_(round_storage(ost.vc[l], dm.dtype))
    if ost.post is not None:
        post = np.nan_to_num(ost.post, nan=0.0)
        st.logits[(t + 1) & 1].copy_(round_storage(post, dm.dtype))
    st.M_tot = sl.sl_compact(st.locked, B, N, st.act_idx, st.act_off, st.m_host)
    st.t = t


def _step_compare(st, ost_before, out, dm, B, N, eps, gate_q, tol_logit):
    """Compare one GPU step with the oracle step that started from the same state."""
    M = len(out.act_idx)
    rows_seq = O.seq_of_rows(out.act_off)
    glob = rows_seq * N + out.act_idx.astype(np.int64)
    cur = host64(st.logits[st.t & 1])    # st.t not yet advanced by the caller
    assert np.max(np.abs(cur[glob] - out.logits)) <= tol_logit
    kl = st.kl[:M].cpu().numpy()
    u = st.u[:M].cpu().numpy()
    if st.t > 0:
        assert np.max(np.abs(kl - out.stats.kl)) <= KL_BAND
    np.testing.assert_allclose(u, out.stats.u, atol=1e-4)
    locked = st.locked.cpu().numpy()
    diff = np.flatnonzero(locked != out.lock.locked)
    for gp in diff:
        i = int(np.flatnonzero(glob == gp)[0])
        near = abs(out.stats.kl[i] - eps) <= KL_BAND or (gate_q >= 0 and abs(out.stats.u[i] - out.lock.gate_thr[rows_seq[i]]) <= GATE_BAND)
        assert near, "lock mismatch at %d kl=%.6g" % (gp, out.stats.kl[i])
    return len(diff)


# lock rules: SureLock (KL test, gate off); the notes page's ablations (消融实验): confidence gate
# only (eps = +inf, gate at the median) and no KV cache (locked positions not attended)
LOOP_RULES = {"surelock": (0.05, -1.0, False), "gate_only": (math.inf, 0.5, False), "no_kv_cache": (0.05, -1.0, True)}


@pytest.mark.parametrize("rule", list(LOOP_RULES))
def test_tiny_loop_teacher_forced(rule):
    """2-layer fp32 model, d=128, 4x32 heads, FFN 384, V=512, N=64 (16 prompt + 48 masked),
    16 steps, 3 unmasks per step; eps=0.05 with the gate off, or one of the ablations."""
    sl = _sl()
    dm = W.TINY
    B, N, T = 1, 64, 16
    eps, gate, no_kv = LOOP_RULES[rule]
    layers, emb, head, om, tok0 = _tiny_setup(dm, B, N, 16)
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                        cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda())
    ost = O.OracleState(B=B, N=N, t=0, locked=np.zeros(B * N, np.uint8),
                        kc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(dm.n_layers)],
                        vc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(dm.n_layers)],
                        tok=tok0.copy(), cand=(tok0 != dm.mask_id).astype(np.uint8),
                        lock_step=np.full(B * N, -1, np.int32))
    total_mismatch, Ms = 0, []
    for t in range(T):
        say("tiny loop step", t)
        _load_state(st, ost, dm, B, N, t)
        post_before = None if ost.post is None else ost.post.copy()
        M_before = st.M_tot
        ost.t = t
        out = O.step(om, ost, eps, gate, True, dm.mask_id, attend_locked=not no_kv)
        tok_o = ost.tok.copy()
        O.sampler_unmask(ost.tok, ost.cand, out.act_idx, out.act_off, N, out.stats.argmax, out.stats.conf,
                         dm.mask_id, 3)
        p = sl.surelock.sl_step_params(eps, gate, dm.mask_id, 1, 3, int(no_kv))
        sl.sl_step(model.s, st.struct(), p, st.ws)
        torch.cuda.synchronize()
        total_mismatch += _step_compare(st, None, out, dm, B, N, eps, gate, 1e-4)
        # sampler: same positions unmasked to the same tokens (teacher-forced, fp32)
        np.testing.assert_array_equal(st.tok.cpu().numpy(), ost.tok)
        Ms.append(M_before)
    assert total_mismatch == 0
    assert all(a >= b for a, b in zip(Ms, Ms[1:]))


def test_tiny_loop_free_running_invariants():
    """The GPU loop on its own: monotone A_t, frozen posterior and cache rows of locked positions."""
    sl = _sl()
    dm = W.TINY
    B, N, T, eps = 2, 64, 16, 0.05
    layers, emb, head, om, tok0 = _tiny_setup(dm, B, N, 16)
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                        cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda())
    frozen = {}
    prevM = st.M_tot
    for t in range(T):
        say("free loop step", t)
        locked_before = st.locked.clone()
        st.step(eps, -1.0, dm.mask_id, True, 3)
        torch.cuda.synchronize()
        assert st.M_tot <= prevM
        prevM = st.M_tot
        assert bool(torch.all(st.locked >= locked_before))
        new = torch.nonzero(st.locked > locked_before).flatten().tolist()
        for g in new:
            buf = t & 1
            frozen[g] = (st.logits[buf][g].clone(), st.k_cache[:, g // N, g % N].clone(),
                         st.v_cache[:, g // N, g % N].clone(), buf)
            assert int(st.lock_step[g]) == t
        for g, (p, k, v, buf) in frozen.items():
            assert torch.equal(st.logits[buf][g], p)
            assert torch.equal(st.k_cache[:, g // N, g % N], k)
            assert torch.equal(st.v_cache[:, g // N, g % N], v)
    assert len(frozen) > 0


def test_step_with_every_position_locked_is_a_no_op():
    """M_tot = 0 (every position locked): the step launches nothing and changes nothing."""
    sl = _sl()
    dm = W.TINY
    B, N = 2, 64
    layers, emb, head, om, tok0 = _tiny_setup(dm, B, N, 16)
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                        cand=torch.ones(B * N, dtype=torch.uint8, device="cuda"),
                        locked=torch.ones(B * N, dtype=torch.uint8, device="cuda"))
    assert st.M_tot == 0
    for t in range(2):
        st.logits[t].fill_(3.0)
    before = [x.clone() for x in (st.tok, st.locked, st.k_cache, st.v_cache, st.logits[0], st.logits[1])]
    for t in range(2):
        assert st.step(0.05, 0.5, dm.mask_id, True, 3) == 0
    torch.cuda.synchronize()
    after = (st.tok, st.locked, st.k_cache, st.v_cache, st.logits[0], st.logits[1])
    assert all(torch.equal(a, b) for a, b in zip(before, after))
    np.testing.assert_array_equal(st.act_off.cpu().numpy(), np.zeros(B + 1, np.int32))


def test_tiny_loop_is_deterministic():
    """Two free-running loops from the same start take the same lock decisions and produce the same
    tokens, masks and posteriors, bit for bit."""
    sl = _sl()
    dm = W.TINY
    B, N, T = 2, 64, 12
    layers, emb, head, om, tok0 = _tiny_setup(dm, B, N, 16)
    model = _dev_model(dm, layers, emb, head, rope_n=N)
    runs = []
    for r in range(2):
        say("deterministic loop run", r)
        st = sl.DeviceState(model, B, N, tok=torch.from_numpy(tok0.copy()).cuda(),
                            cand=torch.from_numpy((tok0 != dm.mask_id).astype(np.uint8)).cuda())
        Ms = [st.step(0.05, 0.5, dm.mask_id, True, 3) for _ in range(T)]
        torch.cuda.synchronize()
        runs.append((Ms, st.tok.clone(), st.locked.clone(), st.lock_step.clone(), st.logits[0].clone(),
                     st.logits[1].clone()))
    assert runs[0][0] == runs[1][0]
    assert all(torch.equal(a, b) for a, b in zip(runs[0][1:], runs[1][1:]))


# ------------------------------------------------------------------ batched ragged step with LM head and lock
@pytest.mark.parametrize("dm,B,N,gate,ms", [
    (W.Dims(n_layers=1, d=256, n_heads=2, head_dim=128, ffn=512, vocab=2048, dtype="bf16"), 3, 128, 0.5, None),
    (W.Dims(n_layers=2, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16"), 2, 192, -1.0, None),
    # one sequence fully locked (no active row) between two active ones
    (W.Dims(n_layers=1, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16"), 3, 128, 0.5, [40, 0, 100]),
])
def test_batched_ragged_step(dm, B, N, gate, ms):
    sl = _sl()
    say("batched step", B, N, gate, ms)
    eps = 0.05
    Ms = W.ragged_ms(B, N, key=B * N) if ms is None else ms
    case = W.layer_case(dm, N, Ms, key=B + N)
    layers = [W.layer_weights(dm, l) for l in range(dm.n_layers)]
    head = W.lm_head_weights(dm)
    od = _odims(dm)
    L64 = [{k: O.widen(v, dm.dtype) for k, v in L.items()} for L in layers]
    om = O.OracleModel(od, dm.n_layers, lambda l: L64[l], None, O.widen(head, dm.dtype))
    locked = np.ones(B * N, np.uint8)
    for b in range(B):
        locked[b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]]] = 0
    K0 = [O.widen(case.k_cache, dm.dtype) for _ in range(dm.n_layers)]
    V0 = [O.widen(case.v_cache, dm.dtype) for _ in range(dm.n_layers)]
    h_in = O.widen(case.h_in, dm.dtype)
    # previous posterior: the oracle's logits of this very step plus N(0, 0.05^2) drift, rounded
    probe = O.OracleState(B=B, N=N, t=0, locked=locked.copy(), kc=[k.copy() for k in K0],
                          vc=[v.copy() for v in V0], h_in=h_in)
    z0 = O.step(om, probe, 0.0, -1.0, do_lock=False).logits
    rows_seq = O.seq_of_rows(case.act_off)
    glob = rows_seq * N + case.act_idx.astype(np.int64)
    prev_full = np.zeros((B * N, dm.vocab))
    prev_full[glob] = z0 + W.normal(W.rng(W.SEED_DRIFT, 42), z0.shape, 0.05)
    prev_st = W.to_storage(prev_full.astype(np.float32), dm.dtype)
    prev64 = O.widen(prev_st, dm.dtype)
    # oracle step at t=1 against that previous posterior
    ost = O.OracleState(B=B, N=N, t=1, locked=locked.copy(), kc=[k.copy() for k in K0],
                        vc=[v.copy() for v in V0], h_in=h_in, post=prev64.copy())
    out = O.step(om, ost, eps, gate, True, -1)
    # GPU
    model = _dev_model(dm, layers, None, head, rope_n=N)
    kc = torch.stack([dev(case.k_cache, dm.dtype)] * dm.n_layers)
    vc = torch.stack([dev(case.v_cache, dm.dtype)] * dm.n_layers)
    st = sl.DeviceState(model, B, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, dm.dtype),
                        k_cache=kc, v_cache=vc)
    st.logits[0].copy_(dev(prev_st, dm.dtype))     # buffer (t+1)%2 = 0 holds p_{t-1} at t = 1
    st.t = 1
    p = sl.surelock.sl_step_params(eps, gate, -1, 1, 0)
    sl.sl_step(model.s, st.struct(), p, st.ws)
    torch.cuda.synchronize()
    st.M_tot = st.m_host.value
    cur = host64(st.logits[1])
    assert np.max(np.abs(cur[glob] - out.logits)) <= 2e-2
    M = len(glob)
    kl = st.kl[:M].cpu().numpy()
    assert np.max(np.abs(kl - out.stats.kl)) <= KL_BAND
    g_locked = st.locked.cpu().numpy()
    diff = np.flatnonzero(g_locked != out.lock.locked)
    for gp in diff:
        i = int(np.flatnonzero(glob == gp)[0])
        near = abs(out.stats.kl[i] - eps) <= KL_BAND or (gate >= 0 and abs(out.stats.u[i] - out.lock.gate_thr[rows_seq[i]]) <= GATE_BAND)
        assert near
    ri, ro = O.active_set(g_locked, B, N)
    np.testing.assert_array_equal(st.act_off.cpu().numpy(), ro)
    np.testing.assert_array_equal(st.act_idx[:st.M_tot].cpu().numpy(), ri)


@pytest.mark.slow
def test_batched_step_full_shape_with_head():
    """The batched ragged workload at full size: 8 sequences x N=2048 (active fraction per sequence
    uniform on [0.05, 0.8]), one LLaDA-8B-shaped layer, final norm, LM head over V=126464, KL-lock
    (eps 0.05, gate at each sequence's median u) and compaction in one sl_step at t = 1.

    Teacher-forced: the previous posterior is the oracle's own logits of this step plus N(0, 0.05^2)
    drift, so every KL is near 0.00125 and the gate decides the locks.  Logits go through one layer of
    bf16 intermediates, so they are held to the hidden-row bound (relative L2 1e-2, no element beyond
    7 rms).  KL within 1e-3; u and lse within the bound their definitions give from the largest logit
    error.  The gate, lock and compaction are checked exactly against the GPU's own statistics, and
    against the oracle's decisions except where the gap between u and the gate threshold is inside
    what the u error can move."""
    sl = _sl()
    dm = W.LLADA_LAYER
    B, N, eps, gate = 8, 2048, 0.05, 0.5
    Ms = W.ragged_ms(B, N, key=B * N)
    say("batched full step with LM head", Ms)
    case = W.layer_case(dm, N, Ms, key=B * N)
    M = case.M_tot
    Wnp = W.layer_weights(dm, 0)
    head = W.lm_head_weights(dm)
    locked = np.ones(B * N, np.uint8)
    for b in range(B):
        locked[b * N + case.act_idx[case.act_off[b]:case.act_off[b + 1]]] = 0
    rows_seq = O.seq_of_rows(case.act_off)
    glob = rows_seq * N + case.act_idx.astype(np.int64)
    # oracle: hidden rows of the active set, final norm and LM head, then the posterior statistics
    od = _odims(dm)
    W64 = {k: O.widen(v, "bf16") for k, v in Wnp.items()}
    ost = O.OracleState(B=B, N=N, t=0, locked=locked.copy(), kc=[O.widen(case.k_cache, "bf16")],
                        vc=[O.widen(case.v_cache, "bf16")], h_in=O.widen(case.h_in, "bf16"))
    h = O.step(O.OracleModel(od, 1, lambda l: W64), ost, 0.0, -1.0, do_lock=False).h
    del W64, ost
    z = O.rmsnorm(h, dm.rms_eps) @ O.widen(head, "bf16").T
    prev_st = W.to_storage(z.astype(np.float32) + W.normal(W.rng(W.SEED_DRIFT, 4343), z.shape, 0.05), "bf16")
    prev64 = O.widen(prev_st, "bf16")
    ref = O.posterior_stats(z, prev64)
    del prev64
    lr = O.lock_update(locked, case.act_idx, case.act_off, B, N, ref.kl, ref.u, None, eps, gate, True)
    say("oracle done: new locks %d" % int(lr.new_lock.sum()))
    # GPU: the same step at t = 1 with that previous posterior in buffer 0
    model = _dev_model(dm, [Wnp], None, head, rope_n=N)
    H, Dh = dm.n_heads, dm.head_dim
    st = sl.DeviceState(model, B, N, locked=torch.from_numpy(locked).cuda(), h_in=dev(case.h_in, "bf16"),
                        k_cache=dev(case.k_cache, "bf16").reshape(1, B, N, H, Dh),
                        v_cache=dev(case.v_cache, "bf16").reshape(1, B, N, H, Dh),
                        cand=torch.ones(B * N, dtype=torch.uint8, device="cuda"))
    assert st.M_tot == M
    gi = torch.from_numpy(glob).cuda()
    st.logits[0].index_copy_(0, gi, dev(prev_st, "bf16"))
    del prev_st
    st.t = 1
    st.step(eps, gate, -1, True, 0)
    torch.cuda.synchronize()
    cur = host64(st.logits[1].index_select(0, gi))
    l2, rms, mx = check_hidden(cur, z, 1e-2, "logits")
    say("logits: rel L2 %.3e rms %.3e max %.3e" % (l2, rms, mx))
    dz = float(np.max(np.abs(cur - z)))
    del cur, z
    kl, u, lse = st.kl[:M].cpu().numpy(), st.u[:M].cpu().numpy(), st.lse[:M].cpu().numpy()
    assert np.max(np.abs(kl - ref.kl)) <= KL_BAND
    # lse moves by at most the largest logit error; u = 1 - exp(max z - lse) by at most twice that
    assert np.max(np.abs(lse - ref.lse)) <= dz + 1e-4
    du = float(np.max(np.abs(u - ref.u)))
    assert du <= 2 * dz + 1e-5
    # gate, lock and compaction, exactly, on the GPU's own statistics
    thr = st.gate_thr.cpu().numpy()
    g_locked = st.locked.cpu().numpy()
    new = np.zeros(M, dtype=bool)
    for b in range(B):
        s_ = slice(case.act_off[b], case.act_off[b + 1])
        kth = int(np.floor(np.float32(gate) * (Ms[b] - 1)))
        assert thr[b] == np.sort(u[s_])[kth]
        new[s_] = (kl[s_] <= np.float32(eps)) & (u[s_] <= thr[b])
    want = locked.copy()
    want[glob[new]] = 1
    np.testing.assert_array_equal(g_locked, want)
    ri, ro = O.active_set(g_locked, B, N)
    np.testing.assert_array_equal(st.act_off.cpu().numpy(), ro)
    np.testing.assert_array_equal(st.act_idx[:int(ro[-1])].cpu().numpy(), ri)
    # against the oracle's decisions: a row may differ only where |u - q| is within what the errors allow
    band = 2 * du + np.abs(thr - lr.gate_thr)[rows_seq]
    diff = np.flatnonzero(new != lr.new_lock)
    near = np.abs(ref.u - lr.gate_thr[rows_seq]) <= band
    say("lock decisions: gpu %d oracle %d differing %d (u error %.2e)" % (int(new.sum()), int(lr.new_lock.sum()),
                                                                       len(diff), du))
    assert np.all(near[diff])
