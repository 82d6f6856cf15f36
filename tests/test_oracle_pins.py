"""Pins of the CPU oracle against what the SureLock pages and mathematics fix.

Each test ties an oracle function to something other than itself: closed
forms (tests/golden/kl_closed_forms.json), library routines for special cases
(numpy quantile / nonzero, torch rms_norm / scaled_dot_product_attention /
silu), brute force on tiny inputs, and the invariants the pages state
(monotone active set, frozen posterior and cache of locked rows, no locking
=> the dense sampler).  test_planted_mistakes checks that plausible mistakes
in the oracle make these pins fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.surelock_oracle as O
import workloads as W
from tests.dense_ref import dense_block, dense_logits, rope_complex

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kl_closed_forms.json")))


# ------------------------------------------------------------------ storage widening
# bfloat16 is the upper half of an IEEE binary32: sign, 8 exponent bits, 7 mantissa bits.  Hand
# bit patterns and the values the format defines for them.
BF16_PATTERNS = [
    (0x3F80, 1.0), (0xC000, -2.0), (0x3F81, 1.0 + 2.0 ** -7), (0x4049, 3.140625),
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),        # largest finite, 3.3895e38
    (0x0080, 2.0 ** -126),                            # smallest normal
    (0x0001, 2.0 ** -133),                            # smallest subnormal
    (0x8000, -0.0), (0x7F80, math.inf), (0xFF80, -math.inf),
]


def pin_widen_bf16():
    bits = np.array([b for b, _ in BF16_PATTERNS], dtype=np.uint16)
    got = O.widen(bits, "bf16")
    assert got.dtype == np.float64
    for (b, want), g in zip(BF16_PATTERNS, got):
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), (hex(b), g, want)
    nan = O.widen(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")
    assert np.isnan(nan).all()
    # f32 storage is the value itself
    x = np.array([1.5, -2.25e-30, 3.0e38], dtype=np.float32)
    assert np.array_equal(O.widen(x, "f32"), x.astype(np.float64))


def test_widen_bf16_bit_patterns():
    pin_widen_bf16()


# ------------------------------------------------------------------ KL / u / LSE
def pin_kl_closed_forms():
    for c in GOLD["cases"]:
        p, q = np.array(c["p"]), np.array(c["q"])
        # logits are log-probabilities plus an arbitrary per-row shift (softmax is shift invariant)
        z = (np.log(p) + 3.25)[None, :]
        y = (np.log(q) - 1.5)[None, :]
        st = O.posterior_stats(z, y)
        assert abs(st.kl[0] - c["kl"]) < 1e-9, (c, st.kl[0])


def test_kl_closed_forms():
    pin_kl_closed_forms()


def test_kl_self_zero_and_gibbs():
    g = np.random.default_rng(0)
    z = g.normal(0, 2, size=(16, 300))
    y = z + g.normal(0, 0.3, size=z.shape)
    assert np.max(np.abs(O.posterior_stats(z, z).kl)) < 1e-12
    kl = O.posterior_stats(z, y).kl
    assert np.all(kl > 0)
    # second-order expansion: KL(p||q) ~ 1/2 Var_p(log p - log q) for a small drift
    d = 1e-3 * g.normal(size=z.shape)
    zp = z + d
    p = np.exp(zp - O.logsumexp_rows(zp)[:, None])
    var = (p * d * d).sum(1) - (p * d).sum(1) ** 2
    np.testing.assert_allclose(O.posterior_stats(zp, z).kl, 0.5 * var, rtol=2e-2)


def test_first_step_never_locks():
    st = O.posterior_stats(np.zeros((2, 5)), None)
    assert np.all(np.isinf(st.kl))


def test_u_lse_closed_forms():
    c = GOLD["confidence"]
    z = np.log(np.array(c["p"]))[None, :] + 7.0
    st = O.posterior_stats(z, None)
    assert abs(st.u[0] - c["u"]) < 1e-12
    st2 = O.posterior_stats(np.array([[0.0, math.log(3.0)]]), None)
    assert abs(st2.lse[0] - math.log(4.0)) < 1e-12
    # large-magnitude logits: LSE stays finite and exact (max shift)
    st3 = O.posterior_stats(np.array([[1000.0, 1000.0]]), None)
    assert abs(st3.lse[0] - (1000.0 + math.log(2.0))) < 1e-9


def test_argmax_excludes_mask_and_ties_low():
    z = np.array([[0.1, 2.0, 2.0, 5.0]])     # mask id 3 holds the global max
    st = O.posterior_stats(z, None, mask_id=3)
    assert st.argmax[0] == 1                  # lowest id among the tied non-mask maxima
    p = np.exp(z[0] - z[0].max()); p /= p.sum()
    assert abs(st.conf[0] - p[1]) < 1e-12
    assert abs(st.u[0] - (1 - p[3])) < 1e-12  # u uses the max over all ids, mask included


# ------------------------------------------------------------------ gate / lock / compaction
def test_gate_hand_list():
    g = GOLD["gate"]
    u = np.array(g["u"])
    q = O.gate_threshold(u, g["m"])
    assert q == g["q"]
    assert int((u <= q).sum()) == g["n_pass"]


def test_gate_matches_numpy_lower_quantile():
    rng = np.random.default_rng(1)
    for n in (1, 2, 3, 7, 100, 1639):
        u = rng.random(n)
        for m in (0.0, 0.25, 0.5, 0.9, 1.0):
            assert O.gate_threshold(u, m) == np.quantile(u, float(np.float32(m)), method="lower")


def _brute_active(locked, B, N):
    idx, off = [], [0]
    for b in range(B):
        for i in range(N):
            if locked[b * N + i] == 0:
                idx.append(i)
        off.append(len(idx))
    return np.array(idx, dtype=np.int32), np.array(off, dtype=np.int32)


def test_active_set_brute_force():
    rng = np.random.default_rng(2)
    for B, N, p in [(1, 1, 0.5), (1, 17, 0.3), (3, 40, 0.6), (4, 33, 0.0), (2, 50, 1.0)]:
        locked = (rng.random(B * N) < p).astype(np.uint8)
        a, o = O.active_set(locked, B, N)
        ba, bo = _brute_active(locked, B, N)
        np.testing.assert_array_equal(a, ba)
        np.testing.assert_array_equal(o, bo)


def test_lock_update_rules():
    rng = np.random.default_rng(3)
    B, N = 2, 30
    locked = (rng.random(B * N) < 0.4).astype(np.uint8)
    act, off = O.active_set(locked, B, N)
    M = len(act)
    kl = rng.random(M) * 0.1
    u = rng.random(M)
    cand = (rng.random(B * N) < 0.7).astype(np.uint8)
    eps = 0.05
    r = O.lock_update(locked, act, off, B, N, kl, u, cand, eps, 0.5, True)
    rows_seq = np.repeat(np.arange(B), np.diff(off))
    glob = rows_seq * N + act
    for i in range(M):                           # brute force, row by row
        b = rows_seq[i]
        us = np.sort(u[off[b]:off[b + 1]])
        q = us[int(math.floor(0.5 * (len(us) - 1)))]
        want = bool(cand[glob[i]]) and kl[i] <= eps and u[i] <= q
        assert r.new_lock[i] == want
    assert np.all(r.locked >= locked)            # monotone: never unlocks
    np.testing.assert_array_equal(r.act_idx, _brute_active(r.locked, B, N)[0])
    # eps <= 0 or no previous posterior: nothing locks
    for e, hp in ((0.0, True), (-1.0, True), (eps, False)):
        r0 = O.lock_update(locked, act, off, B, N, kl, u, cand, e, 0.5, hp)
        assert not r0.new_lock.any()
        np.testing.assert_array_equal(r0.locked, locked)
    # gate off: KL alone decides
    r2 = O.lock_update(locked, act, off, B, N, kl, u, None, eps, -1.0, True)
    np.testing.assert_array_equal(r2.new_lock, kl <= eps)


def test_sampler_top_k_brute_force():
    rng = np.random.default_rng(4)
    B, N, V = 2, 12, 9
    mask = V - 1
    tok = rng.integers(0, V - 1, size=B * N).astype(np.int32)
    tok[rng.random(B * N) < 0.6] = mask
    locked = np.zeros(B * N, np.uint8)
    act, off = O.active_set(locked, B, N)
    conf = np.round(rng.random(len(act)), 1)     # many ties: exercises the position tie-break
    am = rng.integers(0, V - 1, size=len(act))
    tok2, cand = tok.copy(), np.zeros(B * N, np.uint8)
    O.sampler_unmask(tok2, cand, act, off, N, am, conf, mask, 3)
    for b in range(B):
        cands = [(-conf[r], act[r], r) for r in range(off[b], off[b + 1]) if tok[b * N + act[r]] == mask]
        chosen = sorted(cands)[:3]
        for _, p, r in chosen:
            assert tok2[b * N + p] == am[r] and cand[b * N + p] == 1
        changed = set(np.flatnonzero(tok2[b * N:(b + 1) * N] != tok[b * N:(b + 1) * N]))
        assert changed <= {p for _, p, _ in chosen}


# ------------------------------------------------------------------ transformer pieces
def test_rmsnorm_matches_torch():
    h = np.random.default_rng(5).normal(size=(7, 64)) * 3
    ref = F.rms_norm(torch.tensor(h), (64,), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rmsnorm(h, 1e-5), ref, rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    g = np.linspace(-40, 40, 801)
    np.testing.assert_allclose(O.silu(g), F.silu(torch.tensor(g)).numpy(), rtol=1e-13, atol=1e-15)


def pin_rope():
    rng = np.random.default_rng(6)
    H, Dh, th = 2, 16, 10000.0
    x = rng.normal(size=(5, H, Dh))
    pos = np.array([0, 1, 7, 100, 4095])
    r = O.rope(x, pos, th)
    np.testing.assert_allclose(r[0], x[0], atol=0)                    # position 0: identity
    half = Dh // 2
    n_in = x[..., :half] ** 2 + x[..., half:] ** 2
    n_out = r[..., :half] ** 2 + r[..., half:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)               # each pair is rotated
    q, k = rng.normal(size=(1, H, Dh)), rng.normal(size=(1, H, Dh))
    for (m, n, s) in ((3, 10, 5), (0, 40, 17), (123, 7, 1000)):       # relative-position property
        a = (O.rope(q, np.array([m]), th) * O.rope(k, np.array([n]), th)).sum()
        b = (O.rope(q, np.array([m + s]), th) * O.rope(k, np.array([n + s]), th)).sum()
        assert abs(a - b) < 1e-9
    for j in (0, 1, 5):                                               # frequency of pair j
        e = np.zeros((1, 1, Dh)); e[0, 0, j] = 1.0
        dlt = 37
        dot = (O.rope(e, np.array([dlt]), th) * e).sum()
        assert abs(dot - math.cos(dlt * th ** (-2.0 * j / Dh))) < 1e-12
    # agrees with the complex-multiplication form used by the dense reference
    ref = rope_complex(torch.tensor(x), torch.tensor(pos), th).numpy()
    np.testing.assert_allclose(r, ref, rtol=1e-12, atol=1e-12)


def test_rope_properties():
    pin_rope()


def pin_attention():
    rng = np.random.default_rng(7)
    N, H, Dh = 6, 2, 4
    q, K, V = rng.normal(size=(N, H, Dh)), rng.normal(size=(N, H, Dh)), rng.normal(size=(N, H, Dh))
    o = O.attention(q, K, V, 1.0 / math.sqrt(Dh))
    for i in range(N):                                                # explicit loops
        for h in range(H):
            s = [sum(q[i, h, c] * K[j, h, c] for c in range(Dh)) / math.sqrt(Dh) for j in range(N)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            tot = sum(e)
            for c in range(Dh):
                want = sum(e[j] * V[j, h, c] for j in range(N)) / tot
                assert abs(o[i, h, c] - want) < 1e-12
    # M = N equals torch dense attention
    ref = F.scaled_dot_product_attention(torch.tensor(q).transpose(0, 1), torch.tensor(K).transpose(0, 1),
                                         torch.tensor(V).transpose(0, 1)).transpose(0, 1).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # an active row's output does not depend on which other rows are active
    sub = [1, 4]
    np.testing.assert_allclose(O.attention(q[sub], K, V, 1.0 / math.sqrt(Dh)), o[sub], rtol=1e-13, atol=1e-14)


def test_attention_pins():
    pin_attention()


# ------------------------------------------------------------------ layer / step vs dense
def _tiny_model(n_layers=2, d=64, H=2, Dh=32, Fd=96, V=50, key=0):
    dm = W.Dims(n_layers=n_layers, d=d, n_heads=H, head_dim=Dh, ffn=Fd, vocab=V, dtype="f32", weight_std=0.05)
    layers = [{k: O.widen(v, "f32") for k, v in W.layer_weights(dm, l, seed=10 + key).items()}
              for l in range(n_layers)]
    emb = O.widen(W.embed_weights(dm, seed=10 + key), "f32")
    head = O.widen(W.lm_head_weights(dm, seed=10 + key), "f32")
    od = O.OracleDims(d, H, Dh, Fd, V, dm.rms_eps, dm.rope_theta)
    return dm, od, layers, emb, head


def pin_layer_dense():
    dm, od, layers, _, _ = _tiny_model(n_layers=1)
    N = 12
    h = np.random.default_rng(8).normal(size=(N, od.d))
    Kc = np.zeros((N, od.n_heads, od.head_dim)); Vc = np.zeros_like(Kc)
    out = O.layer_forward(h, np.arange(N), layers[0], Kc, Vc, od)
    ref, k, v = dense_block(torch.tensor(h), layers[0], od.n_heads, od.rms_eps, od.rope_theta)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Kc, k.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Vc, v.numpy(), rtol=1e-11, atol=1e-11)
    # subset of rows against the cache of the full pass: same outputs for those rows
    sub = np.array([0, 5, 11])
    Kc2, Vc2 = Kc.copy(), Vc.copy()
    out2 = O.layer_forward(h[sub], sub, layers[0], Kc2, Vc2, od)
    np.testing.assert_allclose(out2, out[sub], rtol=1e-11, atol=1e-11)


def test_layer_equals_dense_block():
    pin_layer_dense()


def pin_no_kv_cache_ablation():
    """The no-KV-cache ablation (zhaoyang97 notes, 消融实验: locked positions cannot be attended)
    equals a dense block over the active rows alone at their own positions, and never reads the
    cache rows of locked positions (NaN there changes nothing)."""
    dm, od, layers, _, _ = _tiny_model(n_layers=1)
    N = 12
    h = np.random.default_rng(9).normal(size=(N, od.d))
    sub = np.array([1, 2, 6, 7, 10])
    Kc = np.full((N, od.n_heads, od.head_dim), np.nan); Vc = Kc.copy()
    out = O.layer_forward(h[sub], sub, layers[0], Kc, Vc, od, attend_locked=False)
    ref, k, v = dense_block(torch.tensor(h[sub]), layers[0], od.n_heads, od.rms_eps, od.rope_theta, pos=sub)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(Kc[sub], k.numpy(), rtol=1e-11, atol=1e-11)
    # with every position active the ablation is the ordinary layer
    Kc2 = np.zeros((N, od.n_heads, od.head_dim)); Vc2 = np.zeros_like(Kc2)
    Kc3, Vc3 = Kc2.copy(), Vc2.copy()
    np.testing.assert_allclose(O.layer_forward(h, np.arange(N), layers[0], Kc2, Vc2, od, attend_locked=False),
                               O.layer_forward(h, np.arange(N), layers[0], Kc3, Vc3, od), rtol=1e-13, atol=1e-13)


def test_no_kv_cache_ablation():
    pin_no_kv_cache_ablation()


def test_gate_only_rule_is_eps_infinity():
    """Confidence gate only (zhaoyang97 notes, 消融实验) as eps = +inf with the gate on: candidates
    lock exactly when u <= q_m (brute force); KL only is the gate off."""
    rng = np.random.default_rng(21)
    B, N = 2, 40
    locked = (rng.random(B * N) < 0.3).astype(np.uint8)
    ai, ao = O.active_set(locked, B, N)
    M = len(ai)
    kl = rng.random(M) * 0.2
    u = rng.random(M)
    cand = (rng.random(B * N) < 0.7).astype(np.uint8)
    lr = O.lock_update(locked, ai, ao, B, N, kl, u, cand, np.inf, 0.5, True)
    for b in range(B):
        rows = range(ao[b], ao[b + 1])
        us = sorted(u[r] for r in rows)
        q = us[int(np.floor(0.5 * (len(us) - 1)))]
        for r in rows:
            g = b * N + ai[r]
            assert lr.new_lock[r] == bool(cand[g] and u[r] <= q)
    # KL only: gate off, eps finite
    lr2 = O.lock_update(locked, ai, ao, B, N, kl, u, cand, 0.1, -1.0, True)
    glob = O.seq_of_rows(ao) * N + ai
    np.testing.assert_array_equal(lr2.new_lock, (cand[glob] != 0) & (kl <= 0.1))


def test_eps_zero_step_equals_dense_sampler():
    dm, od, layers, emb, head = _tiny_model()
    B, N, T = 2, 16, 4
    tok0 = W.prompt_tokens(dm, B, N, 5, key=3)
    model = O.OracleModel(od, dm.n_layers, lambda l: layers[l], emb, head)
    recs = O.run_loop(model, tok0, B, N, T, eps=0.0, gate_m=-1.0, unmask_k=3)
    for r in recs:
        assert r.M == B * N and r.new_locks == 0
    # replay the tokens each step saw through the dense model
    tok = tok0.copy()
    for r in recs:
        for b in range(B):
            ref = dense_logits(tok[b * N:(b + 1) * N], emb, layers, head, od.n_heads, od.rms_eps, od.rope_theta)
            np.testing.assert_allclose(r.logits[b * N:(b + 1) * N], ref, rtol=1e-10, atol=1e-10)
        tok = r.tok


def test_loop_invariants_with_locking():
    dm, od, layers, emb, head = _tiny_model(V=40)
    B, N, T = 2, 24, 10
    tok0 = W.prompt_tokens(dm, B, N, 8, key=4)
    model = O.OracleModel(od, dm.n_layers, lambda l: layers[l], emb, head)
    snaps = {}
    prev = {"locked": np.zeros(B * N, np.uint8), "cand": (tok0 != dm.mask_id)}
    total_locks = [0]

    def on_step(rec, st):
        # monotone: the lock mask never clears, A_{t+1} within A_t
        assert np.all(st.locked >= prev["locked"])
        newly = np.flatnonzero(st.locked & ~prev["locked"])
        # only candidates (unmasked in this step's input) lock
        assert np.all(prev["cand"][newly])
        total_locks[0] += len(newly)
        for g in newly:
            snaps[int(g)] = (st.post[g].copy(), [st.kc[l].reshape(B * N, -1)[g].copy() for l in range(dm.n_layers)],
                             [st.vc[l].reshape(B * N, -1)[g].copy() for l in range(dm.n_layers)])
        for g, (p, ks, vs) in snaps.items():   # frozen posterior and cache, bitwise
            assert np.array_equal(st.post[g], p)
            for l in range(dm.n_layers):
                assert np.array_equal(st.kc[l].reshape(B * N, -1)[g], ks[l])
                assert np.array_equal(st.vc[l].reshape(B * N, -1)[g], vs[l])
        prev["locked"] = st.locked.copy()
        prev["cand"] = st.cand.astype(bool).copy()
        assert np.all((st.tok != dm.mask_id) == st.cand.astype(bool))   # cand <=> unmasked

    recs = O.run_loop(model, tok0, B, N, T, eps=0.05, gate_m=-1.0, unmask_k=3, on_step=on_step)
    Ms = [r.M for r in recs]
    assert all(a >= b for a, b in zip(Ms, Ms[1:]))
    assert total_locks[0] > 0, "the random model should lock some positions at eps=0.05"


def test_layer_flops_model():
    od = O.OracleDims(4096, 32, 128, 12288, 126464, 1e-5, 1e4)
    # 8 d^2 + 6 d F + 4 N d = 453.0 MFLOP per row at d = 4096, F = 12288, N = 1024
    assert abs(O.layer_flops(od, 1, 1024) / 1e6 - 453.0) < 0.1


# ------------------------------------------------------------------ planted mistakes
def _expect_fail(fn):
    with pytest.raises(AssertionError):
        fn()


def test_planted_mistakes(monkeypatch):
    """Plausible oracle mistakes are caught by the pins above."""
    good_widen = O.widen
    for bad in (lambda a, dt: (np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64),
                lambda a, dt: np.asarray(a, np.uint16).view(np.float16).astype(np.float64)):
        monkeypatch.setattr(O, "widen", lambda a, dt, bad=bad: bad(a, dt) if dt == "bf16" else good_widen(a, dt))
        _expect_fail(pin_widen_bf16)
    monkeypatch.setattr(O, "widen", good_widen)

    good_stats = O.posterior_stats

    def reversed_kl(z, y, mask_id=-1, chunk=64):
        s = good_stats(z, y, mask_id, chunk)
        if y is not None:
            s.kl = good_stats(y, z, mask_id, chunk).kl
        return s
    monkeypatch.setattr(O, "posterior_stats", reversed_kl)
    _expect_fail(pin_kl_closed_forms)
    monkeypatch.setattr(O, "posterior_stats", good_stats)

    good_rope = O.rope

    def rope_bad_sign(x, pos, theta):
        Dh = x.shape[-1]; half = Dh // 2
        inv = theta ** (-(np.arange(half) * 2.0) / Dh)
        ang = np.asarray(pos, float)[:, None] * inv[None, :]
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        x1, x2 = x[..., :half], x[..., half:]
        return np.concatenate([x1 * c + x2 * s, x2 * c + x1 * s], axis=-1)   # sign dropped
    monkeypatch.setattr(O, "rope", rope_bad_sign)
    _expect_fail(pin_rope)
    _expect_fail(pin_layer_dense)
    monkeypatch.setattr(O, "rope", good_rope)

    good_attn = O.attention

    def attn_no_scale(q, K, V, scale):
        return good_attn(q, K, V, 1.0)
    monkeypatch.setattr(O, "attention", attn_no_scale)
    _expect_fail(pin_attention)
    _expect_fail(pin_layer_dense)
    monkeypatch.setattr(O, "attention", good_attn)

    def attn_keys_transposed(q, K, V, scale):        # heads and positions confused
        return good_attn(q, np.transpose(K, (1, 0, 2))[: K.shape[0]].reshape(K.shape) if K.shape[0] == K.shape[1]
                         else K[::-1], V, scale)
    monkeypatch.setattr(O, "attention", attn_keys_transposed)
    _expect_fail(pin_layer_dense)
    monkeypatch.setattr(O, "attention", good_attn)

    good_silu = O.silu
    monkeypatch.setattr(O, "silu", lambda g: g / (1 + np.exp(g)))  # wrong sign in the sigmoid
    _expect_fail(pin_layer_dense)
    monkeypatch.setattr(O, "silu", good_silu)

    good_layer = O.layer_forward

    def layer_attends_everything(h, pos, W, Kc, Vc, dm, attend_locked=True):   # ablation flag ignored
        return good_layer(h, pos, W, Kc, Vc, dm)
    monkeypatch.setattr(O, "layer_forward", layer_attends_everything)
    _expect_fail(pin_no_kv_cache_ablation)
    monkeypatch.setattr(O, "layer_forward", good_layer)
