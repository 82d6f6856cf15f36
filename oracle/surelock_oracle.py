"""Oracle: a plain, slow CPU reference of the SureLock decoding step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
call it.  It shares no code with the HIP library and never imports it.

All arithmetic is NumPy float64 on the exact values the GPU receives (bf16
bit patterns are widened exactly), with no intermediate rounding.  Each
function cites the passage of the SureLock pages (arXiv 2602.06412 summaries)
that defines what it computes.  Where the pages leave a step open, the
reading taken is stated in the docstring.

Pins (the tests that tie this oracle to something other than itself) live in
tests/test_oracle_pins.py.  Every function below is pinned; the lock
trajectories a trained LLaDA-8B would produce are not reproducible here
(parity unpinned for that, by construction: no weights exist).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable

import numpy as np


# ------------------------------------------------------------------ storage
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a storage array (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ------------------------------------------------------------------ A_t / L_t
def active_set(locked: np.ndarray, B: int, N: int):
    """Active set A_t: the positions not in the locked set L_t, ascending, per sequence.

    SureLock keeps an active set (computed) and a locked set (skipped, K/V
    cached) at every step (zhaoyang97 notes, "整体框架" framework section).
    Returns (act_idx int32 [M_tot] positions within their sequence,
    act_off int32 [B+1] offsets of each sequence's slice).
    """
    lk = np.asarray(locked).reshape(B, N)
    parts = [np.flatnonzero(lk[b] == 0) for b in range(B)]
    act_off = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        act_off[b + 1] = act_off[b] + len(parts[b])
    act_idx = np.concatenate(parts).astype(np.int32) if B else np.zeros(0, np.int32)
    return act_idx, act_off


def seq_of_rows(act_off: np.ndarray) -> np.ndarray:
    """Sequence index of every row of a compact active list."""
    B = len(act_off) - 1
    return np.repeat(np.arange(B), np.diff(act_off))


# ------------------------------------------------------------------ posterior statistics
def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = z.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))[..., 0]


@dataclass
class PosteriorStats:
    kl: np.ndarray      # D_t = KL(p_t || p_{t-1}) per row (nats); +inf without a previous posterior
    u: np.ndarray       # 1 - max_v p_t(v)
    lse: np.ndarray     # log-sum-exp of the current logits
    argmax: np.ndarray  # argmax over v != mask id (lowest id on ties)
    conf: np.ndarray    # p_t(argmax)


def posterior_stats(z: np.ndarray, y: np.ndarray | None, mask_id: int = -1,
                    chunk: int = 64) -> PosteriorStats:
    """Per-row posterior, step KL and confidence statistic.

    p_t = softmax(z) over the vocabulary.  The lock criterion is the step KL
    D_t = KL(p_t || p_{t-1}) = sum_v p_t(v) (log p_t(v) - log p_{t-1}(v))
    (zhaoyang97 notes, "锁定判据：步间 KL 散度"; gist.science/it §2, lock
    criterion).  Natural log.  The confidence statistic is
    u_t = 1 - max_v p_t(v) (zhaoyang97 notes, "可选置信度门控").
    Without a previous posterior (first step) KL is +inf, so nothing locks.
    The sampler's argmax excludes the [MASK] id; the softmax normalisation
    includes it.  z, y: float64 [M][V] (y may be None).
    """
    M = z.shape[0]
    kl = np.full(M, np.inf)
    u = np.empty(M)
    lse = np.empty(M)
    am = np.empty(M, dtype=np.int64)
    conf = np.empty(M)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        zc = np.asarray(z[r0:r1], dtype=np.float64)
        a = logsumexp_rows(zc)
        logp = zc - a[:, None]
        p = np.exp(logp)
        lse[r0:r1] = a
        u[r0:r1] = 1.0 - np.exp(zc.max(axis=1) - a)
        if y is not None:
            yc = np.asarray(y[r0:r1], dtype=np.float64)
            logq = yc - logsumexp_rows(yc)[:, None]
            kl[r0:r1] = (p * (logp - logq)).sum(axis=1)
        zm = zc
        if 0 <= mask_id < zc.shape[1]:
            zm = zc.copy()
            zm[:, mask_id] = -np.inf
        k = zm.argmax(axis=1)
        am[r0:r1] = k
        conf[r0:r1] = np.exp(zc[np.arange(r1 - r0), k] - a)
    return PosteriorStats(kl, u, lse, am, conf)


# ------------------------------------------------------------------ gate, lock, compaction
def gate_rank(m: float, count: int) -> int:
    """Rank of the gate quantile: floor(m*(count-1)), m taken as the float32 value given."""
    return int(np.floor(float(np.float32(m)) * (count - 1)))


def gate_threshold(u: np.ndarray, m: float) -> float:
    """q_m(u_t): the m-quantile of u over the active rows of one sequence.

    The gate compares u against a quantile of u_t over the active tokens
    (zhaoyang97 notes, "可选置信度门控"; gist.science/it §2: a percentile
    among the active tokens).  Estimator (the pages do not fix one): lower
    nearest rank, element floor(m*(M-1)) of u sorted ascending.
    """
    if len(u) == 0:
        return np.inf
    return float(np.sort(u)[gate_rank(m, len(u))])


@dataclass
class LockResult:
    locked: np.ndarray      # uint8 [B*N] after the update
    new_lock: np.ndarray    # bool [M_tot], rows that locked at this step
    gate_thr: np.ndarray    # float64 [B] (inf when the gate is off)
    act_idx: np.ndarray     # next active list
    act_off: np.ndarray


def lock_update(locked: np.ndarray, act_idx: np.ndarray, act_off: np.ndarray, B: int, N: int,
                kl: np.ndarray, u: np.ndarray, cand: np.ndarray | None, eps: float,
                gate_m: float, have_prev: bool) -> LockResult:
    """Permanent, monotone lock update followed by compaction of the next active set.

    A position locks when its step KL is at most eps (formula "≤ ε",
    zhaoyang97 notes, "锁定判据"), AND-ed with the optional gate
    u <= q_m(u_t) (zhaoyang97 notes, "可选置信度门控"; gist.science/it §2:
    two conditions).  Only unmasked positions may lock (paperdance abstract:
    "the posterior at an unmasked position"); cand marks them (None = every
    active row).  Locks are never undone, so the active set only shrinks
    (zhaoyang97 notes, "永久锁定机制" and "关键发现").
    Readings: eps <= 0 disables locking; gate_m < 0 disables the gate;
    without a previous posterior nothing locks.  The notes page's ablations
    (zhaoyang97 notes, 消融实验) are settings of the same rule: KL only is
    the gate off; confidence gate only is eps = +inf (the KL test always
    passes) with the gate on.
    """
    locked = np.array(locked, dtype=np.uint8, copy=True)
    M = len(act_idx)
    new_lock = np.zeros(M, dtype=bool)
    thr = np.full(B, np.inf)
    rows_seq = seq_of_rows(act_off)
    glob = rows_seq * N + act_idx.astype(np.int64)
    if gate_m >= 0:
        for b in range(B):
            sl = slice(act_off[b], act_off[b + 1])
            thr[b] = gate_threshold(u[sl], gate_m)
    if eps > 0 and have_prev and M:
        is_cand = np.ones(M, dtype=bool) if cand is None else (np.asarray(cand)[glob] != 0)
        ok = is_cand & (kl <= eps)
        if gate_m >= 0:
            ok &= u <= thr[rows_seq]
        new_lock = ok
        locked[glob[ok]] = 1
    nidx, noff = active_set(locked, B, N)
    return LockResult(locked, new_lock, thr, nidx, noff)


# ------------------------------------------------------------------ transformer pieces
def rmsnorm(h: np.ndarray, eps: float) -> np.ndarray:
    """x = h / sqrt(mean(h^2) + eps) (unit gain)."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half form, absolute position = sequence index.

    x: [M][H][Dh]; pair j (j < Dh/2) is (x_j, x_{j+Dh/2}), rotated by the
    angle pos * theta^(-2j/Dh).
    """
    Dh = x.shape[-1]
    half = Dh // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / Dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, scale: float) -> np.ndarray:
    """Bidirectional softmax attention of M active queries over all N cached keys.

    o_i = sum_j softmax_j(q_i . K[j] * scale) V[j], per head, no mask: every
    active row attends to every position, locked ones through their cached
    K/V (zhaoyang97 notes, "永久锁定机制": K^all[L_t] <- C.k[L_t]); the cost is
    O(M N d) instead of O(N^2 d) (paperdance abstract).
    q: [M][H][Dh]; Kc, Vc: [N][H][Dh].  Returns [M][H][Dh].
    """
    qh = np.transpose(q, (1, 0, 2))            # H M Dh
    kh = np.transpose(Kc, (1, 2, 0))           # H Dh N
    vh = np.transpose(Vc, (1, 0, 2))           # H N Dh
    s = (qh @ kh) * scale                      # H M N
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.transpose(p @ vh, (1, 0, 2))


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g), evaluated without overflow for either sign."""
    e = np.exp(-np.abs(g))
    return g * np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


@dataclass
class OracleDims:
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float


def layer_forward(h: np.ndarray, pos: np.ndarray, W: dict, Kc: np.ndarray, Vc: np.ndarray,
                  dm: OracleDims, attend_locked: bool = True) -> np.ndarray:
    """One transformer block for the active rows of one sequence; updates the cache in place.

    Active rows compute their Q projection and FFN; their fresh K/V are written
    into the layer's cache at their positions, and their queries attend over
    all N cached rows (zhaoyang97 notes, "永久锁定机制"; gist.science/it §2,
    lock action: K/V cached for every layer, Q projection and FFN skipped for
    locked rows).  Block: pre-RMSNorm, QKV + RoPE, attention, O projection +
    residual, pre-RMSNorm, SwiGLU FFN + residual.
    attend_locked=False is the "no KV cache" ablation of the notes page
    (zhaoyang97 notes, 消融实验): locked positions cannot be attended, so the
    active rows attend over the active positions only (their fresh K/V).
    h: [M][d] float64; W: float64 [out][in] matrices; Kc, Vc: [N][H][Dh].
    """
    M = h.shape[0]
    H, Dh = dm.n_heads, dm.head_dim
    x = rmsnorm(h, dm.rms_eps)
    q = (x @ W["wq"].T).reshape(M, H, Dh)
    k = (x @ W["wk"].T).reshape(M, H, Dh)
    v = (x @ W["wv"].T).reshape(M, H, Dh)
    q = rope(q, pos, dm.rope_theta)
    k = rope(k, pos, dm.rope_theta)
    Kc[pos] = k
    Vc[pos] = v
    if attend_locked:
        o = attention(q, Kc, Vc, 1.0 / np.sqrt(Dh))
    else:
        o = attention(q, Kc[pos], Vc[pos], 1.0 / np.sqrt(Dh))
    o = o.reshape(M, H * Dh)
    h = h + o @ W["wo"].T
    x2 = rmsnorm(h, dm.rms_eps)
    a = silu(x2 @ W["wg"].T) * (x2 @ W["wu"].T)
    return h + a @ W["wd"].T


# ------------------------------------------------------------------ one SureLock step
@dataclass
class OracleModel:
    dims: OracleDims
    n_layers: int
    layer: Callable[[int], dict]          # l -> dict of float64 [out][in] matrices
    embed: np.ndarray | None = None       # float64 [V][d]
    lm_head: np.ndarray | None = None     # float64 [V][d]


@dataclass
class OracleState:
    B: int
    N: int
    t: int
    locked: np.ndarray                    # uint8 [B*N]
    kc: list                              # per layer float64 [B][N][H][Dh]
    vc: list
    tok: np.ndarray | None = None         # int32 [B*N]
    cand: np.ndarray | None = None        # uint8 [B*N]; None = every active row is a candidate
    h_in: np.ndarray | None = None        # float64 [B*N][d] layer-0 input rows (instead of embed[tok])
    post: np.ndarray | None = None        # float64 [B*N][V] logits of each row's last computed step
    lock_step: np.ndarray | None = None   # int32 [B*N], -1 = not locked


@dataclass
class StepOut:
    act_idx: np.ndarray
    act_off: np.ndarray
    h: np.ndarray                         # [M_tot][d] final hidden rows
    logits: np.ndarray | None             # [M_tot][V]
    stats: PosteriorStats | None
    lock: LockResult | None


def step(model: OracleModel, st: OracleState, eps: float, gate_m: float,
         do_lock: bool = True, mask_id: int = -1, prev_logits: np.ndarray | None = None,
         attend_locked: bool = True) -> StepOut:
    """One SureLock iteration on the oracle state (modified in place).

    1. gather A_t; 2. layer-0 input for the active rows (embedding of the
    current token, or given hidden rows); 3. every layer on the active rows
    only, refreshing their cache rows; 4. final RMSNorm and LM head;
    5. posterior statistics against the previous posterior; 6-7. gate and
    monotone lock update; 8. posterior store: only active rows are written,
    so a locked row keeps the posterior of its lock step (zhaoyang97 notes,
    "永久锁定机制": p_hat_t = p_{t*}); 9. next active set.
    prev_logits ([M_tot][V]) overrides st.post as the previous posterior.
    attend_locked=False: the no-KV-cache ablation (see layer_forward).
    """
    dm = model.dims
    B, N = st.B, st.N
    act_idx, act_off = active_set(st.locked, B, N)
    M = len(act_idx)
    rows_seq = seq_of_rows(act_off)
    glob = rows_seq * N + act_idx.astype(np.int64)
    if st.h_in is not None:
        h = np.asarray(st.h_in[glob], dtype=np.float64)
    else:
        h = model.embed[st.tok[glob]].astype(np.float64)
    for l in range(model.n_layers):
        W = model.layer(l)
        for b in range(B):
            sl = slice(act_off[b], act_off[b + 1])
            if act_off[b + 1] > act_off[b]:
                h[sl] = layer_forward(h[sl], act_idx[sl], W, st.kc[l][b], st.vc[l][b], dm, attend_locked)
    out = StepOut(act_idx, act_off, h, None, None, None)
    if model.lm_head is None:
        return out
    z = rmsnorm(h, dm.rms_eps) @ model.lm_head.T
    out.logits = z
    have_prev = st.t > 0
    y = None
    if have_prev:
        y = prev_logits if prev_logits is not None else st.post[glob]
    stats = posterior_stats(z, y, mask_id)
    out.stats = stats
    if st.post is None:
        st.post = np.full((B * N, dm.vocab), np.nan)
    st.post[glob] = z
    if do_lock:
        lr = lock_update(st.locked, act_idx, act_off, B, N, stats.kl, stats.u, st.cand,
                         eps, gate_m, have_prev)
        if st.lock_step is not None:
            st.lock_step[glob[lr.new_lock]] = st.t
        st.locked = lr.locked
        out.lock = lr
    return out


def sampler_unmask(tok: np.ndarray, cand: np.ndarray, act_idx: np.ndarray, act_off: np.ndarray,
                   N: int, argmax: np.ndarray, conf: np.ndarray, mask_id: int, k: int):
    """Iterative-unmasking sampler step (baseline MDLM sampler; paperdance abstract).

    Per sequence, among the active rows whose token is [MASK], the k with the
    largest confidence p_t(argmax) are unmasked to their argmax token (ties:
    lowest position).  Unmasked positions become lock candidates from the next
    step on.  Returns the global positions unmasked.
    """
    B = len(act_off) - 1
    picked = []
    for b in range(B):
        rows = np.arange(act_off[b], act_off[b + 1])
        pos = act_idx[rows].astype(np.int64) + b * N
        msk = tok[pos] == mask_id
        rows, pos = rows[msk], pos[msk]
        if len(rows) == 0:
            continue
        order = np.lexsort((pos, -conf[rows]))[:k]
        for o in order:
            tok[pos[o]] = int(argmax[rows[o]])
            cand[pos[o]] = 1
            picked.append(int(pos[o]))
    return picked


@dataclass
class LoopRecord:
    t: int
    M: int
    new_locks: int
    act_idx: np.ndarray
    act_off: np.ndarray
    locked: np.ndarray
    tok: np.ndarray
    logits: np.ndarray
    stats: PosteriorStats


def run_loop(model: OracleModel, tok0: np.ndarray, B: int, N: int, T: int, eps: float,
             gate_m: float, unmask_k: int, on_step: Callable | None = None,
             attend_locked: bool = True) -> list:
    """The MDLM sampler loop with SureLock: T steps of (SureLock step, unmask k).

    Candidates at step t are the positions already unmasked in the step's
    input tokens (prompt included); masked positions never lock.
    """
    dm = model.dims
    mask_id = dm.vocab - 1
    st = OracleState(B=B, N=N, t=0, locked=np.zeros(B * N, np.uint8),
                     kc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(model.n_layers)],
                     vc=[np.zeros((B, N, dm.n_heads, dm.head_dim)) for _ in range(model.n_layers)],
                     tok=np.array(tok0, dtype=np.int32, copy=True),
                     cand=(np.asarray(tok0) != mask_id).astype(np.uint8),
                     lock_step=np.full(B * N, -1, np.int32))
    recs = []
    for t in range(T):
        st.t = t
        out = step(model, st, eps, gate_m, True, mask_id, attend_locked=attend_locked)
        sampler_unmask(st.tok, st.cand, out.act_idx, out.act_off, N, out.stats.argmax,
                       out.stats.conf, mask_id, unmask_k)
        rec = LoopRecord(t, len(out.act_idx), int(out.lock.new_lock.sum()), out.act_idx, out.act_off,
                         st.locked.copy(), st.tok.copy(), out.logits, out.stats)
        recs.append(rec)
        if on_step is not None:
            on_step(rec, st)
    return recs


def layer_flops(dm: OracleDims, M: int, N: int) -> float:
    """Algorithmic FLOPs of one layer step for M active rows against N keys.

    QKV 6Md^2, O 2Md^2, FFN 6MdF, attention 4MNd (scores and weighted sum);
    the O(MNd) attention and O(Md^2) FFN terms of the pages' cost model.
    """
    d, F = dm.d, dm.ffn
    return float(M) * (8.0 * d * d + 6.0 * d * F + 4.0 * N * d)
