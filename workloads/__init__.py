"""Seeded synthetic inputs for the SureLock decoding step.

This module only draws random numbers, rounds them to the storage type and
picks seeded subsets.  It holds none of the method's arithmetic, so both the
CPU oracle and the GPU tests can use it without sharing any computation.

Shapes and distributions follow the workloads the SureLock pages describe
(LLaDA-8B layer shape: d=4096, 32 heads x 128, SwiGLU 12288, vocabulary
126464) with random weights, since no trained weights or datasets exist here.

Seeds (one root per purpose, child streams via SeedSequence spawn keys):
  0 weights, 1 activations / logits, 2 caches, 3 active / locked sets,
  4 "+8" spike tokens, 5 logit drift, 6 prompt tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

SEED_WEIGHTS = 0
SEED_ACT = 1
SEED_CACHE = 2
SEED_SETS = 3
SEED_SPIKE = 4
SEED_DRIFT = 5
SEED_PROMPT = 6


def rng(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, key...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


# ---------------------------------------------------------------- storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even), returned as uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draw -> storage array (uint16 bf16 bits, or float32)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact float64 values (for host-side inspection only)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ---------------------------------------------------------------- model dims
@dataclass(frozen=True)
class Dims:
    n_layers: int
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str  # "bf16" or "f32": storage of weights, activations, caches, logits
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    weight_std: float = 0.02

    @property
    def mask_id(self) -> int:
        return self.vocab - 1


# Tiny 2-layer fp32 model of the sampler-loop workload.
TINY = Dims(n_layers=2, d=128, n_heads=4, head_dim=32, ffn=384, vocab=512, dtype="f32")
# One LLaDA-8B-shaped layer (bf16).
LLADA_LAYER = Dims(n_layers=1, d=4096, n_heads=32, head_dim=128, ffn=12288, vocab=126464, dtype="bf16")
# Whole 32-layer LLaDA-8B-shaped model (bf16).
LLADA_8B = replace(LLADA_LAYER, n_layers=32)

LAYER_MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def layer_shapes(dm: Dims) -> dict:
    """Weight shapes, stored [out_features][in_features] (row = output column)."""
    d, f = dm.d, dm.ffn
    return {"wq": (d, d), "wk": (d, d), "wv": (d, d), "wo": (d, d),
            "wg": (f, d), "wu": (f, d), "wd": (d, f)}


def layer_weights(dm: Dims, layer: int, seed: int = SEED_WEIGHTS) -> dict:
    """Storage-format weights of one layer, N(0, weight_std), seeded per (layer, matrix)."""
    out = {}
    for mi, (name, shape) in enumerate(layer_shapes(dm).items()):
        out[name] = to_storage(normal(rng(seed, layer, mi), shape, dm.weight_std), dm.dtype)
    return out


def embed_weights(dm: Dims, seed: int = SEED_WEIGHTS) -> np.ndarray:
    return to_storage(normal(rng(seed, 1000, 0), (dm.vocab, dm.d), dm.weight_std), dm.dtype)


def lm_head_weights(dm: Dims, seed: int = SEED_WEIGHTS) -> np.ndarray:
    return to_storage(normal(rng(seed, 1000, 1), (dm.vocab, dm.d), dm.weight_std), dm.dtype)


# ---------------------------------------------------------------- sets
def choose_active(N: int, M: int, seed: int = SEED_SETS, key: int = 0) -> np.ndarray:
    """M distinct positions of [0, N), uniformly without replacement, ascending (int32)."""
    perm = rng(seed, key).permutation(N)
    return np.sort(perm[:M]).astype(np.int32)


def locked_from_active(N: int, act: np.ndarray) -> np.ndarray:
    locked = np.ones(N, dtype=np.uint8)
    locked[act] = 0
    return locked


def random_mask(n: int, p_locked: float, seed: int, key: int = 0) -> np.ndarray:
    return (rng(seed, key).random(n) < p_locked).astype(np.uint8)


# ---------------------------------------------------------------- KL-lock pass workload
@dataclass
class KLLockCase:
    B: int
    N: int
    V: int
    locked: np.ndarray     # uint8 [B*N], lock mask before the pass
    act_idx: np.ndarray    # int32 [M_tot], ascending positions per sequence
    act_off: np.ndarray    # int32 [B+1]
    cur: np.ndarray        # storage [M_tot][V], logits of the active rows at step t
    prev: np.ndarray       # storage [M_tot][V], logits of the same rows at step t-1
    cand: np.ndarray | None  # uint8 [B*N] or None (= every active row is a candidate)
    dtype: str

    @property
    def M_tot(self) -> int:
        return int(self.act_off[-1])


def kl_lock_mask(N: int, B: int = 1, locked_frac=0.6, key: int = 0):
    """floor(locked_frac*N) positions per sequence locked by a seeded permutation.

    locked_frac is one fraction for every sequence or a sequence of B of them.
    Returns (locked uint8 [B*N], act_idx int32 [M_tot], act_off int32 [B+1])."""
    fr = np.broadcast_to(np.asarray(locked_frac, dtype=np.float64), (B,))
    locked = np.zeros(B * N, dtype=np.uint8)
    acts, offs = [], [0]
    for b in range(B):
        perm = rng(SEED_SETS, key, b).permutation(N)
        nl = int(np.floor(fr[b] * N))
        locked[b * N + perm[:nl]] = 1
        act = np.sort(perm[nl:]).astype(np.int32)
        acts.append(act)
        offs.append(offs[-1] + len(act))
    act_idx = np.concatenate(acts).astype(np.int32) if B else np.zeros(0, np.int32)
    return locked, act_idx, np.asarray(offs, dtype=np.int32)


def kl_lock_case(N: int = 4096, V: int = 126464, B: int = 1, locked_frac=0.6,
                 spike_frac: float = 0.7, spike: float = 8.0, std: float = 2.0,
                 drift: float = 0.05, dtype: str = "bf16", cand_frac: float | None = None,
                 key: int = 0) -> KLLockCase:
    """Logits for the KL-lock pass.

    Per sequence: floor(locked_frac*N) positions already locked (seeded
    permutation); cur ~ N(0, std^2) per entry; round(spike_frac*N) seeded rows
    get +spike at one seeded token (same token in both steps); prev = cur +
    N(0, drift^2).  Only active rows are materialised.
    """
    locked, act_idx, act_off = kl_lock_mask(N, B, locked_frac, key)
    acts = [act_idx[act_off[b]:act_off[b + 1]] for b in range(B)]
    spike_rows = np.zeros(B * N, dtype=bool)
    spike_tok = np.zeros(B * N, dtype=np.int64)
    for b in range(B):
        gs = rng(SEED_SPIKE, key, b)
        rows = gs.permutation(N)[: int(round(spike_frac * N))]
        spike_rows[b * N + rows] = True
        spike_tok[b * N:(b + 1) * N] = gs.integers(0, V, size=N)
    M = len(act_idx)
    glob = np.concatenate([b * N + a for b, a in enumerate(acts)]) if M else np.zeros(0, np.int64)
    cur = np.empty((M, V), dtype=np.uint16 if dtype == "bf16" else np.float32)
    prev = np.empty_like(cur)
    CH = 256
    for r0 in range(0, M, CH):
        r1 = min(M, r0 + CH)
        c32 = normal(rng(SEED_ACT, key, r0), (r1 - r0, V), std)
        rows = glob[r0:r1]
        sp = spike_rows[rows]
        c32[np.nonzero(sp)[0], spike_tok[rows[sp]]] += np.float32(spike)
        p32 = c32 + normal(rng(SEED_DRIFT, key, r0), (r1 - r0, V), drift)
        cur[r0:r1] = to_storage(c32, dtype)
        prev[r0:r1] = to_storage(p32, dtype)
    cand = None
    if cand_frac is not None:
        cand = (rng(SEED_SETS, key, 9999).random(B * N) < cand_frac).astype(np.uint8)
    return KLLockCase(B, N, V, locked, act_idx, act_off, cur, prev, cand, dtype)


# ---------------------------------------------------------------- layer-step workload
@dataclass
class LayerCase:
    dims: Dims
    B: int
    N: int
    act_idx: np.ndarray    # int32 [M_tot]
    act_off: np.ndarray    # int32 [B+1]
    h_in: np.ndarray       # storage [B*N][d]: hidden rows (only active rows are read)
    k_cache: np.ndarray    # storage [B][N][H][Dh] (one layer); locked rows hold the cached K
    v_cache: np.ndarray

    @property
    def M_tot(self) -> int:
        return int(self.act_off[-1])


def layer_case(dims: Dims, N: int, Ms, key: int = 0) -> LayerCase:
    """Hidden rows N(0,1), cached K/V N(0,1), active sets uniform without replacement."""
    Ms = [Ms] if np.isscalar(Ms) else list(Ms)
    B = len(Ms)
    acts = [choose_active(N, int(M), SEED_SETS, key * 64 + b) for b, M in enumerate(Ms)]
    act_idx = np.concatenate(acts).astype(np.int32) if B else np.zeros(0, np.int32)
    act_off = np.concatenate([[0], np.cumsum([len(a) for a in acts])]).astype(np.int32)
    H, Dh, d = dims.n_heads, dims.head_dim, dims.d
    h_in = to_storage(normal(rng(SEED_ACT, key, 7), (B * N, d), 1.0), dims.dtype)
    kc = to_storage(normal(rng(SEED_CACHE, key, 0), (B, N, H, Dh), 1.0), dims.dtype)
    vc = to_storage(normal(rng(SEED_CACHE, key, 1), (B, N, H, Dh), 1.0), dims.dtype)
    return LayerCase(dims, B, N, act_idx, act_off, h_in, kc, vc)


def ragged_fracs(B: int, lo: float = 0.05, hi: float = 0.8, key: int = 0) -> np.ndarray:
    """Per-sequence active fractions drawn uniformly from [lo, hi]."""
    return rng(SEED_SETS, 500, key).uniform(lo, hi, size=B)


def ragged_ms(B: int, N: int, lo: float = 0.05, hi: float = 0.8, key: int = 0) -> list:
    return [int(round(f * N)) for f in ragged_fracs(B, lo, hi, key)]


# ---------------------------------------------------------------- sampler-loop workload
def prompt_tokens(dims: Dims, B: int, N: int, n_prompt: int, key: int = 0) -> np.ndarray:
    """int32 [B*N]: n_prompt ids uniform on [0, V-1) followed by [MASK] (= V-1)."""
    tok = np.full((B, N), dims.mask_id, dtype=np.int32)
    tok[:, :n_prompt] = rng(SEED_PROMPT, key).integers(0, dims.vocab - 1, size=(B, n_prompt))
    return tok.reshape(-1)
