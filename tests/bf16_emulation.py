"""CPU model of the rounding the HIP path does when it stores in bfloat16.

Test infrastructure: it derives the floating-point bounds of the bf16 parity
tests.  It runs the same SureLock layer / model computation as the oracle, in
float64, but rounds a value to bfloat16 (round to nearest even, through fp32)
at each point where the kernels store that value in bf16:

  * the RMSNorm output x that feeds every projection (pre-attention, pre-FFN,
    final norm before the LM head);
  * q, k and v after RoPE (k and v are also what the K/V cache holds);
  * the attention probabilities P = exp(s - m) that feed the P.V product
    (the row sum l is taken from the unrounded values), and the attention
    output o;
  * the SwiGLU activation SiLU(x W_g) * (x W_u);
  * the logits.
The residual stream stays unrounded (the kernels keep it in fp32).  With
rnd=False nothing is rounded and the model equals the oracle's float64 step;
tests/test_bf16_emulation.py pins that.  The deviation of the rounded model
from the oracle is what bf16 storage alone costs; a correct kernel matches it
in distribution, and a test's bound is a stated margin over it.

Nothing here imports the oracle or the HIP library.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 -> bfloat16 (round to nearest even) -> float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.float32)
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _r(x, rnd):
    return round_bf16(x) if rnd else x


def _mm(a, b):
    """a @ b in float64 through torch (multithreaded BLAS)."""
    ta = torch.from_numpy(a) if a.flags.c_contiguous or a.flags.f_contiguous else torch.from_numpy(a.copy())
    tb = torch.from_numpy(b) if b.flags.c_contiguous or b.flags.f_contiguous else torch.from_numpy(b.copy())
    return (ta @ tb).numpy()


def _rmsnorm(h, eps):
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def _rope(x, pos, theta):
    Dh = x.shape[-1]
    half = Dh // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / Dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _silu(g):
    e = np.exp(-np.abs(g))
    return g * np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def attention(q, Kc, Vc, scale, rnd=True):
    """q [M][H][Dh], Kc/Vc [N][H][Dh] -> o [M][H][Dh]; P rounded before P.V, l from unrounded P,
    output rounded."""
    qh = np.transpose(q, (1, 0, 2))
    kh = np.transpose(Kc, (1, 2, 0))
    vh = np.transpose(Vc, (1, 0, 2))
    s = np.stack([_mm(qh[h], kh[h]) for h in range(qh.shape[0])]) * scale
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    l = p.sum(axis=-1, keepdims=True)
    pr = _r(p, rnd)
    o = np.stack([_mm(pr[h], vh[h]) for h in range(pr.shape[0])]) / l
    return _r(np.transpose(o, (1, 0, 2)), rnd)


@dataclass
class Dims:
    d: int
    n_heads: int
    head_dim: int
    ffn: int
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0


def layer(h, pos, W, Kc, Vc, dm: Dims, rnd=True, attend_locked=True):
    """One block for the active rows of one sequence.  h [M][d] float64 residual rows; W float64
    [out][in]; Kc, Vc [N][H][Dh] updated in place at pos (with the stored, rounded k and v)."""
    M = h.shape[0]
    H, Dh = dm.n_heads, dm.head_dim
    x = _r(_rmsnorm(h, dm.rms_eps), rnd)
    q = _r(_rope(_mm(x, W["wq"].T).reshape(M, H, Dh), pos, dm.rope_theta), rnd)
    k = _r(_rope(_mm(x, W["wk"].T).reshape(M, H, Dh), pos, dm.rope_theta), rnd)
    v = _r(_mm(x, W["wv"].T).reshape(M, H, Dh), rnd)
    Kc[pos] = k
    Vc[pos] = v
    if attend_locked:
        o = attention(q, Kc, Vc, 1.0 / np.sqrt(Dh), rnd)
    else:
        o = attention(q, Kc[pos], Vc[pos], 1.0 / np.sqrt(Dh), rnd)
    h = h + _mm(o.reshape(M, H * Dh), W["wo"].T)
    x2 = _r(_rmsnorm(h, dm.rms_eps), rnd)
    a = _r(_silu(_mm(x2, W["wg"].T)) * _mm(x2, W["wu"].T), rnd)
    return h + _mm(a, W["wd"].T)


def logits(h, head, eps, rnd=True, f32=False):
    """Final RMSNorm and LM head: z = bf16(bf16(rmsnorm(h)) W_out^T).  f32=True takes the product in
    float32 (used at full vocabulary, where the float64 product would dominate the test's time; the
    fp32 rounding is far below bf16's)."""
    x = _r(_rmsnorm(h, eps), rnd)
    if f32:
        z = (torch.from_numpy(x.astype(np.float32)) @ torch.from_numpy(np.asarray(head, np.float32)).T)
        z = z.numpy().astype(np.float64)
    else:
        z = _mm(x, np.asarray(head).T)
    return _r(z, rnd)


def step_rows(h_rows, act_idx, act_off, layers_fn, n_layers, kc, vc, dm: Dims, rnd=True, attend_locked=True):
    """The layers of one SureLock step over the active rows of B sequences (compact order).
    kc / vc: per layer float64 [B][N][H][Dh], updated in place.  layers_fn(l) -> float64 weights."""
    h = np.array(h_rows, dtype=np.float64, copy=True)
    B = len(act_off) - 1
    for l in range(n_layers):
        W = layers_fn(l)
        for b in range(B):
            s = slice(act_off[b], act_off[b + 1])
            if act_off[b + 1] > act_off[b]:
                h[s] = layer(h[s], act_idx[s], W, kc[l][b], vc[l][b], dm, rnd, attend_locked)
    return h


@dataclass
class ErrStats:
    rel_l2: float
    rms: float
    max: float
    n: int


def err_stats(got, ref) -> ErrStats:
    d = np.asarray(got, np.float64) - np.asarray(ref, np.float64)
    nr = float(np.linalg.norm(ref))
    return ErrStats(float(np.linalg.norm(d)) / (nr if nr > 0 else 1.0),
                    float(np.sqrt(np.mean(d * d))) if d.size else 0.0,
                    float(np.abs(d).max()) if d.size else 0.0, int(d.size))


# Margin of a bf16 kernel result over the emulated error: the two errors are independent
# realisations of the same roundings, so their relative L2 and their maxima agree within a few
# percent on the large cases; the margin also covers small cases (a few hundred elements), where
# both statistics fluctuate.
MARGIN = 1.25
# Floor of the max-abs bound in emulated standard deviations: on a case of a few hundred elements
# the emulation's own maximum can sit well below the tail the kernel may draw.
MAX_FLOOR_SIGMAS = 5.0


def bounds(emu: ErrStats, margin: float = MARGIN):
    """(relative L2 bound, max-abs bound) for a kernel result, from the emulated error."""
    return margin * emu.rel_l2, margin * max(emu.max, MAX_FLOOR_SIGMAS * emu.rms)


def check(got, ref, emu: ErrStats, what: str, margin: float = MARGIN) -> ErrStats:
    """Assert that got deviates from ref no more than the emulation (with the margin) does."""
    g = err_stats(got, ref)
    l2_b, mx_b = bounds(emu, margin)
    assert g.rel_l2 <= l2_b, "%s: relative L2 %.3e > %.3e (emulated %.3e)" % (what, g.rel_l2, l2_b, emu.rel_l2)
    assert g.max <= mx_b, "%s: max |d| %.3e > %.3e (emulated max %.3e, rms %.3e)" % (
        what, g.max, mx_b, emu.max, emu.rms)
    return g
