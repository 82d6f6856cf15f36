"""Independent dense reference used only to pin the oracle.

A plain bidirectional transformer evaluated on ALL N positions with PyTorch
CPU float64 library operators (rms_norm, scaled_dot_product_attention, silu,
matmul) and RoPE written as complex multiplication.  The SureLock pages state
that with no locking the sampler is the ordinary one (paperdance abstract:
"relative to the same sampler without locking"), so the oracle's step with
eps = 0 / M = N must equal this dense forward.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """x [N][H][Dh]; pair (x_j, x_{j+Dh/2}) as the complex number x_j + i x_{j+Dh/2}."""
    Dh = x.shape[-1]
    half = Dh // 2
    freqs = torch.pow(torch.tensor(theta, dtype=torch.float64),
                      -torch.arange(0, Dh, 2, dtype=torch.float64) / Dh)
    rot = torch.polar(torch.ones(len(pos), half, dtype=torch.float64),
                      pos.to(torch.float64)[:, None] * freqs[None, :])[:, None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def dense_block(h: torch.Tensor, W: dict, n_heads: int, eps: float, theta: float, pos=None):
    """h [N][d] -> (h_out [N][d], k [N][H][Dh], v [N][H][Dh]); pos = the rows' RoPE positions
    (default 0 .. N-1)."""
    N, d = h.shape
    Dh = d // n_heads
    pos = torch.arange(N) if pos is None else torch.as_tensor(np.asarray(pos, dtype=np.int64))
    x = F.rms_norm(h, (d,), eps=eps)
    q = (x @ _t(W["wq"]).T).view(N, n_heads, Dh)
    k = (x @ _t(W["wk"]).T).view(N, n_heads, Dh)
    v = (x @ _t(W["wv"]).T).view(N, n_heads, Dh)
    q = rope_complex(q, pos, theta)
    k = rope_complex(k, pos, theta)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    h = h + o.transpose(0, 1).reshape(N, d) @ _t(W["wo"]).T
    x2 = F.rms_norm(h, (d,), eps=eps)
    h = h + (F.silu(x2 @ _t(W["wg"]).T) * (x2 @ _t(W["wu"]).T)) @ _t(W["wd"]).T
    return h, k, v


def dense_logits(tok: np.ndarray, embed, layers: list, lm_head, n_heads: int, eps: float, theta: float):
    """Full-sequence forward of one sequence: tok [N] -> logits [N][V] (float64 numpy)."""
    h = _t(embed)[torch.as_tensor(np.asarray(tok, dtype=np.int64))]
    for W in layers:
        h, _, _ = dense_block(h, W, n_heads, eps, theta)
    d = h.shape[1]
    return (F.rms_norm(h, (d,), eps=eps) @ _t(lm_head).T).numpy()
