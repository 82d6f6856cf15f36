"""Device buffers of a SureLock model and sampler state (allocation and marshalling only).

DeviceModel holds the weights and the RoPE table on the GPU and the sl_model
struct that points at them; DeviceState holds the per-sequence state of the
sampler (tokens, lock mask, active list, per-layer K/V caches, the
double-buffered posterior store and the per-row statistics) and the sl_state
struct.  All arithmetic happens in libsurelock.so.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import surelock as S


def _dptr(t):
    return None if t is None else t.data_ptr()


class DeviceModel:
    def __init__(self, *, dtype: torch.dtype, n_layers: int, d: int, n_heads: int, head_dim: int, ffn: int,
                 vocab: int, rms_eps: float, rope_theta: float, layers: list, embed=None, lm_head=None,
                 rope_n: int, device="cuda"):
        self.dtype = dtype
        self.layers = layers                       # list of dict name -> device tensor [out][in]
        self.embed = embed
        self.lm_head = lm_head
        self.dims = dict(n_layers=n_layers, d=d, n_heads=n_heads, head_dim=head_dim, ffn=ffn, vocab=vocab)
        self.rope = torch.empty(rope_n, head_dim // 2, 2, dtype=torch.float32, device=device)
        S.sl_rope_table(rope_n, head_dim, rope_theta, self.rope)
        self._arr = (S.sl_layer_weights * n_layers)()
        for l, W in enumerate(layers):
            for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
                t = W[name]
                if t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
                    raise ValueError("layer %d %s must be a contiguous %s device tensor" % (l, name, dtype))
                setattr(self._arr[l], name, t.data_ptr())
        self.s = S.sl_model(S.dtype_code(dtype), n_layers, d, n_heads, head_dim, ffn, vocab, float(rms_eps),
                            C.cast(self._arr, C.POINTER(S.sl_layer_weights)), _dptr(embed), _dptr(lm_head),
                            self.rope.data_ptr(), rope_n)

    def workspace_size(self, B: int, N: int, M_tot: int, minimal: bool = False) -> int:
        """Workspace bytes for a step of at most M_tot rows; minimal: the fixed buffers only
        (split-K residual projections then accumulate with atomics)."""
        if minimal:
            return S.sl_step_workspace_min(self.s, B, N, M_tot)
        return S.sl_step_workspace_size(self.s, B, N, M_tot)


class DeviceState:
    """Sampler state for B sequences of N positions on the GPU."""

    def __init__(self, model: DeviceModel, B: int, N: int, *, tok=None, cand=None, locked=None, h_in=None,
                 k_cache=None, v_cache=None, with_h_out=False, minimal_workspace=False, device="cuda"):
        dm = model.dims
        L, d, H, Dh, V = dm["n_layers"], dm["d"], dm["n_heads"], dm["head_dim"], dm["vocab"]
        dt = model.dtype
        self.model, self.B, self.N = model, B, N
        self.tok = tok
        self.cand = cand
        self.locked = locked if locked is not None else torch.zeros(B * N, dtype=torch.uint8, device=device)
        self.act_idx = torch.empty(B * N, dtype=torch.int32, device=device)
        self.act_off = torch.empty(B + 1, dtype=torch.int32, device=device)
        self.k_cache = k_cache if k_cache is not None else torch.zeros(L, B, N, H, Dh, dtype=dt, device=device)
        self.v_cache = v_cache if v_cache is not None else torch.zeros(L, B, N, H, Dh, dtype=dt, device=device)
        self.h_in = h_in
        self.logits = None
        if model.lm_head is not None:
            self.logits = [torch.zeros(B * N, V, dtype=dt, device=device) for _ in range(2)]
        rows = B * N
        self.kl = torch.zeros(rows, dtype=torch.float32, device=device)
        self.u = torch.zeros(rows, dtype=torch.float32, device=device)
        self.lse = torch.zeros(rows, dtype=torch.float32, device=device)
        self.conf = torch.zeros(rows, dtype=torch.float32, device=device)
        self.argmax = torch.zeros(rows, dtype=torch.int32, device=device)
        self.gate_thr = torch.zeros(B, dtype=torch.float32, device=device)
        self.lock_step = torch.full((rows,), -1, dtype=torch.int32, device=device)
        self.h_out = torch.zeros(rows, d, dtype=torch.float32, device=device) if with_h_out else None
        self.m_host = S.PinnedInt()
        self.M_tot = S.sl_compact(self.locked, B, N, self.act_idx, self.act_off, self.m_host)
        self.t = 0
        # sized for M_tot = B*N, so it serves every later step (M only shrinks)
        self.ws = torch.empty(model.workspace_size(B, N, B * N, minimal_workspace), dtype=torch.uint8,
                              device=device)

    def struct(self) -> S.sl_state:
        st = S.sl_state()
        st.B, st.N, st.M_tot, st.t = self.B, self.N, self.M_tot, self.t
        st.tok, st.cand, st.locked = _dptr(self.tok), _dptr(self.cand), _dptr(self.locked)
        st.act_idx, st.act_off = _dptr(self.act_idx), _dptr(self.act_off)
        st.k_cache, st.v_cache = _dptr(self.k_cache), _dptr(self.v_cache)
        st.h_in, st.h_out = _dptr(self.h_in), _dptr(self.h_out)
        if self.logits is not None:
            st.logits[0], st.logits[1] = self.logits[0].data_ptr(), self.logits[1].data_ptr()
        st.kl, st.u, st.lse, st.conf = _dptr(self.kl), _dptr(self.u), _dptr(self.lse), _dptr(self.conf)
        st.argmax, st.gate_thr, st.lock_step = _dptr(self.argmax), _dptr(self.gate_thr), _dptr(self.lock_step)
        st.m_tot_host = self.m_host.ptr
        return st

    def step(self, eps: float, gate_q: float = -1.0, mask_id: int = -1, do_lock: bool = True,
             unmask_k: int = 0, stream=None, no_kv_cache: bool = False) -> int:
        """One SureLock iteration; returns the new active count.  no_kv_cache: the ablation in
        which positions locked before the step are not attended."""
        p = S.sl_step_params(float(eps), float(gate_q), int(mask_id), int(bool(do_lock)), int(unmask_k),
                             int(bool(no_kv_cache)))
        st = self.struct()
        S.sl_step(self.model.s, st, p, self.ws, stream)
        if do_lock and self.model.lm_head is not None:
            self.M_tot = self.m_host.value
        self.t += 1
        return self.M_tot
