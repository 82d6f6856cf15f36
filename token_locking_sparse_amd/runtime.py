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
                 k_cache=None, v_cache=None, with_h_out=False, minimal_workspace=False, kv_head_major=False,
                 cached_lse=False, device="cuda"):
        """cached_lse: keep a per-position LSE store beside the two posterior buffers, so that each
        step's vocabulary pass takes the previous posterior's LSE from the step that produced it
        (every step with the LM head must then run the pass: do_lock=True)."""
        dm = model.dims
        L, d, H, Dh, V = dm["n_layers"], dm["d"], dm["n_heads"], dm["head_dim"], dm["vocab"]
        dt = model.dtype
        self.model, self.B, self.N = model, B, N
        self.tok = tok
        self.cand = cand
        self.locked = locked if locked is not None else torch.zeros(B * N, dtype=torch.uint8, device=device)
        self.act_idx = torch.empty(B * N, dtype=torch.int32, device=device)
        self.act_off = torch.empty(B + 1, dtype=torch.int32, device=device)
        # token-major [L][B][N][H][Dh], or head-major [L][B][H][N][Dh]
        self.kv_head_major = bool(kv_head_major)
        shape = (L, B, H, N, Dh) if self.kv_head_major else (L, B, N, H, Dh)
        self.k_cache = k_cache if k_cache is not None else torch.zeros(shape, dtype=dt, device=device)
        self.v_cache = v_cache if v_cache is not None else torch.zeros(shape, dtype=dt, device=device)
        self.h_in = h_in
        self.logits = None
        self.lse_pos = None
        if model.lm_head is not None:
            self.logits = [torch.zeros(B * N, V, dtype=dt, device=device) for _ in range(2)]
            if cached_lse:
                self.lse_pos = [torch.zeros(B * N, dtype=torch.float32, device=device) for _ in range(2)]
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
        self.t_dev = None      # device step index (set by CapturedLoop)
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
        st.t_dev = _dptr(self.t_dev)
        st.kv_head_major = int(self.kv_head_major)
        if self.lse_pos is not None:
            st.lse_pos[0], st.lse_pos[1] = self.lse_pos[0].data_ptr(), self.lse_pos[1].data_ptr()
        return st

    def step(self, eps: float, gate_q: float = -1.0, mask_id: int = -1, do_lock: bool = True,
             unmask_k: int = 0, stream=None, no_kv_cache: bool = False, device_m: bool = False,
             fuse_head_kl: bool = False) -> int:
        """One SureLock iteration; returns the new active count.  no_kv_cache: the ablation in
        which positions locked before the step are not attended.  device_m: the count stays on the
        device (M_tot is kept as an upper bound and returned unchanged; no host wait).  fuse_head_kl:
        the LM head computes the vocabulary statistics in its epilogue."""
        p = S.sl_step_params(float(eps), float(gate_q), int(mask_id), int(bool(do_lock)), int(unmask_k),
                             int(bool(no_kv_cache)), int(bool(device_m)), int(bool(fuse_head_kl)))
        st = self.struct()
        if device_m:
            st.m_tot_host = None
        S.sl_step(self.model.s, st, p, self.ws, stream)
        if do_lock and self.model.lm_head is not None and not device_m:
            self.M_tot = self.m_host.value
        self.t += 1
        return self.M_tot


class CapturedLoop:
    """The sampler loop with the active count kept on the device.

    Every step runs with sl_step_params.device_m = 1: the kernels read the live
    count act_off[B] themselves and the host passes only an upper bound, so no
    step waits for the host to read the count back.  Each step is one replay of
    a HIP graph holding the whole step (gather, every layer, LM head, KL-lock,
    sampler and compaction).  Graphs are captured on first use per (capacity,
    step parity): the capacity is the last count the host has seen, rounded up
    to a multiple of `bucket`, and it shrinks as the host learns smaller counts
    from copies of the count that each step queues behind itself.  The host
    keeps at most `depth` steps queued ahead of the last one it has seen
    finish: before queuing step t it waits for step t - depth, whose count
    bounds step t's, while step t - 1 still keeps the GPU busy.  (Without that
    bound the host would queue the whole loop at the first capacity.)  The
    parity picks which posterior buffer is current; the step index that
    lock_step records lives on the device (eager steps of the same state use it
    too).  Replays start once the state has run at least one step (t >= 1), so
    every replayed step has a previous posterior; graphs may be captured before.
    """

    def __init__(self, state: DeviceState, eps: float, gate_q: float = -1.0, mask_id: int = -1,
                 unmask_k: int = 0, no_kv_cache: bool = False, bucket: int = 64, fuse_head_kl: bool = False,
                 depth: int = 2):
        if state.model.lm_head is None:
            raise ValueError("CapturedLoop runs the whole sampler step and needs an LM head")
        self.st = state
        self.p = S.sl_step_params(float(eps), float(gate_q), int(mask_id), 1, int(unmask_k), int(bool(no_kv_cache)), 1,
                                  int(bool(fuse_head_kl)))
        self.bucket = bucket
        self.graphs = {}
        self.known_m = state.M_tot           # an upper bound of the live count
        self.stream = torch.cuda.Stream()
        dev = state.act_off.device
        state.t_dev = torch.full((1,), state.t, dtype=torch.int32, device=dev)
        self.depth = max(1, int(depth))
        self._pending = []                   # (event, pinned slot) of the counts queued steps copy back
        self._pool = [torch.zeros(1, dtype=torch.int32, pin_memory=True) for _ in range(self.depth + 1)]
        self._slot = 0

    def _cap(self) -> int:
        b = self.bucket
        return min(self.st.B * self.st.N, max(b, (self.known_m + b - 1) // b * b))

    def _graph(self, cap: int, parity: int):
        key = (cap, parity)
        g = self.graphs.get(key)
        if g is None:
            st = self.st.struct()
            # the capacity sizes the grids; t only selects the posterior buffers here (t >= 1: a
            # previous posterior exists); no host copy of the count inside a graph
            st.M_tot, st.t, st.m_tot_host = cap, 2 - parity, None
            g = torch.cuda.CUDAGraph()
            self.stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.graph(g, stream=self.stream):
                S.sl_step(self.st.model.s, st, self.p, self.st.ws, stream=self.stream)
            torch.cuda.current_stream().wait_stream(self.stream)
            self.graphs[key] = (g, st)
            g = self.graphs[key]
        return g[0]

    def _learn(self):
        """Wait for the oldest queued step while `depth` are queued, then take every count whose
        copy has completed."""
        while len(self._pending) >= self.depth:
            ev, slot = self._pending.pop(0)
            ev.synchronize()
            self.known_m = min(self.known_m, int(slot[0]))
        while self._pending and self._pending[0][0].query():
            ev, slot = self._pending.pop(0)
            self.known_m = min(self.known_m, int(slot[0]))

    def precapture(self, max_count: int | None = None):
        """Capture the graphs of every capacity up to max_count (default: the current bound), both
        parities, ahead of the loop, so that no capture happens between replays."""
        top = self._cap() if max_count is None else max_count
        for cap in range(self.bucket, top + self.bucket, self.bucket):
            cap = min(cap, self.st.B * self.st.N)
            for parity in (0, 1):
                self._graph(cap, parity)

    def step(self, m_hist: torch.Tensor | None = None):
        """Enqueue one step (a graph replay) on the current stream; m_hist[t] (device int32) receives the
        step's input count when given."""
        st = self.st
        if st.t < 1:
            raise ValueError("replayed steps need a previous posterior: run the first step eagerly")
        cs = torch.cuda.current_stream()
        if m_hist is not None:
            m_hist[st.t:st.t + 1].copy_(st.act_off[st.B:st.B + 1])
        self._learn()
        self._graph(self._cap(), st.t & 1).replay()
        st.t += 1
        slot = self._pool[self._slot % len(self._pool)]   # not in use: at most depth are pending
        self._slot += 1
        slot.copy_(st.act_off[st.B:st.B + 1], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(cs)
        self._pending.append((ev, slot))

    def finish(self) -> int:
        """Wait for the enqueued steps; returns the live count and stores it in the state."""
        torch.cuda.synchronize()
        st = self.st
        st.M_tot = int(st.act_off[st.B].item())
        self.known_m = st.M_tot
        self._pending = []
        return st.M_tot
