"""ctypes binding of libsurelock.so (argument marshalling only).

Every entry point mirrors the C function of the same name in
include/surelock.h; tensors are passed as device pointers and the current
torch stream is passed as the HIP stream.  Every step of the computation runs
in the HIP library: there is no Python or CPU fallback, and a missing library
raises at load time.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsurelock.so")

SL_BF16, SL_F32 = 0, 1
_STATUS = {0: "SL_OK", 1: "SL_ERR_INVALID", 2: "SL_ERR_UNSUPPORTED", 3: "SL_ERR_HIP"}


class SureLockError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s: %s" % (fn, _STATUS.get(status, status), msg))
        self.status = status


class sl_lock_params(C.Structure):
    _fields_ = [("eps", C.c_float), ("gate_q", C.c_float), ("mask_id", C.c_int), ("have_prev", C.c_int)]


class sl_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]


class sl_model(C.Structure):
    _fields_ = [("dtype", C.c_int), ("n_layers", C.c_int), ("d", C.c_int), ("n_heads", C.c_int),
                ("head_dim", C.c_int), ("ffn", C.c_int), ("vocab", C.c_int), ("rms_eps", C.c_float),
                ("layers", C.POINTER(sl_layer_weights)), ("embed", C.c_void_p), ("lm_head", C.c_void_p),
                ("rope", C.c_void_p), ("rope_n", C.c_int)]


class sl_state(C.Structure):
    _fields_ = [("B", C.c_int), ("N", C.c_int), ("M_tot", C.c_int), ("t", C.c_int),
                ("tok", C.c_void_p), ("cand", C.c_void_p), ("locked", C.c_void_p),
                ("act_idx", C.c_void_p), ("act_off", C.c_void_p),
                ("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("h_in", C.c_void_p), ("h_out", C.c_void_p), ("logits", C.c_void_p * 2),
                ("kl", C.c_void_p), ("u", C.c_void_p), ("lse", C.c_void_p), ("conf", C.c_void_p),
                ("argmax", C.c_void_p), ("gate_thr", C.c_void_p), ("lock_step", C.c_void_p),
                ("m_tot_host", C.c_void_p), ("t_dev", C.c_void_p), ("kv_head_major", C.c_int),
                ("lse_pos", C.c_void_p * 2)]


class sl_step_params(C.Structure):
    _fields_ = [("eps", C.c_float), ("gate_q", C.c_float), ("mask_id", C.c_int), ("do_lock", C.c_int),
                ("unmask_k", C.c_int), ("no_kv_cache", C.c_int), ("device_m", C.c_int),
                ("fuse_head_kl", C.c_int)]


EXPORTS = ("sl_status_string", "sl_last_error", "sl_version", "sl_compact", "sl_cache_scatter",
           "sl_attn_active", "sl_attn_workspace_size", "sl_kl_lock", "sl_kl_lock_workspace_size",
           "sl_rope_table", "sl_step", "sl_step_workspace_size", "sl_step_workspace_min", "sl_gemm",
           "sl_gemm_plan", "sl_kl_lock_noalloc", "sl_peak_mfma", "sl_peak_mfma_flops", "sl_peak_stream",
           "sl_peak_gemm_loop", "sl_peak_gemm_loop_flops", "sl_peak_mfma_operands", "sl_gemm_clocked")

_lib = None


def lib():
    """Load libsurelock.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libsurelock.so is not built (expected at %s); run __graft_entry__.build()" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    vp, i, f, sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t
    sig = {
        "sl_status_string": (C.c_char_p, [i]),
        "sl_last_error": (C.c_char_p, []),
        "sl_version": (C.c_char_p, []),
        "sl_compact": (i, [vp, i, i, vp, vp, vp, vp]),
        "sl_cache_scatter": (i, [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]),
        "sl_attn_active": (i, [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, sz, vp]),
        "sl_attn_workspace_size": (sz, [i, i, i, i, i]),
        "sl_kl_lock": (i, [i, vp, vp, i, vp, vp, i, i, i, vp, C.POINTER(sl_lock_params), vp, vp, vp, vp,
                           vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sl_kl_lock_workspace_size": (sz, [i, i, i, i]),
        "sl_kl_lock_noalloc": (i, [i, vp, vp, i, vp, vp, i, i, i, vp, C.POINTER(sl_lock_params), vp, vp, vp, vp,
                                   vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "sl_rope_table": (i, [i, i, f, vp, vp]),
        "sl_step": (i, [C.POINTER(sl_model), C.POINTER(sl_state), C.POINTER(sl_step_params), vp, sz, vp]),
        "sl_step_workspace_size": (sz, [C.POINTER(sl_model), i, i, i]),
        "sl_step_workspace_min": (sz, [C.POINTER(sl_model), i, i, i]),
        "sl_gemm": (i, [i, i, vp, i, i, i, vp, vp, vp, vp, vp, vp, vp, i, i, vp, vp, i, i, vp]),
        "sl_gemm_plan": (i, [i, i, i, i, i, C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int),
                             C.POINTER(C.c_int)]),
        "sl_peak_mfma": (i, [i, i, vp, vp]),
        "sl_peak_mfma_flops": (C.c_double, [i, i]),
        "sl_peak_stream": (i, [vp, vp, sz, i, vp, vp]),
        "sl_peak_gemm_loop": (i, [i, i, i, vp, vp, vp]),
        "sl_peak_gemm_loop_flops": (C.c_double, [i, i]),
        "sl_peak_mfma_operands": (i, [i, i, vp, vp, vp, vp]),
        "sl_gemm_clocked": (i, [i, vp, i, i, i, vp, vp, vp, vp, vp, i, i, vp, i, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


# ------------------------------------------------------------------ helpers
def _ptr(t, name="tensor", dtype=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(fn, st):
    if st != 0:
        raise SureLockError(fn, st, lib().sl_last_error().decode())


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return SL_BF16
    if t == torch.float32:
        return SL_F32
    raise TypeError("storage dtype must be bfloat16 or float32, got %s" % t)


class PinnedInt:
    """A pinned host int32 that receives an active count (m_tot_host)."""

    def __init__(self):
        self.t = torch.zeros(1, dtype=torch.int32, pin_memory=True)

    @property
    def ptr(self):
        return self.t.data_ptr()

    @property
    def value(self) -> int:
        return int(self.t[0])


# ------------------------------------------------------------------ entry points
def sl_compact(locked, B, N, act_idx, act_off, m_tot_host: PinnedInt | None = None, stream=None):
    st = lib().sl_compact(_ptr(locked, "locked", torch.uint8), B, N, _ptr(act_idx, "act_idx", torch.int32),
                          _ptr(act_off, "act_off", torch.int32), m_tot_host.ptr if m_tot_host else None,
                          _stream(stream))
    _check("sl_compact", st)
    return m_tot_host.value if m_tot_host else None


def sl_cache_scatter(k_cache, v_cache, k_new, v_new, act_idx, act_off, B, N, M_tot, H, Dh, stream=None):
    dt = dtype_code(k_cache.dtype)
    st = lib().sl_cache_scatter(dt, _ptr(k_cache, "k_cache", k_cache.dtype), _ptr(v_cache, "v_cache", k_cache.dtype),
                                _ptr(k_new, "k_new", k_cache.dtype, optional=M_tot == 0),
                                _ptr(v_new, "v_new", k_cache.dtype, optional=M_tot == 0),
                                _ptr(act_idx, "act_idx", torch.int32), _ptr(act_off, "act_off", torch.int32),
                                B, N, M_tot, H, Dh, _stream(stream))
    _check("sl_cache_scatter", st)


def sl_attn_workspace_size(B, N, M_tot, H, Dh) -> int:
    return int(lib().sl_attn_workspace_size(B, N, M_tot, H, Dh))


def sl_attn_active(q, k_cache, v_cache, act_off, B, N, M_tot, H, Dh, scale, out, ws, stream=None, key_excl=None):
    """key_excl: optional [B*N] uint8 device tensor; nonzero positions are not attended."""
    dt = dtype_code(k_cache.dtype)
    st = lib().sl_attn_active(dt, _ptr(q, "q", k_cache.dtype, optional=M_tot == 0),
                              _ptr(k_cache, "k_cache", k_cache.dtype), _ptr(v_cache, "v_cache", k_cache.dtype),
                              _ptr(act_off, "act_off", torch.int32),
                              _ptr(key_excl, "key_excl", torch.uint8, optional=True), B, N, M_tot, H, Dh, float(scale),
                              _ptr(out, "out", k_cache.dtype, optional=M_tot == 0), _ptr(ws, "ws"),
                              ws.numel() * ws.element_size(), _stream(stream))
    _check("sl_attn_active", st)


def sl_kl_lock_workspace_size(B, N, M_tot, V) -> int:
    return int(lib().sl_kl_lock_workspace_size(B, N, M_tot, V))


def sl_kl_lock(logits_cur, logits_prev, V, act_idx, act_off, B, N, M_tot, cand, eps, gate_q, mask_id,
               have_prev, locked, kl, u, lse, argmax, conf, gate_thr, new_act_idx, new_act_off, ws,
               m_tot_host: PinnedInt | None = None, stream=None, lse_prev=None, lse_pos=None):
    """lse_prev / lse_pos: optional [B*N] float32 per-position LSE stores (the previous pass's, and
    this pass's); with lse_prev the previous logits' own normaliser is not recomputed."""
    dt = dtype_code(logits_cur.dtype)
    p = sl_lock_params(float(eps), float(gate_q), int(mask_id), int(bool(have_prev)))
    st = lib().sl_kl_lock(dt, _ptr(logits_cur, "logits_cur", logits_cur.dtype),
                          _ptr(logits_prev, "logits_prev", logits_cur.dtype, optional=not have_prev), V,
                          _ptr(act_idx, "act_idx", torch.int32) if M_tot > 0 else None,
                          _ptr(act_off, "act_off", torch.int32), B, N, M_tot, _ptr(cand, "cand", torch.uint8, optional=True), C.byref(p),
                          _ptr(locked, "locked", torch.uint8), _ptr(kl, "kl", torch.float32),
                          _ptr(u, "u", torch.float32), _ptr(lse, "lse", torch.float32),
                          _ptr(argmax, "argmax", torch.int32, optional=True),
                          _ptr(conf, "conf", torch.float32, optional=True),
                          _ptr(lse_prev, "lse_prev", torch.float32, optional=True),
                          _ptr(lse_pos, "lse_pos", torch.float32, optional=True),
                          _ptr(gate_thr, "gate_thr", torch.float32, optional=True),
                          _ptr(new_act_idx, "new_act_idx", torch.int32), _ptr(new_act_off, "new_act_off", torch.int32),
                          m_tot_host.ptr if m_tot_host else None, _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                          _stream(stream))
    _check("sl_kl_lock", st)
    return m_tot_host.value if m_tot_host else None


def sl_kl_lock_noalloc(logits_cur, logits_prev, V, act_idx, act_off, B, N, M_tot, cand, eps, gate_q, mask_id,
                       have_prev, locked, kl, u, lse, argmax, conf, gate_thr, new_act_idx, new_act_off,
                       m_tot_host: PinnedInt | None = None, stream=None, lse_prev=None, lse_pos=None):
    """sl_kl_lock without a workspace argument (the library's own per-GPU scratch array)."""
    dt = dtype_code(logits_cur.dtype)
    p = sl_lock_params(float(eps), float(gate_q), int(mask_id), int(bool(have_prev)))
    st = lib().sl_kl_lock_noalloc(dt, _ptr(logits_cur, "logits_cur", logits_cur.dtype),
                                  _ptr(logits_prev, "logits_prev", logits_cur.dtype, optional=not have_prev), V,
                                  _ptr(act_idx, "act_idx", torch.int32) if M_tot > 0 else None,
                                  _ptr(act_off, "act_off", torch.int32), B, N, M_tot,
                                  _ptr(cand, "cand", torch.uint8, optional=True), C.byref(p),
                                  _ptr(locked, "locked", torch.uint8), _ptr(kl, "kl", torch.float32),
                                  _ptr(u, "u", torch.float32), _ptr(lse, "lse", torch.float32),
                                  _ptr(argmax, "argmax", torch.int32, optional=True),
                                  _ptr(conf, "conf", torch.float32, optional=True),
                                  _ptr(lse_prev, "lse_prev", torch.float32, optional=True),
                                  _ptr(lse_pos, "lse_pos", torch.float32, optional=True),
                                  _ptr(gate_thr, "gate_thr", torch.float32, optional=True),
                                  _ptr(new_act_idx, "new_act_idx", torch.int32),
                                  _ptr(new_act_off, "new_act_off", torch.int32),
                                  m_tot_host.ptr if m_tot_host else None, _stream(stream))
    _check("sl_kl_lock_noalloc", st)
    return m_tot_host.value if m_tot_host else None


def sl_rope_table(n_pos, head_dim, theta, table, stream=None):
    st = lib().sl_rope_table(n_pos, head_dim, float(theta), _ptr(table, "table", torch.float32), _stream(stream))
    _check("sl_rope_table", st)


def sl_step_workspace_size(model: sl_model, B, N, M_tot) -> int:
    return int(lib().sl_step_workspace_size(C.byref(model), B, N, M_tot))


def sl_step_workspace_min(model: sl_model, B, N, M_tot) -> int:
    return int(lib().sl_step_workspace_min(C.byref(model), B, N, M_tot))


def sl_step(model: sl_model, state: sl_state, params: sl_step_params, ws, stream=None):
    st = lib().sl_step(C.byref(model), C.byref(state), C.byref(params), _ptr(ws, "ws"),
                       ws.numel() * ws.element_size(), _stream(stream))
    _check("sl_step", st)


SL_EPI_QKV_ROPE, SL_EPI_RESIDUAL, SL_EPI_SWIGLU, SL_EPI_LOGITS = 0, 1, 2, 3


def sl_gemm_plan(dtype, epilogue, M, K, n_out, with_path=False):
    """(tile rows, tile columns, split-K) that sl_gemm launches for this shape; with_path adds
    1 when the tiles go through registers, 0 for direct global-to-LDS loads."""
    tm, tn, sk, vb = C.c_int(0), C.c_int(0), C.c_int(0), C.c_int(0)
    st = lib().sl_gemm_plan(dtype_code(dtype), int(epilogue), M, K, n_out, C.byref(tm), C.byref(tn), C.byref(sk),
                            C.byref(vb))
    _check("sl_gemm_plan", st)
    return (tm.value, tn.value, sk.value, vb.value) if with_path else (tm.value, tn.value, sk.value)


def sl_gemm(epilogue, A, M, K, n_out, w0, w1=None, w2=None, out0=None, out1=None, out2=None, rope=None,
            d=0, head_dim=0, act_idx=None, act_off=None, B=0, N=0, stream=None):
    dt = dtype_code(A.dtype)
    st = lib().sl_gemm(dt, int(epilogue), _ptr(A, "A", A.dtype), M, K, n_out, _ptr(w0, "w0", A.dtype),
                       _ptr(w1, "w1", A.dtype, optional=True), _ptr(w2, "w2", A.dtype, optional=True),
                       _ptr(out0, "out0"), _ptr(out1, "out1", optional=True), _ptr(out2, "out2", optional=True),
                       _ptr(rope, "rope", torch.float32, optional=True), d, head_dim,
                       _ptr(act_idx, "act_idx", torch.int32, optional=True),
                       _ptr(act_off, "act_off", torch.int32, optional=True), B, N, _stream(stream))
    _check("sl_gemm", st)


# ------------------------------------------------------------------ measurement helpers
def sl_peak_mfma(workgroups: int, iters: int, sink, stream=None) -> float:
    """Launch the register-only MFMA loop; returns the FLOPs it performs."""
    _check("sl_peak_mfma", lib().sl_peak_mfma(workgroups, iters, _ptr(sink, "sink", torch.float32), _stream(stream)))
    return float(lib().sl_peak_mfma_flops(workgroups, iters))


def sl_peak_mfma_operands(workgroups: int, iters: int, operands, sink, clocks=None, stream=None) -> float:
    """The MFMA loop on operands read from `operands` (16 x 256 chunks of 16 bytes); clocks (int64,
    2 x workgroups, optional) receives per workgroup its shader-clock cycles and 100 MHz ticks.
    Returns the FLOPs it performs."""
    if operands.numel() * operands.element_size() < 16 * 256 * 16:
        raise ValueError("operands must hold 16 x 256 chunks of 16 bytes")
    if clocks is not None and (clocks.dtype != torch.int64 or clocks.numel() < 2 * workgroups):
        raise ValueError("clocks must be int64 with 2 x workgroups entries")
    _check("sl_peak_mfma_operands", lib().sl_peak_mfma_operands(workgroups, iters, _ptr(operands, "operands"),
                                                                _ptr(sink, "sink", torch.float32),
                                                                _ptr(clocks, "clocks", optional=True),
                                                                _stream(stream)))
    return float(lib().sl_peak_mfma_flops(workgroups, iters))


def sl_gemm_clocked(epilogue, A, M, K, n_out, w0, w1=None, out0=None, act_idx=None, act_off=None, B=0, N=0,
                    clocks=None, stream=None):
    """sl_gemm (bf16, SwiGLU or logits epilogue) recording per workgroup, in clocks (int64, 4 per
    workgroup): shader-clock cycles, 100 MHz ticks, cycles of the k-tile loop, K elements multiplied."""
    if clocks is None or clocks.dtype != torch.int64 or clocks.numel() < 4:
        raise ValueError("clocks must be an int64 device tensor of 4 x workgroups entries")
    st = lib().sl_gemm_clocked(int(epilogue), _ptr(A, "A", torch.bfloat16), M, K, n_out,
                               _ptr(w0, "w0", torch.bfloat16), _ptr(w1, "w1", torch.bfloat16, optional=True),
                               _ptr(out0, "out0"), _ptr(act_idx, "act_idx", torch.int32, optional=True),
                               _ptr(act_off, "act_off", torch.int32, optional=True), B, N,
                               _ptr(clocks, "clocks"), clocks.numel() // 4, _stream(stream))
    _check("sl_gemm_clocked", st)


def sl_peak_gemm_loop(workgroups: int, tiles: int, with_loads: bool, src, sink, stream=None) -> float:
    """Launch the GEMM tile's LDS-to-MFMA loop alone (with_loads: plus its direct loads, waits and
    barrier, from the L2-resident src); returns the FLOPs it performs."""
    _check("sl_peak_gemm_loop", lib().sl_peak_gemm_loop(workgroups, tiles, int(bool(with_loads)),
                                                        _ptr(src, "src", optional=not with_loads),
                                                        _ptr(sink, "sink", torch.float32), _stream(stream)))
    return float(lib().sl_peak_gemm_loop_flops(workgroups, tiles))


def sl_peak_stream(src, dst, workgroups: int, sink, stream=None):
    """Stream src (read only when dst is None, else copy into dst) with 16-byte non-temporal accesses."""
    nbytes = src.numel() * src.element_size()
    _check("sl_peak_stream", lib().sl_peak_stream(_ptr(src, "src"), _ptr(dst, "dst", optional=True), nbytes,
                                                  workgroups, _ptr(sink, "sink", torch.float32), _stream(stream)))
