"""CPU checks of the C ABI: the library loads and exports every function include/surelock.h declares,
and host-side argument checks reject bad calls before any GPU work (no device needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "surelock.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(sl_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sl_step", "sl_attn_active", "sl_kl_lock", "sl_compact", "sl_cache_scatter"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import token_locking_sparse_amd.surelock as S
    L = S.lib()
    for n in declared_functions():
        assert hasattr(L, n), "libsurelock.so does not export %s" % n
    assert set(S.EXPORTS) <= set(declared_functions())


def test_status_strings_and_host_checks():
    import token_locking_sparse_amd.surelock as S
    L = S.lib()
    assert L.sl_status_string(0) == b"SL_OK"
    assert L.sl_status_string(2) == b"SL_ERR_UNSUPPORTED"
    # NULL pointers are rejected on the host before any launch
    st = L.sl_compact(None, 1, 8, None, None, None, None)
    assert st == 1 and b"NULL" in L.sl_last_error()
    st = L.sl_rope_table(0, 32, ctypes.c_float(1e4), None, None)
    assert st == 1
    p = S.sl_lock_params(0.01, 0.5, -1, 1)
    st = L.sl_kl_lock(7, None, None, 8, None, None, 1, 8, 0, None, ctypes.byref(p), None, None, None, None,
                      None, None, None, None, None, None, None, None, None, 0, None)
    assert st == 1 and b"dtype" in L.sl_last_error()
    # unsupported head_dim
    st = L.sl_attn_active(0, None, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None, 1, 64, 0, 1,
                          48, ctypes.c_float(1.0), None, ctypes.c_void_p(16), 1024, None)
    assert st == 2
    # misaligned exclusion flags
    st = L.sl_attn_active(0, None, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(18),
                          1, 64, 0, 1, 64, ctypes.c_float(1.0), None, ctypes.c_void_p(16), 1 << 20, None)
    assert st == 1 and b"aligned" in L.sl_last_error()
    # a GEMM A operand beyond the 32-bit row offsets (300000 x 8192 bf16 = 4.9 GB) is refused, not launched
    dummy = ctypes.c_void_p(256)
    st = L.sl_gemm(0, 1, dummy, 300000, 8192, 4096, dummy, None, None, dummy, None, None, None, 0, 0, None, None,
                   1, 1, None)
    assert st == 2 and b"4 GiB" in L.sl_last_error()
    # the clock-recording GEMM takes the SwiGLU or logits epilogue only, and a clock record
    st = L.sl_gemm_clocked(0, dummy, 16, 512, 1536, dummy, None, dummy, None, None, 1, 16, dummy, 4, None)
    assert st == 2
    st = L.sl_gemm_clocked(2, dummy, 16, 512, 1536, dummy, dummy, dummy, None, None, 1, 16, None, 0, None)
    assert st == 1 and b"clock" in L.sl_last_error()
    # the operand MFMA loop rotates 8 operand sets: iters must be a multiple of 8
    assert L.sl_peak_mfma_operands(4, 12, dummy, dummy, None, None) == 1


def test_workspace_sizes_are_monotone_in_rows():
    import ctypes

    import token_locking_sparse_amd.surelock as S
    # step workspace: the minimum (fixed buffers) never exceeds the recommended size, which grows with M
    arr = (S.sl_layer_weights * 1)()
    m = S.sl_model(0, 1, 4096, 32, 128, 12288, 126464, 1e-5, ctypes.cast(arr, ctypes.POINTER(S.sl_layer_weights)),
                   None, None, None, 1024)
    sizes = [(S.sl_step_workspace_min(m, 1, 1024, M), S.sl_step_workspace_size(m, 1, 1024, M)) for M in (1, 64, 256, 1024)]
    assert all(0 < lo <= hi for lo, hi in sizes)
    assert all(a[1] <= b[1] for a, b in zip(sizes, sizes[1:]))
    assert sizes[2][1] > sizes[2][0]   # M = 256 splits the residual projections: partial planes reserved
    # a workspace sized for M rows serves every later step with fewer rows, also where the attention's
    # key-split partials make a smaller step need more (M = 128 splits its keys, M = 129 does not)
    dense = [(S.sl_step_workspace_min(m, 1, 1024, M), S.sl_step_workspace_size(m, 1, 1024, M)) for M in range(100, 160)]
    assert all(a[0] <= b[0] and a[1] <= b[1] for a, b in zip(dense, dense[1:]))
    a = S.sl_kl_lock_workspace_size(1, 4096, 100, 126464)
    b = S.sl_kl_lock_workspace_size(1, 4096, 1639, 126464)
    assert b >= a > 0
    # a KL-lock workspace sized for M rows serves every call with fewer: the size never falls with M,
    # across the changes of segments per row (768 rows) and the end of splitting (2048 rows)
    kl_sorted_m = [S.sl_kl_lock_workspace_size(1, 4096, M, 126464) for M in sorted(list(range(1, 2200, 13)) + [767, 768, 2047, 2048, 4096])]
    assert all(x <= y for x, y in zip(kl_sorted_m, kl_sorted_m[1:]))
    assert kl_sorted_m[-1] <= 256 * 1024   # within sl_kl_lock_noalloc's scratch
    assert S.sl_attn_workspace_size(1, 1024, 64, 32, 128) > 0
    # likewise the attention's: key splits come and go with M, the size never falls
    at = [S.sl_attn_workspace_size(1, 1024, M, 32, 128) for M in range(1, 1025, 9)]
    assert all(x <= y for x, y in zip(at, at[1:]))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "token_locking_sparse_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.replace("oracle of", ""), "%s mentions the oracle" % f


def test_gemm_plan_tiles_divide_and_only_residual_splits():
    import torch

    import token_locking_sparse_amd.surelock as S
    d, f, v = 4096, 12288, 126464
    shapes = [(S.SL_EPI_QKV_ROPE, d, 3 * d), (S.SL_EPI_RESIDUAL, d, d), (S.SL_EPI_SWIGLU, d, 2 * f),
              (S.SL_EPI_RESIDUAL, f, d), (S.SL_EPI_LOGITS, d, v)]
    for epi, K, n in shapes:
        for M in (1, 64, 256, 512, 1024, 3000):
            tm, tn, sk, vb = S.sl_gemm_plan(torch.bfloat16, epi, M, K, n, with_path=True)
            assert n % tn == 0 and tm in (64, 128, 256) and tn % 32 == 0
            assert sk >= 1 and (sk == 1 or epi == S.SL_EPI_RESIDUAL)
            assert (K * 2 // 128) // sk >= 1
            assert vb in (0, 1) and (not vb or sk == 1)   # the register path streams the whole K
            assert S.sl_gemm_plan(torch.float32, epi, M, K, n, with_path=True)[3] == 0
    # wide outputs at few rows stream their weights through registers
    assert S.sl_gemm_plan(torch.bfloat16, S.SL_EPI_LOGITS, 16, d, v, with_path=True)[3] == 1
    # residual projections with few row tiles split K to fill the chip
    assert S.sl_gemm_plan(torch.bfloat16, S.SL_EPI_RESIDUAL, 64, f, d)[2] > 1
    with pytest.raises(S.SureLockError):
        S.sl_gemm_plan(torch.bfloat16, S.SL_EPI_SWIGLU, 64, 4096, 100)   # n_out % 64 != 0


def test_gemm_parity_cases_cover_every_tile():
    """The GPU GEMM parity cases reach every tile shape the launcher can pick (checked on the host)."""
    import torch

    import token_locking_sparse_amd.surelock as S
    from tests.test_gpu_kernels import ALL_TILES, GEMM_CASES, tile_of
    epi = {"resid": S.SL_EPI_RESIDUAL, "swiglu": S.SL_EPI_SWIGLU, "qkv": S.SL_EPI_QKV_ROPE, "logits": S.SL_EPI_LOGITS}
    assert {tile_of(S, epi[e], M, K, n) for e, M, K, n in GEMM_CASES} == ALL_TILES
