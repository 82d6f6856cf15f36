"""CPU tests of the bf16-storage emulation that the GPU tests take their floating-point bounds from.

1. Its rounding is bfloat16 round-to-nearest-even (hand values).
2. With rounding off it is the oracle's float64 layer step, so every deviation it reports comes
   from the rounding points alone.
3. At the LLaDA-8B layer shape (d = 4096, 32 x 128 heads, FFN 12288, N = 1024, M = 64 active rows)
   it regenerates the bf16-storage error of the hidden rows quoted for that case: relative L2
   2.79e-3, rms 6.88e-3, max 3.26e-2 over the 64 x 4096 outputs.
"""
import numpy as np

import oracle.surelock_oracle as O
import workloads as W
from tests import bf16_emulation as E


def test_round_bf16_is_round_to_nearest_even():
    u = 2.0 ** -7                                    # bf16 spacing on [1, 2)
    cases = [(1.0, 1.0), (1.0 + u / 2, 1.0),         # a tie rounds to the even mantissa
             (1.0 + 3 * u / 2, 1.0 + 2 * u),         # tie between odd and even: up to even
             (1.0 + 0.26 * u, 1.0), (1.0 + 0.74 * u, 1.0 + u), (-3.14159, -3.140625),
             (3.0e38, 226 * 2.0 ** 120), (0.0, 0.0)]   # 3e38 = 225.7 spacings of 2^120
    for x, want in cases:
        got = float(E.round_bf16(np.array([x]))[0])
        assert got == want, (x, got, want)


def _oracle_dims(dm):
    return O.OracleDims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.vocab, dm.rms_eps, dm.rope_theta)


def _emu_dims(dm):
    return E.Dims(dm.d, dm.n_heads, dm.head_dim, dm.ffn, dm.rms_eps, dm.rope_theta)


def test_emulation_without_rounding_is_the_oracle():
    dm = W.Dims(n_layers=1, d=256, n_heads=2, head_dim=128, ffn=512, vocab=1024, dtype="bf16")
    N, M = 128, 40
    case = W.layer_case(dm, N, [M], key=5)
    Wl = {k: O.widen(v, "bf16") for k, v in W.layer_weights(dm, 0).items()}
    h = O.widen(case.h_in, "bf16")[case.act_idx]
    K, V = O.widen(case.k_cache, "bf16")[0], O.widen(case.v_cache, "bf16")[0]
    for attend_locked in (True, False):
        Ko, Vo, Ke, Ve = K.copy(), V.copy(), K.copy(), V.copy()
        ref = O.layer_forward(h, case.act_idx, Wl, Ko, Vo, _oracle_dims(dm), attend_locked)
        got = E.layer(h, case.act_idx, Wl, Ke, Ve, _emu_dims(dm), rnd=False, attend_locked=attend_locked)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Ke, Ko, rtol=1e-12, atol=1e-12)
        # with rounding on, the cache rows it writes are bf16 values
        Ke2, Ve2 = K.copy(), V.copy()
        E.layer(h, case.act_idx, Wl, Ke2, Ve2, _emu_dims(dm), rnd=True, attend_locked=attend_locked)
        np.testing.assert_array_equal(E.round_bf16(Ke2[case.act_idx]), Ke2[case.act_idx])
    head = O.widen(W.lm_head_weights(dm), "bf16")
    np.testing.assert_allclose(E.logits(h, head, dm.rms_eps, rnd=False), O.rmsnorm(h, dm.rms_eps) @ head.T,
                               rtol=1e-12, atol=1e-12)


def llada_layer_m64_error():
    """bf16-storage error of the LLaDA-8B-shaped layer step at N = 1024, M = 64 (the layer workload's
    inputs, key 64) against the float64 oracle."""
    dm = W.LLADA_LAYER
    M, N = 64, 1024
    case = W.layer_case(dm, N, [M], key=M)
    Wl = {k: O.widen(v, "bf16") for k, v in W.layer_weights(dm, 0).items()}
    h = O.widen(case.h_in, "bf16")[case.act_idx]
    K, V = O.widen(case.k_cache, "bf16")[0], O.widen(case.v_cache, "bf16")[0]
    ref = O.layer_forward(h, case.act_idx, Wl, K.copy(), V.copy(), _oracle_dims(dm))
    emu = E.layer(h, case.act_idx, Wl, K.copy(), V.copy(), _emu_dims(dm))
    return E.err_stats(emu, ref)


def test_emulated_error_at_the_llada_layer_shape():
    s = llada_layer_m64_error()
    assert s.n == 64 * 4096
    assert round(s.rel_l2, 5) == 0.00279, s
    assert round(s.rms, 5) == 0.00688, s
    assert round(s.max, 4) == 0.0326, s
