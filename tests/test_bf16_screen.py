"""Soundness of the step kernel's screen for bf16 parameters (CPU only).

For bf16 parameters the kernel may take a short path for a slice:
- sq = the hardware square root of v: within one ulp on normal inputs (checked on
  the hardware over every normal binary32), and zero for subnormal inputs, which
  the hardware flushes;
- d = fma(sq, a, b), with a = inv_sqrt_bc2 / step_size and b = eps / step_size each
  rounded once to binary32 on the host;
- t = m * rcp(d), with the hardware reciprocal within one ulp on normal inputs up to
  2^126;
- pf = p - t.

It keeps pf only if |t| < min(step_size, 1) 2^127 and both ends of [pf - c, pf + c]
round to the same bf16 bits, with c = |t| 2^-19 + |pf| 2^-22 + 2^-126 (each product
taken exactly, one rounding).

Here the short path is emulated in binary32 with every combination of one-ulp errors
in the square root, the fma and the reciprocal. Wherever the screen passes, its bf16
result must equal the oracle's (the correctly rounded sequence). The inputs put many
exact results next to bf16 rounding boundaries, using updates as large as the
parameters. An unsound width would show up: a screen 16 times narrower passes wrong
results in every case. Two more cases pin the path's other rules:
- a subnormal second moment may take the short path when eps is large enough for
  its flushed square root not to matter;
- the bound on |t| is needed where the sequence's quotient overflows.
"""

import itertools
import math
import os
import re

import numpy as np
import pytest

import oracle

F32 = np.float32
# binary exponents of the screen's two factors, as in the kernel's screen_width()
T_EXP, PF_EXP = -19, -22
# eps >= 2^SUB_EXP * inv_sqrt_bc2 lets subnormal second moments take the short path
SUB_EXP = -39
KERNEL_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "block_wise_bit_adam8bit_amd", "csrc", "qopt_kernels.hip")


def _ulp_step(x, k):
    """x moved by k ulps (k in -1, 0, 1) along the binary32 line where it is finite
    and nonzero; zeros and infinities stay (the hardware square root of 0, and the
    hardware reciprocal of 0 and of infinity, are exact)."""
    if k == 0:
        return x
    moved = np.nextafter(x, F32(np.inf) if k > 0 else F32(-np.inf)).astype(F32)
    return np.where(np.isfinite(x) & (x != 0), moved, x).astype(F32)


def _fma_down(a, b, c):
    """a*b + c with one rounding, then one ulp toward zero: never above the fused
    multiply-add the kernel performs (a, b, c non-negative here)."""
    r = (a.astype(np.float64) * float(b) + c.astype(np.float64)).astype(F32)
    return np.nextafter(r, F32(0)).astype(F32)


def _short_scalars(eps32, ss, isb):
    """The host's folded scalars and path selection, restated: (a, b, t_limit, mode)
    with mode None (no short path), "screen" or "screen+subnormal check"."""
    ss_d = float(ss)
    a = F32(float(isb) / ss_d) if ss_d > 0 else F32(0)
    b = F32(float(eps32) / ss_d) if ss_d > 0 else F32(0)
    t_limit = F32(min(ss_d, 1.0) * 2.0 ** 127)
    a_ok = 2.0 ** -63 <= float(a) <= 2.0 ** 61
    b_ok = float(b) == 0.0 or 2.0 ** -126 <= float(b) <= 2.0 ** 125
    if not (0 < ss_d <= 2.0 ** 20 and a_ok and b_ok):
        return a, b, t_limit, None
    sub_check = float(eps32) != 0.0 and not (float(eps32) >= float(isb) * 2.0 ** SUB_EXP)
    return a, b, t_limit, ("screen+subnormal check" if sub_check else "screen")


def _inputs_from_state(rng, p32, g, cm, cv, am, av, lr, beta1, beta2, eps, step):
    """The moments as the kernel forms them (same binary32 operations), the
    oracle's fp32 result and the step's scalars."""
    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, step=step)
    exact32 = oracle.adam8bit_step(p32, g, cm, cv, am, av, **hp)[0]
    b1, b2, omb1, omb2, eps32, ss, isb = oracle.adam_scalars(lr, beta1, beta2, eps, step)
    m_prev = oracle.dequantize_blockwise(cm, am, oracle.SIGNED)
    v_prev = oracle.dequantize_blockwise(cv, av, oracle.UNSIGNED)
    with np.errstate(over="ignore"):
        m = (b1 * m_prev) + (omb1 * g)
        v = (b2 * v_prev) + (omb2 * (g * g))
    return p32, m, v, (eps32, ss, isb), exact32


def _case(rng, n, lr, beta1, beta2, eps, step):
    p = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, n).astype(F32))
    g = rng.normal(0, 1e-3, n).astype(F32)
    g[rng.choice(n, n // 100, replace=False)] *= 100
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(0, 256, n).astype(np.uint8)
    nb = -(-n // oracle.BLOCK)
    am = (10.0 ** rng.uniform(-5, -2, nb)).astype(F32)
    av = (10.0 ** rng.uniform(-9, -5, nb)).astype(F32)
    return _inputs_from_state(rng, oracle.bf16_to_f32(p), g, cm, cv, am, av,
                              lr, beta1, beta2, eps, step)


def _screen(p32, m, v, scalars, exact32, t_exp=T_EXP, pf_exp=PF_EXP, bound=True):
    """Emulated short path and screen over every one-ulp error combination:
    (number of elements the screen passed with a wrong bf16, elements passed)."""
    eps32, ss, isb = scalars
    a, b, t_limit, mode = _short_scalars(eps32, ss, isb)
    want = oracle.f32_to_bf16_rne(exact32)
    passed_any = np.zeros(p32.size, bool)
    if mode is None:
        return 0, passed_any
    subnormal = (v > 0) & (v < F32(2.0 ** -126))
    usable = ~subnormal if mode == "screen+subnormal check" else np.ones(v.size, bool)
    if not bound:
        t_limit = F32(np.inf)
    wrong = 0
    for ds, dd, dr in itertools.product((-1, 0, 1), repeat=3):
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            sq1 = np.where(subnormal, F32(0), _ulp_step(np.sqrt(v), ds)).astype(F32)
            d = _ulp_step((sq1.astype(np.float64) * float(a) + float(b)).astype(F32), dd)
            r = _ulp_step(F32(1.0) / d, dr)
            t = m * r
            pf = p32 - t
            c = _fma_down(np.abs(t), 2.0 ** t_exp, _fma_down(np.abs(pf), 2.0 ** pf_exp,
                                                              np.full_like(pf, 2.0 ** -126)))
            lo, hi = pf - c, pf + c
            bounded = np.abs(t) < t_limit
        ok = usable & bounded & (oracle.f32_to_bf16_rne(lo) == oracle.f32_to_bf16_rne(hi))
        got = oracle.f32_to_bf16_rne(pf)
        wrong += np.count_nonzero(ok & (got != want))
        passed_any |= ok
    return wrong, passed_any


CASES = [
    (1e-3, 0.9, 0.999, 1e-8, 1),
    (1e-3, 0.9, 0.999, 1e-8, 1000),
    (5e-2, 0.5, 0.75, 1e-6, 3),        # updates as large as the parameters
    (2e-2, 0.9, 0.999, 0.0, 7),
]


def _inputs(lr, beta1, beta2, eps, step):
    rng = np.random.default_rng(int(lr * 1e6) + step)
    return _case(rng, 1 << 18, lr, beta1, beta2, eps, step)


@pytest.mark.parametrize("lr,beta1,beta2,eps,step", CASES)
def test_screen_is_sound(lr, beta1, beta2, eps, step):
    p32, m, v, scalars, exact32 = _inputs(lr, beta1, beta2, eps, step)
    # exact results within 16 binary32 ulps of a bf16 rounding boundary: the
    # cases an unsound screen would get wrong
    low = exact32.view(np.uint32) & np.uint32(0xFFFF)
    near = np.abs(low.astype(np.int64) - 0x8000) <= 16
    assert np.count_nonzero(near) > 0
    wrong, passed = _screen(p32, m, v, scalars, exact32)
    assert wrong == 0, f"screen passed {wrong} wrong bf16 results"
    if lr == 1e-3:
        # with ordinary step sizes the short path keeps nearly every element
        assert np.mean(passed) > 0.999


@pytest.mark.parametrize("lr,beta1,beta2,eps,step", CASES)
def test_narrower_screen_is_caught(lr, beta1, beta2, eps, step):
    """The cases are sharp enough to expose a screen 16 times narrower than the
    kernel's (below the error bound): it passes wrong bf16 results."""
    wrong, _ = _screen(*_inputs(lr, beta1, beta2, eps, step), t_exp=T_EXP - 4,
                       pf_exp=PF_EXP - 4)
    assert wrong > 0


def _subnormal_case(eps, lr=5e-2, step=3):
    """Second moments spread over the subnormals and the smallest normals, first
    moments of a comparable size, updates as large as the parameters."""
    rng = np.random.default_rng(77)
    n = 1 << 16
    p = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, n).astype(F32))
    g = (rng.choice([-1.0, 1.0], n) * 10.0 ** rng.uniform(-24, -18, n)).astype(F32)
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(0, 256, n).astype(np.uint8)
    nb = -(-n // oracle.BLOCK)
    am = (10.0 ** rng.uniform(-9, -6, nb)).astype(F32)
    av = (10.0 ** rng.uniform(-44, -36, nb)).astype(F32)
    return _inputs_from_state(rng, oracle.bf16_to_f32(p), g, cm, cv, am, av,
                              lr, 0.5, 0.75, eps, step)


@pytest.mark.parametrize("eps", [1e-8, 1e-6, 0.0])
def test_subnormal_second_moments_without_a_check(eps):
    """No subnormal test runs for eps >= 2^-39 inv_sqrt_bc2, where a flushed square
    root moves the denominator by under 2^-24 of itself, nor for eps = 0, where it
    makes t infinite or NaN and the bound on |t| rejects it.  The screen stays sound."""
    p32, m, v, scalars, exact32 = _subnormal_case(eps)
    assert _short_scalars(*scalars)[3] == "screen"
    subnormal = (v > 0) & (v < F32(2.0 ** -126))
    assert np.count_nonzero(subnormal) > 1000
    wrong, passed = _screen(p32, m, v, scalars, exact32)
    assert wrong == 0
    if eps > 0:
        assert np.count_nonzero(passed & subnormal) > 100


def test_small_eps_needs_the_subnormal_check():
    """With 0 < eps < 2^-39 inv_sqrt_bc2 the flushed square root changes the
    denominator by far more than the bound allows: the kernel checks for subnormal
    second moments, and skipping that check would pass wrong results."""
    p32, m, v, scalars, exact32 = _subnormal_case(1e-30)
    assert _short_scalars(*scalars)[3] == "screen+subnormal check"
    assert _screen(p32, m, v, scalars, exact32)[0] == 0
    eps32, ss, isb = scalars
    a, b, t_limit, _ = _short_scalars(eps32, ss, isb)
    # the same emulation with every lane usable
    subnormal = (v > 0) & (v < F32(2.0 ** -126))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        d = (np.where(subnormal, F32(0), np.sqrt(v)).astype(np.float64) * float(a)
             + float(b)).astype(F32)
        t = m * (F32(1.0) / d)
        pf = p32 - t
        c = _fma_down(np.abs(t), 2.0 ** T_EXP, _fma_down(np.abs(pf), 2.0 ** PF_EXP,
                                                          np.full_like(pf, 2.0 ** -126)))
        ok = (np.abs(t) < t_limit) & (oracle.f32_to_bf16_rne(pf - c) ==
                                      oracle.f32_to_bf16_rne(pf + c))
    want = oracle.f32_to_bf16_rne(exact32)
    assert np.count_nonzero(ok & subnormal & (oracle.f32_to_bf16_rne(pf) != want)) > 0


def _overflow_case():
    """Large first moments over small second moments with eps = 0: m / denominator
    overflows binary32 for part of the elements while step_size * m / denominator
    does not."""
    rng = np.random.default_rng(5)
    n = 1 << 15
    p = oracle.f32_to_bf16_rne(rng.normal(0, 1.0, n).astype(F32))
    g = np.zeros(n, F32)
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(1, 256, n).astype(np.uint8)
    nb = -(-n // oracle.BLOCK)
    am = np.full(nb, 1e30, F32)
    av = (10.0 ** rng.uniform(-22, -16, nb)).astype(F32)
    return _inputs_from_state(rng, oracle.bf16_to_f32(p), g, cm, cv, am, av,
                              1e-3, 0.9, 0.999, 0.0, 1000)


def test_quotient_overflow_needs_the_bound():
    p32, m, v, scalars, exact32 = _overflow_case()
    assert np.count_nonzero(np.isinf(exact32)) > 100          # the sequence overflows
    assert np.count_nonzero(np.isfinite(exact32)) > 100
    assert _screen(p32, m, v, scalars, exact32)[0] == 0
    assert _screen(p32, m, v, scalars, exact32, bound=False)[0] > 0


def test_kernel_uses_the_tested_constants():
    """The exponents tested here are the ones in the kernel's screen_width(), the
    subnormal rule and the bound on |t|."""
    src = open(KERNEL_SRC).read()
    body = src[src.index("float screen_width(float pf, float t)"):]
    body = body[:body.index("}")]
    exps = [int(e) for e in re.findall(r"0x1p(-?\d+)f", body)]
    assert exps == [T_EXP, PF_EXP, -126], exps
    sub = src[src.index("const bool sub_check ="):]
    sub = sub[:sub.index(";")]
    assert f"0x1p{SUB_EXP}" in sub, sub
    lim = src[src.index("k.t_limit ="):]
    lim = lim[:lim.index(";")]
    assert "(ss < 1.0 ? ss : 1.0) * 0x1p127" in lim, lim
    assert math.isclose(float(_short_scalars(F32(1e-8), F32(1e-3), F32(1.0))[2]),
                        1e-3 * 2.0 ** 127, rel_tol=1e-6)
