"""Soundness of the step kernel's screen for bf16 parameters (CPU only).

For bf16 parameters the kernel may compute p - t with the hardware square root and
reciprocal (each within one ulp; checked on the hardware over every normal binary32)
and keep that result only if both ends of [pf - c, pf + c] round to the same bf16
bits, with c = |t| 2^-19 + |pf| 2^-22 + 2^-126 (each product taken exactly, one
rounding).  Here the short path is emulated in binary32 with every combination of
one-ulp errors in the two hardware results, and wherever the screen passes, its bf16
result must equal the oracle's (the correctly rounded sequence).  The inputs put
many exact results next to bf16 rounding boundaries (updates as large as the
parameters), so an unsound width would show: a screen 16 times narrower passes
wrong results in every case.
"""

import itertools
import os
import re

import numpy as np
import pytest

import oracle

F32 = np.float32
# binary exponents of the screen's two factors, as in the kernel's screen_width()
T_EXP, PF_EXP = -19, -22
KERNEL_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "block_wise_bit_adam8bit_amd", "csrc", "qopt_kernels.hip")


def _ulp_step(x, k):
    """x moved by k ulps (k in -1, 0, 1) along the binary32 line."""
    if k == 0:
        return x
    return np.nextafter(x, F32(np.inf) if k > 0 else F32(-np.inf)).astype(F32)


def _fma_down(a, b, c):
    """a*b + c with one rounding, then one ulp toward zero: never above the fused
    multiply-add the kernel performs (a, b, c non-negative here)."""
    r = (a.astype(np.float64) * float(b) + c.astype(np.float64)).astype(F32)
    return np.nextafter(r, F32(0)).astype(F32)


def _case(rng, n, lr, beta1, beta2, eps, step):
    p = oracle.f32_to_bf16_rne(rng.normal(0, 0.02, n).astype(F32))
    g = rng.normal(0, 1e-3, n).astype(F32)
    g[rng.choice(n, n // 100, replace=False)] *= 100
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(0, 256, n).astype(np.uint8)
    nb = -(-n // oracle.BLOCK)
    am = (10.0 ** rng.uniform(-5, -2, nb)).astype(F32)
    av = (10.0 ** rng.uniform(-9, -5, nb)).astype(F32)
    hp = dict(lr=lr, beta1=beta1, beta2=beta2, eps=eps, step=step)
    p32 = oracle.bf16_to_f32(p)
    exact32 = oracle.adam8bit_step(p32, g, cm, cv, am, av, **hp)[0]
    # the moments, as the kernel forms them (same binary32 operations)
    b1, b2, omb1, omb2, eps32, ss, isb = oracle.adam_scalars(lr, beta1, beta2, eps, step)
    m_prev = oracle.dequantize_blockwise(cm, am, oracle.SIGNED)
    v_prev = oracle.dequantize_blockwise(cv, av, oracle.UNSIGNED)
    m = (b1 * m_prev) + (omb1 * g)
    v = (b2 * v_prev) + (omb2 * (g * g))
    return p32, m, v, (eps32, ss, isb), exact32


def _screen(p32, m, v, scalars, exact32, t_exp=T_EXP, pf_exp=PF_EXP):
    """Emulated short path and screen over every one-ulp error combination:
    (number of elements the screen passed with a wrong bf16, elements passed)."""
    eps32, ss, isb = scalars
    want = oracle.f32_to_bf16_rne(exact32)
    usable = (v == 0) | (v >= F32(2.0 ** -96))
    passed_any = np.zeros(p32.size, bool)
    wrong = 0
    for ds, dr in itertools.product((-1, 0, 1), repeat=2):
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            sq1 = _ulp_step(np.sqrt(v), ds)
            denom = (sq1 * isb) + eps32
            r = _ulp_step(F32(1.0) / denom, dr)
            t = ss * (m * r)
            pf = p32 - t
            c = _fma_down(np.abs(t), 2.0 ** t_exp, _fma_down(np.abs(pf), 2.0 ** pf_exp,
                                                              np.full_like(pf, 2.0 ** -126)))
            lo, hi = pf - c, pf + c
        ok = usable & ~np.isnan(pf) & (oracle.f32_to_bf16_rne(lo) == oracle.f32_to_bf16_rne(hi))
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


def test_kernel_uses_the_tested_width():
    """The exponents tested here are the ones in the kernel's screen_width()."""
    src = open(KERNEL_SRC).read()
    body = src[src.index("float screen_width(float pf, float t)"):]
    body = body[:body.index("}")]
    exps = [int(e) for e in re.findall(r"0x1p(-?\d+)f", body)]
    assert exps == [T_EXP, PF_EXP, -126], exps
