"""Pins for the oracle's 8-bit Adam step (CPU only).

Facts from the pages: Adam keeps a first moment (mean of gradients) and a second
moment (uncentred variance) (summary page §1); the 8-bit optimizer dequantizes its
state, updates in higher precision and stores the state back in 8 bits (§2); the
memory accounting of §1 (4 GB per 1B fp32 values, Adam state 50 %, 38 % saving).
Independent yardsticks: closed forms, beta = 0 special cases, torch.optim.Adam on
inputs the 8-bit state represents without loss, exact rational arithmetic.
"""

from fractions import Fraction
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import SIGNED, UNSIGNED, BLOCK

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
# torch.optim.Adam forms 1 - beta in binary64; handing it the binary32 betas makes
# its scalars equal to the binary32 hyper-parameters the 8-bit step uses.
TORCH_BETAS = (float(np.float32(0.9)), float(np.float32(0.999)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _zero_state(n):
    nb = -(-n // BLOCK)
    return (np.zeros(n, np.uint8), np.zeros(n, np.uint8),
            np.zeros(nb, np.float32), np.zeros(nb, np.float32))


def _tol_ok(p, p_ref, lr, rel=1e-6, p_start=None):
    """|p - p_ref| <= rel * max(|p_ref|, lr), or rel * max(|p_ref|, |p_start|, lr)
    when two implementations with different rounding are followed over several
    steps (values that cross zero keep the rounding error of their start)."""
    p = np.asarray(p, np.float64)
    p_ref = np.asarray(p_ref, np.float64)
    scale = np.maximum(np.abs(p_ref), lr)
    if p_start is not None:
        scale = np.maximum(scale, np.abs(np.asarray(p_start, np.float64)))
    return np.all(np.abs(p - p_ref) <= rel * scale)


# ----------------------------------------------------------------- scalars


@pytest.mark.parametrize("t", [1, 2, 3, 10, 1000, 123457, 10 ** 7])
@pytest.mark.parametrize("beta", [0.9, 0.999, 0.5, 0.0])
def test_bias_correction_scalars_against_exact(t, beta):
    """step_size and inv_sqrt_bc2 are within one binary32 ulp of the exact values
    computed with rationals (binary64 only for the final square root)."""
    lr = 1e-3
    b = Fraction(float(np.float32(beta)))
    if b == 0 or t * -math.log2(float(b)) > 400:
        bc = Fraction(1) - (b ** t if b == 0 else Fraction(0))  # b^t < 2^-400
    else:
        bc = 1 - b ** t
    _, _, _, _, _, step_size, inv_sqrt = oracle.adam_scalars(lr, beta, beta, 1e-8, t)
    exact_step = Fraction(float(np.float32(lr))) / bc
    ulp = Fraction(float(np.spacing(step_size)))
    assert abs(Fraction(float(step_size)) - exact_step) <= ulp
    exact_inv = 1.0 / math.sqrt(float(bc))
    assert abs(float(inv_sqrt) - exact_inv) <= 1.01 * float(np.spacing(inv_sqrt))
    if beta == 0.0:
        assert step_size == np.float32(lr) and inv_sqrt == np.float32(1.0)


def test_one_minus_beta_is_exact_for_usual_betas():
    _, _, omb1, omb2, *_ = oracle.adam_scalars(1e-3, 0.9, 0.999, 1e-8, 1)
    assert Fraction(float(omb1)) == 1 - Fraction(float(np.float32(0.9)))
    assert Fraction(float(omb2)) == 1 - Fraction(float(np.float32(0.999)))


# -------------------------------------------------------------------- bf16


def test_bf16_helpers_match_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-30, 1000),
                        [0.0, -0.0, 1.0, 3.0e38]]).astype(np.float32)
    # exact ties: mantissa low half == 0x8000
    ties = (rng.integers(0, 2 ** 16, 500, dtype=np.uint32) << 16) | 0x8000
    ties = ties & 0x7F7FFFFF
    x = np.concatenate([x, ties.astype(np.uint32).view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_rne(x), want)
    back = oracle.bf16_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16)
                          .float().numpy())


# ------------------------------------------------------------- first step


def test_first_step_closed_form_and_torch_adam():
    """From zero state: m = (1-b1) g, v = (1-b2) g^2, so p1 = p0 - lr g / (|g| + eps)."""
    rng = np.random.default_rng(2)
    n = 3 * BLOCK + 11
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    g[::97] *= 100
    p1, cm, cv, am, av = oracle.adam8bit_step(p0, g, *_zero_state(n), step=1, **HP)
    gd = g.astype(np.float64)
    closed = p0 - HP["lr"] * gd / (np.abs(gd) + HP["eps"])
    assert _tol_ok(p1, closed, HP["lr"])
    pt = torch.from_numpy(p0.copy()).requires_grad_(False)
    pt = torch.nn.Parameter(pt)
    opt = torch.optim.Adam([pt], lr=HP["lr"], betas=TORCH_BETAS,
                           eps=HP["eps"], foreach=False)
    pt.grad = torch.from_numpy(g.copy())
    opt.step()
    assert _tol_ok(p1, pt.detach().numpy(), HP["lr"])
    # the stored state is the block-wise quantization of the first moments
    m1 = np.float32(1 - np.float32(0.9)) * g
    c_ref, a_ref = oracle.quantize_blockwise(m1, SIGNED)
    assert np.array_equal(cm, c_ref) and np.array_equal(am, a_ref)


def test_betas_zero_special_case():
    """b1 = b2 = 0: every step is p - lr g / (|g| + eps) whatever the stored state,
    and the stored codes are quantize(g) and quantize(g*g)."""
    rng = np.random.default_rng(4)
    n = 2 * BLOCK + 100
    p = rng.normal(0, 0.02, n).astype(np.float32)
    cm = rng.integers(0, 256, n).astype(np.uint8)
    cv = rng.integers(0, 256, n).astype(np.uint8)
    am = np.abs(rng.normal(0, 1, 3)).astype(np.float32)
    av = np.abs(rng.normal(0, 1, 3)).astype(np.float32)
    hp = dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8)
    for step in (1, 2, 7):
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        p2, cm2, cv2, am2, av2 = oracle.adam8bit_step(p, g, cm, cv, am, av, step=step, **hp)
        gd = g.astype(np.float64)
        assert _tol_ok(p2, p - 1e-3 * gd / (np.abs(gd) + 1e-8), 1e-3)
        assert np.array_equal(cm2, oracle.quantize_blockwise(g, SIGNED)[0])
        assert np.array_equal(cv2, oracle.quantize_blockwise(g * g, UNSIGNED)[0])
        p, cm, cv, am, av = p2, cm2, cv2, am2, av2


# ------------------------------------------------------------ many steps


def test_lossless_blocks_follow_fp32_adam():
    """Gradients whose magnitude is constant within each block (signs fixed per
    element) keep |m| and v equal across the block, so every element sits at the
    block absmax, which the code 1.0 stores exactly.  The 8-bit trajectory then
    equals 32-bit Adam (torch.optim.Adam) up to rounding, step after step."""
    rng = np.random.default_rng(6)
    nblk = 4
    n = nblk * BLOCK
    p = rng.normal(0, 0.02, n).astype(np.float32)
    p_start = p.copy()
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    state = _zero_state(n)
    pt = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.Adam([pt], lr=HP["lr"], betas=TORCH_BETAS,
                           eps=HP["eps"], foreach=False)
    for step in range(1, 21):
        mag = np.repeat(np.abs(rng.normal(0, 1e-3, nblk)).astype(np.float32), BLOCK)
        g = sign * mag
        p, cm, cv, am, av = oracle.adam8bit_step(p, g, *state, step=step, **HP)
        state = (cm, cv, am, av)
        pt.grad = torch.from_numpy(g.copy())
        opt.step()
        assert np.all((cm & 0x7F) == 0x7F) and np.all(cv == 0xFF)
        assert _tol_ok(p, pt.detach().numpy(), HP["lr"], p_start=p_start), step


def test_trajectory_tracks_fp32_adam_statistically():
    """On generic data the 8-bit state differs from fp32 Adam by quantization
    error only: after 10 steps the parameter displacement agrees closely."""
    rng = np.random.default_rng(8)
    n = 16 * BLOCK
    p0 = rng.normal(0, 0.02, n).astype(np.float32)
    p = p0.copy()
    state = _zero_state(n)
    pt = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.Adam([pt], lr=HP["lr"], betas=TORCH_BETAS,
                           eps=HP["eps"], foreach=False)
    for step in range(1, 11):
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        p, *state = oracle.adam8bit_step(p, g, *state, step=step, **HP)
        pt.grad = torch.from_numpy(g)
        opt.step()
    d8 = p.astype(np.float64) - p0
    d32 = pt.detach().numpy().astype(np.float64) - p0
    rel = np.linalg.norm(d8 - d32) / np.linalg.norm(d32)
    assert rel < 0.05, rel


def test_parameter_path_within_binary64_yardstick():
    """The binary32 update is within a few ulps of the same update in binary64."""
    rng = np.random.default_rng(10)
    n = 4 * BLOCK
    p = rng.normal(0, 0.02, n).astype(np.float32)
    state = _zero_state(n)
    for step in range(1, 6):
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        cm, cv, am, av = state
        m_prev = oracle.dequantize_blockwise(cm, am, SIGNED)
        v_prev = oracle.dequantize_blockwise(cv, av, UNSIGNED)
        b1, b2, omb1, omb2, *_ = oracle.adam_scalars(step=step, **HP)
        m = (b1 * m_prev) + (omb1 * g)
        v = (b2 * v_prev) + (omb2 * (g * g))
        p_new, *state = oracle.adam8bit_step(p, g, *state, step=step, **HP)
        ref = oracle.adam_update_f64(p, m, v, step=step, **HP)
        upd = np.abs(ref - p)
        err = np.abs(p_new.astype(np.float64) - ref)
        assert np.all(err <= 2 ** -24 * np.abs(ref) + 8 * 2 ** -24 * upd + 1e-30)
        assert _tol_ok(p_new, ref, HP["lr"])
        p = p_new


def test_bf16_params_round_once():
    rng = np.random.default_rng(12)
    n = BLOCK + 5
    p32 = rng.normal(0, 0.02, n).astype(np.float32)
    pb = oracle.f32_to_bf16_rne(p32)
    g = oracle.f32_to_bf16_rne(rng.normal(0, 5e-4, n).astype(np.float32))
    out_b = oracle.adam8bit_step(pb, g, *_zero_state(n), step=1, param_dtype="bf16",
                                 grad_dtype="bf16", **HP)
    out_f = oracle.adam8bit_step(oracle.bf16_to_f32(pb), oracle.bf16_to_f32(g),
                                 *_zero_state(n), step=1, **HP)
    assert np.array_equal(out_b[0], oracle.f32_to_bf16_rne(out_f[0]))
    for a, b in zip(out_b[1:], out_f[1:]):
        assert np.array_equal(a, b)


def test_zero_blocks_stay_zero_and_rows_decay():
    """A block with zero gradient and zero state stays zero and p does not move; a
    block with zero gradient but nonzero state decays and p still moves."""
    rng = np.random.default_rng(13)
    n = 3 * BLOCK
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = np.zeros(n, np.float32)
    g[2 * BLOCK:] = rng.normal(0, 1e-3, BLOCK)
    p1, cm, cv, am, av = oracle.adam8bit_step(p, g, *_zero_state(n), step=1, **HP)
    assert np.array_equal(p1[: 2 * BLOCK], p[: 2 * BLOCK])
    assert am[0] == 0 and av[0] == 0 and not cm[:BLOCK].any()
    g2 = np.zeros(n, np.float32)
    p2, cm2, cv2, am2, av2 = oracle.adam8bit_step(p1, g2, cm, cv, am, av, step=2, **HP)
    assert np.array_equal(p2[: 2 * BLOCK], p[: 2 * BLOCK])
    assert am2[2] < am[2] and av2[2] < av[2]
    assert np.any(p2[2 * BLOCK:] != p1[2 * BLOCK:])


def test_multi_tensor_blocks_restart_per_tensor():
    rng = np.random.default_rng(14)
    sizes = [2049, 5, 4096]
    ts = []
    for n in sizes:
        ts.append((rng.normal(0, 0.02, n).astype(np.float32),
                   rng.normal(0, 1e-3, n).astype(np.float32), *_zero_state(n)))
    multi = oracle.adam8bit_step_multi(ts, step=1, **HP)
    for t, out in zip(ts, multi):
        single = oracle.adam8bit_step(*t, step=1, **HP)
        for a, b in zip(out, single):
            assert np.array_equal(a, b)
    # concatenating would share blocks across tensor boundaries: different absmax
    cat = [np.concatenate([t[i] for t in ts]) for i in range(2)]
    one = oracle.adam8bit_step(cat[0], cat[1], *_zero_state(sum(sizes)), step=1, **HP)
    assert one[3].size != sum(o[3].size for o in multi)


def test_memory_accounting_matches_page():
    """Bytes per parameter of the buffers the step touches reproduce the page's
    accounting: fp32 Adam state is half the memory of weights + grads + state, and
    8-bit block-wise state saves about 38 %."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    n = 10 ** 9
    nb = -(-n // BLOCK)
    w = g = 4 * n
    fp32_state = 2 * 4 * n
    assert fp32_state / 1e9 == 2 * facts["fp32_gb_per_billion_params"]["value"]
    assert fp32_state / (w + g + fp32_state) == facts["adam_state_share_fp32"]["value"]
    cm, cv, am, av = _zero_state(BLOCK * 4)
    per_param_state = (cm.nbytes + cv.nbytes + am.nbytes + av.nbytes) / (BLOCK * 4)
    q8_state = per_param_state * n
    saving = 1 - (w + g + q8_state) / (w + g + fp32_state)
    assert abs(saving - facts["memory_saving_8bit_vs_32bit"]["value"]) < 0.01
    assert nb * 2 * 4 / n < 0.004
