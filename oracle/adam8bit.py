"""Oracle: one 8-bit Adam step with block-wise dynamic-tree state (test infrastructure only).

Source: 8-bit optimizers summary page.
* §1: Adam keeps, per parameter, the first moment (running mean of the
  gradients) and the second moment (uncentred variance of the gradients).
* §2 (opening paragraph): the optimizer state is stored in low precision in GPU
  memory, dequantized to a higher precision to update the parameters, and stored
  back in low precision.
* §2 "Block-wise Quantization" and "Dynamic Quantization": the first moment uses
  the signed dynamic-tree code, the always-positive second moment the unsigned one,
  both in blocks of 2048 with a per-block absmax (blockwise.py).
Master weights are fp32 (the DeepSpeed / FSDP mixed-precision page: both
frameworks keep fp32 master parameters for the optimizer step); bf16 parameters
are also supported, updated in place.

Readings where the pages are silent:
* Textbook Adam with bias correction, epsilon added outside the square root, no
  weight decay:  p <- p - lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps).
* The update uses the fp32 moments before they are requantized; requantization only
  affects the next step.
* Hyper-parameters are binary32 values.  b^t is evaluated in binary64 by
  square-and-multiply over the bits of t (least significant bit first), and
  step_size = fl32(lr / (1 - b1^t)), inv_sqrt_bc2 = fl32(1 / sqrt(1 - b2^t)) are
  evaluated in binary64 and rounded once.  1 - b1 and 1 - b2 are binary32
  subtractions.
* Per element, binary32, one rounding per operation, in this order:
      g      = fp32(grad)                              (bf16 -> fp32 is exact)
      m_prev = table_s[cm] * Am        v_prev = table_u[cv] * Av
      m      = (b1 * m_prev) + ((1 - b1) * g)
      v      = (b2 * v_prev) + ((1 - b2) * (g * g))
      denom  = (sqrt(v) * inv_sqrt_bc2) + eps          (correctly rounded sqrt)
      u      = m / denom                               (correctly rounded divide)
      p'     = p - (step_size * u)
  bf16 parameters: p is widened exactly, p' is rounded to bf16 (nearest, ties to
  even).  Then m and v are requantized block-wise (signed / unsigned).
* Blocks of zero gradient still get the full update (m and v decay, p moves).
"""

import math

import numpy as np

from .codebook import BLOCK, SIGNED, UNSIGNED, decode_table
from .blockwise import quantize_blockwise

F32 = np.float32


def _pow_f64(b, t):
    """b^t in binary64, square-and-multiply over the bits of t from the lowest."""
    result = 1.0
    base = float(b)
    e = int(t)
    while e:
        if e & 1:
            result = result * base
        base = base * base
        e >>= 1
    return result


def adam_scalars(lr, beta1, beta2, eps, step):
    """Per-step binary32 scalars: (b1, b2, omb1, omb2, eps, step_size, inv_sqrt_bc2)."""
    if int(step) < 1:
        raise ValueError("step is 1-based")
    b1, b2 = F32(beta1), F32(beta2)
    lr32, eps32 = F32(lr), F32(eps)
    bc1 = 1.0 - _pow_f64(float(b1), step)
    bc2 = 1.0 - _pow_f64(float(b2), step)
    step_size = F32(float(lr32) / bc1)
    inv_sqrt_bc2 = F32(1.0 / math.sqrt(bc2))
    omb1 = F32(1.0) - b1
    omb2 = F32(1.0) - b2
    return b1, b2, omb1, omb2, eps32, step_size, inv_sqrt_bc2


def bf16_to_f32(u16):
    """Widen bf16 bit patterns (uint16) to fp32, exactly."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x):
    """Round fp32 to bf16 bit patterns (uint16), nearest with ties to even.

    Finite inputs only (NaN handling is outside the contract).
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))
    return ((bits + bias) >> np.uint64(16)).astype(np.uint16)


def _expand_absmax(absmax, n):
    return np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)[:n]


def adam8bit_step(p, g, cm, cv, am, av, *, lr, beta1, beta2, eps, step,
                  param_dtype="f32", grad_dtype="f32"):
    """One 8-bit Adam step on one tensor; returns (p', cm', cv', am', av').

    p: fp32 array (param_dtype "f32") or bf16 bit patterns as uint16 ("bf16").
    g: fp32 array or bf16 bit patterns.  cm, cv: uint8 codes.  am, av: fp32 absmax
    with ceil(n / 2048) entries.  Inputs are not modified.
    Parity: pinned (closed-form first step, beta = 0 special case, lossless
    constant-magnitude blocks against torch.optim.Adam over many steps, binary64
    evaluation of the update within its error bound).
    """
    b1, b2, omb1, omb2, eps32, step_size, inv_sqrt_bc2 = adam_scalars(
        lr, beta1, beta2, eps, step)
    p = np.asarray(p).reshape(-1)
    n = p.size
    p32 = bf16_to_f32(p) if param_dtype == "bf16" else np.asarray(p, dtype=F32)
    g32 = bf16_to_f32(g) if grad_dtype == "bf16" else np.asarray(g, dtype=F32)
    g32 = g32.reshape(-1)
    cm = np.asarray(cm, dtype=np.uint8).reshape(-1)
    cv = np.asarray(cv, dtype=np.uint8).reshape(-1)
    if not (g32.size == cm.size == cv.size == n):
        raise ValueError("size mismatch")
    nb = -(-n // BLOCK)
    if np.size(am) != nb or np.size(av) != nb:
        raise ValueError("absmax arrays must hold ceil(n / 2048) entries")

    m_prev = decode_table(SIGNED)[cm] * _expand_absmax(am, n)
    v_prev = decode_table(UNSIGNED)[cv] * _expand_absmax(av, n)
    m = (b1 * m_prev) + (omb1 * g32)
    v = (b2 * v_prev) + (omb2 * (g32 * g32))
    denom = (np.sqrt(v) * inv_sqrt_bc2) + eps32
    u = m / denom
    p_new32 = p32 - (step_size * u)
    p_new = f32_to_bf16_rne(p_new32) if param_dtype == "bf16" else p_new32

    cm_new, am_new = quantize_blockwise(m, SIGNED)
    cv_new, av_new = quantize_blockwise(v, UNSIGNED)
    return p_new, cm_new, cv_new, am_new, av_new


def adam8bit_step_multi(tensors, **hp):
    """Multi-tensor step: every tensor is independent and shares t and the
    hyper-parameters.  ``tensors`` is a list of (p, g, cm, cv, am, av)."""
    return [adam8bit_step(*t, **hp) for t in tensors]


def adam_update_f64(p32, m32, v32, *, lr, beta1, beta2, eps, step):
    """The same parameter update from the same binary32 p, m, v, evaluated in
    binary64 with exact bias corrections: a yardstick for the binary32 rounding
    error of ``adam8bit_step``'s parameter path (pinning only)."""
    b1 = float(F32(beta1))
    b2 = float(F32(beta2))
    t = int(step)
    bc1 = 1.0 - b1 ** t
    bc2 = 1.0 - b2 ** t
    p = np.asarray(p32, dtype=np.float64)
    m = np.asarray(m32, dtype=np.float64)
    v = np.asarray(v32, dtype=np.float64)
    denom = np.sqrt(v) / math.sqrt(bc2) + float(F32(eps))
    return p - (float(F32(lr)) / bc1) * m / denom
