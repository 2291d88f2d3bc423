"""Moment codec for optimizer checkpoints: fp32 Adam moments <-> block-wise 8-bit state.

The checkpoint-compression page (ExCP, information.bz) stores optimizer momentum as a
codebook plus one index per element.  Here the codebook is the dynamic-tree code of
the 8-bit optimizer summary page (§2 "Dynamic Quantization") and the indices are its
code bytes, with one fp32 absmax per 2048-element block (§2 "Block-wise
Quantization"): the first moment through the signed code, the second moment through
the unsigned one.  fp32 moments (4 bytes per value) become 1 byte per value plus
4 bytes per block.  Both directions run in libqopt's quantize / dequantize kernels;
this module only arranges tensors.

A 32-bit Adam checkpoint converted this way is exactly the state ``Adam8bit`` keeps,
so training can switch optimizers mid-run; the reverse direction gives fp32 moments
that ``torch.optim.Adam`` can load.
"""

import torch

from .functional import (SIGNED, UNSIGNED, nblocks, qopt_dequantize_blockwise,
                         qopt_dequantize_blockwise_multi, qopt_quantize_blockwise,
                         qopt_quantize_blockwise_multi)


def compress_moments(exp_avg, exp_avg_sq):
    """Block-wise 8-bit codes of one parameter's Adam moments (GPU tensors of any
    float dtype and shape; widened to fp32, which is exact for bf16 and fp16).
    Returns {"m_codes", "m_absmax", "v_codes", "v_absmax"}, flat."""
    if exp_avg.shape != exp_avg_sq.shape:
        raise ValueError("exp_avg and exp_avg_sq must have the same shape")
    m = exp_avg.detach().reshape(-1).to(torch.float32).contiguous()
    v = exp_avg_sq.detach().reshape(-1).to(torch.float32).contiguous()
    m_codes, m_absmax = qopt_quantize_blockwise(m, SIGNED)
    v_codes, v_absmax = qopt_quantize_blockwise(v, UNSIGNED)
    return {"m_codes": m_codes, "m_absmax": m_absmax, "v_codes": v_codes, "v_absmax": v_absmax}


def decompress_moments(state, shape=None, dtype=torch.float32):
    """fp32 (or ``dtype``) moments from block-wise 8-bit codes: (exp_avg, exp_avg_sq)."""
    m = qopt_dequantize_blockwise(state["m_codes"], state["m_absmax"], SIGNED)
    v = qopt_dequantize_blockwise(state["v_codes"], state["v_absmax"], UNSIGNED)
    if shape is not None:
        m, v = m.view(shape), v.view(shape)
    if dtype != torch.float32:
        m, v = m.to(dtype), v.to(dtype)
    return m, v


def compress_moments_multi(pairs):
    """``compress_moments`` for many parameters at once: ``pairs`` is a list of
    (exp_avg, exp_avg_sq) on one GPU; two multi-tensor codec calls in all."""
    flat, out = [], []
    for m, v in pairs:
        if m.shape != v.shape:
            raise ValueError("exp_avg and exp_avg_sq must have the same shape")
        m = m.detach().reshape(-1).to(torch.float32).contiguous()
        v = v.detach().reshape(-1).to(torch.float32).contiguous()
        n = m.numel()
        st = {"m_codes": torch.empty(n, dtype=torch.uint8, device=m.device),
              "m_absmax": torch.empty(nblocks(n), dtype=torch.float32, device=m.device),
              "v_codes": torch.empty(n, dtype=torch.uint8, device=m.device),
              "v_absmax": torch.empty(nblocks(n), dtype=torch.float32, device=m.device)}
        flat.append((m, v))
        out.append(st)
    qopt_quantize_blockwise_multi([(m, st["m_codes"], st["m_absmax"])
                                   for (m, _), st in zip(flat, out)], SIGNED)
    qopt_quantize_blockwise_multi([(v, st["v_codes"], st["v_absmax"])
                                   for (_, v), st in zip(flat, out)], UNSIGNED)
    return out


def decompress_moments_multi(states, shapes=None):
    """``decompress_moments`` for many parameters at once (fp32 results)."""
    outs = []
    for st in states:
        n = st["m_codes"].numel()
        dev = st["m_codes"].device
        outs.append((torch.empty(n, dtype=torch.float32, device=dev),
                     torch.empty(n, dtype=torch.float32, device=dev)))
    qopt_dequantize_blockwise_multi([(m, st["m_codes"], st["m_absmax"])
                                     for (m, _), st in zip(outs, states)], SIGNED)
    qopt_dequantize_blockwise_multi([(v, st["v_codes"], st["v_absmax"])
                                     for (_, v), st in zip(outs, states)], UNSIGNED)
    if shapes is not None:
        outs = [(m.view(s), v.view(s)) for (m, v), s in zip(outs, shapes)]
    return outs
