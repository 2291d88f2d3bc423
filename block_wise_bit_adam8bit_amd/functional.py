"""Tensor-level wrappers with the C ABI's names (include/qopt.h).

Each function checks shapes, dtypes and devices, allocates outputs with torch when
the caller did not pass them, and calls libqopt on torch's current stream.  No
arithmetic of the method happens here.
"""

import ctypes
import threading

import torch

from . import _lib
from ._lib import LIB, QOPT_BLOCK, QOPT_CB_SIGNED, QOPT_CB_UNSIGNED, QOPT_F32, QOPT_BF16

SIGNED = QOPT_CB_SIGNED
UNSIGNED = QOPT_CB_UNSIGNED

_DTYPES = {torch.float32: QOPT_F32, torch.bfloat16: QOPT_BF16}
_cb_lock = threading.Lock()
_cb_cache = {}


def nblocks(n):
    return -(-int(n) // QOPT_BLOCK)


def qopt_codebook_build(kind):
    """Host codebook of ``kind`` (a ctypes ``qopt_codebook``)."""
    cb = _lib.qopt_codebook()
    _lib.check("qopt_codebook_build", LIB.qopt_codebook_build(int(kind), ctypes.byref(cb)))
    return cb


def codebook_bytes(kind):
    """The host codebook as a uint8 CPU tensor (the exact bytes a device copy holds)."""
    cb = qopt_codebook_build(kind)
    raw = ctypes.string_at(ctypes.addressof(cb), ctypes.sizeof(cb))
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8)


def codebook(kind, device=None):
    """Device copy of the codebook of ``kind`` on ``device`` (built and uploaded once
    per process and device; 16-byte aligned)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    if device.type != "cuda":
        raise ValueError("codebooks live in GPU memory")
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    key = (int(kind), device.index)
    with _cb_lock:
        t = _cb_cache.get(key)
        if t is None:
            t = codebook_bytes(kind).to(device)
            assert t.data_ptr() % 16 == 0
            _cb_cache[key] = t
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_cuda(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU")
        if t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def qopt_quantize_blockwise(x, kind=SIGNED, codes=None, absmax=None):
    """Block-wise quantization of a fp32 tensor: returns (codes uint8 [n],
    absmax fp32 [ceil(n / 2048)]), flattened."""
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    n = x.numel()
    if codes is None:
        codes = torch.empty(n, dtype=torch.uint8, device=x.device)
    if absmax is None:
        absmax = torch.empty(nblocks(n), dtype=torch.float32, device=x.device)
    if codes.numel() != n or codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8 with n elements")
    if absmax.numel() != nblocks(n) or absmax.dtype != torch.float32:
        raise ValueError("absmax must be float32 with ceil(n / 2048) elements")
    dev = _check_cuda(x, codes, absmax)
    cb = codebook(kind, dev)
    with torch.cuda.device(dev):
        rc = LIB.qopt_quantize_blockwise(_ptr(cb), _ptr(x), n, _ptr(codes), _ptr(absmax),
                                         ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_quantize_blockwise", rc)
    return codes, absmax


def qopt_dequantize_blockwise(codes, absmax, kind=SIGNED, out=None):
    """Inverse of qopt_quantize_blockwise: returns fp32 [n]."""
    if codes.dtype != torch.uint8 or absmax.dtype != torch.float32:
        raise TypeError("codes must be uint8 and absmax float32")
    n = codes.numel()
    if absmax.numel() != nblocks(n):
        raise ValueError("absmax must hold ceil(n / 2048) elements")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=codes.device)
    if out.numel() != n or out.dtype != torch.float32:
        raise ValueError("out must be float32 with n elements")
    dev = _check_cuda(codes, absmax, out)
    cb = codebook(kind, dev)
    with torch.cuda.device(dev):
        rc = LIB.qopt_dequantize_blockwise(_ptr(cb), _ptr(codes), _ptr(absmax), n, _ptr(out),
                                           ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_dequantize_blockwise", rc)
    return out


def _codec_array(triples):
    """ctypes array of qopt_codec_tensor from (values, codes, absmax) triples."""
    arr = (_lib.qopt_codec_tensor * len(triples))()
    dev = None
    for i, (vals, codes, absmax) in enumerate(triples):
        n = vals.numel()
        if vals.dtype != torch.float32 or codes.dtype != torch.uint8 or \
                absmax.dtype != torch.float32:
            raise TypeError("values must be float32, codes uint8, absmax float32")
        if codes.numel() != n or absmax.numel() != nblocks(n):
            raise ValueError("codes must hold n and absmax ceil(n / 2048) elements")
        d = _check_cuda(vals, codes, absmax)
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError("all tensors of one call must be on the same GPU")
        arr[i] = _lib.qopt_codec_tensor(vals.data_ptr(), codes.data_ptr(), absmax.data_ptr(), n)
    return arr, dev


def qopt_quantize_blockwise_multi(triples, kind=SIGNED):
    """Quantize many fp32 tensors in few launches: ``triples`` is a list of
    (x, codes, absmax) with preallocated uint8 codes [n] and fp32 absmax
    [ceil(n / 2048)], written in place."""
    arr, dev = _codec_array(triples)
    if dev is None:
        return
    with torch.cuda.device(dev):
        rc = LIB.qopt_quantize_blockwise_multi(_ptr(codebook(kind, dev)), arr, len(arr),
                                               ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_quantize_blockwise_multi", rc)


def qopt_dequantize_blockwise_multi(triples, kind=SIGNED):
    """Dequantize many tensors in few launches: ``triples`` is a list of
    (y, codes, absmax) with preallocated fp32 outputs y [n], written in place."""
    arr, dev = _codec_array(triples)
    if dev is None:
        return
    with torch.cuda.device(dev):
        rc = LIB.qopt_dequantize_blockwise_multi(_ptr(codebook(kind, dev)), arr, len(arr),
                                                 ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_dequantize_blockwise_multi", rc)


def make_tensor_array(tensors):
    """ctypes array of qopt_tensor from tuples (param, grad, m_codes, v_codes,
    m_absmax, v_absmax); checks every tuple and returns (array, pdtype, gdtype, device)."""
    if not tensors:
        return (_lib.qopt_tensor * 0)(), QOPT_F32, QOPT_F32, None
    arr = (_lib.qopt_tensor * len(tensors))()
    pdt = gdt = dev = None
    for i, (p, g, cm, cv, am, av) in enumerate(tensors):
        n = p.numel()
        if p.dtype not in _DTYPES or g.dtype not in _DTYPES:
            raise TypeError("params and grads must be float32 or bfloat16")
        if pdt is None:
            pdt, gdt = _DTYPES[p.dtype], _DTYPES[g.dtype]
        elif (_DTYPES[p.dtype], _DTYPES[g.dtype]) != (pdt, gdt):
            raise TypeError("one call takes one (param dtype, grad dtype) pair")
        if g.numel() != n or cm.numel() != n or cv.numel() != n:
            raise ValueError("param, grad and code tensors must have the same size")
        if cm.dtype != torch.uint8 or cv.dtype != torch.uint8:
            raise TypeError("codes must be uint8")
        if am.dtype != torch.float32 or av.dtype != torch.float32:
            raise TypeError("absmax must be float32")
        if am.numel() != nblocks(n) or av.numel() != nblocks(n):
            raise ValueError("absmax must hold ceil(n / 2048) elements")
        d = _check_cuda(p, g, cm, cv, am, av)
        if dev is None:
            dev = d
        elif d != dev:
            raise ValueError("all tensors of one call must be on the same GPU")
        arr[i] = _lib.qopt_tensor(p.data_ptr(), g.data_ptr(), cm.data_ptr(), cv.data_ptr(),
                                  am.data_ptr(), av.data_ptr(), n)
    return arr, pdt, gdt, dev


def qopt_adam8bit_launch_count(tensors, _prepared=None):
    """Kernel launches one qopt_adam8bit_step call makes for this tensor list."""
    arr, pdt, gdt, dev = _prepared if _prepared is not None else make_tensor_array(tensors)
    out = ctypes.c_int64(0)
    _lib.check("qopt_adam8bit_launch_count",
               LIB.qopt_adam8bit_launch_count(arr, len(arr), pdt, gdt, ctypes.byref(out)))
    return out.value


def qopt_adam8bit_traffic_probe(tensors, _prepared=None):
    """Measurement aid: the bytes of one qopt_adam8bit_step over these tensors, moved
    with the step's launch plan and access pattern but no arithmetic (every buffer
    keeps its contents), on torch's current stream."""
    arr, pdt, gdt, dev = _prepared if _prepared is not None else make_tensor_array(tensors)
    if dev is None:
        return
    with torch.cuda.device(dev):
        rc = LIB.qopt_adam8bit_traffic_probe(arr, len(arr), pdt, gdt,
                                             ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_adam8bit_traffic_probe", rc)


def qopt_adam8bit_step(tensors, *, lr, beta1, beta2, eps, step, _prepared=None):
    """One fused 8-bit Adam step over a list of (param, grad, m_codes, v_codes,
    m_absmax, v_absmax) tuples, updated in place on torch's current stream."""
    arr, pdt, gdt, dev = _prepared if _prepared is not None else make_tensor_array(tensors)
    if dev is None:
        return
    hp = _lib.qopt_adam_hparams(float(lr), float(beta1), float(beta2), float(eps), int(step))
    with torch.cuda.device(dev):
        rc = LIB.qopt_adam8bit_step(arr, len(arr), pdt, gdt, _ptr(codebook(SIGNED, dev)),
                                    _ptr(codebook(UNSIGNED, dev)), ctypes.byref(hp),
                                    ctypes.c_void_p(_lib.stream_handle(dev)))
    _lib.check("qopt_adam8bit_step", rc)


def qopt_pattern_probe_names():
    """Descriptions of the bytes-only access patterns (a measurement aid)."""
    return [LIB.qopt_pattern_probe_name(i).decode() for i in range(LIB.qopt_pattern_probe_count())]


def qopt_pattern_probe(pattern, params, grads, m_codes, v_codes):
    """Measurement aid: one pass of access pattern ``pattern`` over flat buffers holding
    whole blocks (fp32 params, bf16 grads, uint8 codes), every buffer left as it was."""
    n = params.numel()
    if n % QOPT_BLOCK or grads.numel() != n or m_codes.numel() != n or v_codes.numel() != n:
        raise ValueError("the probe moves whole blocks of equally long flat buffers")
    if params.dtype != torch.float32 or grads.dtype != torch.bfloat16 or \
            m_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("the probe moves fp32 params, bf16 grads and uint8 codes")
    rc = LIB.qopt_pattern_probe(int(pattern), _ptr(params), _ptr(grads), _ptr(m_codes),
                                _ptr(v_codes), n // QOPT_BLOCK,
                                ctypes.c_void_p(_lib.stream_handle(params.device)))
    _lib.check("qopt_pattern_probe", rc)
