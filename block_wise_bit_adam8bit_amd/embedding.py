"""Stable Embedding layer: wrappers with the C ABI's names (include/qopt_embedding.h),
an autograd function and a torch module.

The layer is the one of the 8-bit optimizers summary page, §2 "Stable Embedding
Layer": a Xavier-uniform initialised table followed by a layer normalisation, which
the YaLM-100B training page ("Stabilizations. LayerNorm") also places right after
the embedding.  Every step runs in libqopt's HIP kernels; torch allocates outputs,
workspaces and zeroed gradient buffers and supplies the current stream.
"""

import ctypes

import torch

from . import _lib
from ._lib import LIB, QOPT_BF16, QOPT_F32

_DT = {torch.float32: QOPT_F32, torch.bfloat16: QOPT_BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _check(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _dtype_code(t, what):
    if t.dtype not in _DT:
        raise TypeError(f"{what} must be float32 or bfloat16, not {t.dtype}")
    return _DT[t.dtype]


def qopt_embedding_xavier_init(weight, seed=0):
    """Fill a [rows, dim] table in place with the Xavier-uniform values of ``seed``."""
    _check(weight)
    if weight.dim() != 2:
        raise ValueError("the table must be 2-D [rows, dim]")
    rows, dim = weight.shape
    _lib.check("qopt_embedding_xavier_init",
               LIB.qopt_embedding_xavier_init(_ptr(weight), _dtype_code(weight, "weight"), rows,
                                              dim, int(seed) & 0xFFFFFFFFFFFFFFFF,
                                              _lib.stream_handle(weight.device)))
    return weight


def qopt_stable_embedding_forward(weight, idx, gamma, beta, eps=1e-5, out_dtype=None, *,
                                  save_stats=True, bad_count=None, out=None, mean=None,
                                  rstd=None):
    """LayerNorm(weight[idx]): returns (out [*idx.shape, dim], mean, rstd), the last
    two [idx.numel()] float32 (None unless ``save_stats``).  ``bad_count`` (int32
    [1] on the device) counts out-of-range indices, whose rows come out NaN.  Output
    buffers may be passed in (``out``, ``mean``, ``rstd``)."""
    out_dtype = weight.dtype if out_dtype is None else out_dtype
    _check(weight, idx, gamma, beta, bad_count)
    if weight.dim() != 2:
        raise ValueError("the table must be 2-D [rows, dim]")
    if idx.dtype != torch.int64:
        raise TypeError("indices must be int64")
    rows, dim = weight.shape
    if gamma.shape != (dim,) or beta.shape != (dim,) or gamma.dtype != torch.float32 \
            or beta.dtype != torch.float32:
        raise ValueError("gamma and beta must be float32 [dim]")
    if bad_count is not None and (bad_count.dtype != torch.int32 or bad_count.numel() < 1):
        raise ValueError("bad_count must be an int32 device tensor")
    ntok = idx.numel()
    if out is None:
        out = torch.empty(*idx.shape, dim, dtype=out_dtype, device=weight.device)
    elif out.shape != (*idx.shape, dim) or out.dtype != out_dtype:
        raise ValueError("out must have shape [*idx.shape, dim] and dtype out_dtype")
    if save_stats:
        if mean is None:
            mean = torch.empty(ntok, dtype=torch.float32, device=weight.device)
        if rstd is None:
            rstd = torch.empty(ntok, dtype=torch.float32, device=weight.device)
        if mean.shape != (ntok,) or rstd.shape != (ntok,) or mean.dtype != torch.float32 \
                or rstd.dtype != torch.float32:
            raise ValueError("mean and rstd must be float32 [ntokens]")
    else:
        mean = rstd = None
    _check(out, mean, rstd)
    _lib.check("qopt_stable_embedding_forward",
               LIB.qopt_stable_embedding_forward(
                   _ptr(weight), _dtype_code(weight, "weight"), rows, dim, _ptr(idx), ntok,
                   _ptr(gamma), _ptr(beta), float(eps), _ptr(out), _dtype_code(out, "output"),
                   _ptr(mean), _ptr(rstd), _ptr(bad_count), _lib.stream_handle(weight.device)))
    return out, mean, rstd


def backward_workspace_bytes(ntokens, dim):
    n = ctypes.c_size_t(0)
    _lib.check("qopt_stable_embedding_backward_workspace",
               LIB.qopt_stable_embedding_backward_workspace(int(ntokens), int(dim),
                                                            ctypes.byref(n)))
    return n.value


def qopt_stable_embedding_backward(weight, idx, gamma, mean, rstd, dout, dweight=None, *,
                                   dgamma=None, dbeta=None, workspace=None):
    """Gradients for upstream ``dout`` [*idx.shape, dim]: returns (dweight [rows, dim]
    float32, accumulated into ``dweight`` if given, else into zeros; dgamma, dbeta
    [dim] float32).  ``dgamma``, ``dbeta`` and a uint8 ``workspace`` of at least
    backward_workspace_bytes(ntokens, dim) bytes may be passed in."""
    rows, dim = weight.shape
    ntok = idx.numel()
    if dweight is None:
        dweight = torch.zeros(rows, dim, dtype=torch.float32, device=weight.device)
    if dweight.dtype != torch.float32 or dweight.shape != (rows, dim):
        raise ValueError("dweight must be float32 [rows, dim]")
    if dout.shape != (*idx.shape, dim):
        raise ValueError("dout must have shape [*idx.shape, dim]")
    _check(weight, idx, gamma, mean, rstd, dout, dweight)
    if dgamma is None:
        dgamma = torch.empty(dim, dtype=torch.float32, device=weight.device)
    if dbeta is None:
        dbeta = torch.empty(dim, dtype=torch.float32, device=weight.device)
    if dgamma.shape != (dim,) or dbeta.shape != (dim,) or dgamma.dtype != torch.float32 \
            or dbeta.dtype != torch.float32:
        raise ValueError("dgamma and dbeta must be float32 [dim]")
    ws = workspace
    if ws is None:
        ws = torch.empty(max(backward_workspace_bytes(ntok, dim), 16), dtype=torch.uint8,
                         device=weight.device)
    _check(dgamma, dbeta, ws)
    _lib.check("qopt_stable_embedding_backward",
               LIB.qopt_stable_embedding_backward(
                   _ptr(weight), _dtype_code(weight, "weight"), rows, dim, _ptr(idx), ntok,
                   _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dout), _dtype_code(dout, "dout"),
                   _ptr(dweight), _ptr(dgamma), _ptr(dbeta), _ptr(ws), ws.numel(),
                   _lib.stream_handle(weight.device)))
    return dweight, dgamma, dbeta


class StableEmbeddingFunction(torch.autograd.Function):
    """out = LayerNorm(weight[idx]) with gradients for weight, gamma and beta."""

    @staticmethod
    def forward(ctx, idx, weight, gamma, beta, eps, out_dtype, check_indices):
        idx = idx.contiguous()
        bad = torch.zeros(1, dtype=torch.int32, device=weight.device) if check_indices else None
        out, mean, rstd = qopt_stable_embedding_forward(weight, idx, gamma, beta, eps, out_dtype,
                                                        bad_count=bad)
        if check_indices and int(bad.item()):
            raise IndexError(f"{int(bad.item())} embedding indices outside [0, {weight.shape[0]})")
        ctx.save_for_backward(idx, weight, gamma, mean, rstd)
        return out

    @staticmethod
    def backward(ctx, dout):
        idx, weight, gamma, mean, rstd = ctx.saved_tensors
        dout = dout.contiguous()
        if dout.dtype not in _DT:
            dout = dout.float()
        dweight, dgamma, dbeta = qopt_stable_embedding_backward(weight, idx, gamma, mean, rstd,
                                                                dout)
        if weight.dtype != torch.float32:
            dweight = dweight.to(weight.dtype)
        return None, dweight, dgamma, dbeta, None, None, None


class StableEmbedding(torch.nn.Module):
    """Embedding table with Xavier-uniform initialisation followed by LayerNorm
    (gamma = 1, beta = 0 at start), on one GPU.

    ``dtype`` is the table's storage (float32 or bfloat16); ``out_dtype`` the
    output's (default: the table's).  The normalisation is computed in float32.
    """

    def __init__(self, num_embeddings, embedding_dim, eps=1e-5, *, device=None,
                 dtype=torch.float32, out_dtype=None, seed=0, check_indices=True):
        super().__init__()
        device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.num_embeddings = int(num_embeddings)
        self.embedding_dim = int(embedding_dim)
        self.eps = float(eps)
        self.out_dtype = dtype if out_dtype is None else out_dtype
        self.seed = int(seed)
        self.check_indices = bool(check_indices)
        self.weight = torch.nn.Parameter(
            torch.empty(self.num_embeddings, self.embedding_dim, dtype=dtype, device=device))
        self.norm_weight = torch.nn.Parameter(
            torch.ones(self.embedding_dim, dtype=torch.float32, device=device))
        self.norm_bias = torch.nn.Parameter(
            torch.zeros(self.embedding_dim, dtype=torch.float32, device=device))
        self.reset_parameters()

    def reset_parameters(self):
        with torch.no_grad():
            qopt_embedding_xavier_init(self.weight, self.seed)
            self.norm_weight.fill_(1.0)
            self.norm_bias.zero_()

    def forward(self, idx):
        return StableEmbeddingFunction.apply(idx, self.weight, self.norm_weight, self.norm_bias,
                                             self.eps, self.out_dtype, self.check_indices)

    def extra_repr(self):
        return (f"{self.num_embeddings}, {self.embedding_dim}, eps={self.eps}, "
                f"dtype={self.weight.dtype}, out_dtype={self.out_dtype}")
