"""The allocation-free Stable Embedding backward (qopt_stable_embedding_backward_noalloc)
against the backward with a caller's workspace, through the C ABI.

On the grouped path (vector widths) both entry points run the same kernels in the same
order, and every result there is reproducible run to run, so all three gradients must
agree bit for bit.  Two calls in a row, the second on a smaller input, show that what
the first call leaves in the shared fixed scratch does not leak into the second.  A
shape whose workspace exceeds the fixed scratch is refused before anything is enqueued.
"""

import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def q():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_wise_bit_adam8bit_amd as q
    torch.cuda.set_device(0)
    return q


def _inputs(rows, dim, ntok, seed, wdt, odt):
    g = torch.Generator(device="cuda").manual_seed(seed)
    w = (torch.rand(rows, dim, device="cuda", generator=g) * 0.1 - 0.05).to(wdt)
    ids = torch.from_numpy(workloads.zipf_token_ids(ntok, rows, seed=seed)).cuda()
    gamma = torch.rand(dim, device="cuda", generator=g) + 0.5
    beta = torch.rand(dim, device="cuda", generator=g) * 0.2 - 0.1
    dout = torch.randn(ntok, dim, device="cuda", generator=g).to(odt)
    return w, ids, gamma, beta, dout


def _noalloc(q, w, ids, gamma, mean, rstd, dout, dweight, dgamma, dbeta):
    from block_wise_bit_adam8bit_amd import _lib
    from block_wise_bit_adam8bit_amd.embedding import _dtype_code
    rows, dim = w.shape
    return _lib.LIB.qopt_stable_embedding_backward_noalloc(
        w.data_ptr(), _dtype_code(w, "weight"), rows, dim, ids.data_ptr(), ids.numel(),
        gamma.data_ptr(), mean.data_ptr(), rstd.data_ptr(), dout.data_ptr(),
        _dtype_code(dout, "dout"), dweight.data_ptr(), dgamma.data_ptr(), dbeta.data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("wdt,odt", [(torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32)])
def test_noalloc_backward_matches_the_workspace_backward(q, wdt, odt):
    from block_wise_bit_adam8bit_amd import _lib
    from block_wise_bit_adam8bit_amd.embedding import backward_workspace_bytes
    # the second call is smaller in every dimension than the first
    for rows, dim, ntok, seed in ((8000, 2048, 24000, 1), (3000, 512, 5000, 2)):
        say(f"no-alloc backward rows {rows} dim {dim} tokens {ntok} {wdt}->{odt}")
        need = backward_workspace_bytes(ntok, dim)
        assert 0 < need <= _lib.QOPT_EMB_STATIC_SCRATCH_BYTES
        w, ids, gamma, beta, dout = _inputs(rows, dim, ntok, seed, wdt, odt)
        out, mean, rstd = q.qopt_stable_embedding_forward(w, ids, gamma, beta, 1e-5, odt)
        base = torch.randn(rows, dim, device="cuda")
        dw_ref, dg_ref, db_ref = q.qopt_stable_embedding_backward(w, ids, gamma, mean, rstd, dout,
                                                                  dweight=base.clone())
        dw = base.clone()
        dg = torch.full((dim,), float("nan"), device="cuda")
        db = torch.full((dim,), float("nan"), device="cuda")
        rc = _noalloc(q, w, ids, gamma, mean, rstd, dout, dw, dg, db)
        assert rc == _lib.QOPT_OK, _lib.status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32))
        assert torch.equal(dg.view(torch.int32), dg_ref.view(torch.int32))
        assert torch.equal(db.view(torch.int32), db_ref.view(torch.int32))


def test_noalloc_backward_refuses_shapes_beyond_its_scratch(q):
    from block_wise_bit_adam8bit_amd import _lib
    from block_wise_bit_adam8bit_amd.embedding import backward_workspace_bytes
    rows, dim, ntok = 1000, 4096, 40000
    assert backward_workspace_bytes(ntok, dim) > _lib.QOPT_EMB_STATIC_SCRATCH_BYTES
    w, ids, gamma, beta, dout = _inputs(rows, dim, ntok, 3, torch.float32, torch.bfloat16)
    out, mean, rstd = q.qopt_stable_embedding_forward(w, ids, gamma, beta, 1e-5, torch.bfloat16)
    dw = torch.zeros(rows, dim, device="cuda")
    dg = torch.full((dim,), 7.0, device="cuda")
    db = torch.full((dim,), 7.0, device="cuda")
    torch.cuda.synchronize()
    rc = _noalloc(q, w, ids, gamma, mean, rstd, dout, dw, dg, db)
    assert rc == _lib.QOPT_ENOSPACE
    assert "scratch" in _lib.status_string(rc)
    torch.cuda.synchronize()
    # nothing was enqueued
    assert not dw.any() and bool((dg == 7.0).all()) and bool((db == 7.0).all())
