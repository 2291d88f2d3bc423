"""Adam8bit: a drop-in replacement for torch.optim.Adam whose two moments are stored
as block-wise dynamic-tree 8-bit codes (the summary page's "two lines of code" swap:
construct this optimizer instead of Adam).

State per parameter (allocated with torch on the parameter's device at its first
step): ``m_codes`` / ``v_codes`` uint8 [n], ``m_absmax`` / ``v_absmax`` fp32
[ceil(n / 2048)], and the integer ``step``.  Zero-filled state is the state before
the first step.  Parameters must be contiguous fp32 or bf16 GPU tensors with dense
fp32 or bf16 gradients; the update runs in libqopt's fused kernel.
"""

import torch

from .functional import make_tensor_array, nblocks, qopt_adam8bit_step

_ABSMAX_KEYS = ("m_absmax", "v_absmax")


class Adam8bit(torch.optim.Optimizer):
    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8):
        if not 0.0 <= lr:
            raise ValueError(f"invalid learning rate {lr}")
        if not 0.0 <= eps:
            raise ValueError(f"invalid epsilon {eps}")
        if not (0.0 <= betas[0] < 1.0 and 0.0 <= betas[1] < 1.0):
            raise ValueError(f"invalid betas {betas}")
        super().__init__(params, dict(lr=lr, betas=tuple(betas), eps=eps))
        self._prepared = {}

    def _init_state(self, p):
        st = self.state[p]
        n = p.numel()
        st["step"] = 0
        st["m_codes"] = torch.zeros(n, dtype=torch.uint8, device=p.device)
        st["v_codes"] = torch.zeros(n, dtype=torch.uint8, device=p.device)
        st["m_absmax"] = torch.zeros(nblocks(n), dtype=torch.float32, device=p.device)
        st["v_absmax"] = torch.zeros(nblocks(n), dtype=torch.float32, device=p.device)
        return st

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for gi, group in enumerate(self.param_groups):
            batches = {}
            for p in group["params"]:
                if p.grad is None:
                    continue
                g = p.grad
                if g.is_sparse:
                    raise RuntimeError("Adam8bit does not take sparse gradients")
                if not p.is_contiguous() or not g.is_contiguous():
                    raise RuntimeError("Adam8bit needs contiguous parameters and gradients")
                st = self.state[p]
                if not st:
                    st = self._init_state(p)
                st["step"] += 1
                key = (p.device, p.dtype, g.dtype, st["step"])
                batches.setdefault(key, []).append(
                    (p.view(-1), g.view(-1), st["m_codes"], st["v_codes"], st["m_absmax"],
                     st["v_absmax"]))
            b1, b2 = group["betas"]
            for key, items in batches.items():
                sig = (gi, key[:3], tuple(t[0].data_ptr() for t in items),
                       tuple(t[1].data_ptr() for t in items))
                prepared = self._prepared.get(sig)
                if prepared is None:
                    prepared = make_tensor_array(items)
                    self._prepared = {k: v for k, v in self._prepared.items() if k[0] != gi}
                    self._prepared[sig] = prepared
                qopt_adam8bit_step(items, lr=group["lr"], beta1=b1, beta2=b2, eps=group["eps"],
                                   step=key[3], _prepared=prepared)
        return loss

    def load_state_dict(self, state_dict):
        # torch casts floating-point state to the parameter's dtype on load; the block
        # maxima must stay fp32, so they travel as int32 bit patterns through it.
        sd = dict(state_dict)
        sd["state"] = {
            k: {kk: (vv.view(torch.int32) if kk in _ABSMAX_KEYS else vv) for kk, vv in v.items()}
            for k, v in state_dict["state"].items()
        }
        super().load_state_dict(sd)
        for st in self.state.values():
            for k in _ABSMAX_KEYS:
                if k in st and st[k].dtype == torch.int32:
                    st[k] = st[k].view(torch.float32)
        self._prepared = {}
