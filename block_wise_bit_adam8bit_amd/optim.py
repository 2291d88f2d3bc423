"""Adam8bit: a drop-in replacement for torch.optim.Adam whose two moments are stored
as block-wise dynamic-tree 8-bit codes.  As the summary page describes the switch, a
training script constructs this optimizer where it constructed Adam and changes
nothing else.

State per parameter (allocated with torch on the parameter's device at its first
step): ``m_codes`` / ``v_codes`` uint8 [n], ``m_absmax`` / ``v_absmax`` fp32
[ceil(n / 2048)], and the integer ``step``.  Zero-filled state is the state before
the first step.  Parameters must be contiguous fp32 or bf16 GPU tensors with dense
fp32 or bf16 gradients; the update runs in libqopt's fused kernel.

The state tensors of the parameters that start together (and of a loaded state
dict) are views of four flat buffers per device, one per kind, each parameter's
codes starting on a 256-byte boundary.  A few large allocations map to larger page
fragments than one allocation per tensor: measured on the Llama-7B set, per-tensor
allocations took 7 times the address-translation misses and a flat state was up to
4 % faster, never slower.
"""

from collections import defaultdict

import torch

from .checkpoint import compress_moments_multi, decompress_moments_multi
from .functional import make_tensor_array, nblocks, qopt_adam8bit_step

_STATE_KEYS = ("m_codes", "v_codes", "m_absmax", "v_absmax")
_CODE_ALIGN = 256  # bytes between the starts of consecutive parameters' codes


def _flat_state(device, counts):
    """Zero-filled state for parameters of the given element counts on one device:
    per parameter (m_codes, v_codes, m_absmax, v_absmax), views of four flat buffers."""
    code_off, blk_off, c, b = [], [], 0, 0
    for n in counts:
        code_off.append(c)
        blk_off.append(b)
        c += -(-n // _CODE_ALIGN) * _CODE_ALIGN
        b += nblocks(n)
    cm = torch.zeros(max(c, 1), dtype=torch.uint8, device=device)
    cv = torch.zeros_like(cm)
    am = torch.zeros(max(b, 1), dtype=torch.float32, device=device)
    av = torch.zeros_like(am)
    return [(cm[o:o + n], cv[o:o + n], am[k:k + nblocks(n)], av[k:k + nblocks(n)])
            for n, o, k in zip(counts, code_off, blk_off)]


def _repack(state):
    """Move the code and absmax tensors of ``state`` (param -> dict) into flat buffers
    per device, values unchanged."""
    by_device = defaultdict(list)
    for p in state:
        by_device[p.device].append(p)
    for dev, ps in by_device.items():
        for p, views in zip(ps, _flat_state(dev, [p.numel() for p in ps])):
            for k, t in zip(_STATE_KEYS, views):
                t.copy_(state[p][k])
                state[p][k] = t


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

    def _init_states(self, params):
        """Zero state for parameters without one, in flat buffers per device."""
        by_device = defaultdict(list)
        for p in params:
            by_device[p.device].append(p)
        for dev, ps in by_device.items():
            for p, views in zip(ps, _flat_state(dev, [p.numel() for p in ps])):
                st = self.state[p]
                st["step"] = 0
                st.update(zip(_STATE_KEYS, views))

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for gi, group in enumerate(self.param_groups):
            live = [p for p in group["params"] if p.grad is not None]
            for p in live:
                if p.grad.is_sparse:
                    raise RuntimeError("Adam8bit does not take sparse gradients")
                if not p.is_contiguous() or not p.grad.is_contiguous():
                    raise RuntimeError("Adam8bit needs contiguous parameters and gradients")
            self._init_states([p for p in live if not self.state[p]])
            batches = {}
            for p in live:
                g = p.grad
                st = self.state[p]
                st["step"] += 1
                key = (p.device, p.dtype, g.dtype, st["step"])
                batches.setdefault(key, []).append(
                    (p.view(-1), g.view(-1), st["m_codes"], st["v_codes"], st["m_absmax"],
                     st["v_absmax"]))
            b1, b2 = group["betas"]
            for key, items in batches.items():
                # launch descriptors are cached per batch (group, device, dtypes and
                # parameters) and rebuilt when its gradients move
                ident = (gi, key[:3], tuple(t[0].data_ptr() for t in items))
                sig = ident + (tuple(t[1].data_ptr() for t in items),)
                prepared = self._prepared.get(sig)
                if prepared is None:
                    prepared = make_tensor_array(items)
                    self._prepared = {k: v for k, v in self._prepared.items()
                                      if k[:3] != ident}
                    self._prepared[sig] = prepared
                qopt_adam8bit_step(items, lr=group["lr"], beta1=b1, beta2=b2, eps=group["eps"],
                                   step=key[3], _prepared=prepared)
        return loss

    def load_state_dict(self, state_dict):
        """Load a state dict made by ``state_dict()``.  torch's own loader casts every
        state tensor to its parameter's dtype, which would turn the uint8 codes and
        fp32 block maxima into parameter-typed values; this one keeps their dtypes and
        only moves them to the parameter's device."""
        saved_groups = state_dict["param_groups"]
        by_id = self._params_by_saved_id(saved_groups)
        state = defaultdict(dict)
        for pid, st in state_dict["state"].items():
            p = by_id[pid]
            new = {k: (v.to(device=p.device) if torch.is_tensor(v) else v) for k, v in st.items()}
            n = p.numel()
            for k, dt, size in (("m_codes", torch.uint8, n), ("v_codes", torch.uint8, n),
                                ("m_absmax", torch.float32, nblocks(n)),
                                ("v_absmax", torch.float32, nblocks(n))):
                t = new.get(k)
                if t is None or t.dtype != dt or t.numel() != size:
                    raise ValueError(f"state '{k}' of a parameter with {n} elements must be "
                                     f"{dt} with {size} elements")
            new["step"] = int(new["step"])
            state[p] = new
        _repack(state)
        self.state = state
        for group, saved in zip(self.param_groups, saved_groups):
            for k, v in saved.items():
                if k != "params":
                    group[k] = v
        self._prepared = {}

    def _params_by_saved_id(self, saved_groups):
        if len(saved_groups) != len(self.param_groups):
            raise ValueError("state dict has a different number of parameter groups")
        by_id = {}
        for group, saved in zip(self.param_groups, saved_groups):
            if len(group["params"]) != len(saved["params"]):
                raise ValueError("state dict has a different number of parameters in a group")
            by_id.update(zip(saved["params"], group["params"]))
        return by_id

    @torch.no_grad()
    def load_fp32_adam_state(self, adam_state_dict):
        """Take over the state of a ``torch.optim.Adam`` state dict with the same
        parameter groups: each parameter's fp32 ``exp_avg`` / ``exp_avg_sq`` are
        quantized block-wise into this optimizer's 8-bit state (the moment codec of
        ``checkpoint.py``), its step count is kept, and lr, betas and eps are taken
        from the Adam groups.  Adam with weight decay or amsgrad has no 8-bit
        equivalent here and is refused."""
        saved_groups = adam_state_dict["param_groups"]
        for g in saved_groups:
            if g.get("amsgrad", False) or g.get("weight_decay", 0.0) != 0.0:
                raise ValueError("only plain Adam (no amsgrad, no weight decay) converts")
        by_id = self._params_by_saved_id(saved_groups)
        state = defaultdict(dict)
        by_device = defaultdict(list)
        for pid, st in adam_state_dict["state"].items():
            p = by_id[pid]
            if st["exp_avg"].numel() != p.numel():
                raise ValueError("moment size differs from its parameter")
            by_device[p.device].append((p, st))
        for dev, items in by_device.items():
            codes = compress_moments_multi([(st["exp_avg"].to(dev), st["exp_avg_sq"].to(dev))
                                            for _, st in items])
            for (p, st), new in zip(items, codes):
                step = st["step"]
                new["step"] = int(step.item() if torch.is_tensor(step) else step)
                state[p] = new
        _repack(state)
        self.state = state
        for group, saved in zip(self.param_groups, saved_groups):
            group["lr"] = saved["lr"]
            group["betas"] = tuple(saved["betas"])
            group["eps"] = saved["eps"]
        self._prepared = {}

    @torch.no_grad()
    def fp32_adam_state_dict(self):
        """A ``torch.optim.Adam``-loadable state dict: the moments dequantized to
        fp32 in each parameter's shape, the step as a float tensor, plain-Adam group
        settings.  (``torch.optim.Adam.load_state_dict`` casts the moments to the
        parameter dtype.)"""
        sd = self.state_dict()
        out_state = {}
        params = [p for g in self.param_groups for p in g["params"]]
        by_device = defaultdict(list)
        for pid, st in sd["state"].items():
            by_device[st["m_codes"].device].append((pid, st))
        for items in by_device.values():
            moments = decompress_moments_multi([st for _, st in items],
                                               shapes=[params[pid].shape for pid, _ in items])
            for (pid, st), (m, v) in zip(items, moments):
                out_state[pid] = {"step": torch.tensor(float(st["step"])), "exp_avg": m,
                                  "exp_avg_sq": v}
        adam_defaults = torch.optim.Adam([torch.zeros(1)]).defaults  # this torch's keys
        groups = []
        for g in sd["param_groups"]:
            ng = dict(adam_defaults)
            ng.update(lr=g["lr"], betas=tuple(g["betas"]), eps=g["eps"], weight_decay=0.0,
                      amsgrad=False, params=list(g["params"]))
            groups.append(ng)
        return {"state": out_state, "param_groups": groups}
