"""Runs the oracle's 8-bit Adam step over a batch of sampled blocks for the full-size
GPU parity tests, in a child process (numpy only; the test process holds the GPU).

    python tests/oracle_blocks_worker.py IN.npz OUT.npz

IN holds p0 (the blocks' parameters before the first step, one full 2048-element
block after another), g1 .. gK (their gradients at each step) and a JSON string of
hyper-parameters, dtypes and the step count.  Blocks are independent and each is a
full block, so the concatenation steps exactly as the blocks do inside their
tensors.  OUT holds the final parameters, codes and block maxima.
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def main(inp, out):
    d = np.load(inp, allow_pickle=False)
    cfg = json.loads(str(d["cfg"]))
    p = d["p0"]
    n = p.size
    assert n % 2048 == 0
    nb = n // 2048
    st = [np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.zeros(nb, np.float32),
          np.zeros(nb, np.float32)]
    for step in range(1, cfg["steps"] + 1):
        with np.errstate(over="ignore"):
            res = oracle.adam8bit_step(p, d[f"g{step}"], *st, step=step, lr=cfg["lr"],
                                       beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
                                       param_dtype=cfg["pdt"], grad_dtype=cfg["gdt"])
        p, st = res[0], list(res[1:])
    np.savez(out, p=p, cm=st[0], cv=st[1], am=st[2], av=st[3])


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
