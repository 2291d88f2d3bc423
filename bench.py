"""Throughput of the fused block-wise 8-bit Adam step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b]

A step is one qopt_adam8bit_step over the whole parameter set (dequantize the 8-bit
moments, update m, v and p, requantize m and v block-wise), inputs resident in HBM.
Default workload: the Llama-shaped 7B parameter set (291 tensors, fp32 master
weights, bf16 gradients with 0.01 % outliers x1000, uint8 moments + fp32 per-block
absmax), state warmed by 5 steps before the warm-up.  Prints one JSON line.

roofline.achieved = algorithmic bytes of the timed launches / their time, measured
with HIP events recorded on the stream the kernels run on (torch's current stream).
Algorithmic bytes per tensor: n * (read p, g, m code, v code + write p, m code,
v code) + ceil(n / 2048) * 16 (read and write both block maxima).
cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_adam8bit_llama7b.json")
KERNEL_SRC = os.path.join(ROOT, "block_wise_bit_adam8bit_amd", "csrc", "qopt_kernels.hip")
METRIC = "8-bit Adam params/s per step and % of HBM roofline (bytes/param) at 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(sizes, pbytes, gbytes):
    total = 0
    for n in sizes:
        nb = -(-n // 2048)
        total += n * (2 * pbytes + gbytes + 4) + nb * 16
    return total


def embedding_bytes(distinct, ntok, dim):
    """Minimal HBM bytes of one Stable Embedding forward and backward (fp32 table, bf16
    outputs and upstream gradients): each distinct row once, token-major arrays once
    (ids 8 B, mean and rstd 4 B each per token); the backward also reads and writes each
    distinct row's fp32 gradient once.  The backward's workspace (sort keys, per-chunk
    partial sums, dgamma / dbeta slots) is the implementation's own overhead and is not
    counted.  Returns (forward, backward)."""
    fwd = distinct * dim * 4 + ntok * dim * 2 + ntok * 16 + 2 * dim * 4
    bwd = distinct * dim * 4 + ntok * dim * 2 + ntok * 16 + distinct * dim * 8 + 3 * dim * 4
    return fwd, bwd


def kernel_code_hash(text=None):
    """sha256 of the step kernel's source with comments removed and whitespace
    collapsed: it changes with the code, not with its comments."""
    if text is None:
        text = open(KERNEL_SRC).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def load_traffic(workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they were
    taken on this workload and on the current kernel code; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_code_sha256") != kernel_code_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def make_workload(name, torch, workloads, layout="flat"):
    """Device tensors of the workload: (tensors, sizes, pdtype, gdtype, label).

    layout "flat": parameters, gradients and each kind of optimizer state in one
    buffer each, every tensor a view (flattened parameters, as sharded data-parallel
    training keeps them).  layout "params": one allocation per parameter and per
    gradient, as a model holds them, with the state as Adam8bit allocates it."""
    if name == "llama7b":
        shapes, pdt, gdt, seed = workloads.llama7b_shapes(), torch.float32, torch.bfloat16, 3
        label = ("llama7b: 291 tensors, 6,738,415,616 params, fp32 params, bf16 grads "
                 "N(0,1e-3) with 0.01% x1000 outliers, uint8 m/v + fp32 absmax per 2048")
    elif name == "llama7b_shard8":
        # one rank's share when 8 ranks split the blocks of the Llama-7B set
        full = workloads.llama7b_shapes()
        pieces = workloads.shard_pieces([n for _, n in full], 8, 0)
        shapes = [(f"{full[i][0]}[{e0}:{e0 + c}]", c) for i, e0, c in pieces]
        pdt, gdt, seed = torch.float32, torch.bfloat16, 3
        label = (f"llama7b_shard8: rank 0 of 8 over the blocks of the Llama-7B set, "
                 f"{len(shapes)} tensor pieces, {sum(c for _, c in shapes):,} params, fp32 "
                 "params, bf16 grads N(0,1e-3) with 0.01% x1000 outliers")
    elif name == "gpt1p3b":
        shapes, pdt, gdt, seed = workloads.gpt1p3b_shapes(), torch.float32, torch.bfloat16, 2
        label = "gpt1p3b: 243 tensors, 1,311,086,592 params, fp32 params, bf16 grads"
    elif name == "flat20b":
        shapes, pdt, gdt, seed = [("flat", workloads.FLAT20B_N)], torch.bfloat16, torch.bfloat16, 4
        label = "flat20b: one flat bf16 buffer of 2e10 params updated in place, bf16 grads"
    else:
        raise SystemExit(f"unknown workload {name}")
    sizes = [n for _, n in shapes]
    total = sum(sizes)
    dev = torch.device("cuda", 0)
    if layout == "params":
        from block_wise_bit_adam8bit_amd.optim import _flat_state
        tensors = []
        for i, n in enumerate(sizes):
            p = torch.empty(n, dtype=pdt, device=dev)
            g = torch.empty(n, dtype=gdt, device=dev)
            workloads.fill_normal_(p, 0.02, seed * 100000 + i)
            workloads.fill_normal_(g, 1e-3, seed * 100000 + 50000 + i)
            if name in ("llama7b", "llama7b_shard8"):
                workloads.scale_random_entries_(g, 1e-4, 1000.0, seed * 100000 + 90000 + i)
            tensors.append((p, g))
        states = _flat_state(dev, sizes)
        tensors = [(p, g, *st) for (p, g), st in zip(tensors, states)]
        return tensors, sizes, pdt, gdt, label + "; one allocation per parameter and gradient"
    P = torch.empty(total, dtype=pdt, device=dev)
    G = torch.empty(total, dtype=gdt, device=dev)
    CM = torch.zeros(total, dtype=torch.uint8, device=dev)
    CV = torch.zeros(total, dtype=torch.uint8, device=dev)
    workloads.fill_normal_(P, 0.02, seed)
    if name == "flat20b":
        workloads.fill_normal_(G, 5e-4, seed * 1000 + 1)
        rows, dim = workloads.FLAT20B_EMBED_ROWS, workloads.FLAT20B_EMBED_DIM
        mask = workloads.sparse_rows_mask(rows, workloads.FLAT20B_ACTIVE_ROWS, seed, dev)
        G[:rows * dim].view(rows, dim)[~mask] = 0
    else:
        workloads.fill_normal_(G, 1e-3, seed * 1000 + 1)
        if name in ("llama7b", "llama7b_shard8"):
            workloads.scale_random_entries_(G, 1e-4, 1000.0, seed * 1000 + 1)
    tensors, off = [], 0
    for n in sizes:
        nb = -(-n // 2048)
        tensors.append((P[off:off + n], G[off:off + n], CM[off:off + n], CV[off:off + n],
                        torch.zeros(nb, dtype=torch.float32, device=dev),
                        torch.zeros(nb, dtype=torch.float32, device=dev)))
        off += n
    return tensors, sizes, pdt, gdt, label


def cpu_baseline(target_seconds=12.0):
    """The oracle, as it stands, on a sample of the llama7b workload: 2048 blocks
    (4,194,304 params) of fp32 params and bf16 gradients, stepped repeatedly."""
    import numpy as np
    import oracle
    import workloads

    n = 2048 * 2048
    p = workloads.host_normal(n, 0.02, 31)
    g = oracle.f32_to_bf16_rne(workloads.host_normal(n, 1e-3, 32))
    st = [np.zeros(n, np.uint8), np.zeros(n, np.uint8), np.zeros(2048, np.float32),
          np.zeros(2048, np.float32)]
    steps, t0 = 0, time.perf_counter()
    while True:
        out = oracle.adam8bit_step(p, g, *st, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
                                   step=steps + 1, grad_dtype="bf16")
        p, st = out[0], list(out[1:])
        steps += 1
        el = time.perf_counter() - t0
        if el >= target_seconds or steps >= 50:
            break
    return {"value": n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} oracle steps over 4,194,304 params (2048 blocks) of the "
                      f"llama7b workload's dtypes (fp32 params, bf16 grads), {el:.1f} s; "
                      f"numpy element-wise ops run on one core of {os.cpu_count()}"}


def calibrate_copy(torch, reps):
    """Plain device copies of a known size: what PMC byte counters read for them
    scales the counters of the step kernel."""
    n = 1 << 30
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch copy_", "bytes_read_per_copy": 4 * n,
                      "bytes_written_per_copy": 4 * n, "copies": reps}), flush=True)


def hbm_reference(torch, reps):
    """Bandwidth of plain torch device operations on 8 GiB fp32 buffers: the
    achievable-bandwidth reference the step is compared with."""
    n = 1 << 31
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ops = {"copy_ (read + write)": (lambda: b.copy_(a), 8 * n),
           "fill_ (write)": (lambda: b.fill_(2.0), 4 * n),
           "sum (read)": (lambda: a.sum(), 4 * n)}
    out = {}
    for name, (fn, nbytes) in ops.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 3), "GB/s": round(nbytes / ms / 1e6, 1),
                     "frac": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    print(json.dumps({"hbm_reference": out, "buffer_bytes": 4 * n}), flush=True)


def placements(torch, workloads, q, args):
    """The step on several copies of the workload held at once.  Each copy is its
    own set of allocations and so its own placement of physical memory; each copy is
    timed in turn, twice, to separate placement from run-to-run noise."""
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    copies = []
    for i in range(args.placements):
        tensors, sizes, pdt, gdt, label = make_workload(args.workload, torch, workloads)
        copies.append((tensors, q.make_tensor_array(tensors)))
        log(f"copy {i} allocated")
    pbytes = 4 if pdt == torch.float32 else 2
    gbytes = 4 if gdt == torch.float32 else 2
    step_bytes = algorithmic_bytes(sizes, pbytes, gbytes)
    step = 0
    for tensors, prepared in copies:
        for _ in range(args.warmup + 1):
            step += 1
            q.qopt_adam8bit_step(tensors, step=step, _prepared=prepared, **hp)
    torch.cuda.synchronize()
    rounds = []
    for _ in range(2):
        row = []
        for tensors, prepared in copies:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                step += 1
                q.qopt_adam8bit_step(tensors, step=step, _prepared=prepared, **hp)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            row.append(round(step_bytes / ms / 1e6, 1))
        rounds.append(row)
    print(json.dumps({"placements": {"workload": label, "copies": args.placements,
                                     "steps_per_timing": args.steps,
                                     "GB/s_per_copy": rounds,
                                     "frac_per_copy": [[round(x / HBM_PEAK_GBS, 4) for x in r]
                                                       for r in rounds]}}), flush=True)


def ceiling(torch, workloads, q, args):
    """The step against qopt_adam8bit_traffic_probe on the same buffers, timed in
    turn: the probe moves exactly the step's bytes with its launch plan, grid and
    access pattern but no arithmetic, so the ratio is how close the step comes to the
    ceiling of its own access pattern on this placement of physical memory."""
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    tensors, sizes, pdt, gdt, label = make_workload(args.workload, torch, workloads, args.layout)
    prepared = q.make_tensor_array(tensors)
    step_bytes = algorithmic_bytes(sizes, 4 if pdt == torch.float32 else 2,
                                   4 if gdt == torch.float32 else 2)
    step = 0

    def run_step():
        nonlocal step
        step += 1
        q.qopt_adam8bit_step(tensors, step=step, _prepared=prepared, **hp)

    def run_probe():
        q.qopt_adam8bit_traffic_probe(tensors, _prepared=prepared)

    for _ in range(5 + args.warmup):
        run_step()
    run_probe()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return step_bytes / (e0.elapsed_time(e1) / args.steps) / 1e6

    rounds = [(timed(run_step), timed(run_probe)) for _ in range(3)]
    print(json.dumps({"ceiling": {
        "workload": label, "layout": args.layout, "steps_per_timing": args.steps,
        "step_GB/s": [round(a, 1) for a, _ in rounds],
        "probe_GB/s": [round(b, 1) for _, b in rounds],
        "step_over_probe": [round(a / b, 4) for a, b in rounds],
        "step_frac_of_8TB/s": [round(a / HBM_PEAK_GBS, 4) for a, _ in rounds]}}), flush=True)


def ceiling_study(torch, workloads, q, args):
    """Bytes-only access patterns for the step's traffic (qopt_pattern_probe), timed
    against the step and its own traffic probe on the same Llama-7B buffers, in a
    shuffled order over several rounds (medians reported).  Every pattern moves the
    step's bytes of one launch's worth of blocks per call over the whole flat set; what
    it writes is what it read."""
    import random
    import statistics
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    tensors, sizes, pdt, gdt, label = make_workload("llama7b", torch, workloads)
    prepared = q.make_tensor_array(tensors)
    step_bytes = algorithmic_bytes(sizes, 4, 2)
    total = sum(sizes)
    flat = [t.as_strided((total,), (1,)) for t in tensors[0][:4]]
    step = 0

    def run_step():
        nonlocal step
        step += 1
        q.qopt_adam8bit_step(tensors, step=step, _prepared=prepared, **hp)

    cands = [("step", run_step),
             ("step traffic probe", lambda: q.qopt_adam8bit_traffic_probe(tensors, _prepared=prepared))]
    for i, name in enumerate(q.qopt_pattern_probe_names()):
        cands.append((f"pattern {i}: {name}", lambda i=i: q.qopt_pattern_probe(i, *flat)))
    for _ in range(5 + args.warmup):
        run_step()
    for _, fn in cands:
        fn()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return step_bytes / (e0.elapsed_time(e1) / args.steps) / 1e6

    res = {name: [] for name, _ in cands}
    rng = random.Random(0)
    for rnd in range(5):
        order = list(range(len(cands)))
        rng.shuffle(order)
        for j in order:
            res[cands[j][0]].append(timed(cands[j][1]))
        log(f"round {rnd} done")
    rows = [{"what": name, "GB/s median": round(statistics.median(v), 1),
             "GB/s min": round(min(v), 1), "GB/s max": round(max(v), 1),
             "frac of 8 TB/s": round(statistics.median(v) / HBM_PEAK_GBS, 4)} for name, v in res.items()]
    best = max(rows[2:], key=lambda r: r["GB/s median"])
    print(json.dumps({"ceiling_study": {
        "workload": label + " (flat buffers, first allocation of the process)",
        "bytes_per_call": step_bytes, "calls_per_timing": args.steps, "rounds": 5,
        "rows": rows, "best_pattern": best["what"], "best_frac": best["frac of 8 TB/s"],
        "step_frac": rows[0]["frac of 8 TB/s"]}}), flush=True)


def bench_codec(torch, workloads, q, args):
    """Block-wise quantize and dequantize of 2^28 values 0.01 * Student-t(3) through
    the signed codebook, and of the same values' magnitudes through the unsigned one
    (one pass of each leg per step; |x| is formed before the timed region)."""
    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    workloads.student_t3_(x, seed=1)
    xa = x.abs()
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(n // 2048, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    legs = {
        "quantize": lambda: q.qopt_quantize_blockwise(x, q.SIGNED, codes=codes, absmax=absmax),
        "dequantize": lambda: q.qopt_dequantize_blockwise(codes, absmax, q.SIGNED, out=y),
        "quantize_unsigned": lambda: q.qopt_quantize_blockwise(xa, q.UNSIGNED, codes=codes,
                                                               absmax=absmax),
        "dequantize_unsigned": lambda: q.qopt_dequantize_blockwise(codes, absmax, q.UNSIGNED,
                                                                   out=y),
    }
    for _ in range(args.warmup + 1):
        for fn in legs.values():
            fn()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # each quantize is timed before the dequantize that reads its codes
    ms = {name: timed(fn) for name, fn in legs.items()}
    total = sum(ms.values())
    byts = n * 5 + (n // 2048) * 4
    out = {"metric": "block-wise dynamic-tree quantize + dequantize values/s at 1 GPU",
           "value": 2 * n / (total * 1e-3), "unit": "values/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(total, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "codec256m: 2^28 fp32 values 0.01*Student-t(3) through the "
                                  "signed codebook, and their magnitudes through the unsigned "
                                  "codebook, 131,072 blocks of 2048 each"},
           "kernels": {name: {"ms": round(t, 4), "GB/s": round(byts / t / 1e6, 1),
                              "frac": round(byts / t / 1e6 / HBM_PEAK_GBS, 4)}
                       for name, t in ms.items()}}
    print(json.dumps(out), flush=True)


def bench_convert(torch, workloads, q, args):
    """Checkpoint moment codec on the Llama-7B set: fp32 Adam moments (m, v) of all
    291 tensors -> block-wise 8-bit state, and back, with preallocated outputs."""
    sizes = [n for _, n in workloads.llama7b_shapes()]
    total = sum(sizes)
    M = torch.empty(total, dtype=torch.float32, device="cuda")
    V = torch.empty(total, dtype=torch.float32, device="cuda")
    workloads.fill_normal_(M, 1e-4, 71)
    workloads.fill_normal_(V, 1e-4, 72)
    V.square_()
    CM = torch.empty(total, dtype=torch.uint8, device="cuda")
    CV = torch.empty_like(CM)
    nbs = [-(-n // 2048) for n in sizes]
    AM = torch.empty(sum(nbs), dtype=torch.float32, device="cuda")
    AV = torch.empty_like(AM)
    views, off, boff = [], 0, 0
    for n, nb in zip(sizes, nbs):
        views.append((slice(off, off + n), slice(boff, boff + nb)))
        off += n
        boff += nb

    m_set = [(M[s], CM[s], AM[bs]) for s, bs in views]
    v_set = [(V[s], CV[s], AV[bs]) for s, bs in views]

    def compress():
        q.qopt_quantize_blockwise_multi(m_set, q.SIGNED)
        q.qopt_quantize_blockwise_multi(v_set, q.UNSIGNED)

    def decompress():
        q.qopt_dequantize_blockwise_multi(m_set, q.SIGNED)
        q.qopt_dequantize_blockwise_multi(v_set, q.UNSIGNED)

    def timed(fn):
        for _ in range(args.warmup + 1):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    tc = timed(compress)
    td = timed(decompress)
    nb_total = sum(nbs)
    byts = 2 * (total * 5 + nb_total * 4)   # each direction, both moments
    out = {"metric": "fp32 Adam moments <-> block-wise 8-bit state conversion, params/s at 1 GPU",
           "value": total / ((tc + td) * 1e-3), "unit": "params/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tc + td, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": "convert7b: m ~ N(0,1e-4), v = N(0,1e-4)^2 for the 291 tensors "
                                  "of the Llama-7B set (6,738,415,616 params), multi-tensor "
                                  "codec calls"},
           "kernels": {"compress": {"ms": round(tc, 3), "GB/s": round(byts / tc / 1e6, 1),
                                    "frac": round(byts / tc / 1e6 / HBM_PEAK_GBS, 4)},
                       "decompress": {"ms": round(td, 3), "GB/s": round(byts / td / 1e6, 1),
                                      "frac": round(byts / td / 1e6 / HBM_PEAK_GBS, 4)}}}
    print(json.dumps(out), flush=True)


def bench_embed(torch, workloads, q, args):
    """Stable Embedding layer at the Llama-7B embedding's shape: Xavier-initialised
    32,000 x 4096 fp32 table, 65,536 Zipf-distributed token ids, LayerNorm forward
    to bf16, and backward from a bf16 upstream gradient; preallocated buffers."""
    cfg = workloads.EMBED7B
    rows, dim, ntok = cfg["rows"], cfg["dim"], cfg["ntokens"]
    w = torch.empty(rows, dim, dtype=torch.float32, device="cuda")
    q.qopt_embedding_xavier_init(w, 11)
    ids_host = workloads.zipf_token_ids(ntok, rows, seed=12)
    ids = torch.from_numpy(ids_host).cuda()
    gamma = torch.ones(dim, device="cuda")
    beta = torch.zeros(dim, device="cuda")
    out = torch.empty(ntok, dim, dtype=torch.bfloat16, device="cuda")
    mean = torch.empty(ntok, device="cuda")
    rstd = torch.empty(ntok, device="cuda")
    dy = torch.empty(ntok, dim, dtype=torch.bfloat16, device="cuda")
    workloads.fill_normal_(dy.view(-1), 1.0, 13)
    dweight = torch.zeros(rows, dim, device="cuda")
    dgamma = torch.empty(dim, device="cuda")
    dbeta = torch.empty(dim, device="cuda")
    from block_wise_bit_adam8bit_amd.embedding import backward_workspace_bytes
    ws = torch.empty(backward_workspace_bytes(ntok, dim), dtype=torch.uint8, device="cuda")

    def fwd():
        q.qopt_stable_embedding_forward(w, ids, gamma, beta, 1e-5, torch.bfloat16,
                                        out=out, mean=mean, rstd=rstd)

    def bwd():
        q.qopt_stable_embedding_backward(w, ids, gamma, mean, rstd, dy, dweight,
                                         dgamma=dgamma, dbeta=dbeta, workspace=ws)

    def timed(fn):
        for _ in range(args.warmup + 1):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    tf = timed(fwd)
    tb = timed(bwd)
    uniq = int(len(set(ids_host.tolist())))
    fwd_bytes, bwd_bytes = embedding_bytes(uniq, ntok, dim)
    # bytes the kernels request (every token's row read, every token's gradient row
    # added), served partly by the caches when ids repeat
    fwd_req = ntok * dim * (4 + 2) + ntok * 16
    bwd_req = ntok * dim * (4 + 2 + 8) + ntok * 16

    def k(ms, b, r):
        return {"ms": round(ms, 4), "GB/s": round(b / ms / 1e6, 1),
                "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4),
                "requested_GB/s": round(r / ms / 1e6, 1)}

    out_line = {"metric": "stable embedding forward + backward tokens/s at 1 GPU",
                "value": ntok / ((tf + tb) * 1e-3), "unit": "tokens/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tf + tb, 4),
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "f32", "data": "synthetic",
                "config": {"workload": f"embed7b: Xavier-initialised {rows} x {dim} fp32 table, "
                                       f"{ntok} Zipf(1) token ids ({uniq} distinct), LayerNorm "
                                       "to bf16, bf16 upstream gradient N(0,1)",
                           "distinct_rows": uniq, "workspace_bytes": ws.numel()},
                "kernels": {"forward": k(tf, fwd_bytes, fwd_req),
                            "backward": k(tb, bwd_bytes, bwd_req)}}
    print(json.dumps(out_line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "llama7b_shard8", "gpt1p3b", "flat20b", "codec256m",
                             "convert7b", "embed7b"])
    ap.add_argument("--layout", default="flat", choices=["flat", "params"],
                    help="flat buffers with views (default), or one allocation per parameter "
                         "and gradient (llama7b, llama7b_shard8, gpt1p3b)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="only time torch's copy_, fill_ and sum over 8 GiB buffers")
    ap.add_argument("--placements", type=int, default=0, metavar="N",
                    help="only time the step on N copies of the workload held at once "
                         "(llama7b or gpt1p3b), each copy in turn")
    ap.add_argument("--ceiling", action="store_true",
                    help="only time the step against the traffic probe (same bytes and access "
                         "pattern, no arithmetic) on the same buffers")
    ap.add_argument("--ceiling-study", action="store_true",
                    help="only time bytes-only access patterns of the step's traffic against "
                         "the step on the Llama-7B buffers")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run torch copies of 4 GiB (for scaling PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the step needs "
              "no communication and is measured at one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import block_wise_bit_adam8bit_amd as q

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        return calibrate_copy(torch, args.steps)
    if args.hbm_reference:
        return hbm_reference(torch, args.steps)
    if args.placements > 0:
        if args.workload not in ("llama7b", "gpt1p3b"):
            raise SystemExit("--placements takes the llama7b or gpt1p3b workload")
        return placements(torch, workloads, q, args)
    if args.ceiling_study:
        return ceiling_study(torch, workloads, q, args)
    if args.ceiling:
        if args.workload not in ("llama7b", "llama7b_shard8", "gpt1p3b", "flat20b"):
            raise SystemExit("--ceiling takes a step workload")
        return ceiling(torch, workloads, q, args)
    if args.workload == "codec256m":
        return bench_codec(torch, workloads, q, args)
    if args.workload == "convert7b":
        return bench_convert(torch, workloads, q, args)
    if args.workload == "embed7b":
        return bench_embed(torch, workloads, q, args)
    log(f"building workload {args.workload}")
    if args.layout != "flat" and args.workload == "flat20b":
        raise SystemExit("--layout params takes a workload made of several parameters")
    tensors, sizes, pdt, gdt, label = make_workload(args.workload, torch, workloads, args.layout)
    prepared = q.make_tensor_array(tensors)
    launches = q.qopt_adam8bit_launch_count(tensors, _prepared=prepared)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    pbytes = 4 if pdt == torch.float32 else 2
    gbytes = 4 if gdt == torch.float32 else 2
    step_bytes = algorithmic_bytes(sizes, pbytes, gbytes)
    nparams = sum(sizes)

    step = 0

    def one_step():
        nonlocal step
        step += 1
        q.qopt_adam8bit_step(tensors, step=step, _prepared=prepared, **hp)

    warm_state = 5 if args.workload != "flat20b" else 0
    log(f"{nparams} params, {launches} launches per step; {warm_state} state-warming steps, "
        f"{args.warmup} warm-up steps, {args.steps} timed steps")
    for _ in range(warm_state + args.warmup):
        one_step()
    torch.cuda.synchronize()

    # one event per step boundary, on the stream the kernels run on
    stream = torch.cuda.current_stream()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events[0].record(stream)
    for i in range(args.steps):
        one_step()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = events[0].elapsed_time(events[-1])
    step_ms = sorted(events[i].elapsed_time(events[i + 1]) for i in range(args.steps))
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed: wall {wall:.4f} s, events {ev_ms:.3f} ms")

    avg_launch_s = ev_ms * 1e-3 / (args.steps * launches)
    launch_bytes = step_bytes / launches
    achieved = launch_bytes / avg_launch_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(args.workload) if args.layout == "flat" else None,
                "kernel": "adam8bit_kernel", "launches_per_step": launches,
                "avg_launch_ms": round(avg_launch_s * 1e3, 4),
                "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
                "step_ms_min": round(step_ms[0], 4),
                "algorithmic_bytes_per_launch": int(launch_bytes)}

    cpu = None
    if not args.no_cpu_baseline:
        del tensors, prepared
        torch.cuda.empty_cache()
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline()

    out = {
        "metric": METRIC,
        "value": nparams / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if pdt == torch.float32 else "bf16",
        "data": "synthetic",
        "config": {"workload": label, "layout": args.layout, "params": nparams,
                   "tensors": len(sizes),
                   "bytes_per_param": round(step_bytes / nparams, 4),
                   "algorithmic_bytes_per_step": step_bytes, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
