"""Benchmark of the tiled attention hot path on one MI355X.

One step = one forward (fa_forward) plus one backward (fa_backward) over one
batch of synthetic inputs already resident in HBM.  The default workload is
the largest point of the metric's sequence-length range: long-context causal
self-attention, B=2, H=8, N=16384, d=64, bf16.

    python bench.py [--steps K] [--warmup W] [--config NAME [--n N --d D]] [--no-sweep]

Prints one JSON line.  ``value`` is algorithmic forward+backward TFLOP/s
(14 * d flops per kept query-key pair) of the whole job.  ``sweep`` repeats
the forward and forward+backward timing at every point of the metric (the
GPT-2-shaped N=1024 workload and the long-context points N = 2K..16K,
d = 64 and 128).  The inference workloads (``--config kv_decode`` /
``kv_chunk``: new queries against a key/value cache, fa_forward_kv;
``varlen_prefill``: packed sequences of several lengths, fa_forward_varlen)
have no backward: there a step is one inference forward and ``value`` its
algorithmic TFLOP/s (4 * d per pair).

Kernel times: each kernel is launched through its own entry point (the
forward, the backward's dQ pass, the backward's dK/dV pass) K times back to
back between two HIP events recorded on the launch stream, so no event sits
between two launches; ``kernels_sum_us`` reports their sum beside the step
time.  ``roofline`` describes the kernel that takes most of the step;
``cpu_baseline`` times the fp64 oracle on the host on a bounded sample of the
same workload.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_io_aware_52_amd import _binding  # noqa: E402
from exact_io_aware_52_amd import (accounting, build_lib, fa_backward, fa_backward_ex,  # noqa: E402
                                   fa_forward_key_groups_for, fa_backward_key_groups_for,
                                   fa_backward_blocksparse_split,
                                   fa_backward_blocksparse_split_workspace_bytes,
                                   fa_backward_dkdv, fa_backward_dq,
                                   fa_backward_workspace_bytes, fa_forward,
                                   fa_forward_blocksparse_split,
                                   fa_forward_blocksparse_split_workspace_bytes, fa_forward_ex,
                                   fa_forward_kv, fa_forward_kv_workspace_bytes,
                                   fa_forward_varlen, fa_forward_block_rows_for, inputs)

PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}   # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0
TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
# Algorithmic flops per kept pair, in units of d, that each kernel performs:
# forward S and PV; the dK/dV pass does the recomputed S, dP, dV and dK; the
# dQ pass contributes the dQ product only (its S and dP repeat the dK/dV pass).
# The split block-sparse backward is one call (both passes and their
# reductions), timed as one unit: 10 d.
KERNEL_FLOPS_PER_PAIR_D = {"fwd": 4, "bwd_dkdv": 8, "bwd_dq": 2, "bwd": 10}
KERNEL_NAMES = {"fwd": "fa_fwd_kernel",
                "bwd": "fa_bwd_split_prep_kernel + fa_bwd_dq_kernel + fa_bwd_dkdv_kernel "
                       "+ fa_bwd_split_reduce_kernel (split backward)",
                "fwd_combine": "fa_fwd_combine_kernel",
                "bwd_dq": "fa_bwd_dq_kernel", "bwd_dkdv": "fa_bwd_dkdv_kernel"}
METRIC = "attention TFLOP/s fwd & fwd+bwd (bf16, d=64, N=1K\u201316K) and % of MFMA peak"


def code_hashes():
    """Hashes of the built kernels' machine code (written by the build)."""
    try:
        with open(build_lib.CODE_MANIFEST) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return {}


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed counter summary, or None when
    there is none or the kernel's machine code differs from the code the
    counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    # the hash of the instance the counters were taken on, else of the template
    inst = fields.get("instance")
    built = code_hashes().get("instance:" + inst if inst else kernel)
    if built is None or fields.get("code_sha256") != built:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def event_time_ms(fn, n):
    """Average milliseconds of fn() over n back-to-back calls, between two
    HIP events on the current stream (the stream the library launches on)."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def make_workload(args):
    if args.config == "long_causal":
        return inputs.workload("long_causal", args.n, args.d)
    if args.config == "block_sparse_long":
        return inputs.workload("block_sparse_long", args.n)
    return inputs.workload(args.config)


def cpu_baseline(prob, budget_s):
    """Time the fp64 oracle (forward + backward, one head at a time) on the
    host for about ``budget_s`` seconds of work; report TFLOP/s."""
    import oracle   # test infrastructure; used only for this reported baseline
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:   # pragma: no cover
        threads = os.cpu_count()
    heads = [(b, h) for b in range(prob.B) for h in range(prob.H)]
    done = 0   # heads processed; passes over the workload repeat until the budget is spent
    pairs = 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        kl = None if prob.key_lens is None else int(prob.key_lens[b])
        q, k, v, do = (x[b, h].astype(np.float64) for x in (prob.q, prob.k, prob.v, prob.do))
        kw = dict(causal=prob.causal, key_len=kl, block_mask=prob.block_mask,
                  block_size=prob.block_size, row_chunk=2048)
        oracle.head_forward(q, k, v, float(prob.scale), **kw)
        oracle.head_backward(q, k, v, do, float(prob.scale), **kw)
        pairs += accounting.kept_pairs_head(prob.N, prob.causal, kl, prob.block_mask,
                                            prob.block_size)
        done += 1
    dt = time.perf_counter() - t0
    flops = 14 * prob.d * pairs
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} heads ({done / len(heads):.2f} passes over the {len(heads)} heads of "
                      f"the same workload), fp64 forward+backward, {dt:.1f} s"}


def standard_attention_mask(prob, dev):
    """Boolean mask, True where a key is hidden (causal and key padding), or
    None; shaped to broadcast over [B, H, N, N]."""
    mask = None
    if prob.causal:
        mask = torch.ones(prob.N, prob.N, dtype=torch.bool, device=dev).triu_(1)
    if prob.key_lens is not None:
        kl = torch.from_numpy(prob.key_lens).to(dev).long()
        pad = (torch.arange(prob.N, device=dev)[None, :] >= kl[:, None])[:, None, None, :]
        mask = pad if mask is None else mask | pad
    return mask


def standard_forward(q, k, v, scale, mask):
    """Standard attention (the Theta(N d + N^2) side of the IO argument): the
    GEMM writes S = (scale Q) K^T to HBM in the input dtype, a masking pass
    (masked workloads only) rewrites it, softmax reads S and writes P, and the
    second GEMM reads P: 8 bytes per score element at 16 bits, plus 4 for the
    mask.  Library GEMMs and elementwise kernels; every transposed operand
    (here K^T, N x d) is made contiguous first."""
    s = torch.matmul(q * scale, k.transpose(-1, -2).contiguous())
    if mask is not None:
        s.masked_fill_(mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    return torch.matmul(p, v), p


def standard_backward(q, k, v, do, p, scale):
    """Its backward from the stored P: dV = P^T dO, dP = dO V^T, dS from the
    fused softmax backward (P o (dP - rowsum(dP o P)), the kernel autograd
    uses), dQ = scale dS K, dK = scale dS^T Q.  The products with a
    transposed N x N operand are formed transposed, (dO^T P)^T and
    (Q^T dS)^T, so that only N x d operands are transposed (made contiguous);
    dP and dS go through HBM like S and P."""
    tr = lambda x: x.transpose(-1, -2).contiguous()   # noqa: E731  (N x d operands only)
    dv = tr(torch.matmul(tr(do), p))
    dp = torch.matmul(do, tr(v))
    ds = torch.ops.aten._softmax_backward_data(dp, p, -1, p.dtype)
    dq = torch.matmul(ds, k).mul_(scale)
    dk = tr(torch.matmul(tr(q), ds)).mul_(scale)
    return dq, dk, dv


def bench_standard(args, dev):
    """Standard (materialising) attention on the same workload, timed beside
    the tiled kernels; --phase selects what one step is, so that counter runs
    can attribute HBM bytes per step."""
    prob = make_workload(args)
    if prob.block_mask is not None:
        sys.exit("--standard: block-sparse workloads have no standard counterpart here")
    dt = TORCH_DT[prob.dtype]
    q, k, v, do = (torch.from_numpy(x).to(dt).to(dev) for x in (prob.q, prob.k, prob.v, prob.do))
    mask = standard_attention_mask(prob, dev)
    scale = float(prob.scale)
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).to(dev)

    def std_step():
        _, p = standard_forward(q, k, v, scale, mask)
        if args.phase == "fwdbwd":
            standard_backward(q, k, v, do, p, scale)

    o = torch.empty_like(q)
    lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa_backward_workspace_bytes(prob.B, prob.H, prob.N, prob.d),
                     dtype=torch.uint8, device=dev)

    def flash_step():
        fa_forward(q, k, v, scale=scale, causal=prob.causal, key_lens=kl, o=o, lse=lse)
        if args.phase == "fwdbwd":
            fa_backward(q, k, v, o, do, lse, scale=scale, causal=prob.causal, key_lens=kl,
                        dq=dq, dk=dk, dv=dv, workspace=ws)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base_mem = torch.cuda.memory_allocated(dev)
    for _ in range(args.warmup):
        std_step()
    ms_std = timed(std_step, args.steps)
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_mem
    ms_flash = None
    if not args.standard_only:
        for _ in range(args.warmup):
            flash_step()
        ms_flash = timed(flash_step, args.steps)
    pairs = accounting.kept_pairs(prob)
    flops = (4 if args.phase == "fwd" else 14) * prob.d * pairs
    print(json.dumps({
        "metric": f"standard (materialising) attention beside the tiled kernels, {args.phase}",
        "workload": prob.name, "phase": args.phase, "dtype": prob.dtype,
        "steps": args.steps, "warmup": args.warmup,
        "standard_ms": round(ms_std, 4),
        "standard_tflops": round(flops / (ms_std * 1e-3) / 1e12, 2),
        "standard_extra_device_bytes": int(peak_extra),
        "tiled_ms": None if ms_flash is None else round(ms_flash, 4),
        "speedup": None if ms_flash is None else round(ms_std / ms_flash, 2),
        "standard_model_bytes_fwd": accounting.standard_attention_bytes(prob),
    }), flush=True)


def kv_splits(prob):
    """Key-range splits the library plans for this inference problem (read
    back from its workspace size: splits x rows x (d + 1) fp32 values)."""
    need = fa_forward_kv_workspace_bytes(prob.B, prob.H, prob.Nq, prob.Nk, prob.d,
                                         TORCH_DT[prob.dtype])
    return max(1, need // (prob.B * prob.H * prob.Nq * (prob.d + 1) * 4))


def cpu_baseline_kv(prob, budget_s):
    """The fp64 oracle's inference forward, one head at a time, for about
    ``budget_s`` seconds; TFLOP/s at 4 * d flops per kept pair."""
    import oracle   # test infrastructure; used only for this reported baseline
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:   # pragma: no cover
        threads = os.cpu_count()
    heads = [(b, h) for b in range(prob.B) for h in range(prob.H)]
    done, pairs = 0, 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        b, h = heads[done % len(heads)]
        kl = None if prob.key_lens is None else int(prob.key_lens[b])
        oracle.head_forward_kv(*(x[b, h].astype(np.float64) for x in (prob.q, prob.k, prob.v)),
                               float(prob.scale), causal=prob.causal, key_len=kl)
        L = accounting.kv_fill(prob, b)
        i = np.arange(prob.Nq)
        pairs += int((np.clip(i + L - prob.Nq + 1, 0, L) if prob.causal
                      else np.full(prob.Nq, L)).sum())
        done += 1
    dt = time.perf_counter() - t0
    return {"value": 4 * prob.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} heads ({done / len(heads):.2f} passes over the {len(heads)} heads of "
                      f"the same workload), fp64 inference forward, {dt:.1f} s"}


def bench_kv(args, dev):
    """One step = one fa_forward_kv call (new queries against a key/value
    cache); no backward.  The roofline names the bound with the longer time
    at peak for the forward kernel's work: HBM bytes or matrix flops."""
    prob = inputs.kv_workload(args.config)
    dt = TORCH_DT[prob.dtype]
    q, k, v = (torch.from_numpy(x).to(dt).to(dev) for x in (prob.q, prob.k, prob.v))
    kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(prob.B, prob.H, prob.Nq, dtype=torch.float32, device=dev)
    need = fa_forward_kv_workspace_bytes(prob.B, prob.H, prob.Nq, prob.Nk, prob.d, dt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    scale = float(prob.scale)

    def step():
        fa_forward_kv(q, k, v, scale=scale, causal=prob.causal, key_lens=kl, o=o, lse=lse,
                      workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # The call is the forward kernel plus, when the key range is split, the
    # merge kernel; both are timed together between two events.
    call_us = 1e3 * event_time_ms(step, args.steps)
    splits = kv_splits(prob)
    unit = KERNEL_NAMES["fwd"] + (" + " + KERNEL_NAMES["fwd_combine"] if splits > 1 else "")
    kernels = {"fwd": {"name": unit, "avg_us": call_us}}

    pairs = accounting.kv_kept_pairs(prob)
    flops = 4 * prob.d * pairs
    nbytes = accounting.kv_forward_bytes(prob, splits)
    t_fwd = kernels["fwd"]["avg_us"] * 1e-6
    peak = PEAK_TFLOPS[prob.dtype]
    if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12):
        achieved = nbytes / t_fwd / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / t_fwd / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
    roof["traffic"] = read_traffic(KERNEL_NAMES["fwd"], prob.name) if splits == 1 else None
    roof["kernel"] = unit
    roof["kernel_avg_us"] = round(kernels["fwd"]["avg_us"], 2)
    roof["algorithmic_bytes"] = nbytes
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.dtype,
        "data": "synthetic",
        "config": {"workload": prob.name, "pass": "inference forward (no backward)",
                   "B": prob.B, "H": prob.H, "Nq": prob.Nq, "Nk": prob.Nk, "d": prob.d,
                   "causal": prob.causal, "cache_fill": "key_lens" if prob.key_lens is not None
                   else "full", "key_splits": splits, "parallelism": "none"},
        "hbm_GBps_step": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
        "kernels_us": {v["name"]: round(v["avg_us"], 2) for v in kernels.values()},
        "roofline": roof,
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline_kv(prob, args.cpu_budget)
    print(json.dumps(result), flush=True)


def bench_varlen(args, dev):
    """One step = one fa_forward_varlen call over a packed batch of causal
    sequences; roofline against the matrix peak (4 * d flops per kept pair)."""
    prob = inputs.varlen_workload(args.config)
    dt = TORCH_DT[prob.dtype]
    q, k, v = (torch.from_numpy(x).to(dt).to(dev) for x in (prob.q, prob.k, prob.v))
    cq, ck = (torch.from_numpy(c).to(dev) for c in (prob.cu_q, prob.cu_k))
    o = torch.empty_like(q)
    lse = torch.empty(prob.H, q.shape[1], dtype=torch.float32, device=dev)
    mq = int(prob.lens_q.max())
    scale = float(prob.scale)

    def step():
        fa_forward_varlen(q, k, v, cq, ck, mq, scale=scale, causal=prob.causal, o=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    avg_us = 1e3 * event_time_ms(step, args.steps)   # one kernel per call
    pairs = accounting.varlen_kept_pairs(prob)
    flops = 4 * prob.d * pairs
    peak = PEAK_TFLOPS[prob.dtype]
    achieved = flops / (avg_us * 1e-6) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": read_traffic(KERNEL_NAMES["fwd"], prob.name),
            "kernel": KERNEL_NAMES["fwd"], "kernel_avg_us": round(avg_us, 2)}
    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.dtype,
        "data": "synthetic",
        "config": {"workload": prob.name, "pass": "packed variable-length forward (no backward)",
                   "H": prob.H, "sequences": prob.B, "total_tokens": int(prob.cu_q[-1]),
                   "max_seqlen": mq, "d": prob.d, "causal": prob.causal, "parallelism": "none"},
        "kernels_us": {KERNEL_NAMES["fwd"]: round(avg_us, 2)},
        "roofline": roof,
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline_varlen(prob, args.cpu_budget)
    print(json.dumps(result), flush=True)


def cpu_baseline_varlen(prob, budget_s):
    """The fp64 oracle on (sequence, head) pairs of the same packed batch
    for about ``budget_s`` seconds; TFLOP/s at 4 * d flops per kept pair."""
    import oracle   # test infrastructure; used only for this reported baseline
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:   # pragma: no cover
        threads = os.cpu_count()
    items = [(b, h) for b in range(prob.B) for h in range(prob.H)]
    done, pairs = 0, 0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        b, h = items[done % len(items)]
        q0, q1, k0, k1 = (int(x) for x in (prob.cu_q[b], prob.cu_q[b + 1], prob.cu_k[b],
                                          prob.cu_k[b + 1]))
        oracle.head_forward_kv(prob.q[h, q0:q1].astype(np.float64),
                               prob.k[h, k0:k1].astype(np.float64),
                               prob.v[h, k0:k1].astype(np.float64), float(prob.scale),
                               causal=prob.causal)
        nq, L = q1 - q0, k1 - k0
        i = np.arange(nq)
        pairs += int((np.clip(i + L - nq + 1, 0, L) if prob.causal else np.full(nq, L)).sum())
        done += 1
    dt = time.perf_counter() - t0
    return {"value": 4 * prob.d * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (sequence, head) pairs of the {len(items)} in the same packed batch, "
                      f"fp64 forward, {dt:.1f} s"}


class Runner:
    """Device buffers and launch closures for one self-attention workload."""

    def __init__(self, prob, dev, fwd_block_rows=0, fwd_block_keys=0, bwd_rows=0, key_groups=0):
        self.prob = prob
        dt = TORCH_DT[prob.dtype]
        self.q, self.k, self.v, self.do = (torch.from_numpy(x).to(dt).to(dev)
                                           for x in (prob.q, prob.k, prob.v, prob.do))
        self.kl = None if prob.key_lens is None else torch.from_numpy(prob.key_lens).to(dev)
        self.bm = None if prob.block_mask is None else torch.from_numpy(prob.block_mask).to(dev)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = (torch.empty_like(self.q) for _ in range(3))
        self.ws = torch.empty(fa_backward_workspace_bytes(prob.B, prob.H, prob.N, prob.d),
                              dtype=torch.uint8, device=dev)
        self.scale = float(prob.scale)
        self.rows = fwd_block_rows
        self.fwd_rows = fwd_block_rows or fa_forward_block_rows_for(
            prob.B, prob.H, prob.N, prob.d, dt, prob.block_mask is not None)
        # Keys per K/V tile: 64 by default (16-bit); 32 and 128 run as
        # fa_fwd_keys_kernel with 128-row tiles.
        self.keys = fwd_block_keys
        # Key groups per forward tile (0: the library's choice).
        self.key_groups = key_groups
        # Backward tile heights (dQ query rows, dK/dV keys per work-group) and
        # the key groups the library then chooses.
        self.dq_rows = self.dkdv_rows = bwd_rows
        self.bwd_kgroups = 1 if bwd_rows not in (0, 128) else fa_backward_key_groups_for(
            prob.B, prob.H, prob.N, prob.d, dt, prob.block_mask is not None)
        other_keys = fwd_block_keys not in (0, 64)
        if other_keys:
            self.fwd_rows = 128
        # The long structured masks give one query tile per head the whole key
        # range: its forward is split four ways over work-groups (measured best
        # of 4K, 8K and 16K keys per split at N = 32K and 64K).
        self.key_chunk = 0
        self.fwd_kgroups = key_groups or (fa_forward_key_groups_for(
            prob.B, prob.H, prob.N, prob.d, dt, prob.block_mask is not None)
            if not (fwd_block_rows or other_keys) else 1)
        self.fwd_kernel = ("fa_fwd_keys_kernel" if other_keys else
                           "fa_fwd_kgroups_kernel" if self.fwd_kgroups == 2 else KERNEL_NAMES["fwd"])
        # Their backward is split by kept mask blocks, 64 per work-group (measured
        # at 32K: 911, 979 and 1217 us for 32, 64 and 128 against 1346 unsplit; at
        # 64K all within 1% of unsplit, the passes bound by HBM reads of sparse
        # tiles; 64 keeps the float32 partial workspace at 3 GB for 64K).
        self.chunk_blocks = 0
        if prob.name.startswith("block_sparse_long"):
            self.key_chunk = -(-prob.N // (4 * 64)) * 64
            self.split_ws = torch.empty(max(fa_forward_blocksparse_split_workspace_bytes(
                prob.B, prob.H, prob.N, prob.d, self.key_chunk), 1), dtype=torch.uint8,
                device=dev)
            self.chunk_blocks = 64
            self.bsplit_ws = torch.empty(fa_backward_blocksparse_split_workspace_bytes(
                prob.B, prob.H, prob.N, prob.d, self.chunk_blocks), dtype=torch.uint8,
                device=dev)
        self.kw = dict(scale=self.scale, causal=prob.causal, key_lens=self.kl,
                       block_mask=self.bm, block_size=prob.block_size)
        # At d = 128 the dK/dV pass (16-bit, 128-key tiles, unsplit) splits
        # every query tile between two wave groups (key groups left to the
        # library here, so never 1).
        self.dkdv_split_queries = (prob.dtype != "fp32" and prob.d == 128 and
                                   bwd_rows in (0, 128) and not self.chunk_blocks)

    def fwd(self):
        if self.key_chunk:
            fa_forward_blocksparse_split(self.q, self.k, self.v, self.bm, self.prob.block_size,
                                         key_chunk=self.key_chunk, scale=self.scale,
                                         causal=self.prob.causal, key_lens=self.kl, o=self.o,
                                         lse=self.lse, workspace=self.split_ws)
        else:
            fa_forward_ex(self.q, self.k, self.v, block_rows=self.rows, block_keys=self.keys,
                          key_groups=self.key_groups, o=self.o, lse=self.lse, **self.kw)

    def bwd_dq(self):
        fa_backward_dq(self.q, self.k, self.v, self.o, self.do, self.lse, dq=self.dq,
                       workspace=self.ws, rows=self.dq_rows, **self.kw)

    def bwd_dkdv(self):
        fa_backward_dkdv(self.q, self.k, self.v, self.do, self.ws, dk=self.dk, dv=self.dv,
                         rows=self.dkdv_rows, **self.kw)

    def bwd(self):
        if self.chunk_blocks:
            fa_backward_blocksparse_split(self.q, self.k, self.v, self.o, self.do, self.lse,
                                          self.bm, self.prob.block_size, self.chunk_blocks,
                                          scale=self.scale, causal=self.prob.causal,
                                          key_lens=self.kl, dq=self.dq, dk=self.dk, dv=self.dv,
                                          workspace=self.bsplit_ws)
        else:
            fa_backward_ex(self.q, self.k, self.v, self.o, self.do, self.lse, dq=self.dq,
                           dk=self.dk, dv=self.dv, workspace=self.ws, dq_rows=self.dq_rows,
                           dkdv_rows=self.dkdv_rows, **self.kw)

    def step(self):
        self.fwd()
        self.bwd()


def wall_ms(fn, n):
    """Average milliseconds of fn() over n calls, host clock, synchronised
    on both sides."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n


def measure(run, steps, warmup, kernels=True):
    """Step time, forward time and (optionally) per-kernel times of a Runner."""
    for _ in range(warmup):
        run.step()
    out = {"ms_step": wall_ms(run.step, steps), "ms_fwd": wall_ms(run.fwd, steps)}
    if kernels and run.chunk_blocks:
        out["kernels_us"] = {
            "fwd": 1e3 * event_time_ms(run.fwd, steps),
            "bwd": 1e3 * event_time_ms(run.bwd, steps),
        }
    elif kernels:
        out["kernels_us"] = {
            "fwd": 1e3 * event_time_ms(run.fwd, steps),
            "bwd_dq": 1e3 * event_time_ms(run.bwd_dq, steps),
            "bwd_dkdv": 1e3 * event_time_ms(run.bwd_dkdv, steps),
        }
    return out


def sweep(dev, steps, warmup):
    """Forward and forward+backward TFLOP/s at every point of the metric."""
    points = [("gpt2_small", None, None)] + [("long_causal", n, d) for n, d in inputs.LONG_POINTS]
    rows = []
    for name, n, d in points:
        prob = inputs.workload(name, n, d)
        run = Runner(prob, dev)
        m = measure(run, steps, warmup, kernels=False)
        pairs = accounting.kept_pairs(prob)
        peak = PEAK_TFLOPS[prob.dtype]
        fwd_tf = 4 * prob.d * pairs / (m["ms_fwd"] * 1e-3) / 1e12
        fb_tf = 14 * prob.d * pairs / (m["ms_step"] * 1e-3) / 1e12
        rows.append({"workload": prob.name, "N": prob.N, "d": prob.d, "causal": prob.causal,
                     "fwd_ms": round(m["ms_fwd"], 4), "fwd_tflops": round(fwd_tf, 1),
                     "fwd_frac": round(fwd_tf / peak, 4),
                     "fwdbwd_ms": round(m["ms_step"], 4), "fwdbwd_tflops": round(fb_tf, 1),
                     "fwdbwd_frac": round(fb_tf / peak, 4), "fwd_block_rows": run.fwd_rows})
        print(f"[sweep] {prob.name}: fwd {fwd_tf:.0f} TFLOP/s, fwd+bwd {fb_tf:.0f} TFLOP/s",
              file=sys.stderr, flush=True)
        del run
        torch.cuda.empty_cache()
    return rows


STAMP_SEGMENTS = {(5, 1): "loop", (5, 11): "loop", (1, 2): "wait_tile", (2, 3): "barrier",
                  (3, 4): "math", (4, 1): "loop", (4, 11): "loop", (4, 20): "loop",
                  (11, 12): "wait_tile", (12, 13): "barrier", (13, 14): "math",
                  (14, 11): "loop", (14, 1): "loop", (14, 20): "loop", (20, 21): "epilogue"}


def step_stamps(args, dev):
    """Forward step timeline (the stamps build of the forward kernel): for
    the heaviest, a middle and the lightest work-groups of the grid, waves 0-3
    record the shader clock at each step's start, after its tile wait, after
    its barrier and after its math.  Prints, per work-group and wave, the
    total and median cycles of each segment and the clock they imply."""
    prob = make_workload(args)
    lib = _binding.open_library(build_lib.STAMPS_LIB)
    lib.fa_stamps_arm.argtypes = [ctypes.c_void_p]
    lib.fa_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    run = Runner(prob, dev, args.fwd_block_rows)
    rows = run.fwd_rows
    nwg = prob.B * prob.H * -(-prob.N // rows)
    wgs = np.array([0, 1, 2, nwg // 3, nwg // 2, nwg - 3, nwg - 2, nwg - 1], dtype=np.int32)
    assert lib.fa_stamps_arm(wgs.ctypes.data) == 0
    dt = TORCH_DT[prob.dtype]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bm = None if run.bm is None else ctypes.c_void_p(run.bm.data_ptr())
    kl = None if run.kl is None else ctypes.c_void_p(run.kl.data_ptr())
    code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[dt]

    def fwd():
        assert lib.fa_forward_ex(ctypes.c_void_p(run.q.data_ptr()), ctypes.c_void_p(run.k.data_ptr()),
                                 ctypes.c_void_p(run.v.data_ptr()), ctypes.c_void_p(run.o.data_ptr()),
                                 ctypes.c_void_p(run.lse.data_ptr()), prob.B, prob.H, prob.N, prob.d,
                                 run.scale, int(prob.causal), kl, bm, prob.block_size, rows, 0,
                                 1, code, st) == 0
    for _ in range(max(args.warmup, 1)):
        fwd()
    torch.cuda.synchronize()
    kernel_us = 1e3 * event_time_ms(fwd, max(args.steps, 1))
    buf = np.zeros((32, 3 * 340), dtype=np.uint64)
    assert lib.fa_stamps_read(buf.ctypes.data, buf.nbytes) == 0
    out = []
    for slot, wg in enumerate(wgs):
        for w in range(4):
            r = buf[slot * 4 + w].reshape(-1, 3).astype(np.int64)
            n = int(np.argmax(r[:, 0] == 0)) if (r[:, 0] == 0).any() else len(r)
            r = r[:n]
            if n < 2:
                continue
            cyc, rt, codes = r[:, 0], r[:, 1], r[:, 2]
            seg = {}
            for i in range(n - 1):
                key = STAMP_SEGMENTS.get((int(codes[i]), int(codes[i + 1])))
                if key is None and codes[i] >= 1000:
                    key = "prologue"
                if key:
                    seg.setdefault(key, []).append(int(cyc[i + 1] - cyc[i]))
            ns = 10 * int(rt[-1] - rt[0])
            out.append({"work_group": int(wg), "wave": w,
                        "query_tile": int(codes[0] - 1000) if codes[0] >= 1000 else None,
                        "steps": int(sum(c in (1, 11) for c in codes)),
                        "recorded_events": n, "wall_ns": ns, "cycles": int(cyc[-1] - cyc[0]),
                        "clock_ghz": round((cyc[-1] - cyc[0]) / ns, 3) if ns else None,
                        "segments": {k: {"total": int(sum(v)), "median": float(np.median(v)),
                                         "count": len(v)} for k, v in seg.items()}})
    print(json.dumps({"workload": prob.name, "fwd_block_rows": rows, "work_groups": nwg,
                      "kernel_us_stamps_build": round(kernel_us, 2), "timeline": out}))


RATE_OPS = [  # (op code, name, matrix products and vector instructions per wave per iteration)
    (0, "mfma_32x32x16_bf16", 4, 0), (1, "v_exp_f32", 0, 16), (2, "v_fma_f32", 0, 16),
    (3, "v_add_f32", 0, 16), (4, "v_cvt_pk_bf16_f32", 0, 16),
    (5, "mfma + 4 v_exp_f32 each, one wave", 4, 16), (6, "mfma waves beside v_exp_f32 waves", 4, 16),
    (7, "ds_read_b128", 0, 16), (8, "ds_read_b64_tr_b16", 0, 16)]
LDS_READ_BYTES = {7: 1024, 8: 512}  # per wave instruction


def simd_key(rec):
    """(XCD, shader engine, shader array, CU, SIMD) of a wave from its
    recorded XCC_ID << 32 | HW_ID word (HW_ID: SIMD bits 5:4, CU 11:8, shader
    array 12, shader engine 15:13)."""
    h = int(rec) & 0xFFFFFFFF
    return (int(rec) >> 32, (h >> 13) & 7, (h >> 12) & 1, (h >> 8) & 15, (h >> 4) & 3)


def unit_rates(args, dev):
    """Instruction issue rates from libfa_rates.so: SIMD cycles per wave
    instruction of each kind the attention steps use, at 1, 2 and 4 waves per
    SIMD, with the shader clock the run saw; then a few seconds of matrix
    products alone, launch after launch, for the rate and clock they sustain.
    A SIMD's rate is its waves' instructions over the span from its first
    wave's start to its last wave's end (waves grouped by their hardware
    ids)."""
    if not os.path.exists(build_lib.RATES_LIB):
        raise RuntimeError(f"{build_lib.RATES_LIB} is missing: build it with "
                           "`python -m exact_io_aware_52_amd.build_lib`")
    lib = ctypes.CDLL(build_lib.RATES_LIB)
    lib.fa_rates_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    st = torch.cuda.current_stream()

    def run(op, groups_per_cu, iters):
        wpg = 8 if op == 6 else 4
        grid = cus * groups_per_cu
        sink = torch.empty(grid * 64 * wpg, dtype=torch.float32, device=dev)
        clocks = torch.zeros(grid * wpg * 5, dtype=torch.int64, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        rc = lib.fa_rates_run(op, grid, iters, ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(clocks.data_ptr()), ctypes.c_void_p(st.cuda_stream))
        assert rc == 0, rc
        e1.record(st)
        e1.synchronize()
        c = clocks.view(-1, 5).cpu().numpy().astype(np.int64)
        cyc = c[:, 1] - c[:, 0]
        wall_ns = 10 * (c[:, 3] - c[:, 2])
        mfma_wave = (np.arange(len(c)) % wpg) < 4 if op == 6 else np.full(len(c), op in (0, 5))
        simds = {}
        for i, rec in enumerate(c[:, 4]):
            simds.setdefault(simd_key(rec), []).append(i)
        return {"grid": grid, "c": c, "cycles": cyc, "simds": simds, "mfma_wave": mfma_wave,
                "kernel_ms": e0.elapsed_time(e1),
                "ghz": float(np.median(cyc / np.maximum(wall_ns, 1)))}

    def cu_lds_rate(r, iters, op):
        """Median over CUs of LDS bytes read per cycle (span from the CU's
        first wave start to its last wave end)."""
        c = r["c"]
        cus_ = {}
        for key, idx in r["simds"].items():
            cus_.setdefault(key[:4], []).extend(idx)
        per = [len(idx) * iters * 16 * LDS_READ_BYTES[op] /
               (c[idx, 1].max() - c[idx, 0].min()) for idx in cus_.values()]
        return round(float(np.median(per)), 1)

    def simd_rate(r, iters, n_per_iter, select=None):
        """Median over SIMDs of span cycles per wave instruction, and the
        median number of (selected) waves per SIMD."""
        c = r["c"]
        per, waves = [], []
        for idx in r["simds"].values():
            idx = [i for i in idx if select is None or select[i]]
            if not idx:
                continue
            span = c[idx, 1].max() - c[idx, 0].min()
            per.append(span / (len(idx) * iters * n_per_iter))
            waves.append(len(idx))
        return round(float(np.median(per)), 3), float(np.median(waves))

    rows = []
    for op, name, n_mfma, n_valu in RATE_OPS:
        for per_cu in ([1, 2, 4] if op not in (5, 6) else [1, 2]):
            wps = per_cu * (2 if op == 6 else 1)  # waves per SIMD if spread evenly
            iters = max(2000, 160000 // wps)
            run(op, per_cu, 64)  # warm-up launch
            r = run(op, per_cu, iters)
            row = {"op": name, "work_groups_per_cu": per_cu, "iters": iters,
                   "kernel_ms": round(r["kernel_ms"], 3), "clock_ghz": round(r["ghz"], 3),
                   "simds": len(r["simds"])}
            if op == 6:
                row["mfma_cycles_per_inst"], row["mfma_waves_per_simd"] = simd_rate(
                    r, iters, 4, r["mfma_wave"])
                row["exp_cycles_per_inst"], row["exp_waves_per_simd"] = simd_rate(
                    r, iters, 16, ~r["mfma_wave"])
            elif op == 5:
                row["cycles_per_iter"], row["waves_per_simd"] = simd_rate(r, iters, 1)
            else:
                row["cycles_per_inst"], row["waves_per_simd"] = simd_rate(r, iters,
                                                                          n_mfma or n_valu)
                if op in LDS_READ_BYTES:
                    row["lds_bytes_per_cu_cycle"] = cu_lds_rate(r, iters, op)
                if op == 0:
                    flops = r["grid"] * 4 * iters * 4 * 32 * 32 * 16 * 2
                    row["tflops"] = round(flops / (r["kernel_ms"] * 1e-3) / 1e12, 1)
            rows.append(row)
            print(json.dumps(row), flush=True)
    # matrix products alone for a few seconds: the rate and clock they sustain
    sustained = []
    t_end = time.time() + args.rates_seconds
    while time.time() < t_end:
        r = run(0, 2, 300000)
        flops = r["grid"] * 4 * 300000 * 4 * 32 * 32 * 16 * 2
        sustained.append({"tflops": round(flops / (r["kernel_ms"] * 1e-3) / 1e12, 1),
                          "clock_ghz": round(r["ghz"], 3), "kernel_ms": round(r["kernel_ms"], 2)})
    print(json.dumps({"unit_rates": rows, "compute_units": cus,
                      "mfma_sustained": {"launches": len(sustained), "first": sustained[0],
                                         "last": sustained[-1],
                                         "median_tflops": round(float(np.median(
                                             [x["tflops"] for x in sustained])), 1),
                                         "median_clock_ghz": round(float(np.median(
                                             [x["clock_ghz"] for x in sustained])), 3)}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_causal",
                    choices=["tiny", "gpt2_small", "bert_large_padded", "long_causal",
                             "block_sparse", "block_sparse_long", "kv_decode", "kv_chunk",
                             "varlen_prefill"])
    ap.add_argument("--n", type=int, default=16384)
    ap.add_argument("--d", type=int, default=64)
    ap.add_argument("--fwd-block-rows", type=int, default=0, choices=[0, 64, 128, 256],
                    help="query rows per forward work-group (tile height); 0 = chosen per problem")
    ap.add_argument("--fwd-block-keys", type=int, default=0, choices=[0, 32, 64, 128],
                    help="keys per forward K/V tile (B_c); 0 = the default (64); 32 and 128 "
                         "take 128-row tiles")
    ap.add_argument("--key-groups", type=int, default=0, choices=[0, 1, 2],
                    help="wave groups splitting each forward tile's key range; 0 = the library's "
                         "choice")
    ap.add_argument("--bwd-rows", type=int, default=0, choices=[0, 64, 128, 256],
                    help="backward tile height: query rows per dQ work-group and keys per dK/dV "
                         "work-group; 0 = 128")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of host work for the oracle baseline (0 disables)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the timing sweep over the metric's other points")
    ap.add_argument("--standard", action="store_true",
                    help="time standard (materialising) attention on the workload beside the "
                         "tiled kernels")
    ap.add_argument("--phase", default="fwdbwd", choices=["fwd", "fwdbwd"],
                    help="with --standard: what one step is")
    ap.add_argument("--standard-only", action="store_true",
                    help="with --standard: run only the standard attention (counter runs)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--unit-rates", action="store_true",
                    help="instruction issue rates and the sustained matrix-core rate "
                         "(libfa_rates.so)")
    ap.add_argument("--rates-seconds", type=float, default=4.0,
                    help="with --unit-rates: seconds of back-to-back matrix-product launches")
    ap.add_argument("--step-stamps", action="store_true",
                    help="forward step timeline of chosen work-groups from the stamps build "
                         "(libfa_stamps.so)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "(b, h) heads are independent, so a multi-GPU run would shard heads with no "
              "communication; this build measures the single-GPU kernel.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": 1 << 30, "copy_calib_bytes_written": 1 << 30}))
        return
    if args.unit_rates:
        unit_rates(args, dev)
        return
    if args.step_stamps:
        step_stamps(args, dev)
        return
    if args.standard:
        bench_standard(args, dev)
        return
    if args.config.startswith("kv_"):
        bench_kv(args, dev)
        return
    if args.config.startswith("varlen_"):
        bench_varlen(args, dev)
        return

    prob = make_workload(args)
    run = Runner(prob, dev, args.fwd_block_rows, args.fwd_block_keys, args.bwd_rows,
                 args.key_groups)
    m = measure(run, args.steps, args.warmup)
    ms_step, ms_fwd, kus = m["ms_step"], m["ms_fwd"], m["kernels_us"]
    pairs = accounting.kept_pairs(prob)
    flops_step = 14 * prob.d * pairs
    value = flops_step / (ms_step * 1e-3) / 1e12
    dom = max(kus, key=kus.get)
    fwd_unit = run.fwd_kernel + (" + " + KERNEL_NAMES["fwd_combine"] if run.key_chunk else "")
    names = dict(KERNEL_NAMES, fwd=fwd_unit)
    work = KERNEL_FLOPS_PER_PAIR_D[dom] * prob.d * pairs
    achieved = work / (kus[dom] * 1e-6) / 1e12
    peak = PEAK_TFLOPS[prob.dtype]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": (read_traffic(dict(KERNEL_NAMES, fwd=run.fwd_kernel)[dom], prob.name)
                        if not (dom == "bwd" or (dom == "fwd" and run.key_chunk)) else None),
            "kernel": names[dom], "kernel_avg_us": round(kus[dom], 2),
            "algorithmic_flops_per_launch": work}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prob.dtype,
        "data": "synthetic",
        "config": {"workload": prob.name, "B": prob.B, "H": prob.H, "N": prob.N, "d": prob.d,
                   "causal": prob.causal,
                   "key_padding": prob.key_lens is not None,
                   "block_sparse": prob.block_mask is not None,
                   "fwd_block_rows": run.fwd_rows, "fwd_block_keys": run.keys or 64,
                   "fwd_key_groups": run.fwd_kgroups, "bwd_key_groups": run.bwd_kgroups,
                   "bwd_dkdv_split_queries": run.dkdv_split_queries,
                   "bwd_rows": run.dq_rows or 128,
                   "fwd_key_chunk": run.key_chunk or None,
                   "bwd_chunk_blocks": run.chunk_blocks or None,
                   "parallelism": "none"},
        "fwd_ms": round(ms_fwd, 4),
        "fwd_tflops": round(4 * prob.d * pairs / (ms_fwd * 1e-3) / 1e12, 2),
        "frac_of_peak_fwd": round(4 * prob.d * pairs / (ms_fwd * 1e-3) / 1e12 / peak, 4),
        "frac_of_peak_fwd_bwd": round(value / peak, 4),
        "kernels_us": {names[k]: round(v, 2) for k, v in kus.items()},
        "kernels_sum_us": round(sum(kus.values()), 2),
        "roofline": roof,
    }
    del run
    torch.cuda.empty_cache()
    if not args.no_sweep and args.config == "long_causal":
        result["sweep"] = sweep(dev, max(5, args.steps // 2), max(2, args.warmup // 2))
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(prob, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
