#!/usr/bin/env python3
"""Benchmark of one emulated N-rank tensor-parallel block step on one MI355X.

A step is the whole path: the replicated RMSNorm, N ranks' attention halves (QKV projection,
rotary embedding + paged KV append, owned-head attention, o_proj partial), the local N-way
reduce + residual + RMSNorm, N ranks' FFN halves (gate/up + activation, down partial) and the
final reduce + residual, for one batch of synthetic inputs already resident in HBM.

Default workload: the Llama-3-8B-shaped block at tensor-parallel degree 2, bf16, decode of one
token against a 4096-token KV cache. Timing: every step is captured as a HIP graph; `copies`
independent sets of shards and KV caches (>= 1 GB in total) rotate so repeats cannot be served
from the 256 MB last-level cache. One JSON line on stdout; progress on stderr.

Roofline: the dominant kernel is the gate/up projection (the largest weight stream of a rank).
Its average duration is measured live with HIP events recorded by the library immediately around
its launch, on the launch stream.

``--blocks K`` (K > 1) times a stack of K distinct blocks of the workload's shape instead, chained
as the layers of a decoder (each block's output is the next block's input, every block with its
own shards and KV caches), captured as one HIP graph; ``value`` is then tokens/s through the whole
stack and the stack's own K blocks are the cold rotation.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def weight_bytes(s):
    from tensor_transformer_block_amd.inputs import weight_shapes
    per = {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0}[s.w_dtype]
    return int(sum(o * i for o, i in weight_shapes(s).values()) * per)


def step_bytes(s):
    """Algorithmic HBM bytes of one block step, all N ranks: every shard's weights once, the KV
    read of every attended key (new one included) for all heads, the N partials written and read
    at the activation dtype per half, and the residual read and written per half."""
    act = 4 if s.act_dtype == "f32" else 2
    kv = sum(s.kv_lens) * s.n_kv_heads * s.head_dim * act * 2
    if s.mode == "prefill":
        kv = s.n_tokens * s.n_kv_heads * s.head_dim * act * 2
    a = 4 * s.tp * s.n_tokens * s.d_model * act + 4 * s.n_tokens * s.d_model * act
    return weight_bytes(s) + kv + a


def step_flops(s):
    """Projection FLOPs 2*T*params plus causal attention 4*hd per attended (query, key) pair."""
    params = sum(o * i for o, i in __import__(
        "tensor_transformer_block_amd.inputs", fromlist=["weight_shapes"]).weight_shapes(s).values())
    pairs = 0
    if s.mode == "prefill":
        L = s.kv_lens[0]
        pairs = sum(p + 1 for p in range(L - s.n_tokens, L))
    else:
        pairs = sum(s.kv_lens)
    return 2.0 * s.n_tokens * params + 4.0 * s.head_dim * s.n_heads * pairs


def gate_up_unit(s, ranks=1):
    """Algorithmic bytes and FLOPs of one gate/up launch covering `ranks` ranks (1: one rank's
    launch; tp_degree under the all-ranks schedule): each rank's weight slice once, the input
    rows read once and each rank's activation output written."""
    act = 4 if s.act_dtype == "f32" else 2
    per = {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0}[s.w_dtype]
    fr = s.ffn_dim // s.tp
    wb = 2 * fr * s.d_model * per
    return int(ranks * wb + s.n_tokens * s.d_model * act + ranks * s.n_tokens * fr * act), \
        ranks * 2.0 * s.n_tokens * 2 * fr * s.d_model


SCHEDULE_NAMES = {0: "staged", 1: "one-call, per rank", 2: "one-call, all ranks per launch"}


def step_schedule(blk, staged):
    """The schedule the library gives this block's step (the bench's --staged runs the separate
    calls whatever the library would choose)."""
    from tensor_transformer_block_amd import binding as B
    return 0 if staged else B.tp_step_schedule(blk.desc, blk.batch)


class HipEvents:
    """Timing events created with the HIP runtime (hipEvent_t handles the library can record)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def elapsed_s(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e-3

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def code_text(src):
    """C++ source without its comments, whitespace runs collapsed: what the compiler sees of it,
    so that a comment edit does not count as a kernel change."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, kept whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def code_digest(paths, root):
    """sha256 over the code text of the given sources (repository-relative paths), in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(code_text(open(os.path.join(root, p), encoding="utf-8").read()).encode())
        h.update(b"\n")
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed counter summary, or None when there is no
    summary for this workload or the kernel's code changed since the counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"traffic_gate_up_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        if code_digest(fields["sources"].split(), root) != fields["code_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(inp, seconds):
    """The oracle's explicit N-rank block, fp64 NumPy, on the host cores, for a bounded sample."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    s = inp.shape
    p = oracle.params_f64(inp)
    x = oracle.to_f64(inp.x, s.act_dtype)
    kc, vc = oracle.caches_f64(inp)
    kr, vr = oracle.rank_caches(s, kc, vc)
    rows = None
    if s.mode == "prefill":
        rows = np.array([s.n_tokens - 1])          # the last row attends to every key
    ntok = s.n_tokens if rows is None else len(rows)
    n, t0, steps = 0, time.perf_counter(), []
    while True:
        ts = time.perf_counter()
        oracle.block_sharded(s, p, x, kr, vr, inp.positions, inp.token_seq, rows)
        steps.append(time.perf_counter() - ts)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or (s.mode == "prefill" and n >= 1):
            break
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] or [1])
    blas = sorted({i.get("internal_api", "?") for i in pools if i.get("user_api") == "blas"})
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    sample = (f"{n} full block steps (all {s.tp} ranks) of the same workload" if rows is None else
              f"{n} step(s) of the same workload with the oracle producing {len(rows)} output "
              f"row(s) (K/V and QKV for all {s.n_tokens} tokens)")
    return {"value": round(ntok / float(np.median(steps)), 4), "unit": "tokens/s",
            "cores": int(threads), "kind": "oracle",
            "sample": sample + f"; {el:.1f} s wall, fp64 NumPy; value from the median step",
            "host": {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas}}


def bench_vendor_gemm(args, s):
    """The vendor GEMM library (torch.matmul / torch.bmm in bf16 -> hipBLASLt) on the workload's
    four projections with every rank in one call: the column-parallel QKV and gate/up as one GEMM
    over the ranks' stacked weight slices (they share their input), the row-parallel o_proj and
    down as a batch of N GEMMs (each rank its own input). Random operands; bf16 outputs (the
    block's own row-parallel launches store fp32 partials, twice the output bytes). One JSON line
    with the mean time of 20 calls after 3 warm-ups, and the rate against the bf16 dense peak."""
    import torch
    T, d, N, hd = s.n_tokens, s.d_model, s.tp, s.head_dim
    qkv = (s.n_heads + 2 * s.n_kv_heads) * hd // N
    shapes = [("qkv", 1, T, N * qkv, d), ("o_proj", N, T, d, s.n_heads * hd // N),
              ("gate_up", 1, T, 2 * s.ffn_dim, d), ("down", N, T, d, s.ffn_dim // N)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    out = []
    for name, batch, M, Nc, K in shapes:
        g = torch.Generator(device="cuda").manual_seed(args.seed)
        a = torch.randn(batch, M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(batch, K, Nc, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
        fn = (lambda: torch.matmul(a[0], b[0])) if batch == 1 else (lambda: torch.bmm(a, b))
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(20):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / 20
        fl = 2.0 * batch * M * Nc * K
        out.append({"projection": name, "batch": batch, "m": M, "n": Nc, "k": K, "us": round(us, 1),
                    "tflops": round(fl / us / 1e6, 1), "frac": round(fl / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 3)})
        log(f"vendor GEMM {name}: {us:.1f} us")
        del a, b
    print(json.dumps({"vendor_gemm": out, "workload": s.name, "library": "torch.matmul / torch.bmm (hipBLASLt)",
                      "dtype": "bf16", "peak_tflops": MFMA_BF16_PEAK_TFLOPS}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama3-8b-decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cold-bytes", type=float, default=1.0e9,
                    help="rotate at least this many bytes of distinct shards + KV caches")
    ap.add_argument("--kernel-iters", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--blocks", type=int, default=1,
                    help="time a chained stack of this many distinct blocks (one graph)")
    ap.add_argument("--head", action="store_true",
                    help="with the stack, time a full token step: embedding lookup, the stack, "
                         "final RMSNorm and LM head (replicated head of the family's vocabulary)")
    ap.add_argument("--vocab", type=int, default=0, help="vocabulary of --head (0: the family's)")
    ap.add_argument("--partial-dtype", choices=("f32", "bf16"), default="f32",
                    help="storage of the rank partials (f32: the default of the library)")
    ap.add_argument("--staged", action="store_true",
                    help="issue the step as separate per-rank and reduce calls instead of the "
                         "one-call step (tp_block_step)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the step: time the vendor GEMM library (torch.matmul / bmm, "
                         "bf16, random operands) on the workload's projections with every rank "
                         "in one call, as a reference rate for the chip")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a dispatch of known "
                         "size for scaling hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the N tensor-parallel ranks are emulated in sequence "
              "on a single MI355X; runs on more than one GPU are not part of this build "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceBlock
    from tensor_transformer_block_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()  # fails loudly if the HIP library is missing
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibrate_copy_mib} MiB done")
        del src, dst
    from tensor_transformer_block_amd.inputs import MOE_WORKLOADS
    if args.workload in MOE_WORKLOADS:
        bench_moe(args, *MOE_WORKLOADS[args.workload])
        return
    s = WORKLOADS[args.workload]
    if args.vendor_gemm:
        bench_vendor_gemm(args, s)
        return
    if args.blocks > 1 or args.head:
        bench_stack(args, s)
        return
    log(f"workload {s.name}: generating inputs (seed {args.seed})")
    inp = make_inputs(s, seed=args.seed)
    sb = step_bytes(s)
    resident = weight_bytes(s) + sum(s.kv_lens) * s.n_kv_heads * s.head_dim * (
        4 if s.act_dtype == "f32" else 2) * 2
    copies = max(1, math.ceil(args.cold_bytes / resident))
    log(f"building device block: {copies} cold cop{'y' if copies == 1 else 'ies'} "
        f"x {resident / 1e6:.1f} MB")
    blk = DeviceBlock(inp, copies=copies, partial_dtype=args.partial_dtype)
    torch.cuda.synchronize()

    if args.staged:
        def step(c, timed=None):
            blk.step(c, ffn_events=timed)
    else:
        def step(c, timed=None):
            blk.step_fused(c, timed=timed)

    for c in range(copies):
        step(c)
    torch.cuda.synchronize()
    graphs = []
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                step(c)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        # One graph holding a step on every copy in turn (a stack of `copies` blocks, as the
        # layers of a model would be), so a replay's fixed cost is paid once per `copies` steps.
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi):
            for c in range(copies):
                step(c)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % copies].replay()
        else:
            step(i % copies)

    def run_steps(k):
        """k consecutive steps, from copy 0: whole multi-step replays, then single steps."""
        if graphs:
            for _ in range(k // copies):
                multi.replay()
            for i in range(k % copies):
                graphs[i].replay()
        else:
            for i in range(k):
                step(i % copies)

    log(f"warmup {args.warmup} steps")
    run_steps(args.warmup)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    run_steps(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    tok_s = s.n_tokens / (ms / 1e3)

    # Per-step distribution: single-step replays with an event between consecutive steps (the
    # events cost a few microseconds each, so this loop is kept apart from the timed region).
    n_dist = max(10, min(200, args.steps))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n_dist):
        run(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_dist)])
    dist = {"steps": n_dist, "p10": round(float(np.percentile(per_step, 10)), 5),
            "median": round(float(np.median(per_step)), 5),
            "p90": round(float(np.percentile(per_step, 90)), 5)}

    # The same step launched eagerly (no graph), and one rank's share (its ATTN and FFN halves,
    # eager) at the real shape.
    n_extra = max(5, min(50, args.steps // 10))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(2):
        step(i % copies)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n_extra):
        step(i % copies)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_extra
    e0.record()
    for i in range(n_extra):
        c = i % copies
        blk.attn_half(0, c)
        blk.ffn_half(0, c)
    e1.record()
    torch.cuda.synchronize()
    rank_ms = e0.elapsed_time(e1) / n_extra

    # Dominant kernel: the gate/up projection. The library launches its kernels through
    # hipExtLaunchKernel with these events, so each pair spans that projection's kernel execution
    # on the launch stream (what a profiler's kernel trace reports). The timed launches sit inside
    # whole block steps, launched eagerly behind a backlog of graph replays, so every one runs in
    # the same context as in the timed steps (after the attention half and the reduce).
    if args.staged:
        n_kst = max(1, (args.kernel_iters + s.tp - 1) // s.tp)
        n_kl = n_kst * s.tp
    else:  # the one-call step times one rank's gate/up per step, the ranks in turn
        n_kst = n_kl = max(1, args.kernel_iters)
    log(f"timing the gate/up projection ({n_kl} launches in {n_kst} steps)")
    hev = HipEvents(2 * n_kl)
    for i in range(min(64, args.steps)):
        run(i)
    for i in range(n_kst):
        if args.staged:
            step(i % copies, timed=[(hev.ev[2 * (i * s.tp + r)], hev.ev[2 * (i * s.tp + r) + 1])
                                    for r in range(s.tp)])
        else:
            step(i % copies, timed=(i % s.tp, hev.ev[2 * i], hev.ev[2 * i + 1]))
    torch.cuda.synchronize()
    kdur = [hev.elapsed_s(2 * i, 2 * i + 1) for i in range(n_kl)]
    hev.close()
    kavg = float(np.mean(kdur))
    sched = step_schedule(blk, args.staged)
    all_ranks = sched == 2
    ub, uf = gate_up_unit(s, s.tp if all_ranks else 1)
    if s.mode == "prefill":
        roof = {"bound": "mfma", "achieved": round(uf / kavg / 1e12, 3),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(ub / kavg / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(s.name)
    if all_ranks and s.w_dtype == "q8_0" and s.n_tokens > 4:
        roof["kernel"] = ("gate/up projection (all ranks: the Q8_0 GEMM, with its split-K "
                          "epilogue when K is split)")
    else:
        roof["kernel"] = ("gate/up projection (all ranks, one launch)" if all_ranks
                          else "gate/up projection (one rank)")
    roof["avg_us"] = round(kavg * 1e6, 2)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    step_gbs = sb / (ms / 1e3) / 1e9
    line = {
        "metric": "shard decode tokens/s + achieved HBM GB/s (% of peak); prefill MFMA % peak",
        "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": s.act_dtype, "data": "synthetic",
        "config": {"workload": s.name, "d_model": s.d_model, "n_heads": s.n_heads,
                   "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim, "ffn_dim": s.ffn_dim,
                   "tp_degree_emulated": s.tp, "weights": s.w_dtype, "mode": s.mode,
                   "tokens": s.n_tokens, "kv_len": max(s.kv_lens), "page_size": s.page_size,
                   "cold_copies": copies, "graph": not args.no_graph,
                   "schedule": SCHEDULE_NAMES[sched],
                   "partial_dtype": args.partial_dtype},
        "step_algorithmic_bytes": sb,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_tflops": round(step_flops(s) / (ms / 1e3) / 1e12, 3),
        "wall_s_timed": round(wall, 4),
        "step_ms_dist": dist,
        "eager_ms_per_step": round(eager_ms, 5),
        "rank_share_ms": round(rank_ms, 5),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_stack(args, s):
    """A chained stack of ``args.blocks`` distinct blocks, one graph per stack step."""
    import numpy as np
    import torch
    from tensor_transformer_block_amd.block import BlockStack
    from tensor_transformer_block_amd.inputs import make_stack_inputs

    K = args.blocks
    log(f"workload {s.name}: generating a stack of {K} blocks (seed {args.seed})")
    inps = make_stack_inputs(s, K, seed=args.seed)
    model = None
    if args.head:
        from tensor_transformer_block_amd.block import ModelStep
        from tensor_transformer_block_amd.inputs import VOCAB, make_head_inputs
        vocab = args.vocab or VOCAB[s.name]
        log(f"head: vocab {vocab}")
        head = make_head_inputs(s, vocab, seed=args.seed)
        model = ModelStep(head, inps)
        st = model.stack
        del head
    else:
        st = BlockStack(inps)
    del inps
    stepper = model if model is not None else st
    fused = not args.staged
    stepper_step = stepper.step
    if fused:
        def stepper_step():
            stepper.step(fused=True)
    resident = weight_bytes(s) + sum(s.kv_lens) * s.n_kv_heads * s.head_dim * (
        4 if s.act_dtype == "f32" else 2) * 2
    if K * resident < args.cold_bytes:
        log(f"note: the stack holds {K * resident / 1e6:.0f} MB, less than --cold-bytes")
    stepper_step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        stepper_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            stepper_step()
        torch.cuda.synchronize()
    run = g.replay if g is not None else stepper_step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"timing {args.steps} stack steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps

    # Gate/up launches timed inside eager stack steps, behind a backlog of replays.
    if fused:  # one rank's gate/up per block and stack step, the ranks in turn
        n_st = max(1, (args.kernel_iters + K - 1) // K)
        hev = HipEvents(2 * n_st * K)
    else:
        n_st = max(1, (args.kernel_iters + K * s.tp - 1) // (K * s.tp))
        hev = HipEvents(2 * n_st * K * s.tp)
    for _ in range(min(16, args.steps)):
        run()
    i = 0
    for j in range(n_st):
        x_in = model.x if model is not None else None
        if fused:
            tm = []
            for _b in st.blocks:
                tm.append((j % s.tp, hev.ev[2 * i], hev.ev[2 * i + 1]))
                i += 1
            st.step(x=x_in, fused=True, timed=tm)
            continue
        evs = []
        for _b in st.blocks:
            evs.append([(hev.ev[2 * (i + r)], hev.ev[2 * (i + r) + 1]) for r in range(s.tp)])
            i += s.tp
        st.step(x=x_in, ffn_events=evs)
    torch.cuda.synchronize()
    kavg = float(np.mean([hev.elapsed_s(2 * j, 2 * j + 1) for j in range(i)]))
    hev.close()
    sched = step_schedule(st.blocks[0], not fused)
    all_ranks = sched == 2
    ub, uf = gate_up_unit(s, s.tp if all_ranks else 1)
    if s.mode == "prefill":
        roof = {"bound": "mfma", "achieved": round(uf / kavg / 1e12, 3),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(ub / kavg / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(s.name)
    roof["kernel"] = ("gate/up projection (all ranks of one block, one launch)" if all_ranks
                      else "gate/up projection (one rank of one block)")
    roof["avg_us"] = round(kavg * 1e6, 2)
    sb = K * step_bytes(s)
    head_info = None
    if model is not None:
        # The LM head alone: stream events around eager launches (one kernel per launch, so the
        # pair spans it plus its dispatch), behind a backlog of replays.
        hb = model.head.layout.payload_bytes + s.n_tokens * s.d_model * (
            4 if s.act_dtype == "f32" else 2) + s.n_tokens * model.head.vocab * 4
        sb += hb + s.n_tokens * s.d_model * (4 if s.act_dtype == "f32" else 2)
        n_h = 50
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_h)]
        for _ in range(min(8, args.steps)):
            run()
        for j in range(n_h):
            evs[2 * j].record()
            model.head.logits(model.xn_f, model.logits)
            evs[2 * j + 1].record()
        torch.cuda.synchronize()
        h_ms = float(np.mean([evs[2 * j].elapsed_time(evs[2 * j + 1]) for j in range(n_h)]))
        head_info = {"vocab": model.head.vocab, "lm_head_bytes": hb,
                     "lm_head_us": round(h_ms * 1e3, 2),
                     "lm_head_gbs": round(hb / (h_ms / 1e3) / 1e9, 1)}
    step_gbs = sb / (ms / 1e3) / 1e9
    line = {
        "metric": "shard decode tokens/s + achieved HBM GB/s (% of peak); prefill MFMA % peak",
        "value": round(s.n_tokens / (ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": s.act_dtype,
        "data": "synthetic",
        "config": {"workload": f"{s.name} x{K} blocks" + (" + head" if model else ""),
                   "blocks": K, "head": head_info, "d_model": s.d_model,
                   "n_heads": s.n_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "ffn_dim": s.ffn_dim, "tp_degree_emulated": s.tp, "weights": s.w_dtype,
                   "mode": s.mode, "tokens": s.n_tokens, "kv_len": max(s.kv_lens),
                   "page_size": s.page_size, "graph": not args.no_graph,
                   "schedule": SCHEDULE_NAMES[sched]},
        "step_algorithmic_bytes": sb,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_tflops": round((K * step_flops(s) + (2.0 * s.n_tokens * s.d_model * model.head.vocab
                                                    if model else 0.0)) / (ms / 1e3) / 1e12, 3),
        "ms_per_block": round(ms / K, 5),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_moe(args, s, moe):
    """A block whose FFN half is the expert-sliced MoE (dense attention half, replicated router,
    every rank's slice of the selected experts). Cold rotation over copies of every weight and
    cache, sized by the bytes one step touches (the selected experts, not the whole table)."""
    import numpy as np
    import torch
    from tensor_transformer_block_amd.block import MoEBlock
    from tensor_transformer_block_amd.inputs import make_inputs, make_moe_inputs

    act_b = 4 if s.act_dtype == "f32" else 2
    per = {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0}[s.w_dtype]
    hd, d = s.head_dim, s.d_model
    attn_w = ((s.n_heads + 2 * s.n_kv_heads) * hd * d + d * s.n_heads * hd) * per
    kv = sum(s.kv_lens) * s.n_kv_heads * hd * act_b * 2
    expert_sel = s.n_tokens * moe.top_k * 3 * moe.expert_ffn * d * per   # all ranks together
    router = moe.n_experts * d * act_b
    acts = 4 * s.tp * s.n_tokens * d * act_b + 4 * s.n_tokens * d * act_b
    sb = int(attn_w + kv + expert_sel + router + acts)
    copies = max(1, math.ceil(args.cold_bytes / sb))
    log(f"workload {s.name} (MoE {moe.n_experts} experts, top {moe.top_k}, width "
        f"{moe.expert_ffn}): {copies} cold copies x {sb / 1e6:.1f} MB touched per step")
    inp = make_inputs(s, seed=args.seed)
    minp = make_moe_inputs(s, moe, seed=args.seed)
    mb = MoEBlock(inp, minp, copies=copies)
    del minp
    mstep = mb.step if args.staged else mb.step_fused
    for c in range(copies):
        mstep(c)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(copies):
            mstep(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi):
        for c in range(copies):
            mstep(c)
    torch.cuda.synchronize()

    def run_steps(k):
        for _ in range(max(1, k // copies)):
            multi.replay()
        return max(1, k // copies) * copies

    run_steps(args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record()
    n = run_steps(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / n

    # The dominant kernel: the expert gate/up projection of every rank in one launch (the
    # selected experts' gate and up slices of all ranks), timed with HIP events the library
    # records around that launch inside eager one-call steps, behind a backlog of replays.
    n_st = max(1, args.kernel_iters)
    hev = HipEvents(2 * n_st)
    for _ in range(min(16, args.steps)):
        multi.replay()
    for i in range(n_st):
        mb.step_fused(i % copies, timed=(hev.ev[2 * i], hev.ev[2 * i + 1]))
    torch.cuda.synchronize()
    kavg = float(np.mean([hev.elapsed_s(2 * j, 2 * j + 1) for j in range(n_st)]))
    hev.close()
    # weights of every rank's gate and up slices of the selected experts, each rank's read of the
    # normed input, the activations written
    ub = int(s.n_tokens * moe.top_k * 2 * moe.expert_ffn * d * per + s.tp * s.n_tokens * d * act_b
             + s.n_tokens * moe.top_k * moe.expert_ffn * act_b)
    roof = {"bound": "hbm", "achieved": round(ub / kavg / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = "expert gate/up projection (all ranks, one launch)"
    roof["avg_us"] = round(kavg * 1e6, 2)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        log(f"cpu baseline: oracle MoE block for ~{args.cpu_seconds:.0f} s")
        minp = make_moe_inputs(s, moe, seed=args.seed)
        k, t0 = 0, time.perf_counter()
        while True:
            oracle.run_moe_block(inp, minp)
            k += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        cpu = {"value": round(k * s.n_tokens / el, 4), "unit": "tokens/s", "cores": int(threads),
               "kind": "oracle",
               "sample": f"{k} full MoE block steps (all {s.tp} ranks); {el:.1f} s wall, fp64 NumPy"}

    step_gbs = sb / (ms / 1e3) / 1e9
    line = {
        "metric": "shard decode tokens/s + achieved HBM GB/s (% of peak); prefill MFMA % peak",
        "value": round(s.n_tokens / (ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": n, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": s.act_dtype, "data": "synthetic",
        "config": {"workload": s.name, "d_model": d, "n_heads": s.n_heads,
                   "n_kv_heads": s.n_kv_heads, "head_dim": hd, "n_experts": moe.n_experts,
                   "top_k": moe.top_k, "expert_ffn": moe.expert_ffn, "tp_degree_emulated": s.tp,
                   "weights": s.w_dtype, "mode": s.mode, "tokens": s.n_tokens,
                   "kv_len": max(s.kv_lens), "cold_copies": copies, "graph": True,
                   "schedule": "staged" if args.staged else "one-call"},
        "step_algorithmic_bytes": sb,
        "step_hbm_gbs": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
