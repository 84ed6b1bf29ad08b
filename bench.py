#!/usr/bin/env python3
"""Benchmark one training step (forward + backward) of the d20 decoder block
(B=32, T=2048, width 1280, 10 heads of 128, MLP 5120, bf16) on one MI355X.

Prints ONE JSON line on stdout (details go to stderr):
  value       tokens per second of the whole step (inputs resident in HBM)
  tflops      algorithmic FLOP/s of the step (causal attention counted once:
              per token 72*C^2 for the linear layers + 6*C*(T+1) for attention;
              with a window W, only the visible query-key pairs)
  roofline    the launch site with the largest share of the step, timed with
              hipEvents around each of its launches over a second pass of the
              same K steps (block_timing_*), against the bf16 dense MFMA peak
  cpu_baseline the float64 CPU oracle on a bounded sample of the workload
              (whole sequences of it), on this host's cores

--workload d20_decode measures the KV-cache decode step instead (64
sequences, one new token each, caches of 2048 keys; the ragged 128..2048
variant is reported beside it): decode tokens/s, and the HBM roofline of the
split-KV attention kernel from the cache bytes it must read.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/sec and TFLOP/s per decoder block (d20, T=2048) on 1 MI355X"
# the metric as it reads for each training workload (the d20 bf16 one is the headline)
WORKLOAD_METRIC = {
    "d20_bf16": METRIC,
    "d6_f32": "training tokens/sec and TFLOP/s per decoder block (d6, T=512, fp32) on 1 MI355X",
    "d12_bf16": "training tokens/sec and TFLOP/s per decoder block (d12, T=2048) on 1 MI355X",
    "d26_fp8": "training tokens/sec and TFLOP/s per decoder block (d26, T=2048, E4M3 linear GEMMs) on 1 MI355X",
    "d20_bf16_swa": "training tokens/sec and TFLOP/s per decoder block (d20, T=2048, window 512) on 1 MI355X",
    "d20_bf16_gqa": "training tokens/sec and TFLOP/s per decoder block (d20, T=2048, 2 key/value heads) on 1 MI355X",
}
DECODE_METRIC = "decode tokens/sec per decoder block (d20, batch 64, KV cache 2048) on 1 MI355X"
DECODE_WORKLOAD_METRIC = {
    "d20_decode": DECODE_METRIC,
    "d20_decode_gqa": "decode tokens/sec per decoder block (d20, batch 64, KV cache 2048, 2 key/value heads) on 1 MI355X",
}
HEAD_METRIC = "training tokens/sec of the lm_head + cross-entropy (d20, 65,536 tokens, vocabulary 65,536) on 1 MI355X"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def window_of(sh) -> int:
    """Keys a query can see at most: the window, or T for causal."""
    w = getattr(sh, "window", 0)
    return sh.T if w <= 0 or w >= sh.T else w


def kv_heads(sh) -> int:
    """Key/value heads (grouped-query attention); H without grouping."""
    return getattr(sh, "n_kv_head", 0) or sh.H


def qkv_cols(sh) -> int:
    """Output columns of the fused projection: H query, G key and G value heads of 128."""
    return sh.C + 256 * kv_heads(sh)


def matmul_params(sh) -> int:
    """Weights of the block's four linear layers."""
    return sh.C * (qkv_cols(sh) + sh.C + 2 * sh.F)


def attn_matmul_flops(sh) -> float:
    """FLOPs of one T x T x D attention matmul over all heads and sequences,
    counting only the visible (query, key) pairs: sum_i min(i+1, W) per
    sequence (T(T+1)/2 for causal)."""
    T, W = sh.T, window_of(sh)
    pairs = W * (W + 1) / 2.0 + (T - W) * float(W)
    return 2.0 * sh.B * sh.C * pairs


def linear_flops(sh) -> float:
    """Forward, input-gradient and weight-gradient GEMMs of the four linear
    layers: 6 x their weights per token (72 C^2 without grouping)."""
    return float(sh.B * sh.T) * 6.0 * matmul_params(sh)


def step_flops(sh) -> float:
    # attention: 2 matmuls forward, 4 backward
    return linear_flops(sh) + 6.0 * attn_matmul_flops(sh)


def step_flops_nanochat(sh) -> float:
    """The convention of nanochat's estimate_flops (6 x matmul params + 12*C*W
    per token for attention, W the window or T), which reproduces the depth
    table on the flicky.cc nanochat page."""
    N, C = sh.B * sh.T, sh.C
    return float(N) * (6.0 * matmul_params(sh) + 12.0 * C * window_of(sh))


def site_flops(sh) -> dict:
    """Algorithmic FLOPs of one launch of each launch site."""
    N, C, F = sh.B * sh.T, sh.C, sh.F
    att = attn_matmul_flops(sh)           # one attention matmul over the visible pairs
    g = {
        "gemm_qkv_fwd": 2.0 * N * C * qkv_cols(sh), "gemm_o_fwd": 2.0 * N * C * C,
        "gemm_fc_fwd": 2.0 * N * C * F, "gemm_proj_fwd": 2.0 * N * F * C,
        "attn_fwd": 2 * att,
        "attn_bwd_dkdv": 3 * att,      # dV = P^T dO, dP = dO V^T, dK = dS^T Q
        "attn_bwd_dq": 1 * att,        # dQ = dS K
    }
    for p in ("qkv", "o", "fc", "proj"):
        g[f"gemm_{p}_dgrad"] = g[f"gemm_{p}_fwd"]
        g[f"gemm_{p}_wgrad"] = g[f"gemm_{p}_fwd"]
    return g


def site_bytes(sh) -> dict:
    """Algorithmic HBM bytes per step of the memory-bound launch sites (all
    launches of the site in one step).  fp8 quantiser: weights read for the
    amax and for the codes (2 + 2 B) and written as codes (1 B), and read
    again for the transposed codes of the backward (2 + 1 B); activations
    whose maximum the producer folds in read once (2 B) and written as
    row-major and transposed codes (1 + 1 B); dY read twice (amax, codes)."""
    N, C, F = sh.B * sh.T, sh.C, sh.F
    out = {"rmsnorm_fwd": 2.0 * (2 * N * C * 2 + N * 4), "rmsnorm_bwd": 2.0 * (4 * N * C * 2)}
    if sh.gemm == "fp8":
        w = matmul_params(sh)
        out["fp8_quantize"] = float(w * (5 + 3) + N * C * (3 * 4 + 6 + 4 + 3 * 4) + N * F * (4 + 4))
    return out


def smi_state() -> dict:
    """Clock and power of the GPU as the box's SMI tool reports them (called
    while steps are running, so the figures are those under load)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:   # the report notes the failure instead of failing
        return {"error": f"{type(e).__name__}: {e}"}
    card = next((v for k, v in data.items() if k.startswith("card")), {})
    keep = {k: v for k, v in card.items() if any(w in k.lower() for w in ("sclk", "mclk", "fclk", "power"))}
    return {"tool": "rocm-smi --showclocks --showpower", **keep}


def under_load(launch, seconds: float = 2.0) -> dict:
    """Queue about `seconds` of work (launch() enqueues one step) and read
    the SMI state while it runs."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    launch()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-4)
    for _ in range(max(1, int(seconds / one))):
        launch()
    state = smi_state()
    torch.cuda.synchronize()
    return state


def mfma_rates() -> dict:
    """Achievable matrix-core rate from a register-only MFMA loop
    (block_mfma_probe): 4 workgroups of four waves per CU, best of three."""
    import torch
    import backward_gpt_block_amd as bl
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg, out = 4 * cus, {}
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda:0")
    for kind, name, flop, iters in ((0, "bf16", 2 * 32 * 32 * 16, 20000), (1, "fp8", 2 * 32 * 32 * 64, 10000)):
        best = None
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            bl.block_mfma_probe(kind, wg, iters, sink)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        tf = wg * 4 * iters * 4 * flop / (best * 1e-3) / 1e12
        out[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS[name], 4)}
    out["method"] = "register-only MFMA loop, 4 independent 32x32 chains per wave, 4 waves per SIMD, best of 4"
    return out


def split_timing(fwd, bwd, steps: int) -> dict:
    """Median and minimum of the forward, the backward and their sum over
    `steps` iterations, each bracketed by events on the stream."""
    import statistics
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        fwd()
        e[1].record()
        bwd()
        e[2].record()
    torch.cuda.synchronize()
    f = [e[0].elapsed_time(e[1]) for e in ev]
    b = [e[1].elapsed_time(e[2]) for e in ev]
    t = [x + y for x, y in zip(f, b)]
    r = lambda v: {"median": round(statistics.median(v), 4), "min": round(min(v), 4)}
    return {"iterations": steps, "fwd_ms": r(f), "bwd_ms": r(b), "fwd_bwd_ms": r(t)}


def cpu_baseline(sh, inp, budget_s: float = 12.0) -> dict:
    """Oracle forward + backward on whole sequences of the workload until the
    budget is spent (at least one sequence)."""
    from oracle import block as ob
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    t0 = time.perf_counter()
    nseq = 0
    while nseq < sh.B:
        c = ob.block_fwd(inp["x"][nseq:nseq + 1], *W, H=sh.H, eps=sh.eps, rope_base=sh.rope_base,
                         window=sh.window or None, n_kv_head=sh.n_kv_head or None)
        ob.block_bwd(inp["dy"][nseq:nseq + 1], c, *W, H=sh.H)
        nseq += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": nseq * sh.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nseq} of {sh.B} sequences (T={sh.T}) of the workload, float64 numpy, {dt:.1f} s",
            "seconds": dt, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="d20_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-smi", action="store_true",
                    help="skip the SMI clock/power query (for runs under a profiler, whose preloaded "
                         "library would follow the SMI tool's own start-up)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (the known-size kernel that scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the block step is measured on one GPU's share "
              "(see the sharding notes); --gpus must be 1", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    from blockinputs import DECODE_WORKLOADS, HEAD_WORKLOADS
    if args.workload in DECODE_WORKLOADS:
        return bench_decode(args)
    if args.workload in HEAD_WORKLOADS:
        return bench_head(args)
    return bench_train(args)


COPY_BYTES = 1 << 30


def copy_calibration() -> int:
    """Five copies of 1 GiB between two device buffers: each dispatch reads
    and writes exactly COPY_BYTES, so FETCH_SIZE / WRITE_SIZE of these
    dispatches give the counters' scale."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)
    return 0


def source_digest() -> str:
    """SHA-256 over the HIP sources with comments and blank lines removed: a
    traffic figure measured on other code no longer describes the kernel,
    while an edit of the comments leaves the code (and the figure) as it was."""
    import hashlib
    import re
    h = hashlib.sha256()
    d = os.path.join(ROOT, "backward_gpt_block_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".cuh", ".hip")):
            text = open(os.path.join(d, name), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
            h.update(name.encode())
            h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of launch site `kernel` on `workload` from the
    committed counter summary profiles/<workload>_hbm_traffic.txt, or None
    when there is none or it was measured on other sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    digest, value = None, None
    for line in open(path):
        if line.startswith("source_sha256:"):
            digest = line.split(":", 1)[1].strip()
        elif line.startswith(f"traffic {kernel}:"):
            value = float(line.split(":", 1)[1])
    return value if digest == source_digest() else None


def bench_train(args) -> int:
    import numpy as np
    import torch

    import backward_gpt_block_amd as bl
    from blockinputs import WORKLOADS, make_block_inputs, to_storage

    sh = WORKLOADS[args.workload]
    dt = sh.dtype
    log(f"workload {args.workload}: {sh}")
    t0 = time.perf_counter()
    inp = make_block_inputs(sh, seed=0)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        st = to_storage(a, dt)
        t = torch.from_numpy(st.view(np.int16) if dt == "bf16" else st)
        return (t.view(torch.bfloat16) if dt == "bf16" else t).to("cuda:0")

    x, dy = dev(inp["x"]), dev(inp["dy"])
    W = [dev(inp[k]) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    cfg = bl.BlockConfig(B=sh.B, T=sh.T, C=sh.C, H=sh.H, F=sh.F, eps=sh.eps, rope_base=sh.rope_base,
                         dtype=bl.BLK_BF16 if dt == "bf16" else bl.BLK_F32,
                         gemm=bl.BLK_GEMM_FP8_E4M3 if sh.gemm == "fp8" else bl.BLK_GEMM_NATIVE, window=sh.window,
                         n_kv_head=sh.n_kv_head)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dW = [torch.empty(w.shape, dtype=torch.float32, device="cuda:0") for w in W]
    saved = torch.empty(bl.block_saved_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    scratch = torch.empty(bl.block_scratch_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def fwd():
        bl.block_fwd(cfg, x, *W, y, saved, scratch, stream=stream)

    def bwd():
        bl.block_bwd(cfg, dy, x, *W, saved, dx, *dW, 0, scratch, stream=stream)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps between two synchronisations, hipEvents on the stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"step: {ms:.3f} ms (wall {1e3 * wall / args.steps:.3f} ms)")

    # forward and backward separately: median and minimum over max(K, 20) iterations
    split = split_timing(fwd, bwd, max(args.steps, 20))
    log(f"split: {split}")
    smi = {"skipped": "--no-smi"} if args.no_smi else under_load(step)
    log(f"smi under load: {smi}")
    mfma = mfma_rates()
    log(f"mfma probe: {mfma}")

    # per-launch-site times over a second pass of the same K steps
    bl.block_timing_enable(True)
    for _ in range(args.steps):
        step()
    sites = bl.block_timing_read()
    bl.block_timing_enable(False)
    torch.cuda.synchronize()
    total_inst = sum(v[0] for v in sites.values())
    fl = site_flops(sh)
    log(f"{'site':22s} {'ms/step':>9s} {'share':>6s} {'avg ms':>8s} {'TFLOP/s':>8s}")
    for k, (tot, cnt) in sorted(sites.items(), key=lambda kv: -kv[1][0]):
        avg = tot / cnt
        tf = fl[k] / (avg * 1e-3) / 1e12 if k in fl else float("nan")
        log(f"{k:22s} {tot / args.steps:9.3f} {tot / total_inst:6.1%} {avg:8.3f} {tf:8.1f}")
    dom = max(sites.items(), key=lambda kv: kv[1][0])
    dname, (dtot, dcnt) = dom
    davg_ms = dtot / dcnt
    if dname in fl:
        achieved = fl[dname] / (davg_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS["fp8" if sh.gemm == "fp8" and dname.startswith("gemm") else dt]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(dname, args.workload), "kernel": dname,
                "avg_launch_ms": round(davg_ms, 4), "flops_per_launch": fl[dname]}
    else:
        sb = site_bytes(sh)
        roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": None,
                "traffic": measured_traffic(dname, args.workload), "kernel": dname, "avg_launch_ms": round(davg_ms, 4)}
        if dname in sb:   # bytes of all the site's launches in a step over their time in a step
            gbs = sb[dname] / (dtot / args.steps * 1e-3) / 1e9
            roof.update(achieved=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                        bytes_per_step=sb[dname], launches_per_step=dcnt // args.steps)

    tokens = sh.B * sh.T
    tflops = step_flops(sh) / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16" if dt == "bf16" else dt]
    frac = tflops / peak
    if sh.gemm == "fp8":
        # mixed roofline: the linear layers at the fp8 dense peak, attention at the bf16 one
        t_star = linear_flops(sh) / (PEAK_TFLOPS["fp8"] * 1e12) + 6.0 * attn_matmul_flops(sh) / (PEAK_TFLOPS["bf16"] * 1e12)
        frac = t_star / (ms * 1e-3)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(sh, inp, args.cpu_budget)
        log(f"cpu baseline: {cpu}")
    out = {
        "metric": WORKLOAD_METRIC.get(args.workload, METRIC), "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3+bf16" if sh.gemm == "fp8" else dt,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": sh.B, "T": sh.T, "C": sh.C, "H": sh.H, "D": sh.D, "F": sh.F,
                   "gemm": sh.gemm, "window": window_of(sh), "n_kv_head": kv_heads(sh), "tokens_per_step": tokens,
                   "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2), "frac_of_peak": round(frac, 4),
        "tflops_nanochat_convention": round(step_flops_nanochat(sh) / (ms * 1e-3) / 1e12, 2),
        "roofline": roof, "cpu_baseline": cpu,
        "split": split, "smi_under_load": smi, "mfma_probe": mfma,
    }
    print(json.dumps(out), flush=True)
    return 0


def decode_attn_bytes(sh, lens) -> float:
    """Algorithmic HBM bytes of one decode attention launch: the keys and
    values of the visible slots (0..L_b, or the last W of them) of every
    (sequence, key/value head), bf16, and the q rows of every query head."""
    import numpy as np
    keys = np.asarray(lens, dtype=np.int64) + 1
    if getattr(sh, "window", 0) > 0:
        keys = np.minimum(keys, sh.window)
    kv = 2.0 * kv_heads(sh) * 128 * 2 * float(np.sum(keys))
    return kv + sh.B * sh.H * 128 * 4.0


def decode_step_bytes(sh, lens) -> float:
    """Algorithmic HBM bytes of one decode step: every weight once (bf16),
    the cache reads, the new slot writes, x in and y out."""
    C = sh.C
    w = 2.0 * matmul_params(sh)
    return w + decode_attn_bytes(sh, lens) + sh.B * (2.0 * kv_heads(sh) * 128 * 2 + 2 * C * 2)


def cpu_decode_baseline(sh, inp, lens, budget_s: float) -> dict:
    """Oracle decode on whole sequences of the workload (a sub-batch with its
    own caches) until the budget is spent (at least one sequence)."""
    from oracle import block as ob
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    t0 = time.perf_counter()
    n = 0
    while n < sh.B:
        sl = slice(n, n + 1)
        ob.decode_step(inp["x"][sl], *W, inp["k_cache"][sl], inp["v_cache"][sl], lens[sl], H=sh.H, eps=sh.eps,
                       rope_base=sh.rope_base, window=sh.window or None, n_kv_head=sh.n_kv_head or None)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {sh.B} sequences (cache length {int(lens[0])}) of the workload, float64 numpy, "
                      f"{dt:.1f} s", "seconds": dt, "host_cpus": os.cpu_count()}


def bench_decode(args) -> int:
    import numpy as np
    import torch

    import backward_gpt_block_amd as bl
    from blockinputs import DECODE_WORKLOADS, make_decode_inputs, ragged_lengths, to_storage

    sh = DECODE_WORKLOADS[args.workload]
    log(f"workload {args.workload}: {sh}")
    t0 = time.perf_counter()
    inp = make_decode_inputs(sh, seed=0, cache_len=sh.S_max - 1)
    rag = ragged_lengths(sh.B, 128, sh.S_max - 1, seed=0)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        return torch.from_numpy(to_storage(a, "bf16").view(np.int16)).view(torch.bfloat16).to("cuda:0")

    x = dev(inp["x"])
    W = [dev(inp[k]) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    kc, vc = dev(inp["k_cache"]), dev(inp["v_cache"])
    cfg = bl.DecodeConfig(B=sh.B, C=sh.C, H=sh.H, F=sh.F, S_max=sh.S_max, eps=sh.eps, rope_base=sh.rope_base,
                          window=sh.window, n_kv_head=sh.n_kv_head)
    y = torch.empty_like(x)
    scratch = torch.empty(bl.decode_scratch_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def run(lens_np):
        lens = torch.from_numpy(np.asarray(lens_np, dtype=np.int32)).to("cuda:0")

        def step():
            bl.decode_step(cfg, x, *W, kc, vc, lens, y, scratch, stream=stream)

        for _ in range(args.warmup):
            step()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.steps
        bl.block_timing_enable(True)
        for _ in range(args.steps):
            step()
        sites = bl.block_timing_read()
        bl.block_timing_enable(False)
        torch.cuda.synchronize()
        return ms, sites

    lens_u = inp["cache_len"]
    ms, sites = run(lens_u)
    ms_r, sites_r = run(rag)
    step_b = decode_step_bytes(sh, lens_u)
    log(f"decode step: {ms * 1e3:.1f} us, {step_b / (ms * 1e-3) / 1e9:.0f} GB/s of algorithmic traffic "
        f"({step_b / 1e6:.1f} MB); ragged 128..2048: {ms_r * 1e3:.1f} us")
    total = sum(v[0] for v in sites.values())
    for k, (tot, cnt) in sorted(sites.items(), key=lambda kv: -kv[1][0]):
        log(f"  {k:16s} {1e3 * tot / args.steps:8.1f} us/step {tot / total:6.1%}")
    dname, (dtot, dcnt) = max(sites.items(), key=lambda kv: kv[1][0])
    davg = dtot / dcnt
    roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": None,
            "traffic": measured_traffic(dname, args.workload), "kernel": dname, "avg_launch_ms": round(davg, 5)}
    if dname == "dec_attn":
        b = decode_attn_bytes(sh, lens_u)
        ach = b / (davg * 1e-3) / 1e9
        roof.update(achieved=round(ach, 1), frac=round(ach / HBM_PEAK_GBS, 4), bytes_per_launch=b)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_decode_baseline(sh, inp, lens_u, args.cpu_budget)
        log(f"cpu baseline: {cpu}")
    ra = sites_r.get("dec_attn")
    out = {
        "metric": DECODE_WORKLOAD_METRIC.get(args.workload, DECODE_METRIC), "value": round(sh.B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "B": sh.B, "C": sh.C, "H": sh.H, "D": sh.D, "F": sh.F,
                   "S_max": sh.S_max, "cache_len": int(lens_u[0]), "window": sh.window, "n_kv_head": kv_heads(sh),
                   "parallelism": "none (1 GPU)"},
        "step_gbs": round(step_b / (ms * 1e-3) / 1e9, 1), "step_frac_of_hbm": round(step_b / (ms * 1e-3) / 1e12 / 8.0, 4),
        "ragged_variant": {"cache_len": "uniform 128..2048", "ms_per_step": round(ms_r, 5),
                           "value": round(sh.B / (ms_r * 1e-3), 1),
                           "step_gbs": round(decode_step_bytes(sh, rag) / (ms_r * 1e-3) / 1e9, 1),
                           "attn_gbs": None if ra is None else
                           round(decode_attn_bytes(sh, rag) / (ra[0] / ra[1] * 1e-3) / 1e9, 1)},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_head_baseline(sh, inp, budget_s: float) -> dict:
    """Oracle head forward + backward on the first n rows of the workload,
    n doubling until the budget is spent."""
    import threadpoolctl
    from oracle import lm_head as oh
    n, spent = 16, 0.0
    while True:
        t0 = time.perf_counter()
        loss, c = oh.head_loss(inp["x"][:n], inp["w_lm"], inp["targets"][:n], eps=sh.eps)
        oh.head_loss_bwd(1.0, c, inp["w_lm"])
        spent = time.perf_counter() - t0
        if spent >= budget_s / 3 or 2 * n > sh.N:
            break
        n *= 2
    info = threadpoolctl.threadpool_info()
    cores = max([d.get("num_threads", 1) for d in info] or [1])
    return {"value": round(n / spent, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} rows of the workload (full 65,536-token vocabulary), float64, forward + backward"}


def bench_head(args) -> int:
    import numpy as np
    import torch

    import backward_gpt_block_amd as bl
    from blockinputs import HEAD_WORKLOADS, make_head_inputs, to_storage

    sh = HEAD_WORKLOADS[args.workload]
    log(f"workload {args.workload}: {sh}")
    t0 = time.perf_counter()
    inp = make_head_inputs(sh, seed=0, uncounted=0.0)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        return torch.from_numpy(to_storage(a, "bf16").view(np.int16)).view(torch.bfloat16).to("cuda:0")

    x, w = dev(inp["x"]), dev(inp["w_lm"])
    tg = torch.from_numpy(inp["targets"]).to("cuda:0")
    cfg = bl.HeadConfig(N=sh.N, C=sh.C, V=sh.V, eps=sh.eps)
    loss = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    lse = torch.empty(sh.N, dtype=torch.float32, device="cuda:0")
    dx = torch.empty_like(x)
    dw = torch.empty(w.shape, dtype=torch.float32, device="cuda:0")
    scratch = torch.empty(bl.head_scratch_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        bl.head_loss_fwd(cfg, x, w, tg, loss, lse, scratch, stream=stream)
        bl.head_loss_bwd(cfg, x, w, tg, lse, 1.0, dx, dw, 0, scratch, stream=stream)

    for _ in range(args.warmup):
        step()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    bl.block_timing_enable(True)
    for _ in range(args.steps):
        step()
    sites = bl.block_timing_read()
    bl.block_timing_enable(False)
    torch.cuda.synchronize()
    mm = 2.0 * sh.N * sh.C * sh.V                 # one N x C x V matmul
    alg = 3 * mm                                   # z, dh, dW (the recomputed z is not counted)
    tflops = alg / (ms * 1e-3) / 1e12
    log(f"head step: {ms:.3f} ms, {tflops:.1f} TFLOP/s algorithmic ({alg / 1e12:.2f} TFLOP; "
        f"{4 * mm / (ms * 1e-3) / 1e12:.1f} TFLOP/s executed with the recompute), loss {loss.item():.4f}")
    total = sum(v[0] for v in sites.values())
    gemm_sites = ("gemm_head_fwd", "gemm_head_dz", "gemm_head_dgrad", "gemm_head_wgrad")
    for k, (tot, cnt) in sorted(sites.items(), key=lambda kv: -kv[1][0]):
        tf = mm / (tot / cnt * 1e-3) / 1e12 if k in gemm_sites else float("nan")
        log(f"  {k:18s} {tot / args.steps:8.3f} ms/step {tot / total:6.1%}  {tf:7.1f} TFLOP/s")
    dname, (dtot, dcnt) = max(sites.items(), key=lambda kv: kv[1][0])
    davg = dtot / dcnt
    ach = mm / (davg * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
            "frac": round(ach / PEAK_TFLOPS["bf16"], 4), "traffic": measured_traffic(dname, args.workload),
            "kernel": dname, "avg_launch_ms": round(davg, 4), "flops_per_launch": mm}
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_head_baseline(sh, inp, args.cpu_budget)
        log(f"cpu baseline: {cpu}")
    out = {
        "metric": HEAD_METRIC, "value": round(sh.N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "N": sh.N, "C": sh.C, "V": sh.V, "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2), "frac_of_peak": round(tflops / PEAK_TFLOPS["bf16"], 4),
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
