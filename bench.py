#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one forward pass (fa_fwd) plus one recompute backward pass (fa_bwd's three
launches) over the bf16 causal workload B=2, H=16, N=8192, d=128 with synthetic
Gaussian Q, K, V, dO already resident in HBM. Prints ONE JSON line.

FLOP convention: forward 4*B*H*N_q*N_k*d halved for causal; backward 2.5x forward.
The roofline object describes the dominant kernel, timed with HIP events recorded on
the stream the kernels run on; its achieved rate uses the algorithmic FLOPs of that
kernel (see ALG_FLOPS below). The CPU baseline times the float64 oracle (fwd + bwd)
on a bounded sample of whole (b, h) heads of the same workload. A supplementary list
times the forward on short sequences and decode-like shapes (compulsory-byte GB/s), and
another the forward and backward of the same workload under block-sparse bitmaps, and
the FP8 path (quantiser + FP8 forward) on the same inputs, and a sweep over the five
synthetic workloads (forward of each, backward of the last).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd(+bwd) TFLOP/s and % of MI355X bf16 MFMA peak, B·H·N²·d sweep"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # dense E4M3 MFMA (published 5.0 PFLOP/s)

# HBM traffic of the kernels from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (bytes per
# launch, already scaled by the copy-kernel calibration factor), keyed by the sha256 of
# the kernel source they were measured on. A changed source means stale counters -> null.
TRAFFIC = {
    # kernel: (source hash, bytes read, bytes written) -- profiles/attention_fwd_bwd_bf16_causal_B2H16N8192d128.md
    # (fa_bwd.hip changed after the counters only in instantiations these kernels do not
    # use: their generated code is the same instruction for instruction)
    "fwd": ("ce35e01e02c6d7f7", 477.6e6, 68.2e6),
    "bwd_prep": ("9d7b42bf8f4a1505", 136.3e6, 2.1e6),
    "bwd_dkdv": ("9d7b42bf8f4a1505", 270.9e6, 268.4e6),
    "bwd_dq": ("9d7b42bf8f4a1505", 673.3e6, 134.7e6),
}


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_flash_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SRC = {
    "fwd": ("fa_fwd.hip", "fa_device.h"),
    "bwd_prep": ("fa_bwd.hip", "fa_device.h"),
    "bwd_dkdv": ("fa_bwd.hip", "fa_device.h"),
    "bwd_dq": ("fa_bwd.hip", "fa_device.h"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-shapes", action="store_true",
                    help="skip the supplementary short-N and decode-like forward timings")
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the supplementary block-sparse fwd/bwd timings")
    ap.add_argument("--sparse-only", action="store_true",
                    help="only time the block-sparse shapes and print them as one JSON line")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the supplementary forward timings of the five workloads")
    ap.add_argument("--sweep-only", action="store_true",
                    help="only time the five workloads and print them as one JSON line")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the supplementary FP8 forward timings")
    ap.add_argument("--fp8-only", action="store_true",
                    help="only time the FP8 path and print it as one JSON line")
    ap.add_argument("--no-bias-tensor", action="store_true",
                    help="skip the supplementary bias-tensor fwd/bwd timings")
    ap.add_argument("--bias-only", action="store_true",
                    help="only time the bias-tensor shapes and print them as one JSON line")
    ap.add_argument("--hbm-only", action="store_true",
                    help="only time the supplementary shapes and print them as one JSON line")
    ap.add_argument("--hbm-filter", default="",
                    help="time only the supplementary shapes whose name contains this text")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the known-size "
                         "reference for scaling FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


def calibrate_copy():
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the attention kernels shard over (batch, head) with no exchange, so a multi-GPU "
              "figure is N independent copies of this one.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.hbm_only:
        import torch
        import exact_io_aware_flash_amd as fa
        fa.load_library()  # fails loudly if the HIP library is missing
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"hbm_shapes": hbm_shapes(fa, torch, args.hbm_filter)}), flush=True)
        return

    import numpy as np
    import torch

    import exact_io_aware_flash_amd as fa
    from synth import WORKLOADS, qkv_inputs

    if args.fp8_only:
        fa.load_library()  # fails loudly if the HIP library is missing
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"fp8": fp8_forward(fa, torch, WORKLOADS[5], qkv_inputs)}), flush=True)
        return
    if args.bias_only:
        fa.load_library()  # fails loudly if the HIP library is missing
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"bias_tensor": bias_tensor_bench(fa, torch)}), flush=True)
        return
    if args.sweep_only:
        fa.load_library()  # fails loudly if the HIP library is missing
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"sweep": workload_sweep(fa, torch)}), flush=True)
        return
    if args.sparse_only:
        fa.load_library()  # fails loudly if the HIP library is missing
        if not torch.cuda.is_available():
            print("no GPU visible", file=sys.stderr)
            sys.exit(1)
        print(json.dumps({"block_sparse": block_sparse(fa, torch, WORKLOADS[5], qkv_inputs)}),
              flush=True)
        return

    fa.load_library()  # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    w = WORKLOADS[5]
    B, H, N, d = w.B, w.H, w.N_q, w.d
    q, k, v, do = (t.to(dev) for t in qkv_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d), dtype=torch.uint8, device=dev)
    kw = dict(causal=True, scale=w.scale)

    phases = [("bwd_prep", fa.FA_BWD_PREP), ("bwd_dkdv", fa.FA_BWD_DKDV), ("bwd_dq", fa.FA_BWD_DQ)]
    names = ["fwd"] + [p[0] for p in phases]

    def step(ev=None):
        if ev is not None:
            ev[0][0].record()
        fa.fa_fwd(q, k, v, out=o, lse=lse, **kw)
        for i, (_, ph) in enumerate(phases):
            if ev is not None:
                ev[i][1].record()
                ev[i + 1][0].record()
            fa.fa_bwd(do, q, k, v, o, lse, grads=grads, workspace=ws, phases=ph, **kw)
        if ev is not None:
            ev[len(phases)][1].record()

    fwd_flops = 4.0 * B * H * N * N * d / 2.0
    bwd_flops = 2.5 * fwd_flops

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    peak_bytes = torch.cuda.max_memory_allocated(dev)
    io_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, do, o, lse) + grads)

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in names]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = {n: float(np.mean([events[s][i][0].elapsed_time(events[s][i][1])
                                 for s in range(args.steps)])) for i, n in enumerate(names)}

    step_flops = fwd_flops + bwd_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # algorithmic work per launch: 2*d FLOP per visible (query, key) pair and product;
    # causal with N_q == N_k has N(N+1)/2 visible pairs per head
    pairs = B * H * N * (N + 1) / 2.0
    ALG_FLOPS = {
        "fwd": 4.0 * d * pairs,          # S = QK^T, O = PV
        "bwd_dkdv": 8.0 * d * pairs,     # S, dP = dO V^T, dV = P^T dO, dK = dS^T Q
        "bwd_dq": 2.0 * d * pairs,       # dQ = dS K (its S and dP recomputation is overhead)
    }
    prep_bytes = 2.0 * B * H * N * d * 2 + 4.0 * B * H * N
    kernels = {}
    for n in names:
        t = kern_ms[n] * 1e-3
        ent = {"avg_us": round(kern_ms[n] * 1e3, 2)}
        if n in ALG_FLOPS:
            ent["alg_tflops"] = round(ALG_FLOPS[n] / t / 1e12, 1)
            ent["frac_bf16_peak"] = round(ALG_FLOPS[n] / t / 1e12 / PEAK_BF16_TFLOPS, 4)
        else:
            ent["alg_gbs"] = round(prep_bytes / t / 1e9, 1)
        kernels[n] = ent
    dom = max((n for n in names if n in ALG_FLOPS), key=lambda n: kern_ms[n])
    achieved = ALG_FLOPS[dom] / (kern_ms[dom] * 1e-3) / 1e12
    def traffic_of(n):
        tr = TRAFFIC.get(n)
        if tr is None or tr[0] != src_hash(*KERNEL_SRC[n]):
            return None  # no counters for this kernel source
        return tr[1] + tr[2]
    for n in names:
        t = traffic_of(n)
        if t is not None:
            kernels[n]["hbm_bytes"] = t
            kernels[n]["hbm_gbs"] = round(t / (kern_ms[n] * 1e-3) / 1e9, 1)
    traffic = traffic_of(dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}

    forms = backward_forms(fa, torch, q, k, v, do, o, lse, grads, ws, kw, bwd_flops)
    hbm = None if args.no_hbm_shapes else hbm_shapes(fa, torch)
    sparse = None if args.no_sparse else block_sparse(fa, torch, w, qkv_inputs)
    fp8 = None if args.no_fp8 else fp8_forward(fa, torch, w, qkv_inputs)
    sweep = None if args.no_sweep else workload_sweep(fa, torch)
    btensor = None if args.no_bias_tensor else bias_tensor_bench(fa, torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, do, args.cpu_seconds)

    fwd_tflops = fwd_flops / (kern_ms["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(kern_ms[p[0]] for p in phases)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "exact attention fwd+bwd, bf16 causal B2 H16 N8192 d128",
                   "B": B, "H": H, "N": N, "d": d, "causal": True,
                   "grad_dtype": "f32", "flop_convention": "fwd 4BHN^2d/2, bwd 2.5x fwd"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tflops, 1),
        "fwd_frac_of_bf16_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
        "kernels": kernels,
        # device memory held during the step: inputs, outputs and gradients, plus the
        # backward workspace (D and the scaled LSE); no N x N matrix is ever allocated
        "memory": {"peak_allocated_bytes": int(peak_bytes), "io_bytes": int(io_bytes),
                   "workspace_bytes": int(ws.numel()),
                   "score_matrix_bytes_bf16": int(2 * B * H * N * N)},
        "backward_forms": forms,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "hbm_shapes": hbm,
        "block_sparse": sparse,
        "fp8": fp8,
        "sweep": sweep,
        "bias_tensor": btensor,
    }
    print(json.dumps(line), flush=True)


def time_us(torch, fn, rounds=5, settle_ms=50.0, round_ms=10.0):
    """Average microseconds per call of `fn` over back-to-back calls, timed with HIP events
    on the launch stream (torch's current stream); median over `rounds`. Back-to-back calls
    keep the GPU busy, as in a real pass: a sync between single calls would let the clocks
    drop and add the host's launch time. The clocks also need tens of milliseconds of load
    to settle (back to back from idle, the causal B2 H16 N8192 d128 forward took 690 us,
    then 490 us after about 30 ms), so the calls
    are first repeated for `settle_ms`, and each round lasts at least `round_ms`."""
    def run(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / n  # ms per call

    run(3)
    est = max(run(3), 1e-3)
    run(min(5000, max(5, math.ceil(settle_ms / est))))
    reps = min(2000, max(10, math.ceil(round_ms / est)))
    ts = sorted(run(reps) * 1e3 for _ in range(rounds))
    return ts[len(ts) // 2]


def backward_forms(fa, torch, q, k, v, do, o, lse, grads, ws, kw, bwd_flops):
    """The whole backward of the main workload in its two forms, each timed by time_us:
    dQ in a separate query-outer pass (deterministic; the timed step above), and dQ added
    with float32 atomics inside the dK/dV pass (FA_BWD_DQ_ATOMIC)."""
    fa.fa_fwd(q, k, v, out=o, lse=lse, **kw)
    out = {}
    for name, ph in (("separate_dq_pass", fa.FA_BWD_ALL),
                     ("dq_atomics_in_dkdv_pass",
                      fa.FA_BWD_PREP | fa.FA_BWD_DKDV | fa.FA_BWD_DQ_ATOMIC)):
        us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads, workspace=ws,
                                              phases=ph, **kw))
        out[name] = {"bwd_us": round(us, 1), "bwd_tflops": round(bwd_flops / (us * 1e-6) / 1e12, 1)}
    return out


def hbm_shapes(fa, torch, only=""):
    """Forward time and compulsory-byte bandwidth on short sequences and decode-like shapes.

    Compulsory bytes: Q, K, V read and O written once (bf16) plus the float32 LSE. Inputs
    are seeded Gaussian bf16 made on the device; each shape is timed by time_us."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1234)
    shapes = [("short-N", 16, 32, n, n, False) for n in (128, 256, 512)]
    shapes += [("decode", 8, 32, nq, nk, True) for nq in (1, 16) for nk in (8192, 32768)]
    # one sequence, few heads: B H = 8 work-groups for the plain forward on 256 CUs
    shapes += [("decode", 1, 8, 1, 131072, True)]
    out = []
    for kind, B, H, nq, nk, causal in shapes:
        d = 128
        name = f"{kind} B{B} H{H} Nq{nq} Nk{nk} d{d}" + (" causal" if causal else "")
        if only and only not in name:
            continue
        q = torch.randn((B, H, nq, d), device=dev, generator=g).to(torch.bfloat16)
        k = torch.randn((B, H, nk, d), device=dev, generator=g).to(torch.bfloat16)
        v = torch.randn((B, H, nk, d), device=dev, generator=g).to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, nq), dtype=torch.float32, device=dev)
        nbytes = 2 * (2 * B * H * nq * d + 2 * B * H * nk * d) + 4 * B * H * nq
        paths = [("fa_fwd", lambda: fa.fa_fwd(q, k, v, causal=causal, out=o, lse=lse))]
        if kind == "decode":
            n = fa.fa_fwd_split_count(B, H, nq, nk, d, 0)
            ws = torch.empty(max(fa.fa_fwd_split_workspace_bytes(B, H, nq, nk, d, 0), 1),
                             dtype=torch.uint8, device=dev)
            paths.append((f"fa_fwd_split(n={n})",
                          lambda: fa.fa_fwd_split(q, k, v, causal=causal, out=o, lse=lse,
                                                  workspace=ws)))
        for path, fn in paths:
            us = time_us(torch, fn)
            out.append({"shape": name, "path": path, "us": round(us, 2),
                        "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)})
        del q, k, v, o, lse
    return out


def block_sparse(fa, torch, w, qkv_inputs):
    """Forward and backward of the main workload under block bitmaps (one per head).

    Seeded random bitmaps of 128 x 128 blocks at several densities, on top of the causal
    mask. Each path is timed by time_us; the rate counts only the visible (query, key)
    pairs, with the same per-pair FLOPs as the dense figures (forward 4d, backward 10d).
    The dense kernels on the same inputs are timed beside them."""
    import numpy as np

    dev = torch.device("cuda:0")
    B, H, N, d = w.B, w.H, w.N_q, w.d
    q, k, v, do = (t.to(dev) for t in qkv_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d), dtype=torch.uint8, device=dev)
    blk = 128
    nb = -(-N // blk)
    r = np.arange(nb)[:, None]
    c = np.arange(nb)[None, :]
    # causal pairs inside block (r, c) of a square N x N head (N a multiple of blk)
    causal_pairs = np.where(c < r, blk * blk, np.where(c == r, blk * (blk + 1) // 2, 0))

    out = []
    for density in (None, 1.0, 0.5, 0.25):
        kw = dict(causal=True, scale=w.scale)
        if density is None:  # no bitmap: the dense kernels
            pairs = B * H * N * (N + 1) / 2.0
        else:
            bm = (np.random.default_rng(4242).random((H, nb, nb)) < density).astype(np.uint8)
            pairs = float(B * (bm * causal_pairs[None]).sum())
            kw["block_mask"] = (torch.from_numpy(bm).to(dev), blk, blk)
        fwd_us = time_us(torch, lambda: fa.fa_fwd(q, k, v, out=o, lse=lse, **kw))
        fa.fa_fwd(q, k, v, out=o, lse=lse, **kw)
        bwd_us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads,
                                                  workspace=ws, **kw))
        out.append({"shape": f"bf16 causal B{B} H{H} N{N} d{d}" + (
                        f", per-head {blk}x{blk} bitmap" if density is not None else ", no bitmap"),
                    "density": density, "visible_frac_of_causal": round(
                        pairs / (B * H * N * (N + 1) / 2.0), 4),
                    "fwd_us": round(fwd_us, 1), "bwd_us": round(bwd_us, 1),
                    "fwd_tflops": round(4.0 * d * pairs / (fwd_us * 1e-6) / 1e12, 1),
                    "bwd_tflops": round(10.0 * d * pairs / (bwd_us * 1e-6) / 1e12, 1)})
    del q, k, v, do, o, lse, grads, ws
    return out


def bias_tensor_bench(fa, torch):
    """The ALiBi-like workload (bf16 B2 H8 N8192 d128, key ranges) with its bias given as
    a float32 tensor [1, H, N, N] (one matrix per head, shared over the batch) instead of
    generated from the slope: forward, backward, backward writing dbias [B, H, N, N], and
    backward writing dbias [1, H, N, N] summed over the batch, each timed by time_us,
    beside the generated-slope forward and backward. Rates count
    the visible (query, key) pairs (forward 4d, backward 10d FLOPs each); the bias bytes
    are 4 per visible pair and (b, h), the dbias bytes the clear of the whole array plus
    4 per visible pair and (b, h)."""
    from synth import WORKLOADS, bias_tensor, key_ranges, qkv_inputs, seed_for

    dev = torch.device("cuda:0")
    w = WORKLOADS[4]
    B, H, N, d = w.B, w.H, w.N_q, w.d
    q, k, v, do = (t.to(dev) for t in qkv_inputs(w, with_dout=True))
    ks, ke = key_ranges(N, N, seed_for(w.wid, 9), 128, N // 2, 64)
    pairs = B * H * float((ke.clamp(0, N) - ks.clamp(0, N)).clamp(min=0).sum())
    rng = dict(key_start=ks.to(dev), key_end=ke.to(dev), scale=w.scale)
    bias = bias_tensor((1, H, N, N), seed_for(w.wid, 10), 1.0).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, N, d), dtype=torch.uint8, device=dev)
    dbias = torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    res = {"shape": f"bf16 B{B} H{H} N{N} d{d}, key ranges (visible {pairs / (B * H * N * N):.3f} "
                    "of the pairs)"}
    for name, kw in (("slope", dict(bias_slopes=w.bias_slope)), ("tensor", dict(bias=bias))):
        fwd_us = time_us(torch, lambda: fa.fa_fwd(q, k, v, out=o, lse=lse, **rng, **kw))
        fa.fa_fwd(q, k, v, out=o, lse=lse, **rng, **kw)
        bwd_us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads, workspace=ws,
                                                  **rng, **kw))
        ent = {"fwd_us": round(fwd_us, 1), "bwd_us": round(bwd_us, 1),
               "fwd_visible_tflops": round(4.0 * d * pairs / (fwd_us * 1e-6) / 1e12, 1),
               "bwd_visible_tflops": round(10.0 * d * pairs / (bwd_us * 1e-6) / 1e12, 1)}
        if name == "tensor":
            ent["fwd_bias_gbs"] = round(4.0 * pairs / (fwd_us * 1e-6) / 1e9, 1)
            db_us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads,
                                                     workspace=ws, dbias=dbias, **rng, **kw))
            ent["bwd_dbias_us"] = round(db_us, 1)
            ent["dbias_write_gbs"] = round((4.0 * B * H * N * N + 4.0 * pairs)
                                           / (db_us * 1e-6) / 1e9, 1)
            # the shared bias's own gradient: dbias [1, H, N, N] summed over the batch
            del dbias
            dbias = torch.empty((1, H, N, N), dtype=torch.float32, device=dev)
            ds_us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads,
                                                     workspace=ws, dbias=dbias, **rng, **kw))
            ent["bwd_dbias_summed_over_batch_us"] = round(ds_us, 1)
        res[name] = ent
    del q, k, v, do, o, lse, grads, ws, dbias, bias
    return res


def workload_sweep(fa, torch):
    """Forward of each of the five synthetic workloads (fwd + bwd for the last), timed by
    time_us, in TFLOP/s by the convention (4 B H N_q N_k d, halved for causal; masks and
    bias otherwise not discounted) and by the visible (query, key) pairs (4 d each), both
    also as a fraction of the MFMA peak of the input type."""
    from synth import WORKLOADS, key_ranges, qkv_inputs, seed_for

    dev = torch.device("cuda:0")
    out = []
    for wid in sorted(WORKLOADS):
        w = WORKLOADS[wid]
        q, k, v, do = (t.to(dev) if t is not None else None for t in qkv_inputs(w))
        kw = dict(causal=w.causal, scale=w.scale)
        if w.bias_slope is not None:
            kw["bias_slopes"] = w.bias_slope
        if w.key_range:
            ks, ke = key_ranges(w.N_q, w.N_k, seed_for(w.wid, 9), 128, w.N_k // 2, 64)
            kw.update(key_start=ks.to(dev), key_end=ke.to(dev))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
        fwd_us = time_us(torch, lambda: fa.fa_fwd(q, k, v, out=o, lse=lse, **kw))
        fl = 4.0 * w.B * w.H * w.N_q * w.N_k * w.d * (0.5 if w.causal else 1.0)
        # visible (query, key) pairs per head, for the work actually done
        if w.key_range:
            pairs = float((ke.clamp(0, w.N_k) - ks.clamp(0, w.N_k)).clamp(min=0).sum())
        elif w.causal:
            pairs = w.N_q * (w.N_q + 1) / 2.0 + (w.N_k - w.N_q) * w.N_q
        else:
            pairs = float(w.N_q * w.N_k)
        vis = 4.0 * w.d * pairs * w.B * w.H
        peak = 157.3 if w.dtype == "f32" else PEAK_BF16_TFLOPS  # fp32 / 16-bit dense MFMA
        ent = {"workload": w.name, "fwd_us": round(fwd_us, 1),
               "fwd_tflops": round(fl / (fwd_us * 1e-6) / 1e12, 1),
               "fwd_frac_of_peak": round(fl / (fwd_us * 1e-6) / 1e12 / peak, 4),
               "fwd_visible_tflops": round(vis / (fwd_us * 1e-6) / 1e12, 1),
               "fwd_visible_frac_of_peak": round(vis / (fwd_us * 1e-6) / 1e12 / peak, 4)}
        if w.backward:
            grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
            ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N_q, w.N_k, w.d),
                             dtype=torch.uint8, device=dev)
            fa.fa_fwd(q, k, v, out=o, lse=lse, **kw)
            bwd_us = time_us(torch, lambda: fa.fa_bwd(do, q, k, v, o, lse, grads=grads,
                                                      workspace=ws, **kw))
            ent.update(bwd_us=round(bwd_us, 1),
                       bwd_tflops=round(2.5 * fl / (bwd_us * 1e-6) / 1e12, 1))
        out.append(ent)
        del q, k, v, do, o, lse
    return out


def fp8_forward(fa, torch, w, qkv_inputs):
    """The FP8 path on the main workload's forward (rotated Q and K): the three quantiser
    calls and the FP8 forward, each timed by time_us. The forward's rate uses the same FLOP
    convention as the bf16 figures, against the dense E4M3 MFMA peak; the quantiser's
    bytes are the 16-bit input read and the codes written."""
    from synth import random_signs

    dev = torch.device("cuda:0")
    B, H, N, d = w.B, w.H, w.N_q, w.d
    q, k, v, _ = (t.to(dev) if t is not None else None for t in qkv_inputs(w, with_dout=False))
    signs = random_signs(d, 4243)
    q8, qa = fa.fa_fp8_quantize(q, fa.FA_FP8_Q, signs)
    k8, ka = fa.fa_fp8_quantize(k, fa.FA_FP8_K, signs)
    v8, va = fa.fa_fp8_quantize(v, fa.FA_FP8_V)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    fwd_us = time_us(torch, lambda: fa.fa_fwd_fp8(q8, k8, v8, qa, ka, va, N, N, causal=True,
                                                  scale=w.scale, rotated=True, out=o, lse=lse))
    quant = {}
    for name, x, lay, sg in (("q", q, fa.FA_FP8_Q, signs), ("k", k, fa.FA_FP8_K, signs),
                             ("v", v, fa.FA_FP8_V, None)):
        us = time_us(torch, lambda: fa.fa_fp8_quantize(x, lay, sg))
        nbytes = x.numel() * 3  # 16-bit values read, one-byte codes written
        quant[name] = {"us": round(us, 1), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
    fl = 4.0 * B * H * N * N * d / 2.0
    bf16_fwd_us = time_us(torch, lambda: fa.fa_fwd(q, k, v, causal=True, scale=w.scale,
                                                   out=o, lse=lse))
    return {"shape": f"bf16 causal B{B} H{H} N{N} d{d}, rotated Q/K",
            "fwd_fp8_us": round(fwd_us, 1),
            "fwd_fp8_tflops": round(fl / (fwd_us * 1e-6) / 1e12, 1),
            "fwd_fp8_frac_of_fp8_peak": round(fl / (fwd_us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "fwd_bf16_us": round(bf16_fwd_us, 1),
            "quantise": quant}


def cpu_baseline(w, q, k, v, do, seconds):
    """The float64 oracle (fwd + bwd) on whole heads of the same inputs, until `seconds`."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("internal_api") in ("openblas", "mkl", "blis")), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    el = 0.0
    for (b, h) in heads:
        one = lambda t: t[b:b + 1, h:h + 1].float().cpu().double().numpy()  # noqa: E731
        qn, kn, vn, don = one(q), one(k), one(v), one(do)
        t_start = time.perf_counter()
        oracle.attention_forward(qn, kn, vn, w.scale, causal=True)
        oracle.attention_backward(qn, kn, vn, don, w.scale, causal=True)
        el += time.perf_counter() - t_start
        done += 1
        if el >= seconds:
            break
    per_head = 4.0 * w.N_q * w.N_k * w.d / 2.0 * 3.5  # fwd + bwd, same convention
    return {"value": round(done * per_head / el / 1e12, 5), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle", "cpu": model,
            "sample": f"float64 numpy oracle fwd+bwd of {done} of {len(heads)} (b,h) heads "
                      f"at full N={w.N_q} ({el:.1f} s of oracle wall time)"}


if __name__ == "__main__":
    main()
