#!/usr/bin/env python3
"""Throughput of the VQ decode GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--copies C]

A step is one decode call of one layer: the grouped vq_gemv over the four
4096x4096 2-bit q/k/v/o matrices of a LLaMA-7B layer, batch 1 (workload 2;
--workload selects another, see synth).  Inputs are resident in HBM before
the timed region.  The timed steps rotate through C distinct copies of the
layer's packed indices (>= 2 GiB in total, larger than the 256 MB
Infinity Cache and the L2s) so every step streams its indices from HBM.  The
C calls are captured once in a HIP graph and the graph is replayed; HIP
events on the launch stream bracket the timed replays.

Prints one JSON line:
  value            effective weight-byte throughput (GB/s) of back-to-back
                   layer calls, launch gaps included; us_per_layer beside it
  roofline         the lookup kernel (one launch per call; 16-bit indices add a
                   pre-pass launch, counted in): algorithmic bytes per call
                   over the average call period in the timed
                   region; traffic = HBM bytes per launch from the committed
                   rocprofv3 counter summary, when it was taken on the
                   current kernel source (else null)
  cpu_baseline     the float64 CPU oracle on the same layer, timed on the
                   host (one thread), repeated until >= --cpu-seconds
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, decimal GB/s
METRIC = "µs/layer and effective HBM GB/s (% of peak) for VQ-GEMV at LLaMA-7B, B=1"
CSRC = os.path.join(ROOT, "vector_quantized_decode_amd", "csrc")
# source of each workload's lookup kernel (8-bit indices: output-codebook tile
# kernels; 12- and 16-bit indices: virtual-codebook kernels)
KERNEL_SRC = {1: "vq_kernels_wc.hip", 2: "vq_kernels_wc.hip", 3: "vq_kernels_wc.hip",
              4: "vq_kernels_wc.hip", 5: "vq_kernels.hip", 6: "vq_kernels_wc.hip",
              7: "vq_kernels_wc.hip", 8: "vq_kernels_wc.hip", 9: "vq_kernels_wc.hip",
              10: "vq_kernels_tok.hip"}
PROFILES = os.path.join(ROOT, "profiles")

WORKLOAD_NAMES = {1: "vq-linear-512x512-2bit-b1",
                  2: "llama7b-attn-qkvo-4096x4096-2bit-b1",
                  3: "llama7b-decoder-7-linears-3bit-b1",
                  4: "llama13b-shaped-batched-decode-2bit-d8-b16",
                  5: "gemma2-9b-mlp-rotated-vq-residual-3.125bit-b1",
                 6: "qwen3-30b-a3b-moe-8-experts-gate-up-2bit-b1",
                 7: "qwen3-30b-a3b-moe-8-experts-down-2bit-b1",
                 8: "llama7b-attn-qkvo-4096x4096-2bit-b4",
                 9: "llama7b-mlp-gate-up-silu-fused-2bit-b1",
                  10: "llama7b-attn-qkvo-4096x4096-2bit-b16"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=25600)
    p.add_argument("--warmup", type=int, default=1024)
    p.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--copies", type=int, default=0, help="layer copies (0: enough for 2 GiB)")
    p.add_argument("--no-graph", action="store_true", help="launch from Python instead of a graph")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent on the oracle baseline")
    p.add_argument("--f16-out", action="store_true",
                   help="fp16 outputs (the fp16 epilogue: vq_gemv_f16, vq_gemv_swiglu_f16)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 256 MiB device copy (HBM counter calibration)")
    return p.parse_args()


def kernel_source_sha(workload: int) -> str:
    with open(os.path.join(CSRC, KERNEL_SRC[workload]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload: int):
    """HBM bytes per launch of the lookup kernel from the committed counter
    summary of this workload, if it was taken on the current kernel source."""
    sha = kernel_source_sha(workload)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        text = open(path).read()
        m = re.search(r"traffic-record: workload=(\d+) kernel_sha=(\w+) "
                      r"fetch_bytes=([\d.]+) write_bytes=([\d.]+)", text)
        if m and int(m.group(1)) == workload and m.group(2) == sha:
            return float(m.group(3)) + float(m.group(4)), os.path.basename(path)
    return None, None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus must be 1 (across "
                                   "GPUs a layer's matrices split by output rows, or by K with "
                                   "one all-reduce, each GPU running this path on its shard)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import synth
    import vector_quantized_decode_amd as vq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.workload(args.workload)
    residual = wl.residual
    # more than 4 tokens at d=4, n=8: the matrix-core call, on the row-tile index layout
    tokens = (wl.d, wl.nbits) == (4, 8) and wl.B > 4
    layer_bytes = synth.weight_bytes(args.workload)
    copies = args.copies or max(1, -(-(2 << 30) // layer_bytes))

    # ---- inputs: copy 0 from the seeded generator, packed + laid out by the library
    t0 = time.time()
    mis = [synth.matrix_inputs(args.workload, m) for m in range(wl.count)]
    base = []
    for mi in mis:
        if residual:
            base.append(vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits,
                                         sign_bits=mi.sign_bits, alpha=mi.alpha, group=mi.group,
                                         rht_sign=mi.rht_sign, had_block=mi.had_block, device=dev))
        else:
            base.append(vq.upload_matrix(mi.idx, mi.wc, mi.K, mi.N, mi.d, mi.nbits,
                                         tokens=tokens, device=dev))
    xs = [torch.from_numpy(mi.x).to(dev) for mi in mis]
    # further copies: seeded uniform random bytes in the device layouts (uniform bytes are
    # uniform indices and Bernoulli(0.5) sign bits); alpha is shared
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * args.workload + 99)
    layers = [base]
    for c in range(1, copies):
        lay = []
        for m in base:
            cp = vq.DeviceMatrix(m.K, m.N, m.d, m.nbits,
                                 torch.randint(0, 256, m.wi.shape, dtype=torch.uint8, device=dev,
                                               generator=gen), m.wc)
            if residual:
                cp.signs = torch.randint(0, 256, m.signs.shape, dtype=torch.uint8, device=dev,
                                         generator=gen)
                cp.alpha, cp.group, cp.rht_sign, cp.had_block = m.alpha, m.group, m.rht_sign, m.had_block
            lay.append(cp)
        layers.append(lay)
    f16_out = bool(args.f16_out)
    if f16_out and (residual or wl.B > 4):
        print("--f16-out applies to the plain and fused gate/up workloads", file=sys.stderr)
        sys.exit(2)
    ydt = torch.float16 if f16_out else torch.float32
    ys = [torch.empty((wl.B, m.N), dtype=ydt, device=dev) for m in base]
    ws = vq.alloc_workspace(base, wl.B, residual=residual, device=dev)
    call = vq.vq_gemv_residual if residual else (vq.vq_gemv_f16 if f16_out else vq.vq_gemv)
    if tokens:
        def call(lay, xs_, B_, ys_, ws_, n_, stream=None):
            vq.vq_gemv_tokens(lay, xs_, B_, ys_, stream=stream)
    if wl.gated_pairs:
        # gate/up pairs share the gate's x and write one gated output per pair
        def call(lay, xs_, B_, ys_, ws_, n_, stream=None):
            fn = vq.vq_gemv_swiglu_f16 if f16_out else vq.vq_gemv_swiglu
            fn(lay[0::2], lay[1::2], xs_[0::2], B_, ys_[0::2], ws_, n_, stream=stream)
    torch.cuda.synchronize()
    print(f"# setup: {copies} copies x {layer_bytes} B in {time.time() - t0:.1f} s",
          file=sys.stderr, flush=True)

    # ---- sampled parity check of copy 0 in the timed launch configuration
    parity = None
    if not args.no_check:
        import oracle
        call(layers[0], xs, wl.B, ys, ws, ws.numel())
        torch.cuda.synchronize()
        rng = np.random.default_rng(7)
        worst = 0.0
        ok = True
        for k, (mi, y) in enumerate(zip(mis, ys)):
            rows = np.sort(rng.choice(mi.N, size=min(256, mi.N), replace=False))
            if wl.gated_pairs:
                if k % 2:
                    continue                                  # the up matrix of a pair
                up = mis[k + 1]
                g = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx[rows], 8), rows.size,
                                   mi.K, mi.d, mi.nbits)
                u = oracle.vq_gemv(mi.x, up.wc, oracle.pack_rows(up.idx[rows], 8), rows.size,
                                   mi.K, mi.d, mi.nbits)
                ref = oracle.silu_gated(g, u)
            elif residual:
                ref = oracle.vq_gemv_residual(mi.x, mi.wc, oracle.pack_rows(mi.idx[rows], 8),
                                              oracle.pack_rows(mi.sign_bits[rows], 1),
                                              mi.alpha[rows], mi.rht_sign, mi.had_block,
                                              rows.size, mi.K, mi.d, mi.nbits, mi.group)
            else:
                ref = oracle.vq_gemv(mi.x, mi.wc, oracle.pack_rows(mi.idx[rows], mi.nbits),
                                     rows.size, mi.K, mi.d, mi.nbits)
            got = y.float().cpu().numpy()[:, rows]
            rel, mx, rms = oracle.compare(got, ref)
            worst = max(worst, rel)
            ok = ok and oracle.within_tolerance(got, ref)
        parity = {"sampled_rows_per_matrix": 256, "max_rel_l2": worst, "pass": bool(ok)}
        print(f"# parity (sampled rows): max rel_l2 {worst:.3e} pass={ok}", file=sys.stderr,
              flush=True)

    # ---- graph of one pass over all copies
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    per_graph = copies
    graph = None
    if not args.no_graph:
        with torch.cuda.stream(stream):
            for lay in layers[:2]:            # warm the launch path before capture
                call(lay, xs, wl.B, ys, ws, ws.numel(), stream=stream)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for lay in layers:
                call(lay, xs, wl.B, ys, ws, ws.numel(), stream=torch.cuda.current_stream())
        torch.cuda.synchronize()

    def run_steps(nsteps):
        if graph is not None:
            for _ in range(max(1, nsteps // per_graph)):
                graph.replay()
            return max(1, nsteps // per_graph) * per_graph
        with torch.cuda.stream(stream):
            for i in range(nsteps):
                call(layers[i % copies], xs, wl.B, ys, ws, ws.numel(), stream=stream)
        return nsteps

    with torch.cuda.stream(stream):
        run_steps(max(args.warmup, per_graph))
    torch.cuda.synchronize()

    # ---- timed region: back-to-back layer calls
    with torch.cuda.stream(stream):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        done = run_steps(args.steps)
        ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    us_per_layer = ms * 1e3 / done
    gbs = layer_bytes / (us_per_layer * 1e-6) / 1e9
    print(f"# timed {done} steps in {ms:.2f} ms: {us_per_layer:.3f} us/layer, {gbs:.1f} GB/s",
          file=sys.stderr, flush=True)

    # One call is one launch of the lookup kernel (the 16-bit format adds a
    # pre-pass launch), so the timed region's average call period is that
    # kernel's average duration back to back, plus the pre-pass where there
    # is one (rocprofv3's kernel trace of the same command reports both).
    launch_us = us_per_layer
    kernel_gbs = gbs

    # ---- plain copy of known size: the reference reading of the HBM byte counters
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print("# copy probe: 5 x 256 MiB device copies", file=sys.stderr, flush=True)

    # ---- CPU oracle baseline: the whole layer, one thread, >= cpu-seconds
    cpu = None
    if not args.no_cpu:
        import oracle
        from threadpoolctl import threadpool_limits
        packed = []
        for mi in mis:
            pw = oracle.pack_rows(mi.idx, mi.nbits)
            ps = oracle.pack_rows(mi.sign_bits, 1) if residual else None
            packed.append((pw, ps))

        def one_layer():
            if wl.gated_pairs:
                for k in range(0, len(mis), 2):
                    g, u = mis[k], mis[k + 1]
                    oracle.silu_gated(oracle.vq_gemv(g.x, g.wc, packed[k][0], g.N, g.K, g.d, g.nbits),
                                      oracle.vq_gemv(g.x, u.wc, packed[k + 1][0], g.N, g.K, g.d,
                                                     g.nbits))
                return
            for mi, (pw, ps) in zip(mis, packed):
                if residual:
                    oracle.vq_gemv_residual(mi.x, mi.wc, pw, ps, mi.alpha, mi.rht_sign,
                                            mi.had_block, mi.N, mi.K, mi.d, mi.nbits, mi.group)
                else:
                    oracle.vq_gemv(mi.x, mi.wc, pw, mi.N, mi.K, mi.d, mi.nbits)

        reps = []
        with threadpool_limits(limits=1):
            one_layer()                                   # warm
            t_all = time.perf_counter()
            while not reps or time.perf_counter() - t_all < args.cpu_seconds:
                t = time.perf_counter()
                one_layer()
                reps.append(time.perf_counter() - t)
        med = statistics.median(reps)
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": round(layer_bytes / med / 1e9, 5), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"the whole layer ({wl.count} matrices, {layer_bytes} weight bytes), "
                         f"float64 numpy oracle (unpack, output codebook, lookup sum"
                         f"{', rotation, residual' if residual else ''}) on one thread (BLAS "
                         f"limited to 1), {len(reps)} timed run(s) after 1 warm run, median; "
                         f"host has {cores} cores",
               "us_per_layer": round(med * 1e6, 1)}
        print(f"# cpu oracle: {med * 1e3:.1f} ms/layer over {len(reps)} runs", file=sys.stderr,
              flush=True)

    traffic, traffic_src = committed_traffic(args.workload)
    if f16_out:
        traffic, traffic_src = None, None   # the counters were taken with fp32 outputs
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": done,
        "warmup": args.warmup,
        "ms_per_step": us_per_layer / 1e3,
        "us_per_layer": round(us_per_layer, 4),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "matrices": wl.count,
                   "K_N": [[s.K, s.N] for s in wl.matrices], "d": wl.d, "nbits": wl.nbits,
                   "B": wl.B, "weight_bytes_per_layer": layer_bytes, "layer_copies": copies,
                   "launch": "hip graph" if graph is not None else "stream",
                   "y": "f16" if f16_out else "f32"},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel_us": round(launch_us, 4),
                     "launches_per_call": 2 if wl.nbits == 16 else 1,
                     "algorithmic_bytes_per_launch": layer_bytes,
                     "traffic_source": traffic_src, "kernel_source_sha": kernel_source_sha(args.workload)},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
