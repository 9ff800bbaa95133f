#!/usr/bin/env python3
"""Throughput of the VQ decode GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--repeats R] [--workload 2]

A step is one decode call of one layer: by default the grouped vq_gemv over
the four 4096x4096 2-bit q/k/v/o matrices of a LLaMA-7B layer, batch 1
(workload 2; --workload selects another, see synth).  Inputs are resident in
HBM before any timed region.

Protocol.  C distinct copies of the layer (indices, codebooks, and for the
residual workload signs, scales and rotation signs; >= 2 GiB in total, far
above the 256 MB Infinity Cache and the L2s) are laid out once.  The K timed
steps of a repeat are K back-to-back calls on K consecutive copies; HIP
events on the launch stream bracket each repeat, and the reported period is
the median of R repeats that start at successive copies.  The K calls are
timed two ways: captured in one HIP graph and replayed (an untimed replay of
the previous window first, so the host's submission latency falls outside
the timed span; timing.graph_from_idle reports the repeats without it), and
issued one by one from Python after a spin kernel that lets the host queue
them (timing.stream_launch).  A graph replay carries about 10 us of fixed
cost, which matters for small K; single launches cost slightly more per
call.  value uses the faster of the two medians (timing.reported names it);
the read floor and the dense context are timed the same way.

Prints one JSON line:
  value            weight bytes per layer / median call period (GB/s); us_per_layer
  timing           median, min and max repeat times of both protocols; stream
                   launches from an idle GPU (host submission included); a warm
                   figure (one copy repeated, cache-resident); vq_gemv_oc (the
                   output-codebook tile form) on the plain one-token 8-bit
                   workloads; vq_gemv_shared on workloads with shared codebooks
  roofline         the lookup kernel (one launch per call; 16-bit indices add a
                   pre-pass launch, counted in): algorithmic bytes per call over
                   the median call period.  stream_read_gbs: a plain streaming
                   read (vq_stream_read) of the same copies' device index
                   layouts (plus signs and scales), same K, same protocols, same
                   repeats; frac_of_stream_read = achieved / stream_read_gbs.
                   traffic = HBM bytes per launch from the committed rocprofv3
                   counter summary, when it was taken on the current kernel
                   source (else null)
  context          a dense fp16 GEMV at the same shapes (torch.mm on fp16
                   weights, C' distinct copies >= 2 GiB, same protocols):
                   context, not a target
  cpu_baseline     the float64 CPU oracle on the same layer, timed on the host
                   (one thread), repeated until >= --cpu-seconds
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
# source of each workload's lookup kernel
KERNEL_SRC = {1: "vq_kernels_wc.hip", 2: "vq_kernels_wc.hip", 3: "vq_kernels_wc.hip",
              4: "vq_kernels_wc.hip", 5: "vq_kernels.hip", 6: "vq_kernels_wc.hip",
              7: "vq_kernels_wc.hip", 8: "vq_kernels_tok.hip", 9: "vq_kernels_wc.hip",
              10: "vq_kernels_tok.hip", 11: "vq_kernels_wc.hip"}
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 2 << 30       # distinct layer copies: at least this many weight bytes
MAX_COPIES = 2048          # tiny layers: capped (then the copies are cache-resident)

WORKLOAD_NAMES = {1: "vq-linear-512x512-2bit-b1",
                  2: "llama7b-attn-qkvo-4096x4096-2bit-b1",
                  3: "llama7b-decoder-7-linears-3bit-b1",
                  4: "llama13b-shaped-batched-decode-2bit-d8-b16",
                  5: "gemma2-9b-mlp-rotated-vq-residual-3.125bit-b1",
                  6: "qwen3-30b-a3b-moe-8-experts-gate-up-2bit-b1",
                  7: "qwen3-30b-a3b-moe-8-experts-down-2bit-b1",
                  8: "llama7b-attn-qkvo-4096x4096-2bit-b4",
                  9: "llama7b-mlp-gate-up-silu-fused-2bit-b1",
                  10: "llama7b-attn-qkvo-4096x4096-2bit-b16",
                  11: "llama7b-attn-qkvo-4096x4096-2bit-b1-qkv-shared-codebook"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128, help="calls timed per repeat (exact)")
    p.add_argument("--warmup", type=int, default=128, help="untimed calls before timing (at least)")
    p.add_argument("--repeats", type=int, default=20, help="timed repeats (median reported)")
    p.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOAD_NAMES))
    p.add_argument("--copies", type=int, default=0, help="layer copies (0: enough for 2 GiB)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    p.add_argument("--no-context", action="store_true",
                   help="skip the stream-read floor, plain-stream, warm and dense fp16 runs")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent on the oracle baseline")
    p.add_argument("--f16-out", action="store_true",
                   help="fp16 outputs (the fp16 epilogue: vq_gemv_f16, vq_gemv_swiglu_f16)")
    p.add_argument("--dense-only", action="store_true",
                   help="only the dense fp16 GEMV context run (prints its JSON)")
    p.add_argument("--call", choices=["default", "oc"], default="default",
                   help="oc: time vq_gemv_oc (the output-codebook tile form) instead of vq_gemv "
                        "(d=4, n=8, one token, no residual)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 256 MiB device copy (HBM counter calibration)")
    return p.parse_args()


OC_SRC = "vq_kernels.hip"  # source of vq_gemv_oc's kernel


def kernel_source_sha(workload: int, call: str = "default") -> str:
    src = OC_SRC if call == "oc" else KERNEL_SRC[workload]
    with open(os.path.join(CSRC, src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(workload: int, call: str = "default"):
    """HBM bytes per launch of the lookup kernel from the committed counter
    summary of this workload and call, if it was taken on the current kernel
    source."""
    sha = kernel_source_sha(workload, call)
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        text = open(path).read()
        m = re.search(r"traffic-record: workload=(\d+)(?: call=(\w+))? kernel_sha=(\w+) "
                      r"fetch_bytes=([\d.]+) write_bytes=([\d.]+)", text)
        if m and int(m.group(1)) == workload and (m.group(2) or "default") == call \
                and m.group(3) == sha:
            return float(m.group(4)) + float(m.group(5)), os.path.basename(path)
    return None, None


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """Exactly K calls per repeat, from graphs captured over consecutive
    layer copies.  call_for(c) gives a callable(stream) that launches the
    call on copy c.  With K <= C the copies are cut into C / K windows of K
    (C is rounded up to a multiple of K), one graph each, and repeat r
    replays window r mod (C / K); with K > C a repeat replays a graph of all
    C copies K // C times and a graph of the first K mod C copies once."""

    def __init__(self, torch, call_for, copies: int, K: int, stream, same_copy: bool = False):
        self.torch, self.stream, self.K = torch, stream, K
        if same_copy:
            self.reps = [[self._capture([call_for(0)] * K)]]
        elif K <= copies:
            self.reps = [[self._capture([call_for(w * K + i) for i in range(K)])]
                         for w in range(copies // K)]
        else:
            full = self._capture([call_for(c) for c in range(copies)])
            seq = [full] * (K // copies)
            if K % copies:
                seq.append(self._capture([call_for(c) for c in range(K % copies)]))
            self.reps = [seq]

    def _capture(self, fns):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            s = torch.cuda.current_stream()
            for f in fns:
                f(s)
        torch.cuda.synchronize()
        return g

    def warm(self, steps: int) -> int:
        n = max(len(self.reps), -(-steps // self.K))
        with self.torch.cuda.stream(self.stream):
            for r in range(n):
                for g in self.reps[r % len(self.reps)]:
                    g.replay()
        self.torch.cuda.synchronize()
        return n * self.K

    def time(self, repeats: int, lead_in: bool = True):
        """Per repeat: synchronize, (lead-in) replay the previous window
        untimed, record e0, replay the K timed calls, record e1, synchronize.
        The lead-in keeps the GPU busy while the host submits the timed
        graph, so e0..e1 spans exactly the K calls back to back and not the
        host's submission latency from an idle GPU (lead_in=False measures
        that too)."""
        torch = self.torch
        out = []
        n = len(self.reps)
        for r in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            with torch.cuda.stream(self.stream):
                if lead_in:
                    for g in self.reps[(r - 1) % n]:
                        g.replay()
                e0.record(self.stream)
                for g in self.reps[r % n]:
                    g.replay()
                e1.record(self.stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return out


def time_stream_launches(torch, call_for, copies: int, K: int, repeats: int, stream,
                         lead_in: bool = True):
    """The same K calls issued one by one from Python (prepared ctypes
    arguments), no graph.  With lead_in, a spin kernel (torch.cuda._sleep,
    about 8 us per call) runs before e0 so that the host has queued the K
    calls by the time the GPU reaches them: e0..e1 then spans the K calls
    back to back, not the host's submission rate."""
    out = []
    for r in range(repeats):
        calls = [call_for((r * K + i) % copies) for i in range(K)]
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            if lead_in:
                torch.cuda._sleep(20000 * K)
            e0.record(stream)
            for f in calls:
                f(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def time_both(torch, call_for, copies: int, K: int, repeats: int, warmup: int, stream):
    """Exactly K calls per repeat over the same layer copies, timed two ways:
    one HIP graph of the K calls (Timer), and the K calls issued one by one
    behind a spin lead-in.  A graph replay costs about 10 us of fixed time,
    which a window of few calls cannot amortize; single launches cost a
    little more per call.  Returns the faster protocol's summary, both
    summaries, the faster one's name, the untimed warm-up calls run and the
    Timer."""
    t = Timer(torch, call_for, copies, K, stream)
    warm = t.warm(warmup)
    g = summary(t.time(repeats), K)
    s = dict(summary(time_stream_launches(torch, call_for, copies, K, repeats, stream), K),
             what="the K calls issued one by one after a spin lead-in")
    best, launch = (g, "hip graph") if g["us_per_call"] <= s["us_per_call"] else (s, "stream launches")
    return best, g, s, launch, warm, t


def summary(ms_list, K):
    med = statistics.median(ms_list)
    return {"median_ms": round(med, 5), "min_ms": round(min(ms_list), 5),
            "max_ms": round(max(ms_list), 5), "us_per_call": round(med * 1e3 / K, 4)}


def dense_gemv_run(args) -> dict:
    """Dense fp16 GEMV at the workload's shapes (torch.mm on fp16 [N][K]
    weights with x^T), C' distinct weight copies >= 2 GiB, the same exact-K,
    repeated, graph-replay protocol: context for the quantized call, not a
    target."""
    import torch

    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    try:
        torch.backends.cuda.preferred_blas_library("cublas")   # rocBLAS on ROCm
    except Exception:                                           # older torch: its default
        pass
    wl = synth.workload(args.workload)
    K = args.steps
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * args.workload + 98)
    shapes = [(m.N, m.K) for m in wl.matrices]
    dense_bytes = sum(n * k * 2 for n, k in shapes)
    dcopies = max(1, -(-COPY_BYTES // dense_bytes))
    dws = [[torch.randn(sh, generator=gen, device=dev, dtype=torch.float32).half() for sh in shapes]
           for _ in range(dcopies)]
    xT = [torch.randn((k, wl.B), generator=gen, device=dev, dtype=torch.float32).half()
          for _, k in shapes]
    yd = [torch.empty((n, wl.B), dtype=torch.float16, device=dev) for n, _ in shapes]

    def dense_for(c):
        def f(s, c=c):
            for W, xt, yy in zip(dws[c % dcopies], xT, yd):
                torch.mm(W, xt, out=yy)
        return f

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):                   # the BLAS library sets up eagerly
        for c in range(dcopies):
            dense_for(c)(stream)
    torch.cuda.synchronize()
    dcop = dcopies if K > dcopies else -(-dcopies // K) * K
    ds, dg, dsl, dlaunch, _, _ = time_both(torch, dense_for, dcop, K, args.repeats, args.warmup,
                                           stream)
    return dict(ds, weight_bytes_per_layer=dense_bytes,
                gbs=round(dense_bytes / (ds["us_per_call"] * 1e-6) / 1e9, 1),
                copies=dcopies, launch=dlaunch, graph_us_per_call=dg["us_per_call"],
                stream_launch_us_per_call=dsl["us_per_call"],
                blas="rocBLAS (torch preferred_blas_library)",
                what="torch.mm of fp16 [N][K] weights with x^T, the workload's shapes and "
                     "tokens; context, not target")


def dense_context_subprocess(args) -> dict:
    """dense_gemv_run in a child process, so that a BLAS library that fails
    under graph capture cannot end this run."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--dense-only", "--workload",
           str(args.workload), "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--repeats", str(args.repeats)]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    except subprocess.TimeoutExpired:
        return {"error": "dense fp16 GEMV run timed out"}
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    if r.returncode != 0 or not lines:
        tail = (r.stderr.strip().splitlines() or ["no output"])[-1][:300]
        say(f"# dense fp16 GEMV failed (rc {r.returncode}): {tail}")
        return {"error": f"rc {r.returncode}: {tail}"}
    d = json.loads(lines[-1])
    say(f"# dense fp16 GEMV: {d['us_per_call']:.3f} us/layer, {d['gbs']} GB/s")
    return d


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus must be 1 (across "
                                   "GPUs a layer's matrices split by output rows, or by K with "
                                   "one all-reduce, each GPU running this path on its shard)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.steps < 1 or args.repeats < 1:
        print(json.dumps({"error": "--steps and --repeats must be at least 1"}), flush=True)
        sys.exit(2)
    if args.dense_only:
        print(json.dumps(dense_gemv_run(args)), flush=True)
        return

    import torch

    import synth
    import vector_quantized_decode_amd as vq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.workload(args.workload)
    residual = wl.residual
    # 4 or more tokens at d=4, n=8: the matrix-core call, on the row-tile index
    # layout (from 4 tokens on it measured faster than the dot-product call)
    tokens = (wl.d, wl.nbits) == (4, 8) and wl.B >= 4
    f16_out = bool(args.f16_out)
    if f16_out and (residual or tokens):
        say("--f16-out applies to the plain and fused gate/up workloads")
        sys.exit(2)
    # the plain one-token 8-bit workloads, which vq_gemv_oc also serves
    oc_able = (wl.d, wl.nbits, wl.B) == (4, 8, 1) and not residual and not wl.gated_pairs
    oc = args.call == "oc"
    if oc and (not oc_able or f16_out):
        say("--call oc applies to plain d=4, n=8, one-token workloads with fp32 outputs")
        sys.exit(2)
    layer_bytes = synth.weight_bytes(args.workload)
    K = args.steps
    c0 = args.copies or min(MAX_COPIES, max(1, -(-COPY_BYTES // layer_bytes)))
    copies = c0 if K > c0 else -(-c0 // K) * K

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
    lead = [synth.shared_leader(args.workload, m) for m in range(wl.count)]
    for m, l in enumerate(lead):          # shared groups pass one codebook and one x
        if l != m:
            base[m].wc, xs[m] = base[l].wc, xs[l]
    # Further copies, each with its own weights: seeded uniform random bytes in
    # the device layouts (uniform bytes are uniform indices and Bernoulli(0.5)
    # sign bits), a codebook drawn N(0, 0.02), scales U(0.001, 0.01) laid out by
    # vq_repack_alpha, rotation signs uniform over +-1.
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * args.workload + 99)
    # each matrix's copies are drawn by one generator call and sliced (all
    # slices stay 16-byte aligned): a few launches per matrix, not per copy
    nc = copies - 1
    draws = []
    for mm, m in enumerate(base):
        d = {"wi": torch.randint(0, 256, (nc, *m.wi.shape), dtype=torch.uint8, device=dev,
                                 generator=gen)}
        if lead[mm] == mm:
            d["wc"] = (torch.randn((nc, *m.wc.shape), generator=gen, device=dev,
                                   dtype=torch.float32) * 0.02).half()
        if residual:
            d["signs"] = torch.randint(0, 256, (nc, *m.signs.shape), dtype=torch.uint8, device=dev,
                                       generator=gen)
            d["alpha"] = (torch.rand((nc, m.N, m.K // m.group), generator=gen, device=dev,
                                     dtype=torch.float32) * 0.009 + 0.001).half()
            d["rht"] = torch.randint(0, 2, (nc, m.K), generator=gen, device=dev,
                                     dtype=torch.int8) * 2 - 1
        draws.append(d)
    layers = [base]
    for c in range(1, copies):
        lay = []
        for mm, m in enumerate(base):
            d = draws[mm]
            wc = lay[lead[mm]].wc if lead[mm] != mm else d["wc"][c - 1]
            cp = vq.DeviceMatrix(m.K, m.N, m.d, m.nbits, d["wi"][c - 1], wc)
            if residual:
                cp.signs = d["signs"][c - 1]
                cp.alpha = torch.empty_like(m.alpha)
                vq.vq_repack_alpha(d["alpha"][c - 1], m.N, m.K, m.group, cp.alpha)
                cp.group, cp.had_block = m.group, m.had_block
                cp.rht_sign = d["rht"][c - 1]
            lay.append(cp)
        layers.append(lay)
    ydt = torch.float16 if f16_out else torch.float32
    ys = [torch.empty((wl.B, m.N), dtype=ydt, device=dev) for m in base]
    ws = vq.alloc_workspace(base, wl.B, residual=residual or oc, device=dev)

    prepared = {}

    def call_for(c):
        """A prepared call of the timed kind on layer copy c."""
        if c in prepared:
            return prepared[c]
        lay = layers[c]
        if tokens:
            pc = vq.prepare_gemv_tokens(lay, xs, wl.B, ys)
        elif wl.gated_pairs:
            # gate/up pairs share the gate's x and write one gated output per pair
            pc = vq.prepare_gemv_swiglu(lay[0::2], lay[1::2], xs[0::2], wl.B, ys[0::2], f16=f16_out)
        else:
            name = ("vq_gemv_residual" if residual else "vq_gemv_oc" if oc
                    else "vq_gemv_f16" if f16_out else "vq_gemv")
            pc = vq.prepare_gemv(name, lay, xs, wl.B, ys, ws, ws.numel())
        prepared[c] = pc
        return pc

    torch.cuda.synchronize()
    say(f"# setup: {copies} copies x {layer_bytes} B in {time.time() - t0:.1f} s")

    # ---- sampled parity check of copy 0 in the timed launch configuration
    parity = None
    if not args.no_check:
        import oracle
        call_for(0)(torch.cuda.current_stream())
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
        say(f"# parity (sampled rows): max rel_l2 {worst:.3e} pass={ok}")

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for c in range(min(2, copies)):                   # the launch path before capture
            call_for(c)(stream)
    torch.cuda.synchronize()

    # ---- timed region: exactly K back-to-back calls per repeat
    best, st, sl, launch, warm_done, main_t = time_both(torch, call_for, copies, K, args.repeats,
                                                         args.warmup, stream)
    say(f"# graph: {args.repeats} x {K} steps (median {st['median_ms']:.4f} ms, "
        f"min {st['min_ms']:.4f}, max {st['max_ms']:.4f}): {st['us_per_call']:.3f} us/layer")
    say(f"# stream launches after a lead-in: {args.repeats} x {K} steps (median "
        f"{sl['median_ms']:.4f} ms, min {sl['min_ms']:.4f}, max {sl['max_ms']:.4f}): "
        f"{sl['us_per_call']:.3f} us/layer")
    us_per_layer = best["us_per_call"]
    gbs = layer_bytes / (us_per_layer * 1e-6) / 1e9
    say(f"# timed ({launch}): {us_per_layer:.3f} us/layer, {gbs:.1f} GB/s")
    timing = {"repeats": args.repeats, "steps_per_repeat": K, "warmup_steps_run": warm_done,
              "graph": st, "stream_launch": sl, "reported": launch}
    if not args.no_context:
        idle = summary(main_t.time(args.repeats, lead_in=False), K)
        timing["graph_from_idle"] = dict(idle, what="the same repeats with no lead-in: each "
                                                    "includes the graph's submission latency")
        say(f"# from an idle GPU (submission latency included): {idle['us_per_call']:.3f} us/layer")

    # ---- context: the read floor, plain stream launches, a warm figure, dense fp16
    read_gbs = None
    context = None
    if not args.no_context:
        def bufs_of(lay):
            b, n = [], []
            for m in lay:
                b.append(m.wi)
                n.append(m.wi.numel())
                if residual:
                    b += [m.signs, m.alpha]
                    n += [m.signs.numel(), m.alpha.numel() * 2]
            return b, n

        nb0 = bufs_of(layers[0])[1]
        sink_words = vq.vq_stream_read_sink_words(nb0)
        sink = torch.empty(sink_words, dtype=torch.int32, device=dev)
        read_prepared = {}

        def read_for(c):
            if c not in read_prepared:
                b, n = bufs_of(layers[c])
                read_prepared[c] = vq.prepare_stream_read(b, n, sink, sink_words)
            return read_prepared[c]

        read_bytes = sum(nb0)
        rs, rg, rsl, rlaunch, _, rt = time_both(torch, read_for, copies, K, args.repeats,
                                                args.warmup, stream)
        del rt
        read_gbs = read_bytes / (rs["us_per_call"] * 1e-6) / 1e9
        say(f"# stream read of {read_bytes} B per call ({rlaunch}): {rs['us_per_call']:.3f} us, "
            f"{read_gbs:.1f} GB/s (graph {rg['us_per_call']:.3f}, stream launches "
            f"{rsl['us_per_call']:.3f})")

        sn = summary(time_stream_launches(torch, call_for, copies, K, args.repeats, stream,
                                          lead_in=False), K)
        say(f"# stream launches from an idle GPU (host submission rate included): "
            f"{sn['us_per_call']:.3f} us/layer")
        wt = Timer(torch, call_for, copies, K, stream, same_copy=True)
        wt.warm(args.warmup)
        ws_ = summary(wt.time(args.repeats), K)
        say(f"# warm (copy 0 repeated): {ws_['us_per_call']:.3f} us/layer")
        del wt
        timing["stream_launch_from_idle"] = sn
        timing["warm_same_copy"] = ws_
        if wl.shared and not residual and not tokens and not wl.gated_pairs:
            # the same calls through vq_gemv_shared (shared matrices merged into units)
            merged = {}

            def merged_for(c):
                if c not in merged:
                    merged[c] = vq.prepare_gemv("vq_gemv_shared", layers[c], xs, wl.B, ys, ws,
                                                ws.numel())
                return merged[c]

            ms_, _, _, mlaunch, _, mt = time_both(torch, merged_for, copies, K, args.repeats,
                                                  args.warmup, stream)
            del mt
            timing["vq_gemv_shared"] = dict(ms_, launch=mlaunch,
                                            what="the same calls with the matrices that share a "
                                                 "codebook and x merged into units")
            say(f"# vq_gemv_shared (merged units): {ms_['us_per_call']:.3f} us/layer")
        if oc_able and not oc and not f16_out:
            # the same calls in the output-codebook tile form (vq_gemv_oc)
            ws_oc = vq.alloc_workspace(base, wl.B, residual=True, device=dev)
            oc_calls = {}

            def oc_for(c):
                if c not in oc_calls:
                    oc_calls[c] = vq.prepare_gemv("vq_gemv_oc", layers[c], xs, wl.B, ys, ws_oc,
                                                  ws_oc.numel())
                return oc_calls[c]

            os_, _, _, olaunch, _, ot = time_both(torch, oc_for, copies, K, args.repeats,
                                                  args.warmup, stream)
            del ot
            timing["vq_gemv_oc"] = dict(os_, launch=olaunch,
                                        what="the same calls in the output-codebook tile "
                                                  "form: an OC tile per workgroup in LDS, rows "
                                                  "split along K, a fixed-point atomic per row")
            say(f"# vq_gemv_oc (output-codebook tiles): {os_['us_per_call']:.3f} us/layer")
        timing["stream_read"] = dict(rs, bytes_per_call=read_bytes, launch=rlaunch,
                                     graph_us_per_call=rg["us_per_call"],
                                     stream_launch_us_per_call=rsl["us_per_call"],
                                     what="vq_stream_read over each copy's device index layouts"
                                          + (", signs and scales" if residual else ""))

        if not residual:
            context = {"dense_fp16_gemv": dense_context_subprocess(args)}

    # ---- plain copy of known size: the reference reading of the HBM byte counters
    if args.copy_probe:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        say("# copy probe: 5 x 256 MiB device copies")

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
        say(f"# cpu oracle: {med * 1e3:.1f} ms/layer over {len(reps)} runs")

    traffic, traffic_src = committed_traffic(args.workload, args.call)
    if f16_out:
        traffic, traffic_src = None, None   # the counters were taken with fp32 outputs
    roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic, "kernel_us": round(us_per_layer, 4),
            "launches_per_call": 2 if wl.nbits == 16 else 1,
            "algorithmic_bytes_per_launch": layer_bytes,
            "traffic_source": traffic_src,
            "kernel_source_sha": kernel_source_sha(args.workload, args.call)}
    if read_gbs is not None:
        roof["stream_read_gbs"] = round(read_gbs, 2)
        roof["frac_of_stream_read"] = round(gbs / read_gbs, 4)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": us_per_layer / 1e3,
        "us_per_layer": round(us_per_layer, 4),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if f16_out else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "matrices": wl.count,
                   "K_N": [[s.K, s.N] for s in wl.matrices], "d": wl.d, "nbits": wl.nbits,
                   "B": wl.B, "weight_bytes_per_layer": layer_bytes, "layer_copies": copies,
                   "distinct_codebooks_per_copy": True, "launch": launch,
                   "call": "vq_gemv_oc" if oc else "default",
                   "operands": "f16", "accumulate": "f32", "y": "f16" if f16_out else "f32"},
        "timing": timing,
        "roofline": roof,
        "context": context,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
