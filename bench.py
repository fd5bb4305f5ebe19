#!/usr/bin/env python3
"""Benchmark: TTT-Linear dual-form forward on one MI355X (and, by flag, the other forms and the backward).

One step = one call of the whole hot path (ttt_linear_fwd: every mini-batch of
every (sequence, head) chain) on inputs already resident in HBM.  Prints one
JSON line (rank 0) with tokens/s, the HBM roofline of the kernel (live HIP
event timing) and the fp64 CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--config l1p3b|l125m|long|mlp]
                    [--generic | --primal | --decode | --ln | --chunks N | --save | --bwd | --train]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import ttt_inputs as ti  # noqa: E402

METRIC = "TTT-Linear fwd tokens/sec at B16 H32 d64 T8192 b16; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # fp32 matrix
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30           # size of the calibration copy (read and written once each)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg: ti.Config, eta_strides):
    """Algorithmic bytes and flops of one forward call (the unavoidable work).

    Bytes: read Q, K, V once (bf16 or fp32), write Z once (fp32), read eta
    (per token: 4 B per token-head; otherwise negligible), read W0, write W_final.
    Flops per token-head: TTT-Linear 6 d^2 + 4 d b (W K, W Q, the b x b scores
    and their product with E, and the rank-b state update).  TTT-MLP per
    mini-batch: seven d x dh x b products (W1 K, W1 Q, W2 A_K, W2^T E, W2 A_Q
    and the two rank-b updates), two b x b x d ones (K^T Q and E L2) and two
    b x b x dh ones (D L1 and A_K^T A_Q), at 2 flops per multiply-add.
    """
    th = cfg.B * cfg.H * cfg.T
    in_sz = 2 if cfg.dtype == "bf16" else 4
    eta_b = 4 * th if eta_strides[2] != 0 else 4 * (cfg.H if eta_strides[1] else 1)
    d, b = cfg.d, cfg.b
    if cfg.is_mlp:
        dh = cfg.dh
        w = cfg.H * d * dh * 4 * 2
        wf = cfg.B * cfg.H * d * dh * 4 * 2
        flops_mb = 7 * 2 * d * dh * b + 2 * 2 * d * b * b + 2 * 2 * dh * b * b
        flops = flops_mb * th // b
    else:
        w = cfg.H * d * d * 4
        wf = cfg.B * cfg.H * d * d * 4
        flops = th * (6 * d * d + 4 * d * b)
    bytes_ = th * d * (3 * in_sz + 4) + eta_b + w + wf
    return bytes_, flops


def algorithmic_bwd(cfg: ti.Config, eta_strides, grad_size: int = 4):
    """Algorithmic bytes and flops of one backward call (ttt_linear_bwd).

    Bytes: read Q, K (input dtype), the saved E (fp32), dZ (grad_size), eta;
    write dQ, dK, dV (grad_size) and deta (fp32, per token); read W_final and
    dW_final, write dW0 (fp32 d x d per chain).
    Flops per token-head: 14 d^2 for the seven d x d x b products of a
    mini-batch (rebuilding the start state, A K, W^T dZ, W^T dE, A^T E and the
    two terms of the adjoint update) plus 10 d b for the five b x b x d ones.
    """
    th = cfg.B * cfg.H * cfg.T
    in_sz = 2 if cfg.dtype == "bf16" else 4
    d, b = cfg.d, cfg.b
    eta_b = 4 * th if eta_strides[2] != 0 else 4 * (cfg.H if eta_strides[1] else 1)
    bytes_ = th * d * (2 * in_sz + 4 + grad_size + 3 * grad_size) + eta_b + 4 * th + 3 * cfg.B * cfg.H * d * d * 4
    flops = th * (14 * d * d + 10 * d * b)
    return bytes_, flops


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        db = json.load(fh)
    from test_sequence_layer_amd.profiling import source_hash

    rec = db.get(f"{kernel}|{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


_HOST_THREADS: list = []


def _host_threads(oracle) -> int:
    """OpenMP threads available to the oracle, read once: a call with threads=1
    lowers what the OpenMP runtime reports from then on."""
    if not _HOST_THREADS:
        _HOST_THREADS.append(oracle.max_threads())
    return _HOST_THREADS[0]


def _oracle_subset(cfg: ti.Config, inp_full, chains):
    return ti.Inputs(cfg, chains, inp_full.q[chains], inp_full.k[chains], inp_full.v[chains],
                     inp_full.w1, inp_full.w2, inp_full.eta_buf, inp_full.eta_strides)


def cpu_baseline(cfg: ti.Config, inp_full, sample_chains: int, ln: bool = False):
    """The fp64 oracle timed on all host threads over a sample of chains, and on one
    thread over a 1/threads share of that sample (about the same wall time)."""
    import oracle

    def run(sub, threads):
        t0 = time.perf_counter()
        if ln:  # the layer-norm forms, with the benchmark's gamma = 1, beta = 0
            n = len(sub.chains)
            one, zero = np.ones((n, cfg.d)), np.zeros((n, cfg.d))
            if cfg.is_mlp:
                oracle.mlp_ln_primal(sub.q, sub.k, sub.v, sub.w_rows(1), sub.w_rows(2), one, zero, sub.eta_rows(),
                                     cfg.b, threads=threads)
            else:
                oracle.linear_ln_primal(sub.q, sub.k, sub.v, sub.w_rows(1), one, zero, sub.eta_rows(), cfg.b,
                                        threads=threads)
        else:
            oracle.run_inputs(sub, threads=threads)
        return time.perf_counter() - t0

    chains = ti.sample_chains(cfg, sample_chains)
    threads = _host_threads(oracle)
    dt = run(_oracle_subset(cfg, inp_full, chains), threads)
    chains1 = chains[:max(1, len(chains) // threads)]
    dt1 = run(_oracle_subset(cfg, inp_full, chains1), 1)
    tok = lambda n: n * cfg.T / cfg.H              # noqa: E731  (token = all H heads of one position)
    return {"value": tok(len(chains)) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(chains)} of {cfg.chains} (sequence, head) chains at full T={cfg.T}, "
                      f"fp64 primal form, {dt:.2f} s wall on {threads} threads",
            "cpu_model": _cpu_model(),
            "one_thread": {"value": tok(len(chains1)) / dt1, "unit": "tokens/s",
                           "sample": f"{len(chains1)} chains at full T={cfg.T}, {dt1:.2f} s wall on 1 thread"}}


def cpu_baseline_bwd(cfg: ti.Config, inp_full, sample_chains: int):
    import oracle

    chains = ti.sample_chains(cfg, sample_chains)
    sub = ti.Inputs(cfg, chains, inp_full.q[chains], inp_full.k[chains], inp_full.v[chains],
                    inp_full.w1, inp_full.w2, inp_full.eta_buf, inp_full.eta_strides)
    dz, dwf = ti.upstream_grads(cfg, chains=chains)
    threads = _host_threads(oracle)
    t0 = time.perf_counter()
    oracle.linear_primal_grads(sub.q, sub.k, sub.v, sub.w_rows(), sub.eta_rows(), cfg.b, dz, dwf, threads=threads)
    dt = time.perf_counter() - t0
    tokens = len(chains) * cfg.T / cfg.H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(chains)} of {cfg.chains} (sequence, head) chains at full T={cfg.T}, "
                      f"fp64 reverse pass of the primal loop, {dt:.2f} s wall on {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock settles only after ~50 back-to-back launches (~30 ms at the
    # 1.3B shape: the first launches run up to 40% slower), so warm up with 100.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="l1p3b", choices=sorted(ti.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-chains", type=int, default=512)
    ap.add_argument("--generic", action="store_true", help="time the portable fp32 kernel instead")
    ap.add_argument("--primal", action="store_true",
                    help="time the primal (token-by-token) form instead of the dual form")
    ap.add_argument("--ln", action="store_true",
                    help="layer norm and residual inside f (gamma = 1, beta = 0)")
    ap.add_argument("--chunks", type=int, default=1,
                    help="split each sequence into this many chunks run in parallel (chunked forward)")
    ap.add_argument("--decode", action="store_true",
                    help="time decoding: one token per call for every sequence, state carried in place")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: capture one mini-batch of one-token calls (b calls) in a HIP graph and "
                         "time its replays (no per-call host overhead)")
    ap.add_argument("--save", action="store_true",
                    help="time the forward for training (also writes E for the backward)")
    ap.add_argument("--bwd", action="store_true", help="time the TTT-Linear backward (ttt_linear_bwd)")
    ap.add_argument("--train", action="store_true",
                    help="time forward-for-training + backward (one training step of the layer)")
    ap.add_argument("--no-measured-peak", action="store_true",
                    help="skip measuring the chip's achievable peak (HBM copy or bf16 MFMA loop) "
                         "that roofline.frac_measured is stated against")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reads 1 GiB, writes 1 GiB) so profiler "
                         "HBM counters can be scaled to bytes")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.graph and not args.decode:
        ap.error("--graph applies to --decode")
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (got --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the (sequence, head) chains are independent, so N GPUs would each run this same kernel on "
              "1/N of them with no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    import test_sequence_layer_amd as ttt

    cfg = ti.CONFIGS[args.config]
    log(f"bench: generating {cfg.name} inputs ...")
    t0 = time.perf_counter()
    inp = ti.generate(cfg)
    t = ti.to_device(inp, "cuda:0")
    log(f"bench: inputs ready in {time.perf_counter() - t0:.1f} s")
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    z = torch.empty((B, H, T, d), dtype=torch.float32, device="cuda:0")
    if cfg.is_mlp:
        f1 = torch.empty((B, H, cfg.dh, d), dtype=torch.float32, device="cuda:0")
        f2 = torch.empty((B, H, d, cfg.dh), dtype=torch.float32, device="cuda:0")
        kname = ttt.mlp_kernel_name(B, H, T, d, cfg.dh, cfg.b, eta_strides=inp.eta_strides)
        if args.ln:
            kname += " (layer norm)"
            gam = torch.ones((H, d), dtype=torch.float32, device="cuda:0")
            bet = torch.zeros((H, d), dtype=torch.float32, device="cuda:0")

            def step():
                ttt.mlp_ln_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], gam, bet, t["eta"], cfg.b, z=z,
                               w1_final=f1, w2_final=f2)
        else:
            def step():
                ttt.mlp_fwd(t["q"], t["k"], t["v"], t["w1"], t["w2"], t["eta"], cfg.b, z=z, w1_final=f1,
                            w2_final=f2)
    elif args.decode:
        # one call = one new token for all B*H sequences (T=1), positions advancing
        kname = ttt.linear_kernel_name(B, H, 1, d, cfg.b, 1 if cfg.dtype == "bf16" else 0, 0, (0, 0, 0),
                                       primal=True)
        w = t["w1"].unsqueeze(0).expand(B, -1, -1, -1).contiguous()
        wb = w.clone()
        zt = torch.empty((B, H, 1, d), dtype=torch.float32, device="cuda:0")
        tok = [(t["q"][:, :, i:i + 1].contiguous(), t["k"][:, :, i:i + 1].contiguous(),
                t["v"][:, :, i:i + 1].contiguous(),
                t["eta"][:, :, i:i + 1].contiguous() if t["eta"].dim() == 3 else t["eta"]) for i in range(64)]
        pos = [0]

        def step():
            q1, k1, v1, e1 = tok[pos[0] % 64]
            ttt.linear_decode(q1, k1, v1, e1, w, wb, pos[0], cfg.b, z=zt)
            pos[0] += 1

        if args.graph:
            # b consecutive one-token calls, positions 0 .. b-1 (one mini-batch),
            # captured once; each replay continues the sequences by b tokens
            def calls():
                for i in range(cfg.b):
                    q1, k1, v1, e1 = tok[i]
                    ttt.linear_decode(q1, k1, v1, e1, w, wb, i, cfg.b, z=zt)

            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                calls()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                calls()
            torch.cuda.synchronize()

            def step():
                graph.replay()
    else:
        wf = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda:0")
        kname = ttt.linear_kernel_name(B, H, T, d, cfg.b, 1 if cfg.dtype == "bf16" else 0, 0,
                                       inp.eta_strides, args.generic, args.primal)

        if args.save or args.bwd or args.train:
            e_sv = torch.empty((B, H, T, d), dtype=torch.float32, device="cuda:0")
            ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, z=z, w_final=wf, e_saved=e_sv)
            gen = torch.Generator(device="cuda:0")
            gen.manual_seed(cfg.seed)
            dz = torch.randn((B, H, T, d), generator=gen, device="cuda:0")
            dwf = torch.randn((B, H, d, d), generator=gen, device="cuda:0")
            gout = (torch.empty_like(dz), torch.empty_like(dz), torch.empty_like(dz),
                    torch.empty((B, H, T), dtype=torch.float32, device="cuda:0"), torch.empty_like(dwf))
            if args.save:
                def step():
                    ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, z=z, w_final=wf,
                                        e_saved=e_sv)
            elif args.bwd:
                kname = ttt.linear_bwd_kernel_name(B, H, T, d, cfg.b, 1 if cfg.dtype == "bf16" else 0, 0,
                                                   inp.eta_strides, args.generic)

                def step():
                    ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e_sv, dz, cfg.b, dw_final=dwf,
                                   generic=args.generic, out=gout)
            else:
                def step():
                    ttt.linear_fwd_save(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, z=z, w_final=wf,
                                        e_saved=e_sv)
                    ttt.linear_bwd(t["q"], t["k"], t["eta"], wf, e_sv, dz, cfg.b, dw_final=dwf, out=gout)
        elif args.ln:
            gam = torch.ones((H, d), dtype=torch.float32, device="cuda:0")
            bet = torch.zeros((H, d), dtype=torch.float32, device="cuda:0")

            def step():
                ttt.linear_ln_fwd(t["q"], t["k"], t["v"], t["w1"], gam, bet, t["eta"], cfg.b, z=z, w_final=wf)
        elif args.chunks > 1:
            kname = "ttt_linear_mfma_d64b16"
            ws = torch.empty(ttt.linear_chunked_workspace_bytes(B, H, T, d, cfg.b, args.chunks),
                             dtype=torch.uint8, device="cuda:0")

            def step():
                ttt.linear_fwd_chunked(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, args.chunks,
                                       workspace=ws, z=z, w_final=wf)
        else:
            def step():
                ttt.linear_fwd(t["q"], t["k"], t["v"], t["w1"], t["eta"], cfg.b, z=z, w_final=wf,
                               generic=args.generic, primal=args.primal)
    log(f"bench: kernel {kname}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps      # one call per step (the chunked form: 3 launches)
    ms_per_step = max(wall * 1e3 / args.steps, kernel_ms)
    tokens = B * ((cfg.b if args.graph else 1) if args.decode else T)
    if args.decode and args.graph:
        kernel_ms /= cfg.b  # per launch: one replay is b decode launches
    value = tokens / (ms_per_step / 1e3)

    bytes_, flops = algorithmic(cfg, inp.eta_strides)
    if args.save:
        bytes_ += B * H * T * d * 4                     # E written
    elif args.bwd:
        bytes_, flops = algorithmic_bwd(cfg, inp.eta_strides)
    elif args.train:
        b2, f2 = algorithmic_bwd(cfg, inp.eta_strides)
        bytes_, flops = bytes_ + B * H * T * d * 4 + b2, flops + f2
    if args.decode:
        # per call: read W and write it; read Wb unless the token starts a mini-batch, write
        # Wb only when it does -- three d x d states on average over b calls -- plus one
        # token of Q/K/V in and Z out
        bytes_ = B * H * (3 * d * d * 4 + d * (3 * (2 if cfg.dtype == "bf16" else 4) + 4))
        flops = B * H * 6 * d * d
    achieved = bytes_ / (kernel_ms / 1e3) / 1e9
    # counters are recorded per (kernel, workload) for the plain forward and the
    # backward; the other modes (saving forward, training step, layer norm,
    # chunked, primal, decode, portable kernel) run other code under related
    # names and have no record of their own
    plain = not (args.save or args.train or args.ln or args.chunks > 1 or args.primal or args.decode or args.generic)
    traffic = measured_traffic(kname, cfg.name) if plain else None
    tflops = flops / (kernel_ms / 1e3) / 1e12
    # the binding roofline: bytes / 8 TB/s vs flops / 2.5 PF/s (bf16 MFMA, which every
    # contraction runs on); TTT-Linear is HBM-bound, TTT-MLP MFMA-bound
    if bytes_ / HBM_PEAK_GBS >= flops / BF16_PEAK_TFLOPS / 1e3:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    roof.update({"algorithmic_bytes": bytes_, "algorithmic_flops": flops, "achieved_gbs": round(achieved, 1),
                 "kernel": kname, "kernel_ms": round(kernel_ms, 4)})
    mfma = {"algorithmic_flops": flops, "achieved_tflops": round(tflops, 2),
            "frac_of_bf16_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "frac_of_fp32_peak": round(tflops / FP32_PEAK_TFLOPS, 4)}
    log(f"bench: {kname}: {kernel_ms:.3f} ms/launch, {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of HBM), "
        f"{tflops:.1f} TFLOP/s algorithmic")

    if not args.no_measured_peak:
        # the chip's achievable peak for the binding resource, measured after the
        # timed region on the same device: the fraction against it sits beside
        # the fraction against the published peak
        from test_sequence_layer_amd import peaks

        if roof["bound"] == "hbm":
            pm = peaks.measure_hbm_copy()
            roof.update({"peak_measured": round(pm, 1), "frac_measured": round(achieved / pm, 4),
                         "peak_measured_by": "2 GiB device copy, 16-byte non-temporal loads/stores"})
        else:
            pm = peaks.measure_mfma_bf16()
            roof.update({"peak_measured": round(pm, 1), "frac_measured": round(tflops / pm, 4),
                         "peak_measured_by": "bf16 v_mfma_f32_16x16x32 issue loop, 8 chains per wave"})
        log(f"bench: measured peak {pm:.1f} {roof['unit']} -> {roof['frac_measured']:.1%} of it")

    if args.decode or args.primal:
        roof["note"] = ("decode: one token per call, latency-bound" if args.decode
                        else "primal (token-by-token) form: the baseline the dual form replaces")
        if args.decode and args.graph:
            roof["note"] += f"; timed as replays of a HIP graph of {cfg.b} one-token calls"

    if args.copy_calibration:
        n = COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline and not args.decode:
        log("bench: timing the fp64 oracle on a sample ...")
        if args.bwd:
            cpu = cpu_baseline_bwd(cfg, inp, args.cpu_sample_chains)
        else:
            cpu = cpu_baseline(cfg, inp, args.cpu_sample_chains, ln=args.ln)
        log(f"bench: cpu baseline {cpu['value']:.3e} tokens/s ({cpu['sample']})")

    eta_desc = {(0, 0, 0): "scalar", (0, 1, 0): "per head"}.get(tuple(inp.eta_strides), "per token")
    model = "TTT-MLP" if cfg.is_mlp else "TTT-Linear"
    form = ("decode (graph)" if args.graph else "decode") if args.decode else (
        "primal" if args.primal else ("generic" if args.generic else ""))
    if args.ln:
        form = "layer-norm"
        roof["note"] = ("f(x) = x + LN(W2 GELU(W1 x))" if cfg.is_mlp else "f(x) = x + LN(W x)") + \
            ": layer norm and residual inside f"
    if args.chunks > 1:
        form = f"chunked({args.chunks})"
        roof["note"] = "chunked forward: chunk maps + scan + parallel chunks (3 launches per call)"
    direction = "fwd"
    if args.save:
        form, direction = "", "fwd (saving E for the backward)"
    if args.bwd:
        form, direction = ("generic " if args.generic else ""), "bwd"
        roof["note"] = "backward: dQ, dK, dV, deta, dW0 from dZ and dW_final, state rebuilt from W_final and E"
    if args.train:
        form, direction = "", "fwd+bwd (training step)"
        roof["note"] = "forward saving E, then backward: two launches per step"
    headline = cfg.name == "l1p3b" and not form and direction == "fwd"
    rec = {
        "metric": METRIC if headline else
        f"{model} {form.strip() + ' ' if form.strip() else ''}{direction} tokens/sec ({cfg.name})",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" and not args.generic else "fp32",
        "data": "synthetic (seeded N(0,1/d) Q/K/V, N(0,0.02^2) weights)",
        "config": {"workload": f"{model} dual-form {direction if direction != 'fwd' else 'forward'} B{B} H{H} d{d}"
                               f"{(' dh' + str(cfg.dh)) if cfg.is_mlp else ''} T{T} b{cfg.b}, "
                               f"{cfg.dtype} Q/K/V, fp32 state and Z, {eta_desc} eta",
                   "B": B, "H": H, "d": d, "T": T, "b": cfg.b, "global_batch": B, "seq_len": T,
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "mfma": mfma,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
