#!/usr/bin/env python3
"""KDA forward benchmark on one MI355X.

One step = one kda_prefill call over the packed 32k-token workload (8
sequences, lengths uniform on [1024, 8192] from seed 12 -> 32,677 tokens,
H = 32, d_k = d_v = 128, bf16 q/k/v, fp32 gates and state): every stage of
the chunked prefill runs in that one launch.  The decode-step latency (256
sequences x 32 heads, d = 128, fp32 state carried across steps) is timed in
the same run.  Inputs are seeded synthetic data already resident in HBM.

Prints ONE JSON line.  ``value`` is prefill tokens/s; ``roofline`` is the
prefill kernel against HBM bandwidth (algorithmic bytes / measured kernel
time); ``decode`` holds the decode step's microseconds and its own roofline;
``gdn`` the same prefill with one gate per token and head (Gated DeltaNet);
``backward`` the backward pass (kda_prefill_backward) over the same batch
against the fp32 vector ALU peak;
``cpu_baseline`` is the fp64 oracle on a bounded sample of the same
workload, timed on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, _ROOT)

METRIC = "KDA prefill tokens/s (T=32k,H=32,d=128) + decode step µs; % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (published; counts packed fp32 FMA)
# chunk length of the prefill kernel for bf16 inputs at d_k = 128 (32 tokens;
# 16 where a 32-token chunk's LDS tiles exceed the 160 KB of one CU)
CHUNK = 32


def prefill_bytes(T_tot: int, N: int, H: int, dk: int, dv: int, esize: int,
                  scalar_gate: bool = False) -> int:
    """Algorithmic HBM bytes of one prefill: read q, k, v (esize each), log_alpha
    (fp32: d_k values per token-head, one with a scalar gate), beta (fp32),
    write o (esize) per token-head; read S0 and write S_T (fp32) per
    (sequence, head)."""
    per_token_head = esize * (2 * dk + dv) + 4 * (1 if scalar_gate else dk) + 4 + esize * dv
    return per_token_head * T_tot * H + 2 * 4 * dk * dv * N * H


def prefill_flops(T_tot: int, H: int, dk: int, dv: int, C: int = CHUNK) -> int:
    """Useful MFMA flops of the chunk form per token-head, triangles counted at
    half: Gram products beta K~ K^T and Q~ K^T (2 C d_k), U = T R and A_qk U
    (2 C d_v), K~ S, Q~ S and Kbar^T U (6 d_k d_v)."""
    return (2 * C * dk + 2 * C * dv + 6 * dk * dv) * T_tot * H


def decode_bytes(N: int, H: int, dk: int, dv: int, esize: int) -> int:
    """State read + write (fp32) plus q, k, v, log_alpha, beta, o per (sequence, head)."""
    return (8 * dk * dv + esize * (2 * dk + dv) + 4 * dk + 4 + esize * dv) * N * H


def backward_flops(T_tot: int, H: int, dk: int, dv: int) -> int:
    """fp32 flops of the reverse-mode token recurrence per state element and
    token (an FMA counts 2), without recomputation: the forward states
    (decay 1, prediction 2, update 2) and the reverse step (dq 2, G += q do^T 2,
    de 2, dk 4, dS' 2, dlog_alpha 2, G <- Diag(a) dS' 1)."""
    return 20 * dk * dv * T_tot * H


def backward_bytes(T_tot: int, N: int, H: int, dk: int, dv: int, esize: int) -> int:
    """Algorithmic HBM bytes of one backward: read q, k, v, do (esize),
    log_alpha and beta (fp32); write dq, dk, dv, dlog_alpha, dbeta (fp32) per
    token-head; read S0 and dS_T, write dS0 (fp32) per (sequence, head)."""
    per_token_head = esize * (2 * dk + 2 * dv) + 4 * dk + 4 + 4 * (3 * dk + dv) + 4
    return per_token_head * T_tot * H + 3 * 4 * dk * dv * N * H


_CSRC = os.path.join(_ROOT, "gated_delta_rule_60_amd", "csrc")
_PROFILES = os.path.join(_ROOT, "profiles")


def measured_traffic(kernel: str, workload: str, sources):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this kernel and workload, or None when the kernel sources have
    changed since those counters were taken (or no summary exists)."""
    import hashlib
    import re

    path = os.path.join(_PROFILES, f"{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_bytes = re.search(r"traffic bytes per launch: (\d+)", text)
    m_hash = re.search(r"kernel source sha256 \([^)]*\): ([0-9a-f]{64})", text)
    if not (m_bytes and m_hash):
        return None
    h = hashlib.sha256()
    for s in sources:
        with open(os.path.join(_CSRC, s), "rb") as f:
            h.update(f.read())
    return int(m_bytes.group(1)) if h.hexdigest() == m_hash.group(1) else None


def cpu_baseline(x, seconds: float):
    """Time the fp64 oracle on the benchmark workload, a batch of heads at a
    time (all sequences of each head), until ``seconds`` of wall time have
    passed or every head is done; scale to tokens/s over all H heads."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    H = x.H
    per_batch = max(1, min(H, (2 * threads + x.N - 1) // x.N))
    done, t0 = 0, time.perf_counter()
    while done < H:
        heads = list(range(done, min(H, done + per_batch)))
        mask = np.zeros((x.N, H), bool)
        mask[:, heads] = True
        oracle.prefill(x.q, x.k, x.v, x.log_alpha, x.beta, x.S0, x.cu_seqlens, pair_mask=mask,
                       nthreads=threads)
        done += len(heads)
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    value = x.T_tot * done / H / dt
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle, heads 0..{done - 1} of {H} over all {x.N} sequences "
                      f"({x.T_tot * done} token-heads) in {dt:.1f} s on {threads} threads; "
                      f"scaled to all heads",
            "cpu": cpu}


def bench_prefill(kda, torch, x, steps: int, warmup: int, v_split: int, scalar_gate: bool = False):
    """Event-timed launches of kda_prefill (or gdn_prefill with the gate of
    channel 0 per token and head when ``scalar_gate``)."""

    dev = torch.device("cuda:0")
    td = torch.bfloat16 if x.dtype == "bf16" else torch.float32

    def up(a, dt=torch.float32):
        return torch.from_numpy(a).to(dev).to(dt)

    # two resident input sets, alternated, so a step never starts with the
    # previous step's inputs sitting in the 256 MB MALL
    la = x.log_alpha[:, :, 0].copy() if scalar_gate else x.log_alpha
    run = kda.gdn_prefill_t if scalar_gate else kda.prefill
    sets = []
    for rot in range(2):
        d = dict(q=up(x.q, td), k=up(x.k, td), v=up(x.v, td), log_alpha=up(la),
                 beta=up(x.beta), S0=None if x.S0 is None else up(x.S0),
                 cu_seqlens=torch.from_numpy(x.cu_seqlens).to(dev))
        d["o"] = torch.empty((x.T_tot, x.H, x.d_v), dtype=td, device=dev)
        d["S_T"] = torch.empty((x.N, x.H, x.d_k, x.d_v), dtype=torch.float32, device=dev)
        sets.append(d)
    for i in range(warmup):
        run(**sets[i % 2], v_split=v_split)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        run(**sets[i % 2], v_split=v_split)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    return wall, kernel_ms


def bench_backward(kda, torch, x, steps: int, warmup: int):
    """Event-timed kda_prefill_backward launches over the workload, with
    seeded upstream gradients dL/do and dL/dS_T; one workspace reused."""
    from gated_delta_rule_60_amd import inputs

    dev = torch.device("cuda:0")
    td = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    up = lambda a, dt=torch.float32: torch.from_numpy(a).to(dev).to(dt)
    dO, dST = inputs.make_backward_grads(x, seed=12)
    args = (up(x.q, td), up(x.k, td), up(x.v, td), up(x.log_alpha), up(x.beta),
            None if x.S0 is None else up(x.S0), torch.from_numpy(x.cu_seqlens).to(dev), up(dO, td), up(dST))
    ws = kda.kda_prefill_backward_workspace_size(x.N, x.T_tot, x.H, x.d_k, x.d_v, 0 if x.dtype == "bf16" else 1)
    wbuf = torch.empty(ws, dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        kda.prefill_backward(*args, workspace=wbuf)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        kda.prefill_backward(*args, workspace=wbuf)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev], ws


def bench_decode(kda, torch, steps: int, warmup: int, n_inputs: int):
    from gated_delta_rule_60_amd import inputs

    w = inputs.WORKLOADS["decode_n256_h32_d128_bf16_x1000"]
    N, H, dk, dv = w["N"], w["H"], w["d_k"], w["d_v"]
    dev = torch.device("cuda:0")
    S = torch.from_numpy(inputs.decode_initial_state(N, H, dk, dv, seed=w["seed"],
                                                     s0_std=w["s0_std"])).to(dev)
    step_inputs = []
    for s in range(n_inputs):
        si = inputs.decode_step_inputs(N, H, dk, dv, s, seed=w["seed"], dtype=w["dtype"],
                                       log_alpha_range=w["log_alpha_range"])
        step_inputs.append(dict(q=torch.from_numpy(si.q).to(dev).to(torch.bfloat16),
                                k=torch.from_numpy(si.k).to(dev).to(torch.bfloat16),
                                v=torch.from_numpy(si.v).to(dev).to(torch.bfloat16),
                                log_alpha=torch.from_numpy(si.log_alpha).to(dev),
                                beta=torch.from_numpy(si.beta).to(dev)))
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)
    for i in range(warmup):
        kda.decode_step(**step_inputs[i % n_inputs], S=S, o=o)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        kda.decode_step(**step_inputs[(warmup + i) % n_inputs], S=S, o=o)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return dict(N=N, H=H, dk=dk, dv=dv, wall=wall, us=us)


def calib_copy(torch, gib: float, reps: int):
    """A plain device-to-device copy of known size, for scaling HBM counters;
    also reports the copy's own read+write bandwidth (the practical ceiling of
    a streaming kernel that reads and writes the same number of bytes)."""
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    best = min(ms)
    print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n,
                      "reps": reps, "copy_ms_min": best,
                      "copy_GBps_read_plus_write": 8 * n / (best * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_varlen8_32k_h32_d128_bf16")
    ap.add_argument("--v-split", type=int, default=0, help="0 = the library's default shape")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--decode-inputs", type=int, default=16,
                    help="distinct pre-generated decode-step inputs, cycled")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gdn", action="store_true", help="skip the scalar-gate (Gated DeltaNet) prefill line")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass line")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", type=float, default=0.0,
                    help="only run a plain copy of this many GiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the KDA forward path here has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calib_copy > 0:
        calib_copy(torch, args.calib_copy, max(1, args.steps))
        return

    import gated_delta_rule_60_amd as kda
    from gated_delta_rule_60_amd import inputs

    x = inputs.make_workload(args.workload)
    esize = 2 if x.dtype == "bf16" else 4
    split = args.v_split or kda.kda_prefill_default_split(x.N, x.T_tot, x.H, x.d_k, x.d_v,
                                                          0 if x.dtype == "bf16" else 1)
    wall, kms = bench_prefill(kda, torch, x, args.steps, args.warmup, split)
    ms_per_step = wall * 1e3 / args.steps
    k_avg_ms = sum(kms) / len(kms)
    nbytes = prefill_bytes(x.T_tot, x.N, x.H, x.d_k, x.d_v, esize)
    nflops = prefill_flops(x.T_tot, x.H, x.d_k, x.d_v)
    achieved = nbytes / (k_avg_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": x.T_tot * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": x.dtype,
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": args.workload, "sequences": x.N, "T_tot": x.T_tot, "H": x.H,
                   "d_k": x.d_k, "d_v": x.d_v, "chunk": CHUNK, "v_split": split,
                   "lengths": [int(b - a) for a, b in zip(x.cu_seqlens[:-1], x.cu_seqlens[1:])]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("prefill_kernel", args.workload,
                                                 ["kda_prefill.hip", "kda_device.hpp"]),
                     "kernel": "kda::prefill_kernel", "kernel_ms_avg": k_avg_ms,
                     "kernel_ms_min": min(kms), "alg_bytes_per_launch": nbytes},
        "mfma": {"alg_flops_per_launch": nflops,
                 "achieved_tflops": nflops / (k_avg_ms * 1e-3) / 1e12,
                 "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": nflops / (k_avg_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS},
    }
    if not args.no_decode:
        d = bench_decode(kda, torch, args.decode_steps, 10, args.decode_inputs)
        us = d["us"]
        mean_us = sum(us) / len(us)
        med_us = us[len(us) // 2]
        db = decode_bytes(d["N"], d["H"], d["dk"], d["dv"], 2)
        out["decode"] = {
            "workload": "decode_n256_h32_d128_bf16", "steps": len(us),
            "us_per_step_median": med_us, "us_per_step_mean": mean_us, "us_per_step_min": us[0],
            "roofline": {"bound": "hbm", "achieved": db / (mean_us * 1e-6) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": db / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("decode_step_kernel", "decode_n256_h32_d128_bf16",
                                                     ["kda_decode.hip", "kda_device.hpp"]),
                         "kernel": "kda::decode_step_kernel", "alg_bytes_per_launch": db},
        }
    if not args.no_gdn:
        _, gms = bench_prefill(kda, torch, x, args.steps, args.warmup, split, scalar_gate=True)
        g_avg_ms = sum(gms) / len(gms)
        gb = prefill_bytes(x.T_tot, x.N, x.H, x.d_k, x.d_v, esize, scalar_gate=True)
        gwl = args.workload + "_gdn"
        out["gdn"] = {
            "workload": gwl, "what": "gdn_prefill: one gate per token and head (channel 0 of the workload's gates)",
            "tokens_per_s": x.T_tot / (g_avg_ms * 1e-3), "kernel_ms_avg": g_avg_ms, "kernel_ms_min": min(gms),
            "roofline": {"bound": "hbm", "achieved": gb / (g_avg_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gb / (g_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("prefill_kernel", gwl, ["kda_prefill.hip", "kda_device.hpp"]),
                         "kernel": "kda::prefill_kernel (scalar gate)", "alg_bytes_per_launch": gb},
        }
    if not args.no_backward:
        bms, bws = bench_backward(kda, torch, x, args.backward_steps, 1)
        b_avg = sum(bms) / len(bms)
        bfl = backward_flops(x.T_tot, x.H, x.d_k, x.d_v)
        bby = backward_bytes(x.T_tot, x.N, x.H, x.d_k, x.d_v, esize)
        out["backward"] = {
            "workload": args.workload, "what": "kda_prefill_backward: dq, dk, dv, dlog_alpha, dbeta, dS0",
            "tokens_per_s": x.T_tot / (b_avg * 1e-3), "ms_avg": b_avg, "ms_min": min(bms), "launches": len(bms),
            "workspace_bytes": bws,
            "roofline": {"bound": "alu", "achieved": bfl / (b_avg * 1e-3) / 1e12, "peak": FP32_VALU_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": bfl / (b_avg * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                         "traffic": measured_traffic("prefill_backward", args.workload,
                                                     ["kda_backward.hip", "kda_device.hpp"]),
                         "kernel": "kda::bwd_forward_kernel + kda::bwd_kernel (one call)",
                         "alg_flops_per_launch": bfl, "alg_bytes_per_launch": bby,
                         "hbm_frac": bby / (b_avg * 1e-3) / 1e9 / HBM_PEAK_GBS},
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
