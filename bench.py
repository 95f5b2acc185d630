"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill of the 8K workload (B=1, H=32, T=8192,
d=128, bf16 inputs, fp32 state; P0-P4) followed by one decode step of the
decode workload (256 sequences x 32 heads, 128x128 fp32 states, bf16 token
inputs; D1-D4).  Inputs are synthetic, seeded, and resident in HBM before
timing starts.

Prints one JSON line:
  value        prefill tokens/s of the 8K workload (8192 tokens x 32 heads per
               call) from HIP events around each prefill call
  ms_per_step  wall time of one whole step (prefill + decode step)
  decode       decode state GB/s and tokens/s from HIP events around each step
  roofline     the dominant call (largest share of the step) against its bound
  cpu_baseline the fp64 oracle on the host cores, same prefill workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA


def prefill_algorithmic(T, H, d, n_seqs, init, final):
    """Bytes and MFMA FLOPs of one prefill call: q, k, v (bf16), log_alpha
    (fp32), beta (bf16) read, o (bf16) written per token-head; states fp32."""
    per_tok = 3 * d * 2 + d * 4 + 2 + d * 2
    state = d * d * 4 * n_seqs * H * ((1 if init else 0) + (1 if final else 0))
    flops_per_tok = 2 * (5 * 64 * d + 3 * d * d)
    return T * H * per_tok + state, T * H * flops_per_tok


def decode_algorithmic(N, H, d):
    """Bytes of one decode step: state read + write (fp32), q, k, v, o (bf16),
    log_alpha (fp32), beta (bf16)."""
    return N * H * (2 * d * d * 4 + 4 * d * 2 + d * 4 + 2)


def cpu_baseline(prefill_inputs, seconds_hint=""):
    import oracle
    import torch
    d = prefill_inputs
    host = {k: d[k].cpu() for k in ("q", "k", "v", "log_alpha", "beta")}
    cu = d["cu_seqlens"].cpu().long()
    threads = oracle.default_threads()
    t = time.perf_counter()
    oracle.prefill(host["q"], host["k"], host["v"], host["log_alpha"], host["beta"], cu, None,
                   nthreads=threads, want_final=True)
    dt = time.perf_counter() - t
    T = host["q"].shape[0]
    return {"value": T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 8K prefill workload (T={T}, H={host['q'].shape[1]}, "
                      f"d={host['q'].shape[2]}), fp64 token recurrence, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the operator shards by (sequence, head) with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_88_amd import inputs, kda

    dev = "cuda:0"
    torch.cuda.set_device(0)
    kda.load()
    wl = inputs.WORKLOADS["prefill_8k"]
    P = inputs.prefill_inputs(wl, device=dev)
    T, H, D = P["q"].shape
    o = torch.empty((T, H, D), device=dev, dtype=torch.bfloat16)
    fin = torch.empty((1, H, D, D), device=dev, dtype=torch.float32)
    ws = torch.empty(kda.workspace_size(1, T, H, D, D, torch.bfloat16), device=dev, dtype=torch.uint8)

    dwl = inputs.WORKLOADS["decode_256"]
    n_dec = 64
    Dd = inputs.decode_inputs(dwl, device=dev, steps=n_dec)
    state = Dd["state"]
    od = torch.empty((dwl.num_seqs, dwl.heads, dwl.dv), device=dev, dtype=torch.bfloat16)

    def prefill():
        kda.kda_prefill_varlen(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], P["cu_seqlens"],
                               None, o=o, final_state=fin, workspace=ws)

    def decode(s):
        s %= n_dec
        kda.kda_decode_step(Dd["q"][s], Dd["k"][s], Dd["v"][s], Dd["log_alpha"][s], Dd["beta"][s],
                            state, o=od)

    for s in range(args.warmup):
        prefill()
        decode(s)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record()
        prefill()
        ev[s][1].record()
        decode(args.warmup + s)
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K

    pbytes, pflops = prefill_algorithmic(T, H, D, 1, False, True)
    dbytes = decode_algorithmic(dwl.num_seqs, dwl.heads, dwl.dv)
    pre_gbps = pbytes / (pre_avg * 1e-3) / 1e9
    dec_gbps = dbytes / (dec_avg * 1e-3) / 1e9
    roof_pre = {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(pre_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                "call": "kda_prefill_varlen (prep + state-pass kernels)",
                "mfma_tflops": round(pflops / (pre_avg * 1e-3) / 1e12, 2),
                "mfma_frac": round(pflops / (pre_avg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    roof_dec = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                "call": "kda_decode_step (decode_step_kernel)"}
    dominant = roof_dec if dec_avg > pre_avg else roof_pre

    out = {
        "metric": "KDA prefill tokens/s (H=32,d=128) + decode state GB/s vs HBM peak, 1 GPU",
        "value": round(T / (pre_avg * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised, log_alpha=-exp(U(-5,0)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "prefill_8k + decode_256",
                   "prefill": {"B": 1, "H": H, "T": T, "dk": D, "dv": D, "chunk": 64,
                               "init_state": None, "final_state": True},
                   "decode": {"sequences": dwl.num_seqs, "H": dwl.heads, "dk": dwl.dk,
                              "dv": dwl.dv, "state_MB": round(dwl.num_seqs * dwl.heads * dwl.dk * dwl.dv * 4 / 1e6, 1)}},
        "prefill": {"ms": round(pre_avg, 5), "ms_min": round(min(pre_ms), 5),
                    "tokens_per_s": round(T / (pre_avg * 1e-3), 1), "roofline": roof_pre},
        "decode": {"ms": round(dec_avg, 5), "ms_min": round(min(dec_ms), 5),
                   "value": round(dec_gbps, 1), "unit": "GB/s",
                   "tokens_per_s": round(dwl.num_seqs / (dec_avg * 1e-3), 1), "roofline": roof_dec},
        "roofline": dominant,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(P)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
