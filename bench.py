"""Benchmark of the KDA hot path on one MI355X.

One step = one chunked prefill of the 8K workload (B=1, H=32, T=8192,
d=128, bf16 inputs, fp32 state; chunk map, decay, UT/WY factors, state pass,
output) followed by one decode step of the decode workload (256 sequences x
32 heads, 128x128 fp32 states, bf16 token inputs).  Inputs are synthetic,
seeded, and resident in HBM before timing starts.

Prints one JSON line:
  value        prefill tokens/s of the 8K workload (8192 tokens x 32 heads per
               call) from HIP events around each prefill call
  ms_per_step  wall time of one whole step (prefill + decode step)
  decode       decode state GB/s and tokens/s from HIP events around each step
  roofline     the call with the larger share of the step, against its bound
  varlen_16, long_1m
               the variable-length (16 sequences, lengths U[512, 32768], random
               initial states) and long-context (one 2^20-token sequence,
               H = 16) prefill workloads: tokens/s and HBM fraction per call
  backward     kda_prefill_backward on the 8K workload (gradients of every
               input for seeded upstream gradients), against the fp32 MFMA peak
  cpu_baseline the fp64 oracle on the host cores: the 8K prefill workload
               (headline), plus per_workload rates of the variable-length,
               long-context and decode workloads (the last two on the value
               columns the parity tests check), with the host's CPU model,
               nproc and usable cores
  ceilings     a measured 1 GiB device-to-device copy, beside the 8 TB/s spec;
               every HBM fraction is also given against it (frac_of_copy)

Other modes:
  --part prefill|decode|backward|copy
                               run one leg only (for profiler runs); "copy"
                               is a plain 1 GiB device copy used to calibrate
                               the memory counters
  --traffic [OUTDIR]           run the rocprofv3 FETCH_SIZE / WRITE_SIZE passes
                               as child processes and write the traffic record
                               to OUTDIR/traffic_record.json and to profiles/
                               (this process touches no GPU)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic_prefill_8k_decode_256.json")
COPY_BYTES = 1 << 30


# the device code of the kernels whose memory counters the traffic record holds
TRAFFIC_SOURCES = ("kda_prefill_bf16.hip", "kda_decode.hip", "kda_backward.hip", "kda_device.h",
                   "kda_prefill_common.h")


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one
    space (string and character literals kept as they are)."""
    out, i, n = [], 0, len(src)
    while i < n:
        ch = src[i]
        if ch in "\"'":
            j = i + 1
            while j < n and src[j] != ch:
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
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def source_digest() -> str:
    """sha256 of the sources of the kernels the traffic record covers, their
    comments and layout left out, to tell whether its counters still apply."""
    h = hashlib.sha256()
    for p in sorted(os.path.join(ROOT, "gated_delta_rule_88_amd", "csrc", f) for f in TRAFFIC_SOURCES):
        with open(p, encoding="utf-8") as fh:
            h.update(os.path.basename(p).encode())
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def prefill_algorithmic(T, H, d, n_seqs, init, final):
    """Bytes and MFMA FLOPs of one prefill call: q, k, v (bf16), log_alpha
    (fp32), beta (bf16) read, o (bf16) written per token-head; states fp32."""
    per_tok = 3 * d * 2 + d * 4 + 2 + d * 2
    state = d * d * 4 * n_seqs * H * ((1 if init else 0) + (1 if final else 0))
    flops_per_tok = 2 * (5 * 64 * d + 3 * d * d)
    return T * H * per_tok + state, T * H * flops_per_tok


def backward_algorithmic(T, H, d, n_seqs, C=64):
    """Bytes and MFMA FLOPs of one backward call on full chunks.  Reads q, k,
    v, grad_o (bf16), log_alpha (fp32), beta (bf16); writes fp32 gradients of
    q, k, v, log_alpha, beta; reads dL/dS_T and writes dL/dS_0 (fp32).  FLOPs
    are the dense products of the chunked form: 28 C^2 d + 16 C d^2 + 4 C^3
    per (chunk, head)."""
    per_tok = 3 * d * 2 + d * 4 + 2 + d * 2 + 4 * d * 4 + 4
    state = 2 * d * d * 4 * n_seqs * H
    flops_chunk = 28 * C * C * d + 16 * C * d * d + 4 * C ** 3
    return T * H * per_tok + state, (T // C) * H * flops_chunk


def gdn_prefill_algorithmic(T, H, d, n_seqs, final):
    """Bytes of one Gated DeltaNet prefill call: as the KDA call but one fp32
    gate per token-head."""
    per_tok = 3 * d * 2 + 4 + 2 + d * 2
    return T * H * per_tok + d * d * 4 * n_seqs * H * (1 if final else 0)


def decode_algorithmic(N, H, d):
    """Bytes of one decode step: state read + write (fp32), q, k, v, o (bf16),
    log_alpha (fp32), beta (bf16)."""
    return N * H * (2 * d * d * 4 + 4 * d * 2 + d * 4 + 2)


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cores": usable}


def _host(X, cols=None):
    h = {k: X[k].cpu() for k in ("q", "k", "log_alpha", "beta")}
    h["v"] = X["v"].cpu() if cols is None else X["v"][..., cols].cpu().contiguous()
    init = X.get("init_state")
    h["init_state"] = None if init is None else (init.cpu() if cols is None else init[:, :, cols, :].cpu())
    h["cu"] = X["cu_seqlens"].cpu().long()
    return h


def _oracle_prefill(h, threads, out_rows=None):
    import oracle
    oracle.prefill(h["q"], h["k"], h["v"], h["log_alpha"], h["beta"], h["cu"], h["init_state"],
                   nthreads=threads, want_final=True, out_rows=out_rows)


def cpu_baseline(prefill_inputs, dev):
    """The fp64 oracle on the host cores: the 8K prefill workload repeated
    for about 5 s (the headline figure), then one pass over each of the other
    workloads -- the variable-length batch whole, the long-context sequence
    and the decode sequence on the 16 value columns their parity tests check
    (columns never mix, so a column slice is exactly 1/8 of the work; the
    whole-workload rate is the slice's divided by 8)."""
    import oracle
    import torch
    from gated_delta_rule_88_amd import inputs
    threads = oracle.default_threads()
    h = _host(prefill_inputs)
    T, H, D = h["q"].shape
    reps, t0 = 0, time.perf_counter()
    while reps < 100 and (reps == 0 or time.perf_counter() - t0 < 5.0):
        _oracle_prefill(h, threads)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    per = {"prefill_8k": {"tokens_per_s": round(T / dt, 1), "s": round(dt, 3), "calls": reps,
                          "sample": "whole workload"}}

    X = inputs.prefill_inputs(inputs.WORKLOADS["varlen_16"], device=dev)
    hv = _host(X)
    del X
    t0 = time.perf_counter()
    _oracle_prefill(hv, threads)
    dt = time.perf_counter() - t0
    Tv = hv["q"].shape[0]
    per["varlen_16"] = {"tokens_per_s": round(Tv / dt, 1), "s": round(dt, 3), "tokens": Tv,
                        "sample": "whole workload (16 sequences, initial and final states)"}
    del hv

    wl = inputs.WORKLOADS["long_1m"]
    X = inputs.prefill_inputs(wl, device=dev)
    hl = _host(X, cols=slice(112, 128))
    del X
    torch.cuda.empty_cache()
    Tl = hl["q"].shape[0]
    import numpy as np
    rows = np.unique(np.concatenate([np.arange(0, Tl, 4096), [Tl - 1]]))
    t0 = time.perf_counter()
    _oracle_prefill(hl, threads, out_rows=rows)
    dt = time.perf_counter() - t0
    per["long_1m"] = {"tokens_per_s_columns_112_127": round(Tl / dt, 1),
                      "tokens_per_s": round(Tl / dt / 8, 1), "s": round(dt, 3),
                      "sample": "all 2^20 tokens, value columns 112..127 (1/8 of the work), outputs kept on "
                                "the strided rows t = 0 mod 4096 and T-1; tokens_per_s = column rate / 8"}
    del hl

    dwl = inputs.WORKLOADS["decode_256"]
    Dd = inputs.decode_inputs(dwl, device=dev, steps=64)
    cols = slice(0, 16)
    hd = {k: Dd[k].cpu() for k in ("q", "k", "log_alpha", "beta")}
    hd["v"] = Dd["v"][..., cols].cpu().contiguous()
    ref = Dd["state"][:, :, cols, :].cpu().double().numpy()
    del Dd
    steps = 512
    t0 = time.perf_counter()
    for s in range(steps):
        j = s % 64
        _, ref = oracle.decode_step(hd["q"][j], hd["k"][j], hd["v"][j], hd["log_alpha"][j], hd["beta"][j], ref,
                                    nthreads=threads)
    dt = time.perf_counter() - t0
    ntok = dwl.num_seqs * steps
    per["decode_256"] = {"tokens_per_s_columns_0_15": round(ntok / dt, 1), "tokens_per_s": round(ntok / dt / 8, 1),
                         "s": round(dt, 3),
                         "sample": "512 consecutive steps of 256 sequences x 32 heads (inputs cycling over 64 "
                                   "resident steps, as on the GPU), value columns 0..15 (1/8 of the work); "
                                   "tokens_per_s = column rate / 8"}
    return {"value": per["prefill_8k"]["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole 8K prefill workload (T={T}, H={H}, d={D}, final state), fp64 token "
                      f"recurrence, {per['prefill_8k']['calls']} calls, {per['prefill_8k']['s']:.3f} s each",
            "host": host_info(), "per_workload": per}


def copy_ceiling(dev, K=10):
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = []
    for _ in range(K):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    ms.sort()
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * COPY_BYTES / (ms[K // 2] * 1e-3) / 1e9, 1)


def stored_traffic():
    """Per-call HBM bytes from the stored counter record, if it matches the
    current sources; else None."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != source_digest():
        return None
    return rec


# ---------------------------------------------------------------------------
# --traffic: counter passes in child processes
# ---------------------------------------------------------------------------
# kernels read from each part's run
PART_KERNELS = {"copy": {"copy": "copyBuffer"},
                "prefill": {"prefill": "fused_kernel", "init": "fused_init_kernel"},
                "decode": {"decode": "decode_step_kernel"},
                "backward": {"bprep": "bwd_prep", "bfwd": "bwd_fwd", "bdstate": "bwd_dstate", "bgrad": "bwd_grad"}}


def _counter_pass(counter, part, outdir):
    name = f"{part}_{counter}"
    cmd = ["rocprofv3", "--pmc", counter, "-d", outdir, "-o", name, "--output-format", "csv",
           "--", sys.executable, os.path.join(ROOT, "bench.py"), "--part", part,
           "--steps", "3", "--warmup", "1", "--no-cpu-baseline"]
    env = dict(os.environ, TMPDIR="/tmp")
    print("+", " ".join(cmd), flush=True)
    subprocess.run(["timeout", "-s", "KILL", "120"] + cmd, check=True, cwd="/tmp", env=env)
    rows = []
    for path in glob.glob(os.path.join(outdir, "**", f"{name}_counter_collection.csv"), recursive=True):
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    out = {}
    for key, pat in PART_KERNELS[part].items():
        vals = [float(r["Counter_Value"]) for r in rows if pat in r["Kernel_Name"]
                and r["Counter_Name"] == counter]
        if vals:
            out[key] = sum(vals) / len(vals)   # KiB per dispatch
    # recorded with the repository root and the output directory as $REPO and
    # $OUT, and the interpreter by name
    shown = [("$OUT" + a[len(outdir):]) if a.startswith(outdir) else
             ("$REPO" + a[len(ROOT):]) if a.startswith(ROOT) else
             "python3" if a == sys.executable else a for a in cmd]
    return out, " ".join(shown)


def run_traffic(outdir):
    """Run the counter passes and write the traffic record."""
    outdir = os.path.abspath(outdir)   # the passes run with /tmp as working directory
    os.makedirs(outdir, exist_ok=True)
    rec = {"source_sha": source_digest(), "unit": "KiB per dispatch", "commands": []}
    for part in ("copy", "prefill", "decode", "backward"):
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            vals, cmd = _counter_pass(counter, part, outdir)
            rec["commands"].append(cmd)
            for k, v in vals.items():
                rec.setdefault(k, {})[counter] = v
    copy_kib = COPY_BYTES / 1024
    rec["copy_factor_fetch"] = copy_kib / rec["copy"]["FETCH_SIZE"]
    rec["copy_factor_write"] = copy_kib / rec["copy"]["WRITE_SIZE"]

    def scaled(k):
        c = rec[k]
        return (c["FETCH_SIZE"] * rec["copy_factor_fetch"] + c["WRITE_SIZE"] * rec["copy_factor_write"]) * 1024

    rec["prefill_call_bytes"] = scaled("prefill") + scaled("init")
    rec["decode_call_bytes"] = scaled("decode")
    rec["backward_call_bytes"] = sum(scaled(k) for k in ("bprep", "bfwd", "bdstate", "bgrad"))
    for path in (os.path.join(outdir, "traffic_record.json"), TRAFFIC_RECORD):
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
    print(json.dumps({k: rec[k] for k in ("prefill_call_bytes", "decode_call_bytes", "backward_call_bytes",
                                          "copy_factor_fetch", "copy_factor_write")}), flush=True)


# ---------------------------------------------------------------------------
def backward_report(ms, T, H, D, traffic):
    bbytes, bflops = backward_algorithmic(T, H, D, 1)
    avg = sum(ms) / len(ms)
    tf = bflops / (avg * 1e-3) / 1e12
    moved = traffic.get("backward_call_bytes") if traffic else None
    return {"ms": round(avg, 5), "ms_min": round(min(ms), 5), "calls": len(ms),
            "tokens_per_s": round(T / (avg * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4),
                         "traffic": round(moved) if moved else None,
                         "traffic_GB_s": round(moved / (avg * 1e-3) / 1e9, 1) if moved else None,
                         "algorithmic_flops": bflops, "algorithmic_bytes": bbytes,
                         "hbm_frac": round(bbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
            "launch": "kda_prefill_backward: bwd_prep, bwd_fwd, bwd_dstate, bwd_grad (fp32 MFMA)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--part", choices=("all", "prefill", "decode", "backward", "copy"), default="all")
    ap.add_argument("--traffic", metavar="OUTDIR", nargs="?", const=os.path.join(ROOT, "profile_out", "traffic"))
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(the operator shards by (sequence, head) with no exchange, see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if args.traffic:
        run_traffic(args.traffic)
        return

    import torch
    from gated_delta_rule_88_amd import inputs, kda

    dev = "cuda:0"
    torch.cuda.set_device(0)
    kda.load()

    if args.part == "copy":
        src = torch.ones(COPY_BYTES // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        return

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

    # the same decode workload through a state pool twice its size, sequences
    # scattered over the slots by a seeded permutation
    pool = torch.zeros((2 * dwl.num_seqs,) + tuple(state.shape[1:]), device=dev, dtype=torch.float32)
    g_perm = torch.Generator().manual_seed(5)
    sidx = torch.randperm(2 * dwl.num_seqs, generator=g_perm)[:dwl.num_seqs].to(torch.int32).to(dev)
    pool[sidx.long()] = state

    def decode_pooled(s):
        s %= n_dec
        kda.kda_decode_step_pooled(Dd["q"][s], Dd["k"][s], Dd["v"][s], Dd["log_alpha"][s], Dd["beta"][s],
                                   sidx, pool, o=od)

    # backward of the same prefill for seeded upstream gradients
    g_up = torch.Generator(device=dev).manual_seed(7)
    grad_o = torch.randn((T, H, D), device=dev, generator=g_up).to(torch.bfloat16)
    grad_fin = torch.randn((1, H, D, D), device=dev, generator=g_up)
    f32 = dict(device=dev, dtype=torch.float32)
    grads = {"q": torch.empty((T, H, D), **f32), "k": torch.empty((T, H, D), **f32),
             "v": torch.empty((T, H, D), **f32), "log_alpha": torch.empty((T, H, D), **f32),
             "beta": torch.empty((T, H), **f32), "init_state": torch.empty((1, H, D, D), **f32)}
    ws_b = None

    def backward():
        nonlocal ws_b
        if ws_b is None:
            ws_b = torch.empty(kda.backward_workspace_size(1, T, H, D, D, torch.bfloat16), device=dev,
                               dtype=torch.uint8)
        kda.kda_prefill_backward(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], P["cu_seqlens"], None,
                                 grad_o, grad_fin, grads=grads, workspace=ws_b)

    if args.part == "backward":
        for s in range(args.warmup + args.steps):
            backward()
        torch.cuda.synchronize()
        return

    if args.part in ("prefill", "decode"):
        for s in range(args.warmup + args.steps):
            prefill() if args.part == "prefill" else decode(s)
        torch.cuda.synchronize()
        return

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

    # Gated DeltaNet prefill (one gate per token and head) on the same shape
    la_scalar = P["log_alpha"][..., 0].contiguous()

    def gdn_prefill():
        kda.gdn_prefill_varlen(P["q"], P["k"], P["v"], la_scalar, P["beta"], P["cu_seqlens"],
                               None, o=o, final_state=fin, workspace=ws)

    for s in range(args.warmup):
        gdn_prefill()
        decode(s)
    evg = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for s in range(K):
        evg[s][0].record()
        gdn_prefill()
        evg[s][1].record()
        decode(args.warmup + s)   # streams the caches between calls, as in the main loop
    torch.cuda.synchronize()
    gdn_ms = [e[0].elapsed_time(e[1]) for e in evg]

    # pooled decode, timed on its own
    for s in range(args.warmup):
        decode_pooled(s)
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for s in range(K):
        evp[s][0].record()
        decode_pooled(args.warmup + s)
        evp[s][1].record()
    torch.cuda.synchronize()
    pool_ms = [e[0].elapsed_time(e[1]) for e in evp]

    # the decode workload as a sequence: 512 consecutive steps timed end to
    # end (inputs cycle through the resident steps), three repeats
    seq_steps, seq_ms = 512, []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(seq_steps):
            decode(s)
        e1.record()
        torch.cuda.synchronize()
        seq_ms.append(e0.elapsed_time(e1) / seq_steps)

    # the other two prefill workloads, each timed on its own after one
    # untimed call; inputs are drawn on the GPU and freed afterwards
    def workload_leg(name, calls):
        wl = inputs.WORKLOADS[name]
        X = inputs.prefill_inputs(wl, device=dev)
        Tw, Hw, Dw = X["q"].shape
        Nw = X["cu_seqlens"].shape[0] - 1
        ow = torch.empty((Tw, Hw, Dw), device=dev, dtype=torch.bfloat16)
        fw = torch.empty((Nw, Hw, Dw, Dw), device=dev, dtype=torch.float32)
        ww = torch.empty(kda.workspace_size(Nw, Tw, Hw, Dw, Dw, torch.bfloat16), device=dev, dtype=torch.uint8)

        def run():
            kda.kda_prefill_varlen(X["q"], X["k"], X["v"], X["log_alpha"], X["beta"], X["cu_seqlens"],
                                   X["init_state"], o=ow, final_state=fw, workspace=ww)

        run()
        evw = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(calls)]
        for e in evw:
            e[0].record()
            run()
            e[1].record()
        torch.cuda.synchronize()
        ms = [e[0].elapsed_time(e[1]) for e in evw]
        avg = sum(ms) / len(ms)
        wbytes, _ = prefill_algorithmic(Tw, Hw, Dw, Nw, X["init_state"] is not None, True)
        rec = {"ms": round(avg, 4), "ms_min": round(min(ms), 4), "calls": calls, "tokens": Tw, "sequences": Nw,
               "heads": Hw, "tokens_per_s": round(Tw / (avg * 1e-3), 1),
               "GB_s": round(wbytes / (avg * 1e-3) / 1e9, 1),
               "frac_hbm": round(wbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": wbytes}
        del X, ow, fw, ww
        torch.cuda.empty_cache()
        return rec

    varlen_rec = workload_leg("varlen_16", 5)
    long_rec = workload_leg("long_1m", 3)

    # backward, timed on its own (fewer repeats: it is the longest call).  Its
    # first calls touch a fresh 4 GB workspace and run slower for a few calls
    # (3.51, 3.45, 3.40, 3.38, 3.35 ms in a kernel trace), so four untimed calls
    # come first
    Kb = max(3, K // 4)
    for _ in range(max(args.warmup, 4)):
        backward()
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(Kb)]
    for s in range(Kb):
        evb[s][0].record()
        backward()
        evb[s][1].record()
    torch.cuda.synchronize()
    bwd_ms = [e[0].elapsed_time(e[1]) for e in evb]
    ws_b = None

    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K

    copy_gbps = copy_ceiling(dev)
    pbytes, pflops = prefill_algorithmic(T, H, D, 1, False, True)
    dbytes = decode_algorithmic(dwl.num_seqs, dwl.heads, dwl.dv)
    pre_gbps = pbytes / (pre_avg * 1e-3) / 1e9
    dec_gbps = dbytes / (dec_avg * 1e-3) / 1e9
    traffic = stored_traffic()
    roof_pre = {"bound": "hbm", "achieved": round(pre_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(pre_gbps / HBM_PEAK_GBPS, 4),
                "traffic": round(traffic["prefill_call_bytes"]) if traffic else None,
                "frac_of_copy": round(pre_gbps / copy_gbps, 4),
                "algorithmic_bytes": pbytes,
                "launch": "kda_prefill_varlen: fused_init_kernel, then fused_kernel (prep blocks and "
                          "state-pass blocks in one grid)",
                "mfma_tflops": round(pflops / (pre_avg * 1e-3) / 1e12, 2),
                "mfma_frac": round(pflops / (pre_avg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)}
    roof_dec = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                "traffic": round(traffic["decode_call_bytes"]) if traffic else None,
                "frac_of_copy": round(dec_gbps / copy_gbps, 4),
                "algorithmic_bytes": dbytes,
                "launch": "kda_decode_step: decode_step_kernel"}
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
                              "dv": dwl.dv,
                              "state_MB": round(dwl.num_seqs * dwl.heads * dwl.dk * dwl.dv * 4 / 1e6, 1)}},
        "prefill": {"ms": round(pre_avg, 5), "ms_min": round(min(pre_ms), 5),
                    "ms_median": round(sorted(pre_ms)[K // 2], 5),
                    "tokens_per_s": round(T / (pre_avg * 1e-3), 1), "roofline": roof_pre},
        "decode": {"ms": round(dec_avg, 5), "ms_min": round(min(dec_ms), 5),
                   "ms_median": round(sorted(dec_ms)[K // 2], 5),
                   "sequence_512": {"ms_per_step": round(min(seq_ms), 5),
                                    "GB_s": round(dbytes / (min(seq_ms) * 1e-3) / 1e9, 1),
                                    "frac_hbm": round(dbytes / (min(seq_ms) * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                                    "frac_of_copy": round(dbytes / (min(seq_ms) * 1e-3) / 1e9 / copy_gbps, 4),
                                    "repeats": 3},
                   "value": round(dec_gbps, 1), "unit": "GB/s",
                   "tokens_per_s": round(dwl.num_seqs / (dec_avg * 1e-3), 1), "roofline": roof_dec},
        "gdn_prefill": {"ms": round(sum(gdn_ms) / K, 5), "ms_min": round(min(gdn_ms), 5),
                        "tokens_per_s": round(T / (sum(gdn_ms) / K * 1e-3), 1),
                        "GB_s": round(gdn_prefill_algorithmic(T, H, D, 1, True) / (sum(gdn_ms) / K * 1e-3) / 1e9, 1),
                        "frac_hbm": round(gdn_prefill_algorithmic(T, H, D, 1, True) / (sum(gdn_ms) / K * 1e-3)
                                          / 1e9 / HBM_PEAK_GBPS, 4),
                        "launch": "kda_gdn_prefill_varlen: as the KDA call, one gate per token-head"},
        "decode_pooled": {"ms": round(sum(pool_ms) / K, 5), "ms_min": round(min(pool_ms), 5),
                          "value": round(dbytes / (sum(pool_ms) / K * 1e-3) / 1e9, 1), "unit": "GB/s",
                          "pool_slots": 2 * dwl.num_seqs,
                          "launch": "kda_decode_step_pooled: decode_step_kernel with a slot map"},
        "varlen_16": varlen_rec,
        "long_1m": long_rec,
        "backward": backward_report(bwd_ms, T, H, D, traffic),
        "roofline": dominant,
        "ceilings": {"hbm_spec_GB_s": HBM_PEAK_GBPS, "copy_1GiB_GB_s": copy_gbps,
                     "note": "copy = read + write bytes of a 1 GiB device-to-device copy, median of 10"},
    }
    for rec in (varlen_rec, long_rec):
        rec["frac_of_copy"] = round(rec["GB_s"] / copy_gbps, 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(P, dev)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
