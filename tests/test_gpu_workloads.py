"""Parity at the full workload sizes, in the launch configuration the bench
times.  The oracle is fp64 and token-sequential, so the larger workloads are
checked on a subset of value columns (columns of S never mix in the
recurrence, so a column slice of v and of the initial state gives exactly
those columns of the outputs and final states) and, for the 1M-token
sequence, on a strided subset of output rows."""
import time

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, record, row_rel_err, state_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_TOL = TOL[torch.bfloat16]


def _log(msg):
    print(msg, flush=True)


def _prefill_gpu(d):
    o, f = kda.kda_prefill_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                  d["cu_seqlens"], d["init_state"])
    torch.cuda.synchronize()
    return o, f


def _oracle_cols(d, cols, out_rows=None):
    t = time.time()
    init = None if d["init_state"] is None else d["init_state"][:, :, cols, :].cpu()
    ro, rf = oracle.prefill(d["q"].cpu(), d["k"].cpu(), d["v"][..., cols].cpu(),
                            d["log_alpha"].cpu(), d["beta"].cpu(), d["cu_seqlens"].cpu().long(),
                            init, out_rows=out_rows)
    _log(f"  oracle: {time.time() - t:.1f}s")
    return ro, rf


def test_prefill_8k_full():
    """B=1, H=32, T=8192, d=128, bf16: every output and final state"""
    d = inputs.prefill_inputs(inputs.WORKLOADS["prefill_8k"], device=DEV)
    o, f = _prefill_gpu(d)
    ro, rf = _oracle_cols(d, slice(None))
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    _log(f"prefill_8k: o {eo:.3e} state {es:.3e}")
    record("prefill_8k (all outputs and states)", eo, es, BF16_TOL)
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_varlen_16_full():
    """16 packed sequences, lengths U[512, 32768], H=32, random initial states"""
    d = inputs.prefill_inputs(inputs.WORKLOADS["varlen_16"], device=DEV)
    _log(f"varlen_16: lengths {d['lengths']} total {sum(d['lengths'])}")
    o, f = _prefill_gpu(d)
    cols = slice(48, 64)
    ro, rf = _oracle_cols(d, cols)
    eo, es = row_rel_err(o[..., cols], ro), state_rel_err(f[:, :, cols, :], rf)
    _log(f"varlen_16 cols 48..63: o {eo:.3e} state {es:.3e}")
    record("varlen_16 (cols 48..63)", eo, es, BF16_TOL)
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_long_1m_drift():
    """B=1, H=16, T=2^20, long memory: strided output rows and the final state"""
    wl = inputs.WORKLOADS["long_1m"]
    d = inputs.prefill_inputs(wl, device=DEV)
    o, f = _prefill_gpu(d)
    T = wl.seq_len
    rows = np.unique(np.concatenate([np.arange(0, T, 4096), [T - 1]]))
    cols = slice(112, 128)
    osel = o[torch.from_numpy(rows).to(DEV)][..., cols].cpu()
    fsel = f[:, :, cols, :].cpu()
    del o
    ro, rf = _oracle_cols(d, cols, out_rows=rows)
    eo, es = row_rel_err(osel, ro), state_rel_err(fsel, rf)
    _log(f"long_1m cols 112..127, {len(rows)} rows: o {eo:.3e} state {es:.3e}")
    record("long_1m (cols 112..127, strided rows)", eo, es, BF16_TOL)
    assert eo <= BF16_TOL and es <= BF16_TOL


def test_decode_256_all_steps():
    """256 sequences x 32 heads, 512 consecutive steps"""
    wl = inputs.WORKLOADS["decode_256"]
    d = inputs.decode_inputs(wl, device=DEV)
    state = d["state"].clone()
    cols = slice(0, 16)
    ref = d["state"][:, :, cols, :].cpu().double().numpy()
    steps = wl.decode_steps
    outs = torch.empty((steps, wl.num_seqs, wl.heads, wl.dv), device=DEV, dtype=torch.bfloat16)
    for s in range(steps):
        kda.kda_decode_step(d["q"][s], d["k"][s], d["v"][s], d["log_alpha"][s], d["beta"][s],
                            state, o=outs[s])
    torch.cuda.synchronize()
    host = {k: d[k].cpu() for k in ("q", "k", "log_alpha", "beta")}
    vcols = d["v"][..., cols].cpu()
    outs = outs[..., cols].cpu()
    worst = 0.0
    t = time.time()
    for s in range(steps):
        ro, ref = oracle.decode_step(host["q"][s], host["k"][s], vcols[s], host["log_alpha"][s],
                                     host["beta"][s], ref)
        worst = max(worst, row_rel_err(outs[s], ro))
    es = state_rel_err(state[:, :, cols, :], ref)
    _log(f"decode_256 cols 0..15, {steps} steps: o {worst:.3e} state {es:.3e} "
         f"(oracle {time.time() - t:.1f}s)")
    record("decode_256 (cols 0..15, 512 steps)", worst, es, BF16_TOL)
    assert worst <= BF16_TOL and es <= BF16_TOL
