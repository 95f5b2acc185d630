"""Guard regions and NaN poison around every output buffer: each call writes
all of its outputs (nothing is left holding the poison) and nothing outside
them (the guard words around each buffer keep their sentinel values).  The
outputs are carved out of larger allocations filled with NaN, with a guard
of sentinel values on both sides."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, row_rel_err, state_rel_err
from tests.test_gpu_prefill import make_case, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 256
SENTINEL = 7.0


def guarded(shape, dtype):
    """A NaN-filled view of `shape` inside a buffer with sentinel guards."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), float("nan"), device=DEV, dtype=dtype)
    buf[:GUARD] = SENTINEL
    buf[-GUARD:] = SENTINEL
    return buf, buf[GUARD:GUARD + n].view(shape)


def intact(buf):
    return bool((buf[:GUARD] == SENTINEL).all()) and bool((buf[-GUARD:] == SENTINEL).all())


def all_written(x):
    return bool(torch.isfinite(x.float()).all())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_decode_outputs_guarded(dtype):
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=6, heads=3, dtype="f32" if dtype == torch.float32 else "bf16")
    d = inputs.decode_inputs(wl, steps=2)
    N, H, D = 6, 3, 128
    sbuf, state = guarded((N, H, D, D), torch.float32)
    state.copy_(d["state"].to(DEV))
    ref = d["state"].double().numpy()
    for s in range(2):
        obuf, o = guarded((N, H, D), dtype)
        args = [d[k][s] for k in ("q", "k", "v", "log_alpha", "beta")]
        kda.kda_decode_step(*[a.to(DEV) for a in args], state, o=o)
        torch.cuda.synchronize()
        ro, ref = oracle.decode_step(*args, ref)
        assert all_written(o) and intact(obuf) and intact(sbuf)
        assert row_rel_err(o, ro) <= TOL[dtype] and state_rel_err(state, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_final_state_guarded(dtype):
    lengths = [70, 0, 129]
    d = make_case(lengths, H=2, D=128, dtype=dtype, seed=31)
    g = to_dev(d)
    T, H, D = g["q"].shape
    obuf, o = guarded((T, H, D), dtype)
    fbuf, fin = guarded((3, H, D, D), torch.float32)
    kda.kda_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                           g["init_state"], o=o, final_state=fin)
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(),
                            d["init_state"])
    assert all_written(o) and all_written(fin) and intact(obuf) and intact(fbuf)
    assert torch.equal(fin[1], g["init_state"][1])   # the empty sequence keeps its state
    assert row_rel_err(o, ro) <= TOL[dtype] and state_rel_err(fin, rf) <= TOL[dtype]


def test_pooled_prefill_outputs_guarded():
    """pooled prefill: o fully written; only the named slots of the pool
    change; nothing outside either buffer is touched"""
    lengths = [90, 40]
    d = make_case(lengths, H=2, D=128, dtype=torch.bfloat16, seed=33)
    g = to_dev(d)
    T, H, D = g["q"].shape
    P = 5
    pbuf, pool = guarded((P, H, D, D), torch.float32)
    pool.copy_(0.02 * torch.randn((P, H, D, D), device=DEV))
    before = pool.clone()
    idx = torch.tensor([3, 1], dtype=torch.int32, device=DEV)
    pool[3].copy_(g["init_state"][0])
    pool[1].copy_(g["init_state"][1])
    before = pool.clone()
    obuf, o = guarded((T, H, D), torch.bfloat16)
    kda.kda_prefill_varlen_pooled(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"], idx,
                                  pool, o=o)
    torch.cuda.synchronize()
    ro, rf = oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(),
                            d["init_state"])
    assert all_written(o) and intact(obuf) and intact(pbuf)
    for s in (0, 2, 4):
        assert torch.equal(pool[s], before[s])
    assert row_rel_err(o, ro) <= TOL[torch.bfloat16]
    assert state_rel_err(torch.stack([pool[3], pool[1]]), rf) <= TOL[torch.bfloat16]


def test_pooled_decode_default_output_is_zero_for_skipped_rows():
    """a sequence whose slot index is out of range is skipped on the device;
    the binding's default output buffer shows it as zeros"""
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=3, heads=2)
    d = inputs.decode_inputs(wl, steps=1)
    pool = d["state"].to(DEV).clone()
    idx = torch.tensor([0, 99, 2], dtype=torch.int32, device=DEV)
    args = [d[k][0].to(DEV) for k in ("q", "k", "v", "log_alpha", "beta")]
    o = kda.kda_decode_step_pooled(*args, idx, pool)
    torch.cuda.synchronize()
    assert torch.equal(o[1], torch.zeros_like(o[1]))
    assert all_written(o) and bool((o[0] != 0).any()) and bool((o[2] != 0).any())


@pytest.mark.parametrize("alias", [False, True], ids=["separate", "grad_init_is_grad_final"])
def test_backward_gradients_guarded(alias):
    """every gradient buffer fully written and nothing around it touched;
    grad_init_state may be the grad_final_state buffer itself"""
    lengths = [100, 0, 65]
    d = make_case(lengths, H=2, D=64, dtype=torch.float32, seed=35)
    g = to_dev(d)
    T, H, D = g["q"].shape
    N = len(lengths)
    gen = torch.Generator().manual_seed(36)
    go = torch.randn((T, H, D), generator=gen)
    gf = torch.randn((N, H, D, D), generator=gen)
    bufs, grads = {}, {}
    for name, shape in (("q", (T, H, D)), ("k", (T, H, D)), ("v", (T, H, D)), ("log_alpha", (T, H, D)),
                        ("beta", (T, H))):
        bufs[name], grads[name] = guarded(shape, torch.float32)
    gfbuf, gf_dev = guarded((N, H, D, D), torch.float32)
    gf_dev.copy_(gf.to(DEV))
    if alias:
        grads["init_state"] = gf_dev
    else:
        bufs["init_state"], grads["init_state"] = guarded((N, H, D, D), torch.float32)
    kda.kda_prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"], g["init_state"],
                             go.to(DEV), gf_dev, grads=grads)
    torch.cuda.synchronize()
    ref = oracle.prefill_grad(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(),
                              d["init_state"], go, gf)
    for name in ("q", "k", "v", "log_alpha", "beta", "init_state"):
        assert all_written(grads[name]), name
        assert row_rel_err(grads[name], ref[name]) <= TOL[torch.float32], name
    for name, b in bufs.items():
        assert intact(b), name
    assert intact(gfbuf)
