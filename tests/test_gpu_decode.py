"""GPU parity of kda_decode_step (through the C ABI) against the fp64 oracle."""
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, row_rel_err, state_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_steps(dtype, D):
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=5, heads=3, dk=D, dv=D,
                                                dtype="f32" if dtype == torch.float32 else "bf16")
    d = inputs.decode_inputs(wl, steps=6)
    state = d["state"].to(DEV)
    ref = d["state"].double().numpy()
    for s in range(6):
        args = [d[k][s] for k in ("q", "k", "v", "log_alpha", "beta")]
        o = kda.kda_decode_step(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        ro, ref = oracle.decode_step(*args, ref)
        eo = row_rel_err(o, ro)
        es = state_rel_err(state, ref)
        print(f"decode {dtype} D={D} step {s}: o {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_no_op_is_bitwise():
    """log_alpha = 0 and beta = 0 leave the state bit-identical"""
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=4, heads=2)
    d = inputs.decode_inputs(wl, steps=1)
    state = d["state"].to(DEV)
    before = state.clone()
    args = [d[k][0].to(DEV) for k in ("q", "k", "v", "log_alpha", "beta")]
    args[3].zero_()
    args[4].zero_()
    kda.kda_decode_step(*args, state)
    torch.cuda.synchronize()
    assert torch.equal(state, before)


def test_decode_readback():
    """beta = 1, q := k (unit): the output is v"""
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=8, heads=2, dtype="f32")
    d = inputs.decode_inputs(wl, steps=1)
    state = d["state"].to(DEV)
    q = d["k"][0].to(DEV)
    o = kda.kda_decode_step(q, q.clone(), d["v"][0].to(DEV), d["log_alpha"][0].to(DEV),
                            torch.ones_like(d["beta"][0]).to(DEV), state)
    torch.cuda.synchronize()
    assert row_rel_err(o, d["v"][0]) <= 1e-5


def test_decode_deterministic():
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=16, heads=4)
    d = inputs.decode_inputs(wl, steps=1)
    args = [d[k][0].to(DEV) for k in ("q", "k", "v", "log_alpha", "beta")]
    s1, s2 = d["state"].to(DEV), d["state"].to(DEV)
    o1 = kda.kda_decode_step(*args, s1)
    o2 = kda.kda_decode_step(*args, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
