"""GPU parity of the Gated DeltaNet calls (one gate per token and head:
kda_gdn_prefill_varlen, kda_gdn_decode_step) against the fp64 oracle."""
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, row_rel_err, state_rel_err
from tests.test_gpu_prefill import make_case, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def scalar_gate(d):
    """The same inputs with one gate per (token, head): the first channel's."""
    e = dict(d)
    e["log_alpha"] = d["log_alpha"][..., 0].contiguous()
    return e


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64), (torch.bfloat16, 64)],
                         ids=["bf16-128", "f32-64", "bf16-64"])
def test_gdn_prefill_ragged(dtype, D):
    d = scalar_gate(make_case([1, 63, 64, 65, 0, 200, 129], H=3, D=D, dtype=dtype, seed=210 + D))
    g = to_dev(d)
    o, f = kda.gdn_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                                  g["init_state"])
    torch.cuda.synchronize()
    ro, rf = oracle.prefill_scalar_gate(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                        d["cu_seqlens"].long(), d["init_state"])
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    print(f"gdn prefill {dtype} D={D}: o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_gdn_equals_kda_with_repeated_gate_bitwise():
    """the scalar-gate path computes exactly what the channel-gate path does
    when every channel carries the same gate"""
    d = scalar_gate(make_case([130, 257], H=2, D=128, dtype=torch.bfloat16, seed=221))
    g = to_dev(d)
    o1, f1 = kda.gdn_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                                    g["init_state"])
    la_rep = g["log_alpha"][..., None].expand(-1, -1, 128).contiguous()
    o2, f2 = kda.kda_prefill_varlen(g["q"], g["k"], g["v"], la_rep, g["beta"], g["cu_seqlens"],
                                    g["init_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16-128", "f32-64"])
def test_gdn_decode_steps(dtype, D):
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=5, heads=3, dk=D, dv=D,
                                                dtype="f32" if dtype == torch.float32 else "bf16", seed=230)
    d = inputs.decode_inputs(wl, steps=5)
    state = d["state"].to(DEV)
    ref = d["state"].double().numpy()
    for s in range(5):
        args = [d[k][s] for k in ("q", "k", "v", "log_alpha", "beta")]
        args[3] = args[3][..., 0].contiguous()
        o = kda.gdn_decode_step(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        ro, ref = oracle.decode_step_scalar_gate(*args, ref)
        eo, es = row_rel_err(o, ro), state_rel_err(state, ref)
        print(f"gdn decode {dtype} D={D} step {s}: o {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_gdn_prefill_8k_full():
    """the 8K prefill shape with one gate per token and head"""
    wl = inputs.WORKLOADS["prefill_8k"]
    d = scalar_gate(inputs.prefill_inputs(wl))
    g = to_dev(d)
    o, f = kda.gdn_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"], None)
    torch.cuda.synchronize()
    ro, rf = oracle.prefill_scalar_gate(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                        d["cu_seqlens"].long(), None)
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    print(f"gdn prefill_8k: o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
