"""GPU parity of the raw-input calls (kda_prefill_varlen_raw,
kda_decode_step_raw: q, k made unit length and beta = sigmoid(logit) inside
the kernels) against the fp64 oracle applying the same prologue."""
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, row_rel_err, state_rel_err
from tests.test_gpu_prefill import make_case, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def rawify(d, seed):
    """Scale every q and k vector by a random factor and give beta as a logit,
    rounded to the input dtype."""
    g = torch.Generator().manual_seed(seed)
    e = dict(d)
    dt = d["q"].dtype
    shp = d["q"].shape[:-1] + (1,)
    e["q"] = (d["q"].float() * torch.empty(shp).uniform_(0.1, 8.0, generator=g)).to(dt)
    e["k"] = (d["k"].float() * torch.empty(shp).uniform_(0.1, 8.0, generator=g)).to(dt)
    b = d["beta"].float().clamp(1e-4, 1 - 1e-4)
    e["beta"] = torch.log(b / (1 - b)).to(dt)
    return e


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64), (torch.bfloat16, 64)],
                         ids=["bf16-128", "f32-64", "bf16-64"])
def test_raw_prefill_ragged(dtype, D):
    d = rawify(make_case([1, 63, 64, 65, 0, 200, 129], H=3, D=D, dtype=dtype, seed=310 + D), seed=3)
    g = to_dev(d)
    o, f = kda.kda_prefill_varlen_raw(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                                      g["init_state"])
    torch.cuda.synchronize()
    ro, rf = oracle.prefill_raw(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(),
                                d["init_state"])
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    print(f"raw prefill {dtype} D={D}: o {eo:.3e} state {es:.3e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16-128", "f32-64"])
def test_raw_decode_steps(dtype, D):
    wl = inputs.WORKLOADS["decode_256"].replace(num_seqs=5, heads=3, dk=D, dv=D,
                                                dtype="f32" if dtype == torch.float32 else "bf16", seed=330)
    d = inputs.decode_inputs(wl, steps=4)
    state = d["state"].to(DEV)
    ref = d["state"].double().numpy()
    for s in range(4):
        step = rawify({k: d[k][s] for k in ("q", "k", "v", "log_alpha", "beta")}, seed=40 + s)
        args = [step[k] for k in ("q", "k", "v", "log_alpha", "beta")]
        o = kda.kda_decode_step_raw(*[a.to(DEV) for a in args], state)
        torch.cuda.synchronize()
        ro, ref = oracle.decode_step_raw(*args, ref)
        eo, es = row_rel_err(o, ro), state_rel_err(state, ref)
        print(f"raw decode {dtype} D={D} step {s}: o {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= TOL[dtype] and es <= TOL[dtype]
