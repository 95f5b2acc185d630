"""kda_prefill_varlen_noalloc (the prefill whose workspace is the library's
own scratch array, for callers that cannot allocate) against
kda_prefill_varlen with a caller-owned workspace: the same kernels, so the
outputs and final states must agree bit for bit, and both must meet the
oracle tolerance.  Two calls in a row share the scratch array, the second
with a smaller input."""
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import kda
from tests.parity import TOL, record, row_rel_err, state_rel_err
from tests.test_gpu_prefill import make_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16-128", "f32-64"])
def test_noalloc_prefill_matches_workspace_call(dtype, D):
    for i, lengths in enumerate(([700, 300, 1000, 65], [90, 33])):   # the second call is smaller
        print(f"noalloc {dtype} D={D} call {i}: lengths {lengths}", flush=True)
        d = make_case(lengths, H=4, D=D, dtype=dtype, seed=600 + 10 * i + D)
        g = to_dev(d)
        args = (g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"], g["init_state"])
        o1, f1 = kda.kda_prefill_varlen(*args)
        o2, f2 = kda.kda_prefill_varlen_noalloc(*args)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(f1, f2), f"call {i}: outputs differ"
        ro, rf = oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(),
                                d["init_state"])
        eo, es = row_rel_err(o2, ro), state_rel_err(f2, rf)
        record(f"no-alloc prefill {dtype} D={D} call {i}", eo, es, TOL[dtype])
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_noalloc_prefill_empty_and_oversize():
    """no tokens: final states = initial states; sizes beyond the scratch
    array: KDA_ERR_SCRATCH, raised before any work is enqueued"""
    init = 0.02 * torch.randn((2, 2, 128, 128), device="cuda")
    z = lambda *s, dt=torch.bfloat16: torch.empty(s, device="cuda", dtype=dt)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    o, f = kda.kda_prefill_varlen_noalloc(z(0, 2, 128), z(0, 2, 128), z(0, 2, 128),
                                          z(0, 2, 128, dt=torch.float32), z(0, 2), cu, init)
    torch.cuda.synchronize()
    assert torch.equal(f, init)
    T, H = 16384, 32   # 258 slots x 32 heads of 80.5 KiB records: beyond 384 MiB
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_prefill_varlen_noalloc(z(T, H, 128), z(T, H, 128), z(T, H, 128), z(T, H, 128, dt=torch.float32),
                                       z(T, H), cu, None)
    assert e.value.status == 8
