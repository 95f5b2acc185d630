"""GPU parity of kda_prefill_varlen (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_88_amd import inputs, kda
from tests.parity import TOL, record, row_rel_err, state_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)


def make_case(lengths, H, D, dtype, seed, init_std=0.02, u_range=(-5.0, 0.0)):
    """Seeded varlen inputs on the host (same recipe as the workloads)."""
    wl = inputs.KdaWorkload("case", len(lengths), H, D, D, "f32" if dtype == torch.float32 else "bf16",
                            seq_len=1, u_range=u_range, init_std=init_std, seed=seed)
    g = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    q, k, v, la, beta = inputs._token_tensors(wl, (T,), g, "cpu")
    init = init_std * torch.randn((len(lengths), H, D, D), generator=g) if init_std > 0 else None
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths), 0)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, cu_seqlens=cu, init_state=init)


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_gpu(d, **kw):
    g = to_dev(d)
    o, f = kda.kda_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"],
                                  g["cu_seqlens"], g["init_state"], **kw)
    torch.cuda.synchronize()
    return o, f


def run_oracle(d):
    return oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                          d["cu_seqlens"].long(), d["init_state"])


def check(d, tol, label):
    o, f = run_gpu(d)
    ro, rf = run_oracle(d)
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    _log(f"{label}: max row-rel err o {eo:.3e}, state {es:.3e} (tol {tol:g})")
    record(label, eo, es, tol)
    assert eo <= tol and es <= tol, (label, eo, es)
    return o, f


def test_tiny_workload_f32():
    """chunked C = 64 prefill vs the token recurrence: B=1, H=1, T=256, d=64, fp32"""
    d = inputs.prefill_inputs(inputs.WORKLOADS["tiny"])
    check(d, TOL[torch.float32], "tiny f32")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_ragged_varlen(dtype, D):
    # lengths span: partial chunks, exact chunks, empty sequences, several chunks
    lengths = [1, 63, 64, 65, 0, 200, 129]
    d = make_case(lengths, H=3, D=D, dtype=dtype, seed=100 + D)
    check(d, TOL[dtype], f"ragged varlen {dtype} D={D}")


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64), (torch.bfloat16, 64)],
                         ids=["bf16-128", "f32-64", "bf16-64"])
def test_many_short_sequences(dtype, D):
    """257 sequences (more than the CUs, not a multiple of the 8-way block
    interleave) of seeded lengths 0..150 over H = 5 heads: the chunk-slot map
    and the block order of both kernels at scale, and (bf16) the state pass
    with two value tiles per workgroup, chosen when the slices outnumber the
    CUs"""
    lengths = np.random.default_rng(470 + D).integers(0, 151, size=257).tolist()
    lengths[0], lengths[-1] = 0, 64   # an empty first and an exact-chunk last sequence
    d = make_case(lengths, H=5, D=D, dtype=dtype, seed=471 + D)
    check(d, TOL[dtype], f"257 short sequences {dtype} D={D}")


@pytest.mark.parametrize("nseq,H", [(5, 3), (8, 4), (75, 4)], ids=["1-tile", "2-tile", "4-tile"])
def test_state_pass_slice_widths(nseq, H):
    """the bf16 state pass takes slices of 1, 2 or 4 value tiles: the
    narrowest whose tasks are at most a quarter of the blocks the device
    holds at once (15, 32 and 300 (sequence, head) pairs here, on a 256-CU
    device: 120, 128 and 600 tasks -- the last dealt partly from the state
    ticket); every width must match the oracle"""
    lengths = np.random.default_rng(490 + nseq).integers(1, 200, size=nseq).tolist()
    d = make_case(lengths, H=H, D=128, dtype=torch.bfloat16, seed=491 + nseq)
    check(d, TOL[torch.bfloat16], f"state pass slice width, {nseq} x {H} pairs")


@pytest.mark.parametrize("D", [128, 64])
def test_long_sequences_with_bounded_prep_lead(D):
    """two sequences of 70,000 and 66,000 tokens, 2 heads: sequences this long
    (64K tokens or more on average) make the bf16 prep wait whenever it runs
    more than a fixed number of chunks ahead of the state pass of its head;
    outputs and final states on value columns 32..47 (columns of S never mix,
    so the oracle on a column slice of v and of the initial state gives
    exactly those columns)"""
    lengths = [70000, 66000]
    d = make_case(lengths, H=2, D=D, dtype=torch.bfloat16, seed=497 + (D == 64))
    o, f = run_gpu(d)
    cols = slice(32, 48)
    ro, rf = oracle.prefill(d["q"], d["k"], d["v"][..., cols], d["log_alpha"], d["beta"],
                            d["cu_seqlens"].long(), d["init_state"][:, :, cols, :])
    eo, es = row_rel_err(o[..., cols], ro), state_rel_err(f[:, :, cols, :], rf)
    _log(f"long sequences, bounded prep lead, D={D}: o {eo:.3e} state {es:.3e}")
    record(f"two long sequences, bounded prep lead, D={D} (cols 32..47)", eo, es, TOL[torch.bfloat16])
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)], ids=["bf16-128", "f32-64"])
def test_chunk_counts_around_the_loop_unroll(dtype, D):
    """sequences of 11, 12, 13, 24 and 25 chunks (full and partial last
    chunks): every exit point of a chunk loop that runs several chunk steps
    per iteration, with random initial states"""
    lengths = [11 * 64, 12 * 64, 12 * 64 + 1, 13 * 64 - 5, 24 * 64, 25 * 64 + 3]
    d = make_case(lengths, H=2, D=D, dtype=dtype, seed=480 + D)
    check(d, TOL[dtype], f"chunk counts around the unroll {dtype} D={D}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_zero_initial_state_and_no_final(dtype):
    d = make_case([300], H=2, D=128, dtype=dtype, seed=7, init_std=0.0)
    o, _ = run_gpu(d, want_final=False)
    ro, _ = run_oracle(d)
    assert row_rel_err(o, ro) <= TOL[dtype]


def test_strong_decay_edge_of_domain():
    """log_alpha near the documented lower bound (-2.5) everywhere"""
    d = make_case([192, 77], H=2, D=128, dtype=torch.float32, seed=9, u_range=(0.85, 0.916))
    assert float(d["log_alpha"].min()) >= -2.5
    check(d, TOL[torch.float32], "strong decay f32")


@pytest.mark.parametrize("gate", ["kda", "gdn"])
def test_bf16_strong_decay_edge_of_domain(gate):
    """bf16 path at the bottom of the gate range, log_alpha in (-2.5, -2.34)
    everywhere: the anchored decay factors then span e^(+-78), which only the
    bf16 operands of the prep carry (channel gates and, for Gated DeltaNet,
    one gate per token and head)"""
    d = make_case([192, 77, 130], H=2, D=128, dtype=torch.bfloat16, seed=19, u_range=(0.85, 0.916))
    if gate == "gdn":
        d["log_alpha"] = d["log_alpha"][..., 0].contiguous()
    assert float(d["log_alpha"].min()) >= -2.5
    g = to_dev(d)
    fn = kda.gdn_prefill_varlen if gate == "gdn" else kda.kda_prefill_varlen
    o, f = fn(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"], g["init_state"])
    torch.cuda.synchronize()
    ref = oracle.prefill_scalar_gate if gate == "gdn" else oracle.prefill
    ro, rf = ref(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"].long(), d["init_state"])
    eo, es = row_rel_err(o, ro), state_rel_err(f, rf)
    _log(f"strong decay bf16 {gate}: o {eo:.3e} state {es:.3e}")
    record(f"strong decay bf16 {gate}", eo, es, TOL[torch.bfloat16])
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_status_word_reports_gate_range(dtype):
    """a call inside the gate range leaves the status word 0; a run of
    log_alpha = -6 (gate sums far below -87 across a chunk's anchor) sets its
    gate-range bit and nothing else"""
    lengths = [150, 90]
    d = make_case(lengths, H=2, D=128, dtype=dtype, seed=23)
    T, H, D = d["q"].shape
    g = to_dev(d)
    ws = torch.empty(kda.workspace_size(2, T, H, D, D, dtype), device=DEV, dtype=torch.uint8)
    kda.kda_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                           g["init_state"], workspace=ws)
    assert kda.prefill_status(ws, 2, T, H, D, D, dtype) == 0
    la = g["log_alpha"].clone()
    la[10:60] = -6.0   # the first chunk of sequence 0 around its token 31
    kda.kda_prefill_varlen(g["q"], g["k"], g["v"], la, g["beta"], g["cu_seqlens"], g["init_state"],
                           workspace=ws)
    assert kda.prefill_status(ws, 2, T, H, D, D, dtype) == 2
    # and the next in-range call clears it
    kda.kda_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                           g["init_state"], workspace=ws)
    assert kda.prefill_status(ws, 2, T, H, D, D, dtype) == 0


@pytest.mark.parametrize("scale", [2000.0, 7000.0])
def test_bf16_large_values(scale):
    """bf16 path with values scaled up: the sequential pass multiplies fp16
    operands (U, E, S and the read-out terms), so the results hold while
    those stay below the fp16 range (6.5e4); |v| up to 4.3 * scale here"""
    d = make_case([150, 90], H=2, D=128, dtype=torch.bfloat16, seed=25)
    d["v"] = (d["v"].float() * scale).to(torch.bfloat16)
    d["init_state"] = d["init_state"] * scale
    check(d, TOL[torch.bfloat16], f"bf16 values x{scale:g}")


def test_no_write_identity_is_bitwise():
    """alpha == 1 and beta == 0: the final state is the initial state, bit for bit"""
    d = make_case([100, 64], H=2, D=128, dtype=torch.bfloat16, seed=11)
    d["log_alpha"].zero_()
    d["beta"].zero_()
    _, f = run_gpu(d)
    assert torch.equal(f.cpu(), d["init_state"])


def test_readback_q_equals_k():
    """beta = 1 and unit keys: S_t^T k_t = v_t, so q := k reads back v_t"""
    d = make_case([130, 40], H=2, D=128, dtype=torch.float32, seed=12)
    d["q"] = d["k"].clone()
    d["beta"].fill_(1.0)
    o, _ = run_gpu(d)
    err = row_rel_err(o, d["v"])
    _log(f"readback err {err:.3e}")
    assert err <= 1e-4


def test_deterministic_and_packing_invariant():
    lengths = [150, 70, 255]
    d = make_case(lengths, H=2, D=128, dtype=torch.bfloat16, seed=13)
    o1, f1 = run_gpu(d)
    o2, f2 = run_gpu(d)
    assert torch.equal(o1, o2) and torch.equal(f1, f2), "run-to-run bits differ"
    cu = d["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        s = slice(cu[n], cu[n + 1])
        single = {k: d[k][s].clone() for k in ("q", "k", "v", "log_alpha", "beta")}
        single["cu_seqlens"] = torch.tensor([0, lengths[n]], dtype=torch.int32)
        single["init_state"] = d["init_state"][n:n + 1].clone()
        os_, fs = run_gpu(single)
        assert torch.equal(os_, o1[s]) and torch.equal(fs[0], f1[n]), f"packing changed sequence {n}"


def test_prefix_continuation():
    """prefill(x[:T1]) then prefill(x[T1:], S) matches prefill(x) (prefix checkpoint)"""
    d = make_case([320], H=2, D=128, dtype=torch.float32, seed=14)
    ro, rf = run_oracle(d)
    for t1 in (64, 100):
        a = {k: d[k][:t1].clone() for k in ("q", "k", "v", "log_alpha", "beta")}
        b = {k: d[k][t1:].clone() for k in ("q", "k", "v", "log_alpha", "beta")}
        a["cu_seqlens"] = torch.tensor([0, t1], dtype=torch.int32)
        b["cu_seqlens"] = torch.tensor([0, 320 - t1], dtype=torch.int32)
        a["init_state"] = d["init_state"]
        oa, fa = run_gpu(a)
        b["init_state"] = fa.cpu()
        ob, fb = run_gpu(b)
        o = torch.cat([oa, ob])
        assert row_rel_err(o, ro) <= 1e-4 and state_rel_err(fb, rf) <= 1e-4


def test_in_place_continuation_and_guards():
    """final_state may alias init_state; outputs outside the packed rows and
    the workspace tail are untouched; every valid row is written"""
    d = make_case([90, 33], H=2, D=64, dtype=torch.bfloat16, seed=15)
    g = to_dev(d)
    T, H, D = g["q"].shape
    guard = 64
    obuf = torch.full((T * H * D + 2 * guard,), float("nan"), device=DEV, dtype=torch.bfloat16)
    obuf[:guard] = 7.0
    obuf[-guard:] = 7.0
    o = obuf[guard:guard + T * H * D].view(T, H, D)
    need = kda.workspace_size(2, T, H, D, D, torch.bfloat16)
    wbuf = torch.full((need + 4096,), 0x5A, device=DEV, dtype=torch.uint8)
    state = g["init_state"].clone()
    kda.kda_prefill_varlen(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["cu_seqlens"],
                           state, o=o, final_state=state, workspace=wbuf)
    torch.cuda.synchronize()
    ro, rf = run_oracle(d)
    assert torch.isfinite(o.float()).all()
    assert row_rel_err(o, ro) <= TOL[torch.bfloat16]
    assert state_rel_err(state, rf) <= TOL[torch.bfloat16]
    assert (obuf[:guard] == 7.0).all() and (obuf[-guard:] == 7.0).all()
    assert (wbuf[need:] == 0x5A).all()


def test_empty_token_buffer():
    """total_tokens == 0: only final states (= initial states) are produced"""
    init = 0.02 * torch.randn((3, 2, 128, 128), device=DEV)
    z = lambda *s, dt=torch.bfloat16: torch.empty(s, device=DEV, dtype=dt)
    cu = torch.zeros(4, dtype=torch.int32, device=DEV)
    o, f = kda.kda_prefill_varlen(z(0, 2, 128), z(0, 2, 128), z(0, 2, 128),
                                  z(0, 2, 128, dt=torch.float32), z(0, 2), cu, init)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and torch.equal(f, init)


def test_prefill_then_decode_handoff():
    """prefill of a prefix, then decode steps from its final state, matches the
    oracle over the whole sequence"""
    from gated_delta_rule_88_amd.kda import kda_decode_step
    d = make_case([200], H=2, D=128, dtype=torch.float32, seed=16)
    ro, rf = run_oracle(d)
    t1 = 190
    a = {k: d[k][:t1].clone() for k in ("q", "k", "v", "log_alpha", "beta")}
    a["cu_seqlens"] = torch.tensor([0, t1], dtype=torch.int32)
    a["init_state"] = d["init_state"]
    oa, state = run_gpu(a)
    outs = [oa]
    for t in range(t1, 200):
        s = lambda x: x[t:t + 1].to(DEV).contiguous()
        outs.append(kda_decode_step(s(d["q"]), s(d["k"]), s(d["v"]), s(d["log_alpha"]),
                                    s(d["beta"]), state))
    torch.cuda.synchronize()
    assert row_rel_err(torch.cat(outs), ro) <= 1e-4
    assert state_rel_err(state, rf) <= 1e-4


@pytest.mark.parametrize("nseq,H", [(5, 3), (10, 4), (75, 4)], ids=["1-tile", "2-tile", "4-tile"])
def test_state_pass_slice_widths_d64(nseq, H):
    """as above with d = 64 (four value tiles per head): 15, 40 and 300
    (sequence, head) pairs take slices of 1, 2 and 4 value tiles, the wider
    two with the Qg / Bqk record; ragged lengths and random initial states"""
    lengths = np.random.default_rng(530 + nseq).integers(1, 200, size=nseq).tolist()
    d = make_case(lengths, H=H, D=64, dtype=torch.bfloat16, seed=531 + nseq)
    check(d, TOL[torch.bfloat16], f"state pass slice width, d=64, {nseq} x {H} pairs")
