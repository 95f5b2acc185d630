"""Host-only checks of the C ABI: the library loads, exports what
include/kda.h declares, sizes workspaces, and rejects bad arguments before
any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_88_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH),
                                reason="libkda.so not built (python -m gated_delta_rule_88_amd.build)")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, DTYPE = 0, 1, 2, 3, 4, 5, 6
BF16, F32 = kda.KDA_BF16, kda.KDA_F32


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(kda_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"kda_prefill_varlen", "kda_decode_step", "kda_prefill_workspace_size",
                          "kda_status_string", "kda_version"}
    for name in names:
        assert hasattr(lib, name), f"libkda.so does not export {name}"


def test_status_strings_and_version(lib):
    for s in range(0, 8):
        assert kda.status_string(s)
    assert kda.status_string(99) == "unknown status"
    assert kda.version() >= 100


def test_workspace_size(lib):
    f = lib.kda_prefill_workspace_size
    # bf16: one record per (chunk slot, head) -- W, Q', Kc^T, U, Bqk U (fp16)
    # and e^G (fp32) -- then one int32 chunk-ready flag per (slot, head)
    # (padded to 256 bytes) and a 256-byte header
    rec_bf16_128 = 3 * 16384 + 2 * 16384 + 128 * 4
    items = (8192 // 64 + 1 + 1) * 32
    assert f(1, 8192, 32, 128, 128, BF16) == items * rec_bf16_128 + (items * 4 + 255) // 256 * 256 + 256
    assert f(1, 256, 1, 64, 64, F32) > 0
    assert f(0, 0, 1, 128, 128, BF16) > 0            # one spare slot per head
    assert f(1, 100, 2, 96, 96, BF16) == 0            # unsupported head size
    assert f(1, 100, 2, 128, 64, BF16) == 0           # dk != dv
    assert f(1, 100, 0, 128, 128, BF16) == 0
    assert f(1, 100, 2, 128, 128, 7) == 0
    assert f(1, -1, 2, 128, 128, BF16) == 0


P = ctypes.c_void_p(0x10000)     # aligned fake device pointer (never dereferenced)
MIS = ctypes.c_void_p(0x10008)   # 8-byte aligned only


def prefill(lib, **over):
    args = dict(q=P, k=P, v=P, la=P, beta=P, cu=P, init=None, o=P, fin=P, N=1, T=128, H=2,
                dk=128, dv=128, dtype=BF16, ws=P, wsb=1 << 40, stream=None)
    args.update(over)
    return lib.kda_prefill_varlen(args["q"], args["k"], args["v"], args["la"], args["beta"],
                                  args["cu"], args["init"], args["o"], args["fin"], args["N"],
                                  args["T"], args["H"], args["dk"], args["dv"], args["dtype"],
                                  args["ws"], args["wsb"], args["stream"])


def decode(lib, **over):
    args = dict(q=P, k=P, v=P, la=P, beta=P, state=P, o=P, N=4, H=2, dk=128, dv=128, dtype=BF16,
                stream=None)
    args.update(over)
    return lib.kda_decode_step(args["q"], args["k"], args["v"], args["la"], args["beta"],
                               args["state"], args["o"], args["N"], args["H"], args["dk"],
                               args["dv"], args["dtype"], args["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(la=None), NULL),
    (dict(beta=None), NULL), (dict(cu=None), NULL), (dict(o=None), NULL),
    (dict(N=0), SHAPE), (dict(N=-1), SHAPE), (dict(T=-5), SHAPE), (dict(H=0), SHAPE),
    (dict(T=1 << 31), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(dk=128, dv=64), UNSUP), (dict(dk=256, dv=256), UNSUP),
    (dict(dtype=5), DTYPE),
    (dict(q=MIS), ALIGN), (dict(beta=MIS), ALIGN), (dict(init=MIS), ALIGN), (dict(ws=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=1024), WS),
])
def test_prefill_rejects(lib, over, expect):
    assert prefill(lib, **over) == expect


@pytest.mark.parametrize("over,expect", [
    (dict(q=None), NULL), (dict(state=None), NULL), (dict(o=None), NULL), (dict(beta=None), NULL),
    (dict(N=-1), SHAPE), (dict(H=0), SHAPE), (dict(dk=32, dv=32), UNSUP), (dict(dk=64, dv=128), UNSUP),
    (dict(dtype=2), DTYPE), (dict(state=MIS), ALIGN), (dict(la=MIS), ALIGN),
])
def test_decode_rejects(lib, over, expect):
    assert decode(lib, **over) == expect


def test_decode_zero_sequences_is_a_no_op(lib):
    # nothing to launch: returns before touching HIP
    assert decode(lib, N=0, q=None, state=None) == OK


def prefill_pooled(lib, **over):
    args = dict(q=P, k=P, v=P, la=P, beta=P, cu=P, idx=P, pool=P, slots=4, read=1, o=P, N=1, T=128,
                H=2, dk=128, dv=128, dtype=BF16, ws=P, wsb=1 << 40, stream=None)
    args.update(over)
    return lib.kda_prefill_varlen_pooled(args["q"], args["k"], args["v"], args["la"], args["beta"],
                                         args["cu"], args["idx"], args["pool"], args["slots"],
                                         args["read"], args["o"], args["N"], args["T"], args["H"],
                                         args["dk"], args["dv"], args["dtype"], args["ws"],
                                         args["wsb"], args["stream"])


def decode_pooled(lib, **over):
    args = dict(q=P, k=P, v=P, la=P, beta=P, idx=P, pool=P, slots=8, o=P, N=4, H=2, dk=128, dv=128,
                dtype=BF16, stream=None)
    args.update(over)
    return lib.kda_decode_step_pooled(args["q"], args["k"], args["v"], args["la"], args["beta"],
                                      args["idx"], args["pool"], args["slots"], args["o"], args["N"],
                                      args["H"], args["dk"], args["dv"], args["dtype"], args["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(idx=None), NULL), (dict(pool=None), NULL), (dict(cu=None), NULL), (dict(q=None), NULL),
    (dict(slots=-1), SHAPE), (dict(N=0), SHAPE), (dict(dk=96, dv=96), UNSUP), (dict(dtype=3), DTYPE),
    (dict(idx=MIS), ALIGN), (dict(pool=MIS), ALIGN), (dict(ws=None), WS),
])
def test_prefill_pooled_rejects(lib, over, expect):
    assert prefill_pooled(lib, **over) == expect


@pytest.mark.parametrize("over,expect", [
    (dict(idx=None), NULL), (dict(pool=None), NULL), (dict(o=None), NULL), (dict(slots=-2), SHAPE),
    (dict(N=-1), SHAPE), (dict(dk=64, dv=128), UNSUP), (dict(dtype=9), DTYPE), (dict(idx=MIS), ALIGN),
    (dict(pool=MIS), ALIGN),
])
def test_decode_pooled_rejects(lib, over, expect):
    assert decode_pooled(lib, **over) == expect


def test_decode_pooled_zero_sequences_is_a_no_op(lib):
    assert decode_pooled(lib, N=0, q=None, idx=None, pool=None) == OK


def test_backward_workspace_size(lib):
    f = lib.kda_prefill_backward_workspace_size
    # a window of per-(chunk slot, head) blocks -- 22 fp32 [64 x d] matrices, 9
    # fp32 [64 x 64], the dS_end block [d x d] and the beta, diag(dBq), e^gC
    # vectors -- of at most 512 slots and 8 GiB; then the state entering every
    # chunk slot [d x d] and one [d x d] carry per (sequence, head)
    block_128 = 4 * (22 * 64 * 128 + 9 * 64 * 64 + 128 * 128 + 2 * 64 + 128)
    state = 4 * 128 * 128

    def expect(n, t, h):
        slots = t // 64 + n + 1
        win = max(1, min(slots, 512, (8 << 30) // (h * block_128)))
        return win * h * block_128 + slots * h * state + n * h * state

    assert f(1, 8192, 32, 128, 128, BF16) == expect(1, 8192, 32) == 130 * 32 * (block_128 + state) + 32 * state
    # the variable-length and long-context workloads fit a 288 GB device, at
    # most 0.25 MB per (chunk slot, head)
    for n, t, h in ((16, 270810, 32), (1, 1 << 20, 16)):
        size = f(n, t, h, 128, 128, BF16)
        assert size == expect(n, t, h)
        assert size / ((t // 64 + n + 1) * h) <= 0.25e6
    assert f(1, 256, 1, 64, 64, F32) > 0
    assert f(1, 256, 1, 64, 64, F32) > 0
    assert f(1, 100, 2, 96, 96, BF16) == 0
    assert f(1, 100, 2, 128, 128, 7) == 0
    assert f(1, -1, 2, 128, 128, BF16) == 0


def backward(lib, **over):
    args = dict(q=P, k=P, v=P, la=P, beta=P, cu=P, init=None, go=P, gfin=None, gq=P, gk=P, gv=P, gla=P,
                gbeta=P, ginit=None, N=1, T=128, H=2, dk=128, dv=128, dtype=BF16, ws=P, wsb=1 << 40,
                stream=None)
    args.update(over)
    return lib.kda_prefill_backward(args["q"], args["k"], args["v"], args["la"], args["beta"], args["cu"],
                                    args["init"], args["go"], args["gfin"], args["gq"], args["gk"], args["gv"],
                                    args["gla"], args["gbeta"], args["ginit"], args["N"], args["T"], args["H"],
                                    args["dk"], args["dv"], args["dtype"], args["ws"], args["wsb"],
                                    args["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(q=None), NULL), (dict(go=None), NULL), (dict(gq=None), NULL), (dict(gk=None), NULL),
    (dict(gv=None), NULL), (dict(gla=None), NULL), (dict(gbeta=None), NULL), (dict(cu=None), NULL),
    (dict(N=0), SHAPE), (dict(T=-1), SHAPE), (dict(T=1 << 31), SHAPE), (dict(H=0), SHAPE),
    (dict(dk=96, dv=96), UNSUP), (dict(dk=128, dv=64), UNSUP), (dict(dtype=4), DTYPE),
    (dict(go=MIS), ALIGN), (dict(gfin=MIS), ALIGN), (dict(ginit=MIS), ALIGN), (dict(gbeta=MIS), ALIGN),
    (dict(ws=None), WS), (dict(wsb=4096), WS),
])
def test_backward_rejects(lib, over, expect):
    assert backward(lib, **over) == expect


def test_noalloc_prefill_rejects_before_any_hip_call(lib):
    """kda_prefill_varlen_noalloc: argument checks, and sizes whose workspace
    exceeds the library's scratch array, return before any HIP call"""
    f = lib.kda_prefill_varlen_noalloc
    p = ctypes.c_void_p(0x10000)   # aligned, never dereferenced
    T, H = 16384, 32
    big = lib.kda_prefill_workspace_size(1, T, H, 128, 128, BF16)
    assert big > (384 << 20)
    assert f(p, p, p, p, p, p, None, p, None, 1, T, H, 128, 128, BF16, None) == 8   # KDA_ERR_SCRATCH
    assert f(p, p, p, p, p, None, None, p, None, 1, T, H, 128, 128, BF16, None) == NULL
    assert f(p, p, p, p, p, ctypes.c_void_p(0x10004), None, p, None, 1, T, H, 128, 128, BF16, None) == ALIGN
    assert f(p, p, p, p, p, p, None, p, None, 1, T, H, 96, 96, BF16, None) == UNSUP
    assert kda.status_string(8) == "sizes exceed the no-allocation prefill's scratch array"
