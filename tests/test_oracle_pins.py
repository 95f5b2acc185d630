"""The fp64 oracle against facts fixed outside it (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from tests import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(lib, check):
    check(lib)


def _case(seed, T=50, H=3, dk=16, dv=20):
    rng = np.random.default_rng(seed)
    q, k, v, la, beta = pins._rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    return q, k, v, la, beta, s0


def test_thread_count_does_not_change_bits(lib):
    q, k, v, la, beta, s0 = _case(11)
    cu = [0, 50]
    o1, f1 = oracle.prefill(q, k, v, la, beta, cu, s0, nthreads=1, lib=lib)
    o4, f4 = oracle.prefill(q, k, v, la, beta, cu, s0, nthreads=4, lib=lib)
    assert np.array_equal(o1, o4) and np.array_equal(f1, f4)


def test_bf16_inputs_are_cast_exactly(lib):
    q, k, v, la, beta, s0 = _case(12)
    tb = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    qb, kb, vb, bb = tb(q), tb(k), tb(v), tb(beta)
    la32 = torch.from_numpy(la).to(torch.float32)
    o1, f1 = oracle.prefill(qb, kb, vb, la32, bb, [0, 50], s0, lib=lib)
    o2, f2 = oracle.prefill(qb.double(), kb.double(), vb.double(), la32.double(), bb.double(),
                            [0, 50], s0, lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_out_rows_subset(lib):
    q, k, v, la, beta, s0 = _case(13)
    cu = [0, 20, 20, 50]
    s0 = np.concatenate([s0, s0 * 0.5, s0 * -1.0])
    o, f = oracle.prefill(q, k, v, la, beta, cu, s0, lib=lib)
    rows = [0, 7, 19, 20, 33, 49]
    os_, fs = oracle.prefill(q, k, v, la, beta, cu, s0, out_rows=rows, lib=lib)
    assert np.array_equal(os_, o[rows]) and np.array_equal(fs, f)


def test_decode_step_is_one_token(lib):
    rng = np.random.default_rng(14)
    N, H, dk, dv = 5, 2, 8, 8
    q, k, v, la, beta = pins._rand_inputs(rng, N, H, dk, dv)
    st = rng.standard_normal((N, H, dv, dk))
    o, ns = oracle.decode_step(q, k, v, la, beta, st, lib=lib)
    for n in range(N):
        oi, fi = oracle.prefill(q[n:n + 1], k[n:n + 1], v[n:n + 1], la[n:n + 1], beta[n:n + 1],
                                [0, 1], st[n:n + 1], lib=lib)
        assert np.array_equal(oi[0], o[n]) and np.array_equal(fi[0], ns[n])


def test_rejects_bad_arguments(lib):
    q, k, v, la, beta, s0 = _case(15)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, la, beta, [0, 49], s0, lib=lib)      # cu[-1] != T
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, la, beta, [0, 30, 20, 50], None, lib=lib)  # decreasing
    with pytest.raises(TypeError):
        oracle.prefill(q.astype(np.float32), k, v, la, beta, [0, 50], s0, lib=lib)
