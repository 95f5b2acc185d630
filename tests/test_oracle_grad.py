"""The fp64 gradient oracle against its pins, and plausible mistakes planted
in copies of it (CPU only).

Each mutant is one textual edit of ``oracle/kda_oracle_grad.c`` compiled,
with the unmodified forward oracle, into a temporary library; the real
oracle is never modified.
"""
import os

import numpy as np
import pytest

import oracle
from tests import pins_grad

GRAD_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "kda_oracle_grad.c")


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", pins_grad.ALL_GRAD_CHECKS, ids=lambda f: f.__name__)
def test_grad_pin(lib, check):
    check(lib)


def test_grad_thread_count_does_not_change_bits(lib):
    x, cu, d_o, d_final = pins_grad._case(31, [40, 0, 90], 3, 5, 6)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], cu, x["init_state"], d_o, d_final)
    g1 = oracle.prefill_grad(*args, lib=lib, nthreads=1)
    g4 = oracle.prefill_grad(*args, lib=lib, nthreads=4)
    for name in pins_grad.NAMES:
        assert np.array_equal(g1[name], g4[name]), name


def test_grad_is_linear_in_the_upstream_gradients(lib):
    x, cu, d_o, d_final = pins_grad._case(32, [30, 70], 2, 4, 3)
    base = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], cu, x["init_state"])
    ga = oracle.prefill_grad(*base, d_o, None, lib=lib)
    gb = oracle.prefill_grad(*base, np.zeros_like(d_o), d_final, lib=lib)
    gab = oracle.prefill_grad(*base, d_o, d_final, lib=lib)
    for name in pins_grad.NAMES:
        assert pins_grad._rel(ga[name] + gb[name], gab[name]) < 1e-12, name


# (name, original text, replacement) -- each original must occur exactly once
GRAD_MUTANTS = [
    ("dq_before_write", "acc += St[(int64_t)j * K + i] * dO[j];", "acc += D[(int64_t)j * K + i] * dO[j];"),
    ("no_readout_grad", "B->G[(int64_t)j * K + i] += B->qq[i] * dO[j];", ";"),
    ("dv_without_beta", "= beta * B->de[j];", "= B->de[j];"),
    ("dbeta_sign", "db += B->de[j] * (B->vv[j] - p[j]);", "db += B->de[j] * (B->vv[j] + p[j]);"),
    ("dp_sign", "B->dp[j] = -beta * B->de[j];", "B->dp[j] = beta * B->de[j];"),
    ("dk_drops_read_term", "J->dk[kb + i] = acc1 + acc2;", "J->dk[kb + i] = acc1;"),
    ("dk_drops_write_term", "J->dk[kb + i] = acc1 + acc2;", "J->dk[kb + i] = acc2;"),
    ("dla_on_written_state", "acc += B->dD[(int64_t)j * K + i] * D[(int64_t)j * K + i];",
     "acc += B->dD[(int64_t)j * K + i] * St[(int64_t)j * K + i];"),
    ("state_grad_not_decayed", "B->G[(int64_t)j * K + i] = B->a[i] * B->dD[(int64_t)j * K + i];",
     "B->G[(int64_t)j * K + i] = B->dD[(int64_t)j * K + i];"),
    ("state_grad_skips_read", "B->dD[(int64_t)j * K + i] = B->G[(int64_t)j * K + i] + B->kk[i] * B->dp[j];",
     "B->dD[(int64_t)j * K + i] = B->G[(int64_t)j * K + i];"),
    ("wrong_segment_copy", "memcpy(B->S, B->ckpt + s * KV,", "memcpy(B->S, B->ckpt + (s > 0 ? s - 1 : 0) * KV,"),
    ("final_grad_ignored", "J->d_final ? J->d_final[sbase + x] : 0.0", "0.0"),
]


@pytest.mark.parametrize("name,old,new", GRAD_MUTANTS, ids=[m[0] for m in GRAD_MUTANTS])
def test_grad_pins_catch_mutant(tmp_path, name, old, new):
    text = open(GRAD_SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} must occur once"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(grad_src=str(src), out=str(tmp_path / f"libmut_{name}.so"), force=True))
    caught = []
    for check in pins_grad.ALL_GRAD_CHECKS:
        try:
            check(lib)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no gradient pin caught mutant {name}"
