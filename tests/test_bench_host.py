"""Host-only checks of bench.py: the multi-GPU refusal and the algorithmic
byte and FLOP accounting behind its roofline fractions."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_accounting_matches_the_8k_workload():
    # q, k, v, o bf16 (4 x 256 B), log_alpha fp32 (512 B), beta bf16 (2 B) per
    # token-head, plus the final state; dense MFMA work 2 (5 C d + 3 d^2)
    nbytes, flops = bench.prefill_algorithmic(8192, 32, 128, 1, False, True)
    assert nbytes == 8192 * 32 * 1538 + 32 * 128 * 128 * 4 == 405_274_624
    assert flops == 8192 * 32 * 180_224
    assert abs(flops / 1e9 - 47.24) < 0.01


def test_decode_accounting_matches_the_256_sequence_workload():
    # state read + write (128 KiB) and 1,538 B of token I/O per (sequence, head)
    assert bench.decode_algorithmic(256, 32, 128) == 256 * 32 * (2 * 128 * 128 * 4 + 1538) == 1_086_341_120


def test_backward_accounting():
    nbytes, flops = bench.backward_algorithmic(8192, 32, 128, 1)
    per_chunk = 28 * 64 * 64 * 128 + 16 * 64 * 128 * 128 + 4 * 64 ** 3
    assert per_chunk == 32_505_856
    assert flops == 128 * 32 * per_chunk
    assert nbytes == 8192 * 32 * (3 * 256 + 512 + 2 + 256 + 4 * 512 + 4) + 2 * 32 * 128 * 128 * 4


def test_traffic_record_key_ignores_comments_but_not_code():
    src = 'int a = 1; // gate\n/* block\n   comment */ const char* s = "x // y /* z */";\nchar q = \'"\';  s += 1;\n'
    stripped = bench.strip_comments(src)
    assert stripped == 'int a = 1; const char* s = "x // y /* z */"; char q = \'"\'; s += 1;'
    # comment edits and reflowing leave the key alone; a changed token does not
    assert bench.strip_comments(src.replace("// gate", "// the gate, reworded").replace("  ", " ")) == stripped
    assert bench.strip_comments(src.replace("a = 1", "a = 2")) != stripped
    assert len(bench.source_digest()) == 16
