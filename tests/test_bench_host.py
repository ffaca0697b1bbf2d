"""Host logic of bench.py (CPU only): the work and byte counts behind the
roofline figures, the comment-insensitive kernel hash, and the one-GPU rule."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_swska_pairs_is_the_band_count():
    for T in (1, 5, 64, 300):
        for w in (1, 3, 64, 1000):
            brute = sum(1 for t in range(T) for s in range(T) if t - w < s <= t)
            assert bench.swska_pairs(T, w) == brute


def test_prefill_bytes_per_token_head():
    # q, k, g, tau in (dk each), v in and o out (dv each), bf16; plus the fp32 final state
    assert bench.prefill_bytes(1, 1, 1, 128, 128) == 1536 + 128 * 128 * 4
    assert bench.prefill_bytes(4, 16, 4096, 128, 128) == 406_847_488


def test_decode_bytes_per_head_step():
    # fp32 state read and written, q k g tau v in, o out (bf16)
    assert bench.decode_bytes(1, 1, 128, 128) == 2 * 128 * 128 * 4 + (4 * 128 + 128) * 2 + 128 * 2
    assert bench.decode_bytes(256, 16, 128, 128) == 543_162_368


def test_code_only_ignores_comments_and_whitespace():
    a = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y /* z */";\n'
    b = 'int a=1;\n\n   const char *s = "x // y /* z */";  // other note\n'
    assert bench._code_only(a) == bench._code_only(b) == 'inta=1;constchar*s="x // y /* z */";'
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_swska_decode_bytes_per_sequence_step():
    # key window + one head's value window, q, k_new, v_new in; k_new, v_new to the caches; o out
    w, d = 4096, 128
    assert bench.swska_decode_bytes(1, 1, d, d, w) == 2 * w * d * 2 + d * 2 + 2 * (2 * d * 2) + d * 2


def test_source_hash_covers_every_source_and_its_compiler_options(monkeypatch):
    # the traffic records are tied to the code the counters were taken on: every
    # source of a kernel (the prefill's state pass is a unit of its own) and the
    # per-file compiler options count
    import gated_linear_attention_ddts_amd.build as build
    csrc = os.path.join(ROOT, "gated_linear_attention_ddts_amd", "csrc")
    for kind, files in bench.KERNEL_SOURCES.items():
        assert all(os.path.exists(os.path.join(csrc, f)) for f in files), kind
    assert {"scan_mfma.hip", "scan_state.hip", "scan_mfma.h"} <= set(bench.KERNEL_SOURCES["prefill"])
    before, other = bench.source_hash("prefill"), bench.source_hash("decode")
    flags = dict(build.FILE_FLAGS)
    flags["scan_state.hip"] = ["-mno-amdgpu-ieee", "-fno-honor-nans"]
    monkeypatch.setattr(build, "FILE_FLAGS", flags)
    assert bench.source_hash("prefill") != before
    assert bench.source_hash("decode") == other
    monkeypatch.undo()
    assert bench.source_hash("prefill") == before
