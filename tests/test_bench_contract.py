"""Host-side parts of bench.py: the one-GPU guard, the algorithmic byte counts behind the
roofline lines, and the rule that committed counter summaries count only for the kernel
source they were taken on."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "error" in json.loads(res.stdout.strip().splitlines()[-1])


def test_prefill_algorithmic_bytes():
    """8192 x 96, d = 128: per token and head 2 B x (128 q + 128 k + 128 v) + 4 B x 128 g +
    4 B beta + 2 B x 128 o = 1540 B; plus h0 in and the final state out, 96 x 128 x 128 x 4 B
    each: 1,223,688,192 B (the figure the prefill profiles quote as 1.2237e9)."""
    assert 2 * 384 + 4 * 128 + 4 + 2 * 128 == 1540
    assert bench.algorithmic_bytes(8192, 96, 128, 128, 2, 2) == \
        8192 * 96 * 1540 + 2 * 96 * 128 * 128 * 4 == 1_223_688_192
    # two sequences carry two entering and two final states
    assert bench.algorithmic_bytes(100, 2, 64, 64, 4, 4, n_seqs=2) == \
        100 * 2 * (4 * 192 + 4 * 64 + 4 + 4 * 64) + 2 * 2 * 2 * 64 * 64 * 4


def test_decode_algorithmic_bytes():
    """One request, one head, d = 128, conv width 4, 8 new tokens, 3 accepted drafts:
    state read + state_acc + state written (3 x 64 KiB), conv tail in and out
    (2 x 384 channels x 3 x 4 B), replayed drafts' q, k, v, g (bf16) + beta, the new window's
    q, k, v, g, z (bf16) + beta, bf16 outputs, the taps and the norm weight."""
    expect = (3 * 128 * 128 * 4 + 2 * 384 * 3 * 4 + 3 * (4 * 128 + 1) * 2
              + 8 * (5 * 128 + 1) * 2 + 8 * 128 * 2 + 384 * 4 * 4 + 128 * 4)
    assert bench.decode_bytes(1, 1, 128, 4, 8, 3, 2) == expect


def test_counter_summary_counts_only_for_its_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("__global__ void k() {}\n")
    other = tmp_path / "helper.h"
    other.write_text("#pragma once\n")
    digest = hashlib.sha256(src.read_bytes() + other.read_bytes()).hexdigest()
    assert bench.source_digest((str(src), str(other))) == digest
    counters = tmp_path / "counters.txt"
    counters.write_text(f"# a comment: with a colon\nkernel_source_sha256: {digest}\n"
                        "hbm_bytes_per_launch: 123456\n")
    assert bench.counter_traffic(str(counters), (str(src), str(other))) == 123456.0
    src.write_text("__global__ void k() { /* changed */ }\n")
    assert bench.counter_traffic(str(counters), (str(src), str(other))) is None
    assert bench.counter_traffic(str(tmp_path / "missing.txt"), str(src)) is None


def test_committed_counters_match_the_current_kernels():
    """The summaries under profiles/ were taken on the kernel sources in the tree, so the
    bench line's traffic fields are not null."""
    assert bench.counter_traffic() is not None
    assert bench.counter_traffic(bench.DECODE_COUNTERS, bench.DECODE_SRC) is not None
    assert bench.counter_traffic(bench.RAW_COUNTERS) is not None
    assert bench.counter_traffic(bench.SEGMENT_COUNTERS, bench.SEGMENT_SRC) is not None
    assert bench.counter_traffic(bench.VARLEN_COUNTERS, bench.VARLEN_SRC) is not None
    assert bench.counter_traffic(bench.BACKWARD_COUNTERS, bench.BACKWARD_SRC) is not None


def test_hbm_roofline_object():
    r = bench.hbm_roofline(8e9, 2.0)
    assert r == {"bound": "hbm", "achieved": 4000.0, "peak": 8000.0, "unit": "GB/s",
                 "frac": 0.5, "traffic": None}
