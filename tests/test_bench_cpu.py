"""bench.py's host-side contract, checked without a GPU: it refuses more than one GPU with
a message, its algorithmic byte counts follow from the shapes, and the recorded HBM
traffic is reported only while the chunk-output sources are unchanged."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from state_space_sequence_chunk_amd import inputs as gen  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_at_the_bench_shape():
    w = gen.WORKLOADS["2.7b-bf16"]
    by, fl = bench.algorithmic(w)
    x = 2 * 16384 * 80 * 64 * 2          # bf16 x
    y = 2 * 16384 * 80 * 64 * 4          # fp32 y
    bc = 2 * 16384 * 1 * 128 * 2         # one of B, C
    dec = 2 * 80 * 16384 * 4             # G or dt_t
    states = 2 * 80 * 64 * 64 * 128      # chunk-initial states, elements
    assert by["chunk_out"] == x + 2 * bc + 2 * dec + states * 2 + 80 * 4 + y
    # over segment-relative states (8 segments): plus the 7 states entering segments 1..
    # and each chunk's decay from its segment's start
    by8, _ = bench.algorithmic(w, 8)
    assert by8["chunk_out"] == by["chunk_out"] + 7 * 2 * 80 * 64 * 128 * 2 + 2 * 80 * 64 * 4
    assert by["chunk_state"] == x + bc + dec + 80 * 4 + states * 4
    # the page's per-head dense flops: 2 T^2 S + 2 T S P + 2 T^2 P per (batch, chunk, head)
    assert fl["chunk_out"] == 2 * 64 * 80 * (2.0 * 256 * 256 * 128 + 2.0 * 256 * 128 * 64
                                             + 2.0 * 256 * 256 * 64)
    # backward: inputs read once and gradients written once
    tok = 2 * 16384 * 80
    assert bench.backward_bytes(w) == (tok * 64 * 2 + tok * 2 + 2 * bc + tok * 64 * 4
                                       + 2 * 80 * 64 * 128 * 4 + 2 * 80 * 4
                                       + tok * 64 * 4 + tok * 4 + 2 * 2 * 16384 * 128 * 4
                                       + 2 * 80 * 64 * 128 * 4 + 2 * 80 * 4)


def test_recorded_traffic_is_consistent():
    # reported only for a workload with a counter summary, and then close to the bytes
    # the kernel must move (the counters show no re-reads)
    assert bench.measured_traffic("no-such-workload") is None
    t = bench.measured_traffic("2.7b-bf16")
    if t is not None:
        w = gen.WORKLOADS["2.7b-bf16"]
        # the bench shape takes the segmented state pass: chunk_out also reads the states
        # entering segments 1..
        from state_space_sequence_chunk_amd import ssd
        sh = ssd.make_shape(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                            w.chunk, ssd.SSD_BF16)
        nseg = ssd.segment_plan(sh)[2]
        assert nseg == 6
        by, _ = bench.algorithmic(w, nseg)
        assert abs(t - by["chunk_out"]) <= 0.01 * by["chunk_out"]
