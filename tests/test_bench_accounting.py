"""The benchmark's work accounting reproduces the rates the pages print.

Source: vLLM PR 54513, section "Microbenchmarks" (GB300), stored with its
citation in tests/golden/pr54513_microbench.txt.  Recomputing GB/s (decode)
and TFLOP/s (prefill) from the printed microseconds with bench.py's formulas
must land on the printed rate; visible blocks per prefill row come from the
oracle's metadata."""
import os

import numpy as np

import bench
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pr54513_microbench.txt")


def _rows(kind):
    out = []
    for line in open(GOLDEN):
        parts = line.split()
        if parts and parts[0] == kind:
            out.append(parts[1:])
    return out


def test_decode_bytes_match_published_rates():
    rows = _rows("decode")
    assert len(rows) == 14
    for dql, reqs, mean_ctx, us, gbps in rows:
        dql, reqs, mean_ctx, us, gbps = int(dql), int(reqs), int(mean_ctx), float(us), float(gbps)
        nbytes = bench.decode_bytes(reqs, dql, reqs * mean_ctx / 4.0)
        got = nbytes / (us * 1e-6) / 1e9
        assert abs(got - gbps) / gbps < 0.005, (dql, reqs, mean_ctx, got, gbps)


def test_prefill_flops_match_published_rates():
    rows = _rows("prefill")
    assert len(rows) == 12
    for reqs, qlen, prefix, us, tflops in rows:
        reqs, qlen, prefix, us, tflops = int(reqs), int(qlen), int(prefix), float(us), float(tflops)
        qsl = np.arange(reqs + 1, dtype=np.int32) * qlen
        seq = np.full(reqs, prefix + qlen, np.int32)
        _, _, vis = O.token_metadata(qsl, seq, reqs * qlen)
        got = bench.prefill_flops(int(vis.astype(np.int64).sum())) / (us * 1e-6) / 1e12
        assert abs(got - tflops) / tflops < 0.001, (reqs, qlen, prefix, got, tflops)


def test_topk_and_gpu_count_guard():
    assert bench.topk_bytes(2, 10, 3) == 2 * 10 * 4 + 2 * 3 * 4
    assert bench.main(["--gpus", "2"]) == 2
