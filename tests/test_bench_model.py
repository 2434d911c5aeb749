"""bench.py's algorithmic byte and FLOP model, and its command-line contract (no GPU).

The per-row byte model counts what the method must move: the forward reads V e bytes of
logits and 4 of target and writes 4 of loss and 8 of lse; the VJP reads V e, lse (8),
target (4) and g (4) and writes V e.  The expected totals below are those figures worked
out by hand for each workload shape, in MB of 1e6 bytes.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def mb(x):
    return round(x / 1e6, 1)


@pytest.mark.parametrize("rows,V,e,fwd,vjp", [
    (2048, 151936, 2, 622.4, 1244.7),        # bf16 [2048 x 151,936]
    (8192, 32000, 2, 524.4, 1048.7),         # bf16 [8192 x 32,000]
    (1 << 20, 8, 4, 50.3, 83.9),             # fp32 [1,048,576 x 8]
    (65536, 1024, 4, 269.5, 537.9),          # fp32 [65,536 x 1024]
    (65536, 1024, 2, 135.3, 269.5),          # fp16 [65,536 x 1024]
    (1180, 32768, 4, 154.7, 309.3),          # the [10, 119, 32768][:, :-1] view
    ((1 << 27) + (1 << 20), 8, 4, 6492.8, 10821.3),  # fp32 [135,266,304 x 8]
])
def test_ce_bytes(rows, V, e, fwd, vjp):
    f, v = bench.ce_bytes(rows, V, e)
    assert (mb(f), mb(v)) == (fwd, vjp)


def test_one_kernel_bytes():
    """ce_forward_vjp reads each row once: two thirds of the two calls' row bytes, plus
    20 bytes per row (target, g read; loss, lse written)."""
    assert bench.fused_bytes(2048, 151936, 2) == 2048 * (2 * 151936 * 2 + 20)
    assert mb(bench.fused_bytes(2048, 151936, 2)) == 1244.7
    f, v = bench.ce_bytes(2048, 151936, 2)
    assert abs(bench.fused_bytes(2048, 151936, 2) / (f + v) - 2 / 3) < 1e-4


def test_lce_flops():
    assert bench.lce_flops(8192, 4096, 151936) == 2 * 8192 * 4096 * 151936
    assert abs(bench.lce_flops(8192, 4096, 151936) - 1.0196e13) < 1e9


def test_options_vjp_skips_ignored_rows():
    """Every 16th of 2048 rows ignored: their gradient rows are written (zeros) but their
    logits are not read."""
    V, e = 151936, 2
    f, v = bench.opt_bytes(2048, V, e, ignored=128)
    assert f == 2048 * (V * e + 16)
    assert v == 2048 * (V * e + 12) + 1920 * V * e
    assert mb(v) == 1205.8
    assert bench.opt_bytes(2048, V, e) == (f, 2048 * (2 * V * e + 12))


def test_divergence_bytes():
    V, e = 151936, 4
    assert bench.kl_bytes(512, V, e) == (512 * (2 * V * e + 20), 512 * (3 * V * e + 20))
    assert bench.js_bytes(512, V, e) == (512 * (4 * V * e + 24), 512 * (3 * V * e + 24))
    assert bench.probs_bytes(512, V, e) == (512 * (2 * V * e + 16), 512 * (3 * V * e + 12))


def test_traffic_table_is_keyed_by_current_sources():
    """Each TRAFFIC entry names a kernel whose source hash bench.py can compute; an
    entry whose hash differs is reported as null, never as a stale number."""
    for k, t in bench.TRAFFIC.items():
        sha = bench.source_sha(k)
        assert len(sha) == 16
        assert bench.traffic_for(k) == (t["bytes"] if t["source_sha"] == sha else None)


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert p.returncode == 2
    assert p.stdout == ""
    assert "one GPU" in p.stderr
