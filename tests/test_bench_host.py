"""Host-side checks of bench.py: the single-GPU guard and the algorithmic
work it divides by (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lsh_sparse_attention_hash_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_work_of_the_headline_shape():
    # 1 x 8 x 65,536 tokens, 8 rounds, B = 1,024, bf16: N = 4,194,304 token-rounds
    w = synth.WORKLOADS["long"]
    N, T = w.token_rounds, w.batch * w.heads * w.seq_len
    assert N == 4_194_304 and T == 524_288
    a = bench.algorithmic(w)
    assert a["hash"]["flops"] == N * 64 * 1024                     # N.d.B
    assert a["sort"]["bytes"] == 16 * N                            # keys twice, perm, inv_perm
    assert a["attend"]["bytes"] == 524 * N                         # x, v rows; perm, bucket; o; lse
    assert a["attend"]["flops"] == 32_768 * N                      # 4 x 64 x 2 x 64 per token-round
    assert a["combine"]["bytes"] == 264 * N + 256 * T              # o row, lse, inv_perm; y row
    # x read once, every rotation read, bucket ids written
    assert a["hash"]["bytes"] == T * 128 + 8 * 8 * 512 * 64 * 2 + 4 * N


def test_roofline_time_of_the_headline_shape():
    r = bench.roofline_us(synth.WORKLOADS["long"])
    assert r["hash"] == pytest.approx(274.877906944e9 / 2.5e15 * 1e6, abs=0.01)   # MFMA-bound
    assert r["attend"] == pytest.approx(524 * 4_194_304 / 8e12 * 1e6, abs=0.01)
    assert sum(v for k, v in r.items()) == pytest.approx(548.3, abs=0.2)


def test_set_union_adds_the_round_key_table():
    w = synth.WORKLOADS["long"]
    N, T = w.token_rounds, w.batch * w.heads * w.seq_len
    extra = bench.algorithmic(w, union=True)["attend"]["bytes"] - bench.algorithmic(w)["attend"]["bytes"]
    assert extra == 8 * N + 4 * 8 * T + 4 * 8 * N


def test_local_attention_work_counts_each_window_once():
    w = synth.WORKLOADS["local_long"]          # one chunk before and after, not causal
    a = bench.algorithmic_local(w)
    C = w.seq_len // 64
    keys = (3 * C - 2) * 64                    # the first and last chunk lose one neighbour
    assert a["flops"] == w.batch * w.heads * 64 * keys * 4 * 64
    assert a["bytes"] == w.batch * w.heads * w.seq_len * (2 * 64 * 2 + 4 * 64 + 4)


def test_percentiles():
    p = bench.pct([float(i) for i in range(1, 101)])
    assert p["median"] == pytest.approx(50.5)
    assert p["p10"] == pytest.approx(10.9)
    assert p["p90"] == pytest.approx(90.1)


def test_matrix_core_busy_is_reported_only_for_the_profiled_sources(monkeypatch):
    from lsh_sparse_attention_hash_amd import rocprof_summary
    busy = bench.measured_busy("hash", "long")
    assert busy is not None and 0.0 < busy < 1.0
    k = bench.measured_busy("gemm", "layer_long", "lsh::gemm_bf16_kernel<1, 1>")
    assert k is not None and 0.0 < k < 1.0
    assert bench.measured_busy("hash", "no_such_workload") is None
    monkeypatch.setattr(rocprof_summary, "source_digest", lambda step: "000000000000")
    assert bench.measured_busy("hash", "long") is None
