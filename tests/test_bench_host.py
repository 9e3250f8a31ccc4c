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
    # x, v rows; perm, bucket; fp16 o row; lse -- and v once more for the output scale
    assert a["attend"]["bytes"] == 396 * N + 128 * T
    assert a["attend"]["flops"] == 32_768 * N                      # 4 x 64 x 2 x 64 per token-round
    assert a["combine"]["bytes"] == 136 * N + 256 * T              # fp16 o row, lse, inv_perm; y row
    # fp32 inputs keep fp32 output rows and need no scale pass
    f = bench.algorithmic(synth.WORKLOADS["tiny"])
    tw = synth.WORKLOADS["tiny"]
    Nt, Tt = tw.token_rounds, tw.batch * tw.heads * tw.seq_len
    assert f["attend"]["bytes"] == (2 * 64 * 4 + 8 + 4 * 64 + 4) * Nt
    assert f["combine"]["bytes"] == 264 * Nt + 256 * Tt
    # x read once, every rotation read, bucket ids written
    assert a["hash"]["bytes"] == T * 128 + 8 * 8 * 512 * 64 * 2 + 4 * N
    # fp32 per-round rows for bf16 inputs: the fixed per-token byte counts
    # (524 B per token-round for the attention, 264 + 256 per token-head for
    # the combine), no scale pass
    g = bench.algorithmic(w.replace(o_format="f32"))
    assert g["attend"]["bytes"] == 524 * N
    assert g["combine"]["bytes"] == 264 * N + 256 * T
    assert bench.fixed_count_bytes(w) == {"hash": 128 * T + 4 * N, "sort": 16 * N,
                                     "attend": 524 * N, "combine": 264 * N + 256 * T}


def test_path_target_fractions():
    """Both target branches from per-call times: the attention's flops over
    the bf16 peak, the path's bytes over HBM peak (own and fixed counts)."""
    w = synth.WORKLOADS["long"]
    N, T = w.token_rounds, w.batch * w.heads * w.seq_len
    per = {"hash": 0.4, "sort": 0.025, "attend": 0.35, "combine": 0.145}   # ms
    ns = bench.path_targets(w, per)
    assert ns["attend_mfma_frac"] == pytest.approx(32_768 * N / 0.35e-3 / 2.5e15, abs=1e-4)
    own = 16 * N + 396 * N + 128 * T + 136 * N + 256 * T
    assert ns["path_bytes"] == own
    assert ns["path_hbm_frac"] == pytest.approx(own / 0.52e-3 / 8e12, abs=1e-4)
    fixed = 16 * N + 524 * N + 264 * N + 256 * T
    assert ns["path_hbm_frac_fixed_counts"] == pytest.approx(fixed / 0.52e-3 / 8e12, abs=1e-4)
    assert ns["met"] == (ns["path_hbm_frac"] >= 0.6 or ns["attend_mfma_frac"] >= 0.4)


def test_roofline_time_of_the_headline_shape():
    r = bench.roofline_us(synth.WORKLOADS["long"])
    assert r["hash"] == pytest.approx(274.877906944e9 / 2.5e15 * 1e6, abs=0.01)   # MFMA-bound
    assert r["attend"] == pytest.approx((396 * 4_194_304 + 128 * 524_288) / 8e12 * 1e6, abs=0.01)
    assert sum(r.values()) == pytest.approx(109.95 + 8.39 + 216.0 + 88.1, abs=0.2)


def test_set_union_adds_the_round_key_table():
    w = synth.WORKLOADS["long"]
    N, T = w.token_rounds, w.batch * w.heads * w.seq_len
    extra = bench.algorithmic(w, union=True)["attend"]["bytes"] - bench.algorithmic(w)["attend"]["bytes"]
    # table build; keys of rounds 0..6 stored (8 per token); round r gathers r keys
    assert extra == 8 * N + 4 * 8 * T + 4 * T * (0 + 1 + 2 + 3 + 4 + 5 + 6 + 7)


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


def test_matrix_core_busy_is_reported_only_for_the_profiled_sources(monkeypatch, tmp_path):
    from lsh_sparse_attention_hash_amd import rocprof_summary
    d = rocprof_summary.source_digest("hash")
    g = rocprof_summary.source_digest("gemm")
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "mfma_busy_w.md").write_text(
        "| kernel | launches | dispatch us | clock GHz | MFMA instructions | VALU instructions "
        "| MFMA busy SIMD-cycles | MFMA busy |\n|---|---|---|---|---|---|---|---|\n"
        "| lsh::hash_bf16_kernel | 13 | 400.0 | 2.07 | 1 | 2 | 3 | 0.352 |\n"
        "| lsh::gemm_bf16_kernel<1, 1> | 13 | 100.0 | 2.27 | 1 | 2 | 3 | 0.273 |\n\n"
        "| step | workload | digest | kernel | MFMA busy |\n|---|---|---|---|---|\n"
        f"| hash | w | {d} | lsh::hash_bf16_kernel | 0.352 |\n"
        f"| gemm | w | {g} | lsh::gemm_bf16_kernel<1, 1> | 0.273 |\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_busy("hash", "w") == 0.352
    assert bench.measured_busy("gemm", "w", "lsh::gemm_bf16_kernel<1, 1>") == 0.273
    assert bench.measured_busy("gemm", "w", "lsh::gemm_bf16_kernel<0, 0>") is None
    assert bench.measured_busy("hash", "no_such_workload") is None
    monkeypatch.setattr(rocprof_summary, "source_digest", lambda step: "000000000000")
    assert bench.measured_busy("hash", "w") is None
