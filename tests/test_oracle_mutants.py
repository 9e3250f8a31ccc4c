"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a private copy of oracle/lsh_oracle.c (the
committed file is never touched), builds it with gcc into a temporary
directory and runs the pin suite against that build in a child process.  The
pins pass on the real oracle and must fail on every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lsh_oracle.c")

MUTANTS = {
    "hash_drops_negated_half": (
        "const double c = (t < half) ? s[t] : -s[t - half];",
        "const double c = (t < half) ? s[t] : s[t - half];"),
    "hash_ties_to_highest_index": (
        "if (c > best) { best = c; arg = t; }",
        "if (c >= best) { best = c; arg = t; }"),
    "hash_reads_rotation_transposed": (
        "acc = acc + x[k] * rot_hr[(int64_t)j * d + k];",
        "acc = acc + x[k] * rot_hr[(int64_t)k * half + j];"),
    "sort_unstable_positions": (
        "if (p->pos != q->pos) return p->pos < q->pos ? -1 : 1;",
        "if (p->pos != q->pos) return p->pos < q->pos ? 1 : -1;"),
    "window_without_predecessor": (
        "const int lo = (c > 0) ? (c - 1) * s->chunk : 0;",
        "const int lo = c * s->chunk;"),
    "window_wraps_to_last_chunk": (
        "const int lo = (c > 0) ? (c - 1) * s->chunk : 0;",
        "const int lo = (c > 0) ? (c - 1) * s->chunk : s->len - s->chunk;"),
    "bucket_mask_dropped": (
        "if (bk[j] != bk[i]) continue;", ";"),
    "causal_strict": (
        "if (s->causal && j > i) continue;", "if (s->causal && j >= i) continue;"),
    # (Comparing sorted slots instead of positions is NOT a mistake: inside one
    # bucket the sort keeps position order, so the two tests agree.)
    "causal_ignored": (
        "if (s->causal && j > i) continue;", ";"),
    "self_mask_ignored": (
        "if (s->self_mask && j == i) continue;", ";"),
    "keys_not_normalised": (
        "score[a] = dot / nj * inv_sqrt_d;", "score[a] = dot * inv_sqrt_d;"),
    "no_sqrt_d_scale": (
        "score[a] = dot / nj * inv_sqrt_d;", "score[a] = dot / nj;"),
    "lse_without_max": (
        "const double l = mx + log(sum);", "const double l = log(sum);"),
    "combine_uniform_weights": (
        "const double w = exp(lse[seg * L + slot] - mx);", "const double w = 1.0;"),
    "combine_skips_unsort": (
        "const int64_t slot = inv_perm[seg * L + i];", "const int64_t slot = i;"),
    "self_only_returns_zero": (
        "for (int k = 0; k < d; ++k) y[k] = v[(bh * L + i) * d + k];",
        "for (int k = 0; k < d; ++k) y[k] = 0.0;"),
    "union_keeps_keys_of_earlier_rounds": (
        "      if (!found_earlier(s, buckets, inv_perm, bh, r, i, cand[a])) cand[kept++] = cand[a];",
        "      cand[kept++] = cand[a];"),
    "union_earlier_round_ignores_bucket": (
        "    if (bk[i] != bk[j]) continue;\n    const int c = ip[i] / s->chunk;",
        "    const int c = ip[i] / s->chunk;"),
    "union_earlier_window_without_predecessor": (
        "    const int first = (c > 0) ? (c - 1) * s->chunk : 0;\n    if (ip[j] >= first",
        "    const int first = c * s->chunk;\n    if (ip[j] >= first"),
    # attending each key in its LAST round gives the same y: only the
    # per-round pins can tell
    "union_keeps_keys_in_their_last_round": (
        "  for (int q = 0; q < r; ++q) {", "  for (int q = r + 1; q < s->rounds; ++q) {"),
    "union_drops_the_own_round": (
        "  for (int q = 0; q < r; ++q) {", "  for (int q = 0; q <= r; ++q) {"),
    "local_ignores_following_chunks": (
        "const int c_hi = (c + after < nchunks - 1) ? c + after : nchunks - 1;",
        "const int c_hi = c;"),
    "local_one_chunk_too_few_before": (
        "const int c_lo = (c - before > 0) ? c - before : 0;",
        "const int c_lo = (c - before > 0) ? c - before + 1 : 0;"),
    "local_causal_ignored": (
        "if (s->causal && j > i) return 0;", ";"),
    "local_self_mask_ignored": (
        "if (s->self_mask && j == i) return 0;", ";"),
    "local_empty_row_returns_zero": (
        "for (int k = 0; k < d; ++k) y[k] = vs[(int64_t)i * d + k];",
        "for (int k = 0; k < d; ++k) y[k] = 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "lsh_oracle_mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "liblsh_oracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", str(path), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, LSH_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"


LAYER_SRC = os.path.join(ROOT, "oracle", "layer.py")
LAYER_MUTANTS = {
    "inverse_adds_attention": (
        "    x1 = y1 - attention(x2, w, cfg)", "    x1 = y1 + attention(x2, w, cfg)"),
    "inverse_ffn_of_x2": (
        "    x2 = y2 - ffn(y1, w, cfg.get(\"ffn_chunk\"))",
        "    x2 = y2 - ffn(y2, w, cfg.get(\"ffn_chunk\"))"),
    "forward_ffn_of_x1": (
        "    y2 = x2 + ffn(y1, w, cfg.get(\"ffn_chunk\"))",
        "    y2 = x2 + ffn(x1, w, cfg.get(\"ffn_chunk\"))"),
    "ffn_without_relu": (
        "h = bf16_round(np.maximum(oracle.linear(xb, w[\"w_1\"], w[\"b_1\"]), 0.0))",
        "h = bf16_round(oracle.linear(xb, w[\"w_1\"], w[\"b_1\"]))"),
    "ffn_without_first_bias": (
        "oracle.linear(xb, w[\"w_1\"], w[\"b_1\"])", "oracle.linear(xb, w[\"w_1\"])"),
    "ffn_hidden_not_rounded": (
        "h = bf16_round(np.maximum(", "h = (np.maximum("),
    "heads_interleaved": (
        "return np.ascontiguousarray(t.reshape(b, L, heads, HEAD_DIM).transpose(0, 2, 1, 3))",
        "return np.ascontiguousarray(t.reshape(b, L, HEAD_DIM, heads).transpose(0, 3, 1, 2))"),
    "round_ties_away": (
        "return np.ldexp(np.rint(m * 256.0) / 256.0, e)",
        "return np.ldexp(np.trunc(m * 256.0 + np.copysign(0.5, m)) / 256.0, e)"),
}


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_layer_pins_catch_mutant(name, tmp_path):
    old, new = LAYER_MUTANTS[name]
    src = open(LAYER_SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "layer_mutant.py"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, LSH_ORACLE_LAYER=str(path), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_layer_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
