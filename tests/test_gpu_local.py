"""GPU parity of local chunked attention (lsh_local_attend) against the fp64
oracle: y and lse within max abs 1e-5 (fp32 inputs) / 2e-2 (bf16 inputs),
lse = -inf exactly where the oracle's is, and y = v bit for bit on rows that
keep no key."""
import sys

import numpy as np
import pytest
import torch

from lsh_sparse_attention_hash_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lsh_sparse_attention_hash_amd import binding
    return binding


def local_workload(name, b, h, L, before, after, causal, self_mask, dtype, seed, **kw):
    return synth.Workload(name, b, h, L, 64, 1, 1, 64, causal, self_mask, dtype, seed,
                          look_before=before, look_after=after, **kw)


def run_local(B, w, inp):
    cfg = B.config_for(w)
    qk = B.to_device(inp["qk"], w.dtype)
    v = B.to_device(inp["v"], w.dtype)
    loc = B.Local(cfg, w.look_before, w.look_after)
    loc.run(qk, v)
    torch.cuda.synchronize()
    return loc


def host(t):
    return t.detach().cpu().numpy()


def check(y, lse, y_ref, lse_ref, v, tol, what):
    ninf = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf), f"{what}: -inf pattern differs"
    err_l = np.abs(lse[~ninf] - lse_ref[~ninf]).max(initial=0.0)
    assert err_l <= tol, f"{what}: lse err {err_l}"
    err_y = np.abs(y - y_ref).max(initial=0.0)
    assert err_y <= tol, f"{what}: y err {err_y}"
    # rows with no key return their own value exactly
    assert np.array_equal(y[ninf], v[ninf]), f"{what}: empty rows differ from v"
    return err_y


CASES = {
    "tiny_f32": local_workload("l_tiny", 1, 1, 1024, 1, 1, False, True, "f32", 31),
    "f32_causal": local_workload("l_f32c", 2, 2, 64 * 9, 2, 0, True, False, "f32", 32),
    "bf16_both_sides": local_workload("l_b11", 2, 4, 4096, 1, 1, False, True, "bf16", 33),
    "bf16_causal_back3": local_workload("l_c3", 1, 8, 4096, 3, 0, True, True, "bf16", 34),
    "bf16_ahead_only": local_workload("l_a2", 1, 2, 64 * 11, 0, 2, False, False, "bf16", 35),
    "bf16_own_chunk": local_workload("l_00", 1, 3, 64 * 5, 0, 0, True, True, "bf16", 36),
    "bf16_whole_window": local_workload("l_all", 1, 2, 1024, 100, 100, False, False, "bf16", 37),
    "bf16_single_chunk": local_workload("l_one", 2, 2, 64, 2, 2, True, True, "bf16", 38),
    "bf16_clusters": local_workload("l_cl", 1, 2, 4096, 2, 1, False, True, "bf16", 39,
                                    n_clusters=8),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_local_parity(B, name):
    w = CASES[name]
    say(f"[local] {w}")
    inp = synth.make_inputs(w)
    loc = run_local(B, w, inp)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    y_ref, lse_ref = oracle.local_attend(qk, v, w.chunk_len, w.look_before, w.look_after,
                                         w.causal, w.self_mask)
    err = check(host(loc.y), host(loc.lse), y_ref, lse_ref, v, TOL[w.dtype], name)
    say(f"[local] {name}: y max abs err {err:.3g}")


def test_local_one_back_matches_the_lsh_path_without_hashing(B):
    """before = 1, after = 0 is LSH attention with one bucket and one round:
    both GPU paths agree with each other and with the oracle."""
    w = local_workload("l_lsh", 1, 4, 2048, 1, 0, True, True, "bf16", 40)
    inp = synth.make_inputs(w)
    loc = run_local(B, w, inp)
    cfg = B.config_for(w)
    f = B.Forward(cfg)
    f.run(B.to_device(inp["qk"], w.dtype), B.to_device(inp["v"], w.dtype), None)
    torch.cuda.synchronize()
    assert np.abs(host(loc.y) - host(f.y)).max() <= 2e-2
    assert np.array_equal(np.isneginf(host(loc.lse)), np.isneginf(host(f.lse)[:, :, 0]))


def test_local_long_full_size_sampled(B):
    """The benchmark shape (8 heads x 65,536 tokens, one chunk each side) at
    full size: sampled rows against the oracle, y finite everywhere."""
    w = synth.WORKLOADS["local_long"]
    say(f"[local-full] {w}")
    inp = synth.make_inputs(w)
    loc = run_local(B, w, inp)
    y = host(loc.y)
    assert np.isfinite(y).all()
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    idx = np.random.default_rng(41).integers(0, w.batch * w.heads * w.seq_len, 3000)
    idx = np.concatenate([idx, [0, w.seq_len - 1, w.seq_len, 7 * w.seq_len + 63]])
    y_ref, lse_ref = oracle.local_attend_rows(qk, v, w.chunk_len, w.look_before, w.look_after,
                                              w.causal, w.self_mask, idx)
    check(y.reshape(-1, 64)[idx], host(loc.lse).ravel()[idx], y_ref, lse_ref,
          v.reshape(-1, 64)[idx], TOL[w.dtype], "local_long")
    say("[local-full] local_long: 3004 sampled rows within tolerance")


def test_local_repeat_runs_are_bitwise_identical(B):
    w = local_workload("l_rep", 1, 2, 4096, 2, 1, False, True, "bf16", 42)
    inp = synth.make_inputs(w)
    a = run_local(B, w, inp)
    b = run_local(B, w, inp)
    assert np.array_equal(host(a.y), host(b.y))
    assert np.array_equal(host(a.lse), host(b.lse))
