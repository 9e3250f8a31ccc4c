"""GPU parity of the set reading of the union over hash rounds
(lsh_chunk_attend_union + lsh_unsort_combine) against the fp64 oracle.

Bucket ids, perm and inv_perm bit-exact; per-round o_rounds / lse and y
within max abs 1e-5 (fp32 inputs) / 2e-2 (bf16 inputs); lse = -inf exactly
where the oracle's is."""
import sys

import numpy as np
import pytest
import torch

from lsh_sparse_attention_hash_amd import synth
from o_rounds_layout import read_o_rounds
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


def host(t):
    return t.detach().cpu().numpy()


def run_union(B, w, inp):
    f = B.Forward(B.config_for(w))
    f.run(B.to_device(inp["qk"], w.dtype), B.to_device(inp["v"], w.dtype),
          B.to_device(inp["rot"], w.dtype) if w.n_buckets > 1 else None, union=True)
    torch.cuda.synchronize()
    return f


def close(got, want, tol, what):
    ninf = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf pattern differs"
    err = np.abs(np.asarray(got, np.float64)[~ninf] - want[~ninf]).max(initial=0.0)
    assert err <= tol, f"{what}: max abs err {err} > {tol}"
    return err


CASES = {
    "small": synth.Workload("u_small", 2, 4, 4096, 64, 64, 2, 64, True, True, "bf16", 51),
    "many_repeats": synth.Workload("u_rep", 1, 4, 4096, 64, 16, 4, 64, False, True, "bf16", 52),
    "max_rounds": synth.Workload("u_r16", 1, 2, 2048, 64, 8, 16, 64, True, False, "bf16", 53),
    "no_hashing": synth.Workload("u_b1", 1, 2, 1024, 64, 1, 3, 64, True, True, "bf16", 54),
    "f32": synth.Workload("u_f32", 1, 2, 512, 64, 8, 3, 64, True, True, "f32", 55),
    "clusters": synth.Workload("u_cl", 1, 4, 4096, 64, 64, 4, 64, True, True, "bf16", 56,
                               n_clusters=8),
    "ragged": synth.Workload("u_rag", 3, 1, 64 * 21, 64, 10, 3, 64, False, False, "bf16", 57),
    # 5 to 8 rounds: the round-key table's 8-wide variant with padded slots
    "six_rounds": synth.Workload("u_r6", 1, 2, 2048, 64, 16, 6, 64, True, True, "bf16", 59),
    # many buckets: the hash's quad epilogue and the eight-wave sort scatter
    "many_buckets": synth.Workload("u_b4096", 1, 2, 4096, 64, 4096, 3, 64, True, True, "bf16",
                                   64),
    # bf16 inputs with fp32 per-round rows, 8 rounds, no masks: the 8-wide
    # kernel's least common form
    "eight_rounds_f32_rows": synth.Workload("u_r8f", 1, 2, 2048, 64, 16, 8, 64, False, False,
                                            "bf16", 60, o_format="f32"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_union_parity(B, name):
    w = CASES[name]
    say(f"[union] {w}")
    inp = synth.make_inputs(w)
    f = run_union(B, w, inp)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    rot = synth.to_f64(inp["rot"], w.dtype)
    ref = oracle.forward_union(qk, v, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal,
                               w.self_mask)
    assert np.array_equal(host(f.buckets), ref["buckets"])
    assert np.array_equal(host(f.perm), ref["perm"])
    assert np.array_equal(host(f.inv_perm), ref["inv_perm"])
    tol = TOL[w.dtype]
    close(host(f.lse), ref["lse"], tol, "lse")
    close(read_o_rounds(host(f.o_rounds), w), ref["o_rounds"], tol, "o_rounds")
    err = close(host(f.y), ref["y"], tol, "y")
    multi = oracle.forward(qk, v, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal,
                           w.self_mask)
    say(f"[union] {name}: y err {err:.3g}; set vs multiset readings differ by "
        f"{np.abs(ref['y'] - multi['y']).max():.3g}")


def test_union_with_one_round_matches_the_multiset_kernel(B):
    w = synth.Workload("u_r1", 1, 4, 4096, 64, 64, 1, 64, True, True, "bf16", 58)
    inp = synth.make_inputs(w)
    f = run_union(B, w, inp)
    g = B.Forward(B.config_for(w))
    g.run(B.to_device(inp["qk"], w.dtype), B.to_device(inp["v"], w.dtype),
          B.to_device(inp["rot"], w.dtype))
    torch.cuda.synchronize()
    assert np.array_equal(host(f.perm), host(g.perm))
    assert np.abs(host(f.y) - host(g.y)).max() <= 1e-6


def test_union_long_full_size_sampled(B):
    """The headline shape (8 heads x 65,536 tokens, 1,024 buckets, 8 rounds)
    with the set reading: sampled rows of every step against the oracle."""
    w = synth.WORKLOADS["long"]
    say(f"[union-full] {w}")
    inp = synth.make_inputs(w)
    f = run_union(B, w, inp)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    bk, pm, ip = host(f.buckets), host(f.perm), host(f.inv_perm)
    perm, inv = oracle.sort(bk)
    assert np.array_equal(pm, perm) and np.array_equal(ip, inv)
    g = np.random.default_rng(59)
    rows = g.integers(0, bk.size, 2000)
    o_ref, lse_ref = oracle.attend_union_rows(qk, v, bk, pm, ip, w.n_buckets, w.chunk_len,
                                              w.causal, w.self_mask, rows)
    close(host(f.lse).ravel()[rows], lse_ref, 2e-2, "lse")
    o_all = read_o_rounds(host(f.o_rounds), w)
    close(o_all.reshape(-1, 64)[rows], o_ref, 2e-2, "o_rounds")
    toks = g.integers(0, w.batch * w.heads * w.seq_len, 2000)
    y_ref = oracle.combine_rows(o_all, host(f.lse), ip, v, toks)
    assert np.abs(host(f.y).reshape(-1, 64)[toks] - y_ref).max() <= 1e-5
    say("[union-full] long: 2000 sampled rows of o_rounds / lse / y within tolerance")


@pytest.mark.parametrize("name", ["small", "many_repeats", "clusters"])
def test_union_attention_of_any_permutation(B, name):
    """The set-union attention of permutations that are not the bucket sort
    (every bucket run reversed; a shuffle), with inv_perm their inverse,
    matches the oracle: its tile skipping assumes nothing of the order."""
    w = CASES[name]
    inp = synth.make_inputs(w)
    f = run_union(B, w, inp)
    qk_d, v_d = B.to_device(inp["qk"], w.dtype), B.to_device(inp["v"], w.dtype)
    qk, v = synth.to_f64(inp["qk"], w.dtype), synth.to_f64(inp["v"], w.dtype)
    buckets = host(f.buckets)
    L = buckets.shape[-1]
    pos = np.arange(L)
    rng = np.random.default_rng(w.seed)
    tol = TOL[w.dtype]
    for kind in ("runs_reversed", "shuffled"):
        perm = np.empty_like(buckets)
        for idx in np.ndindex(buckets.shape[:-1]):
            perm[idx] = (np.lexsort((-pos, buckets[idx])) if kind == "runs_reversed"
                         else rng.permutation(L))
        inv = np.empty_like(perm)
        np.put_along_axis(inv, perm.astype(np.int64),
                          np.broadcast_to(pos.astype(np.int32), perm.shape), axis=-1)
        say(f"[union] attention of a {kind} permutation, {w}")
        f.perm.copy_(torch.from_numpy(perm))
        f.inv_perm.copy_(torch.from_numpy(inv))
        f.attend_union(qk_d, v_d)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attend_union(qk, v, buckets, perm, inv, w.n_buckets, w.chunk_len,
                                             w.causal, w.self_mask)
        close(host(f.lse), lse_ref, tol, f"lse ({kind})")
        close(read_o_rounds(host(f.o_rounds), w), o_ref, tol, f"o_rounds ({kind})")


def test_union_round_keys_near_2_pow_30(B):
    """Round keys bucket * (C + 1) + chunk reach 2^30 once B * (C + 1) does
    (here B = 16,384 and C + 1 = 65,537 at 4,194,304 tokens).  Buckets are
    given directly: random in round 0, all 16,383 in round 1, so the round-1
    keys of chunks 49,152 and 49,153 are 2^30 - 1 and 2^30.  The stand-in the
    kernel gives the rounds a test skips must not match them: every row of
    those windows in round 1 (and random rows of both rounds) against the
    oracle."""
    L, nb, R = 4194304, 16384, 2
    w = synth.Workload("u_big_keys", 1, 1, L, 64, nb, R, 64, True, True, "bf16", 63,
                       o_format="f32")
    g = np.random.default_rng(64)
    bk = np.empty((1, 1, R, L), np.int32)
    bk[0, 0, 0] = g.integers(0, nb, L, dtype=np.int32)
    bk[0, 0, 1] = nb - 1
    assert (nb - 1) * (L // 64 + 1) + 49153 == 1 << 30
    perm, inv = oracle.sort(bk)
    qk = synth.bf16_bits(g.standard_normal((1, 1, L, 64)).astype(np.float32))
    v = synth.bf16_bits(g.standard_normal((1, 1, L, 64)).astype(np.float32))
    f = B.Forward(B.config_for(w))
    f.buckets.copy_(torch.from_numpy(bk))
    f.perm.copy_(torch.from_numpy(perm))
    f.inv_perm.copy_(torch.from_numpy(inv))
    f.attend_union(B.to_device(qk, "bf16"), B.to_device(v, "bf16"))
    torch.cuda.synchronize()
    crit = L + np.arange(49151 * 64, 49156 * 64)          # round 1, chunks 49,151 .. 49,155
    rows = np.concatenate([crit, g.integers(0, R * L, 1000)])
    o_ref, lse_ref = oracle.attend_union_rows(synth.to_f64(qk, "bf16"), synth.to_f64(v, "bf16"),
                                              bk, perm, inv, nb, 64, True, True, rows)
    idx = torch.from_numpy(rows).cuda()
    o_gpu = host(f.o_rounds[:R * L * 64 * 4].view(torch.float32).view(R * L, 64)[idx])
    lse_gpu = host(f.lse.view(-1)[idx])
    close(lse_gpu, lse_ref, 2e-2, "lse")
    close(o_gpu, o_ref, 2e-2, "o_rounds")
    # the round-1 windows of those chunks keep their keys
    assert np.isfinite(lse_gpu[64:len(crit)]).all()
    say("[union] round keys at 2^30: 1,320 rows of o_rounds / lse within tolerance")
