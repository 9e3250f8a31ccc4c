"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bar (from the method's contract): bucket ids, perm and inv_perm bit-exact;
o_rounds, lse and y within max abs error 1e-5 for fp32 inputs and 2e-2 for
bf16 inputs; lse = -inf exactly where the oracle's is.

Small and medium problems are compared element by element in full.  The two
largest workloads run at full size in the launch configuration the benchmark
times; there the oracle checks a seeded sample of rows of every step (the
integer steps are also checked in full where the oracle can afford it), each
step fed with the GPU's own (already verified) inputs.
"""
import os
import sys

import numpy as np
import pytest
import torch

from lsh_sparse_attention_hash_amd import synth
from o_rounds_layout import header, read_o_rounds
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


def run_gpu(B, w, inputs):
    cfg = B.config_for(w)
    qk = B.to_device(inputs["qk"], w.dtype)
    v = B.to_device(inputs["v"], w.dtype)
    rot = B.to_device(inputs["rot"], w.dtype)
    f = B.Forward(cfg)
    f.run(qk, v, rot)
    torch.cuda.synchronize()
    return f


def host(t):
    return t.detach().cpu().numpy()


def assert_close_lse(got, want, tol, what):
    ninf_g, ninf_w = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(ninf_g, ninf_w), f"{what}: -inf pattern differs"
    fin = ~ninf_w
    err = np.abs(got[fin] - want[fin]).max(initial=0.0)
    assert err <= tol, f"{what}: max abs err {err}"


def assert_close(got, want, tol, what):
    err = np.abs(np.asarray(got, np.float64) - want).max(initial=0.0)
    assert err <= tol, f"{what}: max abs err {err} > {tol}"
    return err


def full_parity(B, w):
    say(f"[parity] {w}")
    inp = synth.make_inputs(w)
    f = run_gpu(B, w, inp)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    rot = synth.to_f64(inp["rot"], w.dtype)
    ref = oracle.forward(qk, v, rot, w.n_buckets, w.n_rounds, w.chunk_len, w.causal, w.self_mask)
    tol = TOL[w.dtype]
    assert np.array_equal(host(f.buckets), ref["buckets"]), "buckets differ"
    assert np.array_equal(host(f.perm), ref["perm"]), "perm differs"
    assert np.array_equal(host(f.inv_perm), ref["inv_perm"]), "inv_perm differs"
    assert_close_lse(host(f.lse), ref["lse"], tol, "lse")
    o_gpu = read_o_rounds(host(f.o_rounds), w)
    assert_close(o_gpu, ref["o_rounds"], tol, "o_rounds")
    err = assert_close(host(f.y), ref["y"], tol, "y")
    # the combine step alone, on the GPU's own per-round outputs
    y2 = oracle.combine(o_gpu, host(f.lse), host(f.inv_perm), v)
    assert_close(host(f.y), y2, 1e-5, "combine on identical inputs")
    say(f"[parity] {w.name}: y max abs err {err:.3g}, fallback rows {int(host(f.fallback_rows)[0])}")
    return f


@pytest.mark.parametrize("name", ["tiny", "small", "medium"])
def test_workload_full_parity(B, name):
    full_parity(B, synth.WORKLOADS[name])


EDGE = {
    # ragged hash tile (L = 37 chunks), padded direction tile (B/2 = 19), not causal
    "ragged_noncausal": synth.Workload("ragged", 3, 2, 64 * 37, 64, 38, 3, 64, False, False,
                                       "bf16", 11),
    "ragged_self": synth.Workload("ragged_self", 1, 3, 64 * 37, 64, 38, 2, 64, False, True,
                                  "bf16", 12),
    "single_chunk": synth.Workload("single", 2, 2, 64, 64, 4, 2, 64, True, True, "bf16", 13),
    "no_hashing": synth.Workload("b1", 1, 2, 64 * 9, 64, 1, 2, 64, True, True, "bf16", 14),
    "two_buckets": synth.Workload("b2", 1, 2, 64 * 9, 64, 2, 3, 64, False, True, "bf16", 15),
    "max_buckets": synth.Workload("bmax", 1, 1, 2048, 64, 16384, 1, 64, True, True, "bf16", 16),
    "f32_causal_rounds": synth.Workload("f32r", 2, 2, 64 * 7, 64, 8, 3, 64, True, False,
                                        "f32", 17),
    "clusters": synth.Workload("clusters", 1, 2, 4096, 64, 64, 2, 64, True, True, "bf16", 18,
                               n_clusters=4),
    # largest bucket count whose sort ranks equal keys through LDS masks, and
    # the smallest that uses ballots
    "mask_match_limit": synth.Workload("b2048", 1, 2, 4096, 64, 2048, 2, 64, True, True, "bf16",
                                       23),
    "ballot_match": synth.Workload("b4096", 1, 1, 4096, 64, 4096, 1, 64, False, True, "bf16", 24),
    # round counts that leave padded slots in the combine's unrolled loads
    "rounds5": synth.Workload("r5", 1, 2, 64 * 11, 64, 16, 5, 64, True, True, "bf16", 25),
    "rounds12": synth.Workload("r12", 1, 1, 64 * 6, 64, 8, 12, 64, False, False, "bf16", 26),
    # more rounds than the combine unrolls (the running softmax over rounds);
    # bf16 causal attention without the self-mask
    "rounds20": synth.Workload("r20", 1, 2, 64 * 4, 64, 8, 20, 64, True, False, "bf16", 27),
    "f32_rounds18": synth.Workload("f32r18", 1, 1, 64 * 3, 64, 4, 18, 64, False, True, "f32",
                                   28),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_case_parity(B, name):
    full_parity(B, EDGE[name])



def _perm_variants(perm, buckets, seed):
    """Permutations of each segment that are not the (bucket, position) sort:
    every bucket run reversed, buckets in descending order, and a shuffle."""
    rng = np.random.default_rng(seed)
    L = perm.shape[-1]
    pos = np.arange(L)
    rev, desc, shuf = (np.empty_like(perm) for _ in range(3))
    for idx in np.ndindex(perm.shape[:-1]):
        bk = buckets[idx]
        rev[idx] = np.lexsort((-pos, bk)).astype(np.int32)
        desc[idx] = np.lexsort((pos, -bk)).astype(np.int32)
        shuf[idx] = rng.permutation(L).astype(np.int32)
    return {"runs_reversed": rev, "buckets_descending": desc, "shuffled": shuf}


@pytest.mark.parametrize("name", ["small", "ragged_noncausal", "ragged_self", "clusters",
                                  "rounds20"])
def test_attention_of_any_permutation(B, name):
    """The attention step takes the window of every chunk from the permutation
    it is given; its tile skipping must not assume that permutation to be the
    bucket sort (the oracle applies the masks key by key)."""
    w = EDGE.get(name) or synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    f = run_gpu(B, w, inp)
    qk_d = B.to_device(inp["qk"], w.dtype)
    v_d = B.to_device(inp["v"], w.dtype)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    buckets = host(f.buckets)
    tol = TOL[w.dtype]
    for kind, perm in _perm_variants(host(f.perm), buckets, w.seed).items():
        say(f"[parity] attention of a {kind} permutation, {w}")
        f.perm.copy_(torch.from_numpy(perm))
        f.attend(qk_d, v_d)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.attend(qk, v, buckets, perm, w.n_buckets, w.chunk_len, w.causal,
                                       w.self_mask)
        assert_close_lse(host(f.lse), lse_ref, tol, f"lse ({kind})")
        assert_close(read_o_rounds(host(f.o_rounds), w), o_ref, tol, f"o_rounds ({kind})")

def test_empty_problem_is_a_no_op(B):
    w = synth.Workload("empty", 1, 2, 0, 64, 8, 2, 64, True, True, "bf16", 19)
    cfg = B.config_for(w)
    z = torch.zeros(0, device="cuda")
    lib = B.library()
    import ctypes
    assert lib.lsh_hash(ctypes.byref(cfg), None, None, None, None, None) == 0
    assert lib.lsh_sort(ctypes.byref(cfg), None, None, None, None, 0, None) == 0
    del z


def test_repeat_runs_are_bitwise_identical(B):
    w = synth.WORKLOADS["small"]
    inp = synth.make_inputs(w)
    a = run_gpu(B, w, inp)
    outs = [host(t).copy() for t in (a.buckets, a.perm, a.inv_perm, a.o_rounds, a.lse, a.y)]
    for _ in range(3):
        b = run_gpu(B, w, inp)
        for x, t in zip(outs, (b.buckets, b.perm, b.inv_perm, b.o_rounds, b.lse, b.y)):
            assert np.array_equal(x, host(t))


def test_per_round_output_scale(B):
    """bf16 inputs store the per-round outputs as fp16 with one power-of-two
    scale per (batch, head): the header's partial maxima give max |v| of each
    (batch, head) exactly, every stored magnitude stays within rounding of
    2^15, and heads whose v are scaled by 2^40, 2^-60, 2^120 or 2^-100 (or are
    all zero) keep the bf16 tolerance relative to that scale."""
    w = synth.Workload("oscale", 2, 4, 1024, 64, 16, 2, 64, True, True, "bf16", 41)
    inp = synth.make_inputs(w)
    v = synth.to_f64(inp["v"], "bf16")
    shift = np.zeros((w.batch, w.heads))
    # moderate scales, and the ends of the bf16 range: k up to 108 and the
    # exponent clamp at -100
    shift[0, 1], shift[1, 2], shift[0, 3], shift[1, 0] = 40, -60, 120, -100
    v = v * 2.0 ** shift[:, :, None, None]
    v[1, 3] = 0.0
    inp = dict(inp, v=synth.bf16_bits(v.astype(np.float32)))
    assert np.array_equal(synth.to_f64(inp["v"], "bf16"), v)   # the scaling was exact
    f = run_gpu(B, w, inp)
    raw = host(f.o_rounds)
    hdr = header(raw, w)
    assert np.array_equal(hdr.max(axis=2).astype(np.float64), np.abs(v).max(axis=(2, 3)))
    from o_rounds_layout import header_bytes
    n = w.batch * w.heads * w.n_rounds * w.seq_len * w.head_dim
    stored = raw[header_bytes(w): header_bytes(w) + 2 * n].view(np.float16)
    assert np.abs(stored.astype(np.float64)).max() <= 2.0 ** 15 * (1 + 2.0 ** -10)
    ref = oracle.forward(synth.to_f64(inp["qk"], "bf16"), v, synth.to_f64(inp["rot"], "bf16"),
                         w.n_buckets, w.n_rounds, w.chunk_len, w.causal, w.self_mask)
    assert np.array_equal(host(f.buckets), ref["buckets"])
    unit = 2.0 ** shift[:, :, None, None]
    o = read_o_rounds(raw, w).astype(np.float64)
    assert np.abs((o - ref["o_rounds"]) / unit[:, :, None]).max() <= TOL["bf16"]
    assert np.abs((host(f.y) - ref["y"]) / unit).max() <= TOL["bf16"]
    assert not host(f.y)[1, 3].any()


@pytest.mark.parametrize("log2_scale", [30, -60])
def test_scaled_inputs_parity(B, log2_scale):
    """qk scaled by a power of two (exact in bf16): very large scores, and
    scores so small that fp32 sums approach the denormal range (those rows
    must be settled in fp64).  Buckets are scale-invariant."""
    w = synth.Workload(f"scaled{log2_scale}", 1, 2, 2048, 64, 64, 2, 64, True, True, "bf16",
                       24 + abs(log2_scale))
    inp = synth.make_inputs(w)
    scaled = synth.to_f64(inp["qk"], "bf16") * 2.0 ** log2_scale
    inp = dict(inp, qk=synth.bf16_bits(scaled.astype(np.float32)))
    assert np.array_equal(synth.to_f64(inp["qk"], "bf16"), scaled)   # the scaling was exact
    f = run_gpu(B, w, inp)
    ref = oracle.forward(scaled, synth.to_f64(inp["v"], "bf16"), synth.to_f64(inp["rot"], "bf16"),
                         w.n_buckets, w.n_rounds, w.chunk_len, w.causal, w.self_mask)
    assert np.array_equal(host(f.buckets), ref["buckets"])
    assert_close_lse(host(f.lse), ref["lse"], 2e-2 * max(1.0, 2.0 ** log2_scale), "lse")
    assert_close(host(f.y), ref["y"], 2e-2, "y")
    say(f"[scaled 2^{log2_scale}] fallback rows {int(host(f.fallback_rows)[0])}")


def test_hash_matches_exactly_on_skewed_and_tied_inputs(B):
    """Integer-valued bf16 inputs produce exact ties; zero rows tie everywhere."""
    w = synth.Workload("ties", 1, 2, 1024, 64, 64, 2, 64, True, True, "bf16", 20)
    g = np.random.default_rng(21)
    qk = g.integers(-2, 3, size=(1, 2, 1024, 64)).astype(np.float32)
    qk[0, 0, :10] = 0.0
    rot = g.integers(-1, 2, size=(2, 2, 32, 64)).astype(np.float32)
    inp = {"qk": synth.bf16_bits(qk), "v": synth.bf16_bits(g.standard_normal(qk.shape)),
           "rot": synth.bf16_bits(rot)}
    f = run_gpu(B, w, inp)
    ref = oracle.hash(synth.to_f64(inp["qk"], "bf16"), synth.to_f64(inp["rot"], "bf16"), 64, 2)
    assert np.array_equal(host(f.buckets), ref)
    assert int(host(f.fallback_rows)[0]) > 0   # ties can only be settled by the fp64 path


def test_hash_settles_more_uncertain_rows_than_one_list_holds(B):
    """A workgroup of 256 tokens whose rows are all uncertain (zero vectors
    tie everywhere) over 8 rounds lists 2048 rows, more than its LDS list
    holds: the rows that do not fit are found again and settled.  The second
    workgroup's 64 tokens (L = 320) carry integer ties."""
    w = synth.Workload("overflow", 1, 1, 320, 64, 32, 8, 64, True, True, "bf16", 22)
    g = np.random.default_rng(23)
    qk = g.integers(-1, 2, size=(1, 1, 320, 64)).astype(np.float32)
    qk[0, 0, :256] = 0.0
    rot = g.integers(-1, 2, size=(1, 8, 16, 64)).astype(np.float32)
    inp = {"qk": synth.bf16_bits(qk), "v": synth.bf16_bits(g.standard_normal(qk.shape)),
           "rot": synth.bf16_bits(rot)}
    f = run_gpu(B, w, inp)
    ref = oracle.hash(synth.to_f64(inp["qk"], "bf16"), synth.to_f64(inp["rot"], "bf16"), 32, 8)
    assert np.array_equal(host(f.buckets), ref)
    assert (ref[0, 0, :, :256] == 0).all()   # all-zero rows take the first index
    assert int(host(f.fallback_rows)[0]) >= 256 * 8


# --------------------------------------------------------------- full size
def sampled_parity(B, w, n_hash, n_rows, seed):
    say(f"[parity-full] {w}")
    inp = synth.make_inputs(w)
    f = run_gpu(B, w, inp)
    tol = TOL[w.dtype]
    g = np.random.default_rng(seed)
    qk = synth.to_f64(inp["qk"], w.dtype)
    rot = synth.to_f64(inp["rot"], w.dtype)
    bk = host(f.buckets)
    idx = g.integers(0, bk.size, n_hash)
    ref_b = oracle.hash_rows(qk, rot, w.n_buckets, w.n_rounds, idx)
    assert np.array_equal(bk.ravel()[idx], ref_b), "sampled buckets differ"
    say(f"[parity-full] {w.name}: {n_hash} sampled buckets exact")
    perm, inv = oracle.sort(bk)
    assert np.array_equal(host(f.perm), perm), "perm differs"
    assert np.array_equal(host(f.inv_perm), inv), "inv_perm differs"
    say(f"[parity-full] {w.name}: perm / inv_perm exact")
    v = synth.to_f64(inp["v"], w.dtype)
    rows = g.integers(0, bk.size, n_rows)
    o_ref, lse_ref = oracle.attend_rows(qk, v, bk, perm, w.n_buckets, w.chunk_len, w.causal,
                                        w.self_mask, rows)
    lse = host(f.lse).ravel()[rows]
    assert_close_lse(lse, lse_ref, tol, "lse")
    o_all = read_o_rounds(host(f.o_rounds), w)
    o = o_all.reshape(-1, w.head_dim)[rows]
    err_o = assert_close(o, o_ref, tol, "o_rounds")
    toks = g.integers(0, w.batch * w.heads * w.seq_len, n_rows)
    y_ref = oracle.combine_rows(o_all, host(f.lse), inv, v, toks)
    y = host(f.y).reshape(-1, w.head_dim)[toks]
    assert_close(y, y_ref, 1e-5, "combine rows")
    say(f"[parity-full] {w.name}: o err {err_o:.3g}, fallback rows {int(host(f.fallback_rows)[0])}")


def test_long_full_size_sampled(B):
    sampled_parity(B, synth.WORKLOADS["long"], n_hash=20000, n_rows=20000, seed=31)


def test_verylong_full_size_sampled(B):
    sampled_parity(B, synth.WORKLOADS["verylong"], n_hash=4000, n_rows=20000, seed=32)


def test_long_end_to_end_rows(B):
    """End to end at full size: y of sampled tokens from the oracle's own
    hash -> sort -> attend -> combine of the heads they belong to (one head's
    oracle work is affordable)."""
    w = synth.WORKLOADS["long"].replace(heads=1)
    inp = synth.make_inputs(synth.WORKLOADS["long"])
    inp = {"qk": inp["qk"][:, :1].copy(), "v": inp["v"][:, :1].copy(),
           "rot": inp["rot"][:1].copy()}
    f = run_gpu(B, w, inp)
    qk = synth.to_f64(inp["qk"], w.dtype)
    v = synth.to_f64(inp["v"], w.dtype)
    rot = synth.to_f64(inp["rot"], w.dtype)
    bk = oracle.hash(qk, rot, w.n_buckets, w.n_rounds)
    assert np.array_equal(host(f.buckets), bk)
    perm, inv = oracle.sort(bk)
    o, lse = oracle.attend(qk, v, bk, perm, w.n_buckets, w.chunk_len, w.causal, w.self_mask)
    toks = np.random.default_rng(33).integers(0, w.seq_len, 4000)
    y_ref = oracle.combine_rows(o, lse, inv, v, toks)
    assert_close(host(f.y).reshape(-1, 64)[toks], y_ref, TOL["bf16"], "y")
