"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expectation is a closed
form, a hand-worked fixture (tests/golden), an identity of the method, a
textbook special case (dense softmax attention, banded local attention) or a
brute-force enumeration written independently in NumPy below.

Passages (Reformer study note, eightmm.github.io/papers/architectures/reformer,
unless noted):
  "LSH Attention"          h(x) in {1..B}; N_LSH(i) = {j : h(q_i) = h(k_j)};
                           y_i = sum_{j in N(i)} softmax_j(q_i.k_j / sqrt(d_k)) v_j
  "Question"               dense attention A = Q K^T / sqrt(d_k)
  "Shared Query-Key Space" Q = K
  "Sorting and Chunking"   hash -> sort -> bucket-contiguous -> chunked attention
  "Multiple Hash Rounds"   N(i) = union over rounds of N^(r)(i)
  "Implementation Reading" causal masking must survive the sort; same-token policy
  yomu.fyi summary, "Takeaways": local attention over chunks with overlap
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


# ----------------------------------------------------------- brute force
def np_scores(x, d):
    """s[i, j] = x_i . x_j / (max(|x_j|, eps) sqrt(d)) (all pairs)."""
    n = np.maximum(np.sqrt((x * x).sum(-1)), EPS)
    return (x @ x.T) / n[None, :] / math.sqrt(d)


def np_masked_softmax_attention(x, v, allowed):
    """Row-wise softmax attention over the boolean matrix `allowed`;
    rows with no allowed key return (v_i, -inf)."""
    L, d = x.shape
    s = np_scores(x, d)
    y = np.empty_like(v)
    lse = np.empty(L)
    for i in range(L):
        idx = np.nonzero(allowed[i])[0]
        if idx.size == 0:
            y[i] = v[i]
            lse[i] = -np.inf
            continue
        si = s[i, idx]
        m = si.max()
        w = np.exp(si - m)
        lse[i] = m + math.log(w.sum())
        y[i] = (w / w.sum()) @ v[idx]
    return y, lse


def dense_allowed(L, causal, self_mask):
    a = np.ones((L, L), bool)
    if causal:
        a &= np.tril(np.ones((L, L), bool))
    if self_mask:
        a &= ~np.eye(L, dtype=bool)
    return a


def rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------ the hash
def test_hash_closed_form_fixture():
    g = json.load(open(os.path.join(GOLDEN, "hash_closed_form.json")))
    xs = np.array([c["x"] for c in g["cases"]], np.float64)
    rot = np.array(g["rot"], np.float64)[None, None]          # [H=1][R=1][2][2]
    bk = oracle.hash(xs[None, None], rot, 4, 1)[0, 0, 0]
    assert bk.tolist() == [c["bucket"] for c in g["cases"]]
    # the fixture's own candidate vectors agree with x R (stated by hand)
    for c in g["cases"]:
        assert c["c"] == pytest.approx(list(np.concatenate([c["x"], -np.array(c["x"])])))


def test_hash_integer_inputs_brute_force():
    """Small-integer inputs make every dot product exact in any order, so the
    first maximum of [xR; -xR] is fixed exactly (many ties included)."""
    g = np.random.default_rng(7)
    H, R, L, d, B = 2, 3, 257, 64, 16
    x = g.integers(-3, 4, size=(1, H, L, d)).astype(np.float64)
    rot = g.integers(-2, 3, size=(H, R, B // 2, d)).astype(np.float64)
    got = oracle.hash(x, rot, B, R)
    xi = x.astype(np.int64)
    ri = rot.astype(np.int64)
    for h in range(H):
        for r in range(R):
            s = xi[0, h] @ ri[h, r].T                        # exact integers [L][B/2]
            c = np.concatenate([s, -s], axis=1)
            assert np.array_equal(got[0, h, r], np.argmax(c, axis=1))  # first max
    # ties really occur in this case (the tie rule is exercised)
    s = xi[0, 0] @ ri[0, 0].T
    c = np.concatenate([s, -s], axis=1)
    assert ((c == c.max(1, keepdims=True)).sum(1) > 1).any()


def test_hash_b1_is_zero_and_b2_is_sign():
    x = rand(1, 1, 2, 100, 8)
    assert (oracle.hash(x, np.zeros((2, 3, 0, 8)), 1, 3) == 0).all()
    rot = rand(2, 2, 1, 1, 8)
    bk = oracle.hash(x, rot, 2, 1)
    s = np.einsum("bhld,hjd->bhlj", x, rot[:, 0])[..., 0]
    assert np.array_equal(bk[:, :, 0], np.where(s >= 0, 0, 1))


def test_hash_random_matches_matmul_argmax():
    x = rand(3, 2, 2, 300, 64)
    rot = rand(4, 2, 2, 32, 64)
    bk = oracle.hash(x, rot, 64, 2)
    s = np.einsum("bhld,hrjd->bhrlj", x, rot)
    ref = np.argmax(np.concatenate([s, -s], -1), -1)
    assert np.array_equal(bk, ref)


def test_hash_negation_and_scaling_identities():
    x = rand(5, 1, 2, 500, 64)
    rot = rand(6, 2, 3, 16, 64)
    B = 32
    bk = oracle.hash(x, rot, B, 3)
    assert np.array_equal(oracle.hash(-x, rot, B, 3), (bk + B // 2) % B)
    for k in (-7, -1, 1, 3, 20):
        assert np.array_equal(oracle.hash(x * 2.0 ** k, rot, B, 3), bk)


def test_hash_direction_permutation_relabels():
    x = rand(8, 1, 1, 400, 64)
    rot = rand(9, 1, 1, 16, 64)
    B = 32
    p = np.random.default_rng(10).permutation(16)
    bk = oracle.hash(x, rot, B, 1)
    bk2 = oracle.hash(x, rot[:, :, p], B, 1)
    inv = np.argsort(p)                       # new row inv[j] holds old direction j
    lab = np.concatenate([inv, inv + 16])
    assert np.array_equal(bk2, lab[bk])


def test_hash_rows_matches_full():
    x = rand(11, 2, 2, 128, 64)
    rot = rand(12, 2, 2, 8, 64)
    full = oracle.hash(x, rot, 16, 2)
    idx = np.random.default_rng(13).integers(0, full.size, 300)
    assert np.array_equal(oracle.hash_rows(x, rot, 16, 2, idx), full.ravel()[idx])


# ------------------------------------------------------------- the sort
def test_sort_is_the_bucket_position_order():
    g = np.random.default_rng(14)
    L = 999
    bk = np.stack([g.integers(0, 7, L), np.minimum(g.geometric(0.3, L), 40), np.zeros(L, int),
                   np.arange(L)[::-1] % 5]).astype(np.int32).reshape(1, 2, 2, L)
    perm, inv = oracle.sort(bk)
    for s in range(4):
        b = bk.reshape(4, L)[s]
        p = perm.reshape(4, L)[s]
        q = inv.reshape(4, L)[s]
        assert p.tolist() == sorted(range(L), key=lambda i: (b[i], i))
        assert np.array_equal(q[p], np.arange(L))
        assert np.array_equal(np.sort(p), np.arange(L))


# ------------------------------------------------ dense special case (B=1, m=L)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("self_mask", [False, True])
@pytest.mark.parametrize("rounds", [1, 3])
def test_b1_one_chunk_is_dense_attention(causal, self_mask, rounds):
    L, d = 96, 64
    x = rand(20, 1, 2, L, d)
    v = rand(21, 1, 2, L, d)
    out = oracle.forward(x, v, np.zeros((2, rounds, 0, d)), 1, rounds, L, causal, self_mask)
    for h in range(2):
        y, lse = np_masked_softmax_attention(x[0, h], v[0, h], dense_allowed(L, causal, self_mask))
        np.testing.assert_allclose(out["y"][0, h], y, rtol=0, atol=1e-12)
        assert np.array_equal(out["perm"][0, h], np.tile(np.arange(L), (rounds, 1)))
        np.testing.assert_allclose(out["lse"][0, h, 0], lse, rtol=0, atol=1e-12)


def test_softmax_two_keys_fixture():
    g = json.load(open(os.path.join(GOLDEN, "softmax_two_keys.json")))
    x = np.array(g["x"])[None, None]
    v = np.array(g["v"])[None, None]
    out = oracle.forward(x, v, np.zeros((1, 1, 0, 4)), 1, 1, 3, False, True)
    env = {"e": math.e, "sqrt": math.sqrt, "log": math.log}
    y = np.array([[eval(e, {}, env) for e in row] for row in g["y_expr"]])
    lse = np.array([eval(e, {}, env) for e in g["lse_expr"]])
    np.testing.assert_allclose(out["y"][0, 0], y, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["lse"][0, 0, 0], lse, rtol=0, atol=1e-15)


# -------------------------------------- local attention (B=1, m=64 < L)
@pytest.mark.parametrize("causal", [False, True])
def test_b1_chunked_is_banded_local_attention(causal):
    L, d, m = 320, 64, 64
    x = rand(22, 1, 1, L, d)
    v = rand(23, 1, 1, L, d)
    out = oracle.forward(x, v, np.zeros((1, 1, 0, d)), 1, 1, m, causal, True)
    assert np.array_equal(out["perm"][0, 0, 0], np.arange(L))
    ci = np.arange(L) // m
    allowed = (ci[None, :] <= ci[:, None]) & (ci[None, :] >= ci[:, None] - 1)
    allowed &= dense_allowed(L, causal, True)
    y, lse = np_masked_softmax_attention(x[0, 0], v[0, 0], allowed)
    np.testing.assert_allclose(out["y"][0, 0], y, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"][0, 0, 0], lse, rtol=0, atol=1e-12)


# ----------------------------- exact-bucket special case (m = L, any B)
@pytest.mark.parametrize("causal", [False, True])
def test_one_chunk_is_exact_bucket_attention(causal):
    L, d, B, R = 128, 64, 8, 2
    x = rand(24, 1, 1, L, d)
    v = rand(25, 1, 1, L, d)
    rot = rand(26, 1, R, B // 2, d)
    out = oracle.forward(x, v, rot, B, R, L, causal, True)
    for r in range(R):
        bk = out["buckets"][0, 0, r]
        allowed = (bk[:, None] == bk[None, :]) & dense_allowed(L, causal, True)
        _, lse = np_masked_softmax_attention(x[0, 0], v[0, 0], allowed)
        # per-round outputs are in sorted order: map back with perm
        p = out["perm"][0, 0, r]
        np.testing.assert_allclose(out["lse"][0, 0, r], lse[p], rtol=0, atol=1e-12)
        o_nat = np.empty((L, d))
        o_nat[p] = out["o_rounds"][0, 0, r]
        y_r, _ = np_masked_softmax_attention(x[0, 0], v[0, 0], allowed)
        empty = ~allowed.any(1)
        np.testing.assert_allclose(o_nat[~empty], y_r[~empty], rtol=0, atol=1e-12)
        assert (o_nat[empty] == 0).all()


# -------------------------------------------------------- the window rule
@pytest.mark.parametrize("causal,self_mask", [(False, False), (False, True), (True, True),
                                              (True, False)])
def test_candidates_follow_the_window_rule(causal, self_mask):
    L, d, B, R, m = 192, 16, 8, 2, 32
    x = rand(27, 2, 1, L, d)
    rot = rand(28, 1, R, B // 2, d)
    bk = oracle.hash(x, rot, B, R)
    perm, inv = oracle.sort(bk)
    for seg in range(2 * R):
        b, r = seg // R, seg % R
        bkr, invr, pr = bk[b, 0, r], inv[b, 0, r], perm[b, 0, r]
        for slot in range(L):
            i = pr[slot]
            c = slot // m
            want = [j for j in pr  # window order = sorted order
                    if bkr[j] == bkr[i] and c - 1 <= invr[j] // m <= c
                    and (not causal or j <= i) and (not self_mask or j != i)]
            got = oracle.candidates(bk, perm, B, m, causal, self_mask, seg, slot)
            assert got.tolist() == want


def test_only_candidates_influence_a_row():
    """Perturbing v_j moves o_r(i) iff j is a candidate of i in round r."""
    L, d, B, R, m = 128, 16, 4, 1, 32
    x = rand(29, 1, 1, L, d)
    v = rand(30, 1, 1, L, d)
    rot = rand(31, 1, R, B // 2, d)
    bk = oracle.hash(x, rot, B, R)
    perm, _ = oracle.sort(bk)
    o0, _ = oracle.attend(x, v, bk, perm, B, m, True, True)
    for j in (0, 17, 63, 127):
        v2 = v.copy()
        v2[0, 0, j] += 1.0
        o1, _ = oracle.attend(x, v2, bk, perm, B, m, True, True)
        for slot in range(L):
            cand = oracle.candidates(bk, perm, B, m, True, True, 0, slot)
            moved = not np.array_equal(o0[0, 0, 0, slot], o1[0, 0, 0, slot])
            assert moved == (j in cand.tolist())


# ------------------------------------------------------ rounds and combine
def test_identical_rounds_equal_one_round():
    L, d, B, m = 256, 64, 16, 64
    x = rand(32, 1, 2, L, d)
    v = rand(33, 1, 2, L, d)
    rot1 = rand(34, 2, 1, B // 2, d)
    one = oracle.forward(x, v, rot1, B, 1, m, True, True)
    three = oracle.forward(x, v, np.repeat(rot1, 3, axis=1), B, 3, m, True, True)
    np.testing.assert_allclose(three["y"], one["y"], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_combine_is_multiset_softmax(causal):
    """y_i is the softmax over the multiset union of the rounds' candidates."""
    L, d, B, R, m = 192, 32, 8, 3, 32
    x = rand(35, 1, 1, L, d)
    v = rand(36, 1, 1, L, d)
    rot = rand(37, 1, R, B // 2, d)
    out = oracle.forward(x, v, rot, B, R, m, causal, True)
    s = np_scores(x[0, 0], d)
    for i in range(L):
        js = []
        for r in range(R):
            seg = r
            slot = out["inv_perm"][0, 0, r, i]
            js += oracle.candidates(out["buckets"], out["perm"], B, m, causal, True, seg,
                                    slot).tolist()
        if not js:
            np.testing.assert_array_equal(out["y"][0, 0, i], v[0, 0, i])
            continue
        js = np.array(js)
        w = np.exp(s[i, js] - s[i, js].max())
        np.testing.assert_allclose(out["y"][0, 0, i], (w / w.sum()) @ v[0, 0, js], rtol=0,
                                   atol=1e-12)


def test_causal_future_values_never_reach_the_past():
    L, d, B, R, m = 256, 64, 16, 2, 64
    x = rand(38, 1, 1, L, d)
    v = rand(39, 1, 1, L, d)
    rot = rand(40, 1, R, B // 2, d)
    base = oracle.forward(x, v, rot, B, R, m, True, True)["y"]
    for j in (1, 100, 255):
        v2 = v.copy()
        v2[0, 0, j:] = rand(41 + j, L - j, d)
        y2 = oracle.forward(x, v2, rot, B, R, m, True, True)["y"]
        assert np.array_equal(y2[0, 0, :j], base[0, 0, :j])


def test_self_only_token_returns_its_value():
    L, d, B, R, m = 128, 64, 8, 2, 64
    x = rand(42, 1, 1, L, d)
    v = rand(43, 1, 1, L, d)
    out = oracle.forward(x, v, rand(44, 1, R, B // 2, d), B, R, m, True, True)
    # position 0 under a causal self-masked rule has no candidate in any round
    assert (out["lse"][0, 0, np.arange(R), out["inv_perm"][0, 0, :, 0]] == -np.inf).all()
    assert np.array_equal(out["y"][0, 0, 0], v[0, 0, 0])


def test_empty_rounds_have_minus_inf_and_zero_output():
    L, d, B, R, m = 128, 16, 64, 2, 64
    x = rand(45, 1, 1, L, d)
    v = rand(46, 1, 1, L, d)
    out = oracle.forward(x, v, rand(47, 1, R, B // 2, d), B, R, m, False, True)
    lse, o = out["lse"][0, 0], out["o_rounds"][0, 0]
    empty = lse == -np.inf
    assert empty.any() and (~empty).any()
    for r in range(R):
        for slot in range(L):
            n = oracle.candidates(out["buckets"], out["perm"], B, m, False, True, r, slot).size
            assert (n == 0) == empty[r, slot]
    assert (o[empty] == 0).all()


def test_rows_variants_match_full():
    L, d, B, R, m = 256, 64, 16, 2, 64
    x = rand(48, 2, 2, L, d)
    v = rand(49, 2, 2, L, d)
    out = oracle.forward(x, v, rand(50, 2, R, B // 2, d), B, R, m, True, True)
    g = np.random.default_rng(51)
    idx = g.integers(0, out["lse"].size, 200)
    o, lse = oracle.attend_rows(x, v, out["buckets"], out["perm"], B, m, True, True, idx)
    np.testing.assert_array_equal(lse, out["lse"].ravel()[idx])
    np.testing.assert_array_equal(o, out["o_rounds"].reshape(-1, d)[idx])
    idx = g.integers(0, 2 * 2 * L, 200)
    y = oracle.combine_rows(out["o_rounds"], out["lse"], out["inv_perm"], v, idx)
    np.testing.assert_array_equal(y, out["y"].reshape(-1, d)[idx])


def test_invalid_arguments_raise():
    x = rand(52, 1, 1, 100, 8)
    with pytest.raises(ValueError):
        oracle.forward(x, x, np.zeros((1, 1, 1, 8)), 3, 1, 10, False, False)   # odd B
    with pytest.raises(ValueError):
        oracle.forward(x, x, np.zeros((1, 1, 0, 8)), 1, 1, 64, False, False)   # L % m


# ------------------------------------------------ local chunked attention
# yomu.fyi summary ("The Reformer - Pushing the limits of language modeling"),
# "Approach / What changed" and "Takeaways": chunks of length l_c that also
# see a configurable number of preceding and following chunks.
def local_allowed(L, m, before, after, causal, self_mask):
    ci = np.arange(L) // m
    a = (ci[None, :] >= ci[:, None] - before) & (ci[None, :] <= ci[:, None] + after)
    return a & dense_allowed(L, causal, self_mask)


@pytest.mark.parametrize("before,after,causal,self_mask", [
    (1, 1, False, True), (2, 0, True, True), (0, 2, False, False), (0, 0, True, False),
    (3, 1, True, True), (1, 4, False, True)])
def test_local_attention_is_banded_attention(before, after, causal, self_mask):
    L, d, m = 384, 64, 64
    x = rand(60, 2, 1, L, d)
    v = rand(61, 2, 1, L, d)
    y, lse = oracle.local_attend(x, v, m, before, after, causal, self_mask)
    allowed = local_allowed(L, m, before, after, causal, self_mask)
    for b in range(2):
        yb, lb = np_masked_softmax_attention(x[b, 0], v[b, 0], allowed)
        np.testing.assert_allclose(y[b, 0], yb, rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(lse[b, 0]), np.isneginf(lb))
        fin = ~np.isneginf(lb)
        np.testing.assert_allclose(lse[b, 0][fin], lb[fin], rtol=0, atol=1e-12)


def test_local_whole_window_is_dense_attention():
    """A window wider than the sequence is plain softmax attention (textbook
    form: softmax(Q K^T / sqrt(d)) V with Q = X, K = unit-length rows of X)."""
    L, d, m = 256, 64, 64
    x = rand(62, 1, 1, L, d)
    v = rand(63, 1, 1, L, d)
    y, lse = oracle.local_attend(x, v, m, 7, 9, False, False)
    k = x[0, 0] / np.linalg.norm(x[0, 0], axis=1, keepdims=True)
    a = x[0, 0] @ k.T / math.sqrt(d)
    p = np.exp(a - a.max(axis=1, keepdims=True))
    np.testing.assert_allclose(y[0, 0], (p / p.sum(1, keepdims=True)) @ v[0, 0], rtol=0, atol=1e-12)
    ref_lse = a.max(1) + np.log(p.sum(1))
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=0, atol=1e-12)


def test_local_one_chunk_back_is_lsh_without_hashing():
    """before = 1, after = 0 is the LSH path with one bucket and one round."""
    L, d, m = 320, 64, 64
    x = rand(64, 1, 2, L, d)
    v = rand(65, 1, 2, L, d)
    for causal in (False, True):
        y, lse = oracle.local_attend(x, v, m, 1, 0, causal, True)
        out = oracle.forward(x, v, np.zeros((2, 1, 0, d)), 1, 1, m, causal, True)
        np.testing.assert_array_equal(y, out["y"])
        np.testing.assert_array_equal(lse, out["lse"][:, :, 0])


def test_local_single_neighbour_closed_forms():
    """With chunks of one token and the self-mask, a token sees exactly one
    other token: y_i is that token's value and lse_i its single score."""
    L, d = 40, 64
    x = rand(66, 1, 1, L, d)
    v = rand(67, 1, 1, L, d)
    X, V = x[0, 0], v[0, 0]

    def score(i, j):
        return float(X[i] @ X[j]) / (math.sqrt(float(X[j] @ X[j])) * 8.0)

    y, lse = oracle.local_attend(x, v, 1, 1, 0, True, True)       # previous token only
    assert np.array_equal(y[0, 0, 0], V[0]) and lse[0, 0, 0] == -np.inf
    np.testing.assert_array_equal(y[0, 0, 1:], V[:-1])
    np.testing.assert_allclose(lse[0, 0, 1:], [score(i, i - 1) for i in range(1, L)],
                               rtol=0, atol=1e-13)
    y, lse = oracle.local_attend(x, v, 1, 0, 1, False, True)      # next token only
    np.testing.assert_array_equal(y[0, 0, :-1], V[1:])
    assert np.array_equal(y[0, 0, -1], V[-1]) and lse[0, 0, -1] == -np.inf
    y, lse = oracle.local_attend(x, v, 2, 0, 0, False, True)      # chunk partner only
    partner = np.arange(L) ^ 1
    np.testing.assert_array_equal(y[0, 0], V[partner])
    np.testing.assert_allclose(lse[0, 0], [score(i, partner[i]) for i in range(L)],
                               rtol=0, atol=1e-13)


def test_local_rows_match_full_and_bad_arguments_raise():
    L, d, m = 256, 64, 64
    x = rand(68, 2, 2, L, d)
    v = rand(69, 2, 2, L, d)
    y, lse = oracle.local_attend(x, v, m, 1, 2, True, True)
    idx = np.random.default_rng(70).integers(0, 4 * L, 300)
    yr, lr = oracle.local_attend_rows(x, v, m, 1, 2, True, True, idx)
    np.testing.assert_array_equal(yr, y.reshape(-1, d)[idx])
    np.testing.assert_array_equal(lr, lse.ravel()[idx])
    with pytest.raises(ValueError):
        oracle.local_attend(x, v, m, -1, 0, False, False)
    with pytest.raises(ValueError):
        oracle.local_attend(x, v, 100, 1, 0, False, False)   # L % l_c != 0


# ------------------------------------------------- set union over rounds
# Reformer study note, "Multiple Hash Rounds": N(i) is the union over rounds
# of the per-round neighbourhoods.  The set reading counts every key once.
def np_round_candidates(buckets, perm, L, m, causal, self_mask):
    """allowed[r][i][j]: j is a candidate of i in round r (dense, from the
    definition: same bucket, j's sorted slot in the window of i's chunk)."""
    R = buckets.shape[0]
    out = np.zeros((R, L, L), bool)
    for r in range(R):
        slot = np.empty(L, int)
        slot[perm[r]] = np.arange(L)
        c = slot // m
        first = np.maximum(c - 1, 0) * m
        last = (c + 1) * m
        win = (slot[None, :] >= first[:, None]) & (slot[None, :] < last[:, None])
        out[r] = win & (buckets[r][:, None] == buckets[r][None, :])
    return out & dense_allowed(L, causal, self_mask)[None]


@pytest.mark.parametrize("causal,self_mask,B,R", [(True, True, 8, 3), (False, True, 4, 4),
                                                  (True, False, 16, 2), (False, False, 2, 5)])
def test_union_is_softmax_over_the_set_of_candidates(causal, self_mask, B, R):
    L, d, m = 256, 64, 64
    x = rand(80 + R, 1, 2, L, d)
    v = rand(81 + R, 1, 2, L, d)
    rot = rand(82 + R, 2, R, B // 2, d)
    out = oracle.forward_union(x, v, rot, B, R, m, causal, self_mask)
    multi = oracle.forward(x, v, rot, B, R, m, causal, self_mask)
    repeats = 0
    for h in range(2):
        cand = np_round_candidates(out["buckets"][0, h], out["perm"][0, h], L, m, causal,
                                   self_mask)
        repeats += int((cand.sum(0) > 1).sum())
        y, lse = np_masked_softmax_attention(x[0, h], v[0, h], cand.any(0))
        np.testing.assert_allclose(out["y"][0, h], y, rtol=0, atol=1e-12)
    assert repeats > 0                                   # the two readings differ here
    assert np.abs(out["y"] - multi["y"]).max() > 1e-3


def test_union_with_one_round_is_the_multiset_path():
    L, d, m = 320, 64, 64
    x = rand(90, 2, 1, L, d)
    v = rand(91, 2, 1, L, d)
    rot = rand(92, 1, 1, 8, d)
    out = oracle.forward_union(x, v, rot, 16, 1, m, True, True)
    multi = oracle.forward(x, v, rot, 16, 1, m, True, True)
    np.testing.assert_array_equal(out["o_rounds"], multi["o_rounds"])
    np.testing.assert_array_equal(out["lse"], multi["lse"])


def test_union_of_identical_rounds_is_one_round():
    """R copies of one rotation: every key of the union is found in round 0,
    so round 0's outputs are the one-round outputs, the later rounds keep no
    key (lse = -inf, o = 0) and y is one round's."""
    L, d, m = 256, 64, 64
    x = rand(93, 1, 1, L, d)
    v = rand(94, 1, 1, L, d)
    one = rand(95, 1, 1, 8, d)
    out = oracle.forward_union(x, v, np.repeat(one, 3, axis=1), 16, 3, m, True, True)
    ref = oracle.forward(x, v, one, 16, 1, m, True, True)
    np.testing.assert_array_equal(out["o_rounds"][:, :, 0], ref["o_rounds"][:, :, 0])
    np.testing.assert_array_equal(out["lse"][:, :, 0], ref["lse"][:, :, 0])
    assert np.isneginf(out["lse"][:, :, 1:]).all()
    assert not out["o_rounds"][:, :, 1:].any()
    np.testing.assert_allclose(out["y"], ref["y"], rtol=0, atol=1e-13)


def test_union_keeps_each_key_in_its_first_round():
    """Per round, the keys kept are the round's candidates that no earlier
    round of the same query has (dense sets from the definition); each round's
    o and lse are the softmax over that set, and the sets partition the union."""
    L, d, m, R, B = 256, 64, 64, 4, 4
    x = rand(100, 1, 1, L, d)
    v = rand(101, 1, 1, L, d)
    rot = rand(102, 1, R, B // 2, d)
    out = oracle.forward_union(x, v, rot, B, R, m, True, True)
    cand = np_round_candidates(out["buckets"][0, 0], out["perm"][0, 0], L, m, True, True)
    seen = np.zeros((L, L), bool)
    dropped = 0
    for r in range(R):
        kept = cand[r] & ~seen
        dropped += int((cand[r] & seen).sum())
        seen |= cand[r]
        o, lse = np_masked_softmax_attention(x[0, 0], v[0, 0], kept)
        fin = ~np.isneginf(lse)
        o[~fin] = 0.0                                    # a round with no key gives o = 0
        slot = out["inv_perm"][0, 0, r]
        np.testing.assert_allclose(out["o_rounds"][0, 0, r][slot], o, rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(out["lse"][0, 0, r][slot]), ~fin)
        np.testing.assert_allclose(out["lse"][0, 0, r][slot][fin], lse[fin], rtol=0, atol=1e-12)
    assert dropped > 0                                   # later rounds do drop keys


def test_union_rows_match_full():
    L, d, m = 256, 64, 64
    x = rand(96, 1, 2, L, d)
    v = rand(97, 1, 2, L, d)
    rot = rand(98, 2, 3, 4, d)
    out = oracle.forward_union(x, v, rot, 8, 3, m, True, True)
    idx = np.random.default_rng(99).integers(0, 2 * 3 * L, 300)
    o, lse = oracle.attend_union_rows(x, v, out["buckets"], out["perm"], out["inv_perm"], 8, m,
                                      True, True, idx)
    np.testing.assert_array_equal(o, out["o_rounds"].reshape(-1, d)[idx])
    np.testing.assert_array_equal(lse, out["lse"].ravel()[idx])
