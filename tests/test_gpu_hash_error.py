"""The matrix-core error model behind the exact bucket hash, measured.

The bucket of a token is the first maximum of [x R ; -x R] with x R an exact
sum (Reformer study note, section "LSH Attention").  The library scores x R on
the bf16 matrix cores with fp32 accumulation and accepts a row without an fp64
recomputation only when the gap between its two best |scores| exceeds 2E, with
E = 64 * 2^-22 * 1.01 * |x| * max_j |R_j| (twice the bound of 64 additions
that each round once by at most one ulp).  Two checks:

* the probe kernel (tests/mfma_probe, same instruction, operand layout and
  accumulation order as the hash) scores more than 10^7 dot products from five
  input families, including heavy cancellation and wide exponent ranges; the
  largest |MFMA - exact| / (64 * 2^-23 * sum_k |x_k R_kj|) must stay below the
  factor 2 the certification allows;
* the hash recomputes the four scores of a row's winning quad of directions
  with chains of v_dot2_f32_bf16 and bounds the other three by those values,
  so the same ratio for the probe's copy of that computation must stay below
  2 too;
* rows built so that their exact top-two gap lies between 2.3E and 3.7E (the
  certified side of the threshold) or between 0.3E and 1.9E (the settled side),
  with alternating-sign components that cancel heavily, must hash exactly like
  the oracle, and the fallback counter must show that the first group was
  certified and the second settled.
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from lsh_sparse_attention_hash_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE = os.path.join(HERE, "mfma_probe", "libmfma_probe.so")
D = 64
UNIT = 64 * 2.0 ** -23      # one ulp per addition, relative to sum_k |x_k R_kj|


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBE):
        raise RuntimeError(f"{PROBE} is missing: run `python tests/mfma_probe/build.py`")
    lib = ctypes.CDLL(PROBE)
    lib.mfma_probe_scores.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_void_p]
    lib.mfma_probe_scores.restype = ctypes.c_int
    lib.mfma_probe_dots.argtypes = lib.mfma_probe_scores.argtypes
    lib.mfma_probe_dots.restype = ctypes.c_int
    return lib


def bf16(a):
    """float values -> (bf16 bit patterns, their exact float64 values)."""
    bits = synth.bf16_bits(np.asarray(a, np.float32))
    return bits, synth.to_f64(bits, "bf16")


def families(g, n_tok, n_dir):
    sgn = (-1.0) ** np.arange(D)
    z = lambda *s: g.standard_normal(s)
    u = lambda lo, hi, *s: 2.0 ** g.integers(lo, hi + 1, s)
    ramp = np.where(np.arange(D) < D // 2, 1.0, -1.0)
    return {
        "normal": (z(n_tok, D), z(n_dir, D)),
        "alternating_cancel": (sgn * (1 + 0.05 * z(n_tok, D)), 1 + 0.05 * z(n_dir, D)),
        "wide_exponents": (z(n_tok, D) * u(-10, 10, n_tok, D), z(n_dir, D) * u(-10, 10, n_dir, D)),
        "ramp_cancel": (ramp * (1 + 0.01 * z(n_tok, D)), 1 + 0.01 * z(n_dir, D)),
        "wide_alternating": (sgn * u(0, 8, n_tok, D) * (1 + 0.1 * z(n_tok, D)),
                             u(0, 8, n_dir, D) * (1 + 0.1 * z(n_dir, D))),
    }


def test_matrix_core_error_within_the_certification_allowance(probe):
    n_tok, n_dir = 32768, 512
    g = np.random.default_rng(71)
    total, worst = 0, {}
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for name, (xs, rs) in families(g, n_tok, n_dir).items():
        xb, x = bf16(xs)
        rb, r = bf16(rs)
        xd = torch.from_numpy(xb.view(np.int16)).cuda()
        rd = torch.from_numpy(rb.view(np.int16)).cuda()
        exact = x @ r.T                     # products exact; fp64 sum error ~1e-14 relative
        absum = np.abs(x) @ np.abs(r).T
        nz = absum > 0
        for kind, fn in (("mfma", probe.mfma_probe_scores), ("dot2", probe.mfma_probe_dots)):
            out = torch.empty((n_tok, n_dir), dtype=torch.float32, device="cuda")
            rc = fn(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(rd.data_ptr()),
                    ctypes.c_void_p(out.data_ptr()), n_tok, n_dir, stream)
            assert rc == 0
            torch.cuda.synchronize()
            t = out.cpu().numpy().astype(np.float64)
            ratio = np.abs(t - exact)[nz] / (UNIT * absum[nz])
            worst[kind, name] = float(ratio.max())
            if kind == "mfma":
                total += int(nz.sum())
            say(f"[{kind} error] {name}: max |{kind} - exact| / (64 2^-23 sum|x R|) = "
                f"{worst[kind, name]:.4f}, mean {ratio.mean():.2e}, exact "
                f"{np.mean(ratio == 0):.3f} of {nz.sum()} scores")
    assert total >= 10 ** 7
    # the certification allows twice the one-ulp-per-addition bound
    assert max(worst.values()) < 2.0, worst


def _near_threshold_rows(g, rot, lo, hi, n):
    """n bf16 rows x whose exact |x.R_0|, |x.R_1| differ by lo..hi times E."""
    sgn = (-1.0) ** np.arange(D)
    out = []
    while sum(len(o) for o in out) < n:
        _, x = bf16(sgn * (1 + 0.05 * g.standard_normal((1 << 18, D))))
        s = np.abs(x @ rot.T)
        e = 64 * 2.0 ** -22 * 1.01 * np.linalg.norm(x, axis=1) * np.linalg.norm(rot, axis=1).max()
        q = np.abs(s[:, 0] - s[:, 1]) / e
        out.append(x[(q > lo) & (q < hi)])
    return np.concatenate(out)[:n]


# (n_buckets, rows of the two directions): B = 4 runs the key epilogue; with
# B = 4096 (the other rows zero) the quad epilogue, once with both directions
# in one quad (tile 5, quad 2, second lane half: the pair is told apart by the
# recomputation) and once in different quads and tiles
@pytest.mark.parametrize("n_buckets,rows", [(4, (0, 1)), (4096, (180, 181)), (4096, (37, 1000))])
def test_rows_near_the_certification_threshold(probe, n_buckets, rows):
    g = np.random.default_rng(72)
    rbits2, rot2 = bf16(1 + 0.05 * g.standard_normal((2, D)))   # the two directions
    n_cert, n_settle = 512, 256
    x = np.concatenate([_near_threshold_rows(g, rot2, 2.3, 3.7, n_cert),
                        _near_threshold_rows(g, rot2, 0.3, 1.9, n_settle)])
    L = n_cert + n_settle
    assert L % 64 == 0
    half = n_buckets // 2
    rbits = np.zeros((half, D), dtype=rbits2.dtype)
    rot = np.zeros((half, D))
    rbits[list(rows)], rot[list(rows)] = rbits2, rot2
    cancel = (np.abs(x) @ np.abs(rot2).T).min(axis=1) / np.abs(x @ rot2.T).max(axis=1)
    say(f"[near threshold] median cancellation sum|x R| / |x.R| = {np.median(cancel):.0f}")
    w = synth.Workload("threshold", 1, 1, L, D, n_buckets, 1, 64, True, True, "bf16", 73)
    from lsh_sparse_attention_hash_amd import binding as B
    cfg = B.config_for(w)
    qk = torch.from_numpy(synth.bf16_bits(x.astype(np.float32)).view(np.int16)).cuda()
    qk = qk.view(torch.bfloat16).reshape(1, 1, L, D)
    rd = torch.from_numpy(rbits.view(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, half, D)
    buckets = torch.empty((1, 1, 1, L), dtype=torch.int32, device="cuda")
    fallback = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.lsh_hash(cfg, qk, rd, buckets, fallback)
    torch.cuda.synchronize()
    ref = oracle.hash(x.reshape(1, 1, L, D), rot.reshape(1, 1, half, D), n_buckets, 1)
    assert np.array_equal(buckets.cpu().numpy(), ref)
    n_fb = int(fallback.cpu()[0])
    say(f"[near threshold] B={n_buckets}, directions {rows}: {n_cert} rows with gap 2.3E..3.7E, "
        f"{n_settle} with 0.3E..1.9E: {n_fb} settled in fp64")
    # every row under 2E must be settled; the rows above it are certified
    # unless the matrix core erred by a sizeable fraction of E
    assert n_settle <= n_fb <= n_settle + n_cert // 4
