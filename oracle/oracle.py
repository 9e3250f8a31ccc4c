"""Python front end of the fp64 CPU oracle (``lsh_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the CPU
baseline of the benchmark may import this module; the product path never does.
It shares nothing with the HIP library: the C file is compiled here with gcc
into ``oracle/liblsh_oracle.so`` and called through ctypes with plain numpy
arrays.  Every floating-point input is upcast exactly to float64 before the
call (bf16 and fp32 values are exact in fp64).

What each function computes, and the passage it follows, is stated in the C
file.  Function map:

    hash(...)      bucket ids             [Reformer note, "LSH Attention"]
    sort(...)      perm, inv_perm         ["Sorting and Chunking"]
    attend(...)    o_rounds, lse (sorted) ["LSH Attention", "Sorting and
                                           Chunking", "Implementation Reading"]
    combine(...)   y                      ["Multiple Hash Rounds"]
    forward(...)   all of the above
    attend_union() o_rounds, lse with set semantics of the round union
                   ["Multiple Hash Rounds"]; forward_union() end to end
    linear()       x W^T + b, token by token            ["Chunked Feed-Forward
                                                          Computation"]
    local_attend() y, lse of local chunked attention (no hashing) [Reformer
                   overview page, "Approach / What changed", "Takeaways"]
    *_rows(...)    the same on a sample of rows (for full-size parity)
    set_threads()  OpenMP thread count of the calls that follow (timing only)
    candidates()   attended positions of one query (window-rule tests)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsh_oracle.c")
_LIB = os.path.join(_HERE, "liblsh_oracle.so")
_lock = threading.Lock()
_lib = None

_I = ctypes.c_int
_I64 = ctypes.c_int64
_P = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    lib.oracle_lsh_hash.argtypes = [_I] * 6 + [_P, _P, _P]
    lib.oracle_lsh_hash_rows.argtypes = [_I] * 6 + [_P, _P, _I64, _P, _P]
    lib.oracle_lsh_sort.argtypes = [_I, _I, _P, _P, _P]
    lib.oracle_lsh_attend.argtypes = [_I] * 9 + [_P] * 6
    lib.oracle_lsh_attend_rows.argtypes = [_I] * 9 + [_P] * 4 + [_I64, _P, _P, _P]
    lib.oracle_lsh_candidates.argtypes = [_I] * 8 + [_P, _P, _I64, _I, _P]
    lib.oracle_lsh_combine.argtypes = [_I] * 5 + [_P] * 5
    lib.oracle_lsh_combine_rows.argtypes = [_I] * 5 + [_P] * 4 + [_I64, _P, _P]
    lib.oracle_lsh_forward.argtypes = [_I] * 9 + [_P] * 9
    lib.oracle_lsh_attend_union.argtypes = [_I] * 9 + [_P] * 7
    lib.oracle_lsh_attend_union_rows.argtypes = [_I] * 9 + [_P] * 5 + [_I64, _P, _P, _P]
    lib.oracle_linear.argtypes = [_I64, _I, _I, _P, _P, _P, _P]
    lib.oracle_local_attend.argtypes = [_I] * 9 + [_P] * 4
    lib.oracle_local_attend_rows.argtypes = [_I] * 9 + [_P, _P, _I64, _P, _P, _P]
    lib.oracle_set_threads.argtypes = [_I]
    for name in ("oracle_lsh_hash", "oracle_lsh_hash_rows", "oracle_lsh_sort",
                 "oracle_lsh_attend", "oracle_lsh_attend_rows",
                 "oracle_lsh_candidates", "oracle_lsh_combine",
                 "oracle_lsh_combine_rows", "oracle_lsh_forward",
                 "oracle_local_attend", "oracle_local_attend_rows",
                 "oracle_lsh_attend_union", "oracle_lsh_attend_union_rows",
                 "oracle_linear", "oracle_set_threads"):
        getattr(lib, name).restype = _I
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            other = os.environ.get("LSH_ORACLE_LIB")
            if other:
                _lib = _bind(ctypes.CDLL(other))
            else:
                build(force=False)
                _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def use_library(path):
    """Point this module at another build of lsh_oracle.c (used by the tests
    that plant a mistake in a private copy of the oracle, which also set
    LSH_ORACLE_LIB for a child process); None restores the default build."""
    global _lib
    with _lock:
        _lib = None if path is None else _bind(ctypes.CDLL(path))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: invalid argument (oracle returned {rc})")


def _dims(qk):
    b, h, L, d = qk.shape
    return int(b), int(h), int(L), int(d)


def _rot(rot, h, n_rounds, n_buckets, d):
    half = n_buckets // 2
    r = _f64(rot) if half > 0 else np.zeros((h, n_rounds, 0, d))
    if r.shape != (h, n_rounds, half, d):
        raise ValueError(f"rot must have shape {(h, n_rounds, half, d)}, got {r.shape}")
    return r


def hash(qk, rot, n_buckets: int, n_rounds: int) -> np.ndarray:
    """buckets[b][h][r][L] (int32) of every token in every round."""
    qk = _f64(qk)
    b, h, L, d = _dims(qk)
    rot = _rot(rot, h, n_rounds, n_buckets, d)
    out = np.empty((b, h, n_rounds, L), np.int32)
    _check(_load().oracle_lsh_hash(b, h, L, d, n_buckets, n_rounds, _ptr(qk), _ptr(rot),
                                   _ptr(out)), "hash")
    return out


def hash_rows(qk, rot, n_buckets: int, n_rounds: int, flat_idx) -> np.ndarray:
    """Bucket ids at flat indices into buckets[b][h][r][L]."""
    qk = _f64(qk)
    b, h, L, d = _dims(qk)
    rot = _rot(rot, h, n_rounds, n_buckets, d)
    idx = _i64(flat_idx).ravel()
    out = np.empty(idx.shape[0], np.int32)
    _check(_load().oracle_lsh_hash_rows(b, h, L, d, n_buckets, n_rounds, _ptr(qk), _ptr(rot),
                                        idx.shape[0], _ptr(idx), _ptr(out)), "hash_rows")
    return out


def sort(buckets):
    """(perm, inv_perm), each shaped like buckets (int32)."""
    bk = _i32(buckets)
    L = bk.shape[-1]
    nseg = bk.size // L
    perm = np.empty_like(bk)
    inv = np.empty_like(bk)
    _check(_load().oracle_lsh_sort(nseg, L, _ptr(bk), _ptr(perm), _ptr(inv)), "sort")
    return perm, inv


def attend(qk, v, buckets, perm, n_buckets: int, chunk: int, causal: bool, self_mask: bool):
    """(o_rounds[b][h][r][L][d], lse[b][h][r][L]) in sorted order, float64."""
    qk, v, bk, pm = _f64(qk), _f64(v), _i32(buckets), _i32(perm)
    b, h, L, d = _dims(qk)
    R = bk.shape[2]
    o = np.empty((b, h, R, L, d))
    lse = np.empty((b, h, R, L))
    _check(_load().oracle_lsh_attend(b, h, L, d, n_buckets, R, chunk, int(causal),
                                     int(self_mask), _ptr(qk), _ptr(v), _ptr(bk), _ptr(pm),
                                     _ptr(o), _ptr(lse)), "attend")
    return o, lse


def attend_rows(qk, v, buckets, perm, n_buckets: int, chunk: int, causal: bool,
                self_mask: bool, flat_idx):
    """(o[n][d], lse[n]) for flat indices seg*L + slot (sorted order)."""
    qk, v, bk, pm = _f64(qk), _f64(v), _i32(buckets), _i32(perm)
    b, h, L, d = _dims(qk)
    R = bk.shape[2]
    idx = _i64(flat_idx).ravel()
    o = np.empty((idx.shape[0], d))
    lse = np.empty(idx.shape[0])
    _check(_load().oracle_lsh_attend_rows(b, h, L, d, n_buckets, R, chunk, int(causal),
                                          int(self_mask), _ptr(qk), _ptr(v), _ptr(bk),
                                          _ptr(pm), idx.shape[0], _ptr(idx), _ptr(o),
                                          _ptr(lse)), "attend_rows")
    return o, lse


def attend_union(qk, v, buckets, perm, inv_perm, n_buckets: int, chunk: int, causal: bool,
                 self_mask: bool):
    """Per-round (o_rounds, lse), sorted order, where each candidate is
    attended only in the first round in which it is a candidate of the query
    (later rounds leave it out); combine() of these is the softmax over the
    SET union of the rounds' candidates."""
    qk, v, bk, pm, ip = _f64(qk), _f64(v), _i32(buckets), _i32(perm), _i32(inv_perm)
    b, h, L, d = _dims(qk)
    R = bk.shape[2]
    o = np.empty((b, h, R, L, d))
    lse = np.empty((b, h, R, L))
    _check(_load().oracle_lsh_attend_union(b, h, L, d, n_buckets, R, chunk, int(causal),
                                           int(self_mask), _ptr(qk), _ptr(v), _ptr(bk), _ptr(pm),
                                           _ptr(ip), _ptr(o), _ptr(lse)), "attend_union")
    return o, lse


def attend_union_rows(qk, v, buckets, perm, inv_perm, n_buckets: int, chunk: int, causal: bool,
                      self_mask: bool, flat_idx):
    """attend_union at flat indices seg*L + slot (sorted order)."""
    qk, v, bk, pm, ip = _f64(qk), _f64(v), _i32(buckets), _i32(perm), _i32(inv_perm)
    b, h, L, d = _dims(qk)
    R = bk.shape[2]
    idx = _i64(flat_idx).ravel()
    o = np.empty((idx.shape[0], d))
    lse = np.empty(idx.shape[0])
    _check(_load().oracle_lsh_attend_union_rows(b, h, L, d, n_buckets, R, chunk, int(causal),
                                                int(self_mask), _ptr(qk), _ptr(v), _ptr(bk),
                                                _ptr(pm), _ptr(ip), idx.shape[0], _ptr(idx),
                                                _ptr(o), _ptr(lse)), "attend_union_rows")
    return o, lse


def candidates(buckets, perm, n_buckets: int, chunk: int, causal: bool, self_mask: bool,
               seg: int, slot: int) -> np.ndarray:
    """Original positions attended by the query at sorted `slot` of segment `seg`."""
    bk, pm = _i32(buckets), _i32(perm)
    b, h, R, L = bk.shape
    out = np.empty(2 * chunk, np.int32)
    n = _load().oracle_lsh_candidates(b, h, L, n_buckets, R, chunk, int(causal),
                                      int(self_mask), _ptr(bk), _ptr(pm), seg, slot, _ptr(out))
    if n < 0:
        raise ValueError("candidates: invalid argument")
    return out[:n].copy()


def combine(o_rounds, lse, inv_perm, v) -> np.ndarray:
    """y[b][h][L][d] (float64) from per-round outputs in sorted order."""
    o, l, inv, v = _f64(o_rounds), _f64(lse), _i32(inv_perm), _f64(v)
    b, h, R, L, d = o.shape
    y = np.empty((b, h, L, d))
    _check(_load().oracle_lsh_combine(b, h, L, d, R, _ptr(o), _ptr(l), _ptr(inv), _ptr(v),
                                      _ptr(y)), "combine")
    return y


def combine_rows(o_rounds, lse, inv_perm, v, flat_idx) -> np.ndarray:
    """y rows at flat indices (b*H + h)*L + i."""
    o, l, inv, v = _f64(o_rounds), _f64(lse), _i32(inv_perm), _f64(v)
    b, h, R, L, d = o.shape
    idx = _i64(flat_idx).ravel()
    y = np.empty((idx.shape[0], d))
    _check(_load().oracle_lsh_combine_rows(b, h, L, d, R, _ptr(o), _ptr(l), _ptr(inv), _ptr(v),
                                           idx.shape[0], _ptr(idx), _ptr(y)), "combine_rows")
    return y


def forward(qk, v, rot, n_buckets: int, n_rounds: int, chunk: int, causal: bool,
            self_mask: bool) -> dict:
    """All four steps; returns every intermediate (float64 / int32 arrays)."""
    qk, v = _f64(qk), _f64(v)
    b, h, L, d = _dims(qk)
    rot = _rot(rot, h, n_rounds, n_buckets, d)
    R = n_rounds
    out = dict(
        buckets=np.empty((b, h, R, L), np.int32),
        perm=np.empty((b, h, R, L), np.int32),
        inv_perm=np.empty((b, h, R, L), np.int32),
        o_rounds=np.empty((b, h, R, L, d)),
        lse=np.empty((b, h, R, L)),
        y=np.empty((b, h, L, d)),
    )
    _check(_load().oracle_lsh_forward(b, h, L, d, n_buckets, R, chunk, int(causal),
                                      int(self_mask), _ptr(qk), _ptr(v), _ptr(rot),
                                      _ptr(out["buckets"]), _ptr(out["perm"]),
                                      _ptr(out["inv_perm"]), _ptr(out["o_rounds"]),
                                      _ptr(out["lse"]), _ptr(out["y"])), "forward")
    return out


def local_attend(qk, v, chunk: int, before: int, after: int, causal: bool, self_mask: bool):
    """(y[b][h][L][d], lse[b][h][L]) of local chunked attention: each chunk
    sees `before` chunks before it and `after` chunks after it."""
    qk, v = _f64(qk), _f64(v)
    b, h, L, d = _dims(qk)
    y = np.empty((b, h, L, d))
    lse = np.empty((b, h, L))
    _check(_load().oracle_local_attend(b, h, L, d, chunk, before, after, int(causal),
                                       int(self_mask), _ptr(qk), _ptr(v), _ptr(y),
                                       _ptr(lse)), "local_attend")
    return y, lse


def local_attend_rows(qk, v, chunk: int, before: int, after: int, causal: bool,
                      self_mask: bool, flat_idx):
    """(y[n][d], lse[n]) of local attention at flat indices (b*heads + h)*L + i."""
    qk, v = _f64(qk), _f64(v)
    b, h, L, d = _dims(qk)
    idx = _i64(flat_idx).ravel()
    y = np.empty((idx.shape[0], d))
    lse = np.empty(idx.shape[0])
    _check(_load().oracle_local_attend_rows(b, h, L, d, chunk, before, after, int(causal),
                                            int(self_mask), _ptr(qk), _ptr(v), idx.shape[0],
                                            _ptr(idx), _ptr(y), _ptr(lse)), "local_attend_rows")
    return y, lse


def forward_union(qk, v, rot, n_buckets: int, n_rounds: int, chunk: int, causal: bool,
                  self_mask: bool) -> dict:
    """hash -> sort -> attend_union -> combine: y is the softmax over the set
    union of the rounds' candidates."""
    buckets = hash(qk, rot, n_buckets, n_rounds)
    perm, inv_perm = sort(buckets)
    o, lse = attend_union(qk, v, buckets, perm, inv_perm, n_buckets, chunk, causal, self_mask)
    y = combine(o, lse, inv_perm, v)
    return dict(buckets=buckets, perm=perm, inv_perm=inv_perm, o_rounds=o, lse=lse, y=y)


def linear(a, w, bias=None) -> np.ndarray:
    """a[..., K] @ w[N, K]^T (+ bias[N]) in fp64, each output row from its own
    input row only."""
    a = _f64(a)
    w = _f64(w)
    N, K = w.shape
    rows = a.size // K
    out = np.empty(a.shape[:-1] + (N,))
    b = None if bias is None else _f64(bias)
    _check(_load().oracle_linear(rows, N, K, _ptr(a), _ptr(w), None if b is None else _ptr(b),
                                 _ptr(out)), "linear")
    return out


def set_threads(n: int = 0) -> int:
    """Use n OpenMP threads from the next call on (n < 1: unchanged); returns
    the count in force.  Results do not depend on it."""
    return int(_load().oracle_set_threads(int(n)))
