"""fp64 oracle of one reversible Reformer layer with LSH attention and a
chunked feed-forward map.

TEST INFRASTRUCTURE ONLY: the tests may import this module; the product path
never does.  It shares nothing with the HIP library.  The dense maps run
through ``oracle.linear`` (plain fp64 loops in lsh_oracle.c), the attention
through ``oracle.forward`` (the pinned LSH oracle).

What it computes (Reformer study note, eightmm.github.io):
  "Reversible Residual Layers"  the hidden state is split into (x1, x2);
      y1 = x1 + F(x2), y2 = x2 + G(y1); the inverse is x2 = y2 - G(y1),
      x1 = y1 - F(x2).
  "Chunked Feed-Forward Computation"  G(x_i) = W2 s(W1 x_i + b1) + b2 token by
      token, evaluated over chunks of tokens with the same result.
  F is the LSH attention of this repository ("LSH Attention", "Shared
      Query-Key Space"): qk = x W_qk^T and v = x W_v^T, split into heads of
      64 features (head h = features 64h .. 64h+63), the LSH forward per head,
      the heads concatenated in the same order and mapped by W_o^T.

Readings where the note is silent (listed in the design notes):
  - s is ReLU; there is no layer normalisation inside F or G;
  - weights are stored one row per output feature ([out][in], bf16 values);
  - the precision is part of the definition: every input of a dense map is
    rounded to bf16 (round to nearest, ties to even), qk, v and the hidden
    activation of G are stored in bf16, the residual stream (x1, x2, y1, y2)
    and the outputs of F and G are exact here (fp32 on the GPU).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle

HEAD_DIM = 64


def bf16_round(a) -> np.ndarray:
    """Round to the nearest value with 8 significant bits (bf16), ties to
    even, written from the definition: a = m * 2^e with 0.5 <= |m| < 1, keep
    round_half_even(m * 2^8) / 2^8.  Finite, normal-range values only."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def split_heads(t, heads):
    """[b][L][H*64] -> [b][H][L][64]."""
    b, L, _ = t.shape
    return np.ascontiguousarray(t.reshape(b, L, heads, HEAD_DIM).transpose(0, 2, 1, 3))


def merge_heads(t):
    """[b][H][L][64] -> [b][L][H*64]."""
    b, H, L, d = t.shape
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3).reshape(b, L, H * d))


def project_qkv(x, w_qk, w_v):
    """(qk, v), each [b][H][L][64] with bf16 values."""
    heads = w_qk.shape[0] // HEAD_DIM
    xb = bf16_round(x)
    qk = bf16_round(oracle.linear(xb, w_qk))
    v = bf16_round(oracle.linear(xb, w_v))
    return split_heads(qk, heads), split_heads(v, heads)


def project_out(y_att, w_o):
    """The heads' outputs [b][H][L][64], concatenated and mapped by W_o^T."""
    return oracle.linear(bf16_round(merge_heads(y_att)), w_o)


def attention(x, w, cfg, with_parts=False):
    """F(x) for x [b][L][D]."""
    qk, v = project_qkv(x, w["w_qk"], w["w_v"])
    fw = oracle.forward(qk, v, w["rot"], cfg["n_buckets"], cfg["n_rounds"], HEAD_DIM,
                        cfg["causal"], cfg["self_mask"])
    out = project_out(fw["y"], w["w_o"])
    if with_parts:
        return out, dict(qk=qk, v=v, **fw)
    return out


def ffn(x, w, chunk=None):
    """G(x) for x [b][L][D], evaluated over chunks of `chunk` tokens (all at
    once if None)."""
    b, L, D = x.shape
    rows = x.reshape(b * L, D)
    step = b * L if not chunk else chunk
    out = np.empty((b * L, w["w_2"].shape[0]))
    for s in range(0, b * L, step):
        xb = bf16_round(rows[s:s + step])
        h = bf16_round(np.maximum(oracle.linear(xb, w["w_1"], w["b_1"]), 0.0))
        out[s:s + step] = oracle.linear(h, w["w_2"], w["b_2"])
    return out.reshape(b, L, -1)


def reversible_forward(x1, x2, w, cfg):
    """(y1, y2) = (x1 + F(x2), x2 + G(y1))."""
    y1 = x1 + attention(x2, w, cfg)
    y2 = x2 + ffn(y1, w, cfg.get("ffn_chunk"))
    return y1, y2


def reversible_inverse(y1, y2, w, cfg):
    """(x1, x2) = (y1 - F(x2), y2 - G(y1)), x2 first."""
    x2 = y2 - ffn(y1, w, cfg.get("ffn_chunk"))
    x1 = y1 - attention(x2, w, cfg)
    return x1, x2
