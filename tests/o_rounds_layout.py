"""Host-side reading of the per-round output buffer of lsh_chunk_attend, from
the layout the C ABI documents (include/lsh.h):

* LSH_O_F32 (any input dtype): fp32 rows [b][H][R][L][64];
* LSH_O_F16_SCALED (bf16 inputs): a header of 256 fp32 partial maxima of |v| per (b, h)
  ([b][H][256]) and the int32 exponent k of each (b, h) ([b][H]), padded to a
  multiple of 256 bytes, then fp16 rows [b][H][R][L][64] holding o * 2^-k,
  where k = max(e - 15, -100) and e is the smallest integer with the largest
  partial maximum of (b, h) < 2^e (e = -126 below 2^-126).

The values come back as fp32, which holds fp16 * 2^k exactly.
"""
import math

import numpy as np

V_PARTS = 256


def header_bytes(w):
    if not w.o16:
        return 0
    n = w.batch * w.heads * (V_PARTS * 4 + 4)
    return (n + 255) // 256 * 256


def scale_exponent(vmax):
    """k of a (b, h) from the largest |v| of its rows."""
    if vmax < 2.0 ** -126:
        e = -126
    else:
        e = math.frexp(vmax)[1]   # vmax = m 2^e with 0.5 <= m < 1: the smallest e with vmax < 2^e
    return max(e - 15, -100)


def header(buf, w):
    """The [b][H][256] partial maxima (bf16 inputs)."""
    n = w.batch * w.heads * V_PARTS
    return np.asarray(buf[: n * 4]).view(np.float32).reshape(w.batch, w.heads, V_PARTS)


def head_exponents(buf, w):
    """The [b][H] int32 exponents that follow the partial maxima."""
    n = w.batch * w.heads
    return np.asarray(buf).view(np.uint8).ravel()[n * V_PARTS * 4: n * V_PARTS * 4 + n * 4].view(
        np.int32).reshape(w.batch, w.heads)


def read_o_rounds(buf, w):
    """o as fp32 [b][H][R][L][64] from the raw bytes of the buffer."""
    buf = np.asarray(buf).view(np.uint8).ravel()
    shape = (w.batch, w.heads, w.n_rounds, w.seq_len, w.head_dim)
    n = int(np.prod(shape))
    if not w.o16:
        return buf[: n * 4].view(np.float32).reshape(shape).copy()
    hb = header_bytes(w)
    o = buf[hb: hb + n * 2].view(np.float16).reshape(shape).astype(np.float32)
    hdr = header(buf, w)
    for b in range(w.batch):
        for h in range(w.heads):
            o[b, h] *= np.float32(2.0 ** scale_exponent(float(hdr[b, h].max())))
    return o
