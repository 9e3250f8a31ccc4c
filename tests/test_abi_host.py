"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every entry point include/lsh.h declares, and
reject every invalid argument on the host with the documented status before
any HIP call is made.
"""
import ctypes
import os
import re

import pytest

from lsh_sparse_attention_hash_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lsh.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsh_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = B.library()
    assert lib.lsh_version() == 10000
    for st, text in ((0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape"),
                     (3, b"workspace too small"), (4, b"HIP launch failure")):
        assert lib.lsh_status_string(st) == text


def cfg(**kw):
    """A valid configuration with the given fields overwritten verbatim."""
    c = B.make_config(batch=1, heads=2, seq_len=256, n_buckets=8, n_rounds=2, causal=1,
                      self_mask=1, dtype="bf16")
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def call_hash(c, qk=FAKE, rot=FAKE, out=FAKE):
    return B.library().lsh_hash(ctypes.byref(c), qk, rot, out, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), B.LSH_ERR_UNSUPPORTED),
    (dict(chunk_len=128), B.LSH_ERR_UNSUPPORTED),
    (dict(n_buckets=7), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(n_buckets=0), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(n_buckets=32768), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(n_rounds=0), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(seq_len=100), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(seq_len=-64), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(causal=2), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(batch=1024, heads=1024, seq_len=4096, n_rounds=1), B.LSH_ERR_INVALID_ARGUMENT),
])
def test_invalid_config_rejected_by_every_call(kw, status):
    c = cfg(**kw)
    lib = B.library()
    assert call_hash(c) == status
    assert lib.lsh_sort(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == status
    assert lib.lsh_chunk_attend(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.lsh_unsort_combine(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.lsh_sort_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.lsh_last_error()


def test_null_and_misaligned_pointers_rejected():
    c = cfg()
    assert call_hash(c, qk=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"qk" in B.library().lsh_last_error()
    assert call_hash(c, rot=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert call_hash(c, out=ctypes.c_void_p(0x10004)) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"aligned" in B.library().lsh_last_error()
    lib = B.library()
    assert lib.lsh_hash(ctypes.byref(c), FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert lib.lsh_chunk_attend(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert lib.lsh_unsort_combine(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert lib.lsh_hash(None, FAKE, FAKE, FAKE, None, None) == B.LSH_ERR_INVALID_ARGUMENT


def test_workspace_too_small():
    c = cfg()
    need = B.lsh_sort_workspace_bytes(c)
    assert need > 0
    lib = B.library()
    assert lib.lsh_sort(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        B.LSH_ERR_WORKSPACE_TOO_SMALL


def _sort_tile(S, L, nb):
    """The sort's tile: for B <= 2048 the largest of 1,024 .. 16,384 keys (at
    most 4,096 for B <= 256 and 8,192 for B > 1,024) that leaves at least 256
    tiles in all; otherwise max(1024, B) doubled up to 4,096 while there would
    be more than 1,024 tiles."""
    if nb <= 2048:
        cap = 4096 if nb <= 256 else (16384 if nb <= 1024 else 8192)
        tile = 1024
        while tile < cap and S * -(-L // (2 * tile)) >= 256:
            tile *= 2
        return tile
    tile = 1024
    while tile < nb:
        tile *= 2
    while tile < 4096 and S * L // tile > 1024:
        tile *= 2
    return tile


def test_workspace_bytes_cover_the_count_tables():
    for L, nb, R in ((1024, 16, 1), (4096, 64, 2), (65536, 1024, 8), (524288, 8192, 2),
                     (2048, 16384, 1), (16384, 2048, 4), (192, 38, 3)):
        c = cfg(seq_len=L, n_buckets=nb, n_rounds=R, heads=4)
        S = 4 * R
        tiles = -(-L // _sort_tile(S, L, nb))
        need = 4 * S * nb * tiles + (4 * S * nb if nb > 2048 else 0)   # counts (+ bases)
        assert B.lsh_sort_workspace_bytes(c) >= need
    # the headline shape: 16,384-key tiles, 1 MiB of counts
    assert B.lsh_sort_workspace_bytes(cfg(seq_len=65536, n_buckets=1024, n_rounds=8,
                                          heads=8)) == 64 * 4 * 1024 * 4


def test_per_round_buffer_size():
    """LSH_O_F32 (either input dtype): fp32 rows; LSH_O_F16_SCALED (bf16
    inputs): 256 fp32 partial maxima and one int32 exponent per (batch,
    head), padded to a multiple of 256 bytes, then fp16 rows."""
    for b, H, L, R, dt in ((1, 8, 65536, 8, B.LSH_BF16), (2, 3, 192, 5, B.LSH_BF16),
                           (1, 1, 1024, 1, B.LSH_F32), (3, 2, 448, 3, B.LSH_F32)):
        rows = b * H * R * L * 64
        c = cfg(batch=b, heads=H, seq_len=L, n_rounds=R, dtype=dt)
        assert c.o_format == B.LSH_O_F32            # the zero default
        assert B.lsh_o_rounds_bytes(c) == 4 * rows
        c = cfg(batch=b, heads=H, seq_len=L, n_rounds=R, dtype=dt, o_format=B.LSH_O_F16_SCALED)
        if dt == B.LSH_BF16:
            header = -(-(b * H * (256 * 4 + 4)) // 256) * 256
            assert B.lsh_o_rounds_bytes(c) == header + 2 * rows
        else:
            assert B.lsh_o_rounds_bytes(c) == 0     # unsupported with fp32 inputs
    assert B.lsh_o_rounds_bytes(cfg(seq_len=0)) == 0
    assert B.lsh_o_rounds_bytes(cfg(head_dim=32)) == 0


def test_o_format_is_validated():
    lib = B.library()
    for kw, status in ((dict(o_format=2), B.LSH_ERR_INVALID_ARGUMENT),
                       (dict(o_format=-1), B.LSH_ERR_INVALID_ARGUMENT),
                       (dict(o_format=B.LSH_O_F16_SCALED, dtype=B.LSH_F32),
                        B.LSH_ERR_UNSUPPORTED)):
        c = cfg(**kw)
        assert call_hash(c) == status
        assert lib.lsh_chunk_attend(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    None) == status
        assert lib.lsh_unsort_combine(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None) == status
        assert b"o_format" in lib.lsh_last_error() or b"F16" in lib.lsh_last_error()


def test_empty_problems_are_no_ops():
    lib = B.library()
    for kw in (dict(batch=0), dict(heads=0), dict(seq_len=0)):
        c = cfg(**kw)
        assert call_hash(c, qk=None, rot=None, out=None) == B.LSH_OK
        assert lib.lsh_sort(ctypes.byref(c), None, None, None, None, 0, None) == B.LSH_OK
        assert lib.lsh_chunk_attend(ctypes.byref(c), None, None, None, None, None, None, None) == 0
        assert lib.lsh_unsort_combine(ctypes.byref(c), None, None, None, None, None, None) == 0
        assert lib.lsh_sort_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.lsh_last_error() == b""


def test_b1_needs_no_rotation():
    c = cfg(n_buckets=1)
    # rot may be NULL when B == 1; qk still required
    assert call_hash(c, qk=None, rot=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"qk" in B.library().lsh_last_error()


def call_local(c, before=1, after=1, qk=FAKE, v=FAKE, y=FAKE, lse=FAKE):
    return B.library().lsh_local_attend(ctypes.byref(c), before, after, qk, v, y, lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), B.LSH_ERR_UNSUPPORTED),
    (dict(chunk_len=128), B.LSH_ERR_UNSUPPORTED),
    (dict(seq_len=100), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(causal=2), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(self_mask=-1), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(batch=2048, heads=1024, seq_len=1024), B.LSH_ERR_INVALID_ARGUMENT),
])
def test_local_attend_rejects_invalid_config(kw, status):
    assert call_local(cfg(**kw)) == status
    assert B.library().lsh_last_error()


def test_local_attend_ignores_bucket_and_round_fields():
    # validation stops at the (fake) pointers only if the config itself passed:
    # a NULL y is reported, not the unused n_buckets / n_rounds
    c = cfg(n_buckets=7, n_rounds=0)
    assert call_local(c, y=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"y is NULL" in B.library().lsh_last_error()


def test_local_attend_rejects_bad_windows_and_pointers():
    c = cfg()
    assert call_local(c, before=-1) == B.LSH_ERR_INVALID_ARGUMENT
    assert call_local(c, after=-2) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"n_before" in B.library().lsh_last_error()
    assert call_local(c, qk=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert call_local(c, v=ctypes.c_void_p(0x10008)) == B.LSH_ERR_INVALID_ARGUMENT
    assert call_local(c, lse=None) == B.LSH_ERR_INVALID_ARGUMENT
    assert B.library().lsh_local_attend(None, 1, 1, FAKE, FAKE, FAKE, FAKE, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    for kw in (dict(batch=0), dict(heads=0), dict(seq_len=0)):
        assert call_local(cfg(**kw), qk=None, v=None, y=None, lse=None) == B.LSH_OK


def test_union_attend_limits_and_workspace():
    lib = B.library()
    c = cfg()
    need = B.lsh_union_workspace_bytes(c)
    assert need == 1 * 2 * 256 * 4 * 4          # rounds before the last, padded to 4 keys
    for R, keys in ((5, 4), (6, 8), (9, 8), (10, 16), (16, 16)):
        assert B.lsh_union_workspace_bytes(cfg(n_rounds=R)) == 2 * 256 * keys * 4
    args = [FAKE] * 7
    assert lib.lsh_chunk_attend_union(ctypes.byref(c), *args, FAKE, need - 1, None) == \
        B.LSH_ERR_WORKSPACE_TOO_SMALL
    assert lib.lsh_chunk_attend_union(ctypes.byref(c), *args[:6], None, FAKE, need, None) == \
        B.LSH_ERR_INVALID_ARGUMENT                # NULL lse
    c17 = cfg(n_rounds=17)
    assert B.lsh_union_workspace_bytes(c17) == 0
    assert lib.lsh_chunk_attend_union(ctypes.byref(c17), *args, FAKE, 1 << 30, None) == \
        B.LSH_ERR_UNSUPPORTED
    big = cfg(seq_len=1 << 23, n_buckets=16384, n_rounds=1, heads=1)
    assert lib.lsh_chunk_attend_union(ctypes.byref(big), *args, FAKE, 1 << 40, None) == \
        B.LSH_ERR_UNSUPPORTED
    empty = cfg(seq_len=0)
    assert lib.lsh_chunk_attend_union(ctypes.byref(empty), *([None] * 8), 0, None) == B.LSH_OK


def layer_cfg(**kw):
    c = B.LshLayerConfig(1, 256, 128, 256, 8, 2, 1, 1, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=100), B.LSH_ERR_UNSUPPORTED),
    (dict(d_model=0), B.LSH_ERR_UNSUPPORTED),
    (dict(d_ff=96), B.LSH_ERR_UNSUPPORTED),
    (dict(ffn_chunk=-1), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(seq_len=100), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(n_buckets=7), B.LSH_ERR_INVALID_ARGUMENT),
    (dict(causal=3), B.LSH_ERR_INVALID_ARGUMENT),
])
def test_layer_calls_reject_invalid_config(kw, status):
    lib = B.library()
    c = layer_cfg(**kw)
    w = B.LshLayerWeights(*([0x10000] * 8))
    assert lib.lsh_project_qkv(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert lib.lsh_project_out(ctypes.byref(c), FAKE, FAKE, FAKE, 0, FAKE, None) == status
    assert lib.lsh_ffn(ctypes.byref(c), *([FAKE] * 6), 0, FAKE, FAKE, 1 << 40, None) == status
    assert lib.lsh_reversible_forward(ctypes.byref(c), ctypes.byref(w), *([FAKE] * 5), 1 << 40,
                                      None) == status
    assert lib.lsh_layer_workspace_bytes(ctypes.byref(c)) == 0
    assert lib.lsh_ffn_workspace_bytes(ctypes.byref(c)) == 0


def test_layer_calls_check_pointers_workspace_and_flags():
    lib = B.library()
    c = layer_cfg()
    w = B.LshLayerWeights(*([0x10000] * 8))
    need = B.lsh_layer_workspace_bytes(c)
    assert need > 0
    assert lib.lsh_reversible_inverse(ctypes.byref(c), ctypes.byref(w), *([FAKE] * 5), need - 1,
                                      None) == B.LSH_ERR_WORKSPACE_TOO_SMALL
    assert lib.lsh_reversible_forward(ctypes.byref(c), None, *([FAKE] * 5), need, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    w_bad = B.LshLayerWeights(*([0x10000] * 4 + [0x10004] + [0x10000] * 3))
    assert lib.lsh_reversible_forward(ctypes.byref(c), ctypes.byref(w_bad), *([FAKE] * 5), need,
                                      None) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"w_1" in lib.lsh_last_error()
    assert B.lsh_ffn_workspace_bytes(c) == 256 * 256 * 2
    assert B.lsh_ffn_workspace_bytes(layer_cfg(ffn_chunk=100)) == 100 * 256 * 2
    assert lib.lsh_ffn(ctypes.byref(c), *([FAKE] * 6), 0, FAKE, FAKE, 256 * 256 * 2 - 1, None) == \
        B.LSH_ERR_WORKSPACE_TOO_SMALL
    assert lib.lsh_project_out(ctypes.byref(c), FAKE, FAKE, FAKE, 2, FAKE, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert lib.lsh_project_qkv(ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    e = layer_cfg(seq_len=0)
    assert lib.lsh_reversible_forward(ctypes.byref(e), None, *([None] * 5), 0, None) == B.LSH_OK


def test_static_scratch_sort_validates_before_any_launch():
    """lsh_sort_static_scratch rejects bad arguments like lsh_sort, and a
    configuration whose count tables exceed its 32 MiB static scratch with
    LSH_ERR_WORKSPACE_TOO_SMALL, all on the host."""
    lib = B.library()
    c = cfg()
    assert lib.lsh_sort_static_scratch(ctypes.byref(c), None, FAKE, FAKE, None) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert lib.lsh_sort_static_scratch(ctypes.byref(cfg(n_buckets=7)), FAKE, FAKE, FAKE,
                                       None) == B.LSH_ERR_INVALID_ARGUMENT
    big = cfg(batch=1, heads=8, seq_len=131072, n_buckets=16384, n_rounds=8)
    assert B.lsh_sort_workspace_bytes(big) > 32 << 20
    assert lib.lsh_sort_static_scratch(ctypes.byref(big), FAKE, FAKE, FAKE, None) == \
        B.LSH_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.lsh_last_error()
    empty = cfg(seq_len=0)
    assert lib.lsh_sort_static_scratch(ctypes.byref(empty), None, None, None, None) == B.LSH_OK


def test_rotation_conversion_validates_before_any_launch():
    lib = B.library()
    conv = lambda c, src, dst: lib.lsh_rot_from_columns(ctypes.byref(c), src, dst, None)
    c = cfg()
    assert conv(c, None, FAKE) == B.LSH_ERR_INVALID_ARGUMENT
    assert b"rot_cols" in lib.lsh_last_error()
    assert conv(c, FAKE, None) == B.LSH_ERR_INVALID_ARGUMENT
    assert conv(c, FAKE, ctypes.c_void_p(0x20008)) == B.LSH_ERR_INVALID_ARGUMENT   # misaligned
    # 2 heads x 2 rounds x 4 directions x 64 bf16 = 2,048 bytes: overlapping buffers rejected
    assert conv(c, ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000 + 1024)) == \
        B.LSH_ERR_INVALID_ARGUMENT
    assert b"overlap" in lib.lsh_last_error()
    assert conv(cfg(dtype=7), FAKE, FAKE) == B.LSH_ERR_INVALID_ARGUMENT
    assert conv(cfg(head_dim=32), FAKE, FAKE) == B.LSH_ERR_UNSUPPORTED
    # nothing to convert: no heads, or no hashing
    assert conv(cfg(heads=0), None, None) == B.LSH_OK
    assert conv(cfg(n_buckets=1), None, None) == B.LSH_OK
    assert lib.lsh_rot_from_columns(None, FAKE, FAKE, None) == B.LSH_ERR_INVALID_ARGUMENT
