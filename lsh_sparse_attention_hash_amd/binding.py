"""Thin ctypes binding of liblsh.so (the C ABI in include/lsh.h).

Argument marshalling only: every function takes torch device tensors, checks
that they have the dtype and shape the ABI documents, passes their data
pointers and the current HIP stream to the library and raises LshError on a
non-OK status.  All computation happens in the library's gfx950 kernels; there
is no fallback of any kind.  If liblsh.so is missing the import of this module
fails loudly (build it with ``python -m lsh_sparse_attention_hash_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# LSH_LIBRARY may name another build of the same library (the sanitizer
# tests load a host-side AddressSanitizer build through it)
LIB_PATH = os.environ.get("LSH_LIBRARY") or os.path.join(_PKG, "liblsh.so")

LSH_OK = 0
LSH_ERR_INVALID_ARGUMENT = 1
LSH_ERR_UNSUPPORTED = 2
LSH_ERR_WORKSPACE_TOO_SMALL = 3
LSH_ERR_HIP = 4
LSH_F32 = 0
LSH_BF16 = 1
LSH_O_F32 = 0
LSH_O_F16_SCALED = 1

EXPORTS = ("lsh_hash", "lsh_rot_from_columns", "lsh_sort_workspace_bytes", "lsh_sort", "lsh_sort_static_scratch",
           "lsh_o_rounds_bytes", "lsh_chunk_attend",
           "lsh_unsort_combine", "lsh_union_workspace_bytes", "lsh_chunk_attend_union",
           "lsh_local_attend", "lsh_project_qkv", "lsh_project_out", "lsh_ffn_workspace_bytes",
           "lsh_ffn", "lsh_layer_workspace_bytes", "lsh_reversible_forward",
           "lsh_reversible_inverse", "lsh_status_string", "lsh_last_error", "lsh_version")


class LshError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str):
        super().__init__(f"{call} failed with status {status}: {detail}")
        self.status = status


class LshConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "heads", "seq_len", "head_dim", "n_buckets", "n_rounds", "chunk_len",
        "causal", "self_mask", "dtype", "o_format")]


class LshLayerConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "seq_len", "d_model", "d_ff", "n_buckets", "n_rounds", "causal", "self_mask",
        "ffn_chunk")]


class LshLayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "w_qk", "w_v", "w_o", "rot", "w_1", "b_1", "w_2", "b_2")]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m lsh_sparse_attention_hash_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(LshConfig)
    lib.lsh_hash.argtypes = [cfgp, P, P, P, P, P]
    lib.lsh_rot_from_columns.argtypes = [cfgp, P, P, P]
    lib.lsh_sort_workspace_bytes.argtypes = [cfgp]
    lib.lsh_sort_workspace_bytes.restype = SZ
    lib.lsh_sort.argtypes = [cfgp, P, P, P, P, SZ, P]
    lib.lsh_sort_static_scratch.argtypes = [cfgp, P, P, P, P]
    lib.lsh_o_rounds_bytes.argtypes = [cfgp]
    lib.lsh_o_rounds_bytes.restype = SZ
    lib.lsh_chunk_attend.argtypes = [cfgp, P, P, P, P, P, P, P]
    lib.lsh_unsort_combine.argtypes = [cfgp, P, P, P, P, P, P]
    lib.lsh_local_attend.argtypes = [cfgp, I32, I32, P, P, P, P, P]
    lib.lsh_union_workspace_bytes.argtypes = [cfgp]
    lib.lsh_union_workspace_bytes.restype = SZ
    lib.lsh_chunk_attend_union.argtypes = [cfgp, P, P, P, P, P, P, P, P, SZ, P]
    lcp = ctypes.POINTER(LshLayerConfig)
    lwp = ctypes.POINTER(LshLayerWeights)
    lib.lsh_project_qkv.argtypes = [lcp, P, P, P, P, P, P]
    lib.lsh_project_out.argtypes = [lcp, P, P, P, I32, P, P]
    lib.lsh_ffn_workspace_bytes.argtypes = [lcp]
    lib.lsh_ffn_workspace_bytes.restype = SZ
    lib.lsh_ffn.argtypes = [lcp, P, P, P, P, P, P, I32, P, P, SZ, P]
    lib.lsh_layer_workspace_bytes.argtypes = [lcp]
    lib.lsh_layer_workspace_bytes.restype = SZ
    lib.lsh_reversible_forward.argtypes = [lcp, lwp, P, P, P, P, P, SZ, P]
    lib.lsh_reversible_inverse.argtypes = [lcp, lwp, P, P, P, P, P, SZ, P]
    for f in ("lsh_hash", "lsh_rot_from_columns", "lsh_sort", "lsh_sort_static_scratch", "lsh_chunk_attend", "lsh_unsort_combine",
              "lsh_local_attend", "lsh_chunk_attend_union", "lsh_project_qkv", "lsh_project_out",
              "lsh_ffn", "lsh_reversible_forward", "lsh_reversible_inverse"):
        getattr(lib, f).restype = I32
    lib.lsh_status_string.argtypes = [I32]
    lib.lsh_status_string.restype = ctypes.c_char_p
    lib.lsh_last_error.argtypes = []
    lib.lsh_last_error.restype = ctypes.c_char_p
    lib.lsh_version.argtypes = []
    lib.lsh_version.restype = ctypes.c_int
    return lib


_lib = load_library()


def library() -> ctypes.CDLL:
    return _lib


def make_config(batch, heads, seq_len, n_buckets, n_rounds, causal, self_mask, dtype,
                head_dim=64, chunk_len=64, o_format=LSH_O_F32) -> LshConfig:
    dt = {"bf16": LSH_BF16, "f32": LSH_F32}.get(dtype, dtype)
    of = {"f32": LSH_O_F32, "f16_scaled": LSH_O_F16_SCALED}.get(o_format, o_format)
    return LshConfig(batch, heads, seq_len, head_dim, n_buckets, n_rounds, chunk_len,
                     int(bool(causal)), int(bool(self_mask)), dt, of)


def config_for(w) -> LshConfig:
    """LshConfig of a synth.Workload (per-round output format from w.o16)."""
    return make_config(w.batch, w.heads, w.seq_len, w.n_buckets, w.n_rounds, w.causal,
                       w.self_mask, w.dtype, w.head_dim, w.chunk_len,
                       LSH_O_F16_SCALED if w.o16 else LSH_O_F32)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to liblsh must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblsh must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_of(cfg: LshConfig):
    return torch.bfloat16 if cfg.dtype == LSH_BF16 else torch.float32


def _expect(t, shape, dtype, name):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _check(call, status):
    if status != LSH_OK:
        raise LshError(call, status, _lib.lsh_last_error().decode())


def lsh_hash(cfg: LshConfig, qk, rot, buckets, fallback_rows=None, stream=None):
    b, H, L, d, B, R = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_buckets, cfg.n_rounds
    dt = _dtype_of(cfg)
    _expect(qk, (b, H, L, d), dt, "qk")
    if B > 1:
        _expect(rot, (H, R, B // 2, d), dt, "rot")
    _expect(buckets, (b, H, R, L), torch.int32, "buckets")
    if fallback_rows is not None:
        _expect(fallback_rows, (1,), torch.int32, "fallback_rows")
    _check("lsh_hash", _lib.lsh_hash(ctypes.byref(cfg), _ptr(qk), _ptr(rot) if B > 1 else None,
                                     _ptr(buckets), _ptr(fallback_rows), _stream(stream)))


def lsh_rot_from_columns(cfg: LshConfig, rot_cols, rot_rows, stream=None):
    """rot_cols [H][R][d][B/2] (each rotation as a d x B/2 matrix) -> rot_rows
    [H][R][B/2][d], the layout lsh_hash reads."""
    H, R, d, B = cfg.heads, cfg.n_rounds, cfg.head_dim, cfg.n_buckets
    dt = _dtype_of(cfg)
    if B > 1 and H > 0:
        _expect(rot_cols, (H, R, d, B // 2), dt, "rot_cols")
        _expect(rot_rows, (H, R, B // 2, d), dt, "rot_rows")
    _check("lsh_rot_from_columns",
           _lib.lsh_rot_from_columns(ctypes.byref(cfg), _ptr(rot_cols), _ptr(rot_rows),
                                     _stream(stream)))


def lsh_sort_workspace_bytes(cfg: LshConfig) -> int:
    return int(_lib.lsh_sort_workspace_bytes(ctypes.byref(cfg)))


def lsh_sort(cfg: LshConfig, buckets, perm, inv_perm, workspace, stream=None):
    shape = (cfg.batch, cfg.heads, cfg.n_rounds, cfg.seq_len)
    for t, n in ((buckets, "buckets"), (perm, "perm"), (inv_perm, "inv_perm")):
        _expect(t, shape, torch.int32, n)
    _check("lsh_sort", _lib.lsh_sort(ctypes.byref(cfg), _ptr(buckets), _ptr(perm), _ptr(inv_perm),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def lsh_sort_static_scratch(cfg: LshConfig, buckets, perm, inv_perm, stream=None):
    """lsh_sort with the library's static scratch (no workspace argument)."""
    shape = (cfg.batch, cfg.heads, cfg.n_rounds, cfg.seq_len)
    for t, n in ((buckets, "buckets"), (perm, "perm"), (inv_perm, "inv_perm")):
        _expect(t, shape, torch.int32, n)
    _check("lsh_sort_static_scratch",
           _lib.lsh_sort_static_scratch(ctypes.byref(cfg), _ptr(buckets), _ptr(perm),
                                        _ptr(inv_perm), _stream(stream)))


def lsh_o_rounds_bytes(cfg: LshConfig) -> int:
    return int(_lib.lsh_o_rounds_bytes(ctypes.byref(cfg)))


def _expect_o_rounds(cfg: LshConfig, t):
    """o_rounds is an opaque device byte buffer of lsh_o_rounds_bytes(cfg) bytes
    (fp32 rows, or a header and fp16 rows for LSH_O_F16_SCALED)."""
    need = lsh_o_rounds_bytes(cfg)
    if not (isinstance(t, torch.Tensor) and t.dtype == torch.uint8 and t.is_contiguous()
            and t.numel() >= need):
        raise ValueError(f"o_rounds: expected a contiguous uint8 tensor of >= {need} bytes")


def lsh_chunk_attend(cfg: LshConfig, qk, v, buckets, perm, o_rounds, lse, stream=None):
    b, H, L, d, R = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_rounds
    dt = _dtype_of(cfg)
    _expect(qk, (b, H, L, d), dt, "qk")
    _expect(v, (b, H, L, d), dt, "v")
    _expect(buckets, (b, H, R, L), torch.int32, "buckets")
    _expect(perm, (b, H, R, L), torch.int32, "perm")
    _expect_o_rounds(cfg, o_rounds)
    _expect(lse, (b, H, R, L), torch.float32, "lse")
    _check("lsh_chunk_attend",
           _lib.lsh_chunk_attend(ctypes.byref(cfg), _ptr(qk), _ptr(v), _ptr(buckets), _ptr(perm),
                                 _ptr(o_rounds), _ptr(lse), _stream(stream)))


def lsh_union_workspace_bytes(cfg: LshConfig) -> int:
    return int(_lib.lsh_union_workspace_bytes(ctypes.byref(cfg)))


def lsh_chunk_attend_union(cfg: LshConfig, qk, v, buckets, perm, inv_perm, o_rounds, lse,
                           workspace, stream=None):
    b, H, L, d, R = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_rounds
    dt = _dtype_of(cfg)
    _expect(qk, (b, H, L, d), dt, "qk")
    _expect(v, (b, H, L, d), dt, "v")
    for t, n in ((buckets, "buckets"), (perm, "perm"), (inv_perm, "inv_perm")):
        _expect(t, (b, H, R, L), torch.int32, n)
    _expect_o_rounds(cfg, o_rounds)
    _expect(lse, (b, H, R, L), torch.float32, "lse")
    _check("lsh_chunk_attend_union",
           _lib.lsh_chunk_attend_union(ctypes.byref(cfg), _ptr(qk), _ptr(v), _ptr(buckets),
                                       _ptr(perm), _ptr(inv_perm), _ptr(o_rounds), _ptr(lse),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def lsh_unsort_combine(cfg: LshConfig, o_rounds, lse, inv_perm, v, y, stream=None):
    b, H, L, d, R = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_rounds
    _expect_o_rounds(cfg, o_rounds)
    _expect(lse, (b, H, R, L), torch.float32, "lse")
    _expect(inv_perm, (b, H, R, L), torch.int32, "inv_perm")
    _expect(v, (b, H, L, d), _dtype_of(cfg), "v")
    _expect(y, (b, H, L, d), torch.float32, "y")
    _check("lsh_unsort_combine",
           _lib.lsh_unsort_combine(ctypes.byref(cfg), _ptr(o_rounds), _ptr(lse), _ptr(inv_perm),
                                   _ptr(v), _ptr(y), _stream(stream)))


def lsh_local_attend(cfg: LshConfig, n_before: int, n_after: int, qk, v, y, lse, stream=None):
    b, H, L, d = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim
    dt = _dtype_of(cfg)
    _expect(qk, (b, H, L, d), dt, "qk")
    _expect(v, (b, H, L, d), dt, "v")
    _expect(y, (b, H, L, d), torch.float32, "y")
    _expect(lse, (b, H, L), torch.float32, "lse")
    _check("lsh_local_attend",
           _lib.lsh_local_attend(ctypes.byref(cfg), int(n_before), int(n_after), _ptr(qk), _ptr(v),
                                 _ptr(y), _ptr(lse), _stream(stream)))


class Local:
    """Output buffers of local chunked attention for one problem size."""

    def __init__(self, cfg: LshConfig, n_before: int, n_after: int, device="cuda"):
        b, H, L, d = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim
        self.cfg, self.n_before, self.n_after = cfg, n_before, n_after
        self.y = torch.empty((b, H, L, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((b, H, L), dtype=torch.float32, device=device)
        self._checked = None   # the inputs of the last fully checked call

    @staticmethod
    def _key(qk, v):
        return (qk.data_ptr(), v.data_ptr(), qk.dtype, v.dtype, tuple(qk.shape), tuple(v.shape),
                qk.stride(), v.stride(), qk.device, v.device)

    def run(self, qk, v, stream=None):
        # One call is one short kernel: repeating the Python-side checks for
        # the very tensors checked last time would cost more host time than
        # the kernel takes on the GPU.
        key = self._key(qk, v)
        if key != self._checked:
            lsh_local_attend(self.cfg, self.n_before, self.n_after, qk, v, self.y, self.lse, stream)
            self._checked = key
            return self.y
        _check("lsh_local_attend",
               _lib.lsh_local_attend(ctypes.byref(self.cfg), self.n_before, self.n_after, key[0],
                                     key[1], self.y.data_ptr(), self.lse.data_ptr(),
                                     _stream(stream)))
        return self.y


class Forward:
    """Device buffers for one problem size plus the four calls in order.

    Allocation happens here (torch device memory), never inside the calls;
    ``run`` enqueues hash -> sort -> chunk attention -> unsort + combine on the
    current stream (or ``stream``).
    """

    def __init__(self, cfg: LshConfig, device="cuda"):
        b, H, L, d, R = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_rounds
        self.cfg = cfg
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.buckets = torch.empty((b, H, R, L), **i32)
        self.perm = torch.empty((b, H, R, L), **i32)
        self.inv_perm = torch.empty((b, H, R, L), **i32)
        # per-round outputs: an opaque buffer in the library's layout
        self.o_rounds = torch.empty(max(16, lsh_o_rounds_bytes(cfg)), dtype=torch.uint8,
                                    device=device)
        self.lse = torch.empty((b, H, R, L), **f32)
        self.y = torch.empty((b, H, L, d), **f32)
        nbytes = max(16, lsh_sort_workspace_bytes(cfg))
        self.workspace = torch.empty(((nbytes + 15) // 16) * 16, dtype=torch.uint8, device=device)
        self.fallback_rows = torch.zeros(1, **i32)
        self.union_workspace = None   # allocated by the first attend_union

    def hash(self, qk, rot, stream=None):
        lsh_hash(self.cfg, qk, rot, self.buckets, self.fallback_rows, stream)

    def sort(self, stream=None):
        lsh_sort(self.cfg, self.buckets, self.perm, self.inv_perm, self.workspace, stream)

    def attend(self, qk, v, stream=None):
        lsh_chunk_attend(self.cfg, qk, v, self.buckets, self.perm, self.o_rounds, self.lse, stream)

    def attend_union(self, qk, v, stream=None):
        """The set reading of the union over rounds (see lsh_chunk_attend_union)."""
        if self.union_workspace is None:
            nbytes = lsh_union_workspace_bytes(self.cfg)
            if nbytes == 0:
                raise LshError("lsh_union_workspace_bytes", LSH_ERR_UNSUPPORTED,
                               "shape not supported by the set-union attention")
            self.union_workspace = torch.empty(((nbytes + 15) // 16) * 16, dtype=torch.uint8,
                                               device=self.y.device)
        lsh_chunk_attend_union(self.cfg, qk, v, self.buckets, self.perm, self.inv_perm,
                               self.o_rounds, self.lse, self.union_workspace, stream)

    def combine(self, v, stream=None):
        lsh_unsort_combine(self.cfg, self.o_rounds, self.lse, self.inv_perm, v, self.y, stream)

    def run(self, qk, v, rot, stream=None, union=False):
        self.hash(qk, rot, stream)
        self.sort(stream)
        if union:
            self.attend_union(qk, v, stream)
        else:
            self.attend(qk, v, stream)
        self.combine(v, stream)
        return self.y


# ----------------------------------------------------------------- layer
def make_layer_config(w) -> LshLayerConfig:
    """LshLayerConfig of a synth.LayerWorkload."""
    return LshLayerConfig(w.batch, w.seq_len, w.d_model, w.d_ff, w.n_buckets, w.n_rounds,
                          int(bool(w.causal)), int(bool(w.self_mask)), w.ffn_chunk)


def attention_config(lc: LshLayerConfig) -> LshConfig:
    """The LshConfig of the layer's attention (bf16, d_model / 64 heads)."""
    return make_config(lc.batch, lc.d_model // 64, lc.seq_len, lc.n_buckets, lc.n_rounds,
                       lc.causal, lc.self_mask, "bf16", o_format=LSH_O_F16_SCALED)


def _layer_shapes(lc):
    b, L, D, F, H = lc.batch, lc.seq_len, lc.d_model, lc.d_ff, lc.d_model // 64
    return dict(stream=(b, L, D), heads=(b, H, L, 64))


def lsh_project_qkv(lc: LshLayerConfig, x, w_qk, w_v, qk, v, stream=None):
    sh = _layer_shapes(lc)
    D = lc.d_model
    _expect(x, sh["stream"], torch.float32, "x")
    _expect(w_qk, (D, D), torch.bfloat16, "w_qk")
    _expect(w_v, (D, D), torch.bfloat16, "w_v")
    _expect(qk, sh["heads"], torch.bfloat16, "qk")
    _expect(v, sh["heads"], torch.bfloat16, "v")
    _check("lsh_project_qkv", _lib.lsh_project_qkv(ctypes.byref(lc), _ptr(x), _ptr(w_qk),
                                                   _ptr(w_v), _ptr(qk), _ptr(v), _stream(stream)))


def lsh_project_out(lc: LshLayerConfig, y_att, w_o, resid, subtract, out, stream=None):
    sh = _layer_shapes(lc)
    _expect(y_att, sh["heads"], torch.float32, "y_att")
    _expect(w_o, (lc.d_model, lc.d_model), torch.bfloat16, "w_o")
    _expect(resid, sh["stream"], torch.float32, "resid")
    _expect(out, sh["stream"], torch.float32, "out")
    _check("lsh_project_out", _lib.lsh_project_out(ctypes.byref(lc), _ptr(y_att), _ptr(w_o),
                                                   _ptr(resid), int(bool(subtract)), _ptr(out),
                                                   _stream(stream)))


def lsh_ffn_workspace_bytes(lc: LshLayerConfig) -> int:
    return int(_lib.lsh_ffn_workspace_bytes(ctypes.byref(lc)))


def lsh_ffn(lc: LshLayerConfig, x, w_1, b_1, w_2, b_2, resid, subtract, out, workspace,
            stream=None):
    sh = _layer_shapes(lc)
    D, F = lc.d_model, lc.d_ff
    for t, n in ((x, "x"), (resid, "resid"), (out, "out")):
        _expect(t, sh["stream"], torch.float32, n)
    _expect(w_1, (F, D), torch.bfloat16, "w_1")
    _expect(b_1, (F,), torch.float32, "b_1")
    _expect(w_2, (D, F), torch.bfloat16, "w_2")
    _expect(b_2, (D,), torch.float32, "b_2")
    _check("lsh_ffn", _lib.lsh_ffn(ctypes.byref(lc), _ptr(x), _ptr(w_1), _ptr(b_1), _ptr(w_2),
                                   _ptr(b_2), _ptr(resid), int(bool(subtract)), _ptr(out),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def lsh_layer_workspace_bytes(lc: LshLayerConfig) -> int:
    return int(_lib.lsh_layer_workspace_bytes(ctypes.byref(lc)))


class Layer:
    """Weights (device tensors), workspace and the calls of one reversible
    layer.  ``weights`` maps w_qk, w_v, w_o, rot, w_1, w_2 (bf16) and b_1,
    b_2 (fp32) to device tensors of the shapes in include/lsh.h."""

    def __init__(self, lc: LshLayerConfig, weights: dict, device="cuda"):
        self.cfg = lc
        self.w = weights
        D, F, H = lc.d_model, lc.d_ff, lc.d_model // 64
        for name, shape in (("w_qk", (D, D)), ("w_v", (D, D)), ("w_o", (D, D)),
                            ("w_1", (F, D)), ("w_2", (D, F))):
            _expect(weights[name], shape, torch.bfloat16, name)
        if lc.n_buckets > 1:
            _expect(weights["rot"], (H, lc.n_rounds, lc.n_buckets // 2, 64), torch.bfloat16, "rot")
        _expect(weights["b_1"], (F,), torch.float32, "b_1")
        _expect(weights["b_2"], (D,), torch.float32, "b_2")
        self.cw = LshLayerWeights(*[None if (k == "rot" and lc.n_buckets == 1)
                                    else weights[k].data_ptr()
                                    for k in ("w_qk", "w_v", "w_o", "rot", "w_1", "b_1", "w_2",
                                              "b_2")])
        nbytes = max(16, lsh_layer_workspace_bytes(lc))
        self.workspace = torch.empty(((nbytes + 15) // 16) * 16, dtype=torch.uint8, device=device)

    def _run(self, fn, name, a, b, c, d, stream):
        sh = _layer_shapes(self.cfg)["stream"]
        for t, n in ((a, "in1"), (b, "in2"), (c, "out1"), (d, "out2")):
            _expect(t, sh, torch.float32, n)
        _check(name, fn(ctypes.byref(self.cfg), ctypes.byref(self.cw), _ptr(a), _ptr(b), _ptr(c),
                        _ptr(d), _ptr(self.workspace),
                        self.workspace.numel() * self.workspace.element_size(), _stream(stream)))

    def forward(self, x1, x2, y1, y2, stream=None):
        self._run(_lib.lsh_reversible_forward, "lsh_reversible_forward", x1, x2, y1, y2, stream)

    def inverse(self, y1, y2, x1, x2, stream=None):
        self._run(_lib.lsh_reversible_inverse, "lsh_reversible_inverse", y1, y2, x1, x2, stream)


def layer_weights_to_device(inputs: dict, device="cuda") -> dict:
    """synth.make_layer_inputs weights -> device tensors (bf16 / fp32)."""
    out = {}
    for k in ("w_qk", "w_v", "w_o", "rot", "w_1", "w_2"):
        out[k] = to_device(inputs[k], "bf16", device)
    for k in ("b_1", "b_2"):
        out[k] = to_device(inputs[k], "f32", device)
    return out


def to_device(stored, dtype: str, device="cuda"):
    """numpy storage from synth (uint16 bf16 bits or float32) -> device tensor."""
    import numpy as np
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32))
    return t.to(device)
