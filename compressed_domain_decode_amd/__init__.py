"""compressed_domain_decode_amd -- TurboQuant-style KV-cache compression and
compressed-domain decode attention for MI355X (gfx950).

A thin ctypes binding over libtq.so, whose C ABI is declared in include/tq.h.
Every function here has the name of the C entry point it wraps and does only
argument marshalling: torch tensors supply device pointers and strides, and
torch's current HIP stream is passed through. All computation happens in the
library's HIP kernels. If libtq.so is missing this package raises on import;
there is no fallback path.

Build the library first:  python compressed_domain_decode_amd/build.py
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIB_PATH names another build of the same sources (the sanitizer build of
# the host code used by the CPU tests); by default the in-tree libtq.so.
LIB_PATH = os.environ.get("TQ_LIB_PATH") or os.path.join(_HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_WORKSPACE = -3
TQ_ERR_HIP = -4
TQ_ERR_NOMEM = -5

# C symbols the header declares; the ABI test checks the library exports each.
EXPORTED = (
    "tq_codec_init", "tq_codec_destroy", "tq_codec_tables", "tq_codec_info", "tq_row_bytes",
    "tq_encode", "tq_encode_kv", "tq_attend_workspace_bytes", "tq_decode_attend_multi",
    "tq_attend_multi_workspace_bytes", "tq_decode_attend_mixed", "tq_decode_attend_raw_k",
    "tq_codec_init_prod", "tq_encode_prod", "tq_decode_attend_prod", "tq_decode_attend", "tq_attend_num_splits",
    "tq_status_string", "tq_last_error", "tq_set_split_events", "tq_stream_read",
    "tq_stream_read_resident",
    "tq_cache_init", "tq_cache_destroy", "tq_cache_state", "tq_cache_append",
    "tq_cache_workspace_bytes", "tq_cache_attend", "tq_codec_init_dense",
    "tq_decode_attend_noalloc",
)


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python compressed_domain_decode_amd/build.py` "
        "(the HIP library is required, there is no CPU fallback)")

# The library links libamdhip64.so.7 by soname. torch ships its own copy of the
# HIP runtime; importing torch first makes the loader reuse that copy, so the
# process holds one HIP runtime and device pointers / streams are shared.
import torch  # noqa: E402,F401  (loaded for its HIP runtime, before libtq.so)

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_lib.tq_codec_init.argtypes = [_I, _I, ctypes.c_uint64, ctypes.POINTER(_P)]
_lib.tq_codec_init.restype = _I
_lib.tq_codec_init_dense.argtypes = [_I, _I, _P, ctypes.POINTER(_P)]
_lib.tq_codec_init_dense.restype = _I
_lib.tq_codec_destroy.argtypes = [_P]
_lib.tq_codec_destroy.restype = None
_lib.tq_codec_tables.argtypes = [_P, _P, _P, _P]
_lib.tq_codec_tables.restype = _I
_lib.tq_codec_info.argtypes = [_P, ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_uint64)]
_lib.tq_codec_info.restype = _I
_lib.tq_row_bytes.argtypes = [_I, _I]
_lib.tq_row_bytes.restype = _I
_lib.tq_encode.argtypes = [_P, _P, _I, _I, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64, _P]
_lib.tq_encode.restype = _I


class _EncodeJob(ctypes.Structure):
    """Mirror of tq_encode_job."""
    _fields_ = [("codec", _P), ("x_fp16", _P), ("x_stride_tok", _I64), ("x_stride_head", _I64),
                ("codes", _P), ("c_stride_tok", _I64), ("c_stride_head", _I64),
                ("norms", _P), ("n_stride_tok", _I64), ("n_stride_head", _I64)]


_lib.tq_encode_kv.argtypes = [ctypes.POINTER(_EncodeJob), ctypes.POINTER(_EncodeJob), _I, _I, _P]
_lib.tq_encode_kv.restype = _I
_lib.tq_attend_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.tq_attend_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_attend_num_splits.argtypes = [_I, _I, _I, _I, _I]
_lib.tq_attend_num_splits.restype = _I
_lib.tq_decode_attend.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _I, _P, _I,
                                  ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_attend.restype = _I
_lib.tq_decode_attend_noalloc.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _I, _P, _I,
                                          ctypes.c_float, _P, _P]
_lib.tq_decode_attend_noalloc.restype = _I
TQ_NOALLOC_SCRATCH_BYTES = 8 << 20  # include/tq.h
_lib.tq_decode_attend_multi.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _I,
                                        ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_attend_multi.restype = _I
_lib.tq_decode_attend_mixed.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _I, _P, _I,
                                        _P, _P, _I, _P, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                        _P]
_lib.tq_decode_attend_mixed.restype = _I
_lib.tq_decode_attend_raw_k.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _I, _P, _I,
                                        ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_attend_raw_k.restype = _I
_lib.tq_codec_init_prod.argtypes = [_I, _I, ctypes.c_uint64, ctypes.POINTER(_P)]
_lib.tq_codec_init_prod.restype = _I
_lib.tq_encode_prod.argtypes = [_P, _P, _I, _I, _I64, _I64, _P, _I64, _I64, _P, _I64, _I64,
                                _P, _I64, _I64, _P, _I64, _I64, _P]
_lib.tq_encode_prod.restype = _I
_lib.tq_decode_attend_prod.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P,
                                       _I, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_attend_prod.restype = _I
_lib.tq_attend_multi_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
_lib.tq_attend_multi_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_set_split_events.argtypes = [_P, _P]
_lib.tq_stream_read.restype = _I
_lib.tq_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.tq_stream_read_resident.restype = _I
_lib.tq_stream_read_resident.argtypes = [_P, ctypes.c_size_t, _P, _P]
_lib.tq_set_split_events.restype = _I


class _CacheDesc(ctypes.Structure):
    """Mirror of tq_cache_desc."""
    _fields_ = [("batch", _I), ("n_kv_heads", _I), ("max_ctx", _I), ("group_size", _I),
                ("k_codes", _P), ("k_norms", _P), ("v_codes", _P), ("v_norms", _P),
                ("pending_k", _P), ("pending_v", _P), ("packed_len", _P), ("pending_len", _P)]


_lib.tq_cache_init.argtypes = [_P, _P, ctypes.POINTER(_CacheDesc), ctypes.POINTER(_P)]
_lib.tq_cache_init.restype = _I
_lib.tq_cache_destroy.argtypes = [_P]
_lib.tq_cache_destroy.restype = None
_lib.tq_cache_state.argtypes = [_P, ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.tq_cache_state.restype = _I
_lib.tq_cache_append.argtypes = [_P, _P, _P, _I, _P]
_lib.tq_cache_append.restype = _I
_lib.tq_cache_workspace_bytes.argtypes = [_P, _I]
_lib.tq_cache_workspace_bytes.restype = ctypes.c_size_t
_lib.tq_cache_attend.argtypes = [_P, _P, _I, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_cache_attend.restype = _I
_lib.tq_status_string.argtypes = [_I]
_lib.tq_status_string.restype = ctypes.c_char_p
_lib.tq_last_error.argtypes = []
_lib.tq_last_error.restype = ctypes.c_char_p


def _status_name(s: int) -> str:
    return _lib.tq_status_string(s).decode()


def tq_status_string(status: int) -> str:
    return _status_name(status)


def tq_last_error() -> str:
    return _lib.tq_last_error().decode()


def _check(status: int):
    if status != TQ_OK:
        raise TQError(status, tq_last_error())


def _stream_ptr(stream):
    """A hipStream_t as an int: explicit value, a torch stream, or torch's current one."""
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(fn: str, specs, contiguous: bool = True) -> None:
    """Check (name, tensor, dtype) triples before anything is enqueued: every
    dtype first, then that all tensors sit on the current GPU, then (unless
    contiguous is False) that each is contiguous. The C ABI takes raw pointers
    and byte strides, so a tensor of another dtype or on the host would be
    misread or written past its end by the kernels."""
    import torch
    for name, t, dt in specs:
        if t.dtype != dt:
            raise TQError(TQ_ERR_INVALID_ARG, f"{fn}: {name} must be {dt}, got {t.dtype}")
    for name, t, _ in specs:
        if t.device.type != "cuda":
            raise TQError(TQ_ERR_INVALID_ARG, f"{fn}: {name} must be a GPU tensor, got {t.device}")
    cur = torch.cuda.current_device()
    for name, t, _ in specs:
        if t.device.index != cur:
            raise TQError(TQ_ERR_INVALID_ARG,
                          f"{fn}: {name} is on {t.device}, the current device is cuda:{cur}")
    if contiguous:
        for name, t, _ in specs:
            if not t.is_contiguous():
                raise TQError(TQ_ERR_INVALID_ARG, f"{fn}: {name} must be contiguous")


# ------------------------------------------------------------------ codec

class Codec:
    """Owns one tq_codec handle (host memory only)."""

    def __init__(self, handle: int, dim: int, bits: int, seed: int):
        self._h = ctypes.c_void_p(handle)
        self.dim, self.bits, self.seed = dim, bits, seed

    @property
    def handle(self):
        return self._h

    @property
    def row_bytes(self) -> int:
        return self.dim * self.bits // 8

    def close(self):
        if self._h:
            _lib.tq_codec_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __repr__(self):
        return f"Codec(dim={self.dim}, bits={self.bits}, seed={self.seed})"


def tq_codec_init(dim: int, bits: int, seed: int) -> Codec:
    h = ctypes.c_void_p()
    _check(_lib.tq_codec_init(dim, bits, ctypes.c_uint64(seed), ctypes.byref(h)))
    return Codec(h.value, dim, bits, seed)


class DenseCodec(Codec):
    """A dense-rotation codec (head dims with no Walsh-Hadamard transform)."""

    def __repr__(self):
        return f"DenseCodec(dim={self.dim}, bits={self.bits})"


def tq_codec_init_dense(dim: int, bits: int, rotation) -> DenseCodec:
    """rotation: dim x dim fp64 array (sqrt(dim) times an orthogonal matrix),
    copied by the library."""
    import numpy as _np
    m = _np.ascontiguousarray(rotation, dtype=_np.float64)
    if m.shape != (dim, dim):
        raise ValueError(f"rotation must be {dim} x {dim}, got {m.shape}")
    h = ctypes.c_void_p()
    _check(_lib.tq_codec_init_dense(dim, bits, m.ctypes.data_as(ctypes.c_void_p),
                                    ctypes.byref(h)))
    return DenseCodec(h.value, dim, bits, 0)


class ProdCodec(Codec):
    """A TurboQuant-Prod key codec: `bits` total, codes of bits - 1 bits plus a
    dim-bit sketch and a residual norm per row."""

    def __init__(self, handle: int, dim: int, bits: int, seed: int):
        super().__init__(handle, dim, bits, seed)

    @property
    def row_bytes(self) -> int:
        return self.dim * (self.bits - 1) // 8

    @property
    def sketch_bytes(self) -> int:
        return self.dim // 8

    def __repr__(self):
        return f"ProdCodec(dim={self.dim}, bits={self.bits}, seed={self.seed})"


def tq_codec_init_prod(dim: int, bits: int, seed: int) -> ProdCodec:
    h = ctypes.c_void_p()
    _check(_lib.tq_codec_init_prod(dim, bits, ctypes.c_uint64(seed), ctypes.byref(h)))
    return ProdCodec(h.value, dim, bits, seed)


def tq_encode_prod(codec: ProdCodec, x, codes, sketch, norms, rnorms, stream=None) -> None:
    """Encode x[n_tok][n_head][dim] with a Prod codec into codes
    [n_tok][n_head][row_bytes], sketch [n_tok][n_head][dim/8] (uint8), norms and
    residual norms [n_tok][n_head] (fp32); any strides, last dims contiguous."""
    import torch
    j = _encode_views(codec, x, codes, norms, "tq_encode_prod")
    _require("tq_encode_prod", (("sketch", sketch, torch.uint8), ("rnorms", rnorms, torch.float32)),
             contiguous=False)
    n_tok, n_head = x.shape[0], x.shape[1]
    if tuple(sketch.shape) != (n_tok, n_head, codec.sketch_bytes) or sketch.stride(2) != 1:
        raise TQError(TQ_ERR_INVALID_ARG, "sketch must be [n_tok][n_head][dim/8], row contiguous")
    if tuple(rnorms.shape) != (n_tok, n_head):
        raise TQError(TQ_ERR_INVALID_ARG, "rnorms must be [n_tok][n_head]")
    _check(_lib.tq_encode_prod(j.codec, j.x_fp16, n_tok, n_head, j.x_stride_tok,
                               j.x_stride_head, j.codes, j.c_stride_tok, j.c_stride_head,
                               _ptr(sketch), sketch.stride(0), sketch.stride(1), j.norms,
                               j.n_stride_tok, j.n_stride_head, _ptr(rnorms), rnorms.stride(0),
                               rnorms.stride(1), _stream_ptr(stream)))


def tq_codec_destroy(codec: Codec) -> None:
    codec.close()


def tq_codec_tables(codec: Codec):
    """(signs int8[dim], centroids float32[2^bits], boundaries float32[2^bits-1]) host copies."""
    bits = codec.bits - 1 if isinstance(codec, ProdCodec) else codec.bits  # Lloyd-Max part
    s = np.zeros(codec.dim, np.int8)
    c = np.zeros(1 << bits, np.float32)
    b = np.zeros((1 << bits) - 1, np.float32)
    _check(_lib.tq_codec_tables(codec.handle, s.ctypes.data, c.ctypes.data, b.ctypes.data))
    return s, c, b


def tq_codec_info(codec: Codec):
    d, b, s = _I(), _I(), ctypes.c_uint64()
    _check(_lib.tq_codec_info(codec.handle, ctypes.byref(d), ctypes.byref(b), ctypes.byref(s)))
    return d.value, b.value, s.value


def tq_row_bytes(dim: int, bits: int) -> int:
    return _lib.tq_row_bytes(dim, bits)


# ------------------------------------------------------------------ encode

def _encode_views(codec: Codec, x, codes, norms, fn="tq_encode"):
    import torch
    _require(fn, (("x", x, torch.float16), ("codes", codes, torch.uint8),
                  ("norms", norms, torch.float32)), contiguous=False)
    n_tok, n_head, d = x.shape
    if d != codec.dim or x.stride(2) != 1:
        raise TQError(TQ_ERR_INVALID_ARG, "x must be [n_tok][n_head][dim] with contiguous dim")
    if tuple(codes.shape) != (n_tok, n_head, codec.row_bytes) or codes.stride(2) != 1:
        raise TQError(TQ_ERR_INVALID_ARG, "codes must be [n_tok][n_head][row_bytes], row contiguous")
    if tuple(norms.shape) != (n_tok, n_head):
        raise TQError(TQ_ERR_INVALID_ARG, "norms must be [n_tok][n_head]")
    return _EncodeJob(codec.handle, _ptr(x), x.stride(0), x.stride(1), _ptr(codes),
                      codes.stride(0), codes.stride(1), _ptr(norms), norms.stride(0),
                      norms.stride(1))


def tq_encode(codec: Codec, x, codes, norms, stream=None) -> None:
    """Encode x[n_tok][n_head][dim] (fp16, any strides, last dim contiguous) into
    codes[n_tok][n_head][row_bytes] (uint8) and norms[n_tok][n_head] (fp32).
    Strides are read from the tensors, so views into a [B][H][T][...] cache
    (e.g. cache[b].transpose(0, 1)[t0:t1]) encode in place."""
    j = _encode_views(codec, x, codes, norms)
    n_tok, n_head = x.shape[0], x.shape[1]
    _check(_lib.tq_encode(j.codec, j.x_fp16, n_tok, n_head, j.x_stride_tok, j.x_stride_head,
                          j.codes, j.c_stride_tok, j.c_stride_head, j.norms, j.n_stride_tok,
                          j.n_stride_head, _stream_ptr(stream)))


def tq_encode_kv(kc: Codec, k, k_codes, k_norms, vc: Codec, v, v_codes, v_norms,
                 stream=None) -> None:
    """tq_encode of K (with kc) and of V (with vc) in one launch; k and v have
    the same [n_tok][n_head] grid, the other rules are tq_encode's."""
    if tuple(k.shape[:2]) != tuple(v.shape[:2]):
        raise TQError(TQ_ERR_INVALID_ARG, "k and v must share [n_tok][n_head]")
    jk = _encode_views(kc, k, k_codes, k_norms, "tq_encode_kv")
    jv = _encode_views(vc, v, v_codes, v_norms, "tq_encode_kv")
    _check(_lib.tq_encode_kv(ctypes.byref(jk), ctypes.byref(jv), k.shape[0], k.shape[1],
                             _stream_ptr(stream)))


# ------------------------------------------------------------------ attend

def _attend_tensors(fn, q, k_codes, k_norms, v_codes, v_norms, lengths, out, workspace,
                    extra=()):
    """The dtype / device / layout checks every attend call shares (workspace
    None: the call takes none)."""
    import torch
    specs = [("q", q, torch.float16), ("k_codes", k_codes, torch.uint8),
             ("k_norms", k_norms, torch.float32), ("v_codes", v_codes, torch.uint8),
             ("v_norms", v_norms, torch.float32), ("lengths", lengths, torch.int32),
             ("out", out, torch.float32)]
    if workspace is not None:
        specs.append(("workspace", workspace, torch.uint8))
    _require(fn, tuple(specs) + tuple(extra))


def tq_attend_workspace_bytes(batch: int, n_q_heads: int, n_kv_heads: int, dim: int,
                              max_len: int) -> int:
    return int(_lib.tq_attend_workspace_bytes(batch, n_q_heads, n_kv_heads, dim, max_len))


def tq_attend_num_splits(batch: int, n_q_heads: int, n_kv_heads: int, dim: int,
                         max_len: int) -> int:
    return int(_lib.tq_attend_num_splits(batch, n_q_heads, n_kv_heads, dim, max_len))


def tq_decode_attend(kc: Codec, vc: Codec, q, k_codes, k_norms, v_codes, v_norms, lengths,
                     max_len: int, scale: float, out, workspace, stream=None) -> None:
    """q [B][Hq][d] fp16; codes [B][Hkv][max_ctx][row] uint8; norms [B][Hkv][max_ctx] fp32;
    lengths int32[B] (device); out [B][Hq][d] fp32; workspace uint8 tensor of at least
    tq_attend_workspace_bytes(...) bytes. All contiguous."""
    B, Hq, d = q.shape
    Hkv, max_ctx = k_norms.shape[1], k_norms.shape[2]
    _attend_tensors("tq_decode_attend", q, k_codes, k_norms, v_codes, v_norms, lengths, out,
                    workspace)
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(v_norms.shape) != (B, Hkv, max_ctx) or tuple(out.shape) != (B, Hq, d) or \
       tuple(lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / output shapes disagree")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_decode_attend(kc.handle, vc.handle, _ptr(q), B, Hq, Hkv, _ptr(k_codes),
                                 _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), max_ctx,
                                 _ptr(lengths), int(max_len), float(scale), _ptr(out),
                                 _ptr(workspace), nbytes, _stream_ptr(stream)))


def tq_decode_attend_noalloc(kc: Codec, vc: Codec, q, k_codes, k_norms, v_codes, v_norms,
                             lengths, max_len: int, scale: float, out, stream=None) -> None:
    """tq_decode_attend with the library's fixed per-GPU scratch array in place
    of a workspace (nothing is allocated); the arguments otherwise as there.
    Calls that overlap on one GPU share that array and race."""
    B, Hq, d = q.shape
    Hkv, max_ctx = k_norms.shape[1], k_norms.shape[2]
    _attend_tensors("tq_decode_attend_noalloc", q, k_codes, k_norms, v_codes, v_norms, lengths,
                    out, None)
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(v_norms.shape) != (B, Hkv, max_ctx) or tuple(out.shape) != (B, Hq, d) or \
       tuple(lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / output shapes disagree")
    _check(_lib.tq_decode_attend_noalloc(kc.handle, vc.handle, _ptr(q), B, Hq, Hkv,
                                         _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                         _ptr(v_norms), max_ctx, _ptr(lengths), int(max_len),
                                         float(scale), _ptr(out), _stream_ptr(stream)))


def tq_attend_multi_workspace_bytes(batch: int, n_query_tokens: int, n_q_heads: int,
                                    n_kv_heads: int, dim: int, max_len: int) -> int:
    return int(_lib.tq_attend_multi_workspace_bytes(batch, n_query_tokens, n_q_heads,
                                                    n_kv_heads, dim, max_len))


def tq_decode_attend_multi(kc: Codec, vc: Codec, q, k_codes, k_norms, v_codes, v_norms,
                           lengths, max_len: int, scale: float, out, workspace,
                           stream=None) -> None:
    """q [B][S][Hq][d] fp16 (S query tokens, causal among themselves); out
    [B][S][Hq][d] fp32; lengths count the cache rows including the S new
    ones; the rest as tq_decode_attend."""
    B, S, Hq, d = q.shape
    Hkv, max_ctx = k_norms.shape[1], k_norms.shape[2]
    _attend_tensors("tq_decode_attend_multi", q, k_codes, k_norms, v_codes, v_norms, lengths, out,
                    workspace)
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(v_norms.shape) != (B, Hkv, max_ctx) or tuple(out.shape) != (B, S, Hq, d) or \
       tuple(lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / output shapes disagree")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_decode_attend_multi(kc.handle, vc.handle, _ptr(q), B, S, Hq, Hkv,
                                       _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                       _ptr(v_norms), max_ctx, _ptr(lengths), int(max_len),
                                       float(scale), _ptr(out), _ptr(workspace), nbytes,
                                       _stream_ptr(stream)))


def tq_decode_attend_mixed(kc: Codec, vc: Codec, q, k_codes, k_norms, v_codes, v_norms,
                           lengths, max_len: int, raw_k, raw_v, raw_lengths, scale: float, out,
                           workspace, stream=None) -> None:
    """tq_decode_attend over the packed rows plus raw fp16 rows raw_k / raw_v
    [B][Hkv][max_raw][d] (raw_lengths int32[B] on the device); the softmax runs
    over both. The rest as tq_decode_attend."""
    B, Hq, d = q.shape
    Hkv, max_ctx = k_norms.shape[1], k_norms.shape[2]
    import torch
    _attend_tensors("tq_decode_attend_mixed", q, k_codes, k_norms, v_codes, v_norms, lengths,
                    out, workspace,
                    (("raw_k", raw_k, torch.float16), ("raw_v", raw_v, torch.float16),
                     ("raw_lengths", raw_lengths, torch.int32)))
    max_raw = raw_k.shape[2]
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(v_norms.shape) != (B, Hkv, max_ctx) or tuple(out.shape) != (B, Hq, d) or \
       tuple(lengths.shape) != (B,) or tuple(raw_k.shape) != (B, Hkv, max_raw, d) or \
       tuple(raw_v.shape) != (B, Hkv, max_raw, d) or tuple(raw_lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / raw segment / output shapes disagree")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_decode_attend_mixed(kc.handle, vc.handle, _ptr(q), B, Hq, Hkv, _ptr(k_codes),
                                       _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), max_ctx,
                                       _ptr(lengths), int(max_len), _ptr(raw_k), _ptr(raw_v),
                                       max_raw, _ptr(raw_lengths), float(scale), _ptr(out),
                                       _ptr(workspace), nbytes, _stream_ptr(stream)))


def tq_decode_attend_raw_k(vc: Codec, q, k, v_codes, v_norms, lengths, max_len: int,
                           scale: float, out, workspace, stream=None) -> None:
    """Raw fp16 keys k [B][Hkv][max_ctx][d] with packed values; the rest as
    tq_decode_attend."""
    B, Hq, d = q.shape
    Hkv, max_ctx = v_norms.shape[1], v_norms.shape[2]
    import torch
    _require("tq_decode_attend_raw_k",
             (("q", q, torch.float16), ("k", k, torch.float16), ("v_codes", v_codes, torch.uint8),
              ("v_norms", v_norms, torch.float32), ("lengths", lengths, torch.int32),
              ("out", out, torch.float32), ("workspace", workspace, torch.uint8)))
    if tuple(k.shape) != (B, Hkv, max_ctx, d) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(out.shape) != (B, Hq, d) or tuple(lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / output shapes disagree")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_decode_attend_raw_k(vc.handle, _ptr(q), B, Hq, Hkv, _ptr(k), _ptr(v_codes),
                                       _ptr(v_norms), max_ctx, _ptr(lengths), int(max_len),
                                       float(scale), _ptr(out), _ptr(workspace), nbytes,
                                       _stream_ptr(stream)))


def tq_decode_attend_prod(kc: ProdCodec, vc: Codec, q, k_codes, k_sketch, k_norms, k_rnorms,
                          v_codes, v_norms, lengths, max_len: int, scale: float, out, workspace,
                          stream=None) -> None:
    """TurboQuant-Prod keys (codes, sketch [B][Hkv][T][d/8], norms, residual
    norms) with packed values; the rest as tq_decode_attend."""
    B, Hq, d = q.shape
    Hkv, max_ctx = k_norms.shape[1], k_norms.shape[2]
    import torch
    _attend_tensors("tq_decode_attend_prod", q, k_codes, k_norms, v_codes, v_norms, lengths, out,
                    workspace,
                    (("k_sketch", k_sketch, torch.uint8), ("k_rnorms", k_rnorms, torch.float32)))
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(k_sketch.shape) != (B, Hkv, max_ctx, kc.sketch_bytes) or \
       tuple(k_rnorms.shape) != (B, Hkv, max_ctx) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(out.shape) != (B, Hq, d) or tuple(lengths.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache / output shapes disagree")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_decode_attend_prod(kc.handle, vc.handle, _ptr(q), B, Hq, Hkv, _ptr(k_codes),
                                      _ptr(k_sketch), _ptr(k_norms), _ptr(k_rnorms),
                                      _ptr(v_codes), _ptr(v_norms), max_ctx, _ptr(lengths),
                                      int(max_len), float(scale), _ptr(out), _ptr(workspace),
                                      nbytes, _stream_ptr(stream)))


def tq_set_split_events(before, after) -> None:
    """Record caller-owned hipEvent_t handles (ints) around the split-attend
    kernel of subsequent tq_decode_attend calls on this thread; None, None stops."""
    _check(_lib.tq_set_split_events(before, after))


def tq_stream_read(buf, sink, stream=None, resident=False) -> None:
    """Measurement aid: a plain streaming read of the whole (contiguous, 16-byte
    aligned) device tensor buf; sink is a device tensor of at least 4 bytes.
    resident=True reads with the resident-grid design (tq_stream_read_resident)."""
    name = "tq_stream_read_resident" if resident else "tq_stream_read"
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if buf.device.type != "cuda" or sink.device.type != "cuda":
        raise TQError(TQ_ERR_INVALID_ARG, f"{name}: buf and sink must be GPU tensors")
    nbytes = buf.numel() * buf.element_size()
    _check(getattr(_lib, name)(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nbytes),
                               ctypes.c_void_p(sink.data_ptr()), _stream_ptr(stream)))


def library_path() -> str:
    return LIB_PATH


# ------------------------------------------------------------ two-phase cache

class Cache:
    """Handle of a tq_cache. It keeps the caller's buffers referenced for as
    long as the C object holds their pointers."""

    def __init__(self, handle: int, kc: Codec, vc: Codec, buffers: tuple):
        self._h = handle
        self.kc, self.vc = kc, vc
        self.buffers = buffers

    @property
    def handle(self):
        if not self._h:
            raise TQError(TQ_ERR_INVALID_ARG, "cache already destroyed")
        return self._h

    def close(self):
        if self._h:
            _lib.tq_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tq_cache_init(kc: Codec, vc: Codec, k_codes, k_norms, v_codes, v_norms, pending_k,
                  pending_v, packed_len, pending_len) -> Cache:
    """Two-phase cache over caller-owned buffers: packed cache
    [B][Hkv][max_ctx][row] / [B][Hkv][max_ctx], fp16 pending rows
    [B][Hkv][group_size][d], device int32 length arrays [B]."""
    B, Hkv, max_ctx = k_norms.shape
    G = pending_k.shape[2]
    import torch
    _require("tq_cache_init",
             (("k_codes", k_codes, torch.uint8), ("k_norms", k_norms, torch.float32),
              ("v_codes", v_codes, torch.uint8), ("v_norms", v_norms, torch.float32),
              ("pending_k", pending_k, torch.float16), ("pending_v", pending_v, torch.float16),
              ("packed_len", packed_len, torch.int32), ("pending_len", pending_len, torch.int32)))
    if tuple(k_codes.shape) != (B, Hkv, max_ctx, kc.row_bytes) or \
       tuple(v_codes.shape) != (B, Hkv, max_ctx, vc.row_bytes) or \
       tuple(v_norms.shape) != (B, Hkv, max_ctx) or \
       tuple(pending_k.shape) != (B, Hkv, G, kc.dim) or tuple(pending_v.shape) != (B, Hkv, G, kc.dim) or \
       tuple(packed_len.shape) != (B,) or tuple(pending_len.shape) != (B,):
        raise TQError(TQ_ERR_INVALID_ARG, "cache buffer shapes disagree")
    desc = _CacheDesc(B, Hkv, max_ctx, G, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                      _ptr(v_norms), _ptr(pending_k), _ptr(pending_v), _ptr(packed_len),
                      _ptr(pending_len))
    h = _P()
    _check(_lib.tq_cache_init(kc.handle, vc.handle, ctypes.byref(desc), ctypes.byref(h)))
    return Cache(h.value, kc, vc, (k_codes, k_norms, v_codes, v_norms, pending_k, pending_v,
                                   packed_len, pending_len))


def tq_cache_destroy(cache: Cache) -> None:
    cache.close()


def tq_cache_state(cache: Cache):
    """(rows packed, rows pending) per (sequence, KV head)."""
    a, b = _I(), _I()
    _check(_lib.tq_cache_state(cache.handle, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def tq_cache_append(cache: Cache, k, v, stream=None) -> None:
    """Append k, v [B][Hkv][n][d] fp16 (contiguous) to the cache."""
    import torch
    _require("tq_cache_append", (("k", k, torch.float16), ("v", v, torch.float16)))
    if k.shape != v.shape:
        raise TQError(TQ_ERR_INVALID_ARG, "k and v must be of one shape")
    B, Hkv, n, d = k.shape
    pk = cache.buffers[4]
    if (B, Hkv, d) != (pk.shape[0], pk.shape[1], pk.shape[3]):
        raise TQError(TQ_ERR_INVALID_ARG, "rows do not match the cache's batch / heads / dim")
    _check(_lib.tq_cache_append(cache.handle, _ptr(k), _ptr(v), n, _stream_ptr(stream)))


def tq_cache_workspace_bytes(cache: Cache, n_q_heads: int) -> int:
    return int(_lib.tq_cache_workspace_bytes(cache.handle, n_q_heads))


def tq_cache_attend(cache: Cache, q, scale: float, out, workspace, stream=None) -> None:
    """Decode attention of q [B][Hq][d] over the cache's packed and pending rows."""
    import torch
    _require("tq_cache_attend", (("q", q, torch.float16), ("out", out, torch.float32),
                                 ("workspace", workspace, torch.uint8)))
    B, Hq, d = q.shape
    if tuple(out.shape) != (B, Hq, d):
        raise TQError(TQ_ERR_INVALID_ARG, "out shape disagrees with q")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_cache_attend(cache.handle, _ptr(q), Hq, float(scale), _ptr(out),
                                _ptr(workspace), nbytes, _stream_ptr(stream)))
