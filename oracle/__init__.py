"""CPU oracle for compressed-domain KV decode.

TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library (`compressed_domain_decode_amd`) and imports nothing from it.

The arithmetic lives in `tq_oracle.c` (plain C, fp64, no FMA contraction) and
`codebook.py` (Lloyd-Max fixed point). This module only marshals numpy arrays.

Parity status: every function here is pinned by a `-m "not gpu"` test to
something other than itself (closed forms, a published generator test vector,
brute force, the pages' packing example and storage ratios, algebraic
identities); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from . import codebook

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
# TQ_ORACLE_LIB names another build of tq_oracle.c (the sanitizer run of the
# CPU tests); by default the library beside this file, rebuilt when stale.
_LIB_DEFAULT = os.path.join(_HERE, "_tq_oracle.so")
_LIB = os.environ.get("TQ_ORACLE_LIB") or _LIB_DEFAULT
_lock = threading.Lock()
_lib = None

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_DEFAULT):
        tmp = _LIB_DEFAULT + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_DEFAULT)
    return _LIB_DEFAULT


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _LIB == _LIB_DEFAULT and (not os.path.exists(_LIB) or
                                         os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I = ctypes.c_int
            I64 = ctypes.c_int64
            lib.orc_splitmix64.argtypes = [ctypes.c_uint64, I, P]
            lib.orc_hadamard.argtypes = [I, P]
            lib.orc_hadamard.restype = ctypes.c_int
            lib.orc_bucketize.argtypes = [P, I64, P, I, P]
            lib.orc_signs.argtypes = [ctypes.c_uint64, I, P]
            lib.orc_pack.argtypes = [I, I, P, P]
            lib.orc_unpack.argtypes = [I, I, P, P]
            lib.orc_encode.argtypes = [I, I, P, P, P, I64, I64, P, P, P, P]
            lib.orc_dequant.argtypes = [I, I, P, P, P, P, I64, P]
            att = [I, I, I, P, P, P, P, P, I, I, I, P, P, P, P, I, P, ctypes.c_double, P, I, P]
            lib.orc_attend.argtypes = att
            lib.orc_attend_rotated.argtypes = att
            lib.orc_encode_dense.argtypes = [I, I, P, P, P, I64, I64, P, P, P, P]
            lib.orc_dequant_dense.argtypes = [I, I, P, P, P, P, I64, P]
            lib.orc_tree_sum.argtypes = [P, I]
            lib.orc_tree_sum.restype = ctypes.c_double
            for f in ("orc_signs", "orc_encode", "orc_dequant", "orc_attend", "orc_attend_rotated",
                      "orc_encode_dense", "orc_dequant_dense"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


# ------------------------------------------------------------------ codec

def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.uint64)
    _load().orc_splitmix64(ctypes.c_uint64(seed), n, _p(out))
    return out


def signs(seed: int, dim: int) -> np.ndarray:
    out = np.zeros(dim, dtype=np.int8)
    _check(_load().orc_signs(ctypes.c_uint64(seed), dim, _p(out)), "signs")
    return out


class Codec:
    """(dim, bits, seed) -> sign vector and fp32 codebook, oracle side."""

    def __init__(self, dim: int, bits: int, seed: int):
        self.dim, self.bits, self.seed = dim, bits, seed
        self.signs = signs(seed, dim)
        c, b = codebook.tables(bits)
        self.centroids = np.ascontiguousarray(c, dtype=np.float32)
        self.boundaries = np.ascontiguousarray(b, dtype=np.float32)

    @property
    def row_bytes(self) -> int:
        return self.dim * self.bits // 8


def hadamard(d: int) -> np.ndarray:
    out = np.zeros((d, d), dtype=np.float64)
    _check(_load().orc_hadamard(d, _p(out)), "hadamard")
    return out


def bucketize(z: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float64).reshape(-1)
    b = np.ascontiguousarray(boundaries, dtype=np.float32)
    out = np.zeros(z.size, dtype=np.int32)
    _load().orc_bucketize(_p(z), z.size, _p(b), b.size, _p(out))
    return out


# ------------------------------------------------------------------ packing

def pack(idx: np.ndarray, bits: int) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1)
    d = idx.size
    out = np.zeros(d * bits // 8, dtype=np.uint8)
    _load().orc_pack(d, bits, _p(idx), _p(out))
    return out


def unpack(row: np.ndarray, d: int, bits: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8).reshape(-1)
    out = np.zeros(d, dtype=np.int32)
    _load().orc_unpack(d, bits, _p(row), _p(out))
    return out


# ------------------------------------------------------------------ encode

def encode(codec: Codec, x: np.ndarray, want_z: bool = False):
    """Encode rows of x (..., d), fp16 or values exactly representable in fp64.

    Returns (codes uint8 (..., d*bits/8), norms float32 (...), norms64, [z]).
    """
    x = np.asarray(x)
    lead = x.shape[:-1]
    d = x.shape[-1]
    assert d == codec.dim
    xd = np.ascontiguousarray(x.reshape(-1, d), dtype=np.float64)
    n = xd.shape[0]
    codes = np.zeros((n, codec.row_bytes), dtype=np.uint8)
    norms = np.zeros(n, dtype=np.float32)
    norms64 = np.zeros(n, dtype=np.float64)
    z = np.zeros((n, d), dtype=np.float64) if want_z else None
    _check(_load().orc_encode(d, codec.bits, _p(codec.signs), _p(codec.boundaries), _p(xd),
                              n, d, _p(codes), _p(norms), _p(norms64),
                              _p(z) if want_z else None), "encode")
    out = (codes.reshape(*lead, codec.row_bytes), norms.reshape(lead), norms64.reshape(lead))
    if want_z:
        out = out + (z.reshape(*lead, d),)
    return out


def dequant(codec: Codec, codes: np.ndarray, norms: np.ndarray) -> np.ndarray:
    lead = norms.shape
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, codec.row_bytes)
    nr = np.ascontiguousarray(norms, dtype=np.float32).reshape(-1)
    out = np.zeros((nr.size, codec.dim), dtype=np.float64)
    _check(_load().orc_dequant(codec.dim, codec.bits, _p(codec.signs), _p(codec.centroids),
                               _p(c), _p(nr), nr.size, _p(out)), "dequant")
    return out.reshape(*lead, codec.dim)


# ------------------------------------------------------------------ attention

def _attend(fn, kc: Codec, vc: Codec, q, k_codes, k_norms, v_codes, v_norms, lengths,
            scale=None, bh=None):
    q = np.ascontiguousarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, T = k_norms.shape[1], k_norms.shape[2]
    assert k_codes.shape == (B, Hkv, T, kc.row_bytes)
    assert v_codes.shape == (B, Hkv, T, vc.row_bytes)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kcd = np.ascontiguousarray(k_codes, dtype=np.uint8)
    vcd = np.ascontiguousarray(v_codes, dtype=np.uint8)
    knr = np.ascontiguousarray(k_norms, dtype=np.float32)
    vnr = np.ascontiguousarray(v_norms, dtype=np.float32)
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    if bh is None:
        pairs = None
        n = B * Hq
    else:
        pairs = np.ascontiguousarray(np.asarray(bh, dtype=np.int32).reshape(-1, 2))
        n = pairs.shape[0]
    out = np.zeros((n, d), dtype=np.float64)
    _check(fn(d, kc.bits, vc.bits, _p(kc.signs), _p(kc.centroids), _p(vc.signs),
              _p(vc.centroids), _p(q), B, Hq, Hkv, _p(kcd), _p(knr), _p(vcd), _p(vnr), T,
              _p(ln), float(scale), _p(pairs) if pairs is not None else None, n, _p(out)),
           "attend")
    return out.reshape(B, Hq, d) if bh is None else out


def attend(kc, vc, q, k_codes, k_norms, v_codes, v_norms, lengths, scale=None, bh=None):
    """Softmax attention over the dequantised cache (fp64). q: [B][Hq][d];
    codes [B][Hkv][T][row]; norms [B][Hkv][T]. Returns [B][Hq][d] or [n_bh][d]."""
    return _attend(_load().orc_attend, kc, vc, q, k_codes, k_norms, v_codes, v_norms,
                   lengths, scale, bh)


def attend_rotated(kc, vc, q, k_codes, k_norms, v_codes, v_norms, lengths, scale=None, bh=None):
    """The same attention taken in the rotated basis (fp64)."""
    return _attend(_load().orc_attend_rotated, kc, vc, q, k_codes, k_norms, v_codes, v_norms,
                   lengths, scale, bh)


def attend_causal_queries(kc, vc, q, k_codes, k_norms, v_codes, v_norms, lengths, scale=None):
    """Multi-token decode (PR #232, review threads: the multi-query attention
    path and speculative decoding with draft tokens): S query tokens per
    sequence, causal among themselves. q: [B][S][Hq][d]; lengths[b] counts the
    cache rows including the S new ones. Query token i of sequence b attends
    the first lengths[b] - S + i + 1 rows (none if that is <= 0, a zero row).
    That is S single-query decodes with those lengths, which is how it is
    computed here. Returns [B][S][Hq][d] (fp64)."""
    q = np.asarray(q)
    B, S, Hq, d = q.shape
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros((B, S, Hq, d), dtype=np.float64)
    for i in range(S):
        li = np.maximum(lengths - S + i + 1, 0).astype(np.int32)
        out[:, i] = attend(kc, vc, q[:, i], k_codes, k_norms, v_codes, v_norms, li, scale)
    return out


def attend_mixed(kc, vc, q, k_codes, k_norms, v_codes, v_norms, lengths, raw_k, raw_v,
                 raw_lengths, scale=None):
    """Softmax attention over the union of the packed rows [0, lengths[b]) and
    raw rows raw_k/raw_v [B][Hkv][R][d] [0, raw_lengths[b]) taken as they are:
    an fp16 "sink" prefix kept uncompressed (turboquant-mlx guide,
    --kv-min-tokens) or pending rows not yet batch-compressed (PR #232,
    Design). Written out directly in fp64 over the dequantised packed rows.
    q: [B][Hq][d]; returns [B][Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_norms).shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    k_hat = dequant(kc, k_codes, k_norms)
    v_hat = dequant(vc, v_codes, v_norms)
    rk = np.asarray(raw_k, dtype=np.float64)
    rv = np.asarray(raw_v, dtype=np.float64)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = max(int(lengths[b]), 0)
        R = max(min(int(raw_lengths[b]), rk.shape[2]), 0)
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([k_hat[b, g, :L], rk[b, g, :R]])
            vals = np.concatenate([v_hat[b, g, :L], rv[b, g, :R]])
            if keys.shape[0] == 0:
                continue
            s = scale * (keys @ q[b, h])
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ vals
    return out


def attend_raw_k(vc, q, k, v_codes, v_norms, lengths, scale=None):
    """Raw fp16 keys with packed values (PR #232's raw-K turbo0v* schemes: keys
    kept at FP16, values compressed): softmax over q . k_t for the raw key rows
    k [B][Hkv][T][d], weighting the dequantised value rows. Written out
    directly in fp64. q: [B][Hq][d]; returns [B][Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    k = np.asarray(k, dtype=np.float64)
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = max(int(lengths[b]), 0)
        if L == 0:
            continue
        for g in range(Hkv):
            v_hat = dequant(vc, v_codes[b, g, :L], v_norms[b, g, :L])
            for h in range(g * G, (g + 1) * G):
                s = scale * (k[b, g, :L] @ q[b, h])
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v_hat
    return out


# ------------------------------------------------------------------ dense rotation

class DenseCodec:
    """A codec whose rotation is a dense matrix given by the caller (head dims
    that are not a power of two; PR #232, Known limitations: dense rotation
    otherwise). m is d x d with m / sqrt(d) orthogonal: z = m x / |x|.
    Lloyd-Max tables as for the Walsh-Hadamard codec."""

    def __init__(self, m: np.ndarray, bits: int):
        m = np.ascontiguousarray(m, dtype=np.float64)
        assert m.ndim == 2 and m.shape[0] == m.shape[1]
        self.dim, self.bits, self.m = m.shape[0], bits, m
        c, b = codebook.tables(bits)
        self.centroids = np.ascontiguousarray(c, dtype=np.float32)
        self.boundaries = np.ascontiguousarray(b, dtype=np.float32)

    @property
    def row_bytes(self) -> int:
        return self.dim * self.bits // 8


def tree_sum(v: np.ndarray) -> float:
    """The any-count pairwise tree the dense codec sums squares over."""
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1)
    return float(_load().orc_tree_sum(_p(v), v.size))


def encode_dense(codec: DenseCodec, x: np.ndarray, want_z: bool = False):
    """encode() with the dense rotation: returns (codes, norms, norms64, [z])."""
    x = np.asarray(x)
    lead = x.shape[:-1]
    d = x.shape[-1]
    assert d == codec.dim
    xd = np.ascontiguousarray(x.reshape(-1, d), dtype=np.float64)
    n = xd.shape[0]
    codes = np.zeros((n, codec.row_bytes), dtype=np.uint8)
    norms = np.zeros(n, dtype=np.float32)
    norms64 = np.zeros(n, dtype=np.float64)
    z = np.zeros((n, d), dtype=np.float64) if want_z else None
    _check(_load().orc_encode_dense(d, codec.bits, _p(codec.m), _p(codec.boundaries), _p(xd),
                                    n, d, _p(codes), _p(norms), _p(norms64),
                                    _p(z) if want_z else None), "encode_dense")
    out = (codes.reshape(*lead, codec.row_bytes), norms.reshape(lead), norms64.reshape(lead))
    if want_z:
        out = out + (z.reshape(*lead, d),)
    return out


def dequant_dense(codec: DenseCodec, codes: np.ndarray, norms: np.ndarray) -> np.ndarray:
    lead = np.asarray(norms).shape
    c = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, codec.row_bytes)
    nr = np.ascontiguousarray(norms, dtype=np.float32).reshape(-1)
    out = np.zeros((nr.size, codec.dim), dtype=np.float64)
    _check(_load().orc_dequant_dense(codec.dim, codec.bits, _p(codec.m), _p(codec.centroids),
                                     _p(c), _p(nr), nr.size, _p(out)), "dequant_dense")
    return out.reshape(*lead, codec.dim)


def attend_dense(kc: DenseCodec, vc: DenseCodec, q, k_codes, k_norms, v_codes, v_norms,
                 lengths, scale=None):
    """Softmax attention over the dequantised cache of dense-rotation codecs,
    written out directly in fp64 (the fused kernel's output equals the
    expand-then-attend path: turboquant-mlx KV-cache guide). q: [B][Hq][d];
    codes [B][Hkv][T][row]; norms [B][Hkv][T]. Returns [B][Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_norms).shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = max(int(lengths[b]), 0)
        if L == 0:
            continue
        for g in range(Hkv):
            k_hat = dequant_dense(kc, k_codes[b, g, :L], k_norms[b, g, :L])
            v_hat = dequant_dense(vc, v_codes[b, g, :L], v_norms[b, g, :L])
            for h in range(g * G, (g + 1) * G):
                s = scale * (k_hat @ q[b, h])
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v_hat
    return out


# ------------------------------------------------------------------ TurboQuant-Prod keys

def _wht_ascending(u: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the rows of u (fp64), stages in
    ascending order (pair distance 1, 2, 4, ...), each pair -> (a + b, a - b)."""
    u = np.array(u, dtype=np.float64, copy=True)
    n, d = u.shape
    h = 1
    while h < d:
        v = u.reshape(n, d // (2 * h), 2, h)
        a, b = v[:, :, 0, :].copy(), v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return u


def _pairwise_sum_sq(u: np.ndarray) -> np.ndarray:
    """Sum of squares of each row over the canonical pairwise tree (adjacent
    pairs level by level, in index order)."""
    s = np.asarray(u, dtype=np.float64) ** 2
    while s.shape[1] > 1:
        s = s[:, 0::2] + s[:, 1::2]
    return s[:, 0]


class ProdCodec:
    """TurboQuant-Prod key codec (VeloxQuant "How I built", Stage 3, and its
    TurboQuantProd method: rotation + Lloyd-Max with bits - 1 bits + a 1-bit QJL
    sketch of the residual). The sketch projection is the randomised Hadamard
    H diag(sigma_S), sigma_S the SplitMix64 signs of seed + 1."""

    def __init__(self, dim: int, bits: int, seed: int):
        assert 2 <= bits <= 9
        self.dim, self.bits, self.seed = dim, bits, seed
        self.mse = Codec(dim, bits - 1, seed)
        self.sketch_signs = signs((seed + 1) % (1 << 64), dim)

    @property
    def row_bytes(self) -> int:
        return self.mse.row_bytes

    @property
    def sketch_bytes(self) -> int:
        return self.dim // 8


def encode_prod(pc: ProdCodec, x: np.ndarray):
    """Keys -> (codes of the (bits-1)-bit MSE part, sketch bits, norm N, residual
    norm gamma). In the rotated basis z = H(sigma x) / N the residual is
    rho = z - c[idx]; gamma = |rho| (fp64 over the canonical pairwise tree,
    stored as fp32); sketch bit j is set when (H (sigma_S rho))_j < 0 (LSB-first,
    d bits). The residual in the original basis has norm N gamma / sqrt(d)."""
    x = np.asarray(x)
    lead = x.shape[:-1]
    d = pc.dim
    codes, norms, _, z = encode(pc.mse, x, want_z=True)
    z = z.reshape(-1, d)
    idx = np.stack([unpack(r, d, pc.mse.bits) for r in codes.reshape(-1, pc.row_bytes)]) \
        if z.shape[0] else np.zeros((0, d), dtype=np.int32)
    rho = z - pc.mse.centroids.astype(np.float64)[idx]
    gamma = np.sqrt(_pairwise_sum_sq(rho)) if z.shape[0] else np.zeros(0)
    y = _wht_ascending(rho * pc.sketch_signs[None, :].astype(np.float64))
    neg = (y < 0).astype(np.uint8)
    sketch = np.packbits(neg, axis=1, bitorder="little")
    return (codes, sketch.reshape(*lead, d // 8), norms,
            gamma.astype(np.float32).reshape(lead))


def qjl_estimate(rho_gamma: np.ndarray, sketch_row: np.ndarray, u: np.ndarray) -> float:
    """QJL estimate of <q~, rho> from the sketch bits of rho, its norm gamma and
    u = H (sigma_S q~): sqrt(pi / 2) gamma / d * sum_j sgn_j u_j, sgn_j = -1 for
    a set bit (Zandieh et al.'s asymmetric estimator, unbiased for Gaussian
    projection rows; rows of H diag(sigma_S) have the same second moments)."""
    d = u.shape[0]
    bits = np.unpackbits(np.asarray(sketch_row, dtype=np.uint8), bitorder="little")[:d]
    sgn = 1.0 - 2.0 * bits.astype(np.float64)
    return float(np.sqrt(np.pi / 2) * float(rho_gamma) / d * np.dot(sgn, u))


def attend_prod(pc: ProdCodec, vc: Codec, q, k_codes, k_sketch, k_norms, k_rnorms, v_codes,
                v_norms, lengths, scale=None):
    """Softmax attention whose scores use the Prod estimate of <q, k>:
    <q, k_hat_MSE> + <q, r> with <q, r> = (N / d) <q~, rho> estimated by QJL,
    q~ = H (sigma_K q). Values dequantised as usual. q: [B][Hq][d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = np.asarray(k_norms).shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    Hd = hadamard(d)
    sk = pc.mse.signs.astype(np.float64)
    ss = pc.sketch_signs.astype(np.float64)
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for b in range(B):
        L = max(int(lengths[b]), 0)
        if L == 0:
            continue
        for g in range(Hkv):
            idx = np.stack([unpack(r, d, pc.mse.bits) for r in k_codes[b, g, :L]])
            cen = pc.mse.centroids.astype(np.float64)[idx]
            v_hat = dequant(vc, v_codes[b, g, :L], v_norms[b, g, :L])
            nk = np.asarray(k_norms[b, g, :L], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                qt = Hd @ (sk * q[b, h])
                u = Hd @ (ss * qt)
                s = np.empty(L)
                for t in range(L):
                    est = qjl_estimate(k_rnorms[b, g, t], k_sketch[b, g, t], u)
                    s[t] = scale * nk[t] / d * (cen[t] @ qt + est)
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v_hat
    return out
