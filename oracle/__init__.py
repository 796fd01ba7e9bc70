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
_LIB = os.path.join(_HERE, "_tq_oracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
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
            for f in ("orc_signs", "orc_encode", "orc_dequant", "orc_attend", "orc_attend_rotated"):
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
