"""Seeded synthetic workloads for the compressed-domain KV decode path.

This module only draws inputs. It holds none of the method's arithmetic (no
rotation, codebook, quantisation or attention), so the CPU oracle and the HIP
path can both consume what it produces without sharing any implementation.

The five workloads stand in for the model layers the source pages measure on
(Llama-3.2-3B-shaped and Llama-3-8B-shaped attention layers, a batched ragged
decode and a long-context layer). Only the shapes are taken from those models;
every value is drawn here from a fixed seed:

    rng = numpy.random.default_rng(seed)
    ragged batch only: lens = rng.integers(lo, hi, size=B, endpoint=True)
    K = draw(B, Hkv, T, d); V = draw(B, Hkv, T, d); q = rng.standard_normal((B, Hq, d))
    draw = standard normal, or Student-t(nu) scaled to unit variance
    outlier channels: chK = rng.choice(d, nK, replace=False); K[..., chK] *= sK
                      then chV likewise for V
    everything cast to float16 (round to nearest even)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    dim: int
    ctx: int                      # context per sequence (max for ragged)
    k_bits: int
    v_bits: int
    dist: str = "normal"          # "normal" | "student_t"
    t_nu: float = 5.0
    k_outliers: Tuple[int, float] = (0, 1.0)   # (channels, scale)
    v_outliers: Tuple[int, float] = (0, 1.0)
    ragged: Optional[Tuple[int, int]] = None   # inclusive [lo, hi] lengths
    pending: int = 0              # tokens encoded inside the timed step
    codec_seed: int = 42          # sign-vector seed shared by K and V codecs

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    # tiny: 4 q heads / 2 kv heads, d=64, 256 tokens, K4/V4, 2 outlier ch x8 in K and V
    "tiny_d64_k4v4": Workload("tiny_d64_k4v4", 0, 1, 4, 2, 64, 256, 4, 4,
                              k_outliers=(2, 8.0), v_outliers=(2, 8.0)),
    # Llama-3.2-3B-shaped layer: 24/8 heads, d=128, 4096 tokens, K4/V2, 4 K outlier ch x6
    "llama3b_4k_k4v2": Workload("llama3b_4k_k4v2", 1, 1, 24, 8, 128, 4096, 4, 2,
                                k_outliers=(4, 6.0)),
    # Llama-3-8B-shaped layer: 32/8 heads, d=128, 32768 tokens, K8/V3, Student-t(5),
    # the last 64 tokens are a pending batch encoded inside the timed step
    "llama8b_32k_k8v3": Workload("llama8b_32k_k8v3", 2, 1, 32, 8, 128, 32768, 8, 3,
                                 dist="student_t", pending=64),
    # batched decode: 16 sequences, ragged lengths in [1024, 8192], K3/V3, 3% outlier ch x5
    "batch16_ragged_k3v3": Workload("batch16_ragged_k3v3", 3, 16, 32, 8, 128, 8192, 3, 3,
                                    k_outliers=(round(0.03 * 128), 5.0),
                                    v_outliers=(round(0.03 * 128), 5.0),
                                    ragged=(1024, 8192)),
    # long context: 64/8 heads, d=64, 131072 tokens, K3/V3, 2 outlier ch x8 in K and V
    "long128k_d64_k3v3": Workload("long128k_d64_k3v3", 4, 1, 64, 8, 64, 131072, 3, 3,
                                  k_outliers=(2, 8.0), v_outliers=(2, 8.0)),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    lengths: np.ndarray   # int32 [B]
    k: np.ndarray         # float16 [B, Hkv, T, d]
    v: np.ndarray         # float16 [B, Hkv, T, d]
    q: np.ndarray         # float16 [B, Hq, d]
    k_channels: np.ndarray
    v_channels: np.ndarray


def _draw(rng, wl: Workload, shape):
    if wl.dist == "normal":
        return rng.standard_normal(shape)
    if wl.dist == "student_t":
        # unit variance: Var(t_nu) = nu / (nu - 2)
        return rng.standard_t(wl.t_nu, size=shape) * math.sqrt((wl.t_nu - 2.0) / wl.t_nu)
    raise ValueError(wl.dist)


def generate(wl: Workload) -> Inputs:
    """Draw the workload's inputs in the fixed order stated in the module doc."""
    rng = np.random.default_rng(wl.seed)
    if wl.ragged is not None:
        lo, hi = wl.ragged
        lengths = rng.integers(lo, hi, size=wl.batch, endpoint=True).astype(np.int32)
        T = int(lengths.max())
    else:
        lengths = np.full(wl.batch, wl.ctx, dtype=np.int32)
        T = wl.ctx
    shape = (wl.batch, wl.n_kv_heads, T, wl.dim)
    k = _draw(rng, wl, shape)
    v = _draw(rng, wl, shape)
    q = rng.standard_normal((wl.batch, wl.n_q_heads, wl.dim))
    nk, sk = wl.k_outliers
    ck = rng.choice(wl.dim, nk, replace=False) if nk else np.zeros(0, np.int64)
    if nk:
        k[..., ck] *= sk
    nv, sv = wl.v_outliers
    cv = rng.choice(wl.dim, nv, replace=False) if nv else np.zeros(0, np.int64)
    if nv:
        v[..., cv] *= sv
    return Inputs(wl, lengths, k.astype(np.float16), v.astype(np.float16),
                  q.astype(np.float16), ck, cv)


def small_case(seed: int, batch: int, n_q_heads: int, n_kv_heads: int, dim: int,
               ctx: int, lengths=None, scale_k: float = 1.0, scale_v: float = 1.0):
    """A generic seeded case for parity sweeps: N(0,1) fp16 K, V and q."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = np.full(batch, ctx, dtype=np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    k = (rng.standard_normal((batch, n_kv_heads, ctx, dim)) * scale_k).astype(np.float16)
    v = (rng.standard_normal((batch, n_kv_heads, ctx, dim)) * scale_v).astype(np.float16)
    q = rng.standard_normal((batch, n_q_heads, dim)).astype(np.float16)
    return lengths, k, v, q


def rotation_matrix(dim: int, seed: int) -> np.ndarray:
    """A Haar-random rotation for head dims with no Walsh-Hadamard transform,
    scaled by sqrt(dim): the Q factor of a standard Gaussian matrix with the
    signs of R's diagonal moved into it (Mezzadri 2007), drawn from
    numpy.random.default_rng(seed). It is a random input of the method, drawn
    here once and handed to both sides as the same fp64 matrix."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((dim, dim))
    qm, r = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(r))
    return np.ascontiguousarray(qm * math.sqrt(dim), dtype=np.float64)


def algorithmic_bytes(lengths, n_kv_heads: int, dim: int, k_bits: int, v_bits: int) -> int:
    """Bytes the decode-attend must read: packed K and V codes plus fp32 norms."""
    per_tok = (dim * k_bits // 8 + 4) + (dim * v_bits // 8 + 4)
    return int(np.asarray(lengths, dtype=np.int64).sum()) * n_kv_heads * per_tok
