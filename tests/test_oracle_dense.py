"""Pins of the oracle's dense-rotation codec (head dims with no Walsh-Hadamard
transform; PR #232, Known limitations: dense rotation otherwise).

The dense codec is pinned to things other than itself: with the rotation
m = H diag(sigma) it must reproduce the Walsh-Hadamard codec bit for bit (that
codec is pinned by brute force and closed forms elsewhere); its pairwise norm
tree is exact on integer data; its rotated values, codes and dequantisation
agree with numpy's matrix products and a brute-force nearest-centroid search;
and attention over its cache taken in the rotated basis equals the plain
definition.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import rotation_matrix


def _data(rng, n, d):
    x = rng.standard_normal((n, d))
    x[:, rng.choice(d, 2, replace=False)] *= 6.0
    x[0] = 0.0                      # zero vector: all middle codes, norm 0
    return x.astype(np.float16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_hadamard_matrix_reproduces_wht_codec(d, bits):
    wc = oracle.Codec(d, bits, 42)
    m = oracle.hadamard(d) * wc.signs.astype(np.float64)[None, :]   # H diag(sigma)
    dc = oracle.DenseCodec(m, bits)
    x = _data(np.random.default_rng(d * 10 + bits), 200, d)
    c1, n1, _ = oracle.encode(wc, x)
    c2, n2, _ = oracle.encode_dense(dc, x)
    assert np.array_equal(c1, c2)
    assert np.array_equal(n1.view(np.uint32), n2.view(np.uint32))
    r1 = oracle.dequant(wc, c1, n1)
    r2 = oracle.dequant_dense(dc, c2, n2)
    np.testing.assert_allclose(r2, r1, rtol=0, atol=1e-12 * max(1.0, np.abs(r1).max()))


@pytest.mark.parametrize("d", [1, 7, 96, 160, 255])
def test_tree_sum_exact_on_integers(d):
    v = np.arange(d, dtype=np.float64) ** 2           # sum of squares is an exact integer
    assert oracle.tree_sum(v) == float(sum(i * i for i in range(d)))


def test_tree_sum_order():
    # five values: the first level adds (v0 + v1) and (v2 + v3), each rounding
    # away the 1, and carries v4; the sum of the pairs is 0, and v4 is added last
    v = np.array([1e16, 1.0, 1.0, -1e16, 3.0])
    s01 = 1e16 + 1.0
    s23 = 1.0 + -1e16
    assert oracle.tree_sum(v) == (s01 + s23) + 3.0


@pytest.mark.parametrize("d,bits", [(96, 2), (96, 3), (96, 4), (96, 8), (160, 3), (192, 4),
                                    (32, 2)])
def test_dense_encode_matches_numpy(d, bits):
    m = rotation_matrix(d, 7)
    np.testing.assert_allclose(m @ m.T, d * np.eye(d), atol=1e-10 * d)
    dc = oracle.DenseCodec(m, bits)
    x = _data(np.random.default_rng(d + bits), 300, d)
    codes, norms, norms64, z = oracle.encode_dense(dc, x, want_z=True)
    xd = x.astype(np.float64)
    nref = np.sqrt(np.array([math.fsum(r * r) for r in xd]))
    np.testing.assert_allclose(norms64, nref, rtol=4e-16, atol=0)
    zref = np.where(nref[:, None] > 0, (xd @ m.T) / np.where(nref > 0, nref, 1)[:, None], 0.0)
    np.testing.assert_allclose(z, zref, rtol=0, atol=1e-13)
    # brute force: nearest centroid with the first index winning a tie, except
    # where z lies within rounding of a boundary
    c = dc.centroids.astype(np.float64)
    near = np.argmin(np.abs(zref[..., None] - c[None, None, :]), axis=-1)
    idx = np.stack([oracle.unpack(r, d, bits) for r in codes])
    close = np.min(np.abs(zref[..., None] - dc.boundaries.astype(np.float64)), axis=-1) < 1e-12
    assert np.array_equal(idx[~close], near[~close])
    assert np.all(idx[0] == (1 << (bits - 1)) - 1) and norms[0] == 0.0
    # dequantisation: (N / d) m^T c[idx]
    ref = (norms.astype(np.float64)[:, None] / d) * (c[idx] @ m)
    np.testing.assert_allclose(oracle.dequant_dense(dc, codes, norms), ref, rtol=0, atol=1e-12)


def test_dense_distortion_near_lloyd_max():
    # sanity (not parity): on N(0, I) vectors the per-coordinate error of z is
    # near the Lloyd-Max distortion of a standard normal (3 bits: 0.03455)
    d, bits = 96, 3
    dc = oracle.DenseCodec(rotation_matrix(d, 3), bits)
    x = np.random.default_rng(5).standard_normal((2000, d)).astype(np.float16)
    codes, _, _, z = oracle.encode_dense(dc, x, want_z=True)
    idx = np.stack([oracle.unpack(r, d, bits) for r in codes])
    mse = np.mean((z - dc.centroids.astype(np.float64)[idx]) ** 2)
    assert abs(mse - 0.034548) < 0.003


@pytest.mark.parametrize("d,G", [(96, 3), (160, 2)])
def test_dense_attend_rotated_equals_definition(d, G):
    rng = np.random.default_rng(11)
    B, Hkv, T = 2, 2, 37
    kc = oracle.DenseCodec(rotation_matrix(d, 1), 4)
    vc = oracle.DenseCodec(rotation_matrix(d, 2), 3)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    lengths = np.array([T, 1], dtype=np.int32)
    kco, kn, _ = oracle.encode_dense(kc, k)
    vco, vn, _ = oracle.encode_dense(vc, v)
    out = oracle.attend_dense(kc, vc, q, kco, kn, vco, vn, lengths)
    scale = 1 / math.sqrt(d)
    for b in range(B):
        L = lengths[b]
        for h in range(G * Hkv):
            g = h // G
            qt = (kc.m @ q[b, h].astype(np.float64)) * scale / d       # rotated query
            ik = np.stack([oracle.unpack(r, d, 4) for r in kco[b, g, :L]])
            iv = np.stack([oracle.unpack(r, d, 3) for r in vco[b, g, :L]])
            s = kn[b, g, :L].astype(np.float64) * (kc.centroids.astype(np.float64)[ik] @ qt)
            p = np.exp(s - s.max())
            p /= p.sum()
            a = (p * vn[b, g, :L].astype(np.float64)) @ vc.centroids.astype(np.float64)[iv]
            ref = (vc.m.T @ a) / d
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)
    # length 1: the output is the one dequantised value row
    vh = oracle.dequant_dense(vc, vco[1, :, :1], vn[1, :, :1])
    for h in range(G * Hkv):
        np.testing.assert_allclose(out[1, h], vh[h // G, 0], rtol=0, atol=1e-12)


def test_hadamard_matrix_attend_matches_wht_oracle():
    d, G = 64, 2
    rng = np.random.default_rng(4)
    wk, wv = oracle.Codec(d, 4, 42), oracle.Codec(d, 4, 42)
    m = oracle.hadamard(d) * wk.signs.astype(np.float64)[None, :]
    dk, dv = oracle.DenseCodec(m, 4), oracle.DenseCodec(m, 4)
    k = rng.standard_normal((1, 2, 50, d)).astype(np.float16)
    v = rng.standard_normal((1, 2, 50, d)).astype(np.float16)
    q = rng.standard_normal((1, 2 * G, d)).astype(np.float16)
    L = np.array([50], dtype=np.int32)
    kco, kn, _ = oracle.encode(wk, k)
    vco, vn, _ = oracle.encode(wv, v)
    ref = oracle.attend(wk, wv, q, kco, kn, vco, vn, L)
    out = oracle.attend_dense(dk, dv, q, kco, kn, vco, vn, L)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
