"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself (a published value, a closed form, brute force, an identity)."""
import math

import mpmath
import numpy as np
import pytest

import oracle
from oracle import codebook
from conftest import read_golden


# ------------------------------------------------------------------ sign generator

def test_splitmix64_published_vector():
    rows = read_golden("splitmix64_seed0.txt")
    got = oracle.splitmix64(0, len(rows))
    for seed, i, hexval in rows:
        assert int(seed) == 0
        assert int(got[int(i)]) == int(hexval, 16)


def test_signs_are_top_bit_of_generator_and_balanced():
    raw = oracle.splitmix64(42, 4096)
    s = oracle.signs(42, 4096)
    assert set(np.unique(s)) <= {-1, 1}
    np.testing.assert_array_equal(s == -1, (raw >> np.uint64(63)) == 1)
    # a fair Rademacher draw: |sum| within 4 sigma of 0
    assert abs(int(s.astype(np.int64).sum())) < 4 * math.sqrt(4096)
    # prefixes agree: the d-dim vector is the first d draws
    np.testing.assert_array_equal(oracle.signs(42, 128), s[:128])


# ------------------------------------------------------------------ Walsh-Hadamard

def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(d):
    h = oracle.hadamard(d)
    np.testing.assert_array_equal(h, _sylvester(d))
    np.testing.assert_array_equal(h @ h, d * np.eye(d))          # H H = d I
    np.testing.assert_array_equal(h, h.T)                         # symmetric, so self-inverse / d


def test_butterfly_op_count_matches_pages():
    # "896 ops at d=128" for the O(d log d) transform (VeloxQuant optimization journey)
    assert 128 * int(math.log2(128)) == 896


# ------------------------------------------------------------------ Lloyd-Max codebook

@pytest.mark.parametrize("row", read_golden("lloyd_max_gaussian.txt"))
def test_lloyd_max_published_values(row):
    bits, levels, mse, tol = int(row[0]), [float(v) for v in row[1].split(",")], float(row[2]), float(row[3])
    c = codebook.lloyd_max(bits)
    pos = c[len(c) // 2:]
    np.testing.assert_allclose(pos, levels, atol=tol, rtol=0)
    assert abs(codebook.distortion(c) - mse) < max(tol, 1e-9)


def test_one_bit_closed_form_exact():
    c, b = codebook.tables(1)
    r = math.sqrt(2.0 / math.pi)
    assert c[1] == np.float32(r) and c[0] == -np.float32(r)
    assert b[0] == 0.0


def _cell_moments_by_quadrature(a, b):
    f = lambda x: mpmath.npdf(x)
    g = lambda x: x * mpmath.npdf(x)
    lo = -mpmath.inf if a is None else a
    hi = mpmath.inf if b is None else b
    return mpmath.quad(f, [lo, hi]), mpmath.quad(g, [lo, hi])


@pytest.mark.parametrize("bits", range(1, 9))
def test_lloyd_max_conditions_by_quadrature(bits):
    """Both conditions, checked with numerical integration (not the closed-form
    cell moments the oracle uses): boundaries are midpoints, centroids are the
    conditional means, to 1e-12."""
    c = codebook.lloyd_max_mp(bits)
    n = len(c)
    step = max(1, n // 32)  # every cell for <= 5 bits, a spread of 32+ cells above
    with mpmath.workdps(30):
        b = [(c[i] + c[i + 1]) / 2 for i in range(n - 1)]
        cells = sorted(set(list(range(0, n, step)) + [n - 1, n // 2, n // 2 - 1]))
        for i in cells:
            mass, m1 = _cell_moments_by_quadrature(b[i - 1] if i else None, b[i] if i < n - 1 else None)
            assert abs(m1 / mass - c[i]) < 1e-12, (bits, i)


@pytest.mark.parametrize("bits", range(1, 9))
def test_codebook_symmetry_order_and_fp32_tables(bits):
    c, b = codebook.tables(bits)
    n = 1 << bits
    assert c.dtype == np.float32 and b.dtype == np.float32
    assert c.shape == (n,) and b.shape == (n - 1,)
    np.testing.assert_array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0) and np.all(np.diff(b) > 0)
    assert b[(n - 1) // 2] == 0.0
    # boundaries interleave the centroids
    assert np.all(c[:-1] < b) and np.all(b < c[1:])
    # fp32 rounding of the high-precision fixed point agrees with the fp64 solve
    c64 = codebook.lloyd_max(bits)
    np.testing.assert_array_equal(c, c64.astype(np.float32))


def test_high_bit_distortion_follows_panter_dite():
    # asymptotic MSE of an optimal quantizer of N(0,1): (sqrt(3) pi / 2) 4^-b
    prev = 0.0
    for bits in range(5, 9):
        ratio = codebook.distortion(codebook.lloyd_max(bits)) / (math.sqrt(3) * math.pi / 2 * 4.0 ** -bits)
        assert 0.9 < ratio < 1.0 and ratio > prev
        prev = ratio
    assert prev > 0.99


# ------------------------------------------------------------------ bucketize

@pytest.mark.parametrize("bits", range(1, 9))
def test_boundary_count_equals_argmin(bits):
    c, b = codebook.tables(bits)
    rng = np.random.default_rng(bits)
    z = np.concatenate([rng.standard_normal(20000) * 1.3, c.astype(np.float64),
                        np.array([-50.0, 50.0, 0.0])])
    got = oracle.bucketize(z, b)
    # brute force nearest centroid, first index on ties
    dist = np.abs(z[:, None] - c.astype(np.float64)[None, :])
    want = np.argmin(dist, axis=1)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("bits", range(1, 9))
def test_value_on_a_boundary_goes_to_lower_cell(bits):
    c, b = codebook.tables(bits)
    z = b.astype(np.float64)
    np.testing.assert_array_equal(oracle.bucketize(z, b), np.arange(b.size))
    up = np.nextafter(z, np.inf)
    np.testing.assert_array_equal(oracle.bucketize(up, b), np.arange(b.size) + 1)


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("row", read_golden("pack_examples.txt"))
def test_pack_matches_pages_example(row):
    bits = int(row[0])
    idx = [int(v) for v in row[1].split(",")]
    assert oracle.pack(idx, bits).tobytes().hex() == row[2]
    np.testing.assert_array_equal(oracle.unpack(np.frombuffer(bytes.fromhex(row[2]), np.uint8), len(idx), bits), idx)


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("d", [8, 64, 128, 256])
def test_pack_roundtrip_and_bit_positions(bits, d):
    rng = np.random.default_rng(d * 10 + bits)
    idx = rng.integers(0, 1 << bits, size=d)
    row = oracle.pack(idx, bits)
    assert row.size == d * bits // 8
    np.testing.assert_array_equal(oracle.unpack(row, d, bits), idx)
    # stream bit p = bits*i + k holds bit k of index i (numpy bit view, LSB first)
    stream = np.unpackbits(row, bitorder="little")
    for i in (0, 1, d // 2, d - 1):
        for k in range(bits):
            assert stream[bits * i + k] == (idx[i] >> k) & 1


@pytest.mark.parametrize("row", read_golden("scheme_ratios.txt"))
def test_storage_size_reproduces_published_ratios(row):
    name, kb, vb, ratio = row[0], int(row[1]), int(row[2]), float(row[3])
    d = 128
    x = np.random.default_rng(0).standard_normal((4, d)).astype(np.float16)

    def stored_bytes(bits):
        if bits == 16:
            return 2 * d
        codes, norms, _ = oracle.encode(oracle.Codec(d, bits, 42), x)
        return codes.shape[-1] + norms.itemsize

    r = (2 * d * 2) / (stored_bytes(kb) + stored_bytes(vb))
    if name == "k8v3":
        assert abs(r - ratio) < 0.1   # "2.7x" in prose; the format gives 2.78
    else:
        assert round(r, 1) == ratio, (name, r)


# ------------------------------------------------------------------ encode

@pytest.mark.parametrize("d,bits", [(8, 3), (64, 4), (128, 2), (128, 8), (256, 3), (64, 1)])
def test_encode_against_dense_rotation(d, bits):
    codec = oracle.Codec(d, bits, 42)
    rng = np.random.default_rng(d + bits)
    x = (rng.standard_normal((200, d)) * rng.uniform(0.01, 30, size=(200, 1))).astype(np.float16)
    codes, norms, norms64, z = oracle.encode(codec, x, want_z=True)
    xd = x.astype(np.float64)
    # R = H diag(sigma) / sqrt(d) is orthonormal; z = sqrt(d) R x / |x|
    r = _sylvester(d) * codec.signs[None, :].astype(np.float64) / math.sqrt(d)
    np.testing.assert_allclose(r @ r.T, np.eye(d), atol=1e-14)
    exact_norm = np.array([math.sqrt(math.fsum(v * v for v in row)) for row in xd])
    np.testing.assert_allclose(norms64, exact_norm, rtol=2e-16, atol=0)
    np.testing.assert_array_equal(norms, exact_norm.astype(np.float32))
    zt = math.sqrt(d) * (xd @ r.T) / exact_norm[:, None]
    np.testing.assert_allclose(z, zt, rtol=1e-14, atol=1e-14)
    idx = np.stack([oracle.unpack(cr, d, bits) for cr in codes])
    np.testing.assert_array_equal(idx, oracle.bucketize(z, codec.boundaries).reshape(idx.shape))


def test_norm_uses_canonical_pairwise_tree():
    # magnitudes chosen so summation order changes the fp64 result
    d = 8
    x = np.array([60000.0, 0.0001, 0.0001, 0.0001, 3.0, 0.0002, 0.0003, 1.0], dtype=np.float16)
    sq = x.astype(np.float64) ** 2
    level = list(sq)
    while len(level) > 1:
        level = [level[2 * i] + level[2 * i + 1] for i in range(len(level) // 2)]
    _, _, n64 = oracle.encode(oracle.Codec(d, 4, 1), x[None, :])
    assert n64[0] == math.sqrt(level[0])


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_zero_vector_and_scale_invariance(bits):
    d = 64
    codec = oracle.Codec(d, bits, 7)
    codes, norms, _ = oracle.encode(codec, np.zeros((1, d), np.float16))
    assert norms[0] == 0.0
    np.testing.assert_array_equal(oracle.unpack(codes[0], d, bits), np.full(d, (1 << (bits - 1)) - 1))
    x = np.random.default_rng(3).standard_normal((16, d)).astype(np.float16)
    c1, n1, _ = oracle.encode(codec, x)
    c2, n2, _ = oracle.encode(codec, (x.astype(np.float32) * 4).astype(np.float16))  # exact power-of-2 scale
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(n2, n1 * 4)


def test_basis_vector_rotates_to_plus_minus_one():
    d, bits = 128, 4
    codec = oracle.Codec(d, bits, 42)
    x = np.zeros((d, d), np.float16)
    np.fill_diagonal(x, 1.0)
    _, norms, _, z = oracle.encode(codec, x, want_z=True)
    np.testing.assert_array_equal(norms, np.ones(d, np.float32))
    np.testing.assert_array_equal(z, codec.signs[:, None] * _sylvester(d))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantisation_error_matches_distortion(bits):
    # rotated unit-scaled coordinates of isotropic input are ~N(0,1): the
    # mean squared error per coordinate is the codebook's distortion
    d = 128
    codec = oracle.Codec(d, bits, 42)
    x = np.random.default_rng(11).standard_normal((2000, d)).astype(np.float16)
    codes, _, _, z = oracle.encode(codec, x, want_z=True)
    idx = np.stack([oracle.unpack(c, d, bits) for c in codes])
    err = np.mean((z - codec.centroids[idx]) ** 2)
    dist = codebook.distortion(codebook.lloyd_max(bits))
    assert abs(err - dist) < 0.05 * dist


# ------------------------------------------------------------------ dequant + attention

def _brute_force_attention(q, k_hat, v_hat, lengths, group, scale):
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hq):
            L = lengths[b]
            if L == 0:
                continue
            kk = k_hat[b, h // group, :L]
            vv = v_hat[b, h // group, :L]
            s = scale * (kk @ q[b, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = p @ vv
    return out


def _encode_cache(codec, x):
    codes, norms, _ = oracle.encode(codec, x)
    return codes, norms


@pytest.mark.parametrize("d", [8, 16])
@pytest.mark.parametrize("kb,vb", [(1, 1), (2, 3), (3, 5), (4, 4), (8, 3), (6, 7), (5, 8)])
def test_attention_brute_force_tiny(d, kb, vb):
    rng = np.random.default_rng(d * 100 + kb * 10 + vb)
    B, Hq, Hkv, T = 1, 2, 1, 8
    lengths = np.array([T])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, kb, 5), oracle.Codec(d, vb, 6)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    # explicit dequantisation: x_hat = |x| R^T c[idx] / sqrt(d), R = H diag(sigma)/sqrt(d)
    def deq(codec, codes, norms):
        r = _sylvester(d) * codec.signs[None, :].astype(np.float64) / math.sqrt(d)
        idx = np.stack([oracle.unpack(cr, d, codec.bits) for cr in codes.reshape(-1, codec.row_bytes)])
        cen = codec.centroids.astype(np.float64)[idx]
        return (norms.reshape(-1, 1).astype(np.float64) * (cen @ r) / math.sqrt(d)).reshape(*norms.shape, d)
    k_hat, v_hat = deq(kc, kcodes, knorms), deq(vc, vcodes, vnorms)
    np.testing.assert_allclose(oracle.dequant(kc, kcodes, knorms), k_hat, rtol=1e-13, atol=1e-13)
    want = _brute_force_attention(q.astype(np.float64), k_hat, v_hat, lengths, Hq // Hkv, 1 / math.sqrt(d))
    got = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d,kb,vb,G", [(64, 4, 4, 2), (128, 4, 2, 3), (128, 8, 3, 4), (64, 3, 3, 8)])
def test_rotated_domain_equals_dequantise_then_attend(d, kb, vb, G):
    rng = np.random.default_rng(d + kb + vb + G)
    B, Hkv, T = 2, 2, 96
    Hq = Hkv * G
    lengths = np.array([96, 37])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, kb, 42), oracle.Codec(d, vb, 42)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    a = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    r = oracle.attend_rotated(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    np.testing.assert_allclose(r, a, rtol=1e-11, atol=1e-12)


def _cache(d=64, kb=4, vb=3, B=2, Hq=4, Hkv=2, T=40, seed=0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, kb, 42), oracle.Codec(d, vb, 42)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    return kc, vc, q, kcodes, knorms, vcodes, vnorms


def test_special_cases_length_one_zero_query_empty():
    kc, vc, q, kcodes, knorms, vcodes, vnorms = _cache()
    v_hat = oracle.dequant(vc, vcodes, vnorms)
    # length 1: the output is the single dequantised value row
    out = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, np.array([1, 1]))
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v_hat[b, h // 2, 0], rtol=1e-13, atol=1e-14)
    # zero query: uniform weights, the output is the mean of the value rows
    lengths = np.array([40, 13])
    out = oracle.attend(kc, vc, np.zeros_like(q), kcodes, knorms, vcodes, vnorms, lengths)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v_hat[b, h // 2, :lengths[b]].mean(0), rtol=1e-12, atol=1e-13)
    # empty sequence: a zero row
    out = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, np.array([0, 5]))
    assert np.all(out[0] == 0.0) and np.any(out[1] != 0.0)


def test_gqa_mapping_and_split_invariance():
    kc, vc, q, kcodes, knorms, vcodes, vnorms = _cache(Hq=6, Hkv=2)
    q[:, 1] = q[:, 0]       # heads 0,1,2 read KV head 0; heads 3,4,5 read KV head 1
    q[:, 4] = q[:, 3]
    lengths = np.array([40, 29])
    out = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    np.testing.assert_array_equal(out[:, 1], out[:, 0])
    np.testing.assert_array_equal(out[:, 4], out[:, 3])
    assert not np.allclose(out[:, 0], out[:, 3])
    # selected (b, h) pairs give the same rows as the full call
    bh = [(1, 5), (0, 2), (1, 0)]
    sel = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, bh=bh)
    for i, (b, h) in enumerate(bh):
        np.testing.assert_array_equal(sel[i], out[b, h])
    # log-sum-exp merge of two halves of the context equals the whole
    scale = 1 / math.sqrt(64)
    k_hat = oracle.dequant(kc, kcodes, knorms)
    v_hat = oracle.dequant(vc, vcodes, vnorms)
    b, h = 0, 2
    s = scale * k_hat[b, h // 3, :40] @ q[b, h].astype(np.float64)
    parts = []
    for lo, hi in [(0, 17), (17, 40)]:
        m = s[lo:hi].max()
        e = np.exp(s[lo:hi] - m)
        parts.append((m, e.sum(), e @ v_hat[b, h // 3, lo:hi]))
    M = max(p[0] for p in parts)
    L = sum(p[1] * math.exp(p[0] - M) for p in parts)
    A = sum(p[2] * math.exp(p[0] - M) for p in parts)
    np.testing.assert_allclose(A / L, out[b, h], rtol=1e-12, atol=1e-13)


def test_rows_beyond_length_are_ignored():
    kc, vc, q, kcodes, knorms, vcodes, vnorms = _cache()
    lengths = np.array([23, 40])
    a = oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    kcodes2, knorms2 = kcodes.copy(), knorms.copy()
    kcodes2[0, :, 23:] = 0xFF
    knorms2[0, :, 23:] = np.nan
    b = oracle.attend(kc, vc, q, kcodes2, knorms2, vcodes, vnorms, lengths)
    np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------ multi-token decode

def _causal_mask_attention(q, k_hat, v_hat, lengths, group, scale):
    """Brute force with an explicit (query token, row) mask: query token i of
    S sits at position lengths[b] - S + i and sees the rows at or before it."""
    B, S, Hq, d = q.shape
    T = k_hat.shape[2]
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for i in range(S):
            pos = lengths[b] - S + i
            visible = np.arange(T) <= pos
            for h in range(Hq):
                if not visible.any():
                    continue
                s = scale * (k_hat[b, h // group] @ q[b, i, h])
                s = np.where(visible, s, -np.inf)
                p = np.exp(s - s.max())
                out[b, i, h] = (p / p.sum()) @ v_hat[b, h // group]
    return out


@pytest.mark.parametrize("d,kb,vb,G,S", [(8, 3, 2, 2, 3), (16, 8, 3, 4, 4), (8, 4, 4, 1, 2)])
def test_causal_queries_against_masked_brute_force(d, kb, vb, G, S):
    rng = np.random.default_rng(d * 1000 + kb * 100 + vb * 10 + S)
    B, Hkv, T = 3, 2, 9
    Hq = G * Hkv
    lengths = np.array([T, S, 1])            # full, exactly the new rows, fewer rows than S
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, S, Hq, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, kb, 3), oracle.Codec(d, vb, 4)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    k_hat = oracle.dequant(kc, kcodes, knorms)
    v_hat = oracle.dequant(vc, vcodes, vnorms)
    want = _causal_mask_attention(q.astype(np.float64), k_hat, v_hat, lengths, G, 1 / math.sqrt(d))
    got = oracle.attend_causal_queries(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # sequence 2 has one row: only the last query token sees it
    assert np.all(got[2, :S - 1] == 0.0) and np.any(got[2, S - 1] != 0.0)


def test_one_query_token_is_the_single_decode():
    rng = np.random.default_rng(11)
    d, B, Hkv, G, T = 16, 2, 2, 2, 12
    lengths = np.array([12, 5])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, 1, G * Hkv, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, 4, 1), oracle.Codec(d, 3, 2)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    one = oracle.attend_causal_queries(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    ref = oracle.attend(kc, vc, q[:, 0], kcodes, knorms, vcodes, vnorms, lengths)
    assert np.array_equal(one[:, 0], ref)


# ------------------------------------------------------------------ packed + raw fp16 rows

@pytest.mark.parametrize("d,kb,vb,G", [(16, 4, 3, 2), (8, 8, 2, 1), (16, 3, 3, 4)])
def test_mixed_segments_reduce_to_known_attention(d, kb, vb, G):
    rng = np.random.default_rng(d * 31 + kb * 7 + vb + G)
    B, Hkv, T, R = 3, 2, 10, 4
    Hq = G * Hkv
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kc, vc = oracle.Codec(d, kb, 8), oracle.Codec(d, vb, 9)
    kcodes, knorms = _encode_cache(kc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    lengths = np.array([T, 7, 0])
    rk = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    rv = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    # no raw rows: the packed-cache attention
    none = oracle.attend_mixed(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv,
                               np.zeros(B, dtype=np.int32))
    np.testing.assert_allclose(none, oracle.attend(kc, vc, q, kcodes, knorms, vcodes, vnorms,
                                                   lengths), rtol=1e-12, atol=1e-13)
    # rows moved from the packed cache to the raw segment, as their decoded
    # values, leave the attention unchanged
    k_hat = oracle.dequant(kc, kcodes, knorms)
    v_hat = oracle.dequant(vc, vcodes, vnorms)
    moved = oracle.attend_mixed(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths - 3 * (lengths > 3),
                                k_hat[:, :, 4:7], v_hat[:, :, 4:7], np.array([0, 3, 0]))
    np.testing.assert_allclose(moved[1], none[1], rtol=1e-12, atol=1e-13)
    # raw rows only (sequence 2 has no packed row): plain attention over them
    raw_only = oracle.attend_mixed(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv,
                                   np.array([R, R, R]))
    want = _brute_force_attention(q.astype(np.float64), rk.astype(np.float64),
                                  rv.astype(np.float64), np.array([R] * B), G, 1 / math.sqrt(d))
    np.testing.assert_allclose(raw_only[2], want[2], rtol=1e-12, atol=1e-13)
    # neither: a zero row
    assert np.all(oracle.attend_mixed(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv,
                                      np.array([0, 0, 0]))[2] == 0.0)


# ------------------------------------------------------------------ raw fp16 keys

@pytest.mark.parametrize("d,vb,G", [(16, 4, 2), (8, 2, 1), (16, 3, 4)])
def test_raw_keys_against_brute_force_and_special_cases(d, vb, G):
    rng = np.random.default_rng(d * 17 + vb * 5 + G)
    B, Hkv, T = 2, 2, 9
    Hq = G * Hkv
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    vc = oracle.Codec(d, vb, 12)
    vcodes, vnorms = _encode_cache(vc, v)
    lengths = np.array([T, 4])
    # explicit dequantisation of V and a dense softmax with the fp16 keys
    r = _sylvester(d) * vc.signs[None, :].astype(np.float64) / math.sqrt(d)
    idx = np.stack([oracle.unpack(cr, d, vb) for cr in vcodes.reshape(-1, vc.row_bytes)])
    v_hat = (vnorms.reshape(-1, 1).astype(np.float64) *
             (vc.centroids.astype(np.float64)[idx] @ r) / math.sqrt(d)).reshape(B, Hkv, T, d)
    want = _brute_force_attention(q.astype(np.float64), k.astype(np.float64), v_hat, lengths, G,
                                  1 / math.sqrt(d))
    got = oracle.attend_raw_k(vc, q, k, vcodes, vnorms, lengths)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # one row: the output is that row's dequantised value
    one = oracle.attend_raw_k(vc, q, k, vcodes, vnorms, np.array([1, 1]))
    np.testing.assert_allclose(one[0, 0], v_hat[0, 0, 0], rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ TurboQuant-Prod keys

@pytest.mark.parametrize("d,bits", [(16, 4), (64, 3), (128, 2), (32, 9)])
def test_prod_residual_reconstructs_and_sketch_is_dense_product(d, bits):
    rng = np.random.default_rng(d + bits)
    x = (rng.standard_normal((40, d)) * rng.uniform(0.1, 5, (40, 1))).astype(np.float16)
    pc = oracle.ProdCodec(d, bits, 21)
    codes, sketch, norms, gam = oracle.encode_prod(pc, x)
    _, _, n64, z = oracle.encode(pc.mse, x, want_z=True)
    idx = np.stack([oracle.unpack(r, d, bits - 1) for r in codes])
    rho = z - pc.mse.centroids.astype(np.float64)[idx]
    # x = (N / d) sigma H (c[idx] + rho): the residual completes the MSE part
    H = _sylvester(d)
    rec = (n64[:, None] / d) * pc.mse.signs[None, :] * ((pc.mse.centroids.astype(np.float64)[idx] + rho) @ H)
    np.testing.assert_allclose(rec, x.astype(np.float64), rtol=1e-12, atol=1e-12)
    # gamma is |rho|, and N gamma / sqrt(d) the residual norm in the original basis
    np.testing.assert_allclose(gam, np.linalg.norm(rho, axis=1), rtol=1e-6)
    k_hat = oracle.dequant(pc.mse, codes, norms)
    np.testing.assert_allclose(norms * gam / math.sqrt(d),
                               np.linalg.norm(x.astype(np.float64) - k_hat, axis=1), rtol=1e-5)
    # sketch bits: signs of the dense product H diag(sigma_S) rho
    y = (rho * pc.sketch_signs[None, :]) @ H
    bits_dense = np.packbits((y < 0).astype(np.uint8), axis=1, bitorder="little")
    clear = np.abs(y) > 1e-9 * np.abs(y).max()
    got = np.unpackbits(sketch, axis=1, bitorder="little")[:, :d]
    want = np.unpackbits(bits_dense, axis=1, bitorder="little")[:, :d]
    assert np.array_equal(got[clear], want[clear])


@pytest.mark.parametrize("d,bits,seed", [(64, 3, 5), (128, 2, 6), (128, 4, 7), (256, 3, 8)])
def test_prod_sketch_signs_exact_outside_butterfly_error_bound(d, bits, seed):
    """Each sketch bit against the exact sign of y_j = sum_i H_ji sigma_S,i rho_i.
    Every term +-rho_i is an fp64 number, and math.fsum returns the correctly
    rounded sum of its terms, so its sign is the sign of the exact sum. The
    oracle's butterfly adds log2(d) times per output, each addition off by at
    most one rounding, so |y_hat - y| <= gamma_k sum_i |rho_i| with k = log2 d
    and gamma_k = k u / (1 - k u), u = 2^-53. Wherever |y| exceeds that bound the
    bit must be the exact sign; entries under it are counted and must be rare."""
    rng = np.random.default_rng(seed)
    n = 60
    x = (rng.standard_normal((n, d)) * rng.uniform(0.05, 20.0, (n, 1))).astype(np.float16)
    x[0] = 0.0                                    # zero vector: rho = -c[idx], no zero sums
    pc = oracle.ProdCodec(d, bits, 31 + seed)
    codes, sketch, norms, gam = oracle.encode_prod(pc, x)
    _, _, _, z = oracle.encode(pc.mse, x, want_z=True)
    idx = np.stack([oracle.unpack(r, d, bits - 1) for r in codes])
    rho = z - pc.mse.centroids.astype(np.float64)[idx]
    H = _sylvester(d)
    k = int(math.log2(d))
    u = 2.0 ** -53
    gamma_k = k * u / (1.0 - k * u)
    got = np.unpackbits(sketch, axis=1, bitorder="little")[:, :d]
    # the zero vector: rho = -c[2^(b-2) - 1] in every coordinate, so every partial
    # sum of the butterfly is an exact multiple of it and y_j = 0 exactly where
    # (H sigma_S)_j = 0; the bit is then (0 < 0) = 0
    y0 = np.array([math.fsum((H[j] * rho[0] * pc.sketch_signs).tolist()) for j in range(d)])
    assert np.array_equal(got[0], (y0 < 0).astype(np.uint8))
    under = 0
    for r in range(1, n):
        terms = rho[r] * pc.sketch_signs.astype(np.float64)   # exact: a sign flip
        bound = gamma_k * float(np.abs(terms).sum()) * (1.0 + 4.0 * d * u)  # + slack of the bound's own sum
        for j in range(d):
            y = math.fsum((H[j] * terms).tolist())               # H_ji = +-1: exact terms
            if abs(y) > bound:
                assert got[r, j] == (1 if y < 0 else 0), (r, j, y, bound)
            else:
                under += 1
    print(f"d={d} bits={bits}: {under} of {(n - 1) * d} entries within the butterfly error bound")
    assert under <= (n - 1) * d // 1000


def test_prod_sketch_sign_pin_catches_a_wrong_bit():
    """The exact-sign check above fails on a sketch computed from rho with one
    coordinate's sign flipped (a plausible indexing mistake), so it can see
    more than its own output."""
    d, bits = 64, 3
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, d)).astype(np.float16)
    pc = oracle.ProdCodec(d, bits, 9)
    _, _, _, z = oracle.encode(pc.mse, x, want_z=True)
    codes, sketch, _, _ = oracle.encode_prod(pc, x)
    idx = np.stack([oracle.unpack(r, d, bits - 1) for r in codes])
    rho = z - pc.mse.centroids.astype(np.float64)[idx]
    bad = rho.copy()
    bad[:, 5] = -bad[:, 5]
    H = _sylvester(d)
    terms = bad * pc.sketch_signs.astype(np.float64)
    exact = np.array([[math.fsum((H[j] * terms[r]).tolist()) for j in range(d)]
                      for r in range(4)])
    got = np.unpackbits(sketch, axis=1, bitorder="little")[:, :d]
    assert np.any(got != (exact < 0))


def test_qjl_estimate_is_unbiased_over_sketch_draws():
    """Average of the estimate over random sketch sign vectors approaches
    <q~, rho>: a wrong sign or a missing sqrt(pi/2) fails it."""
    rng = np.random.default_rng(7)
    d = 64
    rho = rng.standard_normal(d) * 0.3
    qt = rng.standard_normal(d) * 2.0 + 0.8 * rho / np.linalg.norm(rho) * 6
    H = _sylvester(d)
    ests = []
    for _ in range(4000):
        ss = rng.choice([-1.0, 1.0], size=d)
        y = H @ (ss * rho)
        sketch = np.packbits((y < 0).astype(np.uint8), bitorder="little")
        ests.append(oracle.qjl_estimate(np.linalg.norm(rho), sketch, H @ (ss * qt)))
    ests = np.asarray(ests)
    true = float(qt @ rho)
    assert abs(ests.mean() - true) < 4 * ests.std() / math.sqrt(len(ests)) + 0.02 * abs(true)


@pytest.mark.parametrize("d,bits,vb,G", [(16, 4, 3, 2), (8, 3, 2, 1)])
def test_prod_attention_brute_force_tiny(d, bits, vb, G):
    rng = np.random.default_rng(d * 7 + bits + vb)
    B, Hkv, T = 1, 2, 7
    Hq = G * Hkv
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    pc, vc = oracle.ProdCodec(d, bits, 3), oracle.Codec(d, vb, 4)
    kcodes, ksk, knorms, krn = oracle.encode_prod(pc, k)
    vcodes, vnorms = _encode_cache(vc, v)
    lengths = np.array([T])
    got = oracle.attend_prod(pc, vc, q, kcodes, ksk, knorms, krn, vcodes, vnorms, lengths)
    # explicit: rotated query, sketch projection, estimate, dense softmax
    H = _sylvester(d)
    v_hat = oracle.dequant(vc, vcodes, vnorms)
    want = np.zeros((B, Hq, d))
    for h in range(Hq):
        g = h // G
        qt = H @ (pc.mse.signs * q[0, h].astype(np.float64))
        u = H @ (pc.sketch_signs * qt)
        s = []
        for t in range(T):
            idx = oracle.unpack(kcodes[0, g, t], d, bits - 1)
            bitsj = np.unpackbits(ksk[0, g, t], bitorder="little")[:d]
            est = math.sqrt(math.pi / 2) * float(krn[0, g, t]) / d * ((1 - 2.0 * bitsj) @ u)
            s.append(float(knorms[0, g, t]) / d * (pc.mse.centroids[idx].astype(np.float64) @ qt + est) / math.sqrt(d))
        s = np.asarray(s)
        p = np.exp(s - s.max())
        want[0, h] = (p / p.sum()) @ v_hat[0, g]
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
