"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed codes byte-identical and norms bit-identical (the contract is
exact, stronger than the required 1e-5 relative); decode-attend outputs within
2e-3 max-abs of the oracle's fp64 result. Oracle inputs never come from the
HIP path: the oracle encodes its own copy of every cache it attends over.
"""
import concurrent.futures as cf
import functools
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import compressed_domain_decode_amd as tq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL = 2e-3


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def codecs(dim, bits, seed=42):
    return tq.tq_codec_init(dim, bits, seed), oracle.Codec(dim, bits, seed)


def gpu_encode_rows(codec, x_np):
    """x_np (N, H, d) fp16 -> (codes (N, H, row), norms (N, H)) via one tq_encode."""
    N, H, d = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    codes = torch.full((N, H, codec.row_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    norms = torch.full((N, H), -1.0, dtype=torch.float32, device=DEV)
    tq.tq_encode(codec, x, codes, norms)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), norms.cpu().numpy()


def gpu_encode_cache(codec, x_dev):
    """x_dev (B, Hkv, T, d) fp16 on device -> device codes (B, Hkv, T, row), norms (B, Hkv, T).
    One call: (B*Hkv) heads of T tokens, written straight into the cache layout."""
    B, H, T, d = x_dev.shape
    codes = torch.empty((B, H, T, codec.row_bytes), dtype=torch.uint8, device=DEV)
    norms = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    xv = x_dev.view(B * H, T, d).permute(1, 0, 2)
    cv = codes.view(B * H, T, codec.row_bytes).permute(1, 0, 2)
    nv = norms.view(B * H, T).permute(1, 0)
    tq.tq_encode(codec, xv, cv, nv)
    return codes, norms


def gpu_attend(kc, vc, q_np, kcodes, knorms, vcodes, vnorms, lengths_np, scale=None, max_len=None):
    B, Hq, d = q_np.shape
    Hkv, T = knorms.shape[1], knorms.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if max_len is None:
        max_len = max(1, int(np.max(lengths_np)))
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to(DEV)
    lengths = torch.from_numpy(np.asarray(lengths_np, dtype=np.int32)).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len), dtype=torch.uint8, device=DEV)
    tq.tq_decode_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, max_len, scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def oracle_threads():
    """Threads for oracle work over independent units (the C oracle runs with
    the GIL released): the cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def map_units(fn, units):
    """fn over every unit on oracle_threads() threads; the first failure raises."""
    with cf.ThreadPoolExecutor(oracle_threads()) as ex:
        return list(ex.map(fn, units))


# ------------------------------------------------------------------ encode

def _encode_inputs(d, seed, n=384):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 2, d)) * rng.uniform(1e-3, 50, size=(n, 1, 1))
    x[0] = 0.0                                   # zero vector
    x[1, 0] = 6e-8                               # fp16 subnormals only
    x[2, 0, :] = 1.0                             # all equal
    x[3, 0] = rng.choice([-65504.0, 65504.0], size=d)  # largest magnitude
    x[4, 0] = 0.0
    x[4, 0, d // 3] = 3.0                        # one-hot
    return x.astype(np.float16)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", range(1, 9))
def test_encode_matches_oracle(d, bits):
    announce(f"encode d={d} bits={bits}")
    g, o = codecs(d, bits)
    x = _encode_inputs(d, d * 10 + bits)
    codes, norms = gpu_encode_rows(g, x)
    oc, on, _ = oracle.encode(o, x)
    assert codes.tobytes() == oc.tobytes()
    assert norms.tobytes() == on.tobytes()


def test_encode_strided_views_and_append():
    announce("encode strided views / append")
    d, bits = 128, 3
    g, o = codecs(d, bits)
    rng = np.random.default_rng(5)
    B, H, T = 2, 3, 200
    x = rng.standard_normal((B, H, T, d)).astype(np.float16)
    codes, norms = gpu_encode_cache(g, to_dev(x))
    torch.cuda.synchronize()
    oc, on, _ = oracle.encode(o, x)
    assert codes.cpu().numpy().tobytes() == oc.tobytes()
    assert norms.cpu().numpy().tobytes() == on.tobytes()
    # append: re-encode tokens 150..199 of sequence 1 into a cleared region
    codes[1, :, 150:] = 0
    norms[1, :, 150:] = 0
    xv = to_dev(x[1]).permute(1, 0, 2)[150:]
    tq.tq_encode(g, xv, codes[1].permute(1, 0, 2)[150:], norms[1].permute(1, 0)[150:])
    torch.cuda.synchronize()
    assert codes.cpu().numpy().tobytes() == oc.tobytes()
    assert norms.cpu().numpy().tobytes() == on.tobytes()


def _bulk_layout_vectors(d):
    """Vectors per launch from which the encoder uses its bulk layout (d/8 lanes
    per vector): 1024 wavefronts of 512/d vectors. Smaller launches use one
    64-lane wavefront per vector."""
    return 1024 * (512 // d)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", range(1, 9))
def test_encode_bulk_layout_matches_oracle(d, bits):
    announce(f"encode bulk layout d={d} bits={bits}")
    g, o = codecs(d, bits)
    n = _bulk_layout_vectors(d) // 2 + 19          # 2 heads: just past the switch, ragged
    x = _encode_inputs(d, d * 100 + bits, n=n)
    codes, norms = gpu_encode_rows(g, x)
    oc, on, _ = oracle.encode(o, x)
    assert codes.tobytes() == oc.tobytes()
    assert norms.tobytes() == on.tobytes()


@pytest.mark.parametrize("d,kb,vb", [(128, 8, 3), (64, 3, 3), (256, 4, 6), (128, 1, 5), (64, 7, 2)])
@pytest.mark.parametrize("T", [72, 1500])
def test_encode_kv_matches_oracle(d, kb, vb, T):
    """One launch for K and V (different bits and seeds) into [B][H][T][row]
    cache views; T=72 runs the 64-lane layout, T=1500 the bulk layout. Then a
    64-token append into cleared rows."""
    announce(f"encode kv d={d} kb={kb} vb={vb} T={T}")
    gk, ok = codecs(d, kb, 42)
    gv, ov = codecs(d, vb, 7)
    B, H, P = 2, 4, 64
    rng = np.random.default_rng(d + kb * 10 + vb + T)
    k = (rng.standard_normal((B, H, T, d)) * rng.uniform(0.01, 20, (B, H, T, 1))).astype(np.float16)
    v = (rng.standard_normal((B, H, T, d)) * rng.uniform(0.01, 20, (B, H, T, 1))).astype(np.float16)
    k[0, 1, 3] = 0.0
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    kd, vd = to_dev(k), to_dev(v)
    kc = torch.full((B, H, T, gk.row_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    vc = torch.full((B, H, T, gv.row_bytes), 0x5A, dtype=torch.uint8, device=DEV)
    kn = torch.full((B, H, T), -1.0, dtype=torch.float32, device=DEV)
    vn = torch.full((B, H, T), -1.0, dtype=torch.float32, device=DEV)

    def views(t0, t1):
        tm = lambda a, row: a.view(B * H, T, *row).permute(1, 0, *range(2, 2 + len(row)))[t0:t1]
        return (tm(kd, (d,)), tm(kc, (gk.row_bytes,)), tm(kn, ()),
                tm(vd, (d,)), tm(vc, (gv.row_bytes,)), tm(vn, ()))

    xk, ck, nk, xv, cv, nv = views(0, T)
    tq.tq_encode_kv(gk, xk, ck, nk, gv, xv, cv, nv)
    torch.cuda.synchronize()
    for got, want in ((kc, okc), (kn, okn), (vc, ovc), (vn, ovn)):
        assert got.cpu().numpy().tobytes() == want.tobytes()
    kc[:, :, T - P:] = 0
    vc[:, :, T - P:] = 0
    kn[:, :, T - P:] = 0
    vn[:, :, T - P:] = 0
    xk, ck, nk, xv, cv, nv = views(T - P, T)
    tq.tq_encode_kv(gk, xk, ck, nk, gv, xv, cv, nv)
    torch.cuda.synchronize()
    for got, want in ((kc, okc), (kn, okn), (vc, ovc), (vn, ovn)):
        assert got.cpu().numpy().tobytes() == want.tobytes()


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_encode_workload_full_size_sampled(name):
    wl = workloads.WORKLOADS[name]
    announce(f"encode full cache {name}")
    inp = workloads.generate(wl)
    rng = np.random.default_rng(99)
    for which, bits, x in (("K", wl.k_bits, inp.k), ("V", wl.v_bits, inp.v)):
        g, o = codecs(wl.dim, bits, wl.codec_seed)
        codes, norms = gpu_encode_cache(g, to_dev(x))
        torch.cuda.synchronize()
        B, H, T, _ = x.shape
        pick = (rng.integers(0, B, 4096), rng.integers(0, H, 4096), rng.integers(0, T, 4096))
        c_np = codes.cpu().numpy()[pick]
        n_np = norms.cpu().numpy()[pick]
        oc, on, _ = oracle.encode(o, x[pick])
        assert c_np.tobytes() == oc.tobytes(), which
        assert n_np.tobytes() == on.tobytes(), which


# ------------------------------------------------------------------ attend

def _oracle_cache(o, x):
    c, n, _ = oracle.encode(o, x)
    return c, n


def _attend_case(d, kb, vb, G, lengths, Hkv=2, seed=0, T=None, kscale=1.0, vscale=1.0):
    lengths = np.asarray(lengths, dtype=np.int32)
    B = lengths.size
    T = T or max(1, int(lengths.max()))
    lens, k, v, q = workloads.small_case(seed, B, Hkv * G, Hkv, d, T, lengths, kscale, vscale)
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    got = gpu_attend(gk, gv, q, kcodes, knorms, vcodes, vnorms, lens)
    okc, okn = _oracle_cache(ok, k)
    ovc, ovn = _oracle_cache(ov, v)
    # the GPU cache the kernel read is the oracle's cache byte for byte
    assert kcodes.cpu().numpy().tobytes() == okc.tobytes()
    assert vcodes.cpu().numpy().tobytes() == ovc.tobytes()
    want = oracle.attend(ok, ov, q, okc, okn, ovc, ovn, lens)
    return got, want


SUPPORTED_SMALL = [
    (64, 4, 4, 2), (64, 3, 3, 8), (64, 4, 4, 1), (64, 3, 3, 4), (64, 8, 3, 4), (64, 2, 2, 2),
    (64, 1, 1, 2), (64, 5, 7, 2), (64, 6, 6, 16), (64, 4, 4, 5), (64, 8, 3, 7),
    (128, 4, 2, 3), (128, 8, 3, 4), (128, 3, 3, 4), (128, 4, 4, 4), (128, 4, 3, 4), (128, 2, 2, 4),
    (128, 8, 4, 4), (128, 4, 4, 8), (128, 8, 3, 8), (128, 4, 2, 1), (128, 3, 3, 2), (128, 8, 3, 6),
    (128, 1, 1, 4), (128, 7, 5, 6), (128, 3, 3, 5), (128, 4, 2, 8),
    (256, 4, 4, 4), (256, 8, 3, 4), (256, 3, 3, 2), (256, 8, 4, 1), (256, 2, 2, 8),
    # PR #232's turbo4v2 / turbo4v3 at head dims 64 and 256
    (64, 4, 2, 3), (64, 4, 3, 4), (256, 4, 2, 4), (256, 4, 3, 2),
]


@pytest.mark.parametrize("d,kb,vb,G", SUPPORTED_SMALL)
def test_attend_matches_oracle_small(d, kb, vb, G):
    announce(f"attend d={d} K{kb} V{vb} G={G}")
    got, want = _attend_case(d, kb, vb, G, lengths=[700, 37, 257], seed=d + kb * 10 + vb + G)
    err = np.abs(got - want).max()
    print(f"  max abs err {err:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err <= ATOL


@pytest.mark.parametrize("d", [64, 128, 256])
def test_attend_every_bit_width_pair(d):
    """Every (K bits, V bits) pair the codecs accept is attended: pairs with a
    matrix-core instance run it, the others the rotation-matrix kernels with
    m = H diag(sigma) built from the codecs' signs. Ragged lengths with a
    single-row sequence, three query heads per KV head."""
    worst = 0.0
    for kb in range(1, 9):
        for vb in range(1, 9):
            announce(f"attend every pair d={d} K{kb} V{vb}")
            got, want = _attend_case(d, kb, vb, 3, lengths=[150, 1], seed=d + 8 * kb + vb)
            assert np.isfinite(got).all(), (kb, vb)
            err = float(np.abs(got - want).max())
            assert err <= ATOL, (kb, vb, err)
            worst = max(worst, err)
    print(f"  d={d}: worst max abs err {worst:.3e} over 64 pairs", flush=True)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("kb", [2, 3, 4, 8])
@pytest.mark.parametrize("vb", [2, 3, 4])
def test_attend_one_head_per_kv_head(d, kb, vb):
    """One query head per KV head at head dims 64, 128 and 256 runs the
    register-held kernel with m = H diag(sigma) formed from the codecs' signs
    (two lanes per token, four at 256; per-lane softmax state) instead of the
    matrix-core kernel: every (K, V) bit pair it has, with several splits, a
    tail inside a wavefront step, a lone token and an empty sequence."""
    lengths = [3000, 65, 1, 0]
    announce(f"attend one head per KV head d={d} K{kb} V{vb} lengths={lengths}")
    got, want = _attend_case(d, kb, vb, 1, lengths=lengths, seed=900 + d + 10 * kb + vb)
    assert np.isfinite(got).all()
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err
    assert np.all(got[3] == 0.0)


@pytest.mark.parametrize("d,kb,vb,G,lengths", [
    (256, 8, 8, 16, [3000, 1234]),   # 16 query heads per KV head, several splits
    (128, 8, 8, 2, [2500, 64]),      # 8-bit V
    (64, 8, 8, 1, [4100, 0]),        # an empty sequence: zero rows
    (128, 6, 5, 7, [777, 1, 300]),
])
def test_attend_fallback_pairs(d, kb, vb, G, lengths):
    announce(f"attend fallback d={d} K{kb} V{vb} G={G} lengths={lengths}")
    got, want = _attend_case(d, kb, vb, G, lengths=lengths, seed=5 * d + kb + vb + G)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() <= ATOL
    for b, L in enumerate(lengths):
        if L == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("d,kb,vb,G", [(128, 8, 3, 4), (64, 3, 3, 8), (128, 4, 2, 3)])
def test_attend_ragged_edge_lengths(d, kb, vb, G):
    lengths = [1, 2, 63, 64, 65, 255, 256, 257, 511, 513, 1024, 1025, 3000]
    announce(f"attend ragged lengths d={d} K{kb} V{vb} G={G}")
    got, want = _attend_case(d, kb, vb, G, lengths=lengths, seed=7)
    assert np.abs(got - want).max() <= ATOL


def test_attend_many_splits_per_head():
    """One KV head and a long context: the planner cuts 64-token-tile ranges
    to fill the CUs, so a head has far more splits than the combine folds in
    one pass (32), with a short last split."""
    announce("attend many splits per head")
    d, kb, vb, G, L = 128, 8, 3, 4, 20000
    assert tq.tq_attend_num_splits(1, G, 1, d, L) > 64
    got, want = _attend_case(d, kb, vb, G, lengths=[L], Hkv=1, seed=23)
    assert np.abs(got - want).max() <= ATOL
    # a batch of two with ragged lengths: the shorter sequence leaves splits empty
    got, want = _attend_case(d, kb, vb, G, lengths=[L, 7001], Hkv=1, seed=24)
    assert np.abs(got - want).max() <= ATOL


def test_attend_zero_length_and_single_token():
    announce("attend zero length / single token")
    d, kb, vb, G = 128, 8, 3, 4
    got, want = _attend_case(d, kb, vb, G, lengths=[0, 1, 5, 0], T=300, seed=3)
    assert np.all(got[0] == 0.0) and np.all(got[3] == 0.0)
    assert np.abs(got - want).max() <= ATOL
    # one token: the output is that token's dequantised V row
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    lens, k, v, q = workloads.small_case(3, 4, 8, 2, d, 300, [0, 1, 5, 0])
    ovc, ovn = _oracle_cache(ov, v)
    v_hat = oracle.dequant(ov, ovc, ovn)
    for h in range(8):
        np.testing.assert_allclose(got[1, h], v_hat[1, h // G, 0], atol=1e-5)


def test_attend_rows_beyond_length_never_read():
    announce("attend poisoned rows beyond length")
    d, kb, vb, G = 128, 8, 3, 4
    gk, _ = codecs(d, kb)
    gv, _ = codecs(d, vb)
    lens, k, v, q = workloads.small_case(11, 3, 8, 2, d, 1500, [1500, 700, 65])
    kc, kn = gpu_encode_cache(gk, to_dev(k))
    vc, vn = gpu_encode_cache(gv, to_dev(v))
    clean = gpu_attend(gk, gv, q, kc, kn, vc, vn, lens)
    for b, L in enumerate(lens):
        kc[b, :, L:] = 0xFF
        vc[b, :, L:] = 0xFF
        kn[b, :, L:] = float("nan")
        vn[b, :, L:] = float("nan")
    dirty = gpu_attend(gk, gv, q, kc, kn, vc, vn, lens, max_len=1500)
    assert clean.tobytes() == dirty.tobytes()


def test_attend_deterministic():
    announce("attend determinism")
    d, kb, vb, G = 64, 3, 3, 8
    gk, _ = codecs(d, kb)
    gv, _ = codecs(d, vb)
    lens, k, v, q = workloads.small_case(4, 2, 16, 2, d, 5000, [5000, 4097])
    kc, kn = gpu_encode_cache(gk, to_dev(k))
    vc, vn = gpu_encode_cache(gv, to_dev(v))
    a = gpu_attend(gk, gv, q, kc, kn, vc, vn, lens)
    b = gpu_attend(gk, gv, q, kc, kn, vc, vn, lens)
    assert a.tobytes() == b.tobytes()


def test_attend_distinct_heads_and_batches():
    """Every (b, h) row differs and matches its own oracle row: a swapped
    batch / head stride cannot hide behind identical data."""
    announce("attend stride order")
    d, kb, vb, G = 128, 4, 2, 3
    got, want = _attend_case(d, kb, vb, G, lengths=[300, 290, 280], Hkv=3, seed=21)
    flat = got.reshape(-1, d)
    assert len({r.tobytes() for r in flat}) == flat.shape[0]
    assert np.abs(got - want).max() <= ATOL


def test_attend_large_scale_inputs():
    announce("attend peaked softmax")
    # scaled keys make the softmax concentrate on few tokens
    got, want = _attend_case(128, 8, 3, 4, lengths=[2000, 999], seed=17, kscale=4.0, vscale=3.0)
    assert np.abs(got - want).max() <= ATOL


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_attend_workload_full_size(name):
    """Full-size cache and launch configuration of each workload; every
    (sequence, KV head) unit against the oracle, which encodes each unit's
    cache itself (those codes checked byte for byte against the GPU cache)."""
    wl = workloads.WORKLOADS[name]
    announce(f"attend full size {name}")
    inp = workloads.generate(wl)
    gk, ok = codecs(wl.dim, wl.k_bits, wl.codec_seed)
    gv, ov = codecs(wl.dim, wl.v_bits, wl.codec_seed)
    kc, kn = gpu_encode_cache(gk, to_dev(inp.k))
    vc, vn = gpu_encode_cache(gv, to_dev(inp.v))
    got = gpu_attend(gk, gv, inp.q, kc, kn, vc, vn, inp.lengths)
    kc_h, vc_h = kc.cpu().numpy(), vc.cpu().numpy()
    del kc, kn, vc, vn
    G = wl.group

    def unit(bg):
        b, g = bg
        L = int(inp.lengths[b])
        okc, okn, _ = oracle.encode(ok, inp.k[b:b + 1, g:g + 1, :L])
        ovc, ovn, _ = oracle.encode(ov, inp.v[b:b + 1, g:g + 1, :L])
        assert kc_h[b, g, :L].tobytes() == okc.tobytes(), bg
        assert vc_h[b, g, :L].tobytes() == ovc.tobytes(), bg
        want = oracle.attend(ok, ov, inp.q[b:b + 1, g * G:(g + 1) * G], okc, okn, ovc, ovn,
                             np.array([L], np.int32))
        return float(np.abs(got[b, g * G:(g + 1) * G] - want[0]).max())

    units = [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)]
    errs = map_units(unit, units)
    worst = max(errs)
    print(f"  {name}: worst max-abs err {worst:.3e} over all {len(units)} units "
          f"({wl.batch * wl.n_q_heads} rows)", flush=True)
    assert np.isfinite(got).all()
    assert worst <= ATOL


# ------------------------------------------------------------------ multi-token decode

def gpu_attend_multi(kc, vc, q_np, kcodes, knorms, vcodes, vnorms, lengths_np, max_len=None):
    B, S, Hq, d = q_np.shape
    Hkv = knorms.shape[1]
    if max_len is None:
        max_len = max(1, int(np.max(lengths_np)))
    q = to_dev(q_np)
    lengths = torch.from_numpy(np.asarray(lengths_np, dtype=np.int32)).to(DEV)
    out = torch.full((B, S, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_multi_workspace_bytes(B, S, Hq, Hkv, d, max_len),
                     dtype=torch.uint8, device=DEV)
    tq.tq_decode_attend_multi(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, max_len,
                              1.0 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,kb,vb,G,S", [(128, 8, 3, 4, 2), (128, 8, 3, 4, 4), (128, 3, 3, 4, 3),
                                         (64, 3, 3, 8, 2), (64, 4, 4, 2, 4), (128, 4, 2, 3, 2),
                                         (64, 6, 6, 4, 4)])
def test_attend_multi_matches_oracle(d, kb, vb, G, S):
    """S causal query tokens per sequence: ragged lengths over several tiles and
    splits, a sequence with exactly S rows and one with fewer rows than S (its
    first query tokens see nothing: zero rows)."""
    announce(f"attend multi d={d} kb={kb} vb={vb} G={G} S={S}")
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(d + 7 * kb + 13 * vb + 17 * G + S)
    B, Hkv, T = 4, 2, 2500
    Hq = G * Hkv
    lengths = np.array([T, 1337, S, max(1, S - 2)])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, S, Hq, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    got = gpu_attend_multi(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths)
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    want = oracle.attend_causal_queries(ok, ov, q, okc, okn, ovc, ovn, lengths)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= ATOL
    invisible = np.maximum(lengths[3] - S + np.arange(S) + 1, 0) == 0
    assert np.all(got[3][invisible] == 0.0)


def test_attend_multi_one_token_equals_single_decode():
    announce("attend multi S=1 vs single decode")
    d, kb, vb, G = 128, 8, 3, 4
    gk, _ = codecs(d, kb)
    gv, _ = codecs(d, vb)
    rng = np.random.default_rng(99)
    B, Hkv, T = 2, 2, 3000
    lengths = np.array([3000, 2049])
    k = to_dev(rng.standard_normal((B, Hkv, T, d)).astype(np.float16))
    v = to_dev(rng.standard_normal((B, Hkv, T, d)).astype(np.float16))
    q = rng.standard_normal((B, 1, G * Hkv, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(gk, k)
    vcodes, vnorms = gpu_encode_cache(gv, v)
    multi = gpu_attend_multi(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths)
    single = gpu_attend(gk, gv, q[:, 0], kcodes, knorms, vcodes, vnorms, lengths)
    assert multi[:, 0].tobytes() == single.tobytes()


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_attend_multi_workload_full_size(name):
    """The most query tokens (4, else 2) a multi-token kernel covers for each
    workload at full size; every (sequence, KV head) unit against the oracle."""
    wl = workloads.WORKLOADS[name]
    G = wl.n_q_heads // wl.n_kv_heads
    gk, ok = codecs(wl.dim, wl.k_bits, wl.codec_seed)
    gv, ov = codecs(wl.dim, wl.v_bits, wl.codec_seed)
    inp = workloads.generate(wl)
    rng = np.random.default_rng(5)
    kc, kn = gpu_encode_cache(gk, to_dev(inp.k))
    vc, vn = gpu_encode_cache(gv, to_dev(inp.v))
    got = None
    for S in (4, 2):
        if G * S > 16:
            continue
        announce(f"attend multi full size {name} S={S}")
        q = rng.standard_normal((wl.batch, S, wl.n_q_heads, wl.dim)).astype(np.float16)
        try:
            got = gpu_attend_multi(gk, gv, q, kc, kn, vc, vn, inp.lengths)
            break
        except tq.TQError as e:
            if e.status != tq.TQ_ERR_UNSUPPORTED:
                raise
    assert got is not None, "no multi-token kernel for this workload"
    del kc, kn, vc, vn

    def unit(bg):
        b, g = bg
        L = int(inp.lengths[b])
        okc, okn, _ = oracle.encode(ok, inp.k[b:b + 1, g:g + 1, :L])
        ovc, ovn, _ = oracle.encode(ov, inp.v[b:b + 1, g:g + 1, :L])
        qs = q[b:b + 1, :, g * G:(g + 1) * G]
        want = oracle.attend_causal_queries(ok, ov, qs, okc, okn, ovc, ovn, np.array([L]))
        return float(np.max(np.abs(got[b:b + 1, :, g * G:(g + 1) * G] - want)))

    errs = map_units(unit, [(b, g) for b in range(wl.batch) for g in range(wl.n_kv_heads)])
    assert max(errs) <= ATOL


# ------------------------------------------------------------------ packed + raw fp16 rows

def gpu_attend_mixed(kc, vc, q_np, kcodes, knorms, vcodes, vnorms, lengths_np, rk_np, rv_np,
                     rlen_np, max_len=None):
    B, Hq, d = q_np.shape
    Hkv = knorms.shape[1]
    if max_len is None:
        max_len = max(1, int(np.max(lengths_np)))
    lengths = torch.from_numpy(np.asarray(lengths_np, dtype=np.int32)).to(DEV)
    rlen = torch.from_numpy(np.asarray(rlen_np, dtype=np.int32)).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len), dtype=torch.uint8,
                     device=DEV)
    tq.tq_decode_attend_mixed(kc, vc, to_dev(q_np), kcodes, knorms, vcodes, vnorms, lengths,
                              max_len, to_dev(rk_np), to_dev(rv_np), rlen, 1.0 / math.sqrt(d),
                              out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,kb,vb,G", [(128, 8, 3, 4), (64, 4, 4, 2), (128, 4, 2, 3),
                                       (256, 3, 3, 4), (64, 3, 3, 8)])
def test_attend_mixed_matches_oracle(d, kb, vb, G):
    """Packed rows plus raw fp16 rows: a 128-row sink prefix with a long packed
    part, a short pending suffix (37 rows), raw rows only, and packed rows
    only (raw length 0), with raw segments over more than one 64-row step."""
    announce(f"attend mixed d={d} kb={kb} vb={vb} G={G}")
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(d + 3 * kb + 5 * vb + 7 * G)
    B, Hkv, T, R = 4, 2, 2100, 150
    Hq = G * Hkv
    lengths = np.array([T, 1500, 0, 777])
    rlen = np.array([128, 37, R, 0])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    rk = (rng.standard_normal((B, Hkv, R, d)) * 1.5).astype(np.float16)
    rv = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    got = gpu_attend_mixed(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv, rlen)
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    want = oracle.attend_mixed(ok, ov, q, okc, okn, ovc, ovn, lengths, rk, rv, rlen)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= ATOL
    # raw length 0: the same bits as the packed-only call
    single = gpu_attend(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths)
    assert got[3].tobytes() == single[3].tobytes()


def test_attend_mixed_no_rows_is_zero_and_raw_clamped():
    announce("attend mixed: no rows, raw length beyond max_raw")
    d, kb, vb, G = 128, 8, 3, 4
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(3)
    B, Hkv, T, R = 2, 1, 300, 70
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    rk = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    rv = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    lengths, rlen = np.array([0, 300]), np.array([0, 1000])   # 1000 is clamped to R
    got = gpu_attend_mixed(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv, rlen,
                           max_len=T)
    assert np.all(got[0] == 0.0)
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    want = oracle.attend_mixed(ok, ov, q, okc, okn, ovc, ovn, lengths, rk, rv, np.array([0, R]))
    assert np.max(np.abs(got[1] - want[1])) <= ATOL


def test_attend_mixed_maximum_raw_rows():
    """The raw segment at its maximum, 4096 fp16 rows per (sequence, KV head),
    with a packed part, against the oracle."""
    announce("attend mixed: 4096 raw rows")
    d, kb, vb, G = 128, 4, 2, 3
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(29)
    B, Hkv, T, R = 1, 2, 1000, 4096
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    rk = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    rv = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    lengths, rlen = np.array([T]), np.array([R])
    got = gpu_attend_mixed(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv, rlen)
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    want = oracle.attend_mixed(ok, ov, q, okc, okn, ovc, ovn, lengths, rk, rv, rlen)
    assert np.max(np.abs(got - want)) <= ATOL


def test_attend_mixed_raw_rows_past_length_unused():
    """Raw rows at or past raw_lengths (and packed rows past lengths) hold NaN:
    the result equals the one with clean buffers, bit for bit."""
    announce("attend mixed: NaN past the raw and packed lengths")
    d, kb, vb, G = 128, 4, 2, 3
    gk, _ = codecs(d, kb)
    gv, _ = codecs(d, vb)
    rng = np.random.default_rng(11)
    B, Hkv, T, R = 3, 2, 700, 96
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    rk = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    rv = rng.standard_normal((B, Hkv, R, d)).astype(np.float16)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    lengths, rlen = np.array([700, 300, 0]), np.array([5, 70, 96])
    kcodes, knorms = gpu_encode_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    clean = gpu_attend_mixed(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, rk, rv, rlen)
    rk2, rv2 = rk.copy(), rv.copy()
    for b in range(B):
        rk2[b, :, rlen[b]:] = np.nan
        rv2[b, :, rlen[b]:] = np.nan
        knorms[b, :, lengths[b]:] = float("nan")
        vnorms[b, :, lengths[b]:] = float("nan")
    poisoned = gpu_attend_mixed(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, rk2, rv2, rlen)
    assert np.all(np.isfinite(poisoned))
    assert poisoned.tobytes() == clean.tobytes()


def test_attend_mixed_workload_sink_prefix_full_size():
    """The 32K K8/V3 workload with its first 128 tokens kept as fp16 rows (the
    guide's --kv-min-tokens 128): every KV head against the oracle."""
    wl = workloads.WORKLOADS["llama8b_32k_k8v3"]
    announce(f"attend mixed full size {wl.name} sink 128")
    G = wl.n_q_heads // wl.n_kv_heads
    gk, ok = codecs(wl.dim, wl.k_bits, wl.codec_seed)
    gv, ov = codecs(wl.dim, wl.v_bits, wl.codec_seed)
    inp = workloads.generate(wl)
    S = 128
    kc, kn = gpu_encode_cache(gk, to_dev(np.ascontiguousarray(inp.k[:, :, S:])))
    vc, vn = gpu_encode_cache(gv, to_dev(np.ascontiguousarray(inp.v[:, :, S:])))
    rk = np.ascontiguousarray(inp.k[:, :, :S])
    rv = np.ascontiguousarray(inp.v[:, :, :S])
    lengths = inp.lengths - S
    got = gpu_attend_mixed(gk, gv, inp.q, kc, kn, vc, vn, lengths, rk, rv,
                           np.full(wl.batch, S, dtype=np.int32))
    del kc, kn, vc, vn

    def unit(g):
        L = int(lengths[0])
        okc, okn, _ = oracle.encode(ok, inp.k[0:1, g:g + 1, S:S + L])
        ovc, ovn, _ = oracle.encode(ov, inp.v[0:1, g:g + 1, S:S + L])
        want = oracle.attend_mixed(ok, ov, inp.q[0:1, g * G:(g + 1) * G], okc, okn, ovc, ovn,
                                   np.array([L]), rk[0:1, g:g + 1], rv[0:1, g:g + 1],
                                   np.array([S]))
        return float(np.max(np.abs(got[0:1, g * G:(g + 1) * G] - want)))

    assert max(map_units(unit, range(wl.n_kv_heads))) <= ATOL


# ------------------------------------------------------------------ raw fp16 keys

def gpu_attend_raw_k(vc, q_np, k_dev, vcodes, vnorms, lengths_np, max_len=None):
    B, Hq, d = q_np.shape
    Hkv = vnorms.shape[1]
    if max_len is None:
        max_len = max(1, int(np.max(lengths_np)))
    lengths = torch.from_numpy(np.asarray(lengths_np, dtype=np.int32)).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len), dtype=torch.uint8,
                     device=DEV)
    tq.tq_decode_attend_raw_k(vc, to_dev(q_np), k_dev, vcodes, vnorms, lengths, max_len,
                              1.0 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,vb,G", [(128, 4, 4), (128, 2, 3), (128, 4, 8), (64, 4, 2), (64, 4, 8),
                                    (64, 2, 3)])
def test_attend_raw_k_matches_oracle(d, vb, G):
    """Raw fp16 keys with packed values (turbo0v4 / turbo0v2) over ragged lengths
    spanning several tiles and splits, a length-1 and an empty sequence."""
    announce(f"attend raw K d={d} vb={vb} G={G}")
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(d + 11 * vb + 13 * G)
    B, Hkv, T = 4, 2, 2300
    Hq = G * Hkv
    lengths = np.array([T, 1100, 1, 0])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    got = gpu_attend_raw_k(gv, q, to_dev(k), vcodes, vnorms, lengths)
    ovc, ovn, _ = oracle.encode(ov, v)
    want = oracle.attend_raw_k(ov, q, k, ovc, ovn, lengths)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= ATOL
    assert np.all(got[3] == 0.0)


def test_attend_raw_k_llama8b_shape_32k():
    """32K context, 32/8 heads, d=128, fp16 K and 4-bit V (turbo0v4), the 32K
    workload's synthetic K/V: every KV head against the oracle."""
    wl = workloads.WORKLOADS["llama8b_32k_k8v3"]
    announce("attend raw K 32K turbo0v4")
    G = wl.n_q_heads // wl.n_kv_heads
    gv, ov = codecs(wl.dim, 4, wl.codec_seed)
    inp = workloads.generate(wl)
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(inp.v))
    got = gpu_attend_raw_k(gv, inp.q, to_dev(inp.k), vcodes, vnorms, inp.lengths)
    del vcodes, vnorms

    def unit(g):
        L = int(inp.lengths[0])
        ovc, ovn, _ = oracle.encode(ov, inp.v[0:1, g:g + 1, :L])
        want = oracle.attend_raw_k(ov, inp.q[0:1, g * G:(g + 1) * G], inp.k[0:1, g:g + 1, :L],
                                   ovc, ovn, np.array([L]))
        return float(np.max(np.abs(got[0:1, g * G:(g + 1) * G] - want)))

    assert max(map_units(unit, range(wl.n_kv_heads))) <= ATOL


# ------------------------------------------------------------------ TurboQuant-Prod keys

@functools.lru_cache(maxsize=None)
def prod_codecs(dim, bits, seed=42):
    return tq.tq_codec_init_prod(dim, bits, seed), oracle.ProdCodec(dim, bits, seed)


def gpu_encode_prod_rows(codec, x_np):
    N, H, d = x_np.shape
    x = to_dev(x_np)
    codes = torch.full((N, H, codec.row_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    sketch = torch.full((N, H, codec.sketch_bytes), 0x5A, dtype=torch.uint8, device=DEV)
    norms = torch.full((N, H), -1.0, dtype=torch.float32, device=DEV)
    rnorms = torch.full((N, H), -1.0, dtype=torch.float32, device=DEV)
    tq.tq_encode_prod(codec, x, codes, sketch, norms, rnorms)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), sketch.cpu().numpy(), norms.cpu().numpy(), rnorms.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("n", [384, None])
def test_encode_prod_matches_oracle(d, bits, n):
    """Codes, sketch bits, norms and residual norms bit-exact, in both encode
    layouts (n = None: just past the switch to the bulk layout)."""
    n = n or _bulk_layout_vectors(d) // 2 + 19
    announce(f"encode prod d={d} bits={bits} n={n}")
    g, o = prod_codecs(d, bits)
    x = _encode_inputs(d, d * 1000 + bits, n=n)
    codes, sketch, norms, rn = gpu_encode_prod_rows(g, x)
    oc, osk, on, orn = oracle.encode_prod(o, x)
    assert codes.tobytes() == oc.tobytes()
    assert norms.tobytes() == on.tobytes()
    assert rn.tobytes() == orn.tobytes()
    assert sketch.tobytes() == osk.tobytes()


def gpu_encode_prod_cache(codec, x_dev):
    B, H, T, d = x_dev.shape
    codes = torch.empty((B, H, T, codec.row_bytes), dtype=torch.uint8, device=DEV)
    sketch = torch.empty((B, H, T, codec.sketch_bytes), dtype=torch.uint8, device=DEV)
    norms = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    rnorms = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    tm = lambda a, *row: a.view(B * H, T, *row).permute(1, 0, *range(2, 2 + len(row)))
    tq.tq_encode_prod(codec, tm(x_dev, d), tm(codes, codec.row_bytes),
                      tm(sketch, codec.sketch_bytes), tm(norms), tm(rnorms))
    return codes, sketch, norms, rnorms


@pytest.mark.parametrize("d,kb,vb,G", [(128, 4, 4, 4), (128, 4, 4, 8), (128, 3, 3, 4),
                                       (64, 4, 4, 2)])
def test_attend_prod_matches_oracle(d, kb, vb, G):
    """Prod keys (codes + sketch + residual norms from the GPU encode, checked
    bit-exact first) with packed values over ragged lengths, several splits, a
    single-row and an empty sequence."""
    announce(f"attend prod d={d} kb={kb} vb={vb} G={G}")
    gk, ok = prod_codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(d + 3 * kb + 5 * vb + 7 * G)
    B, Hkv, T = 4, 2, 2200
    Hq = G * Hkv
    lengths = np.array([T, 1300, 1, 0])
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    kcodes, ksk, knorms, krn = gpu_encode_prod_cache(gk, to_dev(k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(v))
    okc, osk, okn, okr = oracle.encode_prod(ok, k)
    assert kcodes.cpu().numpy().tobytes() == okc.tobytes()
    assert ksk.cpu().numpy().tobytes() == osk.tobytes()
    assert krn.cpu().numpy().tobytes() == okr.tobytes()
    ovc, ovn, _ = oracle.encode(ov, v)
    lengths_d = torch.from_numpy(lengths.astype(np.int32)).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, T), dtype=torch.uint8, device=DEV)
    tq.tq_decode_attend_prod(gk, gv, to_dev(q), kcodes, ksk, knorms, krn, vcodes, vnorms,
                             lengths_d, T, 1.0 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.attend_prod(ok, ov, q, okc, osk, okn, okr, ovc, ovn, lengths)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= ATOL
    assert np.all(got[3] == 0.0)


def test_attend_prod_llama8b_shape_32k():
    """32K context, 32/8 heads, d=128, 4-bit Prod keys (3-bit codes + sketch)
    and 4-bit values over the 32K workload's synthetic K/V: every KV head
    against the oracle, the Prod encode of each head checked bit-exact."""
    wl = workloads.WORKLOADS["llama8b_32k_k8v3"]
    announce("attend prod 32K k4(prod) v4")
    G = wl.n_q_heads // wl.n_kv_heads
    gk, ok = prod_codecs(wl.dim, 4, wl.codec_seed)
    gv, ov = codecs(wl.dim, 4, wl.codec_seed)
    inp = workloads.generate(wl)
    B, Hkv, T = inp.k.shape[:3]
    kcodes, ksk, knorms, krn = gpu_encode_prod_cache(gk, to_dev(inp.k))
    vcodes, vnorms = gpu_encode_cache(gv, to_dev(inp.v))
    lengths_d = torch.from_numpy(inp.lengths.astype(np.int32)).to(DEV)
    out = torch.empty((B, wl.n_q_heads, wl.dim), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, wl.n_q_heads, Hkv, wl.dim, T),
                     dtype=torch.uint8, device=DEV)
    tq.tq_decode_attend_prod(gk, gv, to_dev(inp.q), kcodes, ksk, knorms, krn, vcodes, vnorms,
                             lengths_d, T, 1.0 / math.sqrt(wl.dim), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    kc_h, ks_h, kr_h = kcodes.cpu().numpy(), ksk.cpu().numpy(), krn.cpu().numpy()

    def unit(g):
        L = int(inp.lengths[0])
        okc, osk, okn, okr = oracle.encode_prod(ok, inp.k[0:1, g:g + 1, :L])
        assert kc_h[0, g, :L].tobytes() == okc.tobytes(), g
        assert ks_h[0, g, :L].tobytes() == osk.tobytes(), g
        assert kr_h[0, g, :L].tobytes() == okr.tobytes(), g
        ovc, ovn, _ = oracle.encode(ov, inp.v[0:1, g:g + 1, :L])
        want = oracle.attend_prod(ok, ov, inp.q[0:1, g * G:(g + 1) * G], okc, osk, okn, okr,
                                  ovc, ovn, np.array([L]))
        return float(np.max(np.abs(got[0:1, g * G:(g + 1) * G] - want)))

    assert max(map_units(unit, range(Hkv))) <= ATOL


# ------------------------------------------------------------ two-phase cache

@pytest.mark.parametrize("d,kb,vb,G,gsize,schedule", [
    # a 200-row prompt (3 groups + 8 pending), decode steps up to one row short
    # of a group, the flush, a long append that straddles the pending rows
    (128, 4, 2, 3, 64, [200] + [1] * 55 + [1, 1, 130, 5]),
    (64, 4, 4, 2, 16, [50] + [1] * 13 + [1, 37, 3]),
])
def test_cache_two_phase_matches_oracle(d, kb, vb, G, gsize, schedule):
    """The two-phase cache against its definition: after every append the
    first floor(rows / group) * group rows are packed exactly as the oracle
    encodes them, the rest sit in the pending buffer as fp16, and attention
    over the cache equals the oracle's attention over packed plus raw rows."""
    announce(f"two-phase cache d={d} kb={kb} vb={vb} G={G} group={gsize}")
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(d + gsize)
    B, Hkv, max_ctx = 2, 2, 512
    Hq = G * Hkv
    N = sum(schedule)
    k_all = rng.standard_normal((B, Hkv, N, d)).astype(np.float16)
    v_all = (rng.standard_normal((B, Hkv, N, d)) * 1.5).astype(np.float16)
    kcodes = torch.zeros((B, Hkv, max_ctx, gk.row_bytes), dtype=torch.uint8, device=DEV)
    vcodes = torch.zeros((B, Hkv, max_ctx, gv.row_bytes), dtype=torch.uint8, device=DEV)
    knorms = torch.zeros((B, Hkv, max_ctx), dtype=torch.float32, device=DEV)
    vnorms = torch.zeros((B, Hkv, max_ctx), dtype=torch.float32, device=DEV)
    pk = torch.zeros((B, Hkv, gsize, d), dtype=torch.float16, device=DEV)
    pv = torch.zeros((B, Hkv, gsize, d), dtype=torch.float16, device=DEV)
    plen = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    rlen = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    cache = tq.tq_cache_init(gk, gv, kcodes, knorms, vcodes, vnorms, pk, pv, plen, rlen)
    ws = torch.empty(tq.tq_cache_workspace_bytes(cache, Hq), dtype=torch.uint8, device=DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)

    def attend_and_check(pos):
        q = rng.standard_normal((B, Hq, d)).astype(np.float16)
        tq.tq_cache_attend(cache, to_dev(q), scale, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        n_packed = (pos // gsize) * gsize
        P = pos - n_packed
        assert plen.cpu().tolist() == [n_packed] * B and rlen.cpu().tolist() == [P] * B
        if pos == 0:
            assert np.all(got == 0.0)
            return
        npk = max(n_packed, 1)  # one row encoded, length 0, when nothing is packed
        okc, okn, _ = oracle.encode(ok, k_all[:, :, :npk])
        ovc, ovn, _ = oracle.encode(ov, v_all[:, :, :npk])
        want = oracle.attend_mixed(ok, ov, q, okc, okn, ovc, ovn, np.full(B, n_packed),
                                   k_all[:, :, n_packed:pos], v_all[:, :, n_packed:pos],
                                   np.full(B, P), scale)
        err = float(np.max(np.abs(got - want)))
        assert err <= ATOL, (pos, err)

    attend_and_check(0)                       # empty cache: zero rows
    pos = 0
    checks = {0, len(schedule) - 1, len(schedule) - 2, len(schedule) - 3, len(schedule) - 4,
              len(schedule) // 2}
    for i, n in enumerate(schedule):
        tq.tq_cache_append(cache, to_dev(k_all[:, :, pos:pos + n]), to_dev(v_all[:, :, pos:pos + n]))
        pos += n
        n_packed = (pos // gsize) * gsize
        assert tq.tq_cache_state(cache) == (n_packed, pos - n_packed)
        if i in checks:
            attend_and_check(pos)
    torch.cuda.synchronize()
    n_packed = (pos // gsize) * gsize
    okc, okn, _ = oracle.encode(ok, k_all[:, :, :n_packed])
    ovc, ovn, _ = oracle.encode(ov, v_all[:, :, :n_packed])
    assert kcodes[:, :, :n_packed].cpu().numpy().tobytes() == okc.tobytes()
    assert vcodes[:, :, :n_packed].cpu().numpy().tobytes() == ovc.tobytes()
    assert knorms[:, :, :n_packed].cpu().numpy().tobytes() == okn.tobytes()
    assert vnorms[:, :, :n_packed].cpu().numpy().tobytes() == ovn.tobytes()
    assert np.all(kcodes[:, :, n_packed:].cpu().numpy() == 0)          # nothing past the packed rows
    P = pos - n_packed
    assert pk[:, :, :P].cpu().numpy().tobytes() == np.ascontiguousarray(k_all[:, :, n_packed:pos]).tobytes()
    assert pv[:, :, :P].cpu().numpy().tobytes() == np.ascontiguousarray(v_all[:, :, n_packed:pos]).tobytes()
    cache.close()


# ------------------------------------------------------------ graph replay

def test_graph_replay_matches_eager():
    """The timed step (append encode of K and V, then decode attention) captured
    in a HIP graph: every replay, with eager work and synchronisations between
    replays, gives the same bits as the eager calls, and those match the oracle."""
    announce("graph replay of append + attend")
    d, kb, vb, G = 128, 8, 3, 4
    gk, ok = codecs(d, kb)
    gv, ov = codecs(d, vb)
    rng = np.random.default_rng(77)
    B, Hkv, T, P = 2, 2, 3000, 64
    Hq = G * Hkv
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float16)
    q = to_dev(rng.standard_normal((B, Hq, d)).astype(np.float16))
    kd, vd = to_dev(k), to_dev(v)
    kcodes, knorms = gpu_encode_cache(gk, kd[:, :, :T - P].contiguous())
    vcodes, vnorms = gpu_encode_cache(gv, vd[:, :, :T - P].contiguous())
    full = lambda c, n, row: (torch.cat([c, torch.zeros((B, Hkv, P) + row, dtype=c.dtype, device=DEV)], 2)
                              .contiguous())
    kcodes, vcodes = full(kcodes, None, (gk.row_bytes,)), full(vcodes, None, (gv.row_bytes,))
    knorms, vnorms = full(knorms, None, ()), full(vnorms, None, ())
    lengths = torch.full((B,), T, dtype=torch.int32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, T), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
    tm = lambda x, row: x.view(B * Hkv, T, *row).permute(1, 0, *range(2, 2 + len(row)))[T - P:T]

    def step():
        tq.tq_encode_kv(gk, tm(kd, (d,)), tm(kcodes, (gk.row_bytes,)), tm(knorms, ()),
                        gv, tm(vd, (d,)), tm(vcodes, (gv.row_bytes,)), tm(vnorms, ()))
        tq.tq_decode_attend(gk, gv, q, kcodes, knorms, vcodes, vnorms, lengths, T,
                            1.0 / math.sqrt(d), out, ws)

    step()
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        knorms[:, :, T - P:].fill_(-1.0)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == eager.tobytes(), f"replay {r}"
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    assert kcodes.cpu().numpy().tobytes() == okc.tobytes()
    assert knorms.cpu().numpy().tobytes() == okn.tobytes()
    want = oracle.attend(ok, ov, q.cpu().numpy(), okc, okn, ovc, ovn, np.full(B, T, np.int32))
    assert np.max(np.abs(eager - want)) <= ATOL
