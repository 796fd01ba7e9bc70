"""GPU parity of the dense-rotation codec (head dims with no Walsh-Hadamard
transform) through the C ABI against the CPU oracle.

Bar as for the Walsh-Hadamard path: packed codes byte-identical and norms
bit-identical; decode-attend outputs within 2e-3 max-abs of the oracle's fp64
result. The rotation is the same seeded fp64 matrix on both sides (an input of
the method); the oracle encodes its own copy of every cache it attends over.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import compressed_domain_decode_amd as tq
from workloads import rotation_matrix

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATOL = 2e-3


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def dense_codecs(dim, bits, seed):
    m = rotation_matrix(dim, seed)
    return tq.tq_codec_init_dense(dim, bits, m), oracle.DenseCodec(m, bits)


def _inputs(rng, shape, d):
    x = rng.standard_normal(shape)
    x[..., rng.choice(d, 2, replace=False)] *= 6.0
    return x.astype(np.float16)


def gpu_encode_cache(codec, x_np):
    """x (B, H, T, d) fp16 -> codes (B, H, T, row), norms (B, H, T), one tq_encode
    over token-major views of the head-major cache."""
    B, H, T, d = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    codes = torch.full((B, H, T, codec.row_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    norms = torch.full((B, H, T), -1.0, dtype=torch.float32, device=DEV)
    xv = x.view(B * H, T, d).permute(1, 0, 2)
    cv = codes.view(B * H, T, codec.row_bytes).permute(1, 0, 2)
    nv = norms.view(B * H, T).permute(1, 0)
    tq.tq_encode(codec, xv, cv, nv)
    return codes, norms


def gpu_attend(kc, vc, q_np, kcodes, knorms, vcodes, vnorms, lengths_np, max_len=None):
    B, Hq, d = q_np.shape
    Hkv = knorms.shape[1]
    if max_len is None:
        max_len = max(1, int(np.max(lengths_np)))
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to(DEV)
    lengths = torch.from_numpy(np.asarray(lengths_np, dtype=np.int32)).to(DEV)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len), dtype=torch.uint8,
                     device=DEV)
    tq.tq_decode_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, max_len,
                        1.0 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,bits", [(96, 2), (96, 3), (96, 4), (96, 8), (160, 3), (192, 4),
                                    (32, 1), (224, 5), (256, 6), (128, 7),
                                    # the LDS-staged kernel (d <= 96): every width
                                    (96, 1), (96, 5), (96, 6), (96, 7), (64, 2), (64, 5),
                                    (64, 8), (32, 4), (32, 8)])
def test_dense_encode_matches_oracle(d, bits):
    announce(f"dense encode d={d} bits={bits}")
    g, o = dense_codecs(d, bits, 7)
    rng = np.random.default_rng(d * 16 + bits)
    x = _inputs(rng, (2, 3, 67, d), d)          # 402 vectors: a ragged last workgroup
    x[0, 0, 5] = 0                               # zero vector
    codes, norms = gpu_encode_cache(g, x)
    oc, on, _ = oracle.encode_dense(o, x)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(norms.cpu().numpy().view(np.uint32), on.view(np.uint32))


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4), (256, 8)])
def test_dense_hadamard_matrix_equals_wht_codec_on_gpu(d, bits):
    announce(f"dense H diag(sigma) vs WHT codec d={d} bits={bits}")
    wc = tq.tq_codec_init(d, bits, 42)
    signs = oracle.Codec(d, bits, 42).signs.astype(np.float64)
    m = oracle.hadamard(d) * signs[None, :]
    dc = tq.tq_codec_init_dense(d, bits, m)
    x = _inputs(np.random.default_rng(d + bits), (1, 4, 130, d), d)
    c1, n1 = gpu_encode_cache(wc, x)
    c2, n2 = gpu_encode_cache(dc, x)
    assert torch.equal(c1, c2) and torch.equal(n1, n2)


def _attend_case(d, kb, vb, G, Hkv, lengths, T, seed):
    kc, ko = dense_codecs(d, kb, seed)
    vc, vo = dense_codecs(d, vb, seed + 1)
    rng = np.random.default_rng(seed)
    B = len(lengths)
    k = _inputs(rng, (B, Hkv, T, d), d)
    v = _inputs(rng, (B, Hkv, T, d), d)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(kc, k)
    vcodes, vnorms = gpu_encode_cache(vc, v)
    out = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    okc, okn, _ = oracle.encode_dense(ko, k)
    ovc, ovn, _ = oracle.encode_dense(vo, v)
    ref = oracle.attend_dense(ko, vo, q, okc, okn, ovc, ovn, np.asarray(lengths))
    return out, ref


@pytest.mark.parametrize("d,kb,vb,G,Hkv,lengths,T", [
    (96, 4, 2, 3, 4, [300, 1], 300),             # Phi-3-mini head dim; ragged tail
    (96, 8, 3, 1, 2, [257, 0, 64], 257),         # length 0 -> zero rows; exactly one tile
    (160, 3, 3, 2, 2, [1000], 1000),             # several splits per head
    (192, 4, 4, 4, 2, [777, 129], 777),
    (32, 1, 8, 16, 1, [5000], 5000),             # 16 query heads per KV head, many splits
    (224, 2, 5, 8, 1, [63, 65], 65),
    (192, 3, 4, 1, 3, [400, 129], 400),          # one query head per KV head, d > 128
    (96, 4, 2, 4, 2, [300, 77], 300),            # four per KV head, d <= 128
])
def test_dense_attend_matches_oracle(d, kb, vb, G, Hkv, lengths, T):
    announce(f"dense attend d={d} K{kb}/V{vb} G={G} Hkv={Hkv} lengths={lengths}")
    out, ref = _attend_case(d, kb, vb, G, Hkv, lengths, T, seed=d + kb)
    assert np.isfinite(out).all()
    err = np.abs(out - ref).max()
    assert err <= ATOL, err
    for b, L in enumerate(lengths):
        if L == 0:
            assert np.all(out[b] == 0.0)


@pytest.mark.parametrize("kb", [2, 3, 4, 8])
@pytest.mark.parametrize("vb", [2, 3, 4])
def test_dense_attend_one_head_per_kv_head(kb, vb):
    """Head dim 96 with one query head per KV head runs the register-held
    kernel (two lanes per token, per-lane softmax state): every K/V bit pair it
    has, with ragged tails, a range shorter than one wavefront step, a lone
    token and an empty sequence."""
    d, G, Hkv = 96, 1, 2
    lengths, T = [700, 33, 1, 0], 700
    announce(f"dense attend one head per KV head d={d} K{kb}/V{vb} lengths={lengths}")
    out, ref = _attend_case(d, kb, vb, G, Hkv, lengths, T, seed=400 + 10 * kb + vb)
    assert np.isfinite(out).all()
    err = np.abs(out - ref).max()
    assert err <= ATOL, err
    assert np.all(out[3] == 0.0)


@pytest.mark.parametrize("qmul", [1.0, 24.0])
def test_dense_attend_one_head_per_kv_head_long(qmul):
    """Several splits per sequence, tails that end inside a step, and (qmul 24)
    scores spread over a range of hundreds in base 2, so the lanes' running
    maxima move many times."""
    d, kb, vb, G, Hkv = 96, 4, 3, 1, 3
    lengths, T = [4100, 2049, 95], 4100
    announce(f"dense attend one head per KV head d={d} K{kb}/V{vb} q x {qmul} lengths={lengths}")
    kc, ko = dense_codecs(d, kb, 51)
    vc, vo = dense_codecs(d, vb, 52)
    rng = np.random.default_rng(53)
    B = len(lengths)
    k = _inputs(rng, (B, Hkv, T, d), d)
    v = _inputs(rng, (B, Hkv, T, d), d)
    q = (rng.standard_normal((B, G * Hkv, d)) * qmul).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(kc, k)
    vcodes, vnorms = gpu_encode_cache(vc, v)
    out = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths)
    okc, okn, _ = oracle.encode_dense(ko, k)
    ovc, ovn, _ = oracle.encode_dense(vo, v)
    ref = oracle.attend_dense(ko, vo, q, okc, okn, ovc, ovn, np.asarray(lengths))
    assert np.isfinite(out).all()
    err = np.abs(out - ref).max()
    assert err <= ATOL, err


def test_dense_attend_phi3_mini_shape_sampled():
    """A Phi-3-mini-shaped layer (32 query and 32 KV heads, head dim 96) at 4096
    tokens, K4/V2, in the launch configuration of a full call; sampled KV heads
    checked against the oracle."""
    d, Hkv, G, T = 96, 32, 1, 4096
    announce(f"dense attend phi3-mini shape d={d} Hkv={Hkv} T={T}")
    kc, ko = dense_codecs(d, 4, 5)
    vc, vo = dense_codecs(d, 2, 6)
    rng = np.random.default_rng(17)
    k = _inputs(rng, (1, Hkv, T, d), d)
    v = _inputs(rng, (1, Hkv, T, d), d)
    q = rng.standard_normal((1, Hkv * G, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(kc, k)
    vcodes, vnorms = gpu_encode_cache(vc, v)
    out = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, [T])
    for g in (0, 13, 31):
        okc, okn, _ = oracle.encode_dense(ko, k[:, g:g + 1])
        ovc, ovn, _ = oracle.encode_dense(vo, v[:, g:g + 1])
        assert np.array_equal(kcodes[:, g:g + 1].cpu().numpy(), okc)
        ref = oracle.attend_dense(ko, vo, q[:, g * G:(g + 1) * G], okc, okn, ovc, ovn,
                                  np.array([T]))
        assert np.abs(out[:, g * G:(g + 1) * G] - ref).max() <= ATOL


@pytest.mark.parametrize("G", [3, 1])
def test_dense_attend_rows_beyond_length_never_read(G):
    """Rows past each sequence's length hold 0xFF codes and NaN norms; a device
    length above max_len is clamped to it. The cache is allocated well past
    what the launch covers (max_ctx 1000 against 5 splits of 64 tokens), so
    every read stays in bounds even where a length exceeds max_len. G = 1 runs
    the register-held kernel, whose steps past a range's end read its last row."""
    d, kb, vb, Hkv, T, max_len = 96, 4, 2, 2, 1000, 300
    announce(f"dense attend poisoned rows d={d} G={G} max_ctx={T} max_len={max_len}")
    kc, _ = dense_codecs(d, kb, 31)
    vc, _ = dense_codecs(d, vb, 32)
    rng = np.random.default_rng(33)
    lens = [300, 77, 150]
    B = len(lens)
    k = _inputs(rng, (B, Hkv, T, d), d)
    v = _inputs(rng, (B, Hkv, T, d), d)
    q = rng.standard_normal((B, G * Hkv, d)).astype(np.float16)
    kcodes, knorms = gpu_encode_cache(kc, k)
    vcodes, vnorms = gpu_encode_cache(vc, v)
    clean = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lens, max_len=max_len)
    for b, L in enumerate(lens):
        kcodes[b, :, L:] = 0xFF
        vcodes[b, :, L:] = 0xFF
        knorms[b, :, L:] = float("nan")
        vnorms[b, :, L:] = float("nan")
    dirty = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lens, max_len=max_len)
    assert np.isfinite(dirty).all()
    assert clean.tobytes() == dirty.tobytes()
    # sequence 0 claims 900 rows on the device; max_len 300 bounds what is read
    over = gpu_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, [900, 77, 150],
                      max_len=max_len)
    assert clean.tobytes() == over.tobytes()


def test_dense_codecs_rejected_where_unsupported():
    d = 96
    kc, _ = dense_codecs(d, 4, 1)
    wc = tq.tq_codec_init(128, 4, 42)
    q = torch.zeros((1, 2, d), dtype=torch.float16, device=DEV)
    k = torch.zeros((1, 1, 64, kc.row_bytes), dtype=torch.uint8, device=DEV)
    n = torch.zeros((1, 1, 64), dtype=torch.float32, device=DEV)
    lengths = torch.ones(1, dtype=torch.int32, device=DEV)
    out = torch.zeros((1, 2, d), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(1, 2, 1, d, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(tq.TQError) as e:   # a dense K codec with a WHT V codec of another dim
        tq.tq_decode_attend(kc, wc, q, k, n, k, n, lengths, 64, 0.1, out, ws)
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    with pytest.raises(tq.TQError) as e:   # multi-token decode is not offered for dense codecs
        tq.tq_decode_attend_multi(kc, kc, q.view(1, 2, 1, d), k, n, k, n, lengths, 64, 0.1,
                                  out.view(1, 2, 1, d), ws)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("G", [3, 1])
def test_dense_graph_replay_matches_eager(G):
    """The dense attend captured in a HIP graph: three replays, with eager work
    between them, bitwise equal to the eager call."""
    d, Hkv, T = 96, 2, 700
    announce(f"dense attend graph replay d={d} G={G} T={T}")
    kc, _ = dense_codecs(d, 4, 21)
    vc, _ = dense_codecs(d, 3, 22)
    rng = np.random.default_rng(23)
    k = _inputs(rng, (1, Hkv, T, d), d)
    v = _inputs(rng, (1, Hkv, T, d), d)
    q = torch.from_numpy(rng.standard_normal((1, G * Hkv, d)).astype(np.float16)).to(DEV)
    kcodes, knorms = gpu_encode_cache(kc, k)
    vcodes, vnorms = gpu_encode_cache(vc, v)
    lengths = torch.tensor([T], dtype=torch.int32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(1, G * Hkv, Hkv, d, T), dtype=torch.uint8,
                     device=DEV)
    eager = torch.empty((1, G * Hkv, d), dtype=torch.float32, device=DEV)
    tq.tq_decode_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, T, 0.1, eager, ws)
    torch.cuda.synchronize()
    out = torch.full_like(eager, float("nan"))

    def call():
        tq.tq_decode_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, T, 0.1, out, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        out.fill_(float("nan"))
        ws.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
