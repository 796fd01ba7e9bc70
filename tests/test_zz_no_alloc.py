"""tq_decode_attend_noalloc: the decode attend with the library's fixed per-GPU
scratch array in place of a caller workspace. Through the C ABI it must give
tq_decode_attend's result bit for bit (same kernels, same plan), on two calls
in a row, the second with a smaller input, and stay within the attend
tolerance of the oracle."""
import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import compressed_domain_decode_amd as tq

DEV = "cuda:0"
ATOL = 2e-3


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _encode(codec, x_dev):
    B, H, T, d = x_dev.shape
    codes = torch.empty((B, H, T, codec.row_bytes), dtype=torch.uint8, device=DEV)
    norms = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    tq.tq_encode(codec, x_dev.view(B * H, T, d).permute(1, 0, 2),
                 codes.view(B * H, T, codec.row_bytes).permute(1, 0, 2),
                 norms.view(B * H, T).permute(1, 0))
    return codes, norms


def _case(seed, B, Hq, Hkv, d, T, lengths, kb, vb):
    lengths, k, v, q = workloads.small_case(seed, B, Hq, Hkv, d, T, lengths=lengths)
    kc, vc = tq.tq_codec_init(d, kb, 42), tq.tq_codec_init(d, vb, 42)
    kcodes, knorms = _encode(kc, torch.from_numpy(k).to(DEV))
    vcodes, vnorms = _encode(vc, torch.from_numpy(v).to(DEV))
    qd = torch.from_numpy(q).to(DEV)
    ld = torch.from_numpy(lengths).to(DEV)
    return (kc, vc, qd, kcodes, knorms, vcodes, vnorms, ld), (lengths, k, v, q)


def _run_both(args, max_len, scale):
    kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths = args
    B, Hq, d = q.shape
    Hkv = knorms.shape[1]
    ref = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len), dtype=torch.uint8,
                     device=DEV)
    tq.tq_decode_attend(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, max_len, scale, ref,
                        ws)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_decode_attend_noalloc(kc, vc, q, kcodes, knorms, vcodes, vnorms, lengths, max_len,
                                scale, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref.cpu().numpy()


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    # first call: 2 sequences, ragged, 8 query heads over 2 KV heads, several
    # splits per head; second call: a smaller input on the same array
    big, big_np = _case(11, 2, 8, 2, 128, 3000, [3000, 1777], 4, 2)
    small, small_np = _case(12, 1, 4, 1, 128, 500, [437], 4, 2)
    for tag, args, host, max_len in (("first, B2 T3000", big, big_np, 3000),
                                     ("second, B1 T500", small, small_np, 500)):
        announce(f"noalloc {tag}")
        scale = 1.0 / math.sqrt(128)
        out, ref = _run_both(args, max_len, scale)
        assert np.isfinite(out).all()
        np.testing.assert_array_equal(out, ref)  # same kernels, same plan: bit for bit
        lengths, k, v, q = host
        # the oracle encodes its own copy of the cache
        ok, ov = oracle.Codec(128, 4, 42), oracle.Codec(128, 2, 42)
        kco, kno, _ = oracle.encode(ok, k)
        vco, vno, _ = oracle.encode(ov, v)
        want = oracle.attend(ok, ov, q, kco, kno, vco, vno, lengths, scale)
        assert np.max(np.abs(out - want)) <= ATOL


@pytest.mark.gpu
def test_noalloc_after_larger_call_on_stale_scratch():
    # a long call leaves partials in the array; a shorter one (fewer splits)
    # must not read any of them
    long_args, _ = _case(21, 1, 8, 2, 128, 8192, [8192], 4, 2)
    short_args, _ = _case(22, 1, 8, 2, 128, 1024, [700], 4, 2)
    announce("noalloc stale-scratch pair")
    scale = 1.0 / math.sqrt(128)
    _run_both(long_args, 8192, scale)
    out, ref = _run_both(short_args, 1024, scale)
    np.testing.assert_array_equal(out, ref)


def test_noalloc_rejects_oversize_before_any_device_call():
    # 4096 sequences x 32 query heads x d 128 needs 64 MiB of partials; the
    # size check runs before the scratch lookup, so this runs without a GPU
    kc, vc = tq.tq_codec_init(128, 4, 42), tq.tq_codec_init(128, 2, 42)
    need = tq.tq_attend_workspace_bytes(4096, 32, 8, 128, 64)
    assert need > tq.TQ_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    st = tq._lib.tq_decode_attend_noalloc(kc.handle, vc.handle, fake, 4096, 32, 8, fake, fake,
                                          fake, fake, 64, fake, 64, ctypes.c_float(0.1), fake,
                                          None)
    assert st == tq.TQ_ERR_UNSUPPORTED
    assert "scratch" in tq.tq_last_error()
