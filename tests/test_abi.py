"""C-ABI boundary tests that need no GPU: the library loads, exports every
symbol include/tq.h declares, builds codec tables identical to the oracle's,
and rejects bad arguments before enqueueing anything."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import compressed_domain_decode_amd as tq
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "tq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    declared = _declared_functions()
    assert set(declared) == set(tq.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", tq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(tq.LIB_PATH)
    for f in declared:
        assert hasattr(lib, f)


def test_header_compiles_as_plain_c():
    r = subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-Wall", "-Werror", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_library_has_no_oracle_dependency():
    out = subprocess.run(["nm", "-D", tq.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["ldd", tq.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


@pytest.mark.parametrize("dim", [64, 128, 256])
@pytest.mark.parametrize("bits", range(1, 9))
def test_codec_tables_match_oracle_bitwise(dim, bits):
    c = tq.tq_codec_init(dim, bits, 42)
    s, cent, bnd = tq.tq_codec_tables(c)
    o = oracle.Codec(dim, bits, 42)
    np.testing.assert_array_equal(s, o.signs)
    assert cent.tobytes() == o.centroids.tobytes()
    assert bnd.tobytes() == o.boundaries.tobytes()
    assert tq.tq_codec_info(c) == (dim, bits, 42)
    assert tq.tq_row_bytes(dim, bits) == dim * bits // 8


@pytest.mark.parametrize("seed", [0, 1, 7, 2**63 + 5])
def test_codec_signs_match_oracle_for_seeds(seed):
    c = tq.tq_codec_init(128, 3, seed)
    np.testing.assert_array_equal(tq.tq_codec_tables(c)[0], oracle.signs(seed, 128))


@pytest.mark.parametrize("dim,bits", [(32, 4), (96, 4), (512, 4), (0, 4), (128, 0), (128, 9), (128, -1)])
def test_codec_init_rejects_unsupported(dim, bits):
    with pytest.raises(tq.TQError) as e:
        tq.tq_codec_init(dim, bits, 1)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    assert "tq_codec_init" in tq.tq_last_error()


@pytest.mark.parametrize("dim,bits", [(80, 4), (288, 4), (0, 4), (16, 4), (96, 0), (96, 9)])
def test_codec_init_dense_rejects_unsupported(dim, bits):
    m = np.eye(max(dim, 1)) * np.sqrt(max(dim, 1))
    lib = ctypes.CDLL(tq.LIB_PATH)
    lib.tq_codec_init_dense.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_void_p)]
    h = ctypes.c_void_p(1)
    assert lib.tq_codec_init_dense(dim, bits, m.ctypes.data, ctypes.byref(h)) == \
        tq.TQ_ERR_UNSUPPORTED
    assert h.value is None
    assert "tq_codec_init_dense" in tq.tq_last_error()


def test_codec_init_dense_invalid_arguments():
    lib = ctypes.CDLL(tq.LIB_PATH)
    lib.tq_codec_init_dense.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    m = np.eye(96) * np.sqrt(96)
    h = ctypes.c_void_p()
    assert lib.tq_codec_init_dense(96, 4, m.ctypes.data, None) == tq.TQ_ERR_INVALID_ARG
    assert lib.tq_codec_init_dense(96, 4, None, ctypes.addressof(h)) == tq.TQ_ERR_INVALID_ARG
    bad = m.copy()
    bad[3, 7] = np.nan
    assert lib.tq_codec_init_dense(96, 4, bad.ctypes.data, ctypes.addressof(h)) == \
        tq.TQ_ERR_INVALID_ARG
    bad[3, 7] = np.inf
    assert lib.tq_codec_init_dense(96, 4, bad.ctypes.data, ctypes.addressof(h)) == \
        tq.TQ_ERR_INVALID_ARG
    assert "not finite" in tq.tq_last_error()
    with pytest.raises(ValueError):
        tq.tq_codec_init_dense(96, 4, np.eye(64))


def test_codec_init_null_out():
    lib = ctypes.CDLL(tq.LIB_PATH)
    lib.tq_codec_init.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p]
    assert lib.tq_codec_init(128, 4, 1, None) == tq.TQ_ERR_INVALID_ARG


def test_status_strings():
    for s, name in [(0, "TQ_OK"), (-1, "TQ_ERR_INVALID_ARG"), (-2, "TQ_ERR_UNSUPPORTED"),
                    (-3, "TQ_ERR_WORKSPACE"), (-4, "TQ_ERR_HIP"), (-5, "TQ_ERR_NOMEM")]:
        assert tq.tq_status_string(s) == name


# ---- argument validation: every call below fails before any HIP call is made

_lib = ctypes.CDLL(tq.LIB_PATH)
_lib.tq_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_void_p]
_lib.tq_decode_attend.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + \
    [ctypes.c_void_p] * 4 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_float,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
FAKE = 0x10000  # never dereferenced: validation fails first


def test_encode_validation():
    c = tq.tq_codec_init(128, 4, 1)
    h = c.handle
    assert _lib.tq_encode(None, FAKE, 1, 1, 128, 128, FAKE, 64, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert _lib.tq_encode(h, None, 1, 1, 128, 128, FAKE, 64, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert _lib.tq_encode(h, FAKE, -1, 1, 128, 128, FAKE, 64, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert _lib.tq_encode(h, FAKE, 1, 1, 128, 128, FAKE + 2, 64, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert _lib.tq_encode(h, FAKE, 1, 1, 128, 128, FAKE, 66, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    assert _lib.tq_encode(h, FAKE + 1, 1, 1, 128, 128, FAKE, 64, 64, FAKE, 1, 1, None) == tq.TQ_ERR_INVALID_ARG
    # nothing to do is fine and touches nothing
    assert _lib.tq_encode(h, None, 0, 5, 0, 0, None, 0, 0, None, 0, 0, None) == tq.TQ_OK


def test_encode_kv_validation():
    kc = tq.tq_codec_init(128, 8, 1)
    vc = tq.tq_codec_init(128, 3, 1)
    other = tq.tq_codec_init(64, 3, 1)
    J = tq._EncodeJob
    P = ctypes.POINTER(J)
    f = tq._lib.tq_encode_kv

    def job(c, x=FAKE, codes=FAKE, cst=64, norms=FAKE):
        return J(c.handle if c else None, x, 128, 128, codes, cst, cst, norms, 1, 1)

    def call(k, v, n_tok=1, n_head=1):
        return f(ctypes.byref(k) if k is not None else P(), ctypes.byref(v) if v is not None else P(),
                 n_tok, n_head, None)

    assert call(None, job(vc)) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc), None) == tq.TQ_ERR_INVALID_ARG
    assert call(job(None), job(vc)) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc), job(other)) == tq.TQ_ERR_INVALID_ARG      # dims differ
    assert call(job(kc), job(vc), n_tok=-1) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc), job(vc, x=None)) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc), job(vc, codes=FAKE + 2)) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc, cst=66), job(vc)) == tq.TQ_ERR_INVALID_ARG
    assert call(job(kc), job(vc, norms=FAKE + 2)) == tq.TQ_ERR_INVALID_ARG
    assert "job 1" in tq.tq_last_error()
    # nothing to do is fine and touches nothing
    assert call(job(kc, x=None), job(vc, x=None), n_tok=0) == tq.TQ_OK


def _attend_call(kc, vc, B=1, Hq=4, Hkv=2, max_ctx=256, max_len=256, ws=FAKE, ws_bytes=1 << 30,
                 q=FAKE, out=FAKE):
    return _lib.tq_decode_attend(kc.handle, vc.handle, q, B, Hq, Hkv, FAKE, FAKE, FAKE, FAKE,
                                 max_ctx, FAKE, max_len, 0.125, out, ws, ws_bytes, None)


def test_decode_attend_validation():
    kc, vc = tq.tq_codec_init(64, 4, 42), tq.tq_codec_init(64, 4, 42)
    vc128 = tq.tq_codec_init(128, 4, 42)
    assert _attend_call(kc, vc128) == tq.TQ_ERR_INVALID_ARG          # dim mismatch
    assert _attend_call(kc, vc, Hq=5, Hkv=2) == tq.TQ_ERR_INVALID_ARG  # ratio
    assert _attend_call(kc, vc, Hq=34, Hkv=2) == tq.TQ_ERR_UNSUPPORTED  # group 17
    assert _attend_call(kc, vc, B=0) == tq.TQ_ERR_INVALID_ARG
    assert _attend_call(kc, vc, max_len=300, max_ctx=256) == tq.TQ_ERR_INVALID_ARG
    assert _attend_call(kc, vc, max_len=0) == tq.TQ_ERR_INVALID_ARG
    assert _attend_call(kc, vc, q=None) == tq.TQ_ERR_INVALID_ARG
    assert _attend_call(kc, vc, out=FAKE + 2) == tq.TQ_ERR_INVALID_ARG
    need = tq.tq_attend_workspace_bytes(1, 4, 2, 64, 256)
    assert need > 0
    assert _attend_call(kc, vc, ws_bytes=need - 1) == tq.TQ_ERR_WORKSPACE
    assert _attend_call(kc, vc, ws=None) == tq.TQ_ERR_WORKSPACE
    assert _attend_call(kc, vc, ws=FAKE + 64) == tq.TQ_ERR_INVALID_ARG  # not 256-aligned
    assert "workspace" in tq.tq_last_error() or "aligned" in tq.tq_last_error()


def test_decode_attend_multi_validation():
    kc = tq.tq_codec_init(128, 8, 1)
    vc = tq.tq_codec_init(128, 3, 1)
    f = tq._lib.tq_decode_attend_multi

    def call(S, Hq=32, Hkv=8, ws_bytes=1 << 30):
        return f(kc.handle, vc.handle, FAKE, 1, S, Hq, Hkv, FAKE, FAKE, FAKE, FAKE, 256, FAKE,
                 256, 0.125, FAKE, FAKE, ws_bytes, None)

    assert call(0) == tq.TQ_ERR_INVALID_ARG
    assert call(5) == tq.TQ_ERR_UNSUPPORTED          # 4 heads x 5 query tokens > 16
    assert "query tokens" in tq.tq_last_error()
    v5 = tq.tq_codec_init(128, 5, 1)                 # no K8/V5 kernel at all
    assert f(kc.handle, v5.handle, FAKE, 1, 2, 32, 8, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 256,
             0.125, FAKE, FAKE, 1 << 30, None) == tq.TQ_ERR_UNSUPPORTED
    assert call(4, ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    one = tq.tq_attend_workspace_bytes(1, 32, 8, 128, 4096)
    assert tq.tq_attend_multi_workspace_bytes(1, 1, 32, 8, 128, 4096) == one
    assert tq.tq_attend_multi_workspace_bytes(1, 4, 32, 8, 128, 4096) > one
    assert tq.tq_attend_multi_workspace_bytes(1, 0, 32, 8, 128, 4096) == 0


def test_decode_attend_mixed_validation():
    kc = tq.tq_codec_init(128, 8, 1)
    vc = tq.tq_codec_init(128, 3, 1)
    f = tq._lib.tq_decode_attend_mixed

    def call(rk=FAKE, rv=FAKE, max_raw=128, rlen=FAKE, ws_bytes=1 << 30):
        return f(kc.handle, vc.handle, FAKE, 1, 32, 8, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 256,
                 rk, rv, max_raw, rlen, 0.125, FAKE, FAKE, ws_bytes, None)

    assert call(max_raw=0) == tq.TQ_ERR_INVALID_ARG
    assert call(max_raw=4097) == tq.TQ_ERR_UNSUPPORTED        # raw scores are held in LDS
    assert call(rk=None) == tq.TQ_ERR_INVALID_ARG
    assert call(rlen=None) == tq.TQ_ERR_INVALID_ARG
    assert call(rv=FAKE + 8) == tq.TQ_ERR_INVALID_ARG           # raw rows 16-byte aligned
    assert "raw" in tq.tq_last_error()
    assert call(ws_bytes=16) == tq.TQ_ERR_WORKSPACE


def test_decode_attend_raw_k_validation():
    vc = tq.tq_codec_init(128, 4, 1)
    v3 = tq.tq_codec_init(128, 3, 1)
    f = tq._lib.tq_decode_attend_raw_k

    def call(codec=vc, k=FAKE, Hq=32, ws_bytes=1 << 30):
        return f(codec.handle if codec else None, FAKE, 1, Hq, 8, k, FAKE, FAKE, 256, FAKE, 256,
                 0.125, FAKE, FAKE, ws_bytes, None)

    assert call(codec=None) == tq.TQ_ERR_INVALID_ARG
    assert call(k=None) == tq.TQ_ERR_INVALID_ARG
    assert call(k=FAKE + 8) == tq.TQ_ERR_INVALID_ARG               # 16-byte aligned keys
    assert call(codec=v3) == tq.TQ_ERR_UNSUPPORTED                 # no fp16-K / 3-bit V kernel
    assert call(ws_bytes=16) == tq.TQ_ERR_WORKSPACE


def test_prod_codec_and_encode_validation():
    with pytest.raises(tq.TQError):
        tq.tq_codec_init_prod(128, 1, 0)                  # needs at least 1 + 1 bits
    with pytest.raises(tq.TQError):
        tq.tq_codec_init_prod(128, 9, 0)
    pc = tq.tq_codec_init_prod(128, 4, 7)
    plain = tq.tq_codec_init(128, 3, 7)
    # the MSE part is the plain 3-bit codec with the same seed
    s1, c1, b1 = tq.tq_codec_tables(pc)
    s2, c2, b2 = tq.tq_codec_tables(plain)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2) and np.array_equal(b1, b2)
    f = tq._lib.tq_encode_prod
    args = [FAKE, 1, 1, 128, 128, FAKE, 48, 48, FAKE, 16, 16, FAKE, 1, 1, FAKE, 1, 1, None]
    assert f(pc.handle, *args[:8], None, *args[9:]) == tq.TQ_ERR_INVALID_ARG      # no sketch
    assert f(pc.handle, *args[:14], FAKE + 2, *args[15:]) == tq.TQ_ERR_INVALID_ARG  # rnorms align
    assert f(plain.handle, *args) == tq.TQ_ERR_INVALID_ARG     # plain codec: tq_encode
    assert "tq_encode" in tq.tq_last_error()
    # and a Prod codec is refused by tq_encode
    assert _lib.tq_encode(pc.handle, FAKE, 1, 1, 128, 128, FAKE, 48, 48, FAKE, 1, 1, None) == \
        tq.TQ_ERR_INVALID_ARG


def test_decode_attend_prod_validation():
    pk = tq.tq_codec_init_prod(128, 4, 1)
    plain = tq.tq_codec_init(128, 4, 1)
    vc = tq.tq_codec_init(128, 4, 1)
    f = tq._lib.tq_decode_attend_prod

    def call(kc=pk, sk=FAKE, rn=FAKE, v=vc, ws_bytes=1 << 30):
        return f(kc.handle, v.handle, FAKE, 1, 32, 8, FAKE, sk, FAKE, rn, FAKE, FAKE, 256, FAKE,
                 256, 0.125, FAKE, FAKE, ws_bytes, None)

    assert call(kc=plain) == tq.TQ_ERR_INVALID_ARG            # needs a Prod K codec
    assert call(sk=None) == tq.TQ_ERR_INVALID_ARG
    assert call(sk=FAKE + 8) == tq.TQ_ERR_INVALID_ARG
    assert call(rn=FAKE + 2) == tq.TQ_ERR_INVALID_ARG
    assert call(v=pk) == tq.TQ_ERR_INVALID_ARG                 # V cannot be a Prod codec
    assert call(ws_bytes=16) == tq.TQ_ERR_WORKSPACE
    # a Prod K codec is refused by the plain call
    assert _attend_call(pk, vc) == tq.TQ_ERR_INVALID_ARG


def test_workspace_and_split_plan():
    assert tq.tq_attend_workspace_bytes(1, 4, 3, 64, 10) == 0
    assert tq.tq_attend_workspace_bytes(1, 4, 2, 96, 10) > 0     # dense-rotation dims
    assert tq.tq_attend_workspace_bytes(1, 4, 2, 80, 10) == 0     # not a multiple of 32
    assert tq.tq_attend_workspace_bytes(1, 4, 2, 288, 10) == 0
    for (B, Hq, Hkv, d, L) in [(1, 4, 2, 64, 256), (1, 32, 8, 128, 32768), (16, 32, 8, 128, 8192),
                               (1, 64, 8, 64, 131072), (1, 24, 8, 128, 4096)]:
        S = tq.tq_attend_num_splits(B, Hq, Hkv, d, L)
        ws = tq.tq_attend_workspace_bytes(B, Hq, Hkv, d, L)
        assert S >= 1
        assert ws >= B * Hq * S * (d + 2) * 4
        assert ws % 256 == 0


def test_single_hip_runtime_in_process():
    """The binding must not bring a second HIP runtime next to torch's."""
    import torch  # noqa: F401
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


@pytest.mark.parametrize("name", ["tq_stream_read", "tq_stream_read_resident"])
def test_stream_read_validation(name):
    lib = ctypes.CDLL(tq.LIB_PATH)
    fn = getattr(lib, name)
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert fn(None, 0, None, None) == tq.TQ_OK          # nothing to read
    assert fn(None, 64, FAKE, None) == tq.TQ_ERR_INVALID_ARG
    assert fn(FAKE, 64, None, None) == tq.TQ_ERR_INVALID_ARG
    assert fn(FAKE + 8, 64, FAKE, None) == tq.TQ_ERR_INVALID_ARG  # alignment
    assert fn(FAKE, 60, FAKE, None) == tq.TQ_ERR_INVALID_ARG      # size
    assert name in tq.tq_last_error()


def _cache_desc(**kw):
    d = dict(batch=2, n_kv_heads=2, max_ctx=256, group_size=64, k_codes=FAKE, k_norms=FAKE,
             v_codes=FAKE, v_norms=FAKE, pending_k=FAKE, pending_v=FAKE, packed_len=FAKE,
             pending_len=FAKE)
    d.update(kw)
    return tq._CacheDesc(**d)


def _cache_init(kc, vc, desc):
    h = ctypes.c_void_p()
    st = tq._lib.tq_cache_init(kc.handle if kc else None, vc.handle if vc else None,
                               ctypes.byref(desc) if desc is not None else None, ctypes.byref(h))
    return st, h


def test_cache_validation():
    """Two-phase cache: descriptor checks at init, counts of an empty cache, and
    appends refused (too many rows, bad rows) or empty, none of which launches."""
    kc, vc = tq.tq_codec_init(128, 4, 42), tq.tq_codec_init(128, 2, 42)
    other = tq.tq_codec_init(64, 2, 42)
    prod = tq.tq_codec_init_prod(128, 4, 42)
    E = tq.TQ_ERR_INVALID_ARG
    assert _cache_init(None, vc, _cache_desc())[0] == E
    assert _cache_init(kc, vc, None)[0] == E
    assert _cache_init(kc, other, _cache_desc())[0] == E                    # dims differ
    assert _cache_init(prod, vc, _cache_desc())[0] == E                     # Prod keys
    for bad in (dict(batch=0), dict(n_kv_heads=-1), dict(max_ctx=0), dict(group_size=0),
                dict(group_size=4097), dict(pending_k=None), dict(packed_len=None),
                dict(k_codes=FAKE + 4), dict(pending_v=FAKE + 8), dict(pending_len=FAKE + 2)):
        st, _ = _cache_init(kc, vc, _cache_desc(**bad))
        assert st == E, bad
    assert tq._lib.tq_cache_init(kc.handle, vc.handle, ctypes.byref(_cache_desc()), None) == E

    st, h = _cache_init(kc, vc, _cache_desc(max_ctx=200, group_size=64))
    assert st == tq.TQ_OK and h.value
    cache = tq.Cache(h.value, kc, vc, ())
    assert tq.tq_cache_state(cache) == (0, 0)
    assert tq.tq_cache_workspace_bytes(cache, 4) == tq.tq_attend_workspace_bytes(2, 4, 2, 128, 200)
    app = tq._lib.tq_cache_append
    assert app(h, FAKE, FAKE, 0, None) == tq.TQ_OK                        # nothing to append
    assert app(h, FAKE, FAKE, -1, None) == E
    assert app(h, None, FAKE, 1, None) == E
    assert app(h, FAKE + 8, FAKE, 1, None) == E                           # alignment
    # 256 rows make four groups of 64: 256 packed rows > max_ctx 200
    assert app(h, FAKE, FAKE, 256, None) == E
    assert "max_ctx" in tq.tq_last_error()
    assert tq.tq_cache_state(cache) == (0, 0)                             # nothing changed
    assert app(None, FAKE, FAKE, 1, None) == E
    cache.close()
