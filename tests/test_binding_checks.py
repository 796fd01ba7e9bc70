"""The binding refuses tensors of the wrong dtype or on the host before anything
is enqueued (CPU only: every call here must raise TQError in Python, before
the C entry point is reached)."""
import pytest
import torch

import compressed_domain_decode_amd as tq

B, HQ, HKV, D, T = 1, 4, 2, 64, 64


def _codecs():
    return tq.tq_codec_init(D, 4, 1), tq.tq_codec_init(D, 4, 1)


def _attend_args(kc, vc):
    return dict(
        q=torch.zeros((B, HQ, D), dtype=torch.float16),
        k_codes=torch.zeros((B, HKV, T, kc.row_bytes), dtype=torch.uint8),
        k_norms=torch.zeros((B, HKV, T), dtype=torch.float32),
        v_codes=torch.zeros((B, HKV, T, vc.row_bytes), dtype=torch.uint8),
        v_norms=torch.zeros((B, HKV, T), dtype=torch.float32),
        lengths=torch.full((B,), T, dtype=torch.int32),
        out=torch.zeros((B, HQ, D), dtype=torch.float32),
        workspace=torch.zeros(tq.tq_attend_workspace_bytes(B, HQ, HKV, D, T), dtype=torch.uint8),
    )


def _call_attend(fn_name, kc, vc, a):
    if fn_name == "tq_decode_attend":
        tq.tq_decode_attend(kc, vc, a["q"], a["k_codes"], a["k_norms"], a["v_codes"],
                            a["v_norms"], a["lengths"], T, 0.125, a["out"], a["workspace"])
    else:
        tq.tq_decode_attend_noalloc(kc, vc, a["q"], a["k_codes"], a["k_norms"], a["v_codes"],
                                    a["v_norms"], a["lengths"], T, 0.125, a["out"])


# a wrong dtype of the same element count where sizes allow, else a plain mismatch
WRONG = {
    "q": torch.bfloat16, "k_codes": torch.int8, "k_norms": torch.float16,
    "v_codes": torch.float32, "v_norms": torch.float64, "lengths": torch.int64,
    "out": torch.float16, "workspace": torch.int32,
}


@pytest.mark.parametrize("fn_name", ["tq_decode_attend", "tq_decode_attend_noalloc"])
@pytest.mark.parametrize("name", list(WRONG))
def test_attend_rejects_wrong_dtype(fn_name, name):
    if fn_name == "tq_decode_attend_noalloc" and name == "workspace":
        pytest.skip("the no-alloc call takes no workspace")
    kc, vc = _codecs()
    a = _attend_args(kc, vc)
    a[name] = a[name].to(WRONG[name])
    with pytest.raises(tq.TQError) as e:
        _call_attend(fn_name, kc, vc, a)
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    assert f"{name} must be" in str(e.value)


@pytest.mark.parametrize("fn_name", ["tq_decode_attend", "tq_decode_attend_noalloc"])
def test_attend_rejects_host_tensors(fn_name):
    kc, vc = _codecs()
    with pytest.raises(tq.TQError) as e:
        _call_attend(fn_name, kc, vc, _attend_args(kc, vc))
    assert "must be a GPU tensor" in str(e.value)


def test_multi_mixed_raw_prod_reject_wrong_dtype():
    kc, vc = _codecs()
    a = _attend_args(kc, vc)
    # multi-token: lengths int64
    with pytest.raises(tq.TQError, match="lengths must be"):
        tq.tq_decode_attend_multi(kc, vc, a["q"].reshape(B, 1, HQ, D), a["k_codes"],
                                  a["k_norms"], a["v_codes"], a["v_norms"],
                                  a["lengths"].long(), T, 0.125, a["out"].reshape(B, 1, HQ, D),
                                  a["workspace"])
    # mixed: raw rows in fp32
    raw = torch.zeros((B, HKV, 8, D), dtype=torch.float32)
    with pytest.raises(tq.TQError, match="raw_k must be"):
        tq.tq_decode_attend_mixed(kc, vc, a["q"], a["k_codes"], a["k_norms"], a["v_codes"],
                                  a["v_norms"], a["lengths"], T, raw, raw.half(),
                                  a["lengths"], 0.125, a["out"], a["workspace"])
    # raw keys: keys in fp32
    with pytest.raises(tq.TQError, match="k must be"):
        tq.tq_decode_attend_raw_k(vc, a["q"], torch.zeros((B, HKV, T, D)), a["v_codes"],
                                  a["v_norms"], a["lengths"], T, 0.125, a["out"],
                                  a["workspace"])
    # Prod keys: residual norms in fp16
    pk = tq.tq_codec_init_prod(D, 4, 1)
    with pytest.raises(tq.TQError, match="k_rnorms must be"):
        tq.tq_decode_attend_prod(
            pk, vc, a["q"], torch.zeros((B, HKV, T, pk.row_bytes), dtype=torch.uint8),
            torch.zeros((B, HKV, T, pk.sketch_bytes), dtype=torch.uint8), a["k_norms"],
            torch.zeros((B, HKV, T), dtype=torch.float16), a["v_codes"], a["v_norms"],
            a["lengths"], T, 0.125, a["out"], a["workspace"])


@pytest.mark.parametrize("name,wrong", [("x", torch.float32), ("codes", torch.int16),
                                        ("norms", torch.float16)])
def test_encode_rejects_wrong_dtype(name, wrong):
    c = tq.tq_codec_init(D, 4, 1)
    a = dict(x=torch.zeros((T, HKV, D), dtype=torch.float16),
             codes=torch.zeros((T, HKV, c.row_bytes), dtype=torch.uint8),
             norms=torch.zeros((T, HKV), dtype=torch.float32))
    a[name] = a[name].to(wrong)
    with pytest.raises(tq.TQError, match=f"{name} must be"):
        tq.tq_encode(c, a["x"], a["codes"], a["norms"])
    with pytest.raises(tq.TQError, match=f"{name} must be"):
        tq.tq_encode_kv(c, a["x"], a["codes"], a["norms"], c, a["x"], a["codes"], a["norms"])


def test_encode_rejects_host_tensors():
    c = tq.tq_codec_init(D, 4, 1)
    with pytest.raises(tq.TQError, match="must be a GPU tensor"):
        tq.tq_encode(c, torch.zeros((T, HKV, D), dtype=torch.float16),
                     torch.zeros((T, HKV, c.row_bytes), dtype=torch.uint8),
                     torch.zeros((T, HKV), dtype=torch.float32))


def test_cache_calls_reject_wrong_dtype():
    kc, vc = _codecs()
    G = 16
    bufs = dict(
        k_codes=torch.zeros((B, HKV, T, kc.row_bytes), dtype=torch.uint8),
        k_norms=torch.zeros((B, HKV, T), dtype=torch.float32),
        v_codes=torch.zeros((B, HKV, T, vc.row_bytes), dtype=torch.uint8),
        v_norms=torch.zeros((B, HKV, T), dtype=torch.float32),
        pending_k=torch.zeros((B, HKV, G, D), dtype=torch.float16),
        pending_v=torch.zeros((B, HKV, G, D), dtype=torch.float16),
        packed_len=torch.zeros((B,), dtype=torch.int32),
        pending_len=torch.zeros((B,), dtype=torch.int32),
    )
    bad = dict(bufs, pending_len=bufs["pending_len"].long())
    with pytest.raises(tq.TQError, match="pending_len must be"):
        tq.tq_cache_init(kc, vc, *bad.values())
    with pytest.raises(tq.TQError, match="must be a GPU tensor"):
        tq.tq_cache_init(kc, vc, *bufs.values())
