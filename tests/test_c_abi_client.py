"""The library from plain C: tests/c_abi_client.c (hipMalloc, tq_codec_init,
tq_encode, tq_decode_attend through include/tq.h, no Python and no torch in
that process) on seeded inputs, its outputs checked against the oracle."""
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import workloads
from conftest import ROOT

CLIENT = os.path.join(ROOT, "tests", "_build", "c_abi_client")


def test_c_client_built_and_linked():
    """Built by __graft_entry__.build(); without arguments it prints its usage
    and exits 2 before any HIP call."""
    assert os.path.exists(CLIENT), "run __graft_entry__.build() first"
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("d,kb,vb,G,lengths", [(128, 4, 2, 3, [700, 333]), (64, 8, 3, 4, [1500])])
def test_c_client_matches_oracle(d, kb, vb, G, lengths):
    print(f"[gpu-case] C ABI client d={d} kb={kb} vb={vb} G={G} lengths={lengths}", flush=True)
    Hkv = 2
    B, Hq = len(lengths), G * Hkv
    T = max(lengths)
    lens, k, v, q = workloads.small_case(31 + d, B, Hq, Hkv, d, T, lengths)
    seed = 42
    with tempfile.TemporaryDirectory() as tmp:
        fin, fout = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
        with open(fin, "wb") as f:
            f.write(struct.pack("<7iQ", B, Hq, Hkv, d, T, kb, vb, seed))
            f.write(np.ascontiguousarray(lens, dtype="<i4").tobytes())
            for a in (k, v, q):
                f.write(np.ascontiguousarray(a, dtype="<f2").tobytes())
        r = subprocess.run([CLIENT, fin, fout], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        raw = open(fout, "rb").read()
    kr, vr = d * kb // 8, d * vb // 8
    n = B * Hkv * T
    off = 0

    def take(count, dtype):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    kc = take(n * kr, np.uint8).reshape(B, Hkv, T, kr)
    kn = take(n, "<f4").reshape(B, Hkv, T)
    vc = take(n * vr, np.uint8).reshape(B, Hkv, T, vr)
    vn = take(n, "<f4").reshape(B, Hkv, T)
    out = take(B * Hq * d, "<f4").reshape(B, Hq, d)
    assert off == len(raw)
    ok, ov = oracle.Codec(d, kb, seed), oracle.Codec(d, vb, seed)
    okc, okn, _ = oracle.encode(ok, k)
    ovc, ovn, _ = oracle.encode(ov, v)
    assert kc.tobytes() == okc.tobytes() and vc.tobytes() == ovc.tobytes()
    assert kn.tobytes() == okn.tobytes() and vn.tobytes() == ovn.tobytes()
    want = oracle.attend(ok, ov, q, okc, okn, ovc, ovn, lens)
    assert np.max(np.abs(out - want)) <= 2e-3
