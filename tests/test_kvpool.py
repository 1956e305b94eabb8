"""The library's host block pool (sv_kv_pool) against the oracle's free list,
and the attention entry points' host-side argument checks.  No GPU needed."""
import os

import numpy as np
import pytest

import speculative_decoding_verification_step_amd as sv
from oracle import attention as oa


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIB_PATH):
        pytest.skip("libspecverify.so not built")
    return sv.lib()


def test_pool_matches_oracle_free_list(lib):
    g = np.random.default_rng(0)
    nb, B, mb = 40, 5, 12
    pool, ref = sv.KVPool(nb), oa.BlockPool(nb)
    rows = np.zeros((B, mb), np.int32)
    n = [0] * B
    ref_rows = [[] for _ in range(B)]
    for _ in range(500):
        b = int(g.integers(B))
        tokens = int(g.integers(0, mb * 32 + 1))
        if g.random() < 0.5:
            try:
                ref.reserve(ref_rows[b], tokens, 32, mb)
                ok = True
            except MemoryError:
                ok = False
            if ok:
                n[b] = pool.reserve(rows[b], n[b], tokens)
            else:
                with pytest.raises(sv.SpecVerifyError) as e:
                    pool.reserve(rows[b], n[b], tokens)
                assert e.value.code == sv.SV_ERR_WORKSPACE
        else:
            ref.trim(ref_rows[b], tokens, 32)
            n[b] = pool.trim(rows[b], n[b], tokens)
        assert rows[b, :n[b]].tolist() == ref_rows[b]
        assert pool.free_blocks == len(ref.free)


def test_pool_rejects(lib):
    with pytest.raises(sv.SpecVerifyError):
        sv.KVPool(0)
    pool = sv.KVPool(4)
    row = np.zeros(2, np.int32)
    with pytest.raises(sv.SpecVerifyError):
        pool.reserve(row, 0, -1)
    with pytest.raises(sv.SpecVerifyError):
        pool.reserve(row, 0, 65)          # needs 3 blocks, the row holds 2


def test_attention_host_checks(lib):
    L = lib
    assert L.spec_verify_attention_workspace_bytes(2, 5, 32, 8, 128, 1) == 0     # one split
    assert L.spec_verify_attention_workspace_bytes(2, 5, 32, 8, 128, 256) > 0
    assert L.spec_verify_attention_workspace_bytes(2, 5, 30, 8, 128, 4) == 0     # Hq % Hkv
    F = 0x10000
    args = dict(q=F, kc=F, vc=F, tab=F, ctx=F, B=1, T=1, Hq=8, Hkv=8, Dh=128, mb=4, nb=4,
                scale=0.1, out=F, ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return L.spec_verify_attention(a["q"], a["kc"], a["vc"], a["tab"], a["ctx"], a["B"], a["T"],
                                       a["Hq"], a["Hkv"], a["Dh"], a["mb"], a["nb"], a["scale"],
                                       a["out"], a["ws"], a["wsb"], None)
    assert call(Dh=96) == sv.SV_ERR_UNSUPPORTED
    assert call(Hq=12) == sv.SV_ERR_INVALID_ARG
    assert call(T=0) == sv.SV_ERR_INVALID_ARG
    assert call(q=None) == sv.SV_ERR_INVALID_ARG
    assert call(scale=float("inf")) == sv.SV_ERR_INVALID_ARG
    assert call(mb=1024) == sv.SV_ERR_WORKSPACE           # split context needs a workspace
    assert call(B=0, q=None) == sv.SV_OK                    # empty batch: nothing enqueued
    assert L.spec_verify_kv_commit(None, None, 0, None) == sv.SV_OK
    assert L.spec_verify_kv_commit(None, F, 3, None) == sv.SV_ERR_INVALID_ARG
    assert L.spec_verify_kv_append(F, F, F, F, F, F, 1, 1, 8, 80, 4, 4, None) == sv.SV_ERR_UNSUPPORTED


def test_moe_host_checks(lib):
    L = lib
    d = sv.binding.MoEDesc(256, 128, 16, 4, 2, 100, 1e-5, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    import ctypes
    h = ctypes.c_void_p()
    assert L.sv_moe_create(ctypes.addressof(d), ctypes.byref(h)) == sv.SV_OK
    try:
        assert L.spec_verify_moe_workspace_bytes(h, 1025) == 0
        assert L.spec_verify_moe_forward(h, 0x10000, 1025, 0x10000, None, 0x10000, 1 << 30, None) \
            == sv.SV_ERR_UNSUPPORTED
        assert L.spec_verify_moe_forward(h, 0x10000, 8, 0x10000, None, 0x10000, 16, None) \
            == sv.SV_ERR_WORKSPACE
        assert L.spec_verify_moe_forward(h, None, 0, None, None, None, 0, None) == sv.SV_OK
    finally:
        L.sv_moe_destroy(h)
    for bad in (dict(top_k=9), dict(top_k=17), dict(d=100), dict(ffn=40), dict(n_experts=300)):
        kw = dict(d=256, ffn=128, n_experts=16, top_k=4)
        kw.update(bad)
        dd = sv.binding.MoEDesc(kw["d"], kw["ffn"], kw["n_experts"], kw["top_k"], 2, 100, 1e-5,
                                0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
        h2 = ctypes.c_void_p()
        assert L.sv_moe_create(ctypes.addressof(dd), ctypes.byref(h2)) != sv.SV_OK
