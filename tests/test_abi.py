"""The C-ABI library: it loads, exports every function include/engram.h
declares, and rejects bad host-visible arguments with the documented status
before launching anything (these calls never reach the GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from hashed_gram_embedding_amd import engram as eg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")

pytestmark = pytest.mark.skipif(not os.path.exists(eg.LIB_PATH), reason="libengram.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_[a-z0-9_]+)\s*\(", text)))


def exported_functions():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", eg.LIB_PATH], capture_output=True, text=True).stdout
    return sorted(set(m for m in re.findall(r" T (engram_\w+)", out)))


def test_exports_match_header():
    decl = declared_functions()
    assert len(decl) >= 11
    assert decl == exported_functions()
    assert sorted(eg.exported_names()) == decl
    L = eg.lib()
    for name in decl:
        assert hasattr(L, name)


def test_abi_version():
    assert eg.lib().engram_abi_version() == 6


def _hash_params(**over):
    proj = ctypes.c_void_p(0x1000)
    mult = np.ones((2, 2, 3), dtype=np.uint64)
    prime = np.array([1009, 1013, 1019, 1021], dtype=np.uint32)
    hp = eg.HashParams(proj, 1000, 3, 2, mult.ctypes.data, prime.ctypes.data)
    for k, v in over.items():
        setattr(hp, k, v)
    return hp, (mult, prime)


def _status(fn, *args):
    st = fn(*args)
    return st, eg.last_error()


def test_hash_rejects_bad_arguments():
    L = eg.lib()
    tok = ctypes.c_void_p(0x2000)
    z = ctypes.c_void_p(0x3000)
    hp, keep = _hash_params()
    assert L.engram_hash_indices(tok, 0, 5, None, ctypes.byref(hp), z, None) == eg.OK   # empty: no-op
    st, msg = _status(L.engram_hash_indices, None, 1, 5, None, ctypes.byref(hp), z, None)
    assert st == eg.EINVAL and "tokens" in msg
    st, _ = _status(L.engram_hash_indices, tok, -1, 5, None, ctypes.byref(hp), z, None)
    assert st == eg.EINVAL
    bad, keep2 = _hash_params(max_n=5)
    st, msg = _status(L.engram_hash_indices, tok, 1, 5, None, ctypes.byref(bad), z, None)
    assert st == eg.EUNSUPPORTED and "max_n" in msg
    bad, keep3 = _hash_params(heads=17)
    assert L.engram_hash_indices(tok, 1, 5, None, ctypes.byref(bad), z, None) == eg.EUNSUPPORTED
    prime0 = np.array([1, 1013, 1019, 1021], dtype=np.uint32)
    bad, keep4 = _hash_params(prime=prime0.ctypes.data)
    st, msg = _status(L.engram_hash_indices, tok, 1, 5, None, ctypes.byref(bad), z, None)
    assert st == eg.EINVAL and "prime" in msg
    assert L.engram_hash_indices(tok, 1, 5, None, None, z, None) == eg.EINVAL


def _tables(**over):
    off = np.array([0, 1009, 2022, 3041], dtype=np.int64)
    n = np.array([1009, 1013, 1019, 1021], dtype=np.int64)
    t = eg.Tables(4, 16, eg.F32, 0x10000, off.ctypes.data, n.ctypes.data, 4062, None, None, None, None, 0)
    for k, v in over.items():
        setattr(t, k, v)
    return t, (off, n)


def test_gather_rejects_bad_arguments():
    L = eg.lib()
    z, e = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    t, keep = _tables()
    assert L.engram_gather(z, 0, ctypes.byref(t), eg.F32, e, None) == eg.OK
    assert L.engram_gather(z, 4, ctypes.byref(t), eg.I8, e, None) == eg.EUNSUPPORTED   # out dtype
    t2, k2 = _tables(dim=12)
    assert L.engram_gather(z, 4, ctypes.byref(t2), eg.F32, e, None) == eg.EUNSUPPORTED
    t3, k3 = _tables(total_rows=4000)
    st, msg = _status(L.engram_gather, z, 4, ctypes.byref(t3), eg.F32, e, None)
    assert st == eg.EINVAL and "table 3" in msg
    t4, k4 = _tables(dtype=eg.I8)
    st, msg = _status(L.engram_gather, z, 4, ctypes.byref(t4), eg.BF16, e, None)
    assert st == eg.EINVAL and "row_scale" in msg
    t5, k5 = _tables(rows=0x10008)
    assert L.engram_gather(z, 4, ctypes.byref(t5), eg.F32, e, None) == eg.EINVAL      # misaligned
    t6, k6 = _tables(cache_slot=0x5000)
    st, msg = _status(L.engram_gather, z, 4, ctypes.byref(t6), eg.F32, e, None)
    assert st == eg.EINVAL and "cache" in msg
    assert L.engram_gather(None, 4, ctypes.byref(t), eg.F32, e, None) == eg.EINVAL


def test_project_rejects_bad_arguments():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    assert L.engram_project_kv(p, p, 8, 96, 128, eg.BF16, p, None) == eg.EUNSUPPORTED
    assert L.engram_project_kv(p, p, 8, 128, 100, eg.BF16, p, None) == eg.EUNSUPPORTED
    assert L.engram_project_kv(p, p, 8, 128, 128, eg.I8, p, None) == eg.EUNSUPPORTED
    assert L.engram_project_kv(p, p, 0, 128, 128, eg.BF16, p, None) == eg.OK
    assert L.engram_project_kv(None, p, 8, 128, 128, eg.BF16, p, None) == eg.EINVAL


def _gc(**over):
    g = eg.GateConvParams(1024, 1, 4, 3, 1e-6, eg.BF16, 0x10000)
    for k, v in over.items():
        setattr(g, k, v)
    return g


def test_gate_conv_rejects_bad_arguments_and_small_workspace():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    g = _gc()
    need = L.engram_gate_conv_workspace(2, 10, ctypes.byref(g))
    assert need >= 2 * 2 * 10 * 4
    st, msg = _status(L.engram_gate_conv_forward, p, p, 2, 10, ctypes.byref(g), None, None, None, p, need - 1, None)
    assert st == eg.EINVAL and "workspace" in msg
    for bad in (_gc(d=1000), _gc(kernel_w=1), _gc(kernel_w=9), _gc(dilation=11), _gc(hdtype=eg.I8)):
        assert L.engram_gate_conv_forward(p, p, 2, 10, ctypes.byref(bad), None, None, None, p, need, None) \
            == eg.EUNSUPPORTED
    assert L.engram_gate_conv_forward(p, p, 2, 10, ctypes.byref(_gc(conv_w=None)), None, None, None, p, need,
                                      None) == eg.EINVAL
    st_bad = eg.DecodeStateStruct(0x10000, None, 0x20000)
    assert L.engram_gate_conv_forward(p, p, 2, 10, ctypes.byref(g), ctypes.byref(st_bad), None, None, p, need,
                                      None) == eg.EINVAL


def test_forward_checks_layer_consistency():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=64, hdtype=eg.F32))
    need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
    assert need > 0
    st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need - 256, None)
    assert st == eg.EINVAL and "workspace" in msg
    n_bad = np.array([1009, 1013, 1019, 1000], dtype=np.int64)
    t_bad, _ = _tables(n_rows=n_bad.ctypes.data)
    lay2 = eg.LayerStruct(hp, t_bad, 0x10000, _gc(d=64, hdtype=eg.F32))
    st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay2), None, None, None, p, need, None)
    assert st == eg.EINVAL and "prime" in msg
    t3, _k = _tables(n_tables=3)
    lay3 = eg.LayerStruct(hp, t3, 0x10000, _gc(d=64, hdtype=eg.F32))
    assert L.engram_forward(p, p, 1, 64, ctypes.byref(lay3), None, None, None, p, need, None) == eg.EINVAL
    assert L.engram_forward(p, p, 0, 64, ctypes.byref(lay), None, None, None, None, 0, None) == eg.OK


def test_cache_build_rejects_bad_arguments():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    need = L.engram_cache_build_workspace(4062)
    assert need >= 2 * 4062 * 4
    st, msg = _status(L.engram_cache_build, p, 1, 8, ctypes.byref(hp), ctypes.byref(t), 5000, p, p, None, p, need, None)
    assert st == eg.EINVAL and "cache_n" in msg
    st, msg = _status(L.engram_cache_build, p, 1, 8, ctypes.byref(hp), ctypes.byref(t), 10, p, p, None, p, need - 1,
                      None)
    assert st == eg.EINVAL and "workspace" in msg
    assert L.engram_cache_build(p, 1, 8, ctypes.byref(hp), ctypes.byref(t), 10, None, p, None, p, need, None) \
        == eg.EINVAL
    t8, k8 = _tables(dtype=eg.I8, row_scale=0x20000)
    st, msg = _status(L.engram_cache_build, p, 1, 8, ctypes.byref(hp), ctypes.byref(t8), 10, p, p, None, p, need,
                      None)
    assert st == eg.EINVAL and "cache_scale" in msg
    assert L.engram_cache_build(p, 1, 8, ctypes.byref(hp), None, 10, p, p, None, p, need, None) == eg.EINVAL


def test_host_alloc_rejects_zero_bytes():
    L = eg.lib()
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    assert L.engram_host_alloc(0, ctypes.byref(h), ctypes.byref(d)) == eg.EINVAL
    assert L.engram_host_free(None) == eg.OK


def test_size_limits_are_rejected_before_launch():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    g = _gc()
    need = L.engram_gate_conv_workspace(2, 10, ctypes.byref(g))
    for bad in (_gc(d=eg.MAX_D + 64), _gc(branches=eg.MAX_BRANCHES + 1)):
        assert L.engram_gate_conv_forward(p, p, 2, 10, ctypes.byref(bad), None, None, None, p, need, None) \
            == eg.EUNSUPPORTED
    st, msg = _status(L.engram_gate_conv_forward, p, p, 1, 2 ** 31, ctypes.byref(g), None, None, None, p, need, None)
    assert st == eg.EUNSUPPORTED and "T above" in msg
    st, msg = _status(L.engram_gate_conv_forward, p, p, 65536, 1, ctypes.byref(g), None, None, None, p, need, None)
    assert st == eg.EUNSUPPORTED and "B above" in msg
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=64, hdtype=eg.F32))
    need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
    st, msg = _status(L.engram_forward, p, p, 65536, 1, ctypes.byref(lay), None, None, None, p, need, None)
    assert st == eg.EUNSUPPORTED and "B above" in msg
    # 2 x 2^30 tokens: B and T are each within their limits, but the hashed gather's 2^31
    # tokens per call is not (refused before any launch; the workspace size is only claimed)
    big = L.engram_forward_workspace(2, 2 ** 30, ctypes.byref(lay))
    st, msg = _status(L.engram_forward, p, p, 2, 2 ** 30, ctypes.byref(lay), None, None, None, p, big, None)
    assert st == eg.EUNSUPPORTED and "2^31" in msg
    st, msg = _status(L.engram_retrieve, p, 2, 2 ** 30, ctypes.byref(lay), None, p, None)
    assert st == eg.EUNSUPPORTED and "2^31" in msg


def test_retrieve_and_forward_retrieved_reject_bad_arguments():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=64, hdtype=eg.F32))
    assert L.engram_retrieve(p, 0, 5, ctypes.byref(lay), None, None, None) == eg.OK      # empty: no-op
    st, msg = _status(L.engram_retrieve, p, 1, 5, ctypes.byref(lay), None, None, None)
    assert st == eg.EINVAL and "e must" in msg
    assert L.engram_retrieve(p, 1, 5, ctypes.byref(lay), None, ctypes.c_void_p(0x10008), None) == eg.EINVAL
    assert L.engram_retrieve(p, 1, 5, None, None, p, None) == eg.EINVAL
    need = L.engram_forward_retrieved_workspace(1, 64, ctypes.byref(lay))
    assert 0 < need < L.engram_forward_workspace(1, 64, ctypes.byref(lay))
    st, msg = _status(L.engram_forward_retrieved, p, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need - 256,
                      None)
    assert st == eg.EINVAL and "workspace" in msg
    st, msg = _status(L.engram_forward_retrieved, p, None, p, 1, 64, ctypes.byref(lay), None, None, None, p, need,
                      None)
    assert st == eg.EINVAL and "e and H" in msg
    sd = eg.DecodeStateStruct(0x20000, 0x30000, 0x40000)
    st, msg = _status(L.engram_forward_retrieved, None, p, p, 1, 64, ctypes.byref(lay), ctypes.byref(sd), None, None,
                      p, need, None)
    assert st == eg.EINVAL and "tokens" in msg


def test_cache_update_rejects_bad_arguments():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    t, keep_t = _tables()
    need = L.engram_cache_update_workspace(4062, 100)
    assert need > 0 and L.engram_cache_update_workspace(4062, 5000) == 0
    # (a valid call would launch: only the rejected ones run here)
    st, msg = _status(L.engram_cache_update, ctypes.byref(t), 100, p, p, None, None, 0, p, need, None)
    assert st == eg.EINVAL and "counts" in msg
    st, msg = _status(L.engram_cache_update, ctypes.byref(t), 100, p, p, None, p, 32, p, need, None)
    assert st == eg.EINVAL and "decay_shift" in msg
    st, msg = _status(L.engram_cache_update, ctypes.byref(t), 100, p, p, None, p, 1, p, need - 1, None)
    assert st == eg.EINVAL and "workspace" in msg
    st, msg = _status(L.engram_cache_update, ctypes.byref(t), 5000, p, p, None, p, 1, p, need, None)
    assert st == eg.EINVAL and "cache_n" in msg
    t8, k8 = _tables(dtype=eg.I8, row_scale=0x20000)
    st, msg = _status(L.engram_cache_update, ctypes.byref(t8), 100, p, p, None, p, 1, p, need, None)
    assert st == eg.EINVAL and "cache_scale" in msg
    tc, kc = _tables(access_counts=0x10002)
    st, msg = _status(L.engram_gather, p, 4, ctypes.byref(tc), eg.F32, p, None)
    assert st == eg.EINVAL and "access_counts" in msg


def test_hot_tier_is_validated_before_launch():
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    hot = eg.HotTierStruct()
    hot.n_hot[0] = 10
    hot.pilots[0], hot.slots[0], hot.rows[0] = 0x20000, 0x30000, 0x40000
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=64, hdtype=eg.F32))
    lay.hot = ctypes.pointer(hot)
    need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
    z = ctypes.c_void_p(0x50000)
    # a well-formed tier passes every check (empty call)
    assert L.engram_forward(p, p, 0, 64, ctypes.byref(lay), None, None, None, None, 0, None) == eg.OK
    assert L.engram_hot_lookup(p, 0, 64, None, ctypes.byref(hp), ctypes.byref(hot), z, None) == eg.OK
    cases = [
        (("slots", 0, 0x30010), eg.EINVAL, "aligned"),     # slots not 32-byte aligned
        (("rows", 0, 0x40008), eg.EINVAL, "aligned"),
        (("pilots", 0, None), eg.EINVAL, "pilots"),
        (("n_hot", 0, -1), eg.EINVAL, "n_hot"),
        (("n_hot", 2, 5), eg.EINVAL, "max_n"),             # order 4 beyond max_n = 3
    ]
    for (field, o, v), status, text in cases:
        bad = eg.HotTierStruct()
        ctypes.pointer(bad)[0] = hot
        getattr(bad, field)[o] = v
        if field == "n_hot" and o == 2:
            bad.pilots[2], bad.slots[2], bad.rows[2] = 0x20000, 0x30000, 0x40000
        lay.hot = ctypes.pointer(bad)
        st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need, None)
        assert st == status and text in msg, (field, msg)
        st, msg = _status(L.engram_retrieve, p, 1, 64, ctypes.byref(lay), None, p, None)
        assert st == status and text in msg, (field, msg)
    # int8 tables have no hot tier
    t8, keep_8 = _tables(dtype=eg.I8, row_scale=0x60000)
    lay8 = eg.LayerStruct(hp, t8, 0x10000, _gc(d=64, hdtype=eg.F32))
    lay8.hot = ctypes.pointer(hot)
    st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay8), None, None, None, p, need, None)
    assert st == eg.EUNSUPPORTED and "hot" in msg
    # the lookup alone needs no rows, but a tier and output
    nor = eg.HotTierStruct()
    ctypes.pointer(nor)[0] = hot
    nor.rows[0] = None
    assert L.engram_hot_lookup(p, 1, 64, None, ctypes.byref(hp), ctypes.byref(nor), None, None) == eg.EINVAL
    assert L.engram_hot_lookup(p, 1, 64, None, ctypes.byref(hp), None, z, None) == eg.EINVAL


def test_mxfp8_layer_outside_the_fused_projection_is_rejected():
    """MXFP8 rows are read only by the fused projection (d <= 4096): a wider
    MXFP8 layer is refused before anything launches."""
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables(dtype=eg.BF16, dim=32)       # d_mem = 4 x 32 = 128
    for d, want in ((4096 + 128, eg.EUNSUPPORTED), (4096 * 2, eg.EUNSUPPORTED)):
        lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=d), 0x20000, 0x30000)
        need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
        st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need, None)
        assert st == want and "MXFP8" in msg
        assert L.engram_retrieve(p, 1, 64, ctypes.byref(lay), None, p, None) == want
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=4096), 0x20000, 0x30000)
    assert L.engram_retrieve(p, 0, 64, ctypes.byref(lay), None, p, None) == eg.OK     # d = 4096 passes the checks


def test_packed_mxfp8_weights_are_checked():
    """engram_pack_mxfp8 takes whole 32-row blocks and 256-column step
    groups, and a layer's packed W needs its MXFP8 W and 16-byte alignment;
    all refused before anything launches."""
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    for rows, cols in ((33, 256), (32, 128), (-32, 256), (64, 300)):
        st, msg = _status(L.engram_pack_mxfp8, p, p, rows, cols, p, None)
        assert st == eg.EINVAL and "pack_mxfp8" in msg, (rows, cols)
    assert L.engram_pack_mxfp8(None, None, 0, 256, None, None) == eg.OK          # empty: a no-op
    st, msg = _status(L.engram_pack_mxfp8, None, p, 32, 256, p, None)
    assert st == eg.EINVAL and "non-NULL" in msg
    st, msg = _status(L.engram_pack_mxfp8, ctypes.c_void_p(0x10008), p, 32, 256, p, None)
    assert st == eg.EINVAL and "aligned" in msg
    hp, keep_h = _hash_params()
    t, keep_t = _tables(dtype=eg.BF16, dim=32)
    for w_mx, packed, text in ((None, 0x40000, "needs w_mx"), (0x20000, 0x40008, "aligned")):
        lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=256), w_mx, 0x30000 if w_mx else None, packed)
        need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
        st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need, None)
        assert st == eg.EINVAL and text in msg, msg


def test_packed_bf16_weights_are_checked():
    """engram_pack_bf16 takes whole 32-row blocks and 16-column steps, and a
    layer's packed bf16 W needs a bf16 layer and 16-byte alignment; all
    refused before anything launches."""
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    for rows, cols in ((33, 64), (32, 24), (-32, 64), (64, -16)):
        st, msg = _status(L.engram_pack_bf16, p, rows, cols, p, None)
        assert st == eg.EINVAL and "pack_bf16" in msg, (rows, cols)
    assert L.engram_pack_bf16(None, 0, 64, None, None) == eg.OK          # empty: a no-op
    st, msg = _status(L.engram_pack_bf16, None, 32, 64, p, None)
    assert st == eg.EINVAL and "non-NULL" in msg
    st, msg = _status(L.engram_pack_bf16, p, 32, 64, ctypes.c_void_p(0x10008), None)
    assert st == eg.EINVAL and "aligned" in msg
    hp, keep_h = _hash_params()
    t, keep_t = _tables(dtype=eg.BF16, dim=32)
    for hdtype, packed, text in ((eg.F32, 0x40000, "bf16 layer"), (eg.BF16, 0x40008, "aligned")):
        lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=256, hdtype=hdtype), None, None, None, packed)
        need = L.engram_forward_workspace(1, 64, ctypes.byref(lay))
        st, msg = _status(L.engram_forward, p, p, 1, 64, ctypes.byref(lay), None, None, None, p, need, None)
        assert st == eg.EINVAL and text in msg and "w_packed" in msg, msg


def test_forward_noalloc_rejects_calls_beyond_its_scratch():
    """engram_forward_noalloc checks every host-visible argument, and that the
    call fits the library's fixed scratch, before it touches any device."""
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables()
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=64, hdtype=eg.F32))
    per_tok = L.engram_forward_workspace(1, 1024, ctypes.byref(lay)) / 1024
    T_big = int(eg.NOALLOC_SCRATCH_BYTES / per_tok) + 1024
    assert L.engram_forward_workspace(1, T_big, ctypes.byref(lay)) > eg.NOALLOC_SCRATCH_BYTES
    st, msg = _status(L.engram_forward_noalloc, p, p, 1, T_big, ctypes.byref(lay), None, None, None, None)
    assert st == eg.EINVAL and "scratch" in msg
    assert L.engram_forward_noalloc(p, p, 0, 64, ctypes.byref(lay), None, None, None, None) == eg.OK   # empty
    assert L.engram_forward_noalloc(p, p, 1, 64, None, None, None, None, None) == eg.EINVAL
    st_bad = eg.DecodeStateStruct(None, 0x20000, 0x30000)
    assert L.engram_forward_noalloc(p, p, 1, 64, ctypes.byref(lay), ctypes.byref(st_bad), None, None, None) \
        == eg.EINVAL
    text = open(HEADER).read()
    assert f"#define ENGRAM_NOALLOC_SCRATCH_BYTES (32u << 20)" in text and eg.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_profile_modes_are_checked():
    """engram_profile_enable accepts modes 0, 1 and 2 only; reading with
    profiling off, or before any profiled call, is an error (no GPU work)."""
    L = eg.lib()
    st, msg = _status(L.engram_profile_enable, 3)
    assert st == eg.EINVAL and "mode" in msg
    assert L.engram_profile_enable(-1) == eg.EINVAL
    assert L.engram_profile_enable(0) == eg.OK
    ms = (ctypes.c_float * 4)()
    n = ctypes.c_int32(7)
    st, msg = _status(L.engram_profile_read, ms, None, 4, ctypes.byref(n))
    assert st == eg.EINVAL and n.value == 0
    assert L.engram_profile_read(ms, None, 4, None) == eg.EINVAL


def test_project_ahead_and_forward_projected_are_checked():
    """engram_project_ahead takes 1..ENGRAM_MAX_AHEAD_LAYERS fused bf16 layers,
    a state for every layer or none, and T = 1 with states;
    engram_forward_projected takes a state only for T = 1; all refused before
    anything launches."""
    L = eg.lib()
    p = ctypes.c_void_p(0x10000)
    hp, keep_h = _hash_params()
    t, keep_t = _tables(dtype=eg.BF16, dim=32)
    lay = eg.LayerStruct(hp, t, 0x10000, _gc(d=256))
    arr = (ctypes.POINTER(eg.LayerStruct) * 2)(ctypes.pointer(lay), ctypes.pointer(lay))
    kv = (ctypes.c_void_p * 2)(0x20000, 0x30000)
    need = L.engram_project_ahead_workspace(1, 1, 2, arr)
    assert need > 0
    for n in (0, 9):
        st, msg = _status(L.engram_project_ahead, p, 1, 1, n, arr, None, kv, p, need, None)
        assert st == eg.EINVAL and "n_layers" in msg
    st, msg = _status(L.engram_project_ahead, p, 1, 1, 2, None, None, kv, p, need, None)
    assert st == eg.EINVAL and "non-NULL" in msg
    ids = ctypes.c_void_p(0x40000)
    ds = eg.DecodeStateStruct(ids, 0x50000, 0x60000)
    sts = (ctypes.POINTER(eg.DecodeStateStruct) * 2)(ctypes.pointer(ds), None)
    st, msg = _status(L.engram_project_ahead, p, 1, 1, 2, arr, sts, kv, p, need, None)
    assert st == eg.EINVAL and "every layer or none" in msg
    sts[1] = ctypes.pointer(ds)
    st, msg = _status(L.engram_project_ahead, p, 1, 2, 2, arr, sts, kv, p, need, None)
    assert st == eg.EUNSUPPORTED and "T must be 1" in msg
    f32 = eg.LayerStruct(hp, t, 0x10000, _gc(d=256, hdtype=eg.F32))
    arr_f = (ctypes.POINTER(eg.LayerStruct) * 1)(ctypes.pointer(f32))
    st, msg = _status(L.engram_project_ahead, p, 1, 1, 1, arr_f, None, kv, p, need, None)
    assert st == eg.EUNSUPPORTED and "bf16 H" in msg
    st, msg = _status(L.engram_project_ahead, p, 1, 1, 2, arr, None, kv, p, 0, None)
    assert st == eg.EINVAL and "workspace" in msg
    assert L.engram_project_ahead(p, 0, 1, 2, arr, None, kv, None, 0, None) == eg.OK     # no tokens: a no-op
    need_f = L.engram_forward_projected_workspace(1, 2, ctypes.byref(lay))
    st, msg = _status(L.engram_forward_projected, p, p, 1, 2, ctypes.byref(lay), ctypes.byref(ds), None, None, p,
                      need_f, None)
    assert st == eg.EUNSUPPORTED and "decode state" in msg
    st, msg = _status(L.engram_forward_projected, p, p, 1, 2, ctypes.byref(lay), None, None, None, p, 0, None)
    assert st == eg.EINVAL and "workspace" in msg
