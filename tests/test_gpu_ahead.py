"""GPU: Steps 1-5 of several layers ahead of their hidden states
(engram_project_ahead), then each layer's Steps 6-8 on the float32
projections (engram_forward_projected).  Every layer matches the oracle at
the bf16 tolerances, carrying the decode state through single-token steps;
the launches are the ones the header promises (two for a pair of layers,
one conv per layer in decode)."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def stages(fn):
    eg.profile_enable(True)
    try:
        fn()
        return [n for n, _ in eg.profile_read()]
    finally:
        eg.profile_enable(False)


def test_pack_bf16_layout():
    """engram_pack_bf16: 32-row blocks, 16-column steps, 64 lane slots of 8
    values (lane 32h + r of step s: row 32b + r, columns 32(s/2) + 16h +
    8(s%2) .. +7), bit for bit."""
    rows, cols = 96, 96
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    w = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    packed = torch.empty_like(w)
    eg.pack_bf16(w, packed)
    got = packed.view(torch.int16).cpu().numpy().view(np.uint16).reshape(rows // 32, cols // 16, 2, 32, 8)
    for b in range(rows // 32):
        for s in range(cols // 16):
            for h in range(2):
                c0 = 32 * (s // 2) + 16 * h + 8 * (s % 2)
                assert np.array_equal(got[b, s, h], bits[32 * b:32 * b + 32, c0:c0 + 8]), (b, s, h)


GATHER_THEN_PRODUCT = ["gather2_kernel", "proj_kv_kernel"]
FUSED = ["gather_proj_kernel"]

# (name, config, overrides, bf16 W packed, launches): the float32 products of
# engram_project_ahead against the exact product of the same bf16 operands,
# at K = 1024, 768, 512 and 256 and ragged token counts: with W in fragment
# order, Steps 1-5 in one launch (int8 rows, and bf16 rows of the
# single-branch workload); the fragment-operand product after the gather
# (table dims not a multiple of 32); and the LDS-staged product.
KV_CASES = [
    ("K1024 fused", 3, dict(B=3, T=37), True, FUSED),
    ("K1024 fused 64-token tiles", 3, dict(B=3, T=100), True, FUSED),
    ("K512 fused 64-token tiles", 3, dict(B=2, T=200, table_dim=32), True, FUSED),
    ("K1024 dim 32 fused", 3, dict(B=2, T=45, table_dim=32, heads=16), True, FUSED),
    ("K1024 dim 32 fused 64-token tiles", 3, dict(B=2, T=200, table_dim=32, heads=16), True, FUSED),
    ("K1024 dim 128 fused", 3, dict(B=2, T=45, table_dim=128, heads=4), True, FUSED),
    ("K512 dim 128 fused 64-token tiles", 3, dict(B=2, T=200, table_dim=128, heads=2), True, FUSED),
    ("K1024 lds", 3, dict(B=3, T=37), False, GATHER_THEN_PRODUCT),
    ("K768 frag", 3, dict(B=2, T=50, table_dim=48), True, GATHER_THEN_PRODUCT),
    ("K512 fused", 3, dict(B=2, T=45, table_dim=32), True, FUSED),
    ("K256 frag", 3, dict(B=1, T=70, table_dim=16, branches=2), True, GATHER_THEN_PRODUCT),
    ("bf16 rows fused", 1, dict(B=1, T=100), True, FUSED),
    ("bf16 rows M=4 fused", 2, dict(B=1, T=33), True, FUSED),
]


@pytest.mark.parametrize("name,cfg,kw,packed,want", KV_CASES, ids=[c[0] for c in KV_CASES])
def test_projections_ahead_against_exact_product(name, cfg, kw, packed, want):
    """Every element of kv within the float32 summation bound of the exact
    product: |kv - W e| <= (K + 2) 2^-24 (|W| |e|), per element."""
    log(f"kv ahead: {name}")
    if cfg == 3:
        w = inputs.make_config(3, rows_per_table=997, layers=2, **kw)
    else:
        w = inputs.make_config(cfg, rows_per_table=997, **kw)
    Ls = [eg.Layer(l, "bf16", DEV, bf16_packed=packed) for l in w.layers]
    assert all((L.w_packed is not None) == packed for L in Ls)
    tok = torch.from_numpy(w.tokens).to(DEV)
    names = stages(lambda: eg.project_ahead(tok, Ls))
    assert len(Ls) == 2 or want == FUSED
    assert names == want, names
    kv = eg.project_ahead(tok, Ls)
    torch.cuda.synchronize()
    for li, lay in enumerate(w.layers):
        ref = orc.forward(w.tokens, w.H, lay, "bf16")
        e = ref["e"].reshape(w.B * w.T, -1)
        wa = orc.storage_to_f64(lay.w, "bf16")
        K = e.shape[1]
        bound = (K + 2) * 2.0 ** -24 * (np.abs(e) @ np.abs(wa).T)
        got = kv[li].cpu().numpy().astype(np.float64)
        err = np.abs(got - ref["kv"].reshape(w.B * w.T, -1))
        assert np.all(err <= bound), (name, li, float(np.max(err - bound)))


@pytest.mark.parametrize("mx,packed,S", [(False, True, 256), (False, True, 64), (False, False, 256),
                                          (True, False, 256)],
                         ids=["bf16-fused", "bf16-fused-32-token-tiles", "bf16-lds", "mxfp8"])
def test_decode_two_layers_ahead(mx, packed, S):
    """S sequences with int8 tables: a 16-token prefill per layer through
    engram_forward, then 3 decode steps in which both layers' Steps 1-5 run
    in one launch (two with the LDS-staged or FP8 product) and each layer's
    gate, conv and residual in one; H flows from layer 0 into layer 1 and
    the states advance as in engram_forward.  (At 64 sequences the fused
    launch takes 32-token tiles.)"""
    log(f"decode ahead mx={mx} packed={packed} S={S}")
    w = inputs.make_config(3, B=S, T=3, rows_per_table=997)
    M, d = 1, 1024
    lays = w.layers
    Ls = [eg.Layer(l, "bf16", DEV, mxfp8=mx, bf16_packed=packed) for l in lays]
    sts = [eg.DecodeState(S, 3, M, 9, d, DEV) for _ in Ls]
    osts = [orc.new_state(S, 3, M, 9, d) for _ in Ls]
    gemm = "mxfp8" if mx else "exact"
    ctx = torch.from_numpy(w.context).to(DEV)
    for li, (L, lay) in enumerate(zip(Ls, lays)):
        Hc = eg.to_device(w.H_context, "bf16", DEV)
        eg.forward(ctx, Hc, L, state=sts[li])
        osts[li] = orc.forward(w.context, w.H_context, lay, "bf16", state=osts[li], gemm=gemm)["state"]
    for t in range(3):
        tok_np = np.ascontiguousarray(w.tokens[:, t:t + 1])
        tok = torch.from_numpy(tok_np).to(DEV)
        out = {}
        names = stages(lambda: out.setdefault("kv", eg.project_ahead(tok, Ls, states=sts)))
        assert names == (FUSED if packed else GATHER_THEN_PRODUCT), names
        Hn = np.ascontiguousarray(w.H[:, t:t + 1])
        H = eg.to_device(Hn, "bf16", DEV)
        for li, (L, lay) in enumerate(zip(Ls, lays)):
            h_in = H.view(torch.int16).cpu().numpy().view(np.uint16).copy()
            res = {}
            names = stages(lambda: res.setdefault("ay", eg.forward_projected(out["kv"][li], H, L, S, 1, state=sts[li],
                                                                              want_alpha=True, want_y=True)))
            assert names == ["conv_kernel"], names
            alpha, y = res["ay"]
            torch.cuda.synchronize()
            ref = orc.forward(tok_np, h_in, lay, "bf16", state=osts[li], gemm=gemm)
            osts[li] = ref["state"]
            check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(h_in),
                             tag=f"ahead step {t} layer {li}")
    for li in range(2):
        assert np.array_equal(sts[li].ids.cpu().numpy(), osts[li]["ids"])
        assert np.all(sts[li].pos.cpu().numpy() == 16 + 3)
        conv = sts[li].conv.cpu().numpy().astype(np.float64)
        chrono = np.stack([conv[:, :, (19 - 9 + i) % 9] for i in range(9)], axis=2)
        assert np.max(np.abs(chrono - osts[li]["u"])) <= 1e-2 * np.max(np.abs(osts[li]["u"]))


# Without a state: three four-branch layers (a pair in two launches, then one
# more); the FP8 product; and products above the small-batch range (the
# general product per layer).
CASES = [
    ("3 layers M=4", dict(B=2, T=40, layers=3, branches=4), False, ["gather_proj_kernel", "gather_proj_kernel"]),
    ("3 layers M=4 lds", dict(B=2, T=40, layers=3, branches=4), None, ["gather2_kernel", "proj_kv_kernel",
                                                                       "gather_kernel<hashed>", "proj_kv_kernel"]),
    ("one token M=2", dict(B=64, T=1, layers=2, branches=2), False, ["gather_proj_kernel"]),
    ("mxfp8 2 layers", dict(B=2, T=40, layers=2, branches=2), True, ["gather2_kernel", "proj_kv_kernel"]),
    ("general product", dict(B=1, T=1500, layers=2, branches=1), False, ["gather2_kernel", "gemm_kernel",
                                                                         "gemm_kernel"]),
]


@pytest.mark.parametrize("name,kw,mx,want", CASES, ids=[c[0] for c in CASES])
def test_layers_ahead_without_state(name, kw, mx, want):
    log(f"ahead without state: {name}")
    w = inputs.make_config(3, rows_per_table=997, **kw)
    B, T = w.B, w.T
    lays = w.layers
    # mx None: bf16 without the fragment-ordered W
    Ls = [eg.Layer(l, "bf16", DEV, mxfp8=bool(mx), bf16_packed=mx is not None) for l in lays]
    mx = bool(mx)
    tok = torch.from_numpy(w.tokens).to(DEV)
    out = {}
    names = stages(lambda: out.setdefault("kv", eg.project_ahead(tok, Ls)))
    assert names == want, names
    H = eg.to_device(w.H, "bf16", DEV)
    for li, (L, lay) in enumerate(zip(Ls, lays)):
        h_in = H.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        res = {}
        names = stages(lambda: res.setdefault("ay", eg.forward_projected(out["kv"][li], H, L, B, T, want_alpha=True,
                                                                          want_y=True)))
        assert names == (["conv_kernel"] if T == 1 else ["gate_stats_kernel", "conv_kernel"]), names
        alpha, y = res["ay"]
        torch.cuda.synchronize()
        ref = orc.forward(w.tokens, h_in, lay, "bf16", gemm="mxfp8" if mx else "exact")
        check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(h_in),
                         tag=f"{name} layer {li}")
