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


@pytest.mark.parametrize("mx", [False, True])
def test_decode_two_layers_ahead(mx):
    """256 sequences with int8 tables: a 16-token prefill per layer through
    engram_forward, then 3 decode steps in which both layers' Steps 1-5 run
    in two launches and each layer's gate, conv and residual in one; H flows
    from layer 0 into layer 1 and the states advance as in engram_forward."""
    log(f"decode ahead mx={mx}")
    w = inputs.make_config(3, T=3, rows_per_table=997)
    S, M, d = w.B, 1, 1024
    lays = w.layers
    Ls = [eg.Layer(l, "bf16", DEV, mxfp8=mx) for l in lays]
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
        assert names == ["gather2_kernel", "proj_kv_kernel"], names
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
    ("3 layers M=4", dict(B=2, T=40, layers=3, branches=4), False, ["gather2_kernel", "proj_kv_kernel",
                                                                    "gather_kernel<hashed>", "proj_kv_kernel"]),
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
    Ls = [eg.Layer(l, "bf16", DEV, mxfp8=mx) for l in lays]
    tok = torch.from_numpy(w.tokens).to(DEV)
    out = {}
    names = stages(lambda: out.setdefault("kv", eg.project_ahead(tok, Ls)))
    assert names == want, names
    H = eg.to_device(w.H, "bf16", DEV)
    for li, (L, lay) in enumerate(zip(Ls, lays)):
        h_in = H.view(torch.int16).cpu().numpy().view(np.uint16).copy()
        alpha, y = eg.forward_projected(out["kv"][li], H, L, B, T, want_alpha=True, want_y=True)
        torch.cuda.synchronize()
        ref = orc.forward(w.tokens, h_in, lay, "bf16", gemm="mxfp8" if mx else "exact")
        check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(h_in),
                         tag=f"{name} layer {li}")
