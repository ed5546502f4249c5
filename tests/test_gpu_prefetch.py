"""GPU: one batch's Steps 5-8 with the next batch's Steps 1-4 in the same
launches (engram_forward_retrieved_prefetch).  Whether the next gather runs
inside the conv launch or after it, every output equals
engram_forward_retrieved followed by engram_retrieve, bit for bit, and the
layer matches the oracle."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def stage_names(fn):
    eg.profile_enable(True)
    try:
        fn()
        return [n for n, _ in eg.profile_read()]
    finally:
        eg.profile_enable(False)


@pytest.mark.parametrize("config,B,T,nB,nT,mx,fused", [
    (1, 2, 300, 2, 300, False, True),
    (1, 1, 512, 3, 77, False, True),     # next batch of another shape
    (2, 1, 200, 1, 200, False, True),    # four branches
    (1, 2, 300, 1, 260, True, True),     # MXFP8 rows for the next batch
    (1, 1, 20, 1, 20, False, True),      # fewer strips than XCDs: the plain strip order
])
def test_prefetch_equals_separate_calls(config, B, T, nB, nT, mx, fused):
    log(f"prefetch config={config} B={B} T={T} next={nB}x{nT} mx={mx}")
    w = inputs.make_config(config, B=B, T=T, rows_per_table=997)
    lay = w.layers[0]
    L = eg.Layer(lay, w.dtype, DEV, mxfp8=mx)
    tok = torch.from_numpy(w.tokens).to(DEV)
    rng = np.random.default_rng(7)
    ntok_np = inputs.zipf_tokens(rng, lay.hash.vocab, 1.1, (nB, nT))
    ntok = torch.from_numpy(ntok_np).to(DEV)
    e = eg.rows_buffer(B, T, L, DEV)
    eg.retrieve(tok, L, e)
    H0 = eg.to_device(w.H, w.dtype, DEV)
    # separate calls
    H1 = H0.clone()
    a1, y1 = eg.forward_retrieved(tok, e, H1, L, want_alpha=True, want_y=True)
    ne1 = eg.rows_buffer(nB, nT, L, DEV)
    eg.retrieve(ntok, L, ne1)
    # one call
    H2 = H0.clone()
    ne2 = eg.rows_buffer(nB, nT, L, DEV)
    out = {}

    def call():
        out["ay"] = eg.forward_retrieved_prefetch(tok, e, H2, L, ntok, ne2, want_alpha=True, want_y=True)
    names = stage_names(call)
    a2, y2 = out["ay"]
    torch.cuda.synchronize()
    assert ("conv_gather_kernel" in names) == fused, names
    assert torch.equal(_bits(H1), _bits(H2)) and torch.equal(a1, a2) and torch.equal(y1, y2)
    assert torch.equal(ne1, ne2)
    if not mx:
        ref = orc.forward(w.tokens, w.H, lay, w.dtype)
        check_bf16_layer(to_f64(a2), ref["alpha"], to_f64(y2), ref["Y"], to_f64(H2), orc.storage_to_f64(w.H, w.dtype),
                         tag="prefetch")
        hp, tab = lay.hash, lay.tables
        z = orc.hash_indices(ntok_np, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads)
        ref_e = orc.gather(z, tab.rows, tab.dtype, tab.row_offset, tab.dim, tab.scale, out_dtype="bf16")
        assert np.array_equal(to_f64(ne2).reshape(ref_e.shape), ref_e)


def test_prefetch_with_empty_halves_and_hot_tier():
    log("prefetch edge cases")
    w = inputs.make_config(1, B=1, T=256, rows_per_table=997)
    lay = w.layers[0]
    L = eg.Layer(lay, w.dtype, DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    e = eg.rows_buffer(1, 256, L, DEV)
    eg.retrieve(tok, L, e)
    H0 = eg.to_device(w.H, w.dtype, DEV)
    # no next batch: the plain compute
    H1, H2 = H0.clone(), H0.clone()
    eg.forward_retrieved(tok, e, H1, L)
    eg.forward_retrieved_prefetch(tok, e, H2, L, None, None)
    torch.cuda.synchronize()
    assert torch.equal(_bits(H1), _bits(H2))
    # no current batch: the plain retrieval
    e2 = eg.rows_buffer(1, 256, L, DEV)
    eg.forward_retrieved_prefetch(tok[:, :0].contiguous(), e, H2, L, tok, e2)
    torch.cuda.synchronize()
    assert torch.equal(e, e2)
    # a hot tier: the gather runs after the conv, same results
    keys = {2: np.array([[int(lay.hash.proj[w.tokens[0, 0]]), int(lay.hash.proj[w.tokens[0, 1]])]], np.int32)}
    rows = {2: eg.to_device(inputs.hot_rows(1, 0, 2, 1, lay.hash.heads * lay.tables.dim, "bf16"), "bf16", DEV)}
    L.set_hot(eg.HotTier(keys, rows, device=DEV))
    H3, H4 = H0.clone(), H0.clone()
    ref_e = eg.rows_buffer(1, 256, L, DEV)
    eg.forward_retrieved(tok, e, H3, L)
    eg.retrieve(tok, L, ref_e)
    e4 = eg.rows_buffer(1, 256, L, DEV)
    names = stage_names(lambda: eg.forward_retrieved_prefetch(tok, e, H4, L, tok, e4))
    torch.cuda.synchronize()
    assert "conv_gather_kernel" not in names and "gather_kernel<hashed,hot>" in names
    assert torch.equal(_bits(H3), _bits(H4)) and torch.equal(ref_e, e4)
    assert not torch.equal(ref_e, e)     # the hot row replaced the first token's 2-gram segment


@pytest.mark.parametrize("config,table", [(4, "bf16"), (3, "i8")])
def test_prefetch_of_the_next_layer(config, table):
    """Layer 0's compute carrying layer 1's retrieval of the same tokens (bf16
    or int8 tables): equal to the separate calls, bit for bit."""
    log(f"prefetch next layer config={config}")
    kw = dict(B=1, T=300, layers=2) if config == 4 else dict(B=16, T=1, layers=2)
    w = inputs.make_config(config, rows_per_table=997, **kw)
    assert w.layers[1].tables.dtype == table
    L0, L1 = (eg.Layer(l, "bf16", DEV) for l in w.layers)
    B, T = w.B, w.T
    tok = torch.from_numpy(w.tokens).to(DEV)
    e0 = eg.rows_buffer(B, T, L0, DEV)
    eg.retrieve(tok, L0, e0)
    H0 = eg.to_device(w.H, "bf16", DEV)
    H1, H2 = H0.clone(), H0.clone()
    eg.forward_retrieved(tok, e0, H1, L0)
    ref = eg.rows_buffer(B, T, L1, DEV)
    eg.retrieve(tok, L1, ref)
    got = eg.rows_buffer(B, T, L1, DEV)
    names = stage_names(lambda: eg.forward_retrieved_prefetch(tok, e0, H2, L0, tok, got, next_layer=L1))
    torch.cuda.synchronize()
    assert "conv_gather_kernel" in names, names
    assert torch.equal(_bits(H1), _bits(H2)) and torch.equal(ref, got)


def test_decode_steps_with_the_next_layer_prefetched():
    """Two-layer decode: after a 16-token prefill, each single-token step runs
    layer 0 with layer 1's retrieval (its own id history) inside layer 0's conv
    launch, then layer 1 on those rows.  Hidden states, the rows and both
    decode states equal plain per-layer forwards, bit for bit."""
    log("prefetch decode")
    w = inputs.make_config(3, B=32, rows_per_table=997)
    lays = w.layers
    Ls = [eg.Layer(l, "bf16", DEV) for l in lays]
    S, span, d = w.B, (lays[0].kernel_w - 1) * lays[0].dilation, lays[0].d
    states = {k: [eg.DecodeState(S, 3, 1, span, d, DEV) for _ in Ls] for k in ("plain", "fused")}
    ctx = torch.from_numpy(w.context).to(DEV)
    for k in states:
        Hc = eg.to_device(w.H_context, "bf16", DEV)
        for L, st in zip(Ls, states[k]):
            eg.forward(ctx, Hc, L, state=st)
    rng = np.random.default_rng(21)
    Hp = eg.to_device(w.H, "bf16", DEV)
    Hf = Hp.clone()
    e0 = eg.rows_buffer(S, 1, Ls[0], DEV)
    e1 = eg.rows_buffer(S, 1, Ls[1], DEV)
    fused_seen = False
    for step in range(4):
        tok = torch.from_numpy(inputs.zipf_tokens(rng, 128_000, 1.1, (S, 1))).to(DEV)
        for L, st in zip(Ls, states["plain"]):
            eg.forward(tok, Hp, L, state=st)
        s0, s1 = states["fused"]
        eg.retrieve(tok, Ls[0], e0, state=s0)
        names = stage_names(lambda: eg.forward_retrieved_prefetch(tok, e0, Hf, Ls[0], tok, e1, next_layer=Ls[1],
                                                                  state=s0, next_state=s1))
        fused_seen |= "conv_gather_kernel" in names and "state_commit_kernel" not in names
        eg.forward_retrieved(tok, e1, Hf, Ls[1], state=s1)
        torch.cuda.synchronize()
        assert torch.equal(_bits(Hp), _bits(Hf)), step
        for a, b in zip(states["plain"], states["fused"]):
            assert torch.equal(a.ids, b.ids) and torch.equal(a.pos, b.pos) and torch.equal(a.conv, b.conv), step
    assert fused_seen
