"""GPU: n-gram orders up to N = 4, the largest the library takes (the
benchmark's workloads stop at 3).  Four ids per window, three orders of K = 4
heads of 32 dims (d_mem = 384); indices and rows bit-exact against the
oracle, the layer within the bf16 tolerances, a continued sequence reading
three ids of history, and an Engram-Nine hot tier with 2-, 3- and 4-gram sets
(16 lanes per (token, order), so a wavefront holds four different lookups)."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_order4_indices_rows_and_layer():
    log("order 4: indices, rows, layer")
    w = inputs.make_order4(B=3, T=333)
    lay = w.layers[0]
    hp, tab = lay.hash, lay.tables
    assert hp.max_n == 4 and hp.n_tables == 12
    L = eg.Layer(lay, "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    hist = np.random.default_rng(3).integers(0, hp.vocab_c, size=(3, 3)).astype(np.int32)
    z = eg.hash_indices(tok, L, torch.from_numpy(hist).to(DEV))
    e = eg.rows_buffer(3, 333, L, DEV)
    eg.retrieve(tok, L, e)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True)
    torch.cuda.synchronize()
    zr = orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 4, hp.heads, hist)
    assert np.array_equal(z.cpu().numpy(), zr)
    ref = orc.forward(w.tokens, w.H, lay, "bf16")
    assert np.array_equal(to_f64(e).reshape(ref["e"].shape), ref["e"])
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H), tag="order4")


def test_order4_continued_sequence():
    """Prefill in two chunks with a decode state (3 ids of history) equals the
    oracle's chunked forward."""
    log("order 4: chunked prefill")
    w = inputs.make_order4(B=2, T=120)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    span = (lay.kernel_w - 1) * lay.dilation
    st = eg.DecodeState(2, 4, 1, span, lay.d, DEV)
    ost = orc.new_state(2, 4, 1, span, lay.d)
    H = eg.to_device(w.H, "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    for lo, hi in ((0, 2), (2, 71), (71, 120)):
        Hc = H[:, lo:hi].contiguous()
        a, y = eg.forward(tok[:, lo:hi].contiguous(), Hc, L, state=st, want_alpha=True, want_y=True)
        torch.cuda.synchronize()
        r = orc.forward(w.tokens[:, lo:hi], w.H[:, lo:hi], lay, "bf16", state=ost)
        ost = r["state"]
        check_bf16_layer(to_f64(a), r["alpha"], to_f64(y), r["Y"], to_f64(Hc), orc.bf16_to_f64(w.H[:, lo:hi]),
                         tag=f"chunk {lo}:{hi}")
    assert np.array_equal(st.ids.cpu().numpy(), ost["ids"])


def test_order4_hot_tier():
    log("order 4: hot tier")
    w = inputs.make_order4(B=2, T=400)
    lay = w.layers[0]
    hp, tab = lay.hash, lay.tables
    xc = orc.compress(w.tokens, hp.proj)
    keys, rows, dev_rows = {}, {}, {}
    for n in (2, 3, 4):
        k = inputs.frequent_ngrams(xc, n, 120)
        pads = [orc.suffix_ngram(xc, b, t, n) for b in range(2) for t in range(n - 1)]
        k = np.concatenate([k, np.array(pads, dtype=np.int32)])
        _, first = np.unique(k, axis=0, return_index=True)
        keys[n] = k[np.sort(first)]
        rows[n] = inputs.hot_rows(5, 0, n, keys[n].shape[0], hp.heads * tab.dim, "bf16")
        dev_rows[n] = eg.to_device(rows[n], "bf16", DEV)
    hot = eg.HotTier(keys, dev_rows, seed=4, device=DEV)
    L = eg.Layer(lay, "bf16", DEV)
    L.set_hot(hot)
    tok = torch.from_numpy(w.tokens).to(DEV)
    got_idx = eg.hot_lookup(tok, L, hot).cpu().numpy()
    e = eg.rows_buffer(2, 400, L, DEV)
    eg.retrieve(tok, L, e)
    torch.cuda.synchronize()
    ref_keys = {n: [tuple(int(v) for v in r) for r in k] for n, k in keys.items()}
    idx = orc.hot_lookup(w.tokens, hp.proj, 4, ref_keys)
    assert np.array_equal(got_idx, idx)
    assert np.all((idx >= 0).any(axis=(0, 1)))          # every order has hits
    z = orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 4, hp.heads)
    ref_e = orc.gather_two_tier(z, idx, tab.rows, "bf16", tab.row_offset, tab.dim, hp.heads, rows, None, "bf16")
    assert np.array_equal(to_f64(e).reshape(ref_e.shape), ref_e)
