"""GPU: the real-time LFU hot cache.  Gathers count row accesses exactly (the
oracle's bincount of the hashed rows); an update re-admits rows exactly as
the oracle's lfu_update (stayers keep their slots, newcomers fill the freed
slots in order, counts aged); the updated cache holds the table rows and
stays transparent to the forward, for HBM and host-resident tables."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


def global_rows(lay, tokens):
    hp, tab = lay.hash, lay.tables
    z = orc.hash_indices(tokens, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads)
    return (z + tab.row_offset).ravel()


def drift_tokens(seed, shape):
    """Zipf(1.1) ids with a seeded shuffle of the vocabulary: the hot rows move."""
    rng = np.random.default_rng(seed)
    toks = inputs.zipf_tokens(rng, 128_000, 1.1, shape)
    perm = rng.permutation(128_000).astype(np.int32)
    return np.ascontiguousarray(perm[toks])


def _u32(x):
    return x.cpu().numpy().view(np.uint32).astype(np.int64)


def test_gather_counts_every_access():
    log("lfu counts")
    w = inputs.make_config(1, B=2, T=200, rows_per_table=997)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    counts = torch.zeros(lay.tables.total_rows, dtype=torch.int32, device=DEV)
    L.set_access_counts(counts)
    tok = torch.from_numpy(w.tokens).to(DEV)
    H = eg.to_device(w.H, "bf16", DEV)
    eg.forward(tok, H, L)
    e = eg.rows_buffer(2, 200, L, DEV)
    eg.retrieve(tok, L, e)
    torch.cuda.synchronize()
    want = 2 * np.bincount(global_rows(lay, w.tokens), minlength=lay.tables.total_rows)
    assert np.array_equal(_u32(counts), want)


@pytest.mark.parametrize("config,host", [(1, False), (3, False), (4, True)])
def test_update_matches_oracle_and_stays_transparent(config, host):
    log(f"lfu update config={config} host={host}")
    kw = {"layers": 1} if config in (3, 4) else {}
    w = inputs.make_config(config, B=2, T=150, rows_per_table=997, **kw)
    lay = w.layers[0]
    tab = lay.tables
    hb = None
    if host:
        hb = eg.HostBuffer(tab.rows.nbytes)
        hb.numpy(tab.rows.dtype, tab.rows.shape)[:] = tab.rows
        L = eg.Layer(lay, "bf16", DEV, rows_ptr=hb.dev)
    else:
        L = eg.Layer(lay, "bf16", DEV)
    try:
        n = tab.total_rows // 10
        warm = drift_tokens(1, (4, 1024))
        slot, rows, scale = eg.cache_build(torch.from_numpy(warm).to(DEV), L, n)
        L.set_cache(slot, rows, scale)
        counts = torch.zeros(tab.total_rows, dtype=torch.int32, device=DEV)
        L.set_access_counts(counts)
        tok0 = torch.from_numpy(w.tokens).to(DEV)
        H0 = eg.to_device(w.H, "bf16", DEV)
        ref_slot = slot.cpu().numpy().astype(np.int64)
        for it, seed in enumerate((2, 3)):
            batch = drift_tokens(seed, (4, 512))
            Hx = eg.to_device(inputs.make_config(1, B=4, T=512, rows_per_table=997).H, "bf16", DEV)
            eg.forward(torch.from_numpy(batch).to(DEV), Hx, L)      # counts accumulate
            torch.cuda.synchronize()
            c_before = _u32(counts)
            eg.cache_update(L, counts, decay_shift=1)
            torch.cuda.synchronize()
            ref_slot, ref_counts = orc.lfu_update(c_before, ref_slot, n, decay_shift=1)
            got = slot.cpu().numpy().astype(np.int64)
            assert np.array_equal(got, ref_slot), f"update {it}"
            assert np.array_equal(_u32(counts), ref_counts)
            adm = np.nonzero(got >= 0)[0]
            sl = torch.from_numpy(got[adm]).to(DEV)
            crow = rows[sl].contiguous()
            crow = crow.view(torch.int16 if tab.dtype == "bf16" else torch.int8).cpu().numpy()
            assert np.array_equal(crow.view(tab.rows.dtype), tab.rows[adm])
            if tab.dtype == "i8":
                assert np.array_equal(scale[sl].cpu().numpy(), tab.scale[adm])
            # transparent: the forward through the updated cache equals the uncached one
            L.set_access_counts(None)
            Hc, Hu = H0.clone(), H0.clone()
            eg.forward(tok0, Hc, L)
            L.set_cache(None, None, None)
            eg.forward(tok0, Hu, L)
            L.set_cache(slot, rows, scale)
            L.set_access_counts(counts)
            torch.cuda.synchronize()
            assert torch.equal(Hc.view(torch.int16), Hu.view(torch.int16))
    finally:
        torch.cuda.synchronize()
        if hb is not None:
            hb.free()
