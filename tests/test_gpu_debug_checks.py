"""GPU: the debug build's precondition checks (libengram_debug.so).  Values
outside their ranges are fed to the debug build only, whose kernels test
each one before the load that uses it and replace it by an in-range value,
so every access stays inside its buffer; each case is compared with the same
call on valid inputs and the error word must hold exactly the expected bit.
Raw token ids are clamped in the release build too, which is also checked."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import build as bld
from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs

from parity import log

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture
def debug_lib():
    release = eg.lib()
    dbg = eg.load_library(bld.LIB_DEBUG)
    eg._lib = dbg
    word = torch.zeros(1, dtype=torch.int32, device=DEV)
    eg.debug_set_error_word(word)
    try:
        assert eg.debug_checks()
        yield release
    finally:
        torch.cuda.synchronize()
        dbg.engram_debug_set_error_word(None)   # tests may have switched the binding to the release build
        eg._lib = release


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_clean_inputs_set_no_bits_and_match_the_release_build(debug_lib):
    log("debug build: clean inputs")
    w = inputs.make_config(1, B=2, T=300, rows_per_table=997)
    L = eg.Layer(w.layers[0], "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    H_dbg = eg.to_device(w.H, "bf16", DEV)
    H_rel = H_dbg.clone()
    eg.forward(tok, H_dbg, L)
    assert eg.debug_read_errors() == 0
    eg._lib = debug_lib                      # the release build on the same inputs
    eg.forward(tok, H_rel, L)
    torch.cuda.synchronize()
    assert _same(H_dbg, H_rel)


def test_out_of_range_tokens_are_clamped_and_reported(debug_lib):
    log("debug build: out-of-range token ids")
    w = inputs.make_config(1, B=2, T=40, rows_per_table=997)
    V = w.layers[0].hash.vocab
    bad = w.tokens.copy()
    bad[0, 3], bad[0, 7], bad[1, 0], bad[1, 20] = -5, V, V + 100, -1
    clamped = np.clip(bad, 0, V - 1)
    L = eg.Layer(w.layers[0], "bf16", DEV)
    H_bad, H_ref = eg.to_device(w.H, "bf16", DEV), eg.to_device(w.H, "bf16", DEV)
    eg.forward(torch.from_numpy(bad).to(DEV), H_bad, L)
    assert eg.debug_read_errors() == eg.ERR_TOKEN
    eg.forward(torch.from_numpy(clamped).to(DEV), H_ref, L)
    assert eg.debug_read_errors() == 0
    assert _same(H_bad, H_ref)
    eg._lib = debug_lib                      # the release build clamps the ids the same way
    H_rel = eg.to_device(w.H, "bf16", DEV)
    eg.forward(torch.from_numpy(bad).to(DEV), H_rel, L)
    torch.cuda.synchronize()
    assert _same(H_rel, H_ref)


def test_out_of_range_row_indices_are_clamped_and_reported(debug_lib):
    log("debug build: out-of-range row indices in engram_gather")
    w = inputs.make_config(1, B=3, T=20, rows_per_table=997)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    p = lay.hash.prime.astype(np.int64)
    rng = np.random.default_rng(3)
    z = np.stack([rng.integers(0, int(q), size=(3, 20)) for q in p], axis=-1)
    z[0, 0, 0], z[0, 1, 5], z[2, 19, 15], z[1, 4, 9] = -1, p[5], 1 << 30, -(1 << 30)
    zc = np.clip(z, 0, p - 1)
    e_bad = eg.gather(torch.from_numpy(z.astype(np.int32)).to(DEV), L, "bf16")
    assert eg.debug_read_errors() == eg.ERR_ROW
    e_ref = eg.gather(torch.from_numpy(zc.astype(np.int32)).to(DEV), L, "bf16")
    assert eg.debug_read_errors() == 0
    assert _same(e_bad, e_ref)


def test_out_of_range_cache_slots_read_as_misses_and_are_reported(debug_lib):
    log("debug build: out-of-range cache slots")
    w = inputs.make_config(1, B=2, T=60, rows_per_table=997)
    lay = w.layers[0]
    tab = lay.tables
    L = eg.Layer(lay, "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    plain = eg.rows_buffer(2, 60, L, DEV)
    eg.retrieve(tok, L, plain)
    rng = np.random.default_rng(5)
    n = tab.total_rows // 3
    cached = np.sort(rng.choice(tab.total_rows, size=n, replace=False))
    slot = np.full(tab.total_rows, -1, dtype=np.int32)
    slot[cached] = np.arange(n, dtype=np.int32)
    crows = np.ascontiguousarray(tab.rows[cached])
    hp = lay.hash
    from oracle import engram_oracle as orc            # which rows the batch reads (test set-up only)
    used = (orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 3, hp.heads) + tab.row_offset).ravel()
    slot[used[0]], slot[used[17]], slot[used[300]] = n, -7, 1 << 30          # outside [-1, n)
    L.set_cache(eg.to_device(slot, "i32", DEV), eg.to_device(crows, "bf16", DEV))
    got = eg.rows_buffer(2, 60, L, DEV)
    eg.retrieve(tok, L, got)
    assert eg.debug_read_errors() == eg.ERR_SLOT
    assert _same(got, plain)


def test_out_of_range_hot_rows_read_as_cold_and_are_reported(debug_lib):
    log("debug build: out-of-range hot-tier rows")
    w = inputs.make_config(1, B=2, T=200, rows_per_table=997)
    lay = w.layers[0]
    hp = lay.hash
    x = hp.proj[w.tokens]
    keys = {n: inputs.frequent_ngrams(x, n, 50) for n in (2, 3)}
    hot = eg.HotTier(keys, None, device=DEV)
    L = eg.Layer(lay, "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    before = eg.hot_lookup(tok, L, hot)
    assert eg.debug_read_errors() == 0
    hits = before[..., 0]
    r = int(hits[hits >= 0][0])                       # a hot row the batch uses (order 2)
    slots = hot.slots[2].view(-1, 8)
    s = int(torch.nonzero(slots[:, 4] == r)[0, 0])
    slots[s, 4] = int(hot.s.n_hot[0]) + 5             # that slot now names a row outside the set
    after = eg.hot_lookup(tok, L, hot)
    assert eg.debug_read_errors() == eg.ERR_HOT_ROW
    expect = before.clone()
    expect[..., 0][before[..., 0] == r] = -1
    assert torch.equal(after, expect)


def test_steps_ahead_out_of_range_tokens_are_clamped_and_reported(debug_lib):
    """The one-launch Steps 1-5 of two decode layers (engram_project_ahead
    with a packed W) checks the raw ids as the gather does, and the decode
    state advances with the clamped ids."""
    log("debug build: out-of-range token ids in the fused Steps 1-5")
    w = inputs.make_config(3, B=64, T=1, rows_per_table=997)
    V = w.layers[0].hash.vocab
    bad = w.tokens.copy()
    bad[0, 0], bad[5, 0], bad[40, 0] = -3, V + 7, V
    clamped = np.clip(bad, 0, V - 1)
    Ls = [eg.Layer(lay, "bf16", DEV) for lay in w.layers]
    assert all(L.w_packed is not None for L in Ls)
    st_bad = [eg.DecodeState(64, 3, 1, 9, 1024, DEV) for _ in Ls]
    st_ref = [eg.DecodeState(64, 3, 1, 9, 1024, DEV) for _ in Ls]
    kv_bad = eg.project_ahead(torch.from_numpy(bad).to(DEV), Ls, states=st_bad)
    assert eg.debug_read_errors() == eg.ERR_TOKEN
    kv_ref = eg.project_ahead(torch.from_numpy(clamped).to(DEV), Ls, states=st_ref)
    assert eg.debug_read_errors() == 0
    torch.cuda.synchronize()
    for a, b, sa, sb in zip(kv_bad, kv_ref, st_bad, st_ref):
        assert torch.equal(a, b)
        assert torch.equal(sa.ids, sb.ids) and torch.equal(sa.pos, sb.pos)
