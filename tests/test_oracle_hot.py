"""Pins for the oracle's Engram-Nine hot tier ("DeepSeek Engram series
guide", experiment 3 "Engram-Nine", Figure 1: two-tier retrieval).

  * a hand-derived worked example (tests/golden/engram_nine_toy.txt), with
    and without a decode history;
  * brute force on a tiny vocabulary: the hot row of every position equals
    the one found by scanning a zero-padded copy of the sequence with a
    sliding window, and reversed n-grams do not match;
  * column placement: e_t assembled segment by segment (the hot row for a
    hot n-gram of order n, the K cold rows otherwise) equals the two-tier
    gather;
  * an empty hot set is the cold layer, bit for bit;
  * when every n-gram is hot and every hot row is zero, the layer leaves H
    unchanged whatever the cold tables hold (the all-zero-table pin of the
    layer, moved to the hot tier);
  * repeated hot n-grams and int8 hot rows are rejected.
"""
import os

import numpy as np
import pytest

from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "engram_nine_toy.txt")


def read_golden():
    sec, out = None, {"hot": {}, "expected": [], "history": None, "expected_hist": []}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("["):
            words = line.strip("[]").split()
            if words[0] == "hot":
                sec = ("hot", int(words[1]))
                out["hot"][int(words[1])] = []
            elif words[0] == "history":
                sec = "expected_hist"
                out["history"] = [int(v) for v in words[1:]]
            else:
                sec = words[0]
            continue
        if sec == "sequence":
            out["sequence"] = [int(v) for v in line.split()]
        elif isinstance(sec, tuple):
            row, gram = line.split(":")
            assert int(row) == len(out["hot"][sec[1]])
            out["hot"][sec[1]].append(tuple(int(v) for v in gram.split()))
        else:
            out[sec].append([int(v) for v in line.split()])
    return out


def test_worked_example():
    g = read_golden()
    tokens = np.array([g["sequence"]], dtype=np.int32)
    proj = np.arange(10, dtype=np.int32)
    r = orc.hot_lookup(tokens, proj, 3, g["hot"])
    exp = np.array(g["expected"])
    assert np.array_equal(exp[:, 0], np.arange(tokens.shape[1]))
    assert np.array_equal(r[0], exp[:, 1:])
    hist = np.array([g["history"]], dtype=np.int32)
    rh = orc.hot_lookup(tokens, proj, 3, g["hot"], hist)
    assert np.array_equal(rh[0], np.array(g["expected_hist"])[:, 1:])


def sliding_rows(xc_padded, n, index, T, max_n):
    """Row of the window ending at each t, from a padded copy of one sequence."""
    win = np.lib.stride_tricks.sliding_window_view(xc_padded, n)   # window q covers q .. q+n-1
    first = max_n - n                                               # window ending at t = 0
    return np.array([index.get(tuple(int(v) for v in win[first + t]), -1) for t in range(T)])


@pytest.mark.parametrize("with_hist", [False, True])
def test_brute_force_tiny_vocabulary(with_hist):
    rng = np.random.default_rng(11)
    B, T, V, Vc, N = 2, 60, 9, 4, 4
    proj = rng.integers(0, Vc, size=V).astype(np.int32)
    tokens = rng.integers(0, V, size=(B, T)).astype(np.int32)
    hist = rng.integers(0, Vc, size=(B, N - 1)).astype(np.int32) if with_hist else None
    hot = {}
    for n in range(2, N + 1):
        allg = [tuple(int(v) for v in g) for g in np.ndindex(*([Vc] * n))]
        pick = rng.permutation(len(allg))[: len(allg) // 2]
        hot[n] = [allg[i] for i in pick]
    r = orc.hot_lookup(tokens, proj, N, hot, hist)
    for n in range(2, N + 1):
        index = {g: i for i, g in enumerate(hot[n])}
        for b in range(B):
            pad = hist[b] if with_hist else np.zeros(N - 1, dtype=np.int32)
            padded = np.concatenate([pad, proj[tokens[b]]])
            assert np.array_equal(r[b, :, n - 2], sliding_rows(padded, n, index, T, N))
    # an asymmetric hot 2-gram matches only in its own order
    tok = np.array([[1, 2, 1, 2]], dtype=np.int32)
    ident = np.arange(3, dtype=np.int32)
    assert list(orc.hot_lookup(tok, ident, 2, {2: [(1, 2)]})[0, :, 0]) == [-1, 0, -1, 0]
    assert list(orc.hot_lookup(tok, ident, 2, {2: [(2, 1)]})[0, :, 0]) == [-1, -1, 0, -1]


def tiny(T=50, **kw):
    return inputs.make_config(0, T=T, **kw)


def hot_sets(w, frac, rng):
    """Hot n-grams: a fraction of the distinct n-grams of the workload plus
    n-grams that never occur; rows N(0, 1) in the tables' storage type."""
    lay = w.layers[0]
    hp, tab = lay.hash, lay.tables
    xc = orc.compress(w.tokens, hp.proj)
    keys, rows = {}, {}
    for n in range(2, hp.max_n + 1):
        seen = sorted({orc.suffix_ngram(xc, b, t, n) for b in range(w.B) for t in range(w.T)})
        pick = [seen[i] for i in rng.permutation(len(seen))[: int(len(seen) * frac)]]
        pick += [tuple(int(v) for v in rng.integers(0, hp.vocab_c, size=n)) for _ in range(5)]
        keys[n] = list(dict.fromkeys(pick))
        width = hp.heads * tab.dim
        vals = rng.standard_normal((len(keys[n]), width)).astype(np.float32)
        rows[n] = inputs.to_bf16_bits(vals) if tab.dtype == "bf16" else vals
    return {"keys": keys, "rows": rows}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hot_rows_replace_exactly_the_heads_of_their_order(dtype):
    w = inputs.make_config(1, T=24, rows_per_table=997, d=128) if dtype == "bf16" else tiny()
    assert w.layers[0].tables.dtype == dtype
    lay = w.layers[0]
    hp, tab = lay.hash, lay.tables
    rng = np.random.default_rng(2)
    hot = hot_sets(w, 0.5, rng)
    z = orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads)
    idx = orc.hot_lookup(w.tokens, hp.proj, hp.max_n, hot["keys"])
    e = orc.gather_two_tier(z, idx, tab.rows, tab.dtype, tab.row_offset, tab.dim, hp.heads, hot["rows"],
                            tab.scale, "f32")
    xc = orc.compress(w.tokens, hp.proj)
    K, dim = hp.heads, tab.dim
    n_hits = 0
    for b in range(w.B):
        for t in range(w.T):
            segs = []
            for n in range(2, hp.max_n + 1):
                g = orc.suffix_ngram(xc, b, t, n)
                if g in hot["keys"][n]:
                    r = hot["keys"][n].index(g)
                    segs.append(orc.storage_to_f64(hot["rows"][n][r], tab.dtype))
                    n_hits += 1
                else:
                    for k in range(K):
                        j = (n - 2) * K + k
                        segs.append(orc.storage_to_f64(tab.rows[tab.row_offset[j] + z[b, t, j]], tab.dtype))
            assert np.array_equal(e[b, t], np.concatenate(segs)), (b, t)
    assert 0 < n_hits < w.B * w.T * (hp.max_n - 1)


def test_empty_hot_set_is_the_cold_layer():
    w = tiny()
    a = orc.forward(w.tokens, w.H, w.layers[0], w.dtype)
    b = orc.forward(w.tokens, w.H, w.layers[0], w.dtype, hot={"keys": {}, "rows": {}})
    for k in ("e", "kv", "alpha", "Y", "H_out"):
        assert np.array_equal(a[k], b[k]), k
    assert np.all(b["hot_idx"] == -1)


def test_all_hot_zero_rows_leave_hidden_unchanged_whatever_the_cold_tables():
    w = tiny(T=40)
    lay = w.layers[0]
    hot = hot_sets(w, 1.0, np.random.default_rng(4))
    for n in hot["rows"]:
        hot["rows"][n] = np.zeros_like(hot["rows"][n])
    out = orc.forward(w.tokens, w.H, lay, w.dtype, hot=hot)
    assert np.all(out["hot_idx"] >= 0)
    assert np.any(lay.tables.rows != 0)
    assert np.all(out["Y"] == 0.0) and np.all(out["alpha"] == 0.5)
    assert np.array_equal(out["H_out"], orc.storage_to_f64(w.H, w.dtype))


def test_rejects_repeated_ngrams_and_int8_rows():
    with pytest.raises(ValueError):
        orc.hot_index([(1, 2), (3, 4), (1, 2)])
    z = np.zeros((1, 1, 2), dtype=np.int64)
    with pytest.raises(ValueError):
        orc.gather_two_tier(z, np.zeros((1, 1, 1), dtype=np.int64), np.zeros((4, 8), np.int8), "i8",
                            np.array([0, 2]), 8, 2, {2: np.zeros((1, 16), np.int8)}, np.ones(4, np.float32))
