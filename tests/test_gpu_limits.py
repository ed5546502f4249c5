"""GPU parity at the library's documented limits (include/engram.h): the most
tables (ENGRAM_MAX_TABLES = 32: orders 2-3 with 16 heads), the most branches
(ENGRAM_MAX_BRANCHES = 64), the widest hidden state (ENGRAM_MAX_D = 65536),
the most sequences (B = 65535, one token each), and a single token.  Each
layer is checked against the oracle at the bf16 tolerances, the gathered
rows bit for bit."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import bits_equal, check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _layer_check(w, tag, rows=True):
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    tok = torch.from_numpy(w.tokens).to(DEV)
    if rows:
        e = eg.rows_buffer(w.B, w.T, L, DEV)
        eg.retrieve(tok, L, e)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True)
    torch.cuda.synchronize()
    log(f"{tag}: oracle")
    ref = orc.forward(w.tokens, w.H, lay, "bf16")
    if rows:
        assert bits_equal(to_f64(e).reshape(ref["e"].shape), ref["e"]), f"{tag}: gathered rows differ"
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H), tag=tag)


@pytest.mark.parametrize("B,T", [(2, 150), (1, 4000)])
def test_most_tables(B, T):
    """32 tables of 32 dims (d_mem = 1024), d = 256; 300 tokens take the
    small-batch projection, 4,000 the large one."""
    log(f"32 tables B={B} T={T}")
    w = inputs.make_shape(B, T, heads=16, dim=32, d=256)
    assert w.layers[0].hash.n_tables == 32
    _layer_check(w, f"32 tables B={B} T={T}")


@pytest.mark.parametrize("B,T", [(1, 40), (1, 300)])
def test_most_branches(B, T):
    """64 branches of d = 128 (W of 65 x 128 rows), each with its own key
    block, gate and conv."""
    log(f"64 branches B={B} T={T}")
    w = inputs.make_shape(B, T, heads=8, dim=16, d=128, branches=64)
    assert w.layers[0].branches == 64
    _layer_check(w, f"64 branches B={B} T={T}", rows=False)


def test_widest_hidden_state():
    """d = 65536 (the separate product, whole-row gate statistics and the
    LDS-tiled conv) on 20 tokens."""
    log("d = 65536")
    w = inputs.make_shape(1, 20, heads=2, dim=64, d=65536)
    _layer_check(w, "d=65536", rows=False)


def test_most_sequences_one_token_each():
    """B = 65535 sequences of one token: every n-gram is padded, the conv sees
    only the current position; the large-tile projection and one-token strips."""
    log("B = 65535, T = 1")
    w = inputs.make_shape(65535, 1, heads=8, dim=16, d=128)
    _layer_check(w, "B=65535 T=1")


def test_single_token():
    log("B = 1, T = 1")
    w = inputs.make_shape(1, 1)
    _layer_check(w, "B=1 T=1")
