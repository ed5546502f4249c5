"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Hash indices and gathered rows must be bit-exact; float
results meet the tolerances in tests/parity.py."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import (bits_equal, check_bf16_layer, check_f32, check_f32_layer, check_kv_bf16, log, to_f64)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def small(config, **kw):
    kw.setdefault("rows_per_table", 997)
    return inputs.make_config(config, **kw)


def dev_tokens(w, tokens=None):
    return torch.from_numpy(np.ascontiguousarray(w.tokens if tokens is None else tokens)).to(DEV)


def dev_H(w, H=None):
    return eg.to_device(w.H if H is None else H, w.dtype, DEV)


# --------------------------------------------------------------------------
# Steps 1-3
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["c0", "c1-primes", "c0-hist", "ragged"])
def test_hash_indices_bit_exact(case):
    log(f"hash case={case}")
    if case == "c1-primes":
        hp = inputs.hash_inputs_for(1)
        tokens = inputs.zipf_tokens(inputs.rng_for(1, 0, inputs.S_TOKENS), 128_000, 1.1, (3, 1000))
    elif case == "ragged":
        hp = inputs.hash_inputs_for(1)
        tokens = inputs.zipf_tokens(inputs.rng_for(1, 5, inputs.S_TOKENS), 128_000, 1.1, (5, 1))
    else:
        hp = inputs.hash_inputs_for(0)
        tokens = inputs.rng_for(0, 0, inputs.S_TOKENS).integers(0, 1000, size=(4, 33), dtype=np.int32)
    hist = None
    if case == "c0-hist":
        hist = np.array([[5, 7], [0, 0], [769, 1], [3, 3]], dtype=np.int32)
    spec = eg.HashSpec(hp, DEV)
    z = eg.hash_indices(torch.from_numpy(tokens).to(DEV), spec,
                        hist=None if hist is None else torch.from_numpy(hist).to(DEV))
    ref = orc.hash_indices(tokens, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads, hist)
    assert np.array_equal(z.cpu().numpy(), ref)


def test_hash_all_bigrams_and_sub_vocab_trigrams():
    """Every 2-gram over V' = 770 and every 3-gram over 64 ids: the GPU index
    equals the oracle's for each enumerated n-gram, for every head."""
    log("hash exhaustive 2-grams (592,900 sequences) and 3-grams (262,144)")
    hp0 = inputs.hash_inputs_for(0)
    ident = inputs.HashInputs(770, 770, 3, hp0.heads, np.arange(770, dtype=np.int32), hp0.mult, hp0.prime)
    a, b = np.meshgrid(np.arange(770), np.arange(770), indexing="ij")
    seq = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.int32)        # x'_0 = a, x'_1 = b
    z = eg.hash_indices(torch.from_numpy(seq).to(DEV), eg.HashSpec(ident, DEV)).cpu().numpy()
    for k in range(ident.heads):
        ref = orc.hash_grams(np.stack([seq[:, 1], seq[:, 0]], 1), ident.mult[0, k], int(ident.prime[k]))
        assert np.array_equal(z[:, 1, k], ref)
    hp1 = inputs.hash_inputs_for(1)
    ident1 = inputs.HashInputs(98_560, 98_560, 3, hp1.heads, np.arange(98_560, dtype=np.int32), hp1.mult,
                               hp1.prime)
    ids = (np.arange(64) * 1531 % 98_560).astype(np.int32)
    g = np.stack(np.meshgrid(ids, ids, ids, indexing="ij"), -1).reshape(-1, 3)   # oldest first
    z = eg.hash_indices(torch.from_numpy(np.ascontiguousarray(g)).to(DEV), eg.HashSpec(ident1, DEV)).cpu().numpy()
    for k in range(hp1.heads):
        j = hp1.heads + k
        ref = orc.hash_grams(g[:, ::-1], hp1.mult[1, k], int(hp1.prime[j]))
        assert np.array_equal(z[:, 2, j], ref)


# --------------------------------------------------------------------------
# Steps 3-4
# --------------------------------------------------------------------------

@pytest.mark.parametrize("config,out", [(0, "f32"), (0, "bf16"), (1, "bf16"), (1, "f32"), (3, "bf16"), (3, "f32")])
def test_gather_bit_exact(config, out):
    log(f"gather config={config} out={out}")
    w = small(config, B=3, T=77, layers=1) if config == 3 else small(config, B=3, T=77)
    lay = w.layers[0]
    hp, tab = lay.hash, lay.tables
    L = eg.Layer(lay, w.dtype, DEV)
    rng = np.random.default_rng(9)
    z = np.stack([rng.integers(0, int(p), size=(3, 77)) for p in hp.prime], axis=-1).astype(np.int32)
    z[0, 0] = 0
    z[0, 1] = (hp.prime - 1).astype(np.int32)                                      # last row of each table
    e = eg.gather(torch.from_numpy(z).to(DEV), L, out)
    ref = orc.gather(z, tab.rows, tab.dtype, tab.row_offset, tab.dim, tab.scale, out)
    assert bits_equal(to_f64(e), ref)


@pytest.mark.parametrize("config", [1, 3])
def test_gather_cache_is_transparent(config):
    """A row read through the HBM hot cache equals the row read from the
    table: 0 %, 30 % and 100 % caches give identical results."""
    log(f"gather cache config={config}")
    w = small(config, B=2, T=100, layers=1) if config == 3 else small(config, B=2, T=100)
    lay = w.layers[0]
    tab = lay.tables
    L = eg.Layer(lay, w.dtype, DEV)
    hp = lay.hash
    z = torch.from_numpy(orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 3, hp.heads).astype(np.int32)).to(DEV)
    plain = to_f64(eg.gather(z, L, "bf16"))
    rng = np.random.default_rng(2)
    for frac in (0.0, 0.3, 1.0):
        n = int(frac * tab.total_rows)
        cached = np.sort(rng.choice(tab.total_rows, size=n, replace=False))
        slot = np.full(tab.total_rows, -1, dtype=np.int32)
        order = rng.permutation(n)
        slot[cached] = order.astype(np.int32)
        crows = np.zeros((max(n, 1), tab.dim), dtype=tab.rows.dtype)
        crows[order] = tab.rows[cached]
        kind = tab.dtype
        cs = None
        if tab.dtype == "i8":
            sc = np.zeros(max(n, 1), dtype=np.float32)
            sc[order] = tab.scale[cached]
            cs = eg.to_device(sc, "f32", DEV)
        L.set_cache(eg.to_device(slot, "i32", DEV), eg.to_device(crows, kind, DEV), cs)
        got = to_f64(eg.gather(z, L, "bf16"))
        assert bits_equal(got, plain), frac
    L.set_cache(None, None)


# --------------------------------------------------------------------------
# Step 5
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n_tok,d_mem,n_out", [(300, 1024, 2048), (37, 1024, 5120), (129, 64, 192), (1, 128, 64),
                                               (4096, 1024, 2048)])
def test_project_kv_bf16(n_tok, d_mem, n_out):
    log(f"project_kv bf16 n_tok={n_tok} d_mem={d_mem} n_out={n_out}")
    rng = inputs.rng_for(99, 0, n_tok)
    e = inputs.normal_bf16_bits(rng, n_tok * d_mem, 0.02).reshape(n_tok, d_mem)
    wt = inputs.normal_bf16_bits(rng, n_out * d_mem, 1 / 32).reshape(n_out, d_mem)
    kv = eg.project_kv(eg.to_device(e, "bf16", DEV), eg.to_device(wt, "bf16", DEV))
    ref = orc.project_kv(orc.bf16_to_f64(e), orc.bf16_to_f64(wt))
    check_kv_bf16(to_f64(kv), ref, d_mem, tag=f"{n_tok}x{d_mem}x{n_out}")


def test_project_kv_f32():
    log("project_kv f32")
    rng = inputs.rng_for(98, 0, 0)
    e = inputs.normal_f32(rng, 65 * 32, 0.02).reshape(65, 32)
    wt = inputs.normal_f32(rng, 128 * 32, 1 / 32).reshape(128, 32)
    kv = eg.project_kv(eg.to_device(e, "f32", DEV), eg.to_device(wt, "f32", DEV))
    check_f32("kv", to_f64(kv), orc.project_kv(e, wt))


# --------------------------------------------------------------------------
# Steps 6-8 on given projections
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,M,d,B,T", [("f32", 1, 64, 2, 50), ("bf16", 1, 1024, 2, 77), ("bf16", 4, 1024, 1, 70),
                                           ("bf16", 2, 128, 3, 5)])
def test_gate_conv_forward(dtype, M, d, B, T):
    log(f"gate_conv dtype={dtype} M={M} d={d} B={B} T={T}")
    rng = inputs.rng_for(97, M, d)
    n_kv = B * T * (1 + M) * d
    if dtype == "bf16":
        kvb = inputs.normal_bf16_bits(rng, n_kv, 0.02).reshape(B, T, (1 + M) * d)
        Hb = inputs.normal_bf16_bits(rng, B * T * M * d, 1.0).reshape(B, T, M, d)
    else:
        kvb = inputs.normal_f32(rng, n_kv, 0.02).reshape(B, T, (1 + M) * d)
        Hb = inputs.normal_f32(rng, B * T * M * d, 1.0).reshape(B, T, M, d)
    conv_w = inputs.normal_f32(rng, M * d * 4, 0.1).reshape(M, d, 4)
    li = small(0 if dtype == "f32" else 1, d=d, branches=M, T=4).layers[0]
    li.conv_w = conv_w
    L = eg.Layer(li, dtype, DEV)
    H = eg.to_device(Hb, dtype, DEV)
    kv = eg.to_device(kvb, dtype, DEV)
    alpha, y = eg.gate_conv_forward(H, kv, L, want_alpha=True, want_y=True)
    ref = orc.gate_conv(orc.storage_to_f64(Hb, dtype), orc.storage_to_f64(kvb, dtype), conv_w, 3, 1e-6)
    h_in = orc.storage_to_f64(Hb, dtype)
    chk = check_f32_layer if dtype == "f32" else check_bf16_layer
    chk(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), h_in, tag="gate_conv")


# --------------------------------------------------------------------------
# Steps 1-8
# --------------------------------------------------------------------------

def _forward_check(w, layer_idx=0, tag=""):
    lay = w.layers[layer_idx]
    L = eg.Layer(lay, w.dtype, DEV)
    H = dev_H(w)
    alpha, y = eg.forward(dev_tokens(w), H, L, want_alpha=True, want_y=True)
    ref = orc.forward(w.tokens, w.H, lay, w.dtype)
    h_in = orc.storage_to_f64(w.H, w.dtype)
    chk = check_f32_layer if w.dtype == "f32" else check_bf16_layer
    chk(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), h_in, tag=tag)
    return ref


@pytest.mark.parametrize("B,T,dim", [(1, 64, 16), (3, 37, 16), (2, 20, 8)])
def test_forward_fp32(B, T, dim):
    log(f"forward fp32 B={B} T={T} table_dim={dim}")
    w = inputs.make_config(0, B=B, T=T, table_dim=dim)
    _forward_check(w, tag="c0")


# Up to 7 * 2^18 token-features (896 tokens at N = 2048, 358 at N = 5120) the
# projection runs the small-batch kernel (64 x 32 tiles, K split over
# wavefronts): (1, 1, 1), (1, 3, 11), (2, 1, 40), (1, 2, 300) and (2, 2, 130);
# (1, 2, 1100) and (2, 1, 900) run the large-tile kernel with a ragged last
# token tile.
@pytest.mark.parametrize("config,B,T", [(1, 2, 300), (1, 1, 1), (1, 3, 11), (2, 1, 40), (2, 2, 130), (1, 2, 1100),
                                        (2, 1, 900)])
def test_forward_bf16(config, B, T):
    log(f"forward bf16 config={config} B={B} T={T}")
    w = small(config, B=B, T=T)
    _forward_check(w, tag=f"c{config}")




# Either side of the switch between the two projection kernels (7 * 2^18
# token-features): 896 / 897 tokens at N = 2048, 358 / 359 at N = 5120.
@pytest.mark.parametrize("config,B,T", [(1, 1, 896), (1, 1, 897), (2, 2, 179), (2, 1, 359)])
def test_forward_bf16_kernel_switch(config, B, T):
    log(f"forward bf16 kernel switch config={config} B={B} T={T}")
    w = small(config, B=B, T=T)
    names = []
    eg.profile_enable(True)
    try:
        _forward_check(w, tag=f"c{config} switch")
        names = [n for n, _ in eg.profile_read()]
    finally:
        eg.profile_enable(False)
    assert "proj_gate_kernel" in names, names

def test_profile_accumulates_back_to_back_calls():
    """Mode 2 keeps the stages of several calls until one read, in launch
    order; the next read starts a new series; mode 1 keeps the last call's."""
    w = small(1, B=1, T=300)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    tok, H = dev_tokens(w), dev_H(w)
    try:
        eg.profile_enable(1)
        eg.forward(tok, H, L)
        one = [n for n, _ in eg.profile_read()]
        eg.profile_enable(2)
        for _ in range(3):
            eg.forward(tok, H, L)
        three = eg.profile_read()
        eg.forward(tok, H, L)
        again = eg.profile_read()
    finally:
        eg.profile_enable(False)
    assert one == ["gather_kernel<hashed>", "proj_gate_kernel", "conv_kernel"], one
    assert [n for n, _ in three] == one * 3
    assert [n for n, _ in again] == one
    assert all(t > 0 for _, t in three + again)


# Narrow tables: d_mem = 16 x 8 = 128 or 16 x 32 = 512 (K of the projection).
# The small-batch kernel's K range per wavefront is then 32 or 128 elements,
# a partial or a whole number of its 64-element load batches; 1,100 tokens at
# d_mem = 128 take the large-tile kernel with two K slices.
@pytest.mark.parametrize("table_dim,B,T", [(8, 2, 40), (32, 1, 300), (8, 1, 1100)])
def test_forward_bf16_narrow_tables(table_dim, B, T):
    log(f"forward bf16 narrow tables table_dim={table_dim} B={B} T={T}")
    w = small(1, B=B, T=T, table_dim=table_dim)
    _forward_check(w, tag=f"c1 table_dim={table_dim}")

# Hidden widths off the fused path (d not a multiple of 128: the separate
# product, then whole-row gate statistics) and several branches in fp32.
@pytest.mark.parametrize("dtype,d,M,B,T", [("bf16", 192, 2, 2, 50), ("bf16", 64, 3, 1, 70), ("f32", 128, 2, 2, 33)])
def test_forward_unfused_widths(dtype, d, M, B, T):
    log(f"forward unfused dtype={dtype} d={d} M={M} B={B} T={T}")
    w = small(0 if dtype == "f32" else 1, B=B, T=T, d=d, branches=M)
    names = []
    eg.profile_enable(True)
    try:
        ref = _forward_check(w, tag=f"unfused d={d}")
        names = [n for n, _ in eg.profile_read()]
    finally:
        eg.profile_enable(False)
    assert "gemm_kernel" in names and "gate_stats_kernel" in names, names
    assert ref["Y"].shape == (B, T, M, d)


# Hidden widths above 2048 on the fused path, bf16 and MXFP8 products, at
# token counts that the small-batch projection would take for narrower
# layers: its 64-column statistics tiles would give the conv more than its
# 64 statistics per row, so these run 128-column tiles.
@pytest.mark.parametrize("d,B,T,mx", [(3072, 2, 75, False), (4096, 1, 150, False), (3072, 3, 40, True),
                                      (4096, 2, 64, True)])
def test_forward_wide_hidden(d, B, T, mx):
    log(f"forward wide hidden d={d} B={B} T={T} mxfp8={mx}")
    w = small(1, B=B, T=T, d=d)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV, mxfp8=mx)
    H = dev_H(w)
    names = []
    eg.profile_enable(True)
    try:
        alpha, y = eg.forward(dev_tokens(w), H, L, want_alpha=True, want_y=True)
        names = [n for n, _ in eg.profile_read()]
    finally:
        eg.profile_enable(False)
    assert "proj_gate_kernel" in names, names
    ref = orc.forward(w.tokens, w.H, lay, "bf16", gemm="mxfp8" if mx else "exact")
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H),
                     tag=f"wide d={d} mx={mx}")


def test_forward_empty_is_noop():
    log("forward empty")
    w = small(1, B=1, T=4)
    L = eg.Layer(w.layers[0], "bf16", DEV)
    H = torch.zeros((0, 4, 1, 1024), dtype=torch.bfloat16, device=DEV)
    tok = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    eg.forward(tok, H, L)
    torch.cuda.synchronize()


@pytest.mark.parametrize("config", [0, 3])
def test_decode_steps_match_oracle(config):
    """Prefill a context with a state, then decode token by token; every step
    matches the oracle and the state matches the oracle's state."""
    log(f"decode config={config}")
    if config == 0:
        w = inputs.make_config(0, B=4, T=12)
        ctx_len = 7
        ctx = w.tokens[:, :ctx_len]
        Hc = w.H[:, :ctx_len]
        steps_tok, steps_H = w.tokens[:, ctx_len:], w.H[:, ctx_len:]
    else:
        w = small(3, B=16, T=6, layers=1, context_len=13)
        ctx, Hc = w.context, w.H_context
        steps_tok, steps_H = w.tokens, w.H
    lay = w.layers[0]
    L = eg.Layer(lay, w.dtype, DEV)
    S = ctx.shape[0]
    st = eg.DecodeState(S, 3, lay.branches, 9, lay.d, DEV)
    ost = orc.new_state(S, 3, lay.branches, 9, lay.d)
    chk = check_f32_layer if w.dtype == "f32" else check_bf16_layer

    def step(tok, Hn, ost, tag):
        H = eg.to_device(Hn, w.dtype, DEV)
        alpha, y = eg.forward(torch.from_numpy(np.ascontiguousarray(tok)).to(DEV), H, L, state=st,
                              want_alpha=True, want_y=True)
        ref = orc.forward(tok, Hn, lay, w.dtype, state=ost)
        chk(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.storage_to_f64(Hn, w.dtype), tag=tag)
        return ref["state"]

    ost = step(ctx, Hc, ost, "prefill")
    for t in range(steps_tok.shape[1]):
        ost = step(steps_tok[:, t:t + 1], steps_H[:, t:t + 1], ost, f"step{t}")
    assert np.array_equal(st.ids.cpu().numpy(), ost["ids"])
    assert np.array_equal(st.pos.cpu().numpy(), ost["pos"])
    conv = st.conv.cpu().numpy().astype(np.float64)          # [S, M, 9, d], slot p % 9
    pos = int(ost["pos"][0])
    chrono = np.stack([conv[:, :, (pos - 9 + i) % 9] for i in range(9)], axis=2)
    tol = 1e-5 if w.dtype == "f32" else 1e-2
    assert np.max(np.abs(chrono - ost["u"])) <= tol * np.max(np.abs(ost["u"]))


def test_hash_indices_full_size_single_branch():
    """T = 4096 tokens hashed into the full 10.3M-row tables: every index
    equals the oracle's (the layer forward at this size is compared on every
    token in test_gpu_fullsize.py)."""
    log("hash indices full-size single-branch")
    w = inputs.make_config(1)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    z_gpu = eg.hash_indices(dev_tokens(w), L).cpu().numpy()
    hp = lay.hash
    assert np.array_equal(z_gpu, orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, 3, hp.heads))


def test_graph_replays_match_eager():
    """The forward captured in a HIP graph gives, on every replay, exactly the
    eager result (the kernels are deterministic and issue no memsets)."""
    log("graph replay vs eager")
    w = small(1, B=2, T=150)
    L = eg.Layer(w.layers[0], "bf16", DEV)
    tok = dev_tokens(w)
    H0 = dev_H(w)
    ws = torch.empty(eg.forward_workspace(w.B, w.T, L), dtype=torch.uint8, device=DEV)
    ref = H0.clone()
    eg.forward(tok, ref, L, ws=ws)
    H = H0.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        eg.forward(tok, H, L, ws=ws, stream=s)
    for r in range(4):
        H.copy_(H0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(H.view(torch.int16), ref.view(torch.int16)), r
        other = H0.clone()
        eg.forward(tok, other, L, ws=ws)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))


# --------------------------------------------------------------------------
# Other conv widths and dilations (the LDS-tiled conv kernel)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,kw,dil,M,d,B,T", [("f32", 3, 2, 1, 64, 2, 40), ("bf16", 2, 1, 2, 128, 2, 33),
                                                  ("bf16", 8, 3, 1, 256, 1, 90), ("f32", 5, 6, 1, 64, 1, 70)])
def test_forward_other_conv_shapes(dtype, kw, dil, M, d, B, T):
    log(f"conv shape dtype={dtype} w={kw} dilation={dil} M={M} d={d}")
    w = small(0 if dtype == "f32" else 1, B=B, T=T, d=d, branches=M)
    lay = w.layers[0]
    lay.kernel_w, lay.dilation = kw, dil
    lay.conv_w = inputs.normal_f32(inputs.rng_for(98, kw, dil), M * d * kw, 0.1).reshape(M, d, kw)
    L = eg.Layer(lay, dtype, DEV)
    H = dev_H(w)
    alpha, y = eg.forward(dev_tokens(w), H, L, want_alpha=True, want_y=True)
    ref = orc.forward(w.tokens, w.H, lay, dtype)
    chk = check_f32_layer if dtype == "f32" else check_bf16_layer
    chk(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.storage_to_f64(w.H, dtype),
        tag=f"w{kw} dil{dil}")


def test_decode_other_conv_shape():
    """w = 3, dilation 2 (span 4): prefill then token-by-token decode equals the oracle."""
    log("decode conv w3 dil2")
    w = small(1, B=3, T=12, rows_per_table=997)
    lay = w.layers[0]
    lay.kernel_w, lay.dilation = 3, 2
    lay.conv_w = inputs.normal_f32(inputs.rng_for(99, 3, 2), lay.d * 3, 0.1).reshape(1, lay.d, 3)
    L = eg.Layer(lay, "bf16", DEV)
    st = eg.DecodeState(3, 3, 1, 4, lay.d, DEV)
    ost = orc.new_state(3, 3, 1, 4, lay.d)
    chunks = [(w.tokens[:, :7], w.H[:, :7])] + [(w.tokens[:, t:t + 1], w.H[:, t:t + 1]) for t in range(7, 12)]
    for ci, (tok, Hn) in enumerate(chunks):
        H = eg.to_device(Hn, "bf16", DEV)
        alpha, y = eg.forward(torch.from_numpy(np.ascontiguousarray(tok)).to(DEV), H, L, state=st,
                              want_alpha=True, want_y=True)
        ref = orc.forward(tok, Hn, lay, "bf16", state=ost)
        ost = ref["state"]
        check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(Hn),
                         tag=f"chunk{ci}")
