"""GPU: the MXFP8 Step 5 (the Guide's FP8 fused W_V / W_K product).  The
quantiser and the gather's MXFP8 output are bit-exact against the oracle;
the layer with the FP8 product matches the oracle's MXFP8 forward at the
bf16 tolerances (only the float32 accumulation order differs)."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_bit_exact(dtype):
    log(f"mxfp8 quantize {dtype}")
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((70, 256)) * np.exp2(rng.integers(-30, 30, (70, 1)))).astype(np.float32)
    x[3, :32] = 0.0                          # all-zero block
    x[4, 32:64] = 0.0
    x[4, 40] = 448.0                         # amax exactly 448: scale byte 127
    x[5, :32] = rng.standard_normal(32).astype(np.float32) * 1e-3
    x[5, 7] = np.float32(-449.0) * 2.0 ** -20
    x[6, :] = 2.0 ** -140                    # float32 subnormals
    if dtype == "bf16":
        xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
        x64 = xt.float().cpu().numpy().astype(np.float64)
    else:
        xt = torch.from_numpy(x).to(DEV)
        x64 = x.astype(np.float64)
    q = torch.empty((70, 256), dtype=torch.uint8, device=DEV)
    s = torch.empty((70, 8), dtype=torch.uint8, device=DEV)
    eg.quantize_mxfp8(xt, q, s)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_mxfp8(x64)
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


def _mx_layer(config, **kw):
    w = inputs.make_config(config, rows_per_table=997, **kw)
    lay = w.layers[0]
    return w, lay, eg.Layer(lay, "bf16", DEV, mxfp8=True)


@pytest.mark.parametrize("config", [1, 3])
def test_retrieve_emits_mxfp8_rows_bit_exact(config):
    """MXFP8 codes and scale bytes of the gathered rows equal the oracle's
    quantisation of the bf16 rows (bf16 tables, and int8 tables whose rows are
    dequantised and rounded to bf16 first)."""
    log(f"mxfp8 gather config={config}")
    w, lay, L = _mx_layer(config, B=2, T=90)
    assert lay.tables.dtype == ("i8" if config == 3 else "bf16")
    tok = torch.from_numpy(w.tokens).to(DEV)
    e = eg.rows_buffer(2, 90, L, DEV)
    eg.retrieve(tok, L, e)
    torch.cuda.synchronize()
    hp, tab = lay.hash, lay.tables
    z = orc.hash_indices(w.tokens, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads)
    ref = orc.gather(z, tab.rows, tab.dtype, tab.row_offset, tab.dim, tab.scale, out_dtype="bf16").reshape(180, -1)
    rq, rs = orc.quantize_mxfp8(ref)
    got = e.cpu().numpy()
    n = ref.size
    assert np.array_equal(got[:n].reshape(rq.shape), rq)
    assert np.array_equal(got[n:n + n // 32].reshape(rs.shape), rs)


@pytest.mark.parametrize("config,B,T", [(1, 2, 300), (1, 1, 5), (2, 2, 130), (1, 3, 700)])
def test_forward_mxfp8_matches_oracle(config, B, T):
    log(f"mxfp8 forward config={config} B={B} T={T}")
    w, lay, L = _mx_layer(config, B=B, T=T)
    tok = torch.from_numpy(w.tokens).to(DEV)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True)
    torch.cuda.synchronize()
    ref = orc.forward(w.tokens, w.H, lay, "bf16", gemm="mxfp8")
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H),
                     tag=f"mxfp8 c{config}")


# Narrower tables (16 x 32 dims: K = 512, four 128-code slices of the FP8
# product; MXFP8 rows need whole 32-value blocks, so 32 dims is the narrowest).
@pytest.mark.parametrize("config,B,T", [(1, 1, 300), (2, 1, 200)])
def test_forward_mxfp8_narrow_tables(config, B, T):
    log(f"mxfp8 forward narrow tables config={config} B={B} T={T}")
    w, lay, L = _mx_layer(config, B=B, T=T, table_dim=32)
    tok = torch.from_numpy(w.tokens).to(DEV)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True)
    torch.cuda.synchronize()
    ref = orc.forward(w.tokens, w.H, lay, "bf16", gemm="mxfp8")
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H),
                     tag=f"mxfp8 narrow c{config}")


@pytest.mark.parametrize("config", [1, 2])
def test_decode_mxfp8_matches_oracle(config):
    """A 7-token prefill with a decode state, then 5 single-token steps, with
    the FP8 product (one ragged token tile per call); every call matches the
    oracle's MXFP8 forward carrying the same state."""
    log(f"mxfp8 decode config={config}")
    w, lay, L = _mx_layer(config, B=3, T=12)
    M, d = lay.branches, lay.d
    st = eg.DecodeState(3, 3, M, 9, d, DEV)
    ost = orc.new_state(3, 3, M, 9, d)
    chunks = [(w.tokens[:, :7], w.H[:, :7])] + [(w.tokens[:, t:t + 1], w.H[:, t:t + 1]) for t in range(7, 12)]
    for ci, (tok, Hn) in enumerate(chunks):
        H = eg.to_device(Hn, "bf16", DEV)
        alpha, y = eg.forward(torch.from_numpy(np.ascontiguousarray(tok)).to(DEV), H, L, state=st,
                              want_alpha=True, want_y=True)
        ref = orc.forward(tok, Hn, lay, "bf16", state=ost, gemm="mxfp8")
        ost = ref["state"]
        check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(Hn),
                         tag=f"mxfp8 decode c{config} chunk{ci}")


def test_pack_mxfp8_layout():
    """engram_pack_mxfp8 writes the operand order that include/engram.h
    documents, built here index by index from the codes and scales."""
    log("mxfp8 pack layout")
    rng = np.random.default_rng(37)
    rows, cols = 96, 768
    q = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    s = rng.integers(0, 256, (rows, cols // 32), dtype=np.uint8)
    packed = torch.empty(rows * cols + rows * cols // 32, dtype=torch.uint8, device=DEV)
    eg.pack_mxfp8(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), packed)
    got = packed.cpu().numpy()
    kk_n = cols // 64
    want = np.empty(rows * cols + rows * cols // 32, dtype=np.uint8)
    for b in range(rows // 32):
        for kk in range(kk_n):
            for lane in range(64):
                row, h = 32 * b + (lane & 31), lane >> 5
                o = ((b * kk_n + kk) * 64 + lane) * 32
                want[o:o + 16] = q[row, 64 * kk + 16 * h:64 * kk + 16 * h + 16]
                want[o + 16:o + 32] = q[row, 64 * kk + 32 + 16 * h:64 * kk + 48 + 16 * h]
        for kq in range(kk_n // 4):
            for lane in range(64):
                row, h = 32 * b + (lane & 31), lane >> 5
                o = rows * cols + ((b * (kk_n // 4) + kq) * 64 + lane) * 4
                for st in range(4):
                    want[o + st] = s[row, 2 * (4 * kq + st) + h]
    assert np.array_equal(got, want)


def _forward(w, L, **kw):
    tok = torch.from_numpy(w.tokens).to(DEV)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True, **kw)
    torch.cuda.synchronize()
    return H, alpha, y


# Token counts that give the resident-token FP8 product enough token tiles
# (at most a quarter of the 256-column passes per workgroup), each with a
# ragged last tile, at every K it is built for.
RESIDENT_CASES = [
    ("K1024 M4", lambda: inputs.make_config(2, B=2, T=3500, rows_per_table=997)),
    ("K512 M4", lambda: inputs.make_config(2, B=2, T=3500, rows_per_table=997, table_dim=32)),
    ("K768 M2", lambda: inputs.make_shape(1, 11000, heads=6, dim=64, d=1024, branches=2)),
    ("K256 M3", lambda: inputs.make_shape(2, 8200, heads=4, dim=32, d=512, branches=3)),
]


@pytest.mark.parametrize("name,make", RESIDENT_CASES, ids=[c[0] for c in RESIDENT_CASES])
def test_resident_fp8_product_is_bit_identical(name, make):
    """With the packed W, multi-branch FP8 layers run the resident-token
    product, whose v and gate sums are formed in the same order as the 128 x
    256 tile kernel's: H, alpha and Y equal the layer without the packed W
    bit for bit, and match the oracle's MXFP8 forward.  A packed W of zeros
    changes the result, so the packed path is the one that ran."""
    log(f"resident fp8 product {name}")
    w = make()
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV, mxfp8=True)
    assert L.w_mx_packed is not None
    L0 = eg.Layer(lay, "bf16", DEV, mxfp8=True, mx_packed=False)
    H, alpha, y = _forward(w, L)
    H0, alpha0, y0 = _forward(w, L0)
    assert torch.equal(H, H0) and torch.equal(alpha, alpha0) and torch.equal(y, y0), name
    zero = torch.zeros_like(L.w_mx_packed)
    L.s.w_mx_packed = zero.data_ptr()
    Hz, _, _ = _forward(w, L)
    assert not torch.equal(Hz, H0), f"{name}: the packed W was not read"
    L.s.w_mx_packed = L.w_mx_packed.data_ptr()
    log(f"{name}: oracle")
    ref = orc.forward(w.tokens, w.H, lay, "bf16", gemm="mxfp8")
    check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(w.H),
                     tag=f"resident {name}")


def test_resident_fp8_decode_with_state_is_bit_identical():
    """A multi-branch FP8 decode over 6,600 sequences (a 3-token prefill, then
    single tokens) runs the resident-token product, the single-token steps
    with the decode state's advance folded into that launch: H, alpha, Y and
    the whole state equal the run without the packed W bit for bit, and the
    first sequences match the oracle carrying the same state."""
    S, T = 6600, 5
    log(f"resident fp8 decode S={S}")
    w = inputs.make_config(2, B=S, T=T, rows_per_table=997)
    lay = w.layers[0]
    M, d = lay.branches, lay.d
    L = eg.Layer(lay, "bf16", DEV, mxfp8=True)
    L0 = eg.Layer(lay, "bf16", DEV, mxfp8=True, mx_packed=False)
    st, st0 = eg.DecodeState(S, 3, M, 9, d, DEV), eg.DecodeState(S, 3, M, 9, d, DEV)
    ns = 4
    ost = orc.new_state(ns, 3, M, 9, d)
    chunks = [(0, 3), (3, 4), (4, 5)]
    for a, b in chunks:
        tok = torch.from_numpy(np.ascontiguousarray(w.tokens[:, a:b])).to(DEV)
        Hn = np.ascontiguousarray(w.H[:, a:b])
        H, H0 = eg.to_device(Hn, "bf16", DEV), eg.to_device(Hn, "bf16", DEV)
        alpha, y = eg.forward(tok, H, L, state=st, want_alpha=True, want_y=True)
        alpha0, y0 = eg.forward(tok, H0, L0, state=st0, want_alpha=True, want_y=True)
        torch.cuda.synchronize()
        tag = f"tokens {a}..{b}"
        assert torch.equal(H, H0) and torch.equal(alpha, alpha0) and torch.equal(y, y0), tag
        assert torch.equal(st.ids, st0.ids) and torch.equal(st.conv, st0.conv) and torch.equal(st.pos, st0.pos), tag
        ref = orc.forward(w.tokens[:ns, a:b], Hn[:ns], lay, "bf16", state=ost, gemm="mxfp8")
        ost = ref["state"]
        check_bf16_layer(to_f64(alpha[:ns]), ref["alpha"], to_f64(y[:ns]), ref["Y"], to_f64(H[:ns]),
                         orc.bf16_to_f64(Hn[:ns]), tag=f"resident decode {tag}")
