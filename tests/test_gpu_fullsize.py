"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, on every token: the gathered rows bit for bit (MXFP8 codes
and scale bytes too), and alpha, Y and H_out element by element against the
oracle, sequence by sequence (the oracle runs each whole sequence)."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import bits_equal, check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def check_rows(e_dev, ref_e, mx, tag):
    """Gathered rows of one sequence: bf16 bit for bit, or the MXFP8 codes and
    scale bytes of the oracle's quantisation of its bf16 rows."""
    if not mx:
        assert bits_equal(to_f64(e_dev), ref_e), f"{tag}: gathered rows differ"
        return
    codes, scales = e_dev
    rq, rs = orc.quantize_mxfp8(ref_e)
    assert np.array_equal(codes.cpu().numpy(), rq), f"{tag}: MXFP8 codes differ"
    assert np.array_equal(scales.cpu().numpy(), rs), f"{tag}: MXFP8 scale bytes differ"


def run_and_check(w, lay, L, tag, mx=False):
    """engram_retrieve (rows) and engram_forward (alpha, Y, H_out) on the whole
    workload, then every sequence against the oracle."""
    B, T = w.B, w.T
    tok = torch.from_numpy(w.tokens).to(DEV)
    e = eg.rows_buffer(B, T, L, DEV)
    eg.retrieve(tok, L, e)
    H = eg.to_device(w.H, "bf16", DEV)
    alpha, y = eg.forward(tok, H, L, want_alpha=True, want_y=True)
    torch.cuda.synchronize()
    d_mem = lay.d_mem
    worst = [0.0, 0.0]
    for b in range(B):
        log(f"{tag}: oracle, sequence {b} of {B}")
        ref = orc.forward(w.tokens[b:b + 1], w.H[b:b + 1], lay, "bf16", gemm="mxfp8" if mx else "exact")
        if mx:
            n = B * T * d_mem
            codes = e[:n].view(B * T, d_mem)[b * T:(b + 1) * T]
            scales = e[n:].view(B * T, d_mem // 32)[b * T:(b + 1) * T]
            check_rows((codes, scales), ref["e"].reshape(T, d_mem), True, f"{tag} b{b}")
        else:
            check_rows(e[b * T:(b + 1) * T], ref["e"].reshape(T, d_mem), False, f"{tag} b{b}")
        da, dy = check_bf16_layer(to_f64(alpha[b:b + 1]), ref["alpha"], to_f64(y[b:b + 1]), ref["Y"],
                                  to_f64(H[b:b + 1]), orc.bf16_to_f64(w.H[b:b + 1]), tag=f"{tag} b{b}")
        worst = [max(worst[0], da), max(worst[1], dy)]
        del ref
    log(f"{tag}: all {B * T} tokens checked; worst alpha err {worst[0]:.2e}, worst Y err {worst[1]:.3f} of tol")


@pytest.mark.parametrize("mx", [False, True])
def test_single_branch_full_size_every_token(mx):
    """The single-branch workload the benchmark's headline line times: B = 1,
    T = 4096, the full 10.3M-row tables; bf16 and the MXFP8 product."""
    log(f"single-branch full size: inputs mxfp8={mx}")
    w = inputs.make_config(1)
    lay = w.layers[0]
    run_and_check(w, lay, eg.Layer(lay, "bf16", DEV, mxfp8=mx), f"c1 mx={mx}", mx)


@pytest.mark.parametrize("mx", [False, True])
def test_multi_branch_full_size_every_token(mx):
    """B = 8, T = 4096, M = 4 branches (shared W_V, four W_K^(m), per-branch
    gate and conv), the full 10.3M-row tables; bf16 and the MXFP8 product."""
    log(f"multi-branch full size: inputs mxfp8={mx}")
    w = inputs.make_config(2)
    lay = w.layers[0]
    run_and_check(w, lay, eg.Layer(lay, "bf16", DEV, mxfp8=mx), f"c2 mx={mx}", mx)


@pytest.mark.parametrize("mx", [False, True])
def test_decode_full_size_every_sequence(mx):
    """256 sequences, int8 rows with per-row scales (703 MB per layer), each
    of the 2 layers: a 16-token prefill with state, then 3 single-token decode
    steps; every sequence matches the oracle at every step, and the state's
    ids, positions and conv ring match (bf16 and the MXFP8 product)."""
    log(f"decode full size: inputs mxfp8={mx}")
    w = inputs.make_config(3, T=3)
    S = w.B
    for li, lay in enumerate(w.layers):
        log(f"decode full size: layer {li}")
        L = eg.Layer(lay, "bf16", DEV, mxfp8=mx)
        st = eg.DecodeState(S, 3, 1, 9, 1024, DEV)
        ost = orc.new_state(S, 3, 1, 9, 1024)
        chunks = [(w.context, w.H_context)] + [(w.tokens[:, t:t + 1], w.H[:, t:t + 1]) for t in range(3)]
        for ci, (tok, Hn) in enumerate(chunks):
            H = eg.to_device(Hn, "bf16", DEV)
            alpha, y = eg.forward(torch.from_numpy(np.ascontiguousarray(tok)).to(DEV), H, L, state=st,
                                  want_alpha=True, want_y=True)
            ref = orc.forward(tok, Hn, lay, "bf16", state=ost, gemm="mxfp8" if mx else "exact")
            ost = ref["state"]
            check_bf16_layer(to_f64(alpha), ref["alpha"], to_f64(y), ref["Y"], to_f64(H), orc.bf16_to_f64(Hn),
                             tag=f"layer{li} chunk{ci}")
        assert np.array_equal(st.ids.cpu().numpy(), ost["ids"])
        assert np.all(st.pos.cpu().numpy() == 16 + 3)
        conv = st.conv.cpu().numpy().astype(np.float64)           # [S, 1, 9, d], position p in slot p % 9
        pos = 16 + 3
        chrono = np.stack([conv[:, :, (pos - 9 + i) % 9] for i in range(9)], axis=2)
        assert np.max(np.abs(chrono - ost["u"])) <= 1e-2 * np.max(np.abs(ost["u"]))


def test_host_table_full_size_with_cache():
    """One layer of 33,556,876 bf16 rows (4.3 GB) in pinned host memory, an
    HBM cache of 10 % of the rows admitted from a 2^22-token warm-up (exact
    LFU ranking checked against the oracle), and a B = 4, T = 4096 forward
    that equals the HBM-table forward bit for bit and matches the oracle on
    every token."""
    log("host table full size: inputs")
    w = inputs.make_config(4, layers=1)
    lay = w.layers[0]
    tab = lay.tables
    hb = eg.HostBuffer(tab.rows.nbytes)
    try:
        hb.numpy(tab.rows.dtype, tab.rows.shape)[:] = tab.rows
        L = eg.Layer(lay, "bf16", DEV, rows_ptr=hb.dev)
        warm = inputs.lfu_warmup_tokens(4, 0, n=1 << 22).reshape(16, -1)
        n_cache = tab.total_rows // 10
        log("host table full size: cache build")
        slot, rows, _ = eg.cache_build(torch.from_numpy(warm).to(DEV), L, n_cache)
        hp = lay.hash
        z = orc.hash_indices(warm, hp.proj, hp.mult, hp.prime, 3, hp.heads)
        ref_slot = orc.lfu_admission(z + tab.row_offset, tab.total_rows, n_cache)
        assert np.array_equal(slot.cpu().numpy(), ref_slot)
        L.set_cache(slot, rows)
        tok = torch.from_numpy(w.tokens).to(DEV)
        H0 = eg.to_device(w.H, "bf16", DEV)
        H2 = H0.clone()
        L_dev = eg.Layer(lay, "bf16", DEV)
        eg.forward(tok, H2, L_dev)
        log("host table full size: forward through the cache, every token against the oracle")
        run_and_check(w, lay, L, "c4")
        H = H0.clone()
        eg.forward(tok, H, L)
        torch.cuda.synchronize()
        assert torch.equal(H.view(torch.int16), H2.view(torch.int16))
        del L_dev
    finally:
        torch.cuda.synchronize()
        hb.free()
