"""engram_forward_noalloc (the layer forward for callers that cannot allocate
device memory) against engram_forward on the same inputs: the same kernels
with the workspace in the library's scratch instead of the caller's, so H,
alpha and Y must be bit-identical; each call is also held to the bf16
tolerances against the oracle.  Calls follow each other on one GPU with
smaller inputs after larger ones, so a call never depends on what an earlier
call left in the shared scratch."""
import numpy as np
import pytest
import torch

from hashed_gram_embedding_amd import engram as eg
from hashed_gram_embedding_amd import inputs
from oracle import engram_oracle as orc

from parity import check_bf16_layer, log, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32 if a.element_size() == 4 else torch.int16),
                       b.view(torch.int32 if b.element_size() == 4 else torch.int16))


@pytest.mark.parametrize("mx", [False, True])
def test_noalloc_equals_forward_on_consecutive_calls(mx):
    for i, (B, T) in enumerate([(1, 4096), (2, 300), (1, 37)]):
        log(f"noalloc call {i}: B={B} T={T} mxfp8={mx}")
        w = inputs.make_config(1, B=B, T=T, rows_per_table=997)
        lay = w.layers[0]
        L = eg.Layer(lay, "bf16", DEV, mxfp8=mx)
        tok = torch.from_numpy(w.tokens).to(DEV)
        H_ref = eg.to_device(w.H, "bf16", DEV)
        H_na = H_ref.clone()
        a_ref, y_ref = eg.forward(tok, H_ref, L, want_alpha=True, want_y=True)
        a_na = torch.full_like(a_ref, float("nan"))
        y_na = torch.full_like(y_ref, float("nan"))
        eg.forward_noalloc(tok, H_na, L, alpha=a_na, y=y_na)
        torch.cuda.synchronize()
        assert _same(H_na, H_ref) and _same(a_na, a_ref) and _same(y_na, y_ref), f"call {i}"
        ref = orc.forward(w.tokens, w.H, lay, "bf16", gemm="mxfp8" if mx else "exact")
        check_bf16_layer(to_f64(a_na), ref["alpha"], to_f64(y_na), ref["Y"], to_f64(H_na), orc.bf16_to_f64(w.H),
                         tag=f"noalloc call {i}")


def test_noalloc_decode_state_equals_forward():
    """A 12-token prefill with a decode state, then three single-token steps:
    the no-allocation call advances its state exactly as engram_forward does."""
    log("noalloc decode")
    w = inputs.make_config(3, B=16, T=3, layers=1, context_len=12, rows_per_table=997)
    lay = w.layers[0]
    L = eg.Layer(lay, "bf16", DEV)
    st_ref = eg.DecodeState(16, 3, 1, 9, lay.d, DEV)
    st_na = eg.DecodeState(16, 3, 1, 9, lay.d, DEV)
    chunks = [(w.context, w.H_context)] + [(w.tokens[:, t:t + 1], w.H[:, t:t + 1]) for t in range(3)]
    for ci, (tk, Hn) in enumerate(chunks):
        tok = torch.from_numpy(np.ascontiguousarray(tk)).to(DEV)
        H_ref = eg.to_device(Hn, "bf16", DEV)
        H_na = H_ref.clone()
        eg.forward(tok, H_ref, L, state=st_ref)
        eg.forward_noalloc(tok, H_na, L, state=st_na)
        torch.cuda.synchronize()
        assert _same(H_na, H_ref), f"chunk {ci}"
        assert torch.equal(st_na.ids, st_ref.ids) and torch.equal(st_na.pos, st_ref.pos)
        assert _same(st_na.conv, st_ref.conv), f"chunk {ci}"
