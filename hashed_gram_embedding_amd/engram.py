"""ctypes binding of libengram.so (C ABI in include/engram.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the layer runs in the library's kernels.
There is no fallback: if the library is missing or a call fails, an error is
raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ENGRAM_DEBUG_CHECKS=1 in the environment loads the debug build instead
# (device-resident preconditions checked into an error word).
LIB_PATH = os.path.join(_HERE, "libengram_debug.so" if os.environ.get("ENGRAM_DEBUG_CHECKS") == "1"
                        else "libengram.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, -1, -2, -3
F32, BF16, I8 = 0, 1, 2
MAX_TABLES, MAX_ORDER = 32, 4
MAX_D, MAX_BRANCHES = 65536, 64

_DT = {"f32": F32, "bf16": BF16, "i8": I8}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8}

c_i32p = ctypes.POINTER(ctypes.c_int32)


class HashParams(ctypes.Structure):
    _fields_ = [("proj", ctypes.c_void_p), ("vocab", ctypes.c_int64), ("max_n", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("mult", ctypes.c_void_p), ("prime", ctypes.c_void_p)]


class Tables(ctypes.Structure):
    _fields_ = [("n_tables", ctypes.c_int32), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rows", ctypes.c_void_p), ("row_offset", ctypes.c_void_p), ("n_rows", ctypes.c_void_p),
                ("total_rows", ctypes.c_int64), ("row_scale", ctypes.c_void_p),
                ("cache_slot", ctypes.c_void_p), ("cache_rows", ctypes.c_void_p),
                ("cache_scale", ctypes.c_void_p), ("cache_n", ctypes.c_int64),
                ("access_counts", ctypes.c_void_p)]


class GateConvParams(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("branches", ctypes.c_int32), ("kernel_w", ctypes.c_int32),
                ("dilation", ctypes.c_int32), ("eps", ctypes.c_float), ("hdtype", ctypes.c_int32),
                ("conv_w", ctypes.c_void_p)]


class HotTierStruct(ctypes.Structure):
    _fields_ = [("n_hot", ctypes.c_int64 * (MAX_ORDER - 1)), ("seed", ctypes.c_uint64 * (MAX_ORDER - 1)),
                ("pilots", ctypes.c_void_p * (MAX_ORDER - 1)), ("slots", ctypes.c_void_p * (MAX_ORDER - 1)),
                ("rows", ctypes.c_void_p * (MAX_ORDER - 1))]


class LayerStruct(ctypes.Structure):
    _fields_ = [("hash", HashParams), ("tables", Tables), ("w", ctypes.c_void_p), ("gc", GateConvParams),
                ("w_mx", ctypes.c_void_p), ("w_mx_scale", ctypes.c_void_p), ("w_mx_packed", ctypes.c_void_p),
                ("w_packed", ctypes.c_void_p), ("hot", ctypes.POINTER(HotTierStruct))]


class DecodeStateStruct(ctypes.Structure):
    _fields_ = [("ids", ctypes.c_void_p), ("conv", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


_lib = None


class EngramError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"engram status {status}: {msg}")
        self.status = status


def lib():
    """Load libengram.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """A build of the library (release or debug) with every entry point's
    signature set; raises if it has not been built."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m hashed_gram_embedding_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "engram_abi_version": (i32, []),
        "engram_last_error": (ctypes.c_char_p, []),
        "engram_hash_indices": (i32, [vp, i64, i64, vp, ctypes.POINTER(HashParams), vp, vp]),
        "engram_gather": (i32, [vp, i64, ctypes.POINTER(Tables), i32, vp, vp]),
        "engram_project_kv": (i32, [vp, vp, i64, i64, i64, i32, vp, vp]),
        "engram_gate_conv_workspace": (sz, [i64, i64, ctypes.POINTER(GateConvParams)]),
        "engram_gate_conv_forward": (i32, [vp, vp, i64, i64, ctypes.POINTER(GateConvParams),
                                           ctypes.POINTER(DecodeStateStruct), vp, vp, vp, sz, vp]),
        "engram_forward_workspace": (sz, [i64, i64, ctypes.POINTER(LayerStruct)]),
        "engram_forward": (i32, [vp, vp, i64, i64, ctypes.POINTER(LayerStruct),
                                 ctypes.POINTER(DecodeStateStruct), vp, vp, vp, sz, vp]),
        "engram_forward_noalloc": (i32, [vp, vp, i64, i64, ctypes.POINTER(LayerStruct),
                                         ctypes.POINTER(DecodeStateStruct), vp, vp, vp]),
        "engram_retrieve": (i32, [vp, i64, i64, ctypes.POINTER(LayerStruct), ctypes.POINTER(DecodeStateStruct), vp,
                                  vp]),
        "engram_forward_retrieved_workspace": (sz, [i64, i64, ctypes.POINTER(LayerStruct)]),
        "engram_forward_retrieved": (i32, [vp, vp, vp, i64, i64, ctypes.POINTER(LayerStruct),
                                           ctypes.POINTER(DecodeStateStruct), vp, vp, vp, sz, vp]),
        "engram_quantize_mxfp8": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "engram_pack_mxfp8": (i32, [vp, vp, i64, i64, vp, vp]),
        "engram_pack_bf16": (i32, [vp, i64, i64, vp, vp]),
        "engram_project_ahead_workspace": (sz, [i64, i64, i32, ctypes.POINTER(ctypes.POINTER(LayerStruct))]),
        "engram_project_ahead": (i32, [vp, i64, i64, i32, ctypes.POINTER(ctypes.POINTER(LayerStruct)),
                                       ctypes.POINTER(ctypes.POINTER(DecodeStateStruct)), ctypes.POINTER(vp), vp, sz,
                                       vp]),
        "engram_forward_projected_workspace": (sz, [i64, i64, ctypes.POINTER(LayerStruct)]),
        "engram_forward_projected": (i32, [vp, vp, i64, i64, ctypes.POINTER(LayerStruct),
                                           ctypes.POINTER(DecodeStateStruct), vp, vp, vp, sz, vp]),
        "engram_forward_retrieved_prefetch": (i32, [vp, vp, vp, i64, i64, ctypes.POINTER(LayerStruct),
                                                    ctypes.POINTER(DecodeStateStruct), vp, vp, vp, sz,
                                                    ctypes.POINTER(LayerStruct), ctypes.POINTER(DecodeStateStruct),
                                                    vp, i64, i64, vp, vp]),
        "engram_cache_update_workspace": (sz, [i64, i64]),
        "engram_cache_update": (i32, [ctypes.POINTER(Tables), i64, vp, vp, vp, vp, i32, vp, sz, vp]),
        "engram_cache_build_workspace": (sz, [i64]),
        "engram_cache_build": (i32, [vp, i64, i64, ctypes.POINTER(HashParams), ctypes.POINTER(Tables), i64, vp, vp, vp,
                                     vp, sz, vp]),
        "engram_hot_buckets": (sz, [i64]),
        "engram_hot_build": (i32, [vp, i64, i32, ctypes.c_uint64, vp, vp, ctypes.POINTER(ctypes.c_uint64)]),
        "engram_hot_lookup": (i32, [vp, i64, i64, vp, ctypes.POINTER(HashParams), ctypes.POINTER(HotTierStruct),
                                    vp, vp]),
        "engram_profile_enable": (i32, [i32]),
        "engram_profile_read": (i32, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), i32,
                                      ctypes.POINTER(i32)]),
        "engram_host_alloc": (i32, [sz, ctypes.POINTER(vp), ctypes.POINTER(vp)]),
        "engram_debug_checks": (i32, []),
        "engram_debug_set_error_word": (i32, [vp]),
        "engram_debug_read_errors": (i32, [ctypes.POINTER(ctypes.c_uint32)]),
        "engram_host_free": (i32, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def exported_names():
    return ["engram_abi_version", "engram_last_error", "engram_hash_indices", "engram_gather",
            "engram_project_kv", "engram_gate_conv_workspace", "engram_gate_conv_forward",
            "engram_forward_workspace", "engram_forward", "engram_forward_noalloc", "engram_retrieve", "engram_forward_retrieved_workspace",
            "engram_forward_retrieved", "engram_cache_build_workspace", "engram_cache_build",
            "engram_cache_update_workspace", "engram_cache_update", "engram_quantize_mxfp8", "engram_pack_mxfp8",
            "engram_pack_bf16",
            "engram_project_ahead_workspace", "engram_project_ahead", "engram_forward_projected_workspace",
            "engram_forward_projected",
            "engram_hot_buckets", "engram_hot_build", "engram_hot_lookup", "engram_forward_retrieved_prefetch",
            "engram_profile_enable", "engram_profile_read",
            "engram_host_alloc", "engram_host_free", "engram_debug_checks", "engram_debug_set_error_word",
            "engram_debug_read_errors"]


def last_error() -> str:
    return lib().engram_last_error().decode()


def _check(status: int):
    if status != OK:
        raise EngramError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def to_device(a: np.ndarray, kind: str, device) -> torch.Tensor:
    """numpy array -> device tensor; kind "bf16" reinterprets uint16 bits."""
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# --------------------------------------------------------------------------
# device-side layer description
# --------------------------------------------------------------------------

class HashSpec:
    """Device copy of P plus the host arrays of the hash parameters."""

    def __init__(self, hp, device="cuda"):
        self.hp = hp
        self.proj = to_device(np.asarray(hp.proj, dtype=np.int32), "i32", device)
        self.mult = np.ascontiguousarray(hp.mult, dtype=np.uint64)
        self.prime = np.ascontiguousarray(hp.prime, dtype=np.uint32)
        self.n_tables = (hp.max_n - 1) * hp.heads
        self.s = HashParams(self.proj.data_ptr(), hp.vocab, hp.max_n, hp.heads,
                            self.mult.ctypes.data, self.prime.ctypes.data)


class Layer:
    """Device copies of one layer's parameters plus the ctypes descriptor.

    Tables live in HBM unless `host_rows` is given: then `rows` must already
    be the device alias of pinned host memory from HostBuffer."""

    def __init__(self, li, hdtype: str, device="cuda", rows_device: Optional[torch.Tensor] = None,
                 rows_ptr: Optional[int] = None, scale_ptr: Optional[int] = None, mxfp8: bool = False,
                 mx_packed: bool = True, bf16_packed: bool = True):
        hp, tab = li.hash, li.tables
        self.li = li
        self.hdtype = _DT[hdtype]
        self.hs = HashSpec(hp, device)
        self.row_offset = np.ascontiguousarray(tab.row_offset, dtype=np.int64)
        self.n_rows = np.ascontiguousarray(tab.n_rows, dtype=np.int64)
        self.table_dtype = _DT[tab.dtype]
        if rows_ptr is None:
            self.rows = rows_device if rows_device is not None else to_device(tab.rows, tab.dtype, device)
            rows_ptr = self.rows.data_ptr()
            self.scale = None
            if tab.dtype == "i8":
                self.scale = to_device(tab.scale.astype(np.float32), "f32", device)
                scale_ptr = self.scale.data_ptr()
        self.w = to_device(li.w, "bf16" if hdtype == "bf16" else "f32", device)
        self.conv_w = to_device(li.conv_w.astype(np.float32), "f32", device)
        self.cache_slot = self.cache_rows = self.cache_scale = None
        self.access_counts = None
        self.hot = None
        self.cache_n = 0
        self.s = LayerStruct()
        self.s.hash = self.hs.s
        self.s.tables = Tables(tab.n_rows.shape[0], tab.dim, self.table_dtype, rows_ptr,
                               self.row_offset.ctypes.data, self.n_rows.ctypes.data, tab.total_rows,
                               scale_ptr, None, None, None, 0)
        self.s.w = self.w.data_ptr()
        self.s.gc = GateConvParams(li.d, li.branches, li.kernel_w, li.dilation, li.eps, self.hdtype,
                                   self.conv_w.data_ptr())
        self.w_packed = None
        if bf16_packed and hdtype == "bf16" and self.w.shape[0] % 32 == 0 and self.w.shape[1] % 16 == 0:
            # the fragment-ordered copy that the decode-size product loads into registers
            self.w_packed = torch.empty_like(self.w)
            pack_bf16(self.w, self.w_packed)
            self.s.w_packed = self.w_packed.data_ptr()
        self.mxfp8 = mxfp8
        if mxfp8:
            n, k = self.w.shape
            self.w_mx = torch.empty((n, k), dtype=torch.uint8, device=device)
            self.w_mx_scale = torch.empty((n, k // 32), dtype=torch.uint8, device=device)
            quantize_mxfp8(self.w, self.w_mx, self.w_mx_scale)
            self.s.w_mx = self.w_mx.data_ptr()
            self.s.w_mx_scale = self.w_mx_scale.data_ptr()
            self.w_mx_packed = None
            if mx_packed and n % 32 == 0 and k % 256 == 0:
                # the fragment-ordered copy that the resident-token FP8 kernel streams
                self.w_mx_packed = torch.empty(n * k + n * k // 32, dtype=torch.uint8, device=device)
                pack_mxfp8(self.w_mx, self.w_mx_scale, self.w_mx_packed)
                self.s.w_mx_packed = self.w_mx_packed.data_ptr()

    def set_cache(self, slot: Optional[torch.Tensor], rows: Optional[torch.Tensor],
                  scale: Optional[torch.Tensor] = None):
        self.cache_slot, self.cache_rows, self.cache_scale = slot, rows, scale
        t = self.s.tables
        t.cache_slot = None if slot is None else slot.data_ptr()
        t.cache_rows = None if rows is None else rows.data_ptr()
        t.cache_scale = None if scale is None else scale.data_ptr()
        self.cache_n = 0 if rows is None else rows.shape[0]
        t.cache_n = self.cache_n

    def set_hot(self, hot: Optional["HotTier"]):
        """Attach an Engram-Nine hot tier (built for this layer's K and dim) or
        detach it (None)."""
        if hot is not None:
            width = self.li.hash.heads * self.li.tables.dim
            for n, k in hot.keys.items():
                r = hot.rows.get(n)
                if r is None or r.dtype != _TORCH_DT[self.table_dtype] or tuple(r.shape) != (k.shape[0], width) \
                        or not r.is_contiguous():
                    raise ValueError(f"hot rows of order {n} must be a contiguous {_TORCH_DT[self.table_dtype]} "
                                     f"tensor [{k.shape[0]}, {width}]")
        self.hot = hot
        self.s.hot = None if hot is None else ctypes.pointer(hot.s)

    def set_access_counts(self, counts: Optional[torch.Tensor]):
        """Per-row access counts (uint32 as int32 [total_rows]) that every gather
        through this layer increments; None stops counting."""
        self.access_counts = counts
        self.s.tables.access_counts = None if counts is None else counts.data_ptr()

    @property
    def M(self):
        return self.li.branches

    @property
    def d(self):
        return self.li.d

    @property
    def d_mem(self):
        return self.li.tables.dim * self.li.tables.n_rows.shape[0]


def hot_build(keys: np.ndarray, seed: int = 0):
    """Minimal perfect hash of one order's hot n-grams (host only).

    keys: int [n_hot, n], n-gram r oldest id first.  Returns (pilots uint32
    [engram_hot_buckets(n_hot)], slots int32 [n_hot, 8], seed_used)."""
    keys = np.ascontiguousarray(keys, dtype=np.int32)
    n_hot, n = keys.shape
    pilots = np.zeros(max(int(lib().engram_hot_buckets(n_hot)), 1), dtype=np.uint32)
    slots = np.zeros((max(n_hot, 1), 8), dtype=np.int32)
    used = ctypes.c_uint64(0)
    _check(lib().engram_hot_build(keys.ctypes.data, n_hot, n, ctypes.c_uint64(seed), pilots.ctypes.data,
                                  slots.ctypes.data, ctypes.byref(used)))
    return pilots, slots, int(used.value)


class HotTier:
    """Device copy of an Engram-Nine hot tier: per order n, the hot n-grams
    (keys[n]: int [n_hot, n], oldest id first) and their rows (rows[n]: a
    device tensor [n_hot, K*dim] of the cold tables' dtype, row r for key r).
    Orders absent from `keys` have no hot set."""

    def __init__(self, keys: dict, rows: Optional[dict] = None, seed: int = 0, device="cuda"):
        self.s = HotTierStruct()
        self.pilots, self.slots, self.rows, self.keys = {}, {}, {}, {}
        for n, k in keys.items():
            k = np.ascontiguousarray(k, dtype=np.int32).reshape(-1, n)
            if k.shape[0] == 0:
                continue
            pilots, slots, used = hot_build(k, seed)
            o = n - 2
            self.keys[n] = k
            self.pilots[n] = to_device(pilots.view(np.int32), "i32", device)
            self.slots[n] = to_device(slots, "i32", device)
            self.s.n_hot[o] = k.shape[0]
            self.s.seed[o] = used
            self.s.pilots[o] = self.pilots[n].data_ptr()
            self.s.slots[o] = self.slots[n].data_ptr()
            if rows is not None:
                r = rows[n]
                assert r.is_contiguous() and r.shape[0] == k.shape[0]
                self.rows[n] = r
                self.s.rows[o] = r.data_ptr()


class DecodeState:
    """Zero-initialised decode state for S sequences (see engram_decode_state)."""

    def __init__(self, S: int, max_n: int, branches: int, span: int, d: int, device="cuda"):
        self.ids = torch.zeros((S, max_n - 1), dtype=torch.int32, device=device)
        self.conv = torch.zeros((S, branches, span, d), dtype=torch.float32, device=device)
        self.pos = torch.zeros(S, dtype=torch.int32, device=device)
        self.s = DecodeStateStruct(self.ids.data_ptr(), self.conv.data_ptr(), self.pos.data_ptr())


class HostBuffer:
    """Pinned, mapped host memory readable by kernels (engram_host_alloc)."""

    def __init__(self, nbytes: int):
        h, d = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().engram_host_alloc(nbytes, ctypes.byref(h), ctypes.byref(d)))
        self.host, self.dev, self.nbytes = h.value, d.value, nbytes

    def numpy(self, dtype, shape):
        buf = (ctypes.c_char * self.nbytes).from_address(self.host)
        return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(shape)

    def free(self):
        if self.host:
            _check(lib().engram_host_free(ctypes.c_void_p(self.host)))
            self.host = self.dev = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# --------------------------------------------------------------------------
# entry points (same names as the C ABI, minus the prefix)
# --------------------------------------------------------------------------

def hash_indices(tokens: torch.Tensor, spec, hist: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """spec: a HashSpec or a Layer."""
    hs = spec.hs if isinstance(spec, Layer) else spec
    B, T = tokens.shape
    if z is None:
        z = torch.empty((B, T, hs.n_tables), dtype=torch.int32, device=tokens.device)
    _check(lib().engram_hash_indices(_ptr(tokens), B, T, _ptr(hist), ctypes.byref(hs.s),
                                     _ptr(z), _stream(stream)))
    return z


def gather(z: torch.Tensor, layer: Layer, out_dtype: str = "bf16", e: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    nt, dim = layer.s.tables.n_tables, layer.s.tables.dim
    n_tok = z.numel() // nt
    if e is None:
        e = torch.empty((*z.shape[:-1], nt * dim), dtype=_TORCH_DT[_DT[out_dtype]], device=z.device)
    _check(lib().engram_gather(_ptr(z), n_tok, ctypes.byref(layer.s.tables), _DT[out_dtype], _ptr(e),
                               _stream(stream)))
    return e


def project_kv(e: torch.Tensor, w: torch.Tensor, kv: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    d_mem = e.shape[-1]
    n_tok = e.numel() // d_mem
    n_out = w.shape[0]
    dt = BF16 if e.dtype == torch.bfloat16 else F32
    if kv is None:
        kv = torch.empty((*e.shape[:-1], n_out), dtype=e.dtype, device=e.device)
    _check(lib().engram_project_kv(_ptr(e), _ptr(w), n_tok, d_mem, n_out, dt, _ptr(kv), _stream(stream)))
    return kv


def gate_conv_forward(H: torch.Tensor, kv: torch.Tensor, layer: Layer, state: Optional[DecodeState] = None,
                      want_alpha: bool = False, want_y: bool = False, stream=None):
    B, T = H.shape[0], H.shape[1]
    M, d = layer.M, layer.d
    alpha = torch.empty((B, T, M), dtype=torch.float32, device=H.device) if want_alpha else None
    y = torch.empty((B, T, M, d), dtype=torch.float32, device=H.device) if want_y else None
    nbytes = lib().engram_gate_conv_workspace(B, T, ctypes.byref(layer.s.gc))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=H.device)
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_gate_conv_forward(_ptr(H), _ptr(kv), B, T, ctypes.byref(layer.s.gc), st,
                                          _ptr(alpha), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return alpha, y


def cache_build(warm_tokens: torch.Tensor, layer: Layer, cache_n: int, stream=None):
    """Static LFU admission: returns (cache_slot [total_rows] int32, cache_rows, cache_scale or None)
    on the device of warm_tokens; attach them with layer.set_cache(...)."""
    dev = warm_tokens.device
    t = layer.s.tables
    total = t.total_rows
    slot = torch.empty(total, dtype=torch.int32, device=dev)
    elt = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8}[t.dtype]
    rows = torch.empty((max(cache_n, 1), t.dim), dtype=elt, device=dev)
    scale = torch.empty(max(cache_n, 1), dtype=torch.float32, device=dev) if t.dtype == I8 else None
    ws = torch.empty(max(lib().engram_cache_build_workspace(total), 256), dtype=torch.uint8, device=dev)
    B, T = warm_tokens.shape
    tab = Tables.from_buffer_copy(t)
    tab.cache_slot = None
    _check(lib().engram_cache_build(_ptr(warm_tokens), B, T, ctypes.byref(layer.s.hash), ctypes.byref(tab), cache_n,
                                    _ptr(slot), _ptr(rows), _ptr(scale), _ptr(ws), ws.numel(), _stream(stream)))
    return slot, rows, scale


def cache_update(layer: Layer, counts: torch.Tensor, decay_shift: int = 0, stream=None):
    """Real-time LFU update of the layer's attached cache (set_cache) from the
    access counts; the slot map and cache rows are updated in place."""
    t = layer.s.tables
    n = layer.cache_n
    ws = torch.empty(max(lib().engram_cache_update_workspace(t.total_rows, n), 256), dtype=torch.uint8,
                     device=counts.device)
    _check(lib().engram_cache_update(ctypes.byref(t), n, _ptr(layer.cache_slot), _ptr(layer.cache_rows),
                                     _ptr(layer.cache_scale), _ptr(counts), decay_shift, _ptr(ws), ws.numel(),
                                     _stream(stream)))


def profile_enable(on=True):
    """on = True / 1: keep the stages of the last call; 2: accumulate the
    stages of back-to-back calls until profile_read; False / 0: off."""
    _check(lib().engram_profile_enable(int(on)))


PROFILE_MAX_STAGES = 2048


def profile_read():
    """[(kernel name, ms)] of the recorded stages (mode 1: the last profiled
    call; mode 2: every call since the previous read)."""
    cap = PROFILE_MAX_STAGES
    ms = (ctypes.c_float * cap)()
    names = (ctypes.c_char_p * cap)()
    n = ctypes.c_int32()
    _check(lib().engram_profile_read(ms, names, cap, ctypes.byref(n)))
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


def forward_workspace(B: int, T: int, layer: Layer) -> int:
    return int(lib().engram_forward_workspace(B, T, ctypes.byref(layer.s)))


def forward(tokens: torch.Tensor, H: torch.Tensor, layer: Layer, state: Optional[DecodeState] = None,
            want_alpha: bool = False, want_y: bool = False, ws: Optional[torch.Tensor] = None, stream=None):
    """One Engram layer; H is updated in place.  Returns (alpha, y) when asked."""
    B, T = tokens.shape
    M, d = layer.M, layer.d
    alpha = torch.empty((B, T, M), dtype=torch.float32, device=H.device) if want_alpha else None
    y = torch.empty((B, T, M, d), dtype=torch.float32, device=H.device) if want_y else None
    if ws is None:
        ws = torch.empty(max(forward_workspace(B, T, layer), 256), dtype=torch.uint8, device=H.device)
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_forward(_ptr(tokens), _ptr(H), B, T, ctypes.byref(layer.s), st, _ptr(alpha), _ptr(y),
                                _ptr(ws), ws.numel(), _stream(stream)))
    return alpha, y


NOALLOC_SCRATCH_BYTES = 32 << 20   # ENGRAM_NOALLOC_SCRATCH_BYTES


def forward_noalloc(tokens: torch.Tensor, H: torch.Tensor, layer: Layer, state: Optional[DecodeState] = None,
                    alpha: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, stream=None):
    """engram_forward_noalloc: the layer with the library's own scratch (no
    device allocation in the call; alpha / y are optional caller buffers)."""
    B, T = tokens.shape
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_forward_noalloc(_ptr(tokens), _ptr(H), B, T, ctypes.byref(layer.s), st, _ptr(alpha),
                                        _ptr(y), _stream(stream)))


def _layer_array(layers):
    arr = (ctypes.POINTER(LayerStruct) * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = ctypes.pointer(L.s)
    return arr


def project_ahead_workspace(B: int, T: int, layers) -> int:
    return lib().engram_project_ahead_workspace(B, T, len(layers), _layer_array(layers))


def kv_buffer(B: int, T: int, layer: Layer, device=None) -> torch.Tensor:
    """float32 [B*T, (1+M)*d]: v, then the M keys (engram_project_ahead)."""
    return torch.empty((B * T, (1 + layer.li.branches) * layer.li.d), dtype=torch.float32, device=device)


def project_ahead(tokens: torch.Tensor, layers, kv=None, states=None, ws: Optional[torch.Tensor] = None,
                  stream=None):
    """Steps 1-5 of several layers over the same tokens [B, T]; returns the
    float32 [v | k] rows of each (engram_project_ahead).  With states, T = 1
    and each state's ids and pos advance here."""
    B, T = tokens.shape
    if kv is None:
        kv = [kv_buffer(B, T, L, tokens.device) for L in layers]
    if ws is None:
        ws = torch.empty(max(project_ahead_workspace(B, T, layers), 256), dtype=torch.uint8, device=tokens.device)
    kv_arr = (ctypes.c_void_p * len(layers))(*[_ptr(k) for k in kv])
    st_arr = None
    if states is not None:
        st_arr = (ctypes.POINTER(DecodeStateStruct) * len(layers))()
        for i, st in enumerate(states):
            st_arr[i] = ctypes.pointer(st.s)
    _check(lib().engram_project_ahead(_ptr(tokens), B, T, len(layers), _layer_array(layers), st_arr, kv_arr,
                                      _ptr(ws), ws.numel(), _stream(stream)))
    return kv


def forward_projected(kv: torch.Tensor, H: torch.Tensor, layer: Layer, B: int, T: int, state=None,
                      want_alpha: bool = False, want_y: bool = False, ws: Optional[torch.Tensor] = None,
                      stream=None):
    """Steps 6-8 of one layer on kv from project_ahead (H updated in place);
    returns (alpha, y) when asked."""
    M, d = layer.li.branches, layer.li.d
    alpha = torch.empty((B, T, M), dtype=torch.float32, device=H.device) if want_alpha else None
    y = torch.empty((B, T, M, d), dtype=torch.float32, device=H.device) if want_y else None
    if ws is None:
        n = lib().engram_forward_projected_workspace(B, T, ctypes.byref(layer.s))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=H.device)
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_forward_projected(_ptr(kv), _ptr(H), B, T, ctypes.byref(layer.s), st, _ptr(alpha), _ptr(y),
                                          _ptr(ws), ws.numel(), _stream(stream)))
    return alpha, y


def rows_buffer(B: int, T: int, layer: Layer, device=None) -> torch.Tensor:
    """A buffer for the gathered rows e of B x T tokens (engram_retrieve); for
    an MXFP8 layer the E4M3 codes followed by the block scale bytes."""
    if layer.mxfp8:
        n = B * T * layer.d_mem
        return torch.empty(n + n // 32, dtype=torch.uint8, device=device)
    dt = torch.bfloat16 if layer.hdtype == BF16 else torch.float32
    return torch.empty((B * T, layer.d_mem), dtype=dt, device=device)


def quantize_mxfp8(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None):
    """MXFP8 of the rows of x (float32 or bfloat16 [rows, cols], cols % 32 == 0)."""
    rows, cols = x.shape
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _check(lib().engram_quantize_mxfp8(_ptr(x), dt, rows, cols, _ptr(q), _ptr(scale), _stream(stream)))


def pack_mxfp8(q: torch.Tensor, scale: torch.Tensor, packed: torch.Tensor, stream=None):
    """The MXFP8 codes q [rows, cols] and scales [rows, cols/32] in the
    matrix cores' operand order (uint8 [rows*cols + rows*cols/32])."""
    rows, cols = q.shape
    _check(lib().engram_pack_mxfp8(_ptr(q), _ptr(scale), rows, cols, _ptr(packed), _stream(stream)))


def pack_bf16(w: torch.Tensor, packed: torch.Tensor, stream=None):
    """The bf16 W [rows, cols] in the matrix cores' operand order (same size)."""
    rows, cols = w.shape
    _check(lib().engram_pack_bf16(_ptr(w), rows, cols, _ptr(packed), _stream(stream)))


def hot_lookup(tokens: torch.Tensor, spec, hot: HotTier, hist: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Hot row of every suffix n-gram, int32 [B, T, N-1] (-1 = cold)."""
    hs = spec.hs if isinstance(spec, Layer) else spec
    B, T = tokens.shape
    if out is None:
        out = torch.empty((B, T, hs.hp.max_n - 1), dtype=torch.int32, device=tokens.device)
    _check(lib().engram_hot_lookup(_ptr(tokens), B, T, _ptr(hist), ctypes.byref(hs.s), ctypes.byref(hot.s),
                                   _ptr(out), _stream(stream)))
    return out


def retrieve(tokens: torch.Tensor, layer: Layer, e: torch.Tensor, state: Optional[DecodeState] = None,
             stream=None):
    """Steps 1-4 into e, from the token ids (and the state's id history) only."""
    B, T = tokens.shape
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_retrieve(_ptr(tokens), B, T, ctypes.byref(layer.s), st, _ptr(e), _stream(stream)))


def forward_retrieved_workspace(B: int, T: int, layer: Layer) -> int:
    return int(lib().engram_forward_retrieved_workspace(B, T, ctypes.byref(layer.s)))


def forward_retrieved(tokens: torch.Tensor, e: torch.Tensor, H: torch.Tensor, layer: Layer,
                      state: Optional[DecodeState] = None, want_alpha: bool = False, want_y: bool = False,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """Steps 5-8 on the rows from retrieve(); H is updated in place.  Returns (alpha, y)."""
    B, T = tokens.shape
    M, d = layer.M, layer.d
    alpha = torch.empty((B, T, M), dtype=torch.float32, device=H.device) if want_alpha else None
    y = torch.empty((B, T, M, d), dtype=torch.float32, device=H.device) if want_y else None
    if ws is None:
        ws = torch.empty(max(forward_retrieved_workspace(B, T, layer), 256), dtype=torch.uint8, device=H.device)
    st = ctypes.byref(state.s) if state is not None else None
    _check(lib().engram_forward_retrieved(_ptr(tokens), _ptr(e), _ptr(H), B, T, ctypes.byref(layer.s), st,
                                          _ptr(alpha), _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return alpha, y


def forward_retrieved_prefetch(tokens: torch.Tensor, e: torch.Tensor, H: torch.Tensor, layer: Layer,
                               next_tokens: Optional[torch.Tensor], next_e: Optional[torch.Tensor],
                               want_alpha: bool = False, want_y: bool = False, ws: Optional[torch.Tensor] = None,
                               next_layer: Optional[Layer] = None, state: Optional[DecodeState] = None,
                               next_state: Optional[DecodeState] = None, stream=None):
    """Steps 5-8 on e (rows of `tokens`, continuing `state` if given) and
    Steps 1-4 of next_tokens with next_layer's tables (default: this layer)
    and next_state's id history into next_e, in the same launches where the
    layers allow.  Returns (alpha, y)."""
    B, T = tokens.shape
    nB, nT = (0, 0) if next_tokens is None else next_tokens.shape
    M, d = layer.M, layer.d
    alpha = torch.empty((B, T, M), dtype=torch.float32, device=H.device) if want_alpha else None
    y = torch.empty((B, T, M, d), dtype=torch.float32, device=H.device) if want_y else None
    if ws is None:
        ws = torch.empty(max(forward_retrieved_workspace(B, T, layer), 256), dtype=torch.uint8, device=H.device)
    nl = None if next_layer is None else ctypes.byref(next_layer.s)
    st = None if state is None else ctypes.byref(state.s)
    nst = None if next_state is None else ctypes.byref(next_state.s)
    _check(lib().engram_forward_retrieved_prefetch(_ptr(tokens), _ptr(e), _ptr(H), B, T, ctypes.byref(layer.s), st,
                                                   _ptr(alpha), _ptr(y), _ptr(ws), ws.numel(), nl, nst,
                                                   _ptr(next_tokens), nB, nT, _ptr(next_e), _stream(stream)))
    return alpha, y


ERR_TOKEN, ERR_ROW, ERR_SLOT, ERR_HOT_ROW = 1, 2, 4, 8


def debug_checks() -> bool:
    """True when the loaded library is the debug build."""
    return bool(lib().engram_debug_checks())


def debug_set_error_word(word: Optional[torch.Tensor]):
    """Debug build: kernels OR their precondition violations into `word` (a
    zeroed int32 device tensor of one element); None stops recording."""
    _check(lib().engram_debug_set_error_word(_ptr(word)))


def debug_read_errors() -> int:
    """Debug build: the error word's bits (ERR_*), cleared afterwards."""
    bits = ctypes.c_uint32(0)
    _check(lib().engram_debug_read_errors(ctypes.byref(bits)))
    return int(bits.value)
