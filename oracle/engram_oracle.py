"""Plain CPU oracle for the Engram conditional-memory forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it; the two meet only through the seeded
inputs in `hashed_gram_embedding_amd.inputs`, which hold none of the method.

What is computed, in the order and notation of "DeepSeek Engram series guide"
(foosynaptic deepseek-tech-notes, section "Engram working principle"):

  Step 1  x'_t = P(x_t)                         vocabulary projection
  Step 2  g_{t,n} = (x'_{t-n+1}, ..., x'_t)     suffix n-grams, n = 2..N
  Step 3  z_{t,n,k} = phi_{n,k}(g_{t,n}),  e_{t,n,k} = E_{n,k}[z_{t,n,k}]
          phi is a multiplicative-XOR hash into a prime-sized table.  The page
          does not give phi; it is fixed here as
              z = (XOR_i  x'_{t-i} * m_{n,k,i}  mod 2^64)  mod p_{n,k}
          with i = 0 the current token and ids before the sequence start
          taken as 0 (or from the decode history).
  Step 4  e_t = concat over n = 2..N (outer), k = 1..K (inner) of e_{t,n,k}
  Step 5  k_t = W_K e_t,  v_t = W_V e_t
  Step 6  alpha_t = sigmoid( RMSNorm(h_t) . RMSNorm(k_t) / sqrt(d) ),
          v~_t = alpha_t v_t
  Step 7  Y = SiLU( Conv1D( RMSNorm(V~) ) ) + V~, depthwise causal conv with
          kernel w = 4 and dilation N
  Step 8  H <- H + Y
  Multi-branch variant (same page, "variant on a multi-branch backbone"):
          per-branch gate alpha^(m) from h^(m) and W_K^(m) e_t, shared W_V,
          u^(m) = alpha^(m) W_V e_t; each branch has its own conv and residual.

Readings where the pages are silent (all listed in the design notes):
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps), over the d channels of one token
    and one branch, with no learned gain.
  * Conv taps follow the cross-correlation convention: weight [.., w-1]
    multiplies the current position, weight [.., j] the position
    (w-1-j)*dilation steps back; positions before the start read 0 (or the
    decode state); there is no bias.
  * int8 rows (lower-precision storage, "Engram module" article section 8,
    and the single select-and-dequantise kernel of the DRAM/SSD offload
    study) dequantise as float32(q) * float32(scale), rounded to bfloat16
    (nearest-even) when the gathered rows are bfloat16.
  * Decode state: the last N-1 compressed ids, and the last (w-1)*N conv
    inputs u = RMSNorm(v~), oldest first.
  * Engram-Nine hot tier (experiment 3 of the guide): the hot set is given
    per order n as a list of n-grams; a hit replaces the K heads of order n,
    i.e. K*d_head columns of e_t, by one hot row ("a single K x d table");
    the fingerprint is read as exact, so membership is exact set membership.

All floating-point arithmetic is float64 on values upcast exactly from their
storage type; hashing is uint64 with wraparound.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------------
# storage-format conversions (exact upcasts, one rounding helper)
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returned as float64.

    A bfloat16 keeps the top 16 bits of a float32.  Rounding to nearest-even
    adds half of the dropped range (0x8000), minus one unless the kept part is
    odd, then truncates.  Finite inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_odd = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_odd) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(a)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Step 1: vocabulary projection
# --------------------------------------------------------------------------

def compress(tokens: np.ndarray, proj: np.ndarray) -> np.ndarray:
    """x'_t = P(x_t) for every token (Step 1)."""
    return np.asarray(proj, dtype=np.int64)[np.asarray(tokens, dtype=np.int64)]


# --------------------------------------------------------------------------
# Step 2: suffix n-grams
# --------------------------------------------------------------------------

def history_id(xc: np.ndarray, b: int, pos: int, hist) -> int:
    """Compressed id at position `pos` of sequence b; pos < 0 reads the decode
    history (oldest first, last entry is position -1) or the pad id 0."""
    if pos >= 0:
        return int(xc[b, pos])
    if hist is None:
        return 0
    h = np.asarray(hist)
    j = h.shape[1] + pos
    return int(h[b, j]) if j >= 0 else 0


def suffix_ngram(xc: np.ndarray, b: int, t: int, n: int, hist=None) -> tuple:
    """g_{t,n} = (x'_{t-n+1}, ..., x'_t) (Step 2), oldest first."""
    return tuple(history_id(xc, b, t - n + 1 + i, hist) for i in range(n))


def shifted_ids(xc: np.ndarray, i: int, hist) -> np.ndarray:
    """Array of x'_{t-i} over all (b, t), with history / pad for t-i < 0."""
    B, T = xc.shape
    out = np.zeros((B, T), dtype=np.int64)
    if i < T:
        out[:, i:] = xc[:, : T - i]
    for t in range(min(i, T)):
        for b in range(B):
            out[b, t] = history_id(xc, b, t - i, hist)
    return out


# --------------------------------------------------------------------------
# Step 3: multiplicative-XOR hash into prime-sized tables
# --------------------------------------------------------------------------

def hash_gram(gram_newest_first, mult_nk: np.ndarray, prime: int) -> int:
    """phi_{n,k}: XOR over i of (id_i * m_{n,k,i}) mod 2^64, then mod p.
    gram_newest_first[0] is x'_t, [1] is x'_{t-1}, ..."""
    acc = np.zeros(1, dtype=np.uint64)
    for i, x in enumerate(gram_newest_first):
        acc ^= np.array([x], dtype=np.uint64) * np.asarray(mult_nk, dtype=np.uint64)[i]
    return int(acc[0] % np.uint64(prime))


def hash_grams(grams_newest_first: np.ndarray, mult_nk: np.ndarray, prime: int) -> np.ndarray:
    """Vectorised phi_{n,k} over an array of n-grams [G, n] (newest first)."""
    g = np.asarray(grams_newest_first, dtype=np.uint64)
    acc = np.zeros(g.shape[0], dtype=np.uint64)
    for i in range(g.shape[1]):
        acc ^= g[:, i] * np.uint64(int(mult_nk[i]))
    return (acc % np.uint64(int(prime))).astype(np.int64)


def hash_indices(tokens: np.ndarray, proj: np.ndarray, mult: np.ndarray, prime: np.ndarray,
                 max_n: int, heads: int, hist=None) -> np.ndarray:
    """z[b, t, j] for table j = (n-2)*K + k (Steps 1-3).

    tokens [B, T] raw ids; hist [B, N-1] compressed ids before t = 0 (oldest
    first) or None for pad 0.  Returns int64 [B, T, (N-1)*K]."""
    xc = compress(tokens, proj)
    B, T = xc.shape
    z = np.zeros((B, T, (max_n - 1) * heads), dtype=np.int64)
    back = [shifted_ids(xc, i, hist).astype(np.uint64) for i in range(max_n)]
    for n in range(2, max_n + 1):
        for k in range(heads):
            acc = np.zeros((B, T), dtype=np.uint64)
            for i in range(n):
                acc ^= back[i] * np.uint64(int(mult[n - 2, k, i]))
            j = (n - 2) * heads + k
            z[:, :, j] = (acc % np.uint64(int(prime[j]))).astype(np.int64)
    return z


# --------------------------------------------------------------------------
# Steps 3-4: table lookup and concatenation
# --------------------------------------------------------------------------

def table_rows_f64(rows: np.ndarray, dtype: str, global_rows: np.ndarray,
                   scale=None, out_dtype: str = "bf16") -> np.ndarray:
    """Values of the requested rows as the gathered output type holds them.

    f32 / bf16 rows are exact copies (an f32 row gathered into a bf16 output
    is rounded to nearest-even); int8 rows are float32(q) * float32(scale),
    rounded to bf16 for a bf16 output."""
    r = np.asarray(rows)[global_rows]
    if dtype == "i8":
        s = np.asarray(scale, dtype=np.float32)[global_rows]
        prod = r.astype(np.float32) * s[..., None]         # one IEEE float32 multiply
        return round_f32_to_bf16(prod) if out_dtype == "bf16" else prod.astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(r)
    if out_dtype == "bf16":
        return round_f32_to_bf16(r)
    return r.astype(np.float64)


def gather(z: np.ndarray, rows: np.ndarray, dtype: str, row_offset: np.ndarray, dim: int,
           scale=None, out_dtype: str = "bf16") -> np.ndarray:
    """e_t = concat_j E_j[z_{t,j}] (Steps 3-4).  z [..., n_tables] local rows;
    returns float64 [..., n_tables * dim]."""
    z = np.asarray(z, dtype=np.int64)
    g = z + np.asarray(row_offset, dtype=np.int64)
    vals = table_rows_f64(rows, dtype, g, scale, out_dtype)   # [..., n_tables, dim]
    return vals.reshape(*z.shape[:-1], z.shape[-1] * dim)


def lfu_admission(global_rows: np.ndarray, total_rows: int, cache_n: int) -> np.ndarray:
    """Static LFU admission of the hot-row cache (Ascend RecSDK Engram article,
    multi-level cache: the most frequently accessed rows live in fast memory).

    Counts the accesses of each row in `global_rows`, admits the cache_n most
    frequent rows (ties: lower row first) and numbers them 0..cache_n-1 in
    ascending row order.  Returns the slot of every row (-1 = not cached)."""
    counts = np.bincount(np.asarray(global_rows, dtype=np.int64).ravel(), minlength=total_rows)
    order = np.lexsort((np.arange(total_rows), -counts))     # by count desc, then row asc
    admitted = np.sort(order[:cache_n])
    slot = np.full(total_rows, -1, dtype=np.int64)
    slot[admitted] = np.arange(cache_n)
    return slot


def lfu_update(counts: np.ndarray, slot_prev: np.ndarray, cache_n: int, decay_shift: int = 0):
    """Real-time LFU update of the hot cache (Ascend RecSDK Engram article,
    multi-level cache: access statistics drive LFU admission and eviction so
    the hot cache stays current).

    The cache_n rows with the highest counts are admitted (ties: lower row
    first).  A cached row that is admitted again keeps its slot; a cached row
    that is not admitted leaves (-1).  The slots nobody keeps, in ascending
    order, go to the newly admitted rows in ascending row order.  Then every
    count is shifted right by decay_shift.  Returns (slot, counts)."""
    counts = np.asarray(counts, dtype=np.int64)
    slot_prev = np.asarray(slot_prev, dtype=np.int64)
    total_rows = counts.shape[0]
    order = np.lexsort((np.arange(total_rows), -counts))     # by count desc, then row asc
    is_admitted = np.zeros(total_rows, dtype=bool)
    is_admitted[order[:cache_n]] = True
    slot = np.where(is_admitted & (slot_prev >= 0), slot_prev, -1)
    kept = np.zeros(cache_n, dtype=bool)
    kept[slot[slot >= 0]] = True
    free_slots = np.nonzero(~kept)[0]                         # ascending
    newcomers = np.nonzero(is_admitted & (slot_prev < 0))[0]  # ascending rows
    slot[newcomers] = free_slots[:newcomers.shape[0]]
    return slot, counts >> decay_shift


# --------------------------------------------------------------------------
# Engram-Nine: a collision-free hot tier over the most frequent n-grams
# ("DeepSeek Engram series guide", experiment 3 "Engram-Nine", its Figure 1:
# two-tier retrieval).  An n-gram g_{t,n} that belongs to the hot set of its
# order n takes one hot row of width K*d_head in place of its K hashed rows;
# every other n-gram keeps the K-head cold lookup.  The page builds the hot
# set's index with a minimal perfect hash plus a fingerprint; what that
# computes is exact set membership and a distinct row per hot n-gram, which
# is what is written out here (a dictionary from n-gram to row).
# --------------------------------------------------------------------------

def hot_index(keys) -> dict:
    """Row of every hot n-gram: keys is a sequence of n-tuples (oldest id
    first); key r gets hot row r.  Duplicate keys are an error."""
    index = {}
    for r, key in enumerate(keys):
        key = tuple(int(v) for v in key)
        if key in index:
            raise ValueError(f"duplicate hot key {key}")
        index[key] = r
    return index


def hot_lookup(tokens: np.ndarray, proj: np.ndarray, max_n: int, hot_keys: dict, hist=None) -> np.ndarray:
    """r[b, t, n-2] = hot row of g_{t,n} in the hot set of order n, or -1 when
    g_{t,n} is not hot (or order n has no hot tier).

    hot_keys maps an order n to its sequence of hot n-tuples (oldest first);
    g_{t,n} is formed exactly as in Step 2, with history / pad for t < n-1."""
    xc = compress(tokens, proj)
    B, T = xc.shape
    out = np.full((B, T, max_n - 1), -1, dtype=np.int64)
    for n in range(2, max_n + 1):
        keys = hot_keys.get(n)
        if keys is None or len(keys) == 0:
            continue
        index = hot_index(keys)
        for b in range(B):
            for t in range(T):
                out[b, t, n - 2] = index.get(suffix_ngram(xc, b, t, n, hist), -1)
    return out


def gather_two_tier(z: np.ndarray, hot_idx: np.ndarray, rows: np.ndarray, dtype: str, row_offset: np.ndarray,
                    dim: int, heads: int, hot_rows: dict, scale=None, out_dtype: str = "bf16") -> np.ndarray:
    """e_t with the hot tier: for order n the K*dim columns of its K heads,
    columns (n-2)*K*dim .. (n-1)*K*dim - 1 of e_t, are the hot row
    hot_rows[n][hot_idx[..., n-2]] when that index is >= 0 and the
    concatenated cold rows E_{n,k}[z_{t,n,k}] otherwise.  Hot rows are stored
    like the cold tables (f32 or bf16 bits)."""
    if dtype == "i8":
        raise ValueError("the hot tier holds f32 or bf16 rows")
    e = gather(z, rows, dtype, row_offset, dim, scale, out_dtype)
    width = heads * dim
    for o in range(hot_idx.shape[-1]):
        hit = hot_idx[..., o] >= 0
        if not hit.any():
            continue
        n = o + 2
        vals = table_rows_f64(hot_rows[n], dtype, hot_idx[..., o][hit], None, out_dtype)
        e[..., o * width:(o + 1) * width][hit] = vals
    return e


# --------------------------------------------------------------------------
# Step 5: key / value projections
# --------------------------------------------------------------------------

def project_kv(e: np.ndarray, w: np.ndarray) -> np.ndarray:
    """[v | k^(0) | ... | k^(M-1)] = e W^T with W stacked [W_V; W_K^(0..M-1)],
    each block [d, d_mem] (Step 5 and the fused-projection remark of the
    multi-branch variant)."""
    return np.asarray(e, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


# --------------------------------------------------------------------------
# Step 6: context-aware gate
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def gate(h: np.ndarray, k: np.ndarray, eps: float) -> np.ndarray:
    """alpha = sigmoid(RMSNorm(h) . RMSNorm(k) / sqrt(d)) over the last axis (Step 6)."""
    d = h.shape[-1]
    return sigmoid(np.sum(rmsnorm(h, eps) * rmsnorm(k, eps), axis=-1) / np.sqrt(d))


# --------------------------------------------------------------------------
# Step 7: short causal depthwise convolution
# --------------------------------------------------------------------------

def short_conv(u: np.ndarray, conv_w: np.ndarray, dilation: int, prev=None) -> np.ndarray:
    """c_t[ch] = sum_j conv_w[ch, j] * u_{t-(w-1-j)*dilation}[ch] (Step 7).

    u [T, d] for one sequence and branch; conv_w [d, w]; prev [(w-1)*dilation, d]
    holds u at positions -(w-1)*dilation .. -1 (oldest first) or None for 0."""
    T, d = u.shape
    w = conv_w.shape[1]
    span = (w - 1) * dilation
    full = np.zeros((span + T, d), dtype=np.float64)
    if prev is not None:
        full[:span] = prev
    full[span:] = u
    c = np.zeros((T, d), dtype=np.float64)
    for j in range(w):
        back = (w - 1 - j) * dilation
        c += conv_w[None, :, j] * full[span - back: span - back + T]
    return c


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


# --------------------------------------------------------------------------
# Steps 1-8: one Engram layer
# --------------------------------------------------------------------------

def new_state(B: int, max_n: int, branches: int, span: int, d: int) -> dict:
    return {"ids": np.zeros((B, max_n - 1), dtype=np.int64),
            "u": np.zeros((B, branches, span, d), dtype=np.float64),
            "pos": np.zeros(B, dtype=np.int64)}


def gate_conv(H: np.ndarray, kv: np.ndarray, conv_w: np.ndarray, dilation: int, eps: float,
              state_u=None) -> dict:
    """Steps 6-8 from given projections, for every branch.

    H [B, T, M, d] and kv [B, T, (1+M)*d] (v, then k^(0..M-1)) as float64;
    conv_w [M, d, w]; state_u [B, M, (w-1)*dilation, d] conv inputs before
    t = 0 (oldest first) or None.  Returns alpha, vt, u, c, Y and H_out."""
    B, T, M, d = H.shape
    v = kv[..., :d]
    alpha = np.zeros((B, T, M))
    vt = np.zeros((B, T, M, d))
    u = np.zeros((B, T, M, d))
    c = np.zeros((B, T, M, d))
    for m in range(M):
        k_m = kv[..., (1 + m) * d:(2 + m) * d]
        alpha[:, :, m] = gate(H[:, :, m, :], k_m, eps)                               # Step 6
        vt[:, :, m, :] = alpha[:, :, m, None] * v
        u[:, :, m, :] = rmsnorm(vt[:, :, m, :], eps)                                 # Step 7
        for b in range(B):
            prev = None if state_u is None else state_u[b, m]
            c[b, :, m, :] = short_conv(u[b, :, m, :], conv_w[m], dilation, prev)
    Y = silu(c) + vt
    return {"alpha": alpha, "vt": vt, "u": u, "c": c, "Y": Y, "H_out": H + Y}       # Step 8


# --------------------------------------------------------------------------
# Step 5 in MXFP8: the fused W_V / W_K product as one FP8 dense GEMM
# --------------------------------------------------------------------------
# The Guide (variant on a multi-branch backbone) suggests fusing W_V with the
# M keys into one FP8 dense GEMM.  The FP8 format is fixed here as OCP MXFP8:
# E4M3 elements (bias 7, no infinities, largest finite 448, subnormals down
# to 2^-9) in blocks of 32 consecutive elements along the contraction axis,
# each block with a power-of-two scale stored as an 8-bit biased exponent
# (byte = exponent + 127).  The scale is the smallest power of two that keeps
# the block's largest magnitude within +-448 (so nothing saturates; OCP's
# floor(log2 amax) - 8 rule would clip up to 12.5 % off the largest element):
# with amax = m 2^E, 0.5 <= m < 1, the exponent is E - 9, plus one when
# m > 0.875.  Elements are v / scale (exact) rounded to nearest-even E4M3.  An
# all-zero block gets scale byte 0 and zero elements.

E4M3_MAX = 448.0


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest-even rounding of float64 values to E4M3, saturated to +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # exponent of the value's binade, never below the smallest normal's (-6)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.ldexp(1.0, (e - 3).astype(np.int64))          # 3 mantissa bits
    r = np.rint(a / quantum) * quantum                          # ties to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are exactly representable in E4M3."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.uint8)
    normal = a >= 2.0 ** -6
    e = np.floor(np.log2(np.where(normal, a, 1.0))).astype(np.int64)
    man = np.where(normal, np.rint((a / np.ldexp(1.0, e) - 1.0) * 8), np.rint(a / 2.0 ** -9)).astype(np.int64)
    out = np.where(normal, ((e + 7) << 3) | man, man).astype(np.uint8)
    return (out | sign).astype(np.uint8)


def e4m3_decode(q: np.ndarray) -> np.ndarray:
    q = np.asarray(q, dtype=np.uint8).astype(np.int64)
    s = np.where(q & 0x80, -1.0, 1.0)
    e = (q >> 3) & 15
    m = q & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return s * mag


def quantize_mxfp8(x: np.ndarray):
    """MXFP8 of x [..., K] with K a multiple of 32: returns (elements uint8
    [..., K], scale bytes uint8 [..., K/32])."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.max(np.abs(blocks), axis=-1)
    m, E = np.frexp(np.where(amax > 0, amax, 1.0))
    exp = np.clip(E - 9 + (m > 0.875), -127, 127)
    scale = np.where(amax > 0, np.ldexp(1.0, exp.astype(np.int64)), 1.0)
    q = round_to_e4m3(blocks / scale[..., None])
    q = np.where(amax[..., None] > 0, q, 0.0)
    sbyte = np.where(amax > 0, exp + 127, 0).astype(np.uint8)
    return e4m3_encode(q).reshape(x.shape), sbyte


def dequantize_mxfp8(q: np.ndarray, sbyte: np.ndarray) -> np.ndarray:
    v = e4m3_decode(q)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    scale = np.ldexp(1.0, sbyte.astype(np.int64) - 127)
    return (blocks * scale[..., None]).reshape(v.shape)


def project_kv_mxfp8(e: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Step 5 with both operands in MXFP8 (blocks along d_mem), products and
    sums exact in float64."""
    eq, es = quantize_mxfp8(e)
    wq, ws = quantize_mxfp8(w)
    return dequantize_mxfp8(eq, es) @ dequantize_mxfp8(wq, ws).T


def forward(tokens: np.ndarray, H: np.ndarray, layer, h_dtype: str, state=None,
            e_dtype=None, gemm: str = "exact", hot=None) -> dict:
    """One Engram layer over tokens [B, T] and hidden states H [B, T, M, d].

    `layer` is a `LayerInputs`-like object (hash, tables, w, conv_w, eps,
    kernel_w, dilation, d, branches).  h_dtype is the storage type of H, W and
    the gathered rows ("f32" or "bf16").  With `state` (see new_state) the
    chunk continues earlier tokens and a new state is returned.
    Returns float64 arrays: z, e, kv, alpha [B,T,M], vt, u, c, Y [B,T,M,d],
    H_out, and `state`.  gemm="mxfp8" takes Step 5 in MXFP8 (project_kv_mxfp8).
    hot = {"keys": {n: n-tuples}, "rows": {n: [n_hot, K*dim] rows}} adds the
    Engram-Nine hot tier (gather_two_tier); the result then also holds hot_idx.
    """
    hp, tab = layer.hash, layer.tables
    B, T = tokens.shape
    span = (layer.kernel_w - 1) * layer.dilation
    hist = None if state is None else state["ids"]
    e_dtype = e_dtype or h_dtype

    z = hash_indices(tokens, hp.proj, hp.mult, hp.prime, hp.max_n, hp.heads, hist)   # Steps 1-3
    if hot is None:
        e = gather(z, tab.rows, tab.dtype, tab.row_offset, tab.dim, tab.scale, e_dtype)  # Steps 3-4
    else:
        hot_idx = hot_lookup(tokens, hp.proj, hp.max_n, hot["keys"], hist)
        e = gather_two_tier(z, hot_idx, tab.rows, tab.dtype, tab.row_offset, tab.dim, hp.heads, hot["rows"],
                            tab.scale, e_dtype)
    w64 = storage_to_f64(layer.w, h_dtype)
    kv = project_kv_mxfp8(e, w64) if gemm == "mxfp8" else project_kv(e, w64)       # Step 5
    out = gate_conv(storage_to_f64(H, h_dtype), kv, layer.conv_w, layer.dilation, layer.eps,
                    None if state is None else state["u"])                           # Steps 6-8
    out.update({"z": z, "e": e, "kv": kv})
    if hot is not None:
        out["hot_idx"] = hot_idx
    if state is not None:
        xc = compress(tokens, hp.proj)
        ids = np.concatenate([state["ids"], xc], axis=1)[:, -(hp.max_n - 1):]
        uu = np.concatenate([state["u"], np.transpose(out["u"], (0, 2, 1, 3))], axis=2)[:, :, -span:]
        out["state"] = {"ids": ids, "u": uu, "pos": state["pos"] + T}
    return out
