"""Seeded synthetic inputs for the Engram conditional-memory layer.

This module draws every input the layer consumes -- token ids, the vocabulary
projection table, hash multipliers, prime table sizes, embedding tables,
hidden states, projection and conv weights, decode context, LFU warm-up
streams and the hot tier's n-gram choice and rows -- and nothing else.  It holds none of the layer's arithmetic (no
hashing, gathering, projection, gating or convolution), so the CPU oracle and
the GPU library can both be fed from it without sharing any of the method.

Sources for the shapes (DeepSeek Engram series guide, "Engram working
principle", Steps 1-7; Ascend RecSDK Engram article, "test results" settings):
  * compressed vocabulary about 23 % smaller than the raw one (Step 1);
  * orders n = 2..N with K heads each, prime-sized tables (Step 3);
  * 512 embedding dims per order split over 8 heads, 10,342,400 table rows in
    total, maximum order 3, sequence length 4096 (RecSDK settings list);
  * hyper-connection backbone with M = 4 residual branches (multi-branch
    variant).
The pages give no dataset that is available here; tokens are i.i.d. draws from
a truncated Zipf(1.1) law over the raw vocabulary, standing in for CCI3-HQ
text.

Random streams: numpy PCG64 seeded by SeedSequence([config, layer, stream]).
bf16 arrays are carried as uint16 bit patterns (numpy has no bfloat16).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import List, Optional

import numpy as np

# stream ids inside SeedSequence([config, layer, stream])
S_TOKENS, S_PROJ, S_MULT, S_TABLES, S_H, S_W, S_CONV, S_LFU, S_CONTEXT, S_HOT, S_UNIFORM, S_RING = range(12)

F32, BF16, I8 = "f32", "bf16", "i8"


def rng_for(config: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, layer, stream])))


# --------------------------------------------------------------------------
# scalar-format helpers for building inputs (input preparation only)
# --------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _is_prime(c: int) -> bool:
    if c < 2:
        return False
    if c % 2 == 0:
        return c == 2
    f = 3
    while f * f <= c:
        if c % f == 0:
            return False
        f += 2
    return True


def primes_from(start: int, count: int) -> List[int]:
    """The `count` smallest primes >= start (trial division)."""
    out = []
    c = max(2, start)
    while len(out) < count:
        if _is_prime(c):
            out.append(c)
        c += 1
    return out


def zipf_tokens(rng: np.random.Generator, vocab: int, s: float, shape) -> np.ndarray:
    """i.i.d. ranks 1..vocab with P(r) proportional to r**-s, returned as ids r-1."""
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -s)
    cdf /= cdf[-1]
    u = rng.random(size=int(np.prod(shape)))
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32).reshape(shape)


def make_projection(rng: np.random.Generator, vocab: int, vocab_c: int) -> np.ndarray:
    """Seeded surjection P: [0, vocab) -> [0, vocab_c).

    A seeded permutation of the raw ids; the first vocab_c permuted ids map one
    to one onto 0..vocab_c-1, the rest map to uniform draws in [0, vocab_c).
    This stands in for the NFKC / lower-casing canonicalisation of a real
    tokenizer (Step 1), which needs tokenizer files.
    """
    perm = rng.permutation(vocab)
    proj = np.empty(vocab, dtype=np.int32)
    proj[perm[:vocab_c]] = np.arange(vocab_c, dtype=np.int32)
    rest = vocab - vocab_c
    if rest > 0:
        proj[perm[vocab_c:]] = rng.integers(0, vocab_c, size=rest, dtype=np.int32)
    return proj


def make_multipliers(rng: np.random.Generator, max_n: int, heads: int) -> np.ndarray:
    """Odd seeded 64-bit multipliers, shape [(N-1), K, N]; entry [n-2, k, i]."""
    m = rng.integers(0, 2 ** 64, size=(max_n - 1, heads, max_n), dtype=np.uint64, endpoint=False)
    return m | np.uint64(1)


# Large arrays are drawn in fixed chunks of GEN_CHUNK values, chunk i from the
# i-th child generator of `rng` (Generator.spawn), and the chunks are filled by
# a thread pool (numpy's generators and ufuncs release the GIL).  The values
# depend only on the seed and the array size, not on the thread count.
GEN_CHUNK = 1 << 22


def gen_threads() -> int:
    """Threads for input generation: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_chunks(rng: np.random.Generator, n: int, chunk: int, fill) -> None:
    """Calls fill(child_rng, start, end) for consecutive chunks of [0, n), each
    with its own spawned child generator, on a thread pool."""
    if n <= 0:
        return
    bounds = [(s, min(n, s + chunk)) for s in range(0, n, chunk)]
    kids = rng.spawn(len(bounds))
    if len(bounds) == 1:
        fill(kids[0], *bounds[0])
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=gen_threads()) as ex:
        list(ex.map(lambda a: fill(a[0], *a[1]), zip(kids, bounds)))


def normal_bf16_bits(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)

    def fill(g, s, e):
        out[s:e] = to_bf16_bits(g.standard_normal(e - s, dtype=np.float32) * np.float32(std))
    fill_chunks(rng, n, GEN_CHUNK, fill)
    return out


def normal_f32(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)

    def fill(g, s, e):
        g.standard_normal(e - s, dtype=np.float32, out=out[s:e])
        out[s:e] *= np.float32(std)
    fill_chunks(rng, n, GEN_CHUNK, fill)
    return out


def quantize_rows_int8(rows: np.ndarray):
    """Symmetric per-row int8: scale = max|row|/127, q = rint(row/scale) clamped
    to [-127, 127] (ties to even).  All-zero rows get scale 0 and q = 0."""
    rows = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(rows), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.rint(rows / safe[:, None])
    q = np.clip(q, -127, 127).astype(np.int8)
    q[scale == 0] = 0
    return q, scale


# --------------------------------------------------------------------------
# input containers
# --------------------------------------------------------------------------

@dataclasses.dataclass
class HashInputs:
    vocab: int              # raw vocabulary size V
    vocab_c: int            # compressed vocabulary size V'
    max_n: int              # N: orders 2..N
    heads: int              # K heads per order
    proj: np.ndarray        # int32 [V]
    mult: np.ndarray        # uint64 [N-1, K, N]
    prime: np.ndarray       # uint32 [(N-1)*K], table j = (n-2)*K + k

    @property
    def n_tables(self) -> int:
        return (self.max_n - 1) * self.heads


@dataclasses.dataclass
class TableInputs:
    dim: int                # columns per row (d_head)
    dtype: str              # F32 | BF16 | I8
    rows: np.ndarray        # [sum_rows, dim]: float32 | uint16 (bf16 bits) | int8
    row_offset: np.ndarray  # int64 [n_tables]: first row of table j in `rows`
    n_rows: np.ndarray      # int64 [n_tables]: rows of table j (its prime)
    scale: Optional[np.ndarray] = None  # float32 [sum_rows] for I8

    @property
    def total_rows(self) -> int:
        return int(self.rows.shape[0])


@dataclasses.dataclass
class LayerInputs:
    hash: HashInputs
    tables: TableInputs
    d: int                  # hidden width per branch
    branches: int           # M
    w: np.ndarray           # [(1+M)*d, d_mem]: rows 0..d-1 W_V, then W_K^(m); float32 or bf16 bits
    conv_w: np.ndarray      # float32 [M, d, kernel_w]; tap kernel_w-1 multiplies the current position
    kernel_w: int = 4
    dilation: int = 3
    eps: float = 1e-6

    @property
    def d_mem(self) -> int:
        return self.tables.dim * self.hash.n_tables


@dataclasses.dataclass
class Workload:
    name: str
    config: int
    dtype: str              # F32 or BF16: storage type of H, W, e and kv
    B: int
    T: int
    tokens: np.ndarray      # int32 [B, T]
    H: np.ndarray           # [B, T, M, d] float32 or bf16 bits
    layers: List[LayerInputs]
    context: Optional[np.ndarray] = None   # int32 [B, Tc] decode warm-up context
    H_context: Optional[np.ndarray] = None  # hidden states for the context
    note: str = ""


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

def _hash_inputs(config, layer, vocab, vocab_c, max_n, heads, prime_start, primes=None):
    proj = make_projection(rng_for(config, layer, S_PROJ), vocab, vocab_c)
    mult = make_multipliers(rng_for(config, layer, S_MULT), max_n, heads)
    if primes is None:
        primes = primes_from(prime_start, (max_n - 1) * heads)
    return HashInputs(vocab, vocab_c, max_n, heads, proj, mult, np.asarray(primes, dtype=np.uint32))


def _tables(config, layer, prime, dim, dtype, std=0.02):
    n_rows = prime.astype(np.int64)
    row_offset = np.concatenate([[0], np.cumsum(n_rows)[:-1]]).astype(np.int64)
    total = int(n_rows.sum())
    rng = rng_for(config, layer, S_TABLES)
    if dtype == F32:
        rows = normal_f32(rng, total * dim, std).reshape(total, dim)
        return TableInputs(dim, F32, rows, row_offset, n_rows)
    if dtype == BF16:
        rows = normal_bf16_bits(rng, total * dim, std).reshape(total, dim)
        return TableInputs(dim, BF16, rows, row_offset, n_rows)
    if dtype == I8:
        q = np.empty((total, dim), dtype=np.int8)
        scale = np.empty(total, dtype=np.float32)

        def fill(g, s, e):
            x = g.standard_normal((e - s) * dim, dtype=np.float32) * np.float32(std)
            q[s:e], scale[s:e] = quantize_rows_int8(x.reshape(e - s, dim))
        fill_chunks(rng, total, max(1, GEN_CHUNK // dim), fill)
        return TableInputs(dim, I8, q, row_offset, n_rows, scale)
    raise ValueError(dtype)


def _layer(config, layer, *, vocab, vocab_c, max_n, heads, prime_start, dim, table_dtype,
           d, branches, store_dtype, w_std, primes=None):
    hp = _hash_inputs(config, layer, vocab, vocab_c, max_n, heads, prime_start, primes)
    tab = _tables(config, layer, hp.prime, dim, table_dtype)
    d_mem = dim * hp.n_tables
    nw = (1 + branches) * d * d_mem
    rng_w = rng_for(config, layer, S_W)
    if store_dtype == BF16:
        w = normal_bf16_bits(rng_w, nw, w_std).reshape((1 + branches) * d, d_mem)
    else:
        w = normal_f32(rng_w, nw, w_std).reshape((1 + branches) * d, d_mem)
    conv_w = normal_f32(rng_for(config, layer, S_CONV), branches * d * 4, 0.1).reshape(branches, d, 4)
    return LayerInputs(hp, tab, d, branches, w, conv_w)


def _hidden(config, shape, dtype):
    rng = rng_for(config, 0, S_H)
    n = int(np.prod(shape))
    if dtype == BF16:
        return normal_bf16_bits(rng, n, 1.0).reshape(shape)
    return normal_f32(rng, n, 1.0).reshape(shape)


CONFIG_NAMES = {
    0: "tiny-fp32",
    1: "single-branch-bf16",
    2: "multi-branch-bf16",
    3: "decode-int8",
    4: "host-table-hbm-cache",
}

C1_PRIME_START = 10_342_400 // 16      # 646,400 rows per table
C4_PRIME_START = (1 << 25) // 16      # 2,097,152 rows per table


def make_config(config: int, *, B: Optional[int] = None, T: Optional[int] = None,
                table_dim: Optional[int] = None, layers: Optional[int] = None,
                context_len: int = 16, uniform_tokens: bool = False,
                rows_per_table: Optional[int] = None, d: Optional[int] = None,
                branches: Optional[int] = None, heads: Optional[int] = None) -> Workload:
    """Build workload `config` (0..4).

    B, T, layers, and (for small tests) the rows per table, the hidden width d,
    the branch count and (configs 1-4) the heads per order may be overridden;
    the tables then hold the first primes >= rows_per_table.
    """
    if config == 0:
        B = B or 1
        T = T or 64
        dim = table_dim or 16
        dd = d or 64
        M = branches or 1
        primes = None if rows_per_table else [1009, 1013, 1019, 1021]
        lay = _layer(0, 0, vocab=1000, vocab_c=770, max_n=3, heads=2,
                     prime_start=rows_per_table or 1000, dim=dim, table_dtype=F32, d=dd,
                     branches=M, store_dtype=F32, w_std=1.0 / 32, primes=primes)
        tokens = rng_for(0, 0, S_TOKENS).integers(0, 1000, size=(B, T), dtype=np.int32)
        H = _hidden(0, (B, T, M, dd), F32)
        return Workload(CONFIG_NAMES[0], 0, F32, B, T, tokens, H, [lay])

    dd = d or 1024
    common = dict(vocab=128_000, vocab_c=98_560, max_n=3, heads=heads or 8, dim=table_dim or 64, d=dd,
                  store_dtype=BF16, w_std=1.0 / 32)
    c1_start = rows_per_table or C1_PRIME_START
    c4_start = rows_per_table or C4_PRIME_START
    if config in (1, 2):
        M = branches or (1 if config == 1 else 4)
        B = B or (1 if config == 1 else 8)
        T = T or 4096
        lay = _layer(config, 0, prime_start=c1_start, table_dtype=BF16, branches=M, **common)
        rng_t = rng_for(config, 0, S_TOKENS)
        if uniform_tokens:
            tokens = rng_t.integers(0, 128_000, size=(B, T), dtype=np.int32)
        else:
            tokens = zipf_tokens(rng_t, 128_000, 1.1, (B, T))
        H = _hidden(config, (B, T, M, dd), BF16)
        return Workload(CONFIG_NAMES[config], config, BF16, B, T, tokens, H, [lay])

    if config == 3:
        S = B or 256
        T = T or 1
        nl = layers or 2
        M = branches or 1
        lays = [_layer(3, l, prime_start=c1_start, table_dtype=I8, branches=M, **common)
                for l in range(nl)]
        tokens = zipf_tokens(rng_for(3, 0, S_TOKENS), 128_000, 1.1, (S, T))
        ctx = zipf_tokens(rng_for(3, 0, S_CONTEXT), 128_000, 1.1, (S, context_len))
        H = _hidden(3, (S, T, M, dd), BF16)
        Hc = normal_bf16_bits(rng_for(3, 1, S_H), S * context_len * M * dd, 1.0).reshape(S, context_len, M, dd)
        return Workload(CONFIG_NAMES[3], 3, BF16, S, T, tokens, H, lays, context=ctx, H_context=Hc,
                        note="decode: each sequence first consumes `context` through prefill")

    if config == 4:
        B = B or 4
        T = T or 4096
        nl = layers or 2
        lays = [_layer(4, l, prime_start=c4_start, table_dtype=BF16, branches=1, **common)
                for l in range(nl)]
        tokens = zipf_tokens(rng_for(4, 0, S_TOKENS), 128_000, 1.1, (B, T))
        H = _hidden(4, (B, T, 1, dd), BF16)
        return Workload(CONFIG_NAMES[4], 4, BF16, B, T, tokens, H, lays)
    raise ValueError(f"unknown config {config}")


def make_order4(B: int, T: int, *, heads: int = 4, dim: int = 32, d: int = 128, branches: int = 1,
                rows_per_table: int = 1009, layers: int = 1) -> Workload:
    """A bf16 variant with n-gram orders 2..4 (N = 4, the largest the library
    takes): K = 4 heads of 32 dims per order (d_mem = 384), prime tables from
    rows_per_table up, hidden width d; tokens Zipf(1.1) over 128,000 raw ids
    projected to 98,560.  Seeds under configuration id 5."""
    lays = [_layer(5, l, vocab=128_000, vocab_c=98_560, max_n=4, heads=heads, prime_start=rows_per_table, dim=dim,
                   table_dtype=BF16, d=d, branches=branches, store_dtype=BF16, w_std=1.0 / 20)
            for l in range(layers)]
    tokens = zipf_tokens(rng_for(5, 0, S_TOKENS), 128_000, 1.1, (B, T))
    H = _hidden(5, (B, T, branches, d), BF16)
    return Workload("order-4-bf16", 5, BF16, B, T, tokens, H, lays)


def make_shape(B: int, T: int, *, max_n: int = 3, heads: int = 8, dim: int = 64, d: int = 1024,
               branches: int = 1, rows_per_table: int = 997, w_std: float = 1.0 / 32) -> Workload:
    """A bf16 layer of any shape the library takes (n-gram orders 2..max_n,
    `heads` tables of `dim` columns per order, hidden width d, `branches`
    branches), for the tests at the library's limits: Zipf(1.1) tokens over
    128,000 raw ids projected to 98,560, prime tables from rows_per_table up.
    Seeds under configuration id 6."""
    lay = _layer(6, 0, vocab=128_000, vocab_c=98_560, max_n=max_n, heads=heads, prime_start=rows_per_table,
                 dim=dim, table_dtype=BF16, d=d, branches=branches, store_dtype=BF16, w_std=w_std)
    tokens = zipf_tokens(rng_for(6, 0, S_TOKENS), 128_000, 1.1, (B, T))
    H = _hidden(6, (B, T, branches, d), BF16)
    return Workload("shape-bf16", 6, BF16, B, T, tokens, H, [lay])


def hash_inputs_for(config: int, layer: int = 0) -> HashInputs:
    """Only the hash inputs of a configuration (no tables), for index tests."""
    if config == 0:
        return _hash_inputs(0, 0, 1000, 770, 3, 2, 1000, [1009, 1013, 1019, 1021])
    start = C4_PRIME_START if config == 4 else C1_PRIME_START
    return _hash_inputs(config, layer, 128_000, 98_560, 3, 8, start)


def uniform_control_tokens(config: int, B: int, T: int, vocab: int = 128_000) -> np.ndarray:
    """Raw ids drawn uniformly from the vocabulary, [B, T]: the no-reuse
    control of the gather's bandwidth."""
    return rng_for(config, 0, S_UNIFORM).integers(0, vocab, size=(B, T), dtype=np.int32)


def lfu_warmup_tokens(config: int, layer: int, n: int = 1 << 24, vocab: int = 128_000) -> np.ndarray:
    """Seeded Zipf(1.1) warm-up stream, shape [1, n], whose row-access counts
    decide the static LFU admission of the HBM hot cache."""
    return zipf_tokens(rng_for(config, layer, S_LFU), vocab, 1.1, (1, n))


# --------------------------------------------------------------------------
# Engram-Nine hot tier ("DeepSeek Engram series guide", experiment 3): the
# hot set is the most frequent n-grams of the training text.  Here it is the
# most frequent windows of a seeded Zipf(1.1) warm-up stream, counted on ids
# the caller has already projected; the hot rows are drawn like table rows.
# --------------------------------------------------------------------------

def hot_warmup_tokens(config: int, layer: int, n: int = 1 << 21, vocab: int = 128_000) -> np.ndarray:
    """Seeded Zipf(1.1) warm-up stream, shape [1, n], whose most frequent
    n-grams form the hot set."""
    return zipf_tokens(rng_for(config, layer, S_HOT), vocab, 1.1, (1, n))


def frequent_ngrams(ids: np.ndarray, n: int, n_hot: int) -> np.ndarray:
    """The n_hot most frequent length-n windows of the rows of ids (int [R, L]);
    windows stay inside a row.  Ties go to the smaller window in lexicographic
    order.  Returns int32 [min(n_hot, distinct), n], most frequent first,
    each window oldest id first."""
    ids = np.asarray(ids, dtype=np.int64)
    rows = [np.lib.stride_tricks.sliding_window_view(r, n) for r in ids if r.shape[0] >= n]
    if not rows or n_hot <= 0:
        return np.zeros((0, n), dtype=np.int32)
    wins = np.concatenate(rows, axis=0)
    if n <= 3 and ids.size and 0 <= ids.min() and ids.max() < (1 << 21):
        # 21 bits per id, oldest id most significant: numeric order of the
        # packed words is the lexicographic order of the windows
        packed = np.zeros(wins.shape[0], dtype=np.int64)
        for i in range(n):
            packed = (packed << 21) | wins[:, i]
        uk, counts = np.unique(packed, return_counts=True)
        uniq = np.stack([(uk >> (21 * (n - 1 - i))) & ((1 << 21) - 1) for i in range(n)], axis=1)
    else:
        uniq, counts = np.unique(wins, axis=0, return_counts=True)     # lexicographic order
    order = np.argsort(-counts, kind="stable")[:n_hot]
    return np.ascontiguousarray(uniq[order].astype(np.int32))


def hot_rows(config: int, layer: int, n: int, n_hot: int, width: int, dtype: str, std: float = 0.02):
    """Hot rows of order n: [n_hot, width] N(0, std), as bf16 bits or float32."""
    rng = rng_for(config, layer, S_HOT * 16 + n)
    if dtype == BF16:
        return normal_bf16_bits(rng, n_hot * width, std).reshape(n_hot, width)
    return normal_f32(rng, n_hot * width, std).reshape(n_hot, width)


# --------------------------------------------------------------------------
# Rotations of distinct batches for timing: batch 0 is the workload's own;
# batch i > 0 is drawn like it from SeedSequence([config, i, S_RING]) (token
# ids) or SeedSequence([config, i, S_RING + 1]) (hidden states).
# --------------------------------------------------------------------------

def token_batch(config: int, i: int, shape, vocab: int = 128_000) -> np.ndarray:
    """Batch i of a rotation of Zipf(1.1) token batches of `shape`."""
    return zipf_tokens(rng_for(config, i, S_RING), vocab, 1.1, shape)


def hidden_batch(config: int, i: int, shape, dtype: str = BF16) -> np.ndarray:
    """Hidden states of batch i of a rotation, N(0, 1), as bf16 bits or float32."""
    rng = rng_for(config, i, S_RING + 1)
    n = int(np.prod(shape))
    if dtype == BF16:
        return normal_bf16_bits(rng, n, 1.0).reshape(shape)
    return normal_f32(rng, n, 1.0).reshape(shape)
