// Steps 3-4 of "DeepSeek Engram series guide", section "Engram working
// principle": e_t = concat over tables j = (n-2)K + k of E_j[z_{t,j}].
//
// Rows may sit in HBM or in pinned host memory read over PCIe through its
// device alias, and an optional HBM hot cache is probed first; int8 rows are
// dequantised on the fly.  This follows the single select-and-dequantise
// kernel that reads HBM or pinned host memory in "Engram embedding
// expansion: co-design for DRAM/SSD offload" (DRAM offload section), with the
// hot-row cache of the Ascend RecSDK Engram article (multi-level cache).
//
// One thread moves 8 consecutive elements of one row: a 16-byte load for
// bf16, 32 bytes for f32, 8 bytes for int8.  Threads are ordered (token,
// table, chunk), so the 8 threads that cover a 128-byte bf16 row are
// adjacent and each wavefront writes a contiguous 1 KiB span of e.
//
// Inside the layer forward the row index is hashed in the same thread
// (Steps 1-3), so the indices never go through memory, and each thread
// serves ITEMS consecutive tokens of one (table, chunk): every phase (token
// ids, P, hot-set probes, cache probes, rows) issues its loads for all items
// before it waits for the first, so a wavefront keeps ITEMS dependent chains
// in flight instead of one.  With access counts given, the first thread of
// each row access adds 1 to the row's count.
//
// With the Engram-Nine hot tier ("DeepSeek Engram series guide", experiment
// 3, Figure 1) the same thread first looks its n-gram up in the hot set of
// its order; on a hit it copies its 8 elements from the n-gram's hot row
// (head k of order n covers columns k*dim .. k*dim+dim-1 of that row) and
// reads no cold row.
#include "device_util.h"
#include "engram_internal.h"
#include "hash_device.h"
#include "hot_device.h"

namespace engram {
namespace {

constexpr int kOutMXFP8 = kGatherOutMXFP8;

template <int IN>
__device__ __forceinline__ void load8(const void* base, const float* scale, int64_t row, int dim,
                                      int col, float* f, uint4* raw_bf16) {
  if constexpr (IN == ENGRAM_BF16) {
    const uint4 q = global_load16(static_cast<const uint16_t*>(base) + row * dim + col);
    *raw_bf16 = q;
    unpack8(q, f);
  } else if constexpr (IN == ENGRAM_F32) {
    const float* p = static_cast<const float*>(base) + row * dim + col;
    const uint4 qa = global_load16(p), qb = global_load16(p + 4);
    const float4 a = make_float4(__uint_as_float(qa.x), __uint_as_float(qa.y), __uint_as_float(qa.z),
                                 __uint_as_float(qa.w));
    const float4 b = make_float4(__uint_as_float(qb.x), __uint_as_float(qb.y), __uint_as_float(qb.z),
                                 __uint_as_float(qb.w));
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + row * dim + col);
    const float s = scale[row];
    const uint32_t w[2] = {q.x, q.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int8_t v = static_cast<int8_t>((w[i >> 2] >> (8 * (i & 3))) & 0xffu);
      f[i] = static_cast<float>(v) * s;
    }
  }
}

// Writes the 8 elements of one thread at element offset `out` of e.
template <int IN, int OUT>
__device__ __forceinline__ void store8(void* e, int64_t out, int64_t mx_scale_base, int c, const float* f,
                                       const uint4& raw, bool live) {
  if constexpr (OUT == kOutMXFP8) {
    // MXFP8 e: 8 codes per thread, the block scale from the 4 threads of the
    // block (rows are whole blocks: dim is a multiple of 32, so the groups
    // of 4 lanes never straddle rows or the grid's end; every lane of the
    // group takes part in the shuffle, stores are predicated)
    uint32_t sb;
    const uint2 q = mx_quantize8(f, &sb);
    uint8_t* eq = static_cast<uint8_t*>(e);
    if (live) {
      *reinterpret_cast<uint2*>(eq + out) = q;
      if ((c & 3) == 0) eq[mx_scale_base + out / 32] = static_cast<uint8_t>(sb);
    }
  } else if constexpr (OUT == ENGRAM_BF16) {
    uint4 q;
    if constexpr (IN == ENGRAM_BF16) q = raw; else q = pack8(f);
    if (live) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(e) + out) = q;
  } else {
    if (live) {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(e) + out);
      p[0] = make_float4(f[0], f[1], f[2], f[3]);
      p[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
}

// Gather from given indices z [n_tok][n_tables]: one (token, table, chunk)
// per thread.
template <int IN, int OUT>
__global__ void __launch_bounds__(256)
gather_kernel(const int32_t* __restrict__ z, int64_t n_tok, TableArgs ta, void* __restrict__ e) {
  const int nt = ta.n_tables;
  const int chunks = ta.dim >> 3;
  const int64_t total = n_tok * nt * chunks;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t tj = gid / chunks;
  const int j = static_cast<int>(tj % nt);
  const int64_t row_offset = ta.row_offset[j];
  int64_t row = row_offset + z[tj];
  const void* src = ta.rows;
  const float* scale = ta.scale;
  if (ta.counts != nullptr && c == 0) atomicAdd(ta.counts + row, 1u);   // access statistics (real-time LFU)
  if (ta.cache_slot != nullptr) {
    const int32_t slot = ta.cache_slot[row];
    if (slot >= 0) {
      src = ta.cache_rows;
      scale = ta.cache_scale;
      row = slot;
    }
  }
  float f[8];
  uint4 raw;
  load8<IN>(src, scale, row, ta.dim, c * 8, f, &raw);
  store8<IN, OUT>(e, tj * ta.dim + c * 8, n_tok * nt * ta.dim, c, f, raw, true);
}

// Steps 1-4 with in-thread hashing; ITEMS consecutive tokens per thread.
// Thread gid serves tokens ITEMS*g .. ITEMS*g + ITEMS-1 of table j, chunk c,
// with (g, j, c) = gid split as [groups][n_tables][chunks]; a wavefront's
// store of one item is a contiguous span of e.  Token counts below 2^31
// (checked by the launcher) keep the index arithmetic in 32 bits.
template <int IN, int OUT, bool HOT, int ITEMS>
__global__ void __launch_bounds__(256)
hashed_gather_kernel(uint32_t n_tok, TableArgs ta, void* __restrict__ e, HashSrc hs) {
  const uint32_t nt = static_cast<uint32_t>(ta.n_tables);
  const uint32_t chunks = static_cast<uint32_t>(ta.dim) >> 3;
  const uint32_t per_group = nt * chunks;
  const uint32_t n_groups = (n_tok + ITEMS - 1) / ITEMS;
  const uint32_t gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_groups * per_group) return;
  const uint32_t g = gid / per_group;
  const uint32_t jc = gid - g * per_group;
  const int j = static_cast<int>(jc / chunks);
  const int c = static_cast<int>(jc - static_cast<uint32_t>(j) * chunks);

  // per-table arguments first: their loads overlap the id loads
  const int64_t row_offset = ta.row_offset[j];
  const TableHash th = table_hash(hs.a, j);
  const uint32_t T = static_cast<uint32_t>(hs.T);
  const int hist_len = hs.a.max_n - 1;

  uint32_t b[ITEMS], t[ITEMS];
  bool live[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const uint32_t tok = g * ITEMS + q;
    live[q] = tok < n_tok;
    const uint32_t tc = live[q] ? tok : n_tok - 1;
    b[q] = tc / T;
    t[q] = tc - b[q] * T;
  }
  // Steps 1-2: ids of the suffix window, newest first (clamped positions,
  // patched from the history below)
  int32_t tk[ITEMS][ENGRAM_MAX_ORDER];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i)
      tk[q][i] = hs.tokens[b[q] * T + (t[q] >= static_cast<uint32_t>(i) ? t[q] - i : 0u)];
  uint32_t x[ITEMS][ENGRAM_MAX_ORDER];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) x[q][i] = static_cast<uint32_t>(hs.proj[tk[q][i]]);
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    if (t[q] < static_cast<uint32_t>(hist_len)) {
#pragma unroll
      for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) {
        const int p = static_cast<int>(t[q]) - i;
        if (p < 0)
          x[q][i] = hs.hist != nullptr && hist_len + p >= 0
                        ? static_cast<uint32_t>(hs.hist[b[q] * hist_len + hist_len + p]) : 0u;
      }
    }
  }
  // Step 3: cold row of every item
  int64_t crow[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) crow[q] = row_offset + hash_of_ids(x[q], th);

  // Engram-Nine: hot row of every item (-1 = cold)
  int32_t hot[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) hot[q] = -1;
  const void* hot_rows = nullptr;
  int hot_col = 0;
  if constexpr (HOT) {
    const int n = th.n;
    const HotOrderArgs o = hot_order(hs.hot, n);
    hot_rows = o.rows;
    hot_col = (j - (n - 2) * hs.hot.heads) * ta.dim + c * 8;
    if (o.n_hot != 0) {
      uint64_t h[ITEMS];
      uint32_t pilot[ITEMS];
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        h[q] = hot_key_hash(x[q], n, o.seed);
        pilot[q] = global_load(o.pilots + hot_range(h[q], o.n_buckets));
      }
      uint4 sa[ITEMS], sb[ITEMS];
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        const uint64_t sl = hot_slot(h[q], pilot[q], o.n_hot);
        sa[q] = global_load16(o.slots + 2 * sl);
        sb[q] = global_load16(o.slots + 2 * sl + 1);
      }
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        uint32_t xm[ENGRAM_MAX_ORDER];
#pragma unroll
        for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) xm[i] = i < n ? x[q][i] : 0u;
        const bool match = sa[q].x == xm[0] && sa[q].y == xm[1] && sa[q].z == xm[2] && sa[q].w == xm[3];
        hot[q] = match ? static_cast<int32_t>(sb[q].x) : -1;
      }
    }
  }

  // Step 4: the source of every item (hot row, HBM cache slot or table row)
  const void* src[ITEMS];
  const float* scale[ITEMS];
  int64_t row[ITEMS];
  int len[ITEMS], col[ITEMS];
  int32_t slot[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) slot[q] = -1;
  if (ta.cache_slot != nullptr) {
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) slot[q] = ta.cache_slot[crow[q]];
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const bool is_hot = HOT && hot[q] >= 0;
    const bool cached = !is_hot && slot[q] >= 0;
    src[q] = is_hot ? hot_rows : (cached ? ta.cache_rows : ta.rows);
    scale[q] = cached ? ta.cache_scale : ta.scale;
    row[q] = is_hot ? hot[q] : (cached ? slot[q] : crow[q]);
    len[q] = is_hot ? hs.hot.width : ta.dim;
    col[q] = is_hot ? hot_col : c * 8;
  }
  float f[ITEMS][8];
  uint4 raw[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) load8<IN>(src[q], scale[q], row[q], len[q], col[q], f[q], &raw[q]);
  if (ta.counts != nullptr && c == 0) {   // access statistics (real-time LFU): cold rows read
#pragma unroll
    for (int q = 0; q < ITEMS; ++q)
      if (live[q] && !(HOT && hot[q] >= 0)) atomicAdd(ta.counts + crow[q], 1u);
  }
  const int64_t dm = static_cast<int64_t>(nt) * ta.dim;
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
    store8<IN, OUT>(e, (static_cast<int64_t>(g) * ITEMS + q) * dm + j * ta.dim + c * 8,
                    static_cast<int64_t>(n_tok) * dm, c, f[q], raw[q], live[q]);
}

template <int IN>
hipError_t launch_in(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out, void* e, hipStream_t s) {
  const int64_t total = n_tok * ta.n_tables * (ta.dim / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  if (out == ENGRAM_BF16)
    launch_k((gather_kernel<IN, ENGRAM_BF16>), grid, dim3(threads), 0, s, z, n_tok, ta, e);
  else
    launch_k((gather_kernel<IN, ENGRAM_F32>), grid, dim3(threads), 0, s, z, n_tok, ta, e);
  return hipGetLastError();
}

template <int IN, int OUT, bool HOT>
hipError_t launch_hashed_items(int64_t n_tok, const TableArgs& ta, void* e, const HashSrc& hs, hipStream_t s) {
  const int64_t per_group = static_cast<int64_t>(ta.n_tables) * (ta.dim / 8);
  // Items per thread, by the wavefronts one item per thread would take:
  // 4 from 16384 wavefronts (8 x 4096 tokens: 26.6 -> 23.0 us, and 44.1 ->
  // 32.6 us with the hot tier, against 1 item), 2 from 4096 (4096 tokens:
  // about 7.0 -> 6.6 us inside the layer, where 4 items gave 6.8-7.8 us), 1
  // below, so that small launches still spread over the CUs.
  const int64_t waves1 = (n_tok * per_group + 63) / 64;
  const int items = waves1 >= 16384 ? 4 : (waves1 >= 4096 ? 2 : 1);
  const int64_t total = (n_tok + items - 1) / items * per_group;
  if (n_tok >= (1ll << 31) || total >= (1ll << 31)) return hipErrorInvalidConfiguration;
  const int threads = 256;
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  const uint32_t n = static_cast<uint32_t>(n_tok);
  if (items == 4)
    launch_k((hashed_gather_kernel<IN, OUT, HOT, 4>), grid, dim3(threads), 0, s, n, ta, e, hs);
  else if (items == 2)
    launch_k((hashed_gather_kernel<IN, OUT, HOT, 2>), grid, dim3(threads), 0, s, n, ta, e, hs);
  else
    launch_k((hashed_gather_kernel<IN, OUT, HOT, 1>), grid, dim3(threads), 0, s, n, ta, e, hs);
  return hipGetLastError();
}

template <int IN, bool HOT>
hipError_t launch_hashed(int64_t n_tok, const TableArgs& ta, int out, void* e, const HashSrc& hs, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (out == kOutMXFP8) return launch_hashed_items<IN, kOutMXFP8, HOT>(n_tok, ta, e, hs, s);
  if (out == ENGRAM_BF16) return launch_hashed_items<IN, ENGRAM_BF16, HOT>(n_tok, ta, e, hs, s);
  return launch_hashed_items<IN, ENGRAM_F32, HOT>(n_tok, ta, e, hs, s);
}

}  // namespace

hipError_t launch_gather(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype,
                         void* e, hipStream_t s) {
  switch (ta.dtype) {
    case ENGRAM_BF16: return launch_in<ENGRAM_BF16>(z, n_tok, ta, out_dtype, e, s);
    case ENGRAM_F32: return launch_in<ENGRAM_F32>(z, n_tok, ta, out_dtype, e, s);
    default: return launch_in<ENGRAM_I8>(z, n_tok, ta, out_dtype, e, s);
  }
}

// The hot tier holds F32 or BF16 rows only (checked by the caller), so int8
// tables have no hot variant.
hipError_t launch_hash_gather(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                              const int32_t* proj, const HashArgs& a, const TableArgs& ta,
                              const HotArgs* hot, int out_dtype, void* e, hipStream_t s) {
  const HashSrc hs{tokens, proj, hist, T, a, hot != nullptr ? *hot : HotArgs{}};
  const int64_t n_tok = B * T;
  if (hot != nullptr) {
    if (ta.dtype == ENGRAM_BF16) return launch_hashed<ENGRAM_BF16, true>(n_tok, ta, out_dtype, e, hs, s);
    if (ta.dtype == ENGRAM_F32) return launch_hashed<ENGRAM_F32, true>(n_tok, ta, out_dtype, e, hs, s);
    return hipErrorInvalidValue;
  }
  switch (ta.dtype) {
    case ENGRAM_BF16: return launch_hashed<ENGRAM_BF16, false>(n_tok, ta, out_dtype, e, hs, s);
    case ENGRAM_F32: return launch_hashed<ENGRAM_F32, false>(n_tok, ta, out_dtype, e, hs, s);
    default: return launch_hashed<ENGRAM_I8, false>(n_tok, ta, out_dtype, e, hs, s);
  }
}

}  // namespace engram
