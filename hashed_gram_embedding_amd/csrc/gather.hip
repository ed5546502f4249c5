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
#include "gather_device.h"

namespace engram {
namespace {

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
  int64_t zj = z[tj];
  if constexpr (kDebugChecks) {
    debug_record(ta.err, range_bit(zj, ta.n_rows[j], kErrRow));
    zj = clamp_index(zj, ta.n_rows[j]);
  }
  int64_t row = row_offset + zj;
  const void* src = ta.rows;
  const float* scale = ta.scale;
  if (ta.counts != nullptr && c == 0) atomicAdd(ta.counts + row, 1u);   // access statistics (real-time LFU)
  if (ta.cache_slot != nullptr) {
    int32_t slot = ta.cache_slot[row];
    if constexpr (kDebugChecks) {
      uint32_t bits = 0;
      slot = checked_slot(slot, ta.cache_n, &bits);
      debug_record(ta.err, bits);
    }
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

// Steps 1-4 with in-thread hashing (hashed_gather_body in gather_device.h).
template <int IN, int OUT, bool HOT, int ITEMS>
__global__ void __launch_bounds__(256)
hashed_gather_kernel(uint32_t n_tok, TableArgs ta, void* __restrict__ e, HashSrc hs) {
  hashed_gather_body<IN, OUT, HOT, ITEMS>(blockIdx.x * blockDim.x + threadIdx.x, n_tok, ta, e, hs);
}

// Two layers' hashed gathers in one launch (the retrieval of several layers
// ahead of their hidden states): workgroups below split serve job a, the rest
// job b.  Both have the same table and row formats.
template <int IN, int OUT, int ITEMS>
__global__ void __launch_bounds__(256)
hashed_gather2_kernel(GatherJob a, GatherJob b, uint32_t split) {
  if (blockIdx.x < split)
    hashed_gather_body<IN, OUT, false, ITEMS>(blockIdx.x * blockDim.x + threadIdx.x, a.n_tok, a.ta, a.e, a.hs);
  else
    hashed_gather_body<IN, OUT, false, ITEMS>((blockIdx.x - split) * blockDim.x + threadIdx.x, b.n_tok, b.ta, b.e,
                                              b.hs);
}

template <int IN, int OUT>
hipError_t launch_gather2_t(const GatherJob& a, const GatherJob& b, hipStream_t s) {
  // one item count for both (layer a's choice; any count is correct)
  const int items = gather_items(a.n_tok, static_cast<int64_t>(a.ta.n_tables) * (a.ta.dim / 8));
  auto blocks = [&](const GatherJob& j) {
    const int64_t per_group = static_cast<int64_t>(j.ta.n_tables) * (j.ta.dim / 8);
    return ((static_cast<int64_t>(j.n_tok) + items - 1) / items * per_group + 255) / 256;
  };
  const int64_t na = blocks(a), nb = blocks(b);
  if (na + nb >= (int64_t{1} << 31) / 256) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(na + nb));
  const uint32_t split = static_cast<uint32_t>(na);
  if (items == 4)
    launch_k((hashed_gather2_kernel<IN, OUT, 4>), grid, dim3(256), 0, s, a, b, split);
  else if (items == 2)
    launch_k((hashed_gather2_kernel<IN, OUT, 2>), grid, dim3(256), 0, s, a, b, split);
  else
    launch_k((hashed_gather2_kernel<IN, OUT, 1>), grid, dim3(256), 0, s, a, b, split);
  return hipGetLastError();
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
  const int items = gather_items(n_tok, per_group);
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
  if (out == kOutFrag16) return launch_hashed_items<IN, kOutFrag16, HOT>(n_tok, ta, e, hs, s);
  if (out == ENGRAM_BF16) return launch_hashed_items<IN, ENGRAM_BF16, HOT>(n_tok, ta, e, hs, s);
  return launch_hashed_items<IN, ENGRAM_F32, HOT>(n_tok, ta, e, hs, s);
}

template <int IN>
hipError_t launch_gather2_in(const GatherJob& a, const GatherJob& b, hipStream_t s) {
  if (a.out_dtype == kOutMXFP8) return launch_gather2_t<IN, kOutMXFP8>(a, b, s);
  if (a.out_dtype == kOutFrag16) return launch_gather2_t<IN, kOutFrag16>(a, b, s);
  if (a.out_dtype == ENGRAM_BF16) return launch_gather2_t<IN, ENGRAM_BF16>(a, b, s);
  return launch_gather2_t<IN, ENGRAM_F32>(a, b, s);
}

}  // namespace

hipError_t launch_hash_gather2(const GatherJob& a, const GatherJob& b, hipStream_t s) {
  if (a.hot || b.hot || a.ta.dtype != b.ta.dtype || a.out_dtype != b.out_dtype) return hipErrorNotSupported;
  if (a.n_tok == 0 && b.n_tok == 0) return hipSuccess;
  switch (a.ta.dtype) {
    case ENGRAM_BF16: return launch_gather2_in<ENGRAM_BF16>(a, b, s);
    case ENGRAM_F32: return launch_gather2_in<ENGRAM_F32>(a, b, s);
    default: return launch_gather2_in<ENGRAM_I8>(a, b, s);
  }
}

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
