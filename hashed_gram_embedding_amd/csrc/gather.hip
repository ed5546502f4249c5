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
// (Steps 1-3), so the indices never go through memory.  With access counts
// given, the first thread of each row access adds 1 to the row's count.
//
// With the Engram-Nine hot tier ("DeepSeek Engram series guide", experiment
// 3, Figure 1) the same thread first looks its n-gram up in the hot set of
// its order; on a hit it copies its 8 elements from the n-gram's hot row
// (head k of order n covers columns k*dim .. k*dim+dim-1 of that row) and
// reads no cold row.  With K*dim/8 = 64 a wavefront holds exactly one
// (token, order), so the lookup is uniform across it.
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

template <int IN, int OUT, bool HASHED, bool HOT>
__global__ void __launch_bounds__(256)
gather_kernel(const int32_t* __restrict__ z, int64_t n_tok, TableArgs ta, void* __restrict__ e,
              HashSrc hs) {
  const int nt = ta.n_tables;
  const int chunks = ta.dim >> 3;
  const int64_t total = n_tok * nt * chunks;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int c = static_cast<int>(gid % chunks);
  const int64_t tj = gid / chunks;
  const int j = static_cast<int>(tj % nt);
  // per-table arguments first: their loads overlap the id loads
  const int64_t row_offset = ta.row_offset[j];
  int32_t zj;
  int32_t hot_row = -1;
  const void* hot_src = nullptr;
  int hot_col = 0;
  if constexpr (HASHED) {
    const TableHash th = table_hash(hs.a, j);
    const int64_t bt = tj / nt;
    const int64_t b = bt / hs.T;
    uint32_t x[ENGRAM_MAX_ORDER];
    window_ids(hs.tokens, hs.proj, hs.hist, hs.a.max_n, b, bt - b * hs.T, hs.T, x);
    zj = hash_of_ids(x, th);
    if constexpr (HOT) {
      const int n = th.n;
      const HotOrderArgs o = hot_order(hs.hot, n);
      hot_row = hot_find(x, n, o);
      hot_src = o.rows;
      hot_col = (j - (n - 2) * hs.hot.heads) * ta.dim + c * 8;
    }
  } else {
    zj = z[tj];
  }
  const void* src = ta.rows;
  const float* scale = ta.scale;
  int64_t row;
  int row_len = ta.dim;
  int col = c * 8;
  if (HOT && hot_row >= 0) {
    src = hot_src;
    row = hot_row;
    row_len = hs.hot.width;
    col = hot_col;
  } else {
    row = row_offset + zj;
    if (ta.counts != nullptr && c == 0) atomicAdd(ta.counts + row, 1u);   // access statistics (real-time LFU)
    if (ta.cache_slot != nullptr) {
      const int32_t slot = ta.cache_slot[row];
      if (slot >= 0) {
        src = ta.cache_rows;
        scale = ta.cache_scale;
        row = slot;
      }
    }
  }
  float f[8];
  uint4 raw;
  load8<IN>(src, scale, row, row_len, col, f, &raw);
  const int64_t out = tj * ta.dim + c * 8;
  if constexpr (OUT == kOutMXFP8) {
    // MXFP8 e: 8 codes per thread, the block scale from the 4 threads of the
    // block (rows are whole blocks: dim is a multiple of 32, so the groups
    // of 4 lanes never straddle rows or the grid's end)
    uint32_t sb;
    const uint2 q = mx_quantize8(f, &sb);
    uint8_t* eq = static_cast<uint8_t*>(e);
    *reinterpret_cast<uint2*>(eq + out) = q;
    if ((c & 3) == 0) eq[n_tok * nt * ta.dim + out / 32] = static_cast<uint8_t>(sb);
  } else if constexpr (OUT == ENGRAM_BF16) {
    uint4 q;
    if constexpr (IN == ENGRAM_BF16) q = raw; else q = pack8(f);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(e) + out) = q;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(e) + out);
    p[0] = make_float4(f[0], f[1], f[2], f[3]);
    p[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

template <int IN, bool HASHED, bool HOT>
hipError_t launch_in(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out, void* e,
                     const HashSrc& hs, hipStream_t s) {
  const int64_t total = n_tok * ta.n_tables * (ta.dim / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  if (out == kOutMXFP8)
    launch_k((gather_kernel<IN, kOutMXFP8, HASHED, HOT>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  else if (out == ENGRAM_BF16)
    launch_k((gather_kernel<IN, ENGRAM_BF16, HASHED, HOT>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  else
    launch_k((gather_kernel<IN, ENGRAM_F32, HASHED, HOT>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  return hipGetLastError();
}

// The hot tier holds F32 or BF16 rows only (checked by the caller), so int8
// tables have no hot variant.
template <bool HASHED, bool HOT>
hipError_t dispatch(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype, void* e,
                    const HashSrc& hs, hipStream_t s) {
  switch (ta.dtype) {
    case ENGRAM_BF16: return launch_in<ENGRAM_BF16, HASHED, HOT>(z, n_tok, ta, out_dtype, e, hs, s);
    case ENGRAM_F32: return launch_in<ENGRAM_F32, HASHED, HOT>(z, n_tok, ta, out_dtype, e, hs, s);
    default:
      if constexpr (HOT) return hipErrorInvalidValue;
      else return launch_in<ENGRAM_I8, HASHED, false>(z, n_tok, ta, out_dtype, e, hs, s);
  }
}

}  // namespace

hipError_t launch_gather(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype,
                         void* e, hipStream_t s) {
  return dispatch<false, false>(z, n_tok, ta, out_dtype, e, HashSrc{}, s);
}

hipError_t launch_hash_gather(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                              const int32_t* proj, const HashArgs& a, const TableArgs& ta,
                              const HotArgs* hot, int out_dtype, void* e, hipStream_t s) {
  HashSrc hs{tokens, proj, hist, T, a, hot != nullptr ? *hot : HotArgs{}};
  if (hot != nullptr) return dispatch<true, true>(nullptr, B * T, ta, out_dtype, e, hs, s);
  return dispatch<true, false>(nullptr, B * T, ta, out_dtype, e, hs, s);
}

}  // namespace engram
