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
#include "device_util.h"
#include "engram_internal.h"
#include "hash_device.h"

namespace engram {
namespace {

constexpr int kOutMXFP8 = kGatherOutMXFP8;

template <int IN>
__device__ __forceinline__ void load8(const void* base, const float* scale, int64_t row, int dim,
                                      int col, float* f, uint4* raw_bf16) {
  if constexpr (IN == ENGRAM_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * dim + col);
    *raw_bf16 = q;
    unpack8(q, f);
  } else if constexpr (IN == ENGRAM_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * dim + col);
    const float4 a = p[0], b = p[1];
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

template <int IN, int OUT, bool HASHED>
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
  int32_t zj;
  if constexpr (HASHED) {
    const int64_t bt = tj / nt;
    const int64_t b = bt / hs.T;
    zj = hash_index(hs.tokens, hs.proj, hs.hist, hs.a, j, b, bt - b * hs.T, hs.T);
  } else {
    zj = z[tj];
  }
  int64_t row = ta.row_offset[j] + zj;
  if (ta.counts != nullptr && c == 0) atomicAdd(ta.counts + row, 1u);   // access statistics (real-time LFU)
  const void* src = ta.rows;
  const float* scale = ta.scale;
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

template <int IN, bool HASHED>
hipError_t launch_in(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out, void* e,
                     const HashSrc& hs, hipStream_t s) {
  const int64_t total = n_tok * ta.n_tables * (ta.dim / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const dim3 grid(static_cast<unsigned>((total + threads - 1) / threads));
  if (out == kOutMXFP8)
    launch_k((gather_kernel<IN, kOutMXFP8, HASHED>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  else if (out == ENGRAM_BF16)
    launch_k((gather_kernel<IN, ENGRAM_BF16, HASHED>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  else
    launch_k((gather_kernel<IN, ENGRAM_F32, HASHED>), grid, dim3(threads), 0, s, z, n_tok, ta, e, hs);
  return hipGetLastError();
}

template <bool HASHED>
hipError_t dispatch(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype, void* e,
                    const HashSrc& hs, hipStream_t s) {
  switch (ta.dtype) {
    case ENGRAM_BF16: return launch_in<ENGRAM_BF16, HASHED>(z, n_tok, ta, out_dtype, e, hs, s);
    case ENGRAM_F32: return launch_in<ENGRAM_F32, HASHED>(z, n_tok, ta, out_dtype, e, hs, s);
    default: return launch_in<ENGRAM_I8, HASHED>(z, n_tok, ta, out_dtype, e, hs, s);
  }
}

}  // namespace

hipError_t launch_gather(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype,
                         void* e, hipStream_t s) {
  return dispatch<false>(z, n_tok, ta, out_dtype, e, HashSrc{}, s);
}

hipError_t launch_hash_gather(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                              const int32_t* proj, const HashArgs& a, const TableArgs& ta,
                              int out_dtype, void* e, hipStream_t s) {
  HashSrc hs{tokens, proj, hist, T, a};
  return dispatch<true>(nullptr, B * T, ta, out_dtype, e, hs, s);
}

}  // namespace engram
