// Steps 1-3 of "DeepSeek Engram series guide", section "Engram working
// principle": vocabulary projection, suffix n-grams and the K-head
// multiplicative-XOR hash into prime-sized tables.
//
// One thread per (token, table j), table index fastest so that the z stores
// of a wavefront are contiguous.  The per-thread work (up to N id loads, N
// 64-bit products, one Barrett reduction) is described in hash_device.h.
#include "engram_internal.h"
#include "hash_device.h"

namespace engram {
namespace {

__global__ void __launch_bounds__(256)
hash_kernel(const int32_t* __restrict__ tokens, int64_t B, int64_t T,
            const int32_t* __restrict__ hist, const int32_t* __restrict__ proj, HashArgs a,
            int32_t* __restrict__ z) {
  const int nt = a.n_tables;
  const int64_t total = B * T * nt;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int j = static_cast<int>(gid % nt);
  const int64_t bt = gid / nt;
  const int64_t b = bt / T;
  const int64_t t = bt - b * T;
  z[gid] = hash_index(tokens, proj, hist, a, j, b, t, T);
}

}  // namespace

hipError_t launch_hash(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                       const int32_t* proj, const HashArgs& a, int32_t* z, hipStream_t s) {
  const int64_t total = B * T * a.n_tables;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  launch_k(hash_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s,
                     tokens, B, T, hist, proj, a, z);
  return hipGetLastError();
}

}  // namespace engram
