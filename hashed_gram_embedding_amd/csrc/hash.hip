// Steps 1-3 of "DeepSeek Engram series guide", section "Engram working
// principle": vocabulary projection, suffix n-grams and the K-head
// multiplicative-XOR hash into prime-sized tables.
//
// One thread per (token, table j).  The thread projects the n ids of its
// suffix window through P (reading the decode history, or pad id 0, before
// the sequence start), XORs the 64-bit wrapped products x' * m_{n,k,i} and
// reduces modulo the table's prime.  The table index is the fastest-varying
// thread coordinate, so the z stores of a wavefront are contiguous.
#include "engram_internal.h"

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
  const int n = a.order[j];
  const int hist_len = a.max_n - 1;
  uint64_t acc = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t p = t - i;
    uint32_t x = 0;
    if (p >= 0) {
      x = static_cast<uint32_t>(proj[tokens[b * T + p]]);
    } else if (hist != nullptr) {
      x = static_cast<uint32_t>(hist[b * hist_len + hist_len + p]);
    }
    acc ^= static_cast<uint64_t>(x) * a.mult[j][i];
  }
  z[gid] = static_cast<int32_t>(acc % static_cast<uint64_t>(a.prime[j]));
}

}  // namespace

hipError_t launch_hash(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                       const int32_t* proj, const HashArgs& a, int32_t* z, hipStream_t s) {
  const int64_t total = B * T * a.n_tables;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(hash_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s,
                     tokens, B, T, hist, proj, a, z);
  return hipGetLastError();
}

}  // namespace engram
