// Device-side Steps 1-3 ("DeepSeek Engram series guide", section "Engram
// working principle"): projection, suffix n-gram and multiplicative-XOR hash
// of one (token, table) pair, shared by the hash and the fused hash+gather
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram_internal.h"

namespace engram {

// x mod p for a 64-bit x and p < 2^31, with inv = floor((2^64-1)/p):
// q = floor(x * inv / 2^64) is floor(x/p) or one less, so r = x - q p lies in
// [0, 2p) and one conditional subtraction finishes (Barrett reduction).
__device__ __forceinline__ uint32_t mod_prime(uint64_t x, uint32_t p, uint64_t inv) {
  const uint64_t q = __umul64hi(x, inv);
  const uint64_t r = x - q * static_cast<uint64_t>(p);
  return static_cast<uint32_t>(r >= p ? r - p : r);
}

// z of table j at position t of sequence b: XOR over i < n of
// x'_{t-i} * m_{j,i} (wrapping in 64 bits), then mod p_j.  Positions before the
// sequence start read the history (oldest first) or the pad id 0.
__device__ __forceinline__ int32_t hash_index(const int32_t* __restrict__ tokens,
                                              const int32_t* __restrict__ proj,
                                              const int32_t* __restrict__ hist, const HashArgs& a,
                                              int j, int64_t b, int64_t t, int64_t T) {
  const int n = a.order[j];
  const int hist_len = a.max_n - 1;
  // Unrolled to the largest order, with clamped (always valid) positions, so
  // that the token loads of all positions and then their P lookups are each
  // issued together; positions before the sequence start are patched from
  // the history afterwards.
  int32_t tok[ENGRAM_MAX_ORDER];
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) {
    const int64_t p = t - i;
    tok[i] = tokens[b * T + (p >= 0 ? p : 0)];
  }
  uint32_t x[ENGRAM_MAX_ORDER];
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) x[i] = static_cast<uint32_t>(proj[tok[i]]);
  if (t < hist_len) {
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) {
      const int64_t p = t - i;
      if (p < 0) x[i] = hist != nullptr && hist_len + p >= 0 ? static_cast<uint32_t>(hist[b * hist_len + hist_len + p]) : 0u;
    }
  }
  uint64_t acc = 0;
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i)
    if (i < n) acc ^= static_cast<uint64_t>(x[i]) * a.mult[j][i];
  return static_cast<int32_t>(mod_prime(acc, a.prime[j], a.inv[j]));
}

}  // namespace engram
