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

// Raw token ids are the caller's contract (0 <= id < vocab); an id outside
// that range is clamped into it, so that P is never read out of bounds (the
// result for such a token is then that of the clamped id), and the debug
// build reports it in the error word.
__device__ __forceinline__ int32_t token_in_vocab(int32_t tk, int32_t vocab, uint32_t* err) {
  debug_record(err, range_bit(tk, vocab, kErrToken));
  return min(max(tk, 0), vocab - 1);
}

// Compressed ids of the suffix window at position t of sequence b, newest
// first: x[i] = x'_{t-i} for i < ENGRAM_MAX_ORDER.  Positions before the
// sequence start read the history (oldest first) or the pad id 0.
__device__ __forceinline__ void window_ids(const int32_t* __restrict__ tokens, const int32_t* __restrict__ proj,
                                           const int32_t* __restrict__ hist, int max_n, int32_t vocab,
                                           uint32_t* err, int64_t b, int64_t t, int64_t T,
                                           uint32_t (&x)[ENGRAM_MAX_ORDER]) {
  const int hist_len = max_n - 1;
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
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) x[i] = static_cast<uint32_t>(proj[token_in_vocab(tok[i], vocab, err)]);
  if (t < hist_len) {
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) {
      const int64_t p = t - i;
      if (p < 0) x[i] = hist != nullptr && hist_len + p >= 0 ? static_cast<uint32_t>(hist[b * hist_len + hist_len + p]) : 0u;
    }
  }
}

// Hash constants of table j.  Kernels read them before the token ids, so
// that these argument loads and the id loads are in flight together.  The
// multipliers of positions i >= n are 0, so every position can be taken
// unconditionally.
struct TableHash {
  uint64_t m[ENGRAM_MAX_ORDER];
  uint64_t inv;
  uint32_t prime;
  int32_t n;
};

__device__ __forceinline__ TableHash table_hash(const HashArgs& a, int j) {
  TableHash th;
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) th.m[i] = a.mult[j][i];
  th.inv = a.inv[j];
  th.prime = a.prime[j];
  th.n = a.order[j];
  return th;
}

// z of a table from the window ids: XOR over i < n of x'_{t-i} * m_i
// (wrapping in 64 bits), then mod p.
__device__ __forceinline__ int32_t hash_of_ids(const uint32_t (&x)[ENGRAM_MAX_ORDER], const TableHash& th) {
  uint64_t acc = 0;
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) acc ^= static_cast<uint64_t>(x[i]) * th.m[i];
  return static_cast<int32_t>(mod_prime(acc, th.prime, th.inv));
}

// z of table j at position t of sequence b.
__device__ __forceinline__ int32_t hash_index(const int32_t* __restrict__ tokens,
                                              const int32_t* __restrict__ proj,
                                              const int32_t* __restrict__ hist, const HashArgs& a,
                                              int j, int64_t b, int64_t t, int64_t T) {
  const TableHash th = table_hash(a, j);
  uint32_t x[ENGRAM_MAX_ORDER];
  window_ids(tokens, proj, hist, a.max_n, a.vocab, a.err, b, t, T, x);
  return hash_of_ids(x, th);
}

}  // namespace engram
