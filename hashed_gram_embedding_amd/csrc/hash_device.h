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

__device__ __forceinline__ WindowSrc window_src(const HashSrc& hs) {
  return WindowSrc{hs.tokens, hs.proj, hs.hist, hs.a.err, static_cast<int32_t>(hs.T), hs.a.max_n, hs.a.vocab};
}

// Steps 1-2 for ITEMS tokens at positions t[q] of sequences b[q], in two
// halves so that a kernel can issue other loads in between.  window_loads
// loads the P values of the window's tokens (xp) and the history ids that
// positions before the sequence start need (hv, 0 where there are none).
// With HIST_ALL the history index does not depend on the token ids, so
// those loads go out just before the token loads, into registers of their
// own, and the P lookups take the second and last memory latency.  (Memory
// reads return in order, so once the P lookups are issued the history has
// arrived.)
// window_select then forms x[q][i] = x'_{t-i}, newest first.
// HIST_ALL: the caller guarantees hs.hist != null and T <= max_n - 1 (every
// token reads history, as in decode), so that the choice below is not a
// branch in the kernel.
template <int ITEMS, bool HIST_ALL = false>
__device__ __forceinline__ void window_loads(const WindowSrc& hs, const uint32_t (&b)[ITEMS],
                                             const uint32_t (&t)[ITEMS], uint32_t (&xp)[ITEMS][ENGRAM_MAX_ORDER],
                                             uint32_t (&hv)[ITEMS][ENGRAM_MAX_ORDER]) {
  const uint32_t T = static_cast<uint32_t>(hs.T);
  const int hl = hs.max_n - 1;
  // every token reads history (decode): loads without branches or selects,
  // so that none waits for another.  For i <= hl and t < i the index
  // hl + t - i is in range; positions i > hl (>= the largest order) enter no
  // hash (their multipliers are 0) and no hot key, so the clamped index
  // serves them as well as the pad would.
  auto hist_all = [&]() {
#pragma unroll
    for (int q = 0; q < ITEMS; ++q)
#pragma unroll
      for (int i = 1; i < ENGRAM_MAX_ORDER; ++i) {
        const int idx = hl + static_cast<int>(t[q]) - i;   // index in the history of position t - i
        hv[q][i] = static_cast<uint32_t>(hs.hist[b[q] * hl + min(max(idx, 0), hl - 1)]);
      }
  };
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) hv[q][i] = 0u;
  if constexpr (HIST_ALL) hist_all();
  int32_t tk[ITEMS][ENGRAM_MAX_ORDER];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i)
      tk[q][i] = hs.tokens[b[q] * T + (t[q] >= static_cast<uint32_t>(i) ? t[q] - i : 0u)];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i)
      xp[q][i] = static_cast<uint32_t>(hs.proj[token_in_vocab(tk[q][i], hs.vocab, hs.err)]);
  // Otherwise the history (if any) is read after the P lookups are issued:
  // its branches ahead of the token loads made the compiler wait, on every
  // path, for the loads issued before them (the callers' table constants)
  // before reading the token ids.
  if constexpr (!HIST_ALL) {
    if (hs.hist != nullptr && T <= static_cast<uint32_t>(hl)) {
      hist_all();
    } else if (hs.hist != nullptr) {
      // only tokens near a sequence start do
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        if (t[q] < static_cast<uint32_t>(hl)) {
#pragma unroll
          for (int i = 1; i < ENGRAM_MAX_ORDER; ++i) {
            const int idx = hl + static_cast<int>(t[q]) - i;
            if (idx >= 0 && idx < hl) hv[q][i] = static_cast<uint32_t>(hs.hist[b[q] * hl + idx]);
          }
        }
      }
    }
  }
}

template <int ITEMS>
__device__ __forceinline__ void window_select(const uint32_t (&t)[ITEMS], const uint32_t (&xp)[ITEMS][ENGRAM_MAX_ORDER],
                                              const uint32_t (&hv)[ITEMS][ENGRAM_MAX_ORDER],
                                              uint32_t (&x)[ITEMS][ENGRAM_MAX_ORDER]) {
#pragma unroll
  for (int q = 0; q < ITEMS; ++q)
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER; ++i)
      x[q][i] = t[q] >= static_cast<uint32_t>(i) ? xp[q][i] : hv[q][i];   // before the start: history or pad 0
}

template <int ITEMS>
__device__ __forceinline__ void window_ids_n(const HashSrc& hs, const uint32_t (&b)[ITEMS],
                                             const uint32_t (&t)[ITEMS], uint32_t (&x)[ITEMS][ENGRAM_MAX_ORDER]) {
  uint32_t xp[ITEMS][ENGRAM_MAX_ORDER], hv[ITEMS][ENGRAM_MAX_ORDER];
  window_loads<ITEMS>(window_src(hs), b, t, xp, hv);
  window_select<ITEMS>(t, xp, hv, x);
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

// Decode-state advance (ProjGateArgs.adv_B > 0), by the threads of
// workgroup 0: ids <- last N-1 of (ids ++ P(tokens)), pos += T.
__device__ __forceinline__ void advance_state(const ProjGateArgs& a, uint32_t bid) {
  if (a.adv_B <= 0 || bid != 0) return;
  const int hl = a.max_n - 1;
  for (int b = threadIdx.x; b < a.adv_B; b += blockDim.x) {
    int32_t next[ENGRAM_MAX_ORDER];
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER - 1; ++i) {
      if (i < hl) {
        const int64_t idx = static_cast<int64_t>(a.adv_T) + i;   // index in (old ids ++ chunk ids)
        next[i] = idx < hl ? a.st_ids[static_cast<int64_t>(b) * hl + idx]
                           : a.proj[token_in_vocab(a.tokens[static_cast<int64_t>(b) * a.adv_T + idx - hl], a.vocab,
                                                   a.err)];
      }
    }
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER - 1; ++i)
      if (i < hl) a.st_ids[static_cast<int64_t>(b) * hl + i] = next[i];
    a.st_pos[b] += a.adv_T;
  }
}

}  // namespace engram
