// Engram-Nine hot tier ("DeepSeek Engram series guide", experiment 3
// "Engram-Nine", Figure 1: two-tier retrieval): the minimal perfect hash that
// indexes the hot n-grams of one order, and the device lookup against it.
//
// The hash is hash-and-displace with one pilot per bucket (the PTHash scheme
// of Pibiri and Trani, SIGIR 2021): an n-gram's 64-bit hash h picks a bucket;
// the bucket's pilot p, found at build time, sends every n-gram of the bucket
// to a distinct slot.  A slot holds the n-gram itself as its fingerprint and
// the n-gram's hot row, so a lookup costs two dependent loads (pilot, then
// the 32-byte slot) and is exact: an n-gram outside the set never matches.
//
// These functions are compiled for the host (the builder) and for the device
// (the lookup); both must give the same slot for every n-gram.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram_internal.h"

namespace engram {

// SplitMix64 finaliser (Steele, Lea and Flood, OOPSLA 2014): a bijection on
// 64-bit words with full avalanche.
__host__ __device__ __forceinline__ uint64_t hot_mix(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

// floor(a * b / 2^64): maps a uniform 64-bit a onto [0, b) (Lemire's
// multiply-shift range reduction).
__host__ __device__ __forceinline__ uint64_t hot_range(uint64_t a, uint64_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umul64hi(a, b);
#else
  return static_cast<uint64_t>((static_cast<unsigned __int128>(a) * b) >> 64);
#endif
}

// Buckets of a hot set of n_hot n-grams: about 4 n-grams per bucket.
__host__ __device__ __forceinline__ uint64_t hot_buckets(uint64_t n_hot) {
  return n_hot <= 4 ? 1 : (n_hot + 3) / 4;
}

// h of an n-gram given newest id first (x[i] = x'_{t-i}, i < n).
template <int MAXN>
__host__ __device__ __forceinline__ uint64_t hot_key_hash(const uint32_t (&x)[MAXN], int n, uint64_t seed) {
  uint64_t h = hot_mix(seed ^ static_cast<uint64_t>(n));
#pragma unroll
  for (int i = 0; i < MAXN; ++i)
    if (i < n) h = hot_mix(h ^ static_cast<uint64_t>(x[i]));
  return h;
}

__host__ __device__ __forceinline__ uint64_t hot_slot(uint64_t h, uint32_t pilot, uint64_t n_hot) {
  return hot_range(hot_mix(h ^ hot_mix(static_cast<uint64_t>(pilot) + 1)), n_hot);
}

// The tier of order n (2 <= n <= ENGRAM_MAX_ORDER).  Selected field by field
// from values the kernel reads at fixed offsets of its arguments, so that a
// per-lane n costs a few selects instead of a dependent load of the
// argument block.
__device__ __forceinline__ uint64_t sgpr64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<uint64_t>(hi) << 32 | lo;
}

template <typename P>
__device__ __forceinline__ P* sgpr_ptr(P* p) {
  return reinterpret_cast<P*>(sgpr64(reinterpret_cast<uint64_t>(p)));
}

template <typename V>
__device__ __forceinline__ V pick3(int n, V a, V b, V c) {
  return n == 2 ? a : (n == 3 ? b : c);
}

__device__ __forceinline__ HotOrderArgs hot_order(const HotArgs& h, int n) {
  static_assert(ENGRAM_MAX_ORDER == 4, "three hot orders");
  HotOrderArgs r;
  r.pilots = pick3(n, sgpr_ptr(h.o[0].pilots), sgpr_ptr(h.o[1].pilots), sgpr_ptr(h.o[2].pilots));
  r.slots = pick3(n, sgpr_ptr(h.o[0].slots), sgpr_ptr(h.o[1].slots), sgpr_ptr(h.o[2].slots));
  r.rows = pick3(n, sgpr_ptr(h.o[0].rows), sgpr_ptr(h.o[1].rows), sgpr_ptr(h.o[2].rows));
  r.seed = pick3(n, sgpr64(h.o[0].seed), sgpr64(h.o[1].seed), sgpr64(h.o[2].seed));
  r.n_hot = pick3(n, sgpr64(h.o[0].n_hot), sgpr64(h.o[1].n_hot), sgpr64(h.o[2].n_hot));
  r.n_buckets = pick3(n, sgpr64(h.o[0].n_buckets), sgpr64(h.o[1].n_buckets), sgpr64(h.o[2].n_buckets));
  return r;
}

// Loads through global (not flat) instructions: every buffer read here is
// device memory or a device alias of pinned host memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T global_load(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ uint4 global_load16(const void* p) {
  const u32x4 v = global_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Hot row of the n-gram whose ids are x (newest first), or -1.
__device__ __forceinline__ int32_t hot_find(const uint32_t (&x)[ENGRAM_MAX_ORDER], int n,
                                            const HotOrderArgs& o, uint32_t* err = nullptr) {
  if (o.n_hot == 0) return -1;
  const uint64_t h = hot_key_hash(x, n, o.seed);
  const uint32_t pilot = global_load(o.pilots + hot_range(h, o.n_buckets));
  const uint64_t s = hot_slot(h, pilot, o.n_hot);
  const uint4 a = global_load16(o.slots + 2 * s);
  const uint4 b = global_load16(o.slots + 2 * s + 1);
  uint32_t xm[ENGRAM_MAX_ORDER];
#pragma unroll
  for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) xm[i] = i < n ? x[i] : 0u;
  static_assert(ENGRAM_MAX_ORDER == 4, "a slot holds four ids");
  const bool match = a.x == xm[0] && a.y == xm[1] && a.z == xm[2] && a.w == xm[3];
  const int32_t row = match ? static_cast<int32_t>(b.x) : -1;
  if constexpr (kDebugChecks) {
    if (row >= 0 && !in_range(row, static_cast<int64_t>(o.n_hot))) {
      debug_record(err, kErrHotRow);
      return -1;
    }
  }
  return row;
}

}  // namespace engram
