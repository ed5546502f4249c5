// Checks of the device-resident preconditions that the C ABI leaves to the
// caller (raw token ids inside the vocabulary, row indices inside their
// table, cache slots inside the cache, hot-tier rows inside the hot set).
//
// In the debug build (ENGRAM_DEBUG_CHECKS defined: libengram_debug.so) the
// kernels test each value before the load that uses it; a value outside its
// range sets a bit in the caller's error word (engram_debug_set_error_word,
// one global atomic OR) and is replaced by one inside the range (an index
// clamped into it; a bad cache slot or hot row read as a miss), so every
// access stays inside its buffer.  In the release build the checks compile
// away; raw token ids are clamped into the vocabulary in both builds.
//
// The range logic is plain host/device code so that it can be tested on the
// host.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define ENGRAM_HD __host__ __device__
#else
#define ENGRAM_HD
#endif

namespace engram {

#ifdef ENGRAM_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif

// Bits of the error word (the same values as ENGRAM_ERR_* in engram.h).
constexpr uint32_t kErrToken = 1u;    // raw token id outside [0, vocab)
constexpr uint32_t kErrRow = 2u;      // row index outside [0, rows of its table)
constexpr uint32_t kErrSlot = 4u;     // cache slot outside [-1, cache_n)
constexpr uint32_t kErrHotRow = 8u;   // hot-tier row outside [0, n_hot)

// v lies in [0, n).
ENGRAM_HD inline bool in_range(int64_t v, int64_t n) { return v >= 0 && v < n; }

// v clamped into [0, n) (n >= 1).
ENGRAM_HD inline int64_t clamp_index(int64_t v, int64_t n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// `bit` when v lies outside [0, n), else 0.
ENGRAM_HD inline uint32_t range_bit(int64_t v, int64_t n, uint32_t bit) { return in_range(v, n) ? 0u : bit; }

// A cache slot read from the slot map: -1 (not cached) and [0, cache_n) are
// valid; anything else is reported with kErrSlot and read as -1 (a miss).
ENGRAM_HD inline int32_t checked_slot(int32_t slot, int64_t cache_n, uint32_t* bits) {
  if (slot == -1 || in_range(slot, cache_n)) return slot;
  *bits |= kErrSlot;
  return -1;
}

#if defined(__HIPCC__)
// Adds bits to the error word (debug build only; one vector atomic).
__device__ __forceinline__ void debug_record(uint32_t* err, uint32_t bits) {
  if constexpr (kDebugChecks) {
    if (bits != 0u && err != nullptr) atomicOr(err, bits);
  }
}
#endif

}  // namespace engram
