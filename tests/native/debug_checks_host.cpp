// Host build of the debug build's range checks (debug_checks.h): edge values
// of every check, compiled with the host compiler and run by
// tests/test_debug_checks.py.
#include <cstdint>
#include <cstdio>

#include "debug_checks.h"

static int failures = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::printf("FAILED line %d: %s\n", __LINE__, #c);            \
      ++failures;                                                   \
    }                                                               \
  } while (0)

int main() {
  using namespace engram;
  // tokens against the vocabulary
  const int64_t V = 128000;
  EXPECT(range_bit(0, V, kErrToken) == 0u);
  EXPECT(range_bit(V - 1, V, kErrToken) == 0u);
  EXPECT(range_bit(V, V, kErrToken) == kErrToken);
  EXPECT(range_bit(-1, V, kErrToken) == kErrToken);
  EXPECT(range_bit(INT32_MIN, V, kErrToken) == kErrToken);
  EXPECT(clamp_index(-5, V) == 0 && clamp_index(V + 7, V) == V - 1 && clamp_index(12345, V) == 12345);
  EXPECT(clamp_index(INT32_MAX, V) == V - 1 && clamp_index(0, 1) == 0 && clamp_index(3, 1) == 0);
  // row indices against a prime-sized table
  const int64_t p = 646403;
  EXPECT(in_range(p - 1, p) && !in_range(p, p) && !in_range(-1, p));
  EXPECT(range_bit(p, p, kErrRow) == kErrRow && range_bit(p - 1, p, kErrRow) == 0u);
  // cache slots: -1 and [0, cache_n) pass; the rest are misses with the bit
  uint32_t bits = 0;
  EXPECT(checked_slot(-1, 10, &bits) == -1 && bits == 0u);
  EXPECT(checked_slot(0, 10, &bits) == 0 && checked_slot(9, 10, &bits) == 9 && bits == 0u);
  EXPECT(checked_slot(10, 10, &bits) == -1 && bits == kErrSlot);
  bits = 0;
  EXPECT(checked_slot(-2, 10, &bits) == -1 && bits == kErrSlot);
  bits = 0;
  EXPECT(checked_slot(0, 0, &bits) == -1 && bits == kErrSlot);   // an empty cache holds no slot
  bits = kErrToken;
  EXPECT(checked_slot(INT32_MAX, 10, &bits) == -1 && bits == (kErrToken | kErrSlot));
  // the bits are distinct
  EXPECT((kErrToken & kErrRow) == 0u && (kErrRow & kErrSlot) == 0u && (kErrSlot & kErrHotRow) == 0u);
  EXPECT(kDebugChecks == false);   // this file is compiled without ENGRAM_DEBUG_CHECKS
  std::printf("%s\n", failures == 0 ? "debug checks: all passed" : "debug checks: FAILURES");
  return failures == 0 ? 0 : 1;
}
