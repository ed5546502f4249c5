// Engram-Nine hot tier ("DeepSeek Engram series guide", experiment 3
// "Engram-Nine", Figure 1: two-tier retrieval): the host build of the
// minimal perfect hash over one order's hot n-grams, and the standalone
// device lookup (the fused lookup sits in the hashed gather).
//
// Build: every n-gram's 64-bit hash h picks one of ceil(n/4) buckets.
// Buckets are placed largest first; for each, pilots 0, 1, 2, .. are tried
// until all of its n-grams land in distinct free slots.  Big buckets go
// while most slots are free; the singletons at the end need about n/free
// tries each, so the whole build is O(n log n) hash evaluations.
#include <algorithm>
#include <cstring>
#include <vector>

#include "engram_internal.h"
#include "hash_device.h"
#include "hot_device.h"

namespace engram {
namespace {

__global__ void __launch_bounds__(256)
hot_lookup_kernel(const int32_t* __restrict__ tokens, int64_t B, int64_t T, const int32_t* __restrict__ hist,
                  const int32_t* __restrict__ proj, int max_n, int32_t vocab, HotArgs h, int32_t* __restrict__ out,
                  uint32_t* err) {
  const int no = max_n - 1;
  const int64_t total = B * T * no;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int o = static_cast<int>(gid % no);
  const int64_t bt = gid / no;
  const int64_t b = bt / T;
  uint32_t x[ENGRAM_MAX_ORDER];
  window_ids(tokens, proj, hist, max_n, vocab, err, b, bt - b * T, T, x);
  out[gid] = hot_find(x, o + 2, hot_order(h, o + 2), err);
}

}  // namespace

hipError_t launch_hot_lookup(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                             const int32_t* proj, int max_n, int32_t vocab, const HotArgs& h, int32_t* out,
                             uint32_t* err, hipStream_t s) {
  const int64_t total = B * T * (max_n - 1);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  launch_k(hot_lookup_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, s, tokens, B, T, hist, proj,
           max_n, vocab, h, out, err);
  return hipGetLastError();
}

HotBuild hot_build(const int32_t* keys, int64_t n_hot, int n, uint64_t seed, uint32_t* pilots,
                   int32_t* slots) {
  const uint64_t m = hot_buckets(static_cast<uint64_t>(n_hot));
  const uint64_t nh = static_cast<uint64_t>(n_hot);
  std::vector<uint64_t> h(nh);
  for (uint64_t r = 0; r < nh; ++r) {
    uint32_t x[ENGRAM_MAX_ORDER] = {0, 0, 0, 0};
    for (int i = 0; i < n; ++i) x[i] = static_cast<uint32_t>(keys[r * n + (n - 1 - i)]);
    h[r] = hot_key_hash(x, n, seed);
  }
  // Equal hashes: the same n-gram twice (the caller's error) or a 64-bit
  // collision of two n-grams (this seed cannot separate them).
  {
    std::vector<uint32_t> byh(nh);
    for (uint64_t r = 0; r < nh; ++r) byh[r] = static_cast<uint32_t>(r);
    std::sort(byh.begin(), byh.end(), [&](uint32_t a, uint32_t b) { return h[a] < h[b] || (h[a] == h[b] && a < b); });
    for (uint64_t q = 1; q < nh; ++q) {
      const uint32_t a = byh[q - 1], b = byh[q];
      if (h[a] != h[b]) continue;
      if (std::memcmp(keys + static_cast<uint64_t>(a) * n, keys + static_cast<uint64_t>(b) * n,
                      sizeof(int32_t) * n) == 0)
        return HotBuild{HotBuild::kDuplicate, a, b};
      return HotBuild{HotBuild::kRetry, a, b};
    }
  }
  // Members of each bucket (counting sort by bucket).
  std::vector<uint32_t> start(m + 1, 0), member(nh);
  std::vector<uint64_t> bucket(nh);
  for (uint64_t r = 0; r < nh; ++r) {
    bucket[r] = hot_range(h[r], m);
    ++start[bucket[r] + 1];
  }
  for (uint64_t b = 0; b < m; ++b) start[b + 1] += start[b];
  {
    std::vector<uint32_t> fill(start.begin(), start.end() - 1);
    for (uint64_t r = 0; r < nh; ++r) member[fill[bucket[r]]++] = static_cast<uint32_t>(r);
  }
  // Buckets by size, largest first, then by index.
  std::vector<uint32_t> order(m);
  for (uint64_t b = 0; b < m; ++b) order[b] = static_cast<uint32_t>(b);
  std::stable_sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) {
    return start[a + 1] - start[a] > start[b + 1] - start[b];
  });
  // Search bound per bucket: the last singleton, with one free slot left,
  // needs n_hot tries on average, and exceeds 16 n_hot with odds e^-16.
  const uint64_t max_pilot = std::min<uint64_t>(0xffffffffull, std::max<uint64_t>(1ull << 24, 16 * nh));
  std::vector<uint8_t> taken(nh, 0);
  std::vector<uint64_t> pos;
  for (uint64_t b = 0; b < m; ++b) pilots[b] = 0;
  for (uint32_t b : order) {
    const uint32_t lo = start[b], size = start[b + 1] - lo;
    if (size == 0) break;  // sorted by size: the rest are empty
    pos.resize(size);
    bool placed = false;
    for (uint64_t p = 0; p < max_pilot; ++p) {
      bool ok = true;
      for (uint32_t q = 0; q < size && ok; ++q) {
        pos[q] = hot_slot(h[member[lo + q]], static_cast<uint32_t>(p), nh);
        if (taken[pos[q]]) ok = false;
        for (uint32_t u = 0; u < q && ok; ++u)
          if (pos[u] == pos[q]) ok = false;
      }
      if (!ok) continue;
      for (uint32_t q = 0; q < size; ++q) taken[pos[q]] = 1;
      pilots[b] = static_cast<uint32_t>(p);
      for (uint32_t q = 0; q < size; ++q) {
        const uint32_t r = member[lo + q];
        int32_t* sl = slots + 8 * pos[q];
        for (int i = 0; i < 8; ++i) sl[i] = 0;
        for (int i = 0; i < n; ++i) sl[i] = keys[static_cast<uint64_t>(r) * n + (n - 1 - i)];
        sl[4] = static_cast<int32_t>(r);
      }
      placed = true;
      break;
    }
    if (!placed) return HotBuild{HotBuild::kRetry, b, 0};
  }
  return HotBuild{HotBuild::kOk, 0, 0};
}

}  // namespace engram
