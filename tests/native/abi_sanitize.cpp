// Host-side exercise of the C ABI for the address and undefined-behaviour
// sanitizers: every entry point with arguments that its host checks must
// reject (no GPU is touched), the workspace sizing calls, and the host build
// of the Engram-Nine minimal perfect hash on a real key set (checked against
// the hash the header defines).  Built with -fsanitize=address,undefined on
// the host code of the library's C-ABI layer and of this driver; run by
// tests/test_sanitize.py.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <set>
#include <vector>

#include "engram.h"

static int failures = 0;
#define EXPECT(c)                                                           \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::printf("FAILED line %d: %s (%s)\n", __LINE__, #c, engram_last_error()); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

// The header's hash of an n-gram (newest id first) and its slot.
static uint64_t mix(uint64_t v) {
  v ^= v >> 30; v *= 0xbf58476d1ce4e5b9ull; v ^= v >> 27; v *= 0x94d049bb133111ebull; v ^= v >> 31;
  return v;
}
static uint64_t range(uint64_t a, uint64_t r) { return static_cast<uint64_t>((static_cast<unsigned __int128>(a) * r) >> 64); }

int main() {
  EXPECT(engram_abi_version() == ENGRAM_ABI_VERSION);
  EXPECT(engram_debug_checks() == 0);
  uint32_t bits = 0;
  EXPECT(engram_debug_set_error_word(nullptr) == ENGRAM_EUNSUPPORTED);
  EXPECT(engram_debug_read_errors(&bits) == ENGRAM_EUNSUPPORTED);

  // ---- descriptors with fake device pointers (never dereferenced) ----
  std::vector<uint64_t> mult(2 * 2 * 3, 1);
  uint32_t prime[4] = {1009, 1013, 1019, 1021};
  engram_hash_params hp{static_cast<const int32_t*>(fake(0x1000)), 1000, 3, 2, mult.data(), prime};
  int64_t off[4] = {0, 1009, 2022, 3041}, nrows[4] = {1009, 1013, 1019, 1021};
  engram_tables tab{};
  tab.n_tables = 4; tab.dim = 16; tab.dtype = ENGRAM_F32; tab.rows = fake(0x10000);
  tab.row_offset = off; tab.n_rows = nrows; tab.total_rows = 4062;
  engram_gate_conv_params gc{64, 1, 4, 3, 1e-6f, ENGRAM_F32, static_cast<const float*>(fake(0x20000))};
  engram_layer L{};
  L.hash = hp; L.tables = tab; L.w = fake(0x30000); L.gc = gc;
  void* p = fake(0x40000);
  int32_t* ip = static_cast<int32_t*>(p);

  // hash
  EXPECT(engram_hash_indices(ip, 1, 8, nullptr, nullptr, ip, nullptr) == ENGRAM_EINVAL);
  engram_hash_params hb = hp; hb.max_n = 5;
  EXPECT(engram_hash_indices(ip, 1, 8, nullptr, &hb, ip, nullptr) == ENGRAM_EUNSUPPORTED);
  hb = hp; hb.vocab = 0;
  EXPECT(engram_hash_indices(ip, 1, 8, nullptr, &hb, ip, nullptr) == ENGRAM_EINVAL);
  hb = hp; hb.vocab = int64_t{1} << 40;
  EXPECT(engram_hash_indices(ip, 1, 8, nullptr, &hb, ip, nullptr) == ENGRAM_EUNSUPPORTED);
  EXPECT(engram_hash_indices(ip, -1, 8, nullptr, &hp, ip, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_hash_indices(nullptr, 1, 8, nullptr, &hp, ip, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_hash_indices(ip, 0, 8, nullptr, &hp, ip, nullptr) == ENGRAM_OK);
  // gather
  EXPECT(engram_gather(ip, 8, nullptr, ENGRAM_BF16, p, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_gather(ip, 8, &tab, ENGRAM_I8, p, nullptr) == ENGRAM_EUNSUPPORTED);
  engram_tables tb = tab; tb.dim = 12;
  EXPECT(engram_gather(ip, 8, &tb, ENGRAM_BF16, p, nullptr) == ENGRAM_EUNSUPPORTED);
  tb = tab; tb.total_rows = 4000;
  EXPECT(engram_gather(ip, 8, &tb, ENGRAM_BF16, p, nullptr) == ENGRAM_EINVAL);
  tb = tab; tb.rows = fake(0x10008);
  EXPECT(engram_gather(ip, 8, &tb, ENGRAM_BF16, p, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_gather(ip, 8, &tab, ENGRAM_BF16, fake(0x40008), nullptr) == ENGRAM_EINVAL);
  // projection
  EXPECT(engram_project_kv(p, p, 8, 100, 64, ENGRAM_BF16, p, nullptr) == ENGRAM_EUNSUPPORTED);
  EXPECT(engram_project_kv(p, p, 8, 128, 64, ENGRAM_I8, p, nullptr) == ENGRAM_EUNSUPPORTED);
  EXPECT(engram_project_kv(nullptr, p, 8, 128, 128, ENGRAM_BF16, p, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_project_kv(p, p, 0, 128, 128, ENGRAM_BF16, p, nullptr) == ENGRAM_OK);
  // gate + conv
  const size_t gws = engram_gate_conv_workspace(2, 10, &gc);
  EXPECT(gws > 0);
  EXPECT(engram_gate_conv_forward(p, p, 2, 10, &gc, nullptr, nullptr, nullptr, p, gws - 1, nullptr) == ENGRAM_EINVAL);
  engram_gate_conv_params gb = gc; gb.kernel_w = 9;
  EXPECT(engram_gate_conv_forward(p, p, 2, 10, &gb, nullptr, nullptr, nullptr, p, gws, nullptr) == ENGRAM_EUNSUPPORTED);
  gb = gc; gb.d = 1000;
  EXPECT(engram_gate_conv_forward(p, p, 2, 10, &gb, nullptr, nullptr, nullptr, p, gws, nullptr) == ENGRAM_EUNSUPPORTED);
  EXPECT(engram_gate_conv_forward(p, p, 65536, 1, &gc, nullptr, nullptr, nullptr, p, gws, nullptr) == ENGRAM_EUNSUPPORTED);
  engram_decode_state bad_st{ip, nullptr, ip};   // no conv ring
  EXPECT(engram_gate_conv_forward(p, p, 2, 10, &gc, &bad_st, nullptr, nullptr, p, gws, nullptr) == ENGRAM_EINVAL);
  // layer forward, split forward, no-allocation forward
  const size_t fws = engram_forward_workspace(1, 64, &L);
  EXPECT(fws > 0 && engram_forward_retrieved_workspace(1, 64, &L) < fws);
  EXPECT(engram_forward(ip, p, 1, 64, &L, nullptr, nullptr, nullptr, p, fws - 256, nullptr) == ENGRAM_EINVAL);
  engram_layer Lb = L; int64_t nbad[4] = {1009, 1013, 1019, 1000}; Lb.tables.n_rows = nbad;
  EXPECT(engram_forward(ip, p, 1, 64, &Lb, nullptr, nullptr, nullptr, p, fws, nullptr) == ENGRAM_EINVAL);
  Lb = L; Lb.w = nullptr;
  EXPECT(engram_forward(ip, p, 1, 64, &Lb, nullptr, nullptr, nullptr, p, fws, nullptr) == ENGRAM_EINVAL);
  Lb = L; Lb.w_mx = static_cast<const uint8_t*>(fake(0x60000));
  EXPECT(engram_forward(ip, p, 1, 64, &Lb, nullptr, nullptr, nullptr, p, fws, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_forward(ip, p, 0, 64, &L, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == ENGRAM_OK);
  EXPECT(engram_forward_noalloc(ip, p, 1, 1 << 20, &L, nullptr, nullptr, nullptr, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_forward_noalloc(ip, p, 1, 64, nullptr, nullptr, nullptr, nullptr, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_retrieve(ip, 1, 5, &L, nullptr, nullptr, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_forward_retrieved(ip, p, nullptr, 1, 64, &L, nullptr, nullptr, nullptr, p, fws, nullptr) ==
         ENGRAM_EINVAL);
  EXPECT(engram_forward_retrieved_prefetch(ip, p, p, 1, 64, &L, nullptr, nullptr, nullptr, p, fws, nullptr, nullptr,
                                           ip, 1, 64, p, nullptr) == ENGRAM_EINVAL);   // next_e == e
  // caches
  const size_t cws = engram_cache_build_workspace(4062);
  EXPECT(cws > 0);
  EXPECT(engram_cache_build(ip, 1, 8, &hp, &tab, 5000, ip, p, nullptr, p, cws, nullptr) == ENGRAM_EINVAL);
  EXPECT(engram_cache_build(ip, 1, 8, &hp, &tab, 10, ip, p, nullptr, p, cws - 1, nullptr) == ENGRAM_EINVAL);
  const size_t uws = engram_cache_update_workspace(4062, 100);
  EXPECT(uws > 0 && engram_cache_update_workspace(4062, 5000) == 0);
  EXPECT(engram_cache_update(&tab, 100, ip, p, nullptr, static_cast<uint32_t*>(p), 40, p, uws, nullptr) ==
         ENGRAM_EINVAL);
  // MXFP8 quantiser, profiling, host memory
  EXPECT(engram_quantize_mxfp8(p, ENGRAM_BF16, 4, 33, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p), nullptr) ==
         ENGRAM_EINVAL);
  float ms[4];
  int32_t ns = 0;
  EXPECT(engram_profile_read(ms, nullptr, 4, &ns) == ENGRAM_EINVAL);
  void *h = nullptr, *d = nullptr;
  EXPECT(engram_host_alloc(0, &h, &d) == ENGRAM_EINVAL);
  EXPECT(engram_host_free(nullptr) == ENGRAM_OK);

  // ---- the hot tier's minimal perfect hash, built on the host ----
  const int n = 3;
  const int64_t n_hot = 50000;
  std::vector<int32_t> keys(n_hot * n);
  uint64_t s = 12345;
  std::set<std::vector<int32_t>> seen;
  for (int64_t r = 0; r < n_hot;) {
    std::vector<int32_t> k(n);
    for (int i = 0; i < n; ++i) { s = mix(s + 0x9e3779b97f4a7c15ull); k[i] = static_cast<int32_t>(s % 98560); }
    if (!seen.insert(k).second) continue;
    std::memcpy(&keys[r * n], k.data(), n * sizeof(int32_t));
    ++r;
  }
  const size_t nb = engram_hot_buckets(n_hot);
  EXPECT(nb == static_cast<size_t>((n_hot + 3) / 4) && engram_hot_buckets(0) == 0 && engram_hot_buckets(3) == 1);
  std::vector<uint32_t> pilots(nb);
  std::vector<engram_hot_slot> slots(n_hot);
  uint64_t used = 0;
  EXPECT(engram_hot_build(keys.data(), n_hot, n, 7, pilots.data(), slots.data(), &used) == ENGRAM_OK);
  std::vector<char> taken(n_hot, 0);
  for (int64_t r = 0; r < n_hot; ++r) {
    uint64_t hh = mix(used ^ static_cast<uint64_t>(n));
    for (int i = 0; i < n; ++i) hh = mix(hh ^ static_cast<uint64_t>(keys[r * n + (n - 1 - i)]));
    const uint64_t slot = range(mix(hh ^ mix(static_cast<uint64_t>(pilots[range(hh, nb)]) + 1)), n_hot);
    EXPECT(slots[slot].row == r);
    EXPECT(!taken[slot]);
    taken[slot] = 1;
    for (int i = 0; i < n; ++i) EXPECT(slots[slot].ids[i] == keys[r * n + (n - 1 - i)]);
  }
  std::vector<int32_t> dup(keys.begin(), keys.begin() + 2 * n);
  std::memcpy(&dup[n], &dup[0], n * sizeof(int32_t));
  EXPECT(engram_hot_build(dup.data(), 2, n, 0, pilots.data(), slots.data(), &used) == ENGRAM_EINVAL);
  keys[5] = -3;
  EXPECT(engram_hot_build(keys.data(), n_hot, n, 0, pilots.data(), slots.data(), &used) == ENGRAM_EINVAL);
  EXPECT(engram_hot_build(keys.data(), n_hot, 5, 0, pilots.data(), slots.data(), &used) == ENGRAM_EINVAL);

  std::printf("%s (%d failures)\n", failures == 0 ? "abi sanitize: all passed" : "abi sanitize: FAILURES", failures);
  return failures == 0 ? 0 : 1;
}
