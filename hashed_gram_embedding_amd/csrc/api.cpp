// C ABI of libengram.so (declared in include/engram.h): argument checks on
// host-visible values, workspace carving and kernel launch order.  Nothing
// here touches device data or synchronises, except engram_host_alloc/free.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "engram.h"
#include "engram_internal.h"
#include "hot_device.h"

#define ENGRAM_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

// Debug build: the caller's device error word (engram_debug_set_error_word),
// passed to every kernel launched after it is set.
std::atomic<uint32_t*> g_err_word{nullptr};

engram_status fail(engram_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

engram_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ENGRAM_OK;
  return fail(ENGRAM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t dtype_size(int dt) {
  switch (dt) {
    case ENGRAM_F32: return 4;
    case ENGRAM_BF16: return 2;
    case ENGRAM_I8: return 1;
    default: return 0;
  }
}

engram_status check_hash(const engram_hash_params* hp, engram::HashArgs* out) {
  if (hp == nullptr) return fail(ENGRAM_EINVAL, "hash params are NULL");
  if (hp->proj == nullptr || hp->mult == nullptr || hp->prime == nullptr)
    return fail(ENGRAM_EINVAL, "hash params: proj, mult and prime must be non-NULL");
  if (hp->vocab <= 0) return fail(ENGRAM_EINVAL, "hash params: vocab must be positive");
  if (hp->vocab > INT32_MAX) return fail(ENGRAM_EUNSUPPORTED, "hash params: vocab above 2^31-1");
  if (hp->max_n < 2 || hp->max_n > ENGRAM_MAX_ORDER)
    return fail(ENGRAM_EUNSUPPORTED, "hash params: max_n=%d outside [2, %d]", hp->max_n, ENGRAM_MAX_ORDER);
  const int nt = (hp->max_n - 1) * hp->heads;
  if (hp->heads < 1 || nt > ENGRAM_MAX_TABLES)
    return fail(ENGRAM_EUNSUPPORTED, "hash params: (max_n-1)*heads=%d outside [1, %d]", nt, ENGRAM_MAX_TABLES);
  if (out != nullptr) *out = engram::HashArgs{};
  for (int n = 2; n <= hp->max_n; ++n) {
    for (int k = 0; k < hp->heads; ++k) {
      const int j = (n - 2) * hp->heads + k;
      const uint32_t p = hp->prime[j];
      if (p < 2 || p > 0x7fffffffu)
        return fail(ENGRAM_EINVAL, "hash params: prime[%d]=%u outside [2, 2^31)", j, p);
      if (out != nullptr) {
        out->prime[j] = p;
        out->inv[j] = ~static_cast<uint64_t>(0) / p;
        out->order[j] = n;
        for (int i = 0; i < n; ++i)
          out->mult[j][i] = hp->mult[(static_cast<int64_t>(n - 2) * hp->heads + k) * hp->max_n + i];
      }
    }
  }
  if (out != nullptr) {
    out->n_tables = nt;
    out->max_n = hp->max_n;
    out->vocab = static_cast<int32_t>(hp->vocab);
    out->err = g_err_word.load();
  }
  return ENGRAM_OK;
}

engram_status check_tables(const engram_tables* tab, engram::TableArgs* out) {
  if (tab == nullptr) return fail(ENGRAM_EINVAL, "tables are NULL");
  if (tab->n_tables < 1 || tab->n_tables > ENGRAM_MAX_TABLES)
    return fail(ENGRAM_EUNSUPPORTED, "tables: n_tables=%d outside [1, %d]", tab->n_tables, ENGRAM_MAX_TABLES);
  if (tab->dim < 8 || tab->dim % 8 != 0)
    return fail(ENGRAM_EUNSUPPORTED, "tables: dim=%d must be a positive multiple of 8", tab->dim);
  if (tab->dtype != ENGRAM_F32 && tab->dtype != ENGRAM_BF16 && tab->dtype != ENGRAM_I8)
    return fail(ENGRAM_EUNSUPPORTED, "tables: unknown dtype %d", static_cast<int>(tab->dtype));
  if (tab->rows == nullptr || tab->row_offset == nullptr || tab->n_rows == nullptr)
    return fail(ENGRAM_EINVAL, "tables: rows, row_offset and n_rows must be non-NULL");
  const size_t row_align = tab->dtype == ENGRAM_I8 ? 8 : 16;
  if (!aligned(tab->rows, row_align))
    return fail(ENGRAM_EINVAL, "tables: rows must be %zu-byte aligned", row_align);
  if (tab->total_rows <= 0) return fail(ENGRAM_EINVAL, "tables: total_rows must be positive");
  for (int j = 0; j < tab->n_tables; ++j) {
    const int64_t off = tab->row_offset[j], n = tab->n_rows[j];
    if (off < 0 || n < 1 || n > 0x7fffffffLL || off + n > tab->total_rows)
      return fail(ENGRAM_EINVAL, "tables: table %d (offset %lld, rows %lld) outside [0, total_rows=%lld)",
                  j, static_cast<long long>(off), static_cast<long long>(n),
                  static_cast<long long>(tab->total_rows));
  }
  if (tab->dtype == ENGRAM_I8 && tab->row_scale == nullptr)
    return fail(ENGRAM_EINVAL, "tables: int8 rows need row_scale");
  if (!aligned(tab->access_counts, 4)) return fail(ENGRAM_EINVAL, "tables: access_counts must be 4-byte aligned");
  if (tab->cache_slot != nullptr) {
    if (tab->cache_rows == nullptr || tab->cache_n < 0)
      return fail(ENGRAM_EINVAL, "tables: a cache needs cache_rows and cache_n >= 0");
    if (!aligned(tab->cache_rows, row_align))
      return fail(ENGRAM_EINVAL, "tables: cache_rows must be %zu-byte aligned", row_align);
    if (tab->dtype == ENGRAM_I8 && tab->cache_scale == nullptr)
      return fail(ENGRAM_EINVAL, "tables: an int8 cache needs cache_scale");
  }
  if (out != nullptr) {
    *out = engram::TableArgs{};
    for (int j = 0; j < tab->n_tables; ++j) {
      out->row_offset[j] = tab->row_offset[j];
      out->n_rows[j] = static_cast<int32_t>(tab->n_rows[j]);
    }
    out->cache_n = tab->cache_slot != nullptr ? tab->cache_n : 0;
    out->err = g_err_word.load();
    out->rows = tab->rows;
    out->scale = tab->row_scale;
    out->cache_slot = tab->cache_slot;
    out->cache_rows = tab->cache_rows;
    out->cache_scale = tab->cache_scale;
    out->counts = tab->access_counts;
    out->n_tables = tab->n_tables;
    out->dim = tab->dim;
    out->dtype = tab->dtype;
  }
  return ENGRAM_OK;
}

engram_status check_gc(const engram_gate_conv_params* p, engram::GateConvArgs* out) {
  if (p == nullptr) return fail(ENGRAM_EINVAL, "gate/conv params are NULL");
  if (p->d < 64 || p->d % 64 != 0 || p->d > ENGRAM_MAX_D)
    return fail(ENGRAM_EUNSUPPORTED, "gate/conv: d=%d must be a multiple of 64 in [64, %d]", p->d, ENGRAM_MAX_D);
  if (p->branches < 1) return fail(ENGRAM_EINVAL, "gate/conv: branches must be >= 1");
  if (p->branches > ENGRAM_MAX_BRANCHES)
    return fail(ENGRAM_EUNSUPPORTED, "gate/conv: branches=%d above %d", p->branches, ENGRAM_MAX_BRANCHES);
  if (p->kernel_w < 2 || p->kernel_w > ENGRAM_MAX_KERNEL_W)
    return fail(ENGRAM_EUNSUPPORTED, "gate/conv: kernel_w=%d outside [2, %d]", p->kernel_w, ENGRAM_MAX_KERNEL_W);
  if (p->dilation < 1 || (p->kernel_w - 1) * p->dilation > ENGRAM_MAX_CONV_SPAN)
    return fail(ENGRAM_EUNSUPPORTED, "gate/conv: (kernel_w-1)*dilation must lie in [1, %d]", ENGRAM_MAX_CONV_SPAN);
  if (!(p->eps >= 0.0f)) return fail(ENGRAM_EINVAL, "gate/conv: eps must be >= 0");
  if (p->hdtype != ENGRAM_F32 && p->hdtype != ENGRAM_BF16)
    return fail(ENGRAM_EUNSUPPORTED, "gate/conv: hdtype must be F32 or BF16");
  if (p->conv_w == nullptr) return fail(ENGRAM_EINVAL, "gate/conv: conv_w is NULL");
  if (out != nullptr) {
    out->d = p->d;
    out->branches = p->branches;
    out->kernel_w = p->kernel_w;
    out->dilation = p->dilation;
    out->eps = p->eps;
    out->hdtype = p->hdtype;
    out->kvdtype = p->hdtype;
    out->conv_w = p->conv_w;
  }
  return ENGRAM_OK;
}

engram_status check_state(const engram_decode_state* st, bool need_ids) {
  if (st == nullptr) return ENGRAM_OK;
  if (st->conv == nullptr || st->pos == nullptr || (need_ids && st->ids == nullptr))
    return fail(ENGRAM_EINVAL, "decode state: ids, conv and pos must be non-NULL");
  if (!aligned(st->conv, 16)) return fail(ENGRAM_EINVAL, "decode state: conv must be 16-byte aligned");
  return ENGRAM_OK;
}

// ---- stage timing (per calling thread) ----
// Mode 1 keeps the stages of the last call (kCallStages); mode 2 keeps every
// stage since the last read, up to kMaxStages (later ones are dropped and
// counted).
constexpr int kCallStages = 12;
constexpr int kMaxStages = 2048;

struct Profiler {
  int mode = 0;                     // 0 off, 1 last call, 2 accumulate until read
  int created = 0;                  // event pairs created
  int n = 0;                        // stages recorded
  int dropped = 0;                  // stages not recorded since the last read (no free event pair)
  const char* pending = nullptr;    // open stage: its kernel has not been launched yet
  hipEvent_t start[kMaxStages];
  hipEvent_t stop[kMaxStages];
  const char* names[kMaxStages];
};

thread_local Profiler g_prof;

// Opens a stage; the next kernel launched on this thread records its events.
void prof_mark(hipStream_t, const char* name) {
  Profiler& p = g_prof;
  if (p.mode != 0) p.pending = name;
}

void prof_begin() {
  Profiler& p = g_prof;
  if (p.mode == 1) {
    p.n = 0;
    p.dropped = 0;
  }
  p.pending = nullptr;
}

}  // namespace

namespace engram {
bool prof_take(hipEvent_t* start, hipEvent_t* stop) {
  Profiler& p = g_prof;
  if (p.mode == 0 || p.pending == nullptr) return false;
  if (p.n >= p.created) {
    ++p.dropped;
    p.pending = nullptr;
    return false;
  }
  *start = p.start[p.n];
  *stop = p.stop[p.n];
  p.names[p.n] = p.pending;
  p.pending = nullptr;
  ++p.n;
  return true;
}
}  // namespace engram

namespace {

// ---- workspace layouts ----
// A bump allocator over the caller's workspace: every region starts on a
// 256-byte boundary.  With base == nullptr it only measures.
struct Carve {
  char* base;
  size_t used = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base == nullptr ? nullptr : reinterpret_cast<T*>(base + used);
    used += align_up(count * sizeof(T));
    return p;
  }
};

struct GcWorkspace {
  float4* stats;   // [n_tok][1+M]
  float* gamma;    // [n_tok][M]
};

GcWorkspace carve_gc(Carve& c, int64_t n_tok, int M) {
  GcWorkspace w;
  w.stats = c.take<float4>(static_cast<size_t>(n_tok) * (1 + M));
  w.gamma = c.take<float>(static_cast<size_t>(n_tok) * M);
  return w;
}

// Fused bf16 path: gathered rows, float32 v, per-tile gate statistics.
bool use_fused(const engram_layer* L) {
  return L->gc.hdtype == ENGRAM_BF16 && L->gc.d % 128 == 0 && L->gc.d <= 4096 &&
         (static_cast<int64_t>(L->tables.n_tables) * L->tables.dim) % 64 == 0;
}

// Workspace of Steps 5-8 (engram_forward_retrieved); engram_forward puts the
// gathered rows e in front of it.
struct ComputeWorkspace {
  float* kv;        // unfused: [n_tok][(1+M)d]; fused: v only, [n_tok][d]
  float4* stats;    // fused: [n_tok][(1+M)d/128] (or fewer tiles); unfused: [n_tok][1+M]
  float* gamma;     // [n_tok][M]
};

ComputeWorkspace carve_compute(Carve& c, int64_t n_tok, const engram_layer* L) {
  const int M = L->gc.branches, d = L->gc.d;
  ComputeWorkspace f;
  if (use_fused(L)) {
    f.kv = c.take<float>(static_cast<size_t>(n_tok) * d);
    f.stats = c.take<float4>(static_cast<size_t>(n_tok) * (1 + M) * d / engram::kProjGateTileF);
  } else {
    f.kv = c.take<float>(static_cast<size_t>(n_tok) * (1 + M) * d);
    f.stats = c.take<float4>(static_cast<size_t>(n_tok) * (1 + M));
  }
  f.gamma = c.take<float>(static_cast<size_t>(n_tok) * M);
  return f;
}

size_t rows_bytes(int64_t n_tok, const engram_layer* L) {
  return static_cast<size_t>(n_tok) * L->tables.n_tables * L->tables.dim * dtype_size(L->gc.hdtype);
}

size_t gc_ws_bytes(int64_t n_tok, int M) {
  Carve c{nullptr};
  carve_gc(c, n_tok, M);
  return c.used;
}

size_t compute_ws_bytes(int64_t n_tok, const engram_layer* L) {
  Carve c{nullptr};
  carve_compute(c, n_tok, L);
  return c.used;
}

size_t forward_ws_bytes(int64_t n_tok, const engram_layer* L) {
  Carve c{nullptr};
  c.take<char>(rows_bytes(n_tok, L));
  carve_compute(c, n_tok, L);
  return c.used;
}

// Steps 6-8 once the gate statistics are in `stats`: conv (+ residual), then
// the decode-state commit.
// next: a hashed gather of another batch to run with this conv (in the same
// launch where a fused form exists, else right after it), or null.
engram_status run_conv_commit(void* H, const void* v, int64_t v_stride, int vdtype, const float4* stats, int qv,
                              int qk, bool mixed, int64_t B, int64_t T, const engram::GateConvArgs& g, engram_decode_state* st,
                              const int32_t* tokens, const int32_t* proj, int32_t max_n, int32_t vocab,
                              float* alpha_out, float* gamma, float* y_out, hipStream_t s,
                              const engram::GatherJob* next = nullptr,
                              bool state_folded = false) {
  engram::ConvArgs ca{};
  ca.H = H;
  ca.v = v;
  ca.v_stride = v_stride;
  ca.stats = stats;
  ca.qv = qv;
  ca.qk = qk;
  ca.mixed = mixed;
  ca.kq0 = mixed ? 0 : qv;
  ca.nq = qv + g.branches * qk;
  ca.B = B;
  ca.T = T;
  ca.g = g;
  ca.has_state = st != nullptr;
  if (st != nullptr) ca.st = engram::StateArgs{st->ids, st->conv, st->pos};
  // decode with the state advance already done by the projection launch: the
  // conv reads pos - T and writes the new conv input itself
  ca.pos_advanced = state_folded;
  ca.commit_u = state_folded;
  ca.alpha_out = alpha_out;
  ca.gamma_out = gamma;
  ca.y_out = y_out;
  engram_status r;
  bool fused = false;
  if (next != nullptr) {
    prof_mark(s, "conv_gather_kernel");
    const hipError_t e = engram::launch_conv_gather(ca, vdtype, *next, s);
    if (e != hipErrorNotSupported) {
      if ((r = hip_status(e, "conv+gather launch")) != ENGRAM_OK) return r;
      fused = true;
    }
  }
  if (!fused) {
    prof_mark(s, "conv_kernel");
    if ((r = hip_status(engram::launch_conv(ca, vdtype, s), "conv launch")) != ENGRAM_OK) return r;
    if (next != nullptr) {
      const engram::HashSrc& hs = next->hs;
      prof_mark(s, next->hot ? "gather_kernel<hashed,hot>" : "gather_kernel<hashed>");
      r = hip_status(engram::launch_hash_gather(hs.tokens, next->n_tok / hs.T, hs.T, hs.hist, hs.proj, hs.a, next->ta,
                                                next->hot ? &hs.hot : nullptr, next->out_dtype, next->e, s),
                     "hash+gather launch");
      if (r != ENGRAM_OK) return r;
    }
  }
  if (st != nullptr && !state_folded) {
    engram::StateArgs sa{tokens != nullptr ? st->ids : nullptr, st->conv, st->pos};
    prof_mark(s, "state_commit_kernel");
    r = hip_status(engram::launch_state_commit(v, v_stride, vdtype, B, T, g, gamma, sa, tokens, proj, max_n, vocab,
                                                    g_err_word.load(), s),
                   "state commit launch");
  }
  prof_mark(s, nullptr);
  return r;
}

// The Engram-Nine hot tier.  tab = NULL when only the lookup runs (then the
// rows are not read and may be NULL).  *any is set when some order has a
// hot set.
engram_status check_hot(const engram_hot_tier* hot, const engram_hash_params* hp, const engram_tables* tab,
                        engram::HotArgs* out, bool* any) {
  *any = false;
  if (out != nullptr) *out = engram::HotArgs{};
  if (hot == nullptr) return ENGRAM_OK;
  for (int o = 0; o < ENGRAM_MAX_ORDER - 1; ++o) {
    const int n = o + 2;
    const int64_t nh = hot->n_hot[o];
    if (nh < 0 || nh > INT32_MAX) return fail(ENGRAM_EINVAL, "hot tier: n_hot of order %d outside [0, 2^31)", n);
    if (nh == 0) continue;
    if (n > hp->max_n) return fail(ENGRAM_EINVAL, "hot tier: order %d has a hot set but max_n is %d", n, hp->max_n);
    if (hot->pilots[o] == nullptr || hot->slots[o] == nullptr || (tab != nullptr && hot->rows[o] == nullptr))
      return fail(ENGRAM_EINVAL, "hot tier: order %d needs pilots, slots and rows", n);
    if (!aligned(hot->slots[o], 32) || !aligned(hot->pilots[o], 4) || !aligned(hot->rows[o], 16))
      return fail(ENGRAM_EINVAL, "hot tier: order %d slots must be 32-byte, pilots 4-byte, rows 16-byte aligned", n);
    *any = true;
    if (out != nullptr) {
      engram::HotOrderArgs& a = out->o[o];
      a.pilots = hot->pilots[o];
      a.slots = reinterpret_cast<const uint4*>(hot->slots[o]);
      a.rows = hot->rows[o];
      a.seed = hot->seed[o];
      a.n_hot = static_cast<uint64_t>(nh);
      a.n_buckets = engram::hot_buckets(static_cast<uint64_t>(nh));
    }
  }
  if (*any && tab != nullptr && tab->dtype != ENGRAM_F32 && tab->dtype != ENGRAM_BF16)
    return fail(ENGRAM_EUNSUPPORTED, "hot tier: needs F32 or BF16 tables");
  if (out != nullptr) {
    out->heads = hp->heads;
    out->width = tab != nullptr ? hp->heads * tab->dim : 0;
  }
  return ENGRAM_OK;
}

engram_status check_layer(const engram_layer* L, engram::HashArgs* ha, engram::TableArgs* ta,
                          engram::GateConvArgs* ga) {
  if (L == nullptr) return fail(ENGRAM_EINVAL, "layer is NULL");
  engram_status r = check_hash(&L->hash, ha);
  if (r != ENGRAM_OK) return r;
  r = check_tables(&L->tables, ta);
  if (r != ENGRAM_OK) return r;
  r = check_gc(&L->gc, ga);
  if (r != ENGRAM_OK) return r;
  const int nt = (L->hash.max_n - 1) * L->hash.heads;
  if (L->tables.n_tables != nt)
    return fail(ENGRAM_EINVAL, "layer: tables.n_tables=%d but the hash has (N-1)*K=%d tables",
                L->tables.n_tables, nt);
  for (int j = 0; j < nt; ++j)
    if (L->tables.n_rows[j] != static_cast<int64_t>(L->hash.prime[j]))
      return fail(ENGRAM_EINVAL, "layer: table %d has %lld rows but prime %u", j,
                  static_cast<long long>(L->tables.n_rows[j]), L->hash.prime[j]);
  if (L->w == nullptr) return fail(ENGRAM_EINVAL, "layer: w is NULL");
  const int64_t d_mem = static_cast<int64_t>(nt) * L->tables.dim;
  if (L->gc.hdtype == ENGRAM_BF16 && d_mem % 64 != 0)
    return fail(ENGRAM_EUNSUPPORTED, "layer: bf16 projections need n_tables*dim (%lld) to be a multiple of 64",
                static_cast<long long>(d_mem));
  if (!aligned(L->w, 16)) return fail(ENGRAM_EINVAL, "layer: w must be 16-byte aligned");
  if ((L->w_mx == nullptr) != (L->w_mx_scale == nullptr))
    return fail(ENGRAM_EINVAL, "layer: w_mx and w_mx_scale must both be set or both be NULL");
  if (L->w_mx != nullptr) {
    // (the MXFP8 rows are read only by the fused projection, which takes d <= 4096)
    if (L->gc.hdtype != ENGRAM_BF16 || L->gc.d % 128 != 0 || L->gc.d > 4096 || L->tables.dim % 32 != 0 ||
        d_mem % 128 != 0)
      return fail(ENGRAM_EUNSUPPORTED,
                  "layer: MXFP8 needs bf16 H, d a multiple of 128 up to 4096, dim a multiple of 32 and d_mem of 128");
    if (!aligned(L->w_mx, 16) || !aligned(L->w_mx_scale, 4))
      return fail(ENGRAM_EINVAL, "layer: w_mx must be 16-byte and w_mx_scale 4-byte aligned");
  }
  if (L->w_mx_packed != nullptr) {
    if (L->w_mx == nullptr) return fail(ENGRAM_EINVAL, "layer: w_mx_packed needs w_mx");
    if (!aligned(L->w_mx_packed, 16)) return fail(ENGRAM_EINVAL, "layer: w_mx_packed must be 16-byte aligned");
  }
  if (L->w_packed != nullptr) {
    if (L->gc.hdtype != ENGRAM_BF16) return fail(ENGRAM_EINVAL, "layer: w_packed needs a bf16 layer");
    if (!aligned(L->w_packed, 16)) return fail(ENGRAM_EINVAL, "layer: w_packed must be 16-byte aligned");
  }
  bool any_hot;
  return check_hot(L->hot, &L->hash, &L->tables, nullptr, &any_hot);
}

}  // namespace

ENGRAM_API int32_t engram_abi_version(void) { return ENGRAM_ABI_VERSION; }

ENGRAM_API const char* engram_last_error(void) { return g_last_error.c_str(); }

ENGRAM_API engram_status engram_hash_indices(const int32_t* tokens, int64_t B, int64_t T,
                                             const int32_t* hist, const engram_hash_params* hp,
                                             int32_t* z, hipStream_t stream) {
  engram::HashArgs ha;
  engram_status r = check_hash(hp, &ha);
  if (r != ENGRAM_OK) return r;
  if (B < 0 || T < 0) return fail(ENGRAM_EINVAL, "hash: B and T must be >= 0");
  if (B * T == 0) return ENGRAM_OK;
  if (tokens == nullptr || z == nullptr) return fail(ENGRAM_EINVAL, "hash: tokens and z must be non-NULL");
  return hip_status(engram::launch_hash(tokens, B, T, hist, hp->proj, ha, z, stream), "hash launch");
}

ENGRAM_API engram_status engram_gather(const int32_t* z, int64_t n_tok, const engram_tables* tab,
                                       engram_dtype out_dtype, void* e, hipStream_t stream) {
  engram::TableArgs ta;
  engram_status r = check_tables(tab, &ta);
  if (r != ENGRAM_OK) return r;
  if (out_dtype != ENGRAM_F32 && out_dtype != ENGRAM_BF16)
    return fail(ENGRAM_EUNSUPPORTED, "gather: out_dtype must be F32 or BF16");
  if (n_tok < 0) return fail(ENGRAM_EINVAL, "gather: n_tok must be >= 0");
  if (n_tok == 0) return ENGRAM_OK;
  if (z == nullptr || e == nullptr) return fail(ENGRAM_EINVAL, "gather: z and e must be non-NULL");
  if (!aligned(e, 16)) return fail(ENGRAM_EINVAL, "gather: e must be 16-byte aligned");
  return hip_status(engram::launch_gather(z, n_tok, ta, out_dtype, e, stream), "gather launch");
}

ENGRAM_API engram_status engram_project_kv(const void* e, const void* w, int64_t n_tok, int64_t d_mem,
                                           int64_t n_out, engram_dtype dtype, void* kv,
                                           hipStream_t stream) {
  if (dtype != ENGRAM_F32 && dtype != ENGRAM_BF16)
    return fail(ENGRAM_EUNSUPPORTED, "project_kv: dtype must be F32 or BF16");
  if (n_tok < 0 || d_mem < 1 || n_out < 1)
    return fail(ENGRAM_EINVAL, "project_kv: need n_tok >= 0, d_mem >= 1, n_out >= 1");
  if (d_mem > 0x7fffffff || n_out > 0x7fffffff) return fail(ENGRAM_EUNSUPPORTED, "project_kv: dims too large");
  if (dtype == ENGRAM_BF16 && (d_mem % 64 != 0 || n_out % 64 != 0))
    return fail(ENGRAM_EUNSUPPORTED, "project_kv: bf16 needs d_mem and n_out to be multiples of 64");
  if (n_tok == 0) return ENGRAM_OK;
  if (e == nullptr || w == nullptr || kv == nullptr)
    return fail(ENGRAM_EINVAL, "project_kv: e, w and kv must be non-NULL");
  if (!aligned(e, 16) || !aligned(w, 16)) return fail(ENGRAM_EINVAL, "project_kv: e and w must be 16-byte aligned");
  return hip_status(engram::launch_project_kv(e, w, n_tok, d_mem, n_out, dtype, dtype, kv, stream),
                    "project_kv launch");
}

ENGRAM_API size_t engram_gate_conv_workspace(int64_t B, int64_t T, const engram_gate_conv_params* p) {
  if (p == nullptr || B < 0 || T < 0 || p->branches < 1) return 0;
  return gc_ws_bytes(B * T, p->branches);
}

ENGRAM_API engram_status engram_gate_conv_forward(void* H, const void* kv, int64_t B, int64_t T,
                                                  const engram_gate_conv_params* p,
                                                  engram_decode_state* st, float* alpha_out,
                                                  float* y_out, void* ws, size_t ws_bytes,
                                                  hipStream_t stream) {
  engram::GateConvArgs g;
  engram_status r = check_gc(p, &g);
  if (r != ENGRAM_OK) return r;
  if ((r = check_state(st, false)) != ENGRAM_OK) return r;
  if (B < 0 || T < 0) return fail(ENGRAM_EINVAL, "gate_conv: B and T must be >= 0");
  if (T > INT32_MAX) return fail(ENGRAM_EUNSUPPORTED, "gate_conv: T above 2^31-1 tokens per sequence");
  if (B > 65535) return fail(ENGRAM_EUNSUPPORTED, "gate_conv: B above 65535 sequences per call");
  if (B * T == 0) return ENGRAM_OK;
  if (H == nullptr || kv == nullptr) return fail(ENGRAM_EINVAL, "gate_conv: H and kv must be non-NULL");
  if (!aligned(H, 16) || !aligned(kv, 16)) return fail(ENGRAM_EINVAL, "gate_conv: H and kv must be 16-byte aligned");
  if (y_out != nullptr && !aligned(y_out, 16)) return fail(ENGRAM_EINVAL, "gate_conv: y_out must be 16-byte aligned");
  const size_t need = gc_ws_bytes(B * T, p->branches);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "gate_conv: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  Carve c{static_cast<char*>(ws)};
  GcWorkspace w = carve_gc(c, B * T, p->branches);
  prof_begin();
  prof_mark(stream, "gate_stats_kernel");
  r = hip_status(engram::launch_gate_stats(H, kv, B * T, g, w.stats, stream), "gate statistics launch");
  if (r != ENGRAM_OK) return r;
  const int64_t stride = static_cast<int64_t>(1 + p->branches) * p->d;
  return run_conv_commit(H, kv, stride, g.kvdtype, w.stats, 1, 1, false, B, T, g, st, nullptr, nullptr, 0, 1, alpha_out,
                         w.gamma, y_out, stream);
}

namespace {

// Argument checks shared by the layer entry points (everything host-visible).
engram_status check_call(const char* who, const engram_layer* L, const engram_decode_state* st, bool state_ids,
                         int64_t B, int64_t T, engram::HashArgs* ha, engram::TableArgs* ta,
                         engram::GateConvArgs* g) {
  engram_status r = check_layer(L, ha, ta, g);
  if (r != ENGRAM_OK) return r;
  if ((r = check_state(st, state_ids)) != ENGRAM_OK) return r;
  if (B < 0 || T < 0) return fail(ENGRAM_EINVAL, "%s: B and T must be >= 0", who);
  if (T > INT32_MAX) return fail(ENGRAM_EUNSUPPORTED, "%s: T above 2^31-1 tokens per sequence", who);
  if (B > 65535) return fail(ENGRAM_EUNSUPPORTED, "%s: B above 65535 sequences per call", who);
  return ENGRAM_OK;
}

// Steps 1-4: indices hashed inside the gather.
engram_status run_retrieve(const int32_t* tokens, int64_t B, int64_t T, const engram_layer* L,
                           const engram::HashArgs& ha, const engram::TableArgs& ta, int hdtype,
                           const engram_decode_state* st, void* e, hipStream_t stream, int out_order = -1) {
  // the hashed gather indexes tokens and (token, table) groups in 32 bits
  if (B * T >= (int64_t{1} << 31))
    return fail(ENGRAM_EUNSUPPORTED, "retrieve: B*T = %lld tokens, above 2^31-1 per call", static_cast<long long>(B * T));
  const int32_t* hist = st != nullptr ? st->ids : nullptr;
  const int out = out_order >= 0 ? out_order : (L->w_mx != nullptr ? engram::kGatherOutMXFP8 : hdtype);
  engram::HotArgs hot;
  bool any_hot;
  const engram_status r = check_hot(L->hot, &L->hash, &L->tables, &hot, &any_hot);
  if (r != ENGRAM_OK) return r;
  prof_mark(stream, any_hot ? "gather_kernel<hashed,hot>" : "gather_kernel<hashed>");
  return hip_status(engram::launch_hash_gather(tokens, B, T, hist, L->hash.proj, ha, ta, any_hot ? &hot : nullptr,
                                               out, e, stream),
                    "hash+gather launch");
}

// Steps 5-8 on gathered rows e.
engram_status run_compute(const int32_t* tokens, const void* e, void* H, int64_t B, int64_t T,
                          const engram_layer* L, engram::GateConvArgs g, engram_decode_state* st,
                          float* alpha_out, float* y_out, const ComputeWorkspace& f, hipStream_t stream,
                          const engram::GatherJob* next = nullptr) {
  const int64_t n_tok = B * T;
  const int64_t d_mem = static_cast<int64_t>(L->tables.n_tables) * L->tables.dim;
  const int M = g.branches, d = g.d;
  const int64_t n_out = static_cast<int64_t>(1 + M) * d;
  engram_status r;
  if (use_fused(L)) {
    // Step 5 with the gate's sums folded into the product's epilogue; only v is stored
    engram::ProjGateArgs pa{};
    const bool mx = L->w_mx != nullptr;
    pa.e = static_cast<const uint16_t*>(e);
    pa.w = static_cast<const uint16_t*>(mx ? static_cast<const void*>(L->w_mx) : L->w);
    if (mx) {
      pa.e_scale = static_cast<const uint8_t*>(e) + n_tok * d_mem;   // after the codes
      pa.w_scale = L->w_mx_scale;
      pa.w_packed = L->w_mx_packed;
    }
    pa.H = static_cast<const uint16_t*>(H);
    pa.v = f.kv;
    pa.stats = f.stats;
    pa.n_tok = n_tok;
    pa.K = static_cast<int>(d_mem);
    pa.N = static_cast<int>(n_out);
    pa.d = d;
    pa.M = M;
    const engram::ProjGateLayout pl =
        engram::proj_gate_layout(n_tok, static_cast<int>(n_out), d, static_cast<int>(d_mem), M, mx);
    // Decode step (T = 1, the strip conv): the state's ids and pos advance in
    // this launch and the conv writes the new ring row, so no commit kernel
    bool fold = false;
    if (st != nullptr && T == 1 && tokens != nullptr && st->ids != nullptr) {
      engram::ConvArgs probe{};
      probe.g = g;
      probe.qv = pl.qv;
      probe.qk = pl.qk;
      probe.mixed = pl.mixed;
      probe.B = B;
      probe.T = T;
      fold = engram::conv_strip_ts(probe) == 1;
    }
    if (fold) {
      pa.st_ids = st->ids;
      pa.st_pos = st->pos;
      pa.tokens = tokens;
      pa.proj = L->hash.proj;
      pa.vocab = static_cast<int32_t>(L->hash.vocab);
      pa.err = g_err_word.load();
      pa.max_n = L->hash.max_n;
      pa.adv_T = static_cast<int32_t>(T);
      pa.adv_B = static_cast<int32_t>(B);
    }
    prof_mark(stream, "proj_gate_kernel");
    r = hip_status(engram::launch_proj_gate(pa, stream), "projection launch");
    if (r != ENGRAM_OK) return r;
    return run_conv_commit(H, f.kv, d, ENGRAM_F32, f.stats, pl.qv, pl.qk, pl.mixed, B, T, g, st, tokens, L->hash.proj,
                           L->hash.max_n, static_cast<int32_t>(L->hash.vocab), alpha_out, f.gamma, y_out, stream, next, fold);
  }
  // Step 5 into float32 projections, then whole-row gate statistics
  prof_mark(stream, "gemm_kernel");
  r = hip_status(engram::launch_project_kv(e, L->w, n_tok, d_mem, n_out, g.hdtype, ENGRAM_F32, f.kv, stream),
                 "project_kv launch");
  if (r != ENGRAM_OK) return r;
  g.kvdtype = ENGRAM_F32;
  prof_mark(stream, "gate_stats_kernel");
  r = hip_status(engram::launch_gate_stats(H, f.kv, n_tok, g, f.stats, stream), "gate statistics launch");
  if (r != ENGRAM_OK) return r;
  return run_conv_commit(H, f.kv, n_out, ENGRAM_F32, f.stats, 1, 1, false, B, T, g, st, tokens, L->hash.proj,
                         L->hash.max_n, static_cast<int32_t>(L->hash.vocab), alpha_out, f.gamma, y_out, stream, next);
}

}  // namespace

ENGRAM_API size_t engram_forward_workspace(int64_t B, int64_t T, const engram_layer* L) {
  if (L == nullptr || B < 0 || T < 0 || L->gc.branches < 1 || L->tables.n_tables < 1) return 0;
  return forward_ws_bytes(B * T, L);
}

ENGRAM_API engram_status engram_forward(const int32_t* tokens, void* H, int64_t B, int64_t T,
                                        const engram_layer* L, engram_decode_state* st,
                                        float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("forward", L, st, true, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  const int64_t n_tok = B * T;
  if (n_tok == 0) return ENGRAM_OK;
  if (tokens == nullptr || H == nullptr) return fail(ENGRAM_EINVAL, "forward: tokens and H must be non-NULL");
  if (!aligned(H, 16)) return fail(ENGRAM_EINVAL, "forward: H must be 16-byte aligned");
  if (y_out != nullptr && !aligned(y_out, 16)) return fail(ENGRAM_EINVAL, "forward: y_out must be 16-byte aligned");
  const size_t need = forward_ws_bytes(n_tok, L);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "forward: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  Carve c{static_cast<char*>(ws)};
  void* e = c.take<char>(rows_bytes(n_tok, L));
  const ComputeWorkspace f = carve_compute(c, n_tok, L);
  prof_begin();
  r = run_retrieve(tokens, B, T, L, ha, ta, g.hdtype, st, e, stream);
  if (r != ENGRAM_OK) return r;
  return run_compute(tokens, e, H, B, T, L, g, st, alpha_out, y_out, f, stream);
}

namespace {

// Scratch of engram_forward_noalloc: a device global, so each GPU holds its
// own copy (at its own address) from the moment the library's code is loaded
// there until the process ends.  On the host `scratch` names a stand-in, not
// device memory: host code takes the array's device address from
// hipGetSymbolAddress, once per device with that device current, and passes
// only that address on.
static __device__ __align__(256) unsigned char scratch[ENGRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch.
engram_status current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ENGRAM_EUNSUPPORTED, "forward_noalloc: device %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256)) return fail(ENGRAM_EHIP, "forward_noalloc: scratch address not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ENGRAM_OK;
}

}  // namespace

ENGRAM_API engram_status engram_forward_noalloc(const int32_t* tokens, void* H, int64_t B, int64_t T,
                                                const engram_layer* L, engram_decode_state* st, float* alpha_out,
                                                float* y_out, hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("forward_noalloc", L, st, true, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  const int64_t n_tok = B * T;
  if (n_tok == 0) return ENGRAM_OK;
  const size_t need = forward_ws_bytes(n_tok, L);
  if (need > ENGRAM_NOALLOC_SCRATCH_BYTES)
    return fail(ENGRAM_EINVAL, "forward_noalloc: the call needs %zu bytes of workspace, above the %u-byte scratch",
                need, ENGRAM_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((r = current_scratch(&ws)) != ENGRAM_OK) return r;
  return engram_forward(tokens, H, B, T, L, st, alpha_out, y_out, ws, ENGRAM_NOALLOC_SCRATCH_BYTES, stream);
}

ENGRAM_API engram_status engram_retrieve(const int32_t* tokens, int64_t B, int64_t T, const engram_layer* L,
                                         const engram_decode_state* st, void* e, hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("retrieve", L, st, true, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  if (B * T == 0) return ENGRAM_OK;
  if (tokens == nullptr || e == nullptr) return fail(ENGRAM_EINVAL, "retrieve: tokens and e must be non-NULL");
  if (!aligned(e, 16)) return fail(ENGRAM_EINVAL, "retrieve: e must be 16-byte aligned");
  prof_begin();
  return run_retrieve(tokens, B, T, L, ha, ta, g.hdtype, st, e, stream);
}

ENGRAM_API size_t engram_forward_retrieved_workspace(int64_t B, int64_t T, const engram_layer* L) {
  if (L == nullptr || B < 0 || T < 0 || L->gc.branches < 1 || L->tables.n_tables < 1) return 0;
  return compute_ws_bytes(B * T, L);
}

ENGRAM_API engram_status engram_forward_retrieved(const int32_t* tokens, const void* e, void* H, int64_t B,
                                                  int64_t T, const engram_layer* L, engram_decode_state* st,
                                                  float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                                                  hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("forward_retrieved", L, st, true, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  const int64_t n_tok = B * T;
  if (n_tok == 0) return ENGRAM_OK;
  if (e == nullptr || H == nullptr) return fail(ENGRAM_EINVAL, "forward_retrieved: e and H must be non-NULL");
  if (st != nullptr && tokens == nullptr)
    return fail(ENGRAM_EINVAL, "forward_retrieved: tokens must be non-NULL with a decode state");
  if (!aligned(H, 16) || !aligned(e, 16))
    return fail(ENGRAM_EINVAL, "forward_retrieved: H and e must be 16-byte aligned");
  if (y_out != nullptr && !aligned(y_out, 16))
    return fail(ENGRAM_EINVAL, "forward_retrieved: y_out must be 16-byte aligned");
  const size_t need = compute_ws_bytes(n_tok, L);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "forward_retrieved: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  Carve c{static_cast<char*>(ws)};
  const ComputeWorkspace f = carve_compute(c, n_tok, L);
  prof_begin();
  return run_compute(tokens, e, H, B, T, L, g, st, alpha_out, y_out, f, stream);
}

ENGRAM_API engram_status engram_forward_retrieved_prefetch(const int32_t* tokens, const void* e, void* H, int64_t B,
                                                           int64_t T, const engram_layer* L, engram_decode_state* st,
                                                           float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                                                           const engram_layer* next_L,
                                                           const engram_decode_state* next_st,
                                                           const int32_t* next_tokens, int64_t next_B, int64_t next_T,
                                                           void* next_e, hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("forward_retrieved_prefetch", L, st, true, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  if (next_st != nullptr && (next_st == st || next_st->ids == nullptr))
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: next_st must have ids and must not be st");
  // the next retrieval's layer (its hash, tables and row format)
  const engram_layer* NL = next_L != nullptr ? next_L : L;
  engram::HashArgs nha;
  engram::TableArgs nta;
  engram::GateConvArgs ng;
  if (NL != L && (r = check_layer(NL, &nha, &nta, &ng)) != ENGRAM_OK) return r;
  if (NL == L) {
    nha = ha;
    nta = ta;
    ng = g;
  }
  if (next_B < 0 || next_T < 0 || next_T > INT32_MAX || next_B > 65535)
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: next_B and next_T outside [0, 65535] x [0, 2^31)");
  const int64_t n_tok = B * T, n_next = next_B * next_T;
  if (n_next > 0) {
    if (next_tokens == nullptr || next_e == nullptr)
      return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: next_tokens and next_e must be non-NULL");
    if (!aligned(next_e, 16)) return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: next_e must be 16-byte aligned");
    if (next_e == e) return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: next_e must not be e");
  }
  engram::GatherJob job{};
  job.ta = nta;
  engram::HotArgs hot;
  bool any_hot;
  if ((r = check_hot(NL->hot, &NL->hash, &NL->tables, &hot, &any_hot)) != ENGRAM_OK) return r;
  job.hs = engram::HashSrc{next_tokens, NL->hash.proj, next_st != nullptr ? next_st->ids : nullptr, next_T, nha, hot};
  job.e = next_e;
  job.n_tok = static_cast<uint32_t>(n_next);
  job.out_dtype = NL->w_mx != nullptr ? engram::kGatherOutMXFP8 : ng.hdtype;
  job.hot = any_hot;
  if (n_next >= (1ll << 31)) return fail(ENGRAM_EUNSUPPORTED, "forward_retrieved_prefetch: next batch too large");
  if (n_tok == 0) {
    if (n_next == 0) return ENGRAM_OK;
    prof_begin();
    return run_retrieve(next_tokens, next_B, next_T, NL, nha, nta, ng.hdtype, next_st, next_e, stream);
  }
  if (e == nullptr || H == nullptr)
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: e and H must be non-NULL");
  if (st != nullptr && tokens == nullptr)
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: tokens must be non-NULL with a decode state");
  if (!aligned(H, 16) || !aligned(e, 16))
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: H and e must be 16-byte aligned");
  if (y_out != nullptr && !aligned(y_out, 16))
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: y_out must be 16-byte aligned");
  const size_t need = compute_ws_bytes(n_tok, L);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "forward_retrieved_prefetch: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                need, ws_bytes);
  Carve c{static_cast<char*>(ws)};
  const ComputeWorkspace f = carve_compute(c, n_tok, L);
  prof_begin();
  return run_compute(tokens, e, H, B, T, L, g, st, alpha_out, y_out, f, stream, n_next > 0 ? &job : nullptr);
}

// ---- Steps 1-5 ahead of the hidden states ----

namespace {

// The gathered rows of each layer, for whole 64-token tiles (the
// fragment-operand product reads whole tiles; the rows past the last token
// only reach output columns that are not stored).
size_t ahead_ws_bytes(int64_t n_tok, int32_t n_layers, const engram_layer* const* layers) {
  Carve c{nullptr};
  for (int l = 0; l < n_layers; ++l) c.take<char>(rows_bytes((n_tok + 63) / 64 * 64, layers[l]));
  return c.used;
}

// The gather job of one layer (cold rows; the hot tier is not supported here).
engram::GatherJob gather_job(const int32_t* tokens, int64_t T, int64_t n_tok, const engram_layer* L,
                             const engram::HashArgs& ha, const engram::TableArgs& ta, int hdtype,
                             const engram_decode_state* st, void* e) {
  engram::GatherJob j{};
  j.ta = ta;
  j.hs = engram::HashSrc{tokens, L->hash.proj, st != nullptr ? st->ids : nullptr, T, ha, engram::HotArgs{}};
  j.e = e;
  j.n_tok = static_cast<uint32_t>(n_tok);
  j.out_dtype = L->w_mx != nullptr ? engram::kGatherOutMXFP8 : hdtype;
  j.hot = false;
  return j;
}

// Whether layer L's product in engram_project_ahead takes the fragment-operand
// kernel (its gathered rows are then written in that kernel's operand order).
bool ahead_frag(const engram_layer* L, int64_t n_tok, int N, int d, int K) {
  return L->w_packed != nullptr && L->w_mx == nullptr && engram::proj_frag_for(n_tok, N, d, K);
}

}  // namespace

ENGRAM_API size_t engram_project_ahead_workspace(int64_t B, int64_t T, int32_t n_layers,
                                                 const engram_layer* const* layers) {
  if (layers == nullptr || B < 0 || T < 0 || n_layers < 1 || n_layers > ENGRAM_MAX_AHEAD_LAYERS) return 0;
  for (int l = 0; l < n_layers; ++l)
    if (layers[l] == nullptr || layers[l]->tables.n_tables < 1) return 0;
  return ahead_ws_bytes(B * T, n_layers, layers);
}

ENGRAM_API engram_status engram_project_ahead(const int32_t* tokens, int64_t B, int64_t T, int32_t n_layers,
                                              const engram_layer* const* layers, engram_decode_state* const* states,
                                              float* const* kv, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_layers < 1 || n_layers > ENGRAM_MAX_AHEAD_LAYERS)
    return fail(ENGRAM_EINVAL, "project_ahead: n_layers must be 1..%d", ENGRAM_MAX_AHEAD_LAYERS);
  if (layers == nullptr || kv == nullptr) return fail(ENGRAM_EINVAL, "project_ahead: layers and kv must be non-NULL");
  engram::HashArgs ha[ENGRAM_MAX_AHEAD_LAYERS];
  engram::TableArgs ta[ENGRAM_MAX_AHEAD_LAYERS];
  engram::GateConvArgs g[ENGRAM_MAX_AHEAD_LAYERS];
  const int64_t n_tok = B * T;
  engram_status r;
  for (int l = 0; l < n_layers; ++l) {
    const engram_layer* L = layers[l];
    if (L == nullptr) return fail(ENGRAM_EINVAL, "project_ahead: layers[%d] is NULL", l);
    engram_decode_state* st = states != nullptr ? states[l] : nullptr;
    if (states != nullptr && st == nullptr)
      return fail(ENGRAM_EINVAL, "project_ahead: states[%d] is NULL (give a state for every layer or none)", l);
    if ((r = check_call("project_ahead", L, st, true, B, T, &ha[l], &ta[l], &g[l])) != ENGRAM_OK) return r;
    if (!use_fused(L))
      return fail(ENGRAM_EUNSUPPORTED, "project_ahead: layer %d needs bf16 H, d a multiple of 128 up to 4096", l);
    if (L->hot != nullptr) return fail(ENGRAM_EUNSUPPORTED, "project_ahead: layer %d has a hot tier", l);
    if (st != nullptr && T != 1) return fail(ENGRAM_EUNSUPPORTED, "project_ahead: with decode states T must be 1");
    if (n_tok > 0 && (kv[l] == nullptr || !aligned(kv[l], 16)))
      return fail(ENGRAM_EINVAL, "project_ahead: kv[%d] must be non-NULL and 16-byte aligned", l);
  }
  if (n_tok == 0) return ENGRAM_OK;
  if (tokens == nullptr) return fail(ENGRAM_EINVAL, "project_ahead: tokens must be non-NULL");
  if (n_tok >= (int64_t{1} << 31))
    return fail(ENGRAM_EUNSUPPORTED, "project_ahead: B*T = %lld tokens, above 2^31-1 per call",
                static_cast<long long>(n_tok));
  const size_t need = ahead_ws_bytes(n_tok, n_layers, layers);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "project_ahead: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  // the product of each layer, and whether it takes the small-batch kernel
  engram::ProjGateArgs pa[ENGRAM_MAX_AHEAD_LAYERS];
  bool small[ENGRAM_MAX_AHEAD_LAYERS], frag[ENGRAM_MAX_AHEAD_LAYERS], fused[ENGRAM_MAX_AHEAD_LAYERS];
  void* e[ENGRAM_MAX_AHEAD_LAYERS];
  Carve c{static_cast<char*>(ws)};
  for (int l = 0; l < n_layers; ++l) {
    const engram_layer* L = layers[l];
    engram_decode_state* st = states != nullptr ? states[l] : nullptr;
    e[l] = c.take<char>(rows_bytes((n_tok + 63) / 64 * 64, L));
    const int64_t d_mem = static_cast<int64_t>(L->tables.n_tables) * L->tables.dim;
    const int M = g[l].branches, d = g[l].d;
    const bool mx = L->w_mx != nullptr;
    engram::ProjGateArgs& p = pa[l];
    p = engram::ProjGateArgs{};
    p.e = static_cast<const uint16_t*>(e[l]);
    p.w = static_cast<const uint16_t*>(mx ? static_cast<const void*>(L->w_mx) : L->w);
    if (mx) {
      p.e_scale = static_cast<const uint8_t*>(e[l]) + n_tok * d_mem;
      p.w_scale = L->w_mx_scale;
    }
    p.kv_out = kv[l];
    p.n_tok = n_tok;
    p.K = static_cast<int>(d_mem);
    p.N = static_cast<int>(static_cast<int64_t>(1 + M) * d);
    p.d = d;
    p.M = M;
    if (st != nullptr) {
      p.st_ids = st->ids;
      p.st_pos = st->pos;
      p.tokens = tokens;
      p.proj = L->hash.proj;
      p.vocab = static_cast<int32_t>(L->hash.vocab);
      p.err = g_err_word.load();
      p.max_n = L->hash.max_n;
      p.adv_T = static_cast<int32_t>(T);
      p.adv_B = static_cast<int32_t>(B);
    }
    small[l] = engram::proj_gate_small_for(n_tok, p.N, d, p.K, mx) && p.K % (mx ? 512 : 64) == 0;
    frag[l] = ahead_frag(L, n_tok, p.N, d, p.K);
    if (frag[l]) p.w_frag = static_cast<const uint16_t*>(L->w_packed);
    fused[l] = frag[l] && engram::ahead_fused_for(ta[l], n_tok, p.N, d, p.K);
    if (!small[l] && (mx || st != nullptr))
      return fail(ENGRAM_EUNSUPPORTED,
                  "project_ahead: layer %d's product (%lld tokens x %d columns) is above the small-batch range, which "
                  "MXFP8 layers and decode states need",
                  l, static_cast<long long>(n_tok), p.N);
  }
  prof_begin();
  for (int l = 0; l < n_layers; l += 2) {
    const bool pair = l + 1 < n_layers;
    // Steps 1-5 of the pair in one launch where both layers allow it
    if (fused[l] && (!pair || fused[l + 1])) {
      engram::AheadJob ja{}, jb{};
      ja.g = gather_job(tokens, T, n_tok, layers[l], ha[l], ta[l], g[l].hdtype,
                        states != nullptr ? states[l] : nullptr, e[l]);
      ja.p = pa[l];
      if (pair) {
        jb.g = gather_job(tokens, T, n_tok, layers[l + 1], ha[l + 1], ta[l + 1], g[l + 1].hdtype,
                          states != nullptr ? states[l + 1] : nullptr, e[l + 1]);
        jb.p = pa[l + 1];
      }
      prof_mark(stream, "gather_proj_kernel");
      const hipError_t he = engram::launch_ahead_fused(ja, pair ? &jb : nullptr, stream);
      if (he != hipErrorNotSupported) {
        if ((r = hip_status(he, "gather+projection launch")) != ENGRAM_OK) return r;
        continue;
      }
    }
    // Steps 1-4 of the pair in one launch where the formats match
    const int out_a = frag[l] ? engram::kGatherOutFrag16 : -1;
    const int out_b = pair && frag[l + 1] ? engram::kGatherOutFrag16 : -1;
    engram::GatherJob ja = gather_job(tokens, T, n_tok, layers[l], ha[l], ta[l], g[l].hdtype,
                                      states != nullptr ? states[l] : nullptr, e[l]);
    if (out_a >= 0) ja.out_dtype = out_a;
    bool gathered = false;
    if (pair) {
      engram::GatherJob jb = gather_job(tokens, T, n_tok, layers[l + 1], ha[l + 1], ta[l + 1], g[l + 1].hdtype,
                                        states != nullptr ? states[l + 1] : nullptr, e[l + 1]);
      if (out_b >= 0) jb.out_dtype = out_b;
      prof_mark(stream, "gather2_kernel");
      const hipError_t he = engram::launch_hash_gather2(ja, jb, stream);
      if (he != hipErrorNotSupported) {
        if ((r = hip_status(he, "two-layer gather launch")) != ENGRAM_OK) return r;
        gathered = true;
      }
    }
    if (!gathered) {
      for (int k = l; k < l + (pair ? 2 : 1); ++k) {
        engram_decode_state* st = states != nullptr ? states[k] : nullptr;
        if ((r = run_retrieve(tokens, B, T, layers[k], ha[k], ta[k], g[k].hdtype, st, e[k], stream,
                              frag[k] ? engram::kGatherOutFrag16 : -1)) != ENGRAM_OK)
          return r;
      }
    }
    // Step 5 of the pair
    if (small[l] && (!pair || small[l + 1])) {
      prof_mark(stream, "proj_kv_kernel");
      const hipError_t he = engram::launch_project_layers(pa[l], pair ? &pa[l + 1] : nullptr, stream);
      if (he != hipErrorNotSupported) {
        if ((r = hip_status(he, "projection launch")) != ENGRAM_OK) return r;
        continue;
      }
    }
    for (int k = l; k < l + (pair ? 2 : 1); ++k) {
      if (small[k]) {
        prof_mark(stream, "proj_kv_kernel");
        r = hip_status(engram::launch_project_layers(pa[k], nullptr, stream), "projection launch");
      } else {
        prof_mark(stream, "gemm_kernel");
        r = hip_status(engram::launch_project_kv(e[k], layers[k]->w, n_tok, pa[k].K, pa[k].N, ENGRAM_BF16, ENGRAM_F32,
                                                 kv[k], stream),
                       "project_kv launch");
      }
      if (r != ENGRAM_OK) return r;
    }
  }
  prof_mark(stream, nullptr);
  return ENGRAM_OK;
}

ENGRAM_API size_t engram_forward_projected_workspace(int64_t B, int64_t T, const engram_layer* L) {
  if (L == nullptr || B < 0 || T < 0 || L->gc.branches < 1) return 0;
  return gc_ws_bytes(B * T, L->gc.branches);
}

ENGRAM_API engram_status engram_forward_projected(const float* kv, void* H, int64_t B, int64_t T,
                                                  const engram_layer* L, engram_decode_state* st, float* alpha_out,
                                                  float* y_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram::GateConvArgs g;
  engram_status r = check_call("forward_projected", L, st, false, B, T, &ha, &ta, &g);
  if (r != ENGRAM_OK) return r;
  if (!use_fused(L))
    return fail(ENGRAM_EUNSUPPORTED, "forward_projected: the layer needs bf16 H, d a multiple of 128 up to 4096");
  const int64_t n_tok = B * T;
  const int M = g.branches, d = g.d;
  // one launch: a single-token chunk whose rows fit one conv workgroup
  const bool one = T == 1 && d <= 1024 && g.kernel_w == 4 && g.dilation == 3;
  if (st != nullptr && !one)
    return fail(ENGRAM_EUNSUPPORTED,
                "forward_projected: with a decode state, T = 1, d <= 1024 and the conv w = 4, dilation 3");
  if (n_tok == 0) return ENGRAM_OK;
  if (kv == nullptr || H == nullptr) return fail(ENGRAM_EINVAL, "forward_projected: kv and H must be non-NULL");
  if (!aligned(H, 16) || !aligned(kv, 16)) return fail(ENGRAM_EINVAL, "forward_projected: H and kv must be 16-byte aligned");
  if (y_out != nullptr && !aligned(y_out, 16))
    return fail(ENGRAM_EINVAL, "forward_projected: y_out must be 16-byte aligned");
  const size_t need = gc_ws_bytes(n_tok, M);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "forward_projected: workspace needs %zu bytes, 256-byte aligned (got %zu)", need,
                ws_bytes);
  Carve c{static_cast<char*>(ws)};
  const GcWorkspace w = carve_gc(c, n_tok, M);
  const int64_t n_out = static_cast<int64_t>(1 + M) * d;
  g.kvdtype = ENGRAM_F32;
  prof_begin();
  if (one) {
    engram::ConvArgs ca{};
    ca.H = H;
    ca.v = kv;
    ca.v_stride = n_out;
    ca.qv = 1;
    ca.qk = 1;
    ca.kq0 = 1;
    ca.nq = 1 + M;
    ca.B = B;
    ca.T = T;
    ca.g = g;
    ca.has_state = st != nullptr;
    if (st != nullptr) ca.st = engram::StateArgs{st->ids, st->conv, st->pos};
    ca.pos_advanced = st != nullptr;   // advanced by engram_project_ahead
    ca.commit_u = st != nullptr;
    ca.sums_from_kv = 1;
    ca.alpha_out = alpha_out;
    ca.gamma_out = w.gamma;
    ca.y_out = y_out;
    prof_mark(stream, "conv_kernel");
    r = hip_status(engram::launch_conv(ca, ENGRAM_F32, stream), "conv launch");
    prof_mark(stream, nullptr);
    return r;
  }
  prof_mark(stream, "gate_stats_kernel");
  r = hip_status(engram::launch_gate_stats(H, kv, n_tok, g, w.stats, stream), "gate statistics launch");
  if (r != ENGRAM_OK) return r;
  return run_conv_commit(H, kv, n_out, ENGRAM_F32, w.stats, 1, 1, false, B, T, g, nullptr, nullptr, L->hash.proj,
                         L->hash.max_n, static_cast<int32_t>(L->hash.vocab), alpha_out, w.gamma, y_out, stream);
}

ENGRAM_API size_t engram_cache_build_workspace(int64_t total_rows) {
  if (total_rows <= 0) return 0;
  return engram::cache_build_workspace(total_rows);
}

ENGRAM_API engram_status engram_cache_build(const int32_t* warm_tokens, int64_t B, int64_t T,
                                            const engram_hash_params* hp, const engram_tables* tab,
                                            int64_t cache_n, int32_t* cache_slot, void* cache_rows,
                                            float* cache_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  engram::HashArgs ha;
  engram::TableArgs ta;
  engram_status r = check_hash(hp, &ha);
  if (r != ENGRAM_OK) return r;
  if (tab == nullptr) return fail(ENGRAM_EINVAL, "cache_build: tables are NULL");
  engram_tables plain = *tab;   // the cache being built is not probed
  plain.cache_slot = nullptr;
  if ((r = check_tables(&plain, &ta)) != ENGRAM_OK) return r;
  if (tab->n_tables != ha.n_tables)
    return fail(ENGRAM_EINVAL, "cache_build: tables.n_tables=%d but the hash has %d tables", tab->n_tables,
                ha.n_tables);
  for (int j = 0; j < ha.n_tables; ++j)
    if (tab->n_rows[j] != static_cast<int64_t>(ha.prime[j]))
      return fail(ENGRAM_EINVAL, "cache_build: table %d has %lld rows but prime %u", j,
                  static_cast<long long>(tab->n_rows[j]), ha.prime[j]);
  if (B < 0 || T < 0) return fail(ENGRAM_EINVAL, "cache_build: B and T must be >= 0");
  if (B * T > 0 && warm_tokens == nullptr) return fail(ENGRAM_EINVAL, "cache_build: warm_tokens is NULL");
  if (cache_n < 0 || cache_n > tab->total_rows || tab->total_rows > 0x7fffffffLL)
    return fail(ENGRAM_EINVAL, "cache_build: need 0 <= cache_n <= total_rows < 2^31");
  if (cache_slot == nullptr || (cache_n > 0 && cache_rows == nullptr))
    return fail(ENGRAM_EINVAL, "cache_build: cache_slot and cache_rows must be non-NULL");
  if (tab->dtype == ENGRAM_I8 && cache_n > 0 && cache_scale == nullptr)
    return fail(ENGRAM_EINVAL, "cache_build: int8 tables need cache_scale");
  if (cache_rows != nullptr && !aligned(cache_rows, 8)) return fail(ENGRAM_EINVAL, "cache_build: cache_rows must be 8-byte aligned");
  const size_t need = engram::cache_build_workspace(tab->total_rows);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "cache_build: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  const int row_bytes = tab->dim * static_cast<int>(dtype_size(tab->dtype));
  return hip_status(engram::launch_cache_build(warm_tokens, B, T, hp->proj, ha, ta, tab->total_rows, row_bytes, cache_n,
                                               cache_slot, cache_rows, tab->dtype == ENGRAM_I8 ? cache_scale : nullptr,
                                               ws, stream),
                    "cache build launch");
}

ENGRAM_API size_t engram_cache_update_workspace(int64_t total_rows, int64_t cache_n) {
  if (total_rows <= 0 || cache_n < 0 || cache_n > total_rows) return 0;
  return engram::cache_update_workspace(total_rows, cache_n);
}

ENGRAM_API engram_status engram_cache_update(const engram_tables* tab, int64_t cache_n, int32_t* cache_slot,
                                             void* cache_rows, float* cache_scale, uint32_t* counts,
                                             int32_t decay_shift, void* ws, size_t ws_bytes, hipStream_t stream) {
  engram::TableArgs ta;
  if (tab == nullptr) return fail(ENGRAM_EINVAL, "cache_update: tables are NULL");
  engram_tables plain = *tab;   // the cache being updated is passed separately
  plain.cache_slot = nullptr;
  plain.access_counts = nullptr;
  engram_status r = check_tables(&plain, &ta);
  if (r != ENGRAM_OK) return r;
  if (cache_n < 0 || cache_n > tab->total_rows || tab->total_rows > 0x7fffffffLL)
    return fail(ENGRAM_EINVAL, "cache_update: need 0 <= cache_n <= total_rows < 2^31");
  if (cache_slot == nullptr || counts == nullptr || (cache_n > 0 && cache_rows == nullptr))
    return fail(ENGRAM_EINVAL, "cache_update: cache_slot, counts and cache_rows must be non-NULL");
  if (tab->dtype == ENGRAM_I8 && cache_n > 0 && cache_scale == nullptr)
    return fail(ENGRAM_EINVAL, "cache_update: int8 tables need cache_scale");
  if (!aligned(cache_rows, 8) || !aligned(counts, 4) || !aligned(cache_slot, 4))
    return fail(ENGRAM_EINVAL, "cache_update: misaligned cache_rows, counts or cache_slot");
  if (decay_shift < 0 || decay_shift > 31) return fail(ENGRAM_EINVAL, "cache_update: decay_shift outside [0, 31]");
  const size_t need = engram::cache_update_workspace(tab->total_rows, cache_n);
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256))
    return fail(ENGRAM_EINVAL, "cache_update: workspace needs %zu bytes, 256-byte aligned (got %zu)", need, ws_bytes);
  const int row_bytes = tab->dim * static_cast<int>(dtype_size(tab->dtype));
  return hip_status(engram::launch_cache_update(ta, tab->total_rows, row_bytes, cache_n, cache_slot, cache_rows,
                                                tab->dtype == ENGRAM_I8 ? cache_scale : nullptr, counts, decay_shift,
                                                ws, stream),
                    "cache update launch");
}

ENGRAM_API engram_status engram_quantize_mxfp8(const void* x, engram_dtype dtype, int64_t rows, int64_t cols,
                                               uint8_t* q, uint8_t* scale, hipStream_t stream) {
  if (dtype != ENGRAM_F32 && dtype != ENGRAM_BF16) return fail(ENGRAM_EUNSUPPORTED, "quantize_mxfp8: dtype F32 or BF16");
  if (rows < 0 || cols < 0 || cols % 32 != 0)
    return fail(ENGRAM_EINVAL, "quantize_mxfp8: rows >= 0 and cols a non-negative multiple of 32");
  if (rows * cols == 0) return ENGRAM_OK;
  if (x == nullptr || q == nullptr || scale == nullptr)
    return fail(ENGRAM_EINVAL, "quantize_mxfp8: x, q and scale must be non-NULL");
  if (!aligned(x, dtype == ENGRAM_F32 ? 32 : 16) || !aligned(q, 8))
    return fail(ENGRAM_EINVAL, "quantize_mxfp8: x must be 16-byte (BF16) or 32-byte (F32) aligned, q 8-byte");
  return hip_status(engram::launch_mx_quantize(x, dtype, rows, cols, q, scale, stream), "quantize launch");
}

ENGRAM_API engram_status engram_pack_bf16(const void* w, int64_t rows, int64_t cols, void* packed,
                                          hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % 32 != 0 || cols % 16 != 0)
    return fail(ENGRAM_EINVAL, "pack_bf16: rows a non-negative multiple of 32 and cols of 16");
  if (rows * cols == 0) return ENGRAM_OK;
  if (w == nullptr || packed == nullptr) return fail(ENGRAM_EINVAL, "pack_bf16: w and packed must be non-NULL");
  if (!aligned(w, 16) || !aligned(packed, 16))
    return fail(ENGRAM_EINVAL, "pack_bf16: w and packed must be 16-byte aligned");
  return hip_status(engram::launch_bf16_pack(static_cast<const uint16_t*>(w), rows, cols,
                                             static_cast<uint16_t*>(packed), stream),
                    "pack launch");
}

ENGRAM_API engram_status engram_pack_mxfp8(const uint8_t* q, const uint8_t* scale, int64_t rows, int64_t cols,
                                           uint8_t* packed, hipStream_t stream) {
  if (rows < 0 || cols < 0 || rows % 32 != 0 || cols % 256 != 0)
    return fail(ENGRAM_EINVAL, "pack_mxfp8: rows a non-negative multiple of 32 and cols of 256");
  if (rows * cols == 0) return ENGRAM_OK;
  if (q == nullptr || scale == nullptr || packed == nullptr)
    return fail(ENGRAM_EINVAL, "pack_mxfp8: q, scale and packed must be non-NULL");
  if (!aligned(q, 16) || !aligned(packed, 16))
    return fail(ENGRAM_EINVAL, "pack_mxfp8: q and packed must be 16-byte aligned");
  return hip_status(engram::launch_mx_pack(q, scale, rows, cols, packed, stream), "pack launch");
}

ENGRAM_API engram_status engram_profile_enable(int32_t on) {
  if (on < 0 || on > 2) return fail(ENGRAM_EINVAL, "profile_enable: mode must be 0, 1 or 2");
  Profiler& p = g_prof;
  const int want = on == 2 ? kMaxStages : (on == 1 ? kCallStages : 0);
  for (; p.created < want; ++p.created) {
    hipError_t e = hipEventCreate(&p.start[p.created]);
    if (e == hipSuccess) e = hipEventCreate(&p.stop[p.created]);
    if (e != hipSuccess) return hip_status(e, "hipEventCreate");
  }
  p.mode = on;
  p.n = 0;
  p.dropped = 0;
  p.pending = nullptr;
  return ENGRAM_OK;
}

ENGRAM_API engram_status engram_profile_read(float* ms, const char** names, int32_t cap, int32_t* n_stages) {
  Profiler& p = g_prof;
  if (n_stages == nullptr || (cap > 0 && ms == nullptr))
    return fail(ENGRAM_EINVAL, "profile_read: n_stages and ms must be non-NULL");
  *n_stages = 0;
  if (p.mode == 0 || p.n < 1) return fail(ENGRAM_EINVAL, "profile_read: no profiled call recorded");
  if (p.dropped != 0) {
    p.n = 0;
    p.dropped = 0;
    return fail(ENGRAM_EINVAL, "profile_read: more stages than the profiler holds since the last read");
  }
  hipError_t e = hipEventSynchronize(p.stop[p.n - 1]);
  if (e != hipSuccess) return hip_status(e, "hipEventSynchronize");
  const int stages = p.n;
  for (int i = 0; i < stages && i < cap; ++i) {
    float t = 0.f;
    e = hipEventElapsedTime(&t, p.start[i], p.stop[i]);
    if (e != hipSuccess) return hip_status(e, "hipEventElapsedTime");
    ms[i] = t;
    if (names != nullptr) names[i] = p.names[i];
  }
  *n_stages = stages;
  if (p.mode == 2) p.n = 0;
  return ENGRAM_OK;
}

ENGRAM_API engram_status engram_host_alloc(size_t bytes, void** host_ptr, void** device_alias) {
  if (host_ptr == nullptr || device_alias == nullptr || bytes == 0)
    return fail(ENGRAM_EINVAL, "host_alloc: need bytes > 0 and non-NULL out pointers");
  *host_ptr = nullptr;
  *device_alias = nullptr;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess) return hip_status(e, "hipHostMalloc");
  void* dptr = nullptr;
  e = hipHostGetDevicePointer(&dptr, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return hip_status(e, "hipHostGetDevicePointer");
  }
  *host_ptr = h;
  *device_alias = dptr;
  return ENGRAM_OK;
}

ENGRAM_API engram_status engram_host_free(void* host_ptr) {
  if (host_ptr == nullptr) return ENGRAM_OK;
  return hip_status(hipHostFree(host_ptr), "hipHostFree");
}

ENGRAM_API size_t engram_hot_buckets(int64_t n_hot) {
  return n_hot <= 0 ? 0 : static_cast<size_t>(engram::hot_buckets(static_cast<uint64_t>(n_hot)));
}

ENGRAM_API engram_status engram_hot_build(const int32_t* keys, int64_t n_hot, int32_t n, uint64_t seed,
                                          uint32_t* pilots, engram_hot_slot* slots, uint64_t* seed_used) {
  static_assert(sizeof(engram_hot_slot) == 32, "a hot slot is 32 bytes");
  if (n < 2 || n > ENGRAM_MAX_ORDER) return fail(ENGRAM_EINVAL, "hot build: n=%d outside [2, %d]", n, ENGRAM_MAX_ORDER);
  if (n_hot < 1 || n_hot > INT32_MAX) return fail(ENGRAM_EINVAL, "hot build: n_hot must be in [1, 2^31)");
  if (keys == nullptr || pilots == nullptr || slots == nullptr || seed_used == nullptr)
    return fail(ENGRAM_EINVAL, "hot build: keys, pilots, slots and seed_used must be non-NULL");
  for (int64_t q = 0; q < n_hot * n; ++q)
    if (keys[q] < 0) return fail(ENGRAM_EINVAL, "hot build: n-gram %lld holds a negative id", static_cast<long long>(q / n));
  for (int attempt = 0; attempt < 16; ++attempt) {
    const uint64_t s = seed + static_cast<uint64_t>(attempt);
    const engram::HotBuild b = engram::hot_build(keys, n_hot, n, s, pilots, reinterpret_cast<int32_t*>(slots));
    if (b.status == engram::HotBuild::kOk) {
      *seed_used = s;
      return ENGRAM_OK;
    }
    if (b.status == engram::HotBuild::kDuplicate)
      return fail(ENGRAM_EINVAL, "hot build: n-grams %u and %u are equal", b.a, b.b);
  }
  return fail(ENGRAM_EUNSUPPORTED, "hot build: no seed in [seed, seed+15] gave a perfect hash");
}

ENGRAM_API engram_status engram_hot_lookup(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                                           const engram_hash_params* hp, const engram_hot_tier* hot,
                                           int32_t* hot_row, hipStream_t stream) {
  engram::HashArgs ha;
  engram_status r = check_hash(hp, &ha);
  if (r != ENGRAM_OK) return r;
  if (hot == nullptr) return fail(ENGRAM_EINVAL, "hot lookup: hot is NULL");
  engram::HotArgs h;
  bool any;
  if ((r = check_hot(hot, hp, nullptr, &h, &any)) != ENGRAM_OK) return r;
  if (B < 0 || T < 0) return fail(ENGRAM_EINVAL, "hot lookup: B and T must be >= 0");
  if (B * T == 0) return ENGRAM_OK;
  if (tokens == nullptr || hot_row == nullptr) return fail(ENGRAM_EINVAL, "hot lookup: tokens and hot_row must be non-NULL");
  prof_begin();
  prof_mark(stream, "hot_lookup_kernel");
  return hip_status(engram::launch_hot_lookup(tokens, B, T, hist, hp->proj, hp->max_n, ha.vocab, h, hot_row,
                                                 g_err_word.load(), stream),
                    "hot lookup launch");
}

ENGRAM_API int32_t engram_debug_checks(void) { return engram::kDebugChecks ? 1 : 0; }

ENGRAM_API engram_status engram_debug_set_error_word(uint32_t* word) {
  if (!engram::kDebugChecks)
    return fail(ENGRAM_EUNSUPPORTED, "debug_set_error_word: this is the release build (use libengram_debug.so)");
  if (!aligned(word, 4)) return fail(ENGRAM_EINVAL, "debug_set_error_word: word must be 4-byte aligned");
  g_err_word.store(word);
  return ENGRAM_OK;
}

ENGRAM_API engram_status engram_debug_read_errors(uint32_t* bits) {
  if (!engram::kDebugChecks)
    return fail(ENGRAM_EUNSUPPORTED, "debug_read_errors: this is the release build (use libengram_debug.so)");
  if (bits == nullptr) return fail(ENGRAM_EINVAL, "debug_read_errors: bits is NULL");
  *bits = 0;
  uint32_t* word = g_err_word.load();
  if (word == nullptr) return fail(ENGRAM_EINVAL, "debug_read_errors: no error word is set");
  engram_status r = hip_status(hipDeviceSynchronize(), "hipDeviceSynchronize");
  if (r != ENGRAM_OK) return r;
  if ((r = hip_status(hipMemcpy(bits, word, sizeof(uint32_t), hipMemcpyDeviceToHost), "hipMemcpy")) != ENGRAM_OK)
    return r;
  return hip_status(hipMemset(word, 0, sizeof(uint32_t)), "hipMemset");
}
