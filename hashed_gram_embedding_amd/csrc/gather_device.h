// Device side of the hashed gather (Steps 1-4 of "DeepSeek Engram series
// guide", section "Engram working principle", with the Engram-Nine hot tier of
// its experiment 3): row loads, the output formats and the per-thread body of
// the kernel, shared by the gather kernel and the conv launch that carries the
// next batch's gather.  The design notes are in gather.hip.
#pragma once

#include "device_util.h"
#include "engram_internal.h"
#include "hash_device.h"
#include "hot_device.h"

namespace engram {

constexpr int kOutMXFP8 = kGatherOutMXFP8;
constexpr int kOutFrag16 = kGatherOutFrag16;

template <int IN>
__device__ __forceinline__ void load8(const void* base, const float* scale, int64_t row, int dim,
                                      int col, float* f, uint4* raw_bf16) {
  if constexpr (IN == ENGRAM_BF16) {
    const uint4 q = global_load16(static_cast<const uint16_t*>(base) + row * dim + col);
    *raw_bf16 = q;
    unpack8(q, f);
  } else if constexpr (IN == ENGRAM_F32) {
    const float* p = static_cast<const float*>(base) + row * dim + col;
    const uint4 qa = global_load16(p), qb = global_load16(p + 4);
    const float4 a = make_float4(__uint_as_float(qa.x), __uint_as_float(qa.y), __uint_as_float(qa.z),
                                 __uint_as_float(qa.w));
    const float4 b = make_float4(__uint_as_float(qb.x), __uint_as_float(qb.y), __uint_as_float(qb.z),
                                 __uint_as_float(qb.w));
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const int8_t*>(base) + row * dim + col);
    const float s = scale[row];
    const uint32_t w[2] = {q.x, q.y};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int8_t v = static_cast<int8_t>((w[i >> 2] >> (8 * (i & 3))) & 0xffu);
      f[i] = static_cast<float>(v) * s;
    }
  }
}

// Writes the 8 elements of one thread at element offset `out` of e.
template <int IN, int OUT>
__device__ __forceinline__ void store8(void* e, int64_t out, int64_t mx_scale_base, int c, const float* f,
                                       const uint4& raw, bool live) {
  if constexpr (OUT == kOutMXFP8) {
    // MXFP8 e: 8 codes per thread, the block scale from the 4 threads of the
    // block (rows are whole blocks: dim is a multiple of 32, so the groups
    // of 4 lanes never straddle rows or the grid's end; every lane of the
    // group takes part in the shuffle, stores are predicated)
    // the codes quantise the bf16 row values the bf16 product would read:
    // int8 and float32 rows are rounded to bf16 (RNE) first
    float fb[8];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      if constexpr (IN == ENGRAM_BF16) {
        fb[i] = f[i];
        fb[i + 1] = f[i + 1];
      } else {
        const uint32_t b = pack_bf16x2(f[i], f[i + 1]);
        fb[i] = __uint_as_float(b << 16);
        fb[i + 1] = __uint_as_float(b & 0xffff0000u);
      }
    }
    uint32_t sb;
    const uint2 q = mx_quantize8(fb, &sb);
    uint8_t* eq = static_cast<uint8_t*>(e);
    if (live) {
      *reinterpret_cast<uint2*>(eq + out) = q;
      if ((c & 3) == 0) eq[mx_scale_base + out / 32] = static_cast<uint8_t>(sb);
    }
  } else if constexpr (OUT == ENGRAM_BF16) {
    uint4 q;
    if constexpr (IN == ENGRAM_BF16) q = raw; else q = pack8(f);
    if (live) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(e) + out) = q;
  } else {
    if (live) {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(e) + out);
      p[0] = make_float4(f[0], f[1], f[2], f[3]);
      p[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
}

// Steps 1-4 with in-thread hashing; ITEMS consecutive tokens per thread.
// Thread gid serves tokens ITEMS*g .. ITEMS*g + ITEMS-1 of table j, chunk c,
// with (g, j, c) = gid split as [groups][n_tables][chunks]; a wavefront's
// store of one item is a contiguous span of e.  Token counts below 2^31
// (checked by the launcher) keep the index arithmetic in 32 bits.
template <int IN, int OUT, bool HOT, int ITEMS>
__device__ __forceinline__ void hashed_gather_body(uint32_t gid, uint32_t n_tok, const TableArgs& ta,
                                                   void* __restrict__ e, const HashSrc& hs) {
  // Every scalar argument the path needs is read in one batch with one wait:
  // the asm statements take them as operands, so all their loads are issued
  // before them.  Left to itself the compiler reads the grid bound's
  // arguments, waits, then reads the rest and waits again, two round trips
  // before the first id load.
  {
    const void* const p0 = hs.tokens;
    const void* const p1 = hs.proj;
    const void* const p2 = hs.hist;
    const void* const p3 = ta.rows;
    const void* const p4 = ta.scale;
    const void* const p5 = ta.cache_slot;
    const void* const p6 = ta.counts;
    const void* const p7 = e;
    const int32_t i0 = ta.n_tables, i1 = ta.dim, i2 = hs.a.max_n, i3 = hs.a.vocab;
    const int64_t i4 = hs.T;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(p5), "s"(p6), "s"(p7));
    asm volatile("" ::"s"(i0), "s"(i1), "s"(i2), "s"(i3), "s"(i4), "s"(n_tok));
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t nt = static_cast<uint32_t>(ta.n_tables);
  const uint32_t chunks = static_cast<uint32_t>(ta.dim) >> 3;
  const uint32_t per_group = nt * chunks;
  const uint32_t n_groups = (n_tok + ITEMS - 1) / ITEMS;
  if (gid >= n_groups * per_group) return;
  const uint32_t g = gid / per_group;
  const uint32_t jc = gid - g * per_group;
  const int j = static_cast<int>(jc / chunks);
  const int c = static_cast<int>(jc - static_cast<uint32_t>(j) * chunks);

  // per-table arguments first: their loads overlap the id loads
  const int64_t row_offset = ta.row_offset[j];
  const TableHash th = table_hash(hs.a, j);
  const uint32_t T = static_cast<uint32_t>(hs.T);

  uint32_t b[ITEMS], t[ITEMS];
  bool live[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const uint32_t tok = g * ITEMS + q;
    live[q] = tok < n_tok;
    const uint32_t tc = live[q] ? tok : n_tok - 1;
    b[q] = tc / T;
    t[q] = tc - b[q] * T;
  }
  // Steps 1-2: ids of the suffix window, newest first
  uint32_t x[ITEMS][ENGRAM_MAX_ORDER];
  window_ids_n<ITEMS>(hs, b, t, x);
  // Step 3: cold row of every item
  int64_t crow[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int32_t z = hash_of_ids(x[q], th);
    if constexpr (kDebugChecks) debug_record(hs.a.err, range_bit(z, th.prime, kErrRow));   // z < p by construction
    crow[q] = row_offset + z;
  }

  // Engram-Nine: hot row of every item (-1 = cold)
  int32_t hot[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) hot[q] = -1;
  const void* hot_rows = nullptr;
  int hot_col = 0;
  if constexpr (HOT) {
    const int n = th.n;
    const HotOrderArgs o = hot_order(hs.hot, n);
    hot_rows = o.rows;
    hot_col = (j - (n - 2) * hs.hot.heads) * ta.dim + c * 8;
    if (o.n_hot != 0) {
      uint64_t h[ITEMS];
      uint32_t pilot[ITEMS];
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        h[q] = hot_key_hash(x[q], n, o.seed);
        pilot[q] = global_load(o.pilots + hot_range(h[q], o.n_buckets));
      }
      uint4 sa[ITEMS], sb[ITEMS];
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        const uint64_t sl = hot_slot(h[q], pilot[q], o.n_hot);
        sa[q] = global_load16(o.slots + 2 * sl);
        sb[q] = global_load16(o.slots + 2 * sl + 1);
      }
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) {
        uint32_t xm[ENGRAM_MAX_ORDER];
#pragma unroll
        for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) xm[i] = i < n ? x[q][i] : 0u;
        const bool match = sa[q].x == xm[0] && sa[q].y == xm[1] && sa[q].z == xm[2] && sa[q].w == xm[3];
        hot[q] = match ? static_cast<int32_t>(sb[q].x) : -1;
        if constexpr (kDebugChecks) {
          if (hot[q] >= 0 && !in_range(hot[q], static_cast<int64_t>(o.n_hot))) {
            debug_record(hs.a.err, kErrHotRow);
            hot[q] = -1;   // read as cold
          }
        }
      }
    }
  }

  // Step 4: the source of every item (hot row, HBM cache slot or table row)
  const void* src[ITEMS];
  const float* scale[ITEMS];
  int64_t row[ITEMS];
  int len[ITEMS], col[ITEMS];
  int32_t slot[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) slot[q] = -1;
  if (ta.cache_slot != nullptr) {
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) slot[q] = ta.cache_slot[crow[q]];
    if constexpr (kDebugChecks) {
      uint32_t bits = 0;
#pragma unroll
      for (int q = 0; q < ITEMS; ++q) slot[q] = checked_slot(slot[q], ta.cache_n, &bits);
      debug_record(ta.err, bits);
    }
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const bool is_hot = HOT && hot[q] >= 0;
    const bool cached = !is_hot && slot[q] >= 0;
    src[q] = is_hot ? hot_rows : (cached ? ta.cache_rows : ta.rows);
    scale[q] = cached ? ta.cache_scale : ta.scale;
    row[q] = is_hot ? hot[q] : (cached ? slot[q] : crow[q]);
    len[q] = is_hot ? hs.hot.width : ta.dim;
    col[q] = is_hot ? hot_col : c * 8;
  }
  float f[ITEMS][8];
  uint4 raw[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) load8<IN>(src[q], scale[q], row[q], len[q], col[q], f[q], &raw[q]);
  if (ta.counts != nullptr && c == 0) {   // access statistics (real-time LFU): cold rows read
#pragma unroll
    for (int q = 0; q < ITEMS; ++q)
      if (live[q] && !(HOT && hot[q] >= 0)) atomicAdd(ta.counts + crow[q], 1u);
  }
  const int64_t dm = static_cast<int64_t>(nt) * ta.dim;
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int64_t tok = static_cast<int64_t>(g) * ITEMS + q;
    const int64_t k = static_cast<int64_t>(j) * ta.dim + c * 8;
    if constexpr (OUT == kOutFrag16) {
      // columns 32q + 16h + 8s .. +7 land in lane slot 32h + tok % 32 of
      // fragment (tok / 32, step 2q + s)
      const int64_t ks = (k >> 5) * 2 + ((k >> 3) & 1);
      const int64_t slot = ((tok >> 5) * (dm >> 4) + ks) * 64 + ((k >> 4) & 1) * 32 + (tok & 31);
      store8<IN, ENGRAM_BF16>(e, slot * 8, 0, c, f[q], raw[q], live[q]);
    } else {
      store8<IN, OUT>(e, tok * dm + k, static_cast<int64_t>(n_tok) * dm, c, f[q], raw[q], live[q]);
    }
  }
}

// Items per thread of the hashed gather for n_tok tokens and per_group
// threads per token (tables x 8-element chunks), by the wavefronts one item
// per thread would take: 4 from 16384 wavefronts (8 x 4096 tokens: 26.6 ->
// 23.0 us, and 44.1 -> 32.6 us with the hot tier, against 1 item), 2 from
// 4096 (4096 tokens: about 7.0 -> 6.6 us inside the layer, where 4 items gave
// 6.8-7.8 us), 1 below, so that small launches still spread over the CUs.
inline int gather_items(int64_t n_tok, int64_t per_group) {
  const int64_t waves1 = (n_tok * per_group + 63) / 64;
  return waves1 >= 16384 ? 4 : (waves1 >= 4096 ? 2 : 1);
}

}  // namespace engram
