// Steps 1-5 of decode-size batches ahead of the hidden states ("DeepSeek
// Engram series guide", section "Engram working principle": Steps 1-4 and
// the products v = W_V e, k^(m) = W_K^(m) e of Step 5 read only the token ids
// and the decode history), into float32 rows of [v | k].
//
// At a few hundred tokens the product is a chain of memory latencies, not a
// bandwidth or matrix-core problem, so both kernels here are built to wait
// on memory as few times as possible:
//   proj_frag2_kernel   both operands in the matrix cores' fragment order (W
//                       from launch_bf16_pack, e from the gather's
//                       kGatherOutFrag16 output): every operand is one
//                       coalesced 1 KiB load straight into registers, all of
//                       a wavefront's loads are issued before its first
//                       matrix operation, and nothing is staged in LDS.
//   ahead_fused_kernel  the same product whose wavefronts hash their tokens
//                       and read their own table rows (Steps 1-4) instead of
//                       loading gathered rows: the gather's launch and its
//                       round trip through memory go, the W loads overlap the
//                       id -> hash -> row chain, and int8 rows are dequantised
//                       in registers (the select-and-dequantise-in-one-kernel
//                       design of the DRAM offload study, "Engram embedding
//                       extension: co-design for efficient DRAM/SSD offload",
//                       decode section).
// A workgroup's 64 x 64 output tile (64 x 32 in small fused launches) is
// split over its 8 wavefronts along K (K/8 each); the 8 partial tiles meet in
// LDS (128 or 64 KiB) at the end.  Tiles run feature tile fastest, so the
// token tiles that share a W tile share the workgroup index modulo 8, and so
// an XCD and its L2.
//
// The K order inside the matrix operations: lane l = 32h + r of K16 step ks
// takes columns 32(ks/2) + 16h + 8(ks%2) .. +7, so that a lane's two steps of
// a 32-column group read 16 consecutive values of one table row (16 bytes of
// an int8 row); W is packed the same way, so the sum is that of W e in
// another order.
#include <atomic>

#include "device_util.h"
#include "engram_internal.h"
#include "gather_device.h"
#include "hash_device.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFragTile = 64;   // features and tokens per workgroup
constexpr int kFragWaves = 8;
constexpr int kFragLds = kFragWaves * 16 * 64 * 16;   // [wave][16 float4][64 lanes] (64 x 64 tiles)

static_assert(sizeof(AheadJob::Head) == 128, "the head is two scalar loads");

// Arrival counts of the fused launches that advance decode states, one per
// token tile of each layer: zero at load, and put back to zero by the last
// workgroup of each tile.
__device__ uint32_t ahead_arrivals[kAheadSlots];
constexpr int kAheadTiles = 64;   // 32-token tiles per layer that a launch with states may have (2048 sequences)

// The 64 x 32TB tile of the 8 wavefronts' partial products acc (K split 8
// ways): summed through LDS and stored as float32 rows of kv_out.
template <int TB>
__device__ __forceinline__ void frag_epilogue(float* kv_out, int N, int64_t n_tok, int tf, int tt,
                                              f32x16_t (&acc)[2][TB]) {
  extern __shared__ float4 frag_part[];   // [wave][j][lane]
  constexpr int NJ = 2 * TB * 4;           // float4s per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // acc[fb][tb][4g + r]: feature 32fb + 8g + 4(lane / 32) + r, token 32tb + lane % 32
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        frag_part[(wave * NJ + (fb * TB + tb) * 4 + g) * 64 + lane] =
            make_float4(acc[fb][tb][4 * g], acc[fb][tb][4 * g + 1], acc[fb][tb][4 * g + 2], acc[fb][tb][4 * g + 3]);
  __syncthreads();
  if constexpr (TB == 2) {
    // thread (j, r): fragment j's float4s of lanes r and r + 32, i.e. 8
    // consecutive features of one token, summed over the wavefronts
    const int j = threadIdx.x >> 5, r = threadIdx.x & 31;
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
#pragma unroll
    for (int w = 0; w < kFragWaves; ++w) {
      const float4 x = frag_part[(w * NJ + j) * 64 + r], y = frag_part[(w * NJ + j) * 64 + 32 + r];
      lo.x += x.x; lo.y += x.y; lo.z += x.z; lo.w += x.w;
      hi.x += y.x; hi.y += y.y; hi.z += y.z; hi.w += y.w;
    }
    const int fb = j >> 3, tb = (j >> 2) & 1, g = j & 3;
    const int64_t tok = static_cast<int64_t>(tt) * 64 + tb * 32 + r;
    if (tok < n_tok) {
      float4* kp = reinterpret_cast<float4*>(kv_out + tok * N + tf * kFragTile + fb * 32 + g * 8);
      kp[0] = lo;
      kp[1] = hi;
    }
  } else {
    // thread (j, l): fragment j's float4 of lane l (lanes l and l + 32 of a
    // wavefront store one token's 8 consecutive features)
    const int j = threadIdx.x >> 6, l = threadIdx.x & 63;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kFragWaves; ++w) {
      const float4 x = frag_part[(w * NJ + j) * 64 + l];
      sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
    }
    const int fb = j >> 2, g = j & 3;
    const int64_t tok = static_cast<int64_t>(tt) * 32 + (l & 31);
    if (tok < n_tok)
      *reinterpret_cast<float4*>(kv_out + tok * N + tf * kFragTile + fb * 32 + g * 8 + 4 * (l >> 5)) = sum;
  }
}

template <int TB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][TB]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// The wavefront index, known to the compiler as uniform (so that what it
// selects, table arguments and base addresses, stays in scalar registers).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// This wavefront's W operands: K16 steps wave*SPW .. +SPW-1 of the 32-row
// blocks 2tf and 2tf+1 (K = 128 SPW), step by step, so that step s waits
// only for its own.
template <int SPW>
__device__ __forceinline__ void load_w(const uint16_t* w_frag, int tf, u32x4_t (&wa)[2][SPW]) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  constexpr int64_t ks_n = 8 * SPW;   // K / 16
  const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(w_frag) + ((2 * tf) * ks_n + wave * SPW) * 64 + lane;
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    wa[0][st] = wp[st * 64];
    wa[1][st] = wp[(ks_n + st) * 64];
  }
}

template <int SPW>
__device__ __forceinline__ void proj_frag_body(const ProjGateArgs& a, uint32_t bid) {
  const int tf = static_cast<int>(bid % static_cast<uint32_t>(a.tiles_f));
  const int tt = static_cast<int>(bid / static_cast<uint32_t>(a.tiles_f));
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int64_t ks_n = a.K / 16;
  const u32x4_t* ep = reinterpret_cast<const u32x4_t*>(a.e) + ((2 * tt) * ks_n + wave * SPW) * 64 + lane;
  u32x4_t wa[2][SPW], eb[2][SPW];
  load_w<SPW>(a.w_frag, tf, wa);
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    eb[0][st] = ep[st * 64];
    eb[1][st] = ep[(ks_n + st) * 64];
  }
  // keep the scheduler from sinking the loads next to their first use
  __builtin_amdgcn_sched_barrier(0);
  f32x16_t acc[2][2];
  zero_acc<2>(acc);
#pragma unroll
  for (int st = 0; st < SPW; ++st)
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wa[fb][st]),
                                                              __builtin_bit_cast(bf16x8_t, eb[tb][st]), acc[fb][tb],
                                                              0, 0, 0);
  frag_epilogue<2>(a.kv_out, a.N, a.n_tok, tf, tt, acc);
  advance_state(a, bid);
}

// One or two layers (workgroups below split serve a, the rest b).
template <int SPW>
__global__ void __launch_bounds__(64 * kFragWaves)
proj_frag2_kernel(ProjGateArgs a, ProjGateArgs b, uint32_t split) {
  if (blockIdx.x < split)
    proj_frag_body<SPW>(a, blockIdx.x);
  else
    proj_frag_body<SPW>(b, blockIdx.x - split);
}

// Row values of the fused kernel: a lane's 16 consecutive values of a
// 32-column group, as loaded (int8 codes with the row's scale, or bf16).
template <int IN>
struct RowRun;
template <>
struct RowRun<ENGRAM_I8> {
  u32x4_t q;
  float s;
};
template <>
struct RowRun<ENGRAM_BF16> {
  u32x4_t lo, hi;
};

// The bf16 operand of half `s` (values 8s .. 8s+7) of a run: int8 codes are
// dequantised as the gather does (one float32 multiply by the row's scale,
// then round to nearest even bf16), bf16 values pass as they are.
template <int IN>
__device__ __forceinline__ u32x4_t run_operand(const RowRun<IN>& v, int s) {
  if constexpr (IN == ENGRAM_I8) {
    const uint32_t w0 = s == 0 ? v.q[0] : v.q[2], w1 = s == 0 ? v.q[1] : v.q[3];
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = static_cast<float>(static_cast<int8_t>((w0 >> (8 * i)) & 0xffu)) * v.s;
      f[4 + i] = static_cast<float>(static_cast<int8_t>((w1 >> (8 * i)) & 0xffu)) * v.s;
    }
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return o;
  } else {
    return s == 0 ? v.lo : v.hi;
  }
}

// Steps 1-5 of one workgroup tile (64 features x 32TB tokens) of one layer;
// tables of dim 32 GPT.
template <int IN, int SPW, bool HIST_ALL, int GPT, int TB>
__device__ __forceinline__ void ahead_fused_body(const AheadJob& J, int tf, int tt) {
  constexpr int NG = SPW / 2;   // 32-column groups per wavefront
  constexpr int DIM = 32 * GPT;
  static_assert(NG % GPT == 0 || GPT > NG, "a wavefront's groups start at a table boundary, or lie in one table");
  const AheadJob::Head hd = J.head;
  const TableArgs& ta = J.g.ta;
  const HashSrc& hs = J.g.hs;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int h = lane >> 5, r = lane & 31;

  // The hash constants and row offsets of this wavefront's tables.
  constexpr int NT = GPT > NG ? 1 : NG / GPT;   // tables per wavefront
  TableHash th[NT];
  int64_t row_off[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int j = (32 * NG * wave) / DIM + u;
    th[u] = table_hash(hs.a, j);
    row_off[u] = ta.row_offset[j];
  }
  // These and the head are read in one batch of scalar loads and one wait:
  // the asm statements take them all as operands, so every load is issued
  // before them.  Left to itself the compiler issues each argument read
  // where its value is first needed and waits for it there, one memory
  // round trip each (several, in a chain, before the first id load).
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(hd.tokens), "s"(hd.proj), "s"(hd.hist), "s"(hd.w_frag), "s"(hd.rows), "s"(hd.scale),
               "s"(hd.kv_out), "s"(hd.st_ids), "s"(hd.st_pos));
  asm volatile("" ::"s"(hd.T), "s"(hd.max_n), "s"(hd.vocab), "s"(hd.n_tok), "s"(hd.N), "s"(hd.tiles_f),
               "s"(hd.has_state), "s"(hd.slot));
  const uint32_t slot = hd.slot;
  const WindowSrc win{hd.tokens, hd.proj, hd.hist, hd.err, hd.T, hd.max_n, hd.vocab};
#pragma unroll
  for (int u = 0; u < NT; ++u)
    asm volatile("" ::"s"(th[u].m[0]), "s"(th[u].m[1]), "s"(th[u].m[2]), "s"(th[u].m[3]), "s"(th[u].inv),
                 "s"(th[u].prime), "s"(row_off[u]));

  // Steps 1-2: the suffix window of this lane's own token: 64tt + 32h + r
  // (TB = 2: the lane pair (r, 32 + r) holds the tile's tokens r and 32 + r
  // between them) or 32tt + r (TB = 1: both lanes of the pair hold token r).
  // Tokens past the end take the last one's; their columns are not stored.
  const uint32_t n_tok = static_cast<uint32_t>(hd.n_tok);
  const uint32_t T = static_cast<uint32_t>(hd.T);
  uint32_t b[1], t[1];
  {
    const uint32_t tok = static_cast<uint32_t>(tt) * (32 * TB) + (TB == 2 ? 32 * h : 0) + r;
    const uint32_t tc = tok < n_tok ? tok : n_tok - 1;
    b[0] = tc / T;
    t[0] = tc - b[0] * T;
  }
  uint32_t xp[1][ENGRAM_MAX_ORDER], hv[1][ENGRAM_MAX_ORDER];
  window_loads<1, HIST_ALL>(win, b, t, xp, hv);
  // With decode states: this workgroup's history reads are done once every
  // wavefront holds hv (the asm makes each wait for it, which costs nothing
  // here: the history returned before the token ids the P lookups needed),
  // so the arrival is counted now and its round trip overlaps the rest; the
  // count is relaxed, as the reads have all returned and it orders nothing
  // but the arrivals themselves.
  uint32_t arrived_before;   // thread 0's count (the other lanes never read it)
  if (hd.has_state) {
    asm volatile("" ::"v"(hv[0][1]), "v"(hv[0][2]), "v"(hv[0][3]) : "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      arrived_before = __hip_atomic_fetch_add(&ahead_arrivals[slot + tt], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  }
  // W after the P lookups: its loads then stream in behind the P and row
  // latencies, and (memory reads retiring in order) waiting for the P values
  // does not wait for W
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t wa[2][SPW];
  load_w<SPW>(hd.w_frag, tf, wa);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t x[1][ENGRAM_MAX_ORDER];
  window_select<1>(t, xp, hv, x);

  // Steps 3-4: this wavefront's groups are columns 32(NG wave + q) .. +31,
  // in table j at column c0 (uniform over the wavefront); lane half h reads
  // the group's values 16h .. 16h+15 of the tile's token rows.  A table's
  // index is hashed once per lane pair and token and traded between the two
  // lanes (v_permlane32_swap), and so (below) the int8 row's scale: TB = 2,
  // each lane hashes its own token for every table; TB = 1, lane half h
  // hashes the token for every other table, from table h.
  RowRun<IN> run[TB][NG];
  float s_own[NG];
  int32_t z_tb[TB][NT];
  if constexpr (TB == 2) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int32_t z = hash_of_ids(x[0], th[u]);
      if constexpr (kDebugChecks) debug_record(hs.a.err, range_bit(z, th[u].prime, kErrRow));   // z < p by construction
      const auto sw = __builtin_amdgcn_permlane32_swap(z, z, false, false);
      const int32_t zp = h ? static_cast<int32_t>(sw[0]) : static_cast<int32_t>(sw[1]);   // the pair lane's
      z_tb[0][u] = h ? zp : z;
      z_tb[TB - 1][u] = h ? z : zp;
      if constexpr (IN == ENGRAM_I8) s_own[u] = hd.scale[row_off[u] + z];
    }
  } else if constexpr (NT == 1) {
    const int32_t z = hash_of_ids(x[0], th[0]);
    if constexpr (kDebugChecks) debug_record(hs.a.err, range_bit(z, th[0].prime, kErrRow));
    z_tb[0][0] = z;
    if constexpr (IN == ENGRAM_I8) s_own[0] = hd.scale[row_off[0] + z];
  } else {
#pragma unroll
    for (int p = 0; p < NT / 2; ++p) {
      TableHash tm = th[2 * p];   // table 2p + h
#pragma unroll
      for (int i = 0; i < ENGRAM_MAX_ORDER; ++i) tm.m[i] = h ? th[2 * p + 1].m[i] : th[2 * p].m[i];
      tm.inv = h ? th[2 * p + 1].inv : th[2 * p].inv;
      tm.prime = h ? th[2 * p + 1].prime : th[2 * p].prime;
      const int32_t z = hash_of_ids(x[0], tm);
      if constexpr (kDebugChecks) debug_record(hs.a.err, range_bit(z, tm.prime, kErrRow));
      const auto sw = __builtin_amdgcn_permlane32_swap(z, z, false, false);
      const int32_t zp = h ? static_cast<int32_t>(sw[0]) : static_cast<int32_t>(sw[1]);   // the pair lane's
      z_tb[0][2 * p] = h ? zp : z;
      z_tb[0][2 * p + 1] = h ? z : zp;
      if constexpr (IN == ENGRAM_I8) s_own[p] = hd.scale[(h ? row_off[2 * p + 1] : row_off[2 * p]) + z];
    }
  }
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    const int k0 = 32 * (NG * wave + q);
    const int j = k0 / DIM;
    const int col = k0 - j * DIM + 16 * h;
    const int u = GPT > NG ? 0 : q / GPT;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t row = row_off[u] + z_tb[tb][u];
      if constexpr (IN == ENGRAM_I8) {
        run[tb][q].q = *reinterpret_cast<const u32x4_t*>(static_cast<const int8_t*>(hd.rows) + row * DIM + col);
      } else {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(hd.rows) + row * DIM + col);
        run[tb][q].lo = p[0];
        run[tb][q].hi = p[1];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (IN == ENGRAM_I8) {
    float sc[TB][NT];
    if constexpr (TB == 2 || NT > 1) {
#pragma unroll
      for (int p = 0; p < (TB == 2 ? NT : NT / 2); ++p) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s_own[p]), __float_as_uint(s_own[p]), false,
                                                          false);
        const float sp = __uint_as_float(h ? sw[0] : sw[1]);
        if constexpr (TB == 2) {
          sc[0][p] = h ? sp : s_own[p];
          sc[TB - 1][p] = h ? s_own[p] : sp;
        } else {
          sc[0][2 * p] = h ? sp : s_own[p];
          sc[0][2 * p + 1] = h ? s_own[p] : sp;
        }
      }
    } else {
      sc[0][0] = s_own[0];
    }
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) run[tb][q].s = sc[tb][GPT > NG ? 0 : q / GPT];
  }

  // Step 5
  f32x16_t acc[2][TB];
  zero_acc<TB>(acc);
#pragma unroll
  for (int st = 0; st < SPW; ++st) {
    u32x4_t eb[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) eb[tb] = run_operand<IN>(run[tb][st >> 1], st & 1);
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[fb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wa[fb][st]),
                                                              __builtin_bit_cast(bf16x8_t, eb[tb]), acc[fb][tb],
                                                              0, 0, 0);
  }
  frag_epilogue<TB>(hd.kv_out, hd.N, hd.n_tok, tf, tt, acc);

  // The decode state (T = 1: token tok is sequence tok) may only advance
  // once every workgroup of this token tile has read its history: the last
  // of the tile's feature workgroups to arrive writes the new ids, which the
  // lanes of its first wavefront already hold (x, newest first), and clears
  // the count.
  if (hd.has_state && wave == 0) {
    // thread 0 holds the count; its wavefront writes (no barrier needed)
    const bool last = __builtin_amdgcn_readfirstlane(arrived_before) == static_cast<uint32_t>(hd.tiles_f) - 1;
    if (last) {
      if (lane == 0) __hip_atomic_store(&ahead_arrivals[slot + tt], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int hl = hd.max_n - 1;
      const int64_t tok = static_cast<int64_t>(tt) * (32 * TB) + (TB == 2 ? 32 * h : 0) + r;   // this lane's own
      if (tok < hd.n_tok && (TB == 2 || h == 0)) {
#pragma unroll
        for (int i = 0; i < ENGRAM_MAX_ORDER - 1; ++i)
          if (i < hl) hd.st_ids[tok * hl + i] = static_cast<int32_t>(x[0][hl - 1 - i]);
        hd.st_pos[tok] += 1;
      }
    }
  }
}

// HIST_ALL: every token of both layers reads decode history (T <= N-1).
// The grid is (feature tile, token tile, layer), so that a workgroup knows
// its tile and layer before it reads any argument.
template <int IN, int SPW, bool HIST_ALL, int GPT, int TB>
__global__ void __launch_bounds__(64 * kFragWaves)
ahead_fused_kernel(AheadJob a, AheadJob b) {
  if (blockIdx.z == 0)
    ahead_fused_body<IN, SPW, HIST_ALL, GPT, TB>(a, blockIdx.x, blockIdx.y);
  else
    ahead_fused_body<IN, SPW, HIST_ALL, GPT, TB>(b, blockIdx.x, blockIdx.y);
}

// Kernels with more than 64 KiB of dynamic LDS, raised once per device.
hipError_t raise_lds(const void* kernel, std::atomic<uint64_t>& attr_set, int bytes = kFragLds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  return hipSuccess;
}

template <int SPW>
hipError_t launch_frag2(const ProjGateArgs& a, const ProjGateArgs& b, hipStream_t s) {
  static std::atomic<uint64_t> attr_set{0};
  const hipError_t e = raise_lds(reinterpret_cast<const void*>(proj_frag2_kernel<SPW>), attr_set);
  if (e != hipSuccess) return e;
  const uint32_t na = static_cast<uint32_t>(a.tiles_f * a.tiles_t), nb = static_cast<uint32_t>(b.tiles_f * b.tiles_t);
  launch_k((proj_frag2_kernel<SPW>), dim3(na + nb), dim3(64 * kFragWaves), kFragLds, s, a, b, na);
  return hipGetLastError();
}

std::atomic<uint32_t> g_next_slot{0};

template <int IN, int SPW, bool HIST_ALL, int GPT, int TB>
hipError_t launch_fused_t(AheadJob a, AheadJob b, hipStream_t s) {
  static std::atomic<uint64_t> attr_set{0};
  constexpr int lds = kFragWaves * 8 * TB * 64 * 16;   // [wave][8 TB float4][64 lanes]
  const hipError_t e =
      raise_lds(reinterpret_cast<const void*>(ahead_fused_kernel<IN, SPW, HIST_ALL, GPT, TB>), attr_set, lds);
  if (e != hipSuccess) return e;
  const uint32_t nb = static_cast<uint32_t>(b.p.tiles_f * b.p.tiles_t);
  // a block of 2 kAheadTiles counts per launch: a's token tiles, then b's
  const uint32_t slot = (g_next_slot.fetch_add(1) % (kAheadSlots / (2 * kAheadTiles))) * (2 * kAheadTiles);
  a.head.slot = slot;
  b.head.slot = slot + kAheadTiles;
  // a's workgroups, then b's (as many: the two layers have the same tiles);
  // workgroup i runs on XCD i % 8, so with 8 | tiles_f the token tiles of a
  // feature tile share an XCD
  launch_k((ahead_fused_kernel<IN, SPW, HIST_ALL, GPT, TB>),
           dim3(static_cast<unsigned>(a.p.tiles_f), static_cast<unsigned>(a.p.tiles_t), nb > 0 ? 2 : 1),
           dim3(64 * kFragWaves), lds, s, a, b);
  return hipGetLastError();
}

template <int IN, int SPW, bool HIST_ALL, int TB>
hipError_t launch_fused_g(const AheadJob& a, const AheadJob& b, hipStream_t s) {
  switch (a.g.ta.dim) {
    case 32: return launch_fused_t<IN, SPW, HIST_ALL, 1, TB>(a, b, s);
    case 64: return launch_fused_t<IN, SPW, HIST_ALL, 2, TB>(a, b, s);
    default: return launch_fused_t<IN, SPW, HIST_ALL, 4, TB>(a, b, s);
  }
}

template <int IN, bool HIST_ALL, int TB>
hipError_t launch_fused_h(const AheadJob& a, const AheadJob& b, hipStream_t s) {
  return a.p.K == 512 ? launch_fused_g<IN, 4, HIST_ALL, TB>(a, b, s) : launch_fused_g<IN, 8, HIST_ALL, TB>(a, b, s);
}

bool hist_all(const AheadJob& x) { return x.g.hs.hist != nullptr && x.g.hs.T <= x.g.hs.a.max_n - 1; }

template <int IN, int TB>
hipError_t launch_fused_in(const AheadJob& a, const AheadJob& b, bool has_b, hipStream_t s) {
  return hist_all(a) && (!has_b || hist_all(b)) ? launch_fused_h<IN, true, TB>(a, b, s)
                                                : launch_fused_h<IN, false, TB>(a, b, s);
}

ProjGateArgs frag_shaped(const ProjGateArgs& x, int tile_t = kFragTile) {
  ProjGateArgs y = x;
  y.tiles_f = y.N / kFragTile;
  y.tiles_t = static_cast<int>((y.n_tok + tile_t - 1) / tile_t);
  return y;
}

}  // namespace

bool proj_frag_for(int64_t n_tok, int N, int d, int K) {
  return K % 128 == 0 && K <= 1024 && N % kFragTile == 0 && proj_gate_small_for(n_tok, N, d, K, false);
}

bool ahead_fused_for(const TableArgs& ta, int64_t n_tok, int N, int d, int K) {
  return proj_frag_for(n_tok, N, d, K) && (K == 512 || K == 1024) && (ta.dim == 32 || ta.dim == 64 || ta.dim == 128) &&
         (ta.dtype == ENGRAM_I8 || ta.dtype == ENGRAM_BF16) && reinterpret_cast<uintptr_t>(ta.rows) % 16 == 0 &&
         ta.cache_slot == nullptr && ta.counts == nullptr;
}

hipError_t launch_project_frag(const ProjGateArgs& in_a, const ProjGateArgs* in_b, hipStream_t s) {
  auto fits = [&](const ProjGateArgs& x) {
    return x.kv_out != nullptr && x.w_frag != nullptr && x.e_scale == nullptr && x.K == in_a.K &&
           proj_frag_for(x.n_tok, x.N, x.d, x.K);
  };
  if (!fits(in_a) || (in_b != nullptr && !fits(*in_b))) return hipErrorNotSupported;
  const ProjGateArgs a = frag_shaped(in_a);
  ProjGateArgs b = in_b != nullptr ? frag_shaped(*in_b) : ProjGateArgs{};
  if (in_b == nullptr) b.tiles_f = b.tiles_t = 0;
  if (a.tiles_t + b.tiles_t == 0) return hipSuccess;
  switch (a.K / 128) {
    case 1: return launch_frag2<1>(a, b, s);
    case 2: return launch_frag2<2>(a, b, s);
    case 3: return launch_frag2<3>(a, b, s);
    case 4: return launch_frag2<4>(a, b, s);
    case 5: return launch_frag2<5>(a, b, s);
    case 6: return launch_frag2<6>(a, b, s);
    case 7: return launch_frag2<7>(a, b, s);
    default: return launch_frag2<8>(a, b, s);
  }
}

hipError_t launch_ahead_fused(const AheadJob& in_a, const AheadJob* in_b, hipStream_t s) {
  auto fits = [&](const AheadJob& x) {
    return x.p.kv_out != nullptr && x.p.w_frag != nullptr && x.p.e_scale == nullptr && !x.g.hot &&
           x.p.K == in_a.p.K && x.g.ta.dtype == in_a.g.ta.dtype && x.g.ta.dim == in_a.g.ta.dim &&
           x.p.n_tok == x.g.n_tok &&
           x.p.K == x.g.ta.n_tables * x.g.ta.dim && ahead_fused_for(x.g.ta, x.p.n_tok, x.p.N, x.p.d, x.p.K);
  };
  // with decode states (T = 1), at most kAheadTiles 32-token tiles
  auto state_fits = [](const AheadJob& x) {
    return x.p.adv_B <= 0 || (x.p.adv_T == 1 && x.p.adv_B == x.p.n_tok && x.p.n_tok <= int64_t{kAheadTiles} * 32);
  };
  if (!fits(in_a) || (in_b != nullptr && !fits(*in_b))) return hipErrorNotSupported;
  if (!state_fits(in_a) || (in_b != nullptr && !state_fits(*in_b))) return hipErrorNotSupported;
  // 64-token tiles, or 32-token ones (64 KiB of LDS, two workgroups per CU)
  // where 64-token tiles would leave CUs without a workgroup.  (At 256
  // tokens x 2048 columns x 2 layers, 32-token tiles measured 12.7 us against
  // 11.1: each workgroup streams its whole W tile, and per CU that doubles.)
  const int64_t wg64 = (in_a.p.N / kFragTile) * ((in_a.p.n_tok + 63) / 64) * (in_b != nullptr ? 2 : 1);
  const int tile_t = wg64 < 256 ? 32 : 64;
  AheadJob a = in_a, b = in_b != nullptr ? *in_b : AheadJob{};
  auto shape = [tile_t](AheadJob& x) {
    x.p = frag_shaped(x.p, tile_t);
    const HashSrc& hs = x.g.hs;
    AheadJob::Head& hd = x.head;
    hd = AheadJob::Head{};
    hd.tokens = hs.tokens;
    hd.proj = hs.proj;
    hd.hist = hs.hist;
    hd.w_frag = x.p.w_frag;
    hd.rows = x.g.ta.rows;
    hd.scale = x.g.ta.scale;
    hd.kv_out = x.p.kv_out;
    hd.st_ids = x.p.st_ids;
    hd.st_pos = x.p.st_pos;
    hd.err = hs.a.err;
    hd.T = static_cast<int32_t>(hs.T);
    hd.max_n = hs.a.max_n;
    hd.vocab = hs.a.vocab;
    hd.n_tok = static_cast<int32_t>(x.p.n_tok);
    hd.N = x.p.N;
    hd.tiles_f = x.p.tiles_f;
    hd.has_state = x.p.adv_B > 0;
  };
  shape(a);
  if (in_b != nullptr) {
    shape(b);
    if (b.p.tiles_f != a.p.tiles_f || b.p.tiles_t != a.p.tiles_t) return hipErrorNotSupported;
  } else {
    b.p.tiles_f = b.p.tiles_t = 0;
  }
  if (a.p.tiles_t == 0) return hipSuccess;
  const bool has_b = in_b != nullptr;
  if (tile_t == 32)
    return a.g.ta.dtype == ENGRAM_I8 ? launch_fused_in<ENGRAM_I8, 1>(a, b, has_b, s)
                                     : launch_fused_in<ENGRAM_BF16, 1>(a, b, has_b, s);
  return a.g.ta.dtype == ENGRAM_I8 ? launch_fused_in<ENGRAM_I8, 2>(a, b, has_b, s)
                                   : launch_fused_in<ENGRAM_BF16, 2>(a, b, has_b, s);
}

}  // namespace engram
