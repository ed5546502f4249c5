// Step 5 of "DeepSeek Engram series guide", section "Engram working
// principle" (v = W_V e, k^(m) = W_K^(m) e, stacked as the multi-branch
// variant suggests), fused with the reductions that Step 6's gate needs, so
// that the keys never leave the matrix cores' accumulators:
//   v tiles  -> v (float32) and per-token partial sums of v^2,
//   k tiles  -> per-token partial sums of h^2, k^2 and h.k over the tile's
//               columns (h read from H here, before anything writes H).
// The conv kernel adds up the partials of each token (a fixed number of
// tiles, so the result is deterministic) to form alpha and RMSNorm(alpha v).
//
// gfx950 bf16 matrix cores: v_mfma_f32_32x32x16_bf16 (measured on MI355X at
// about 1.4x the sustained rate of the 16x16x32 form), float32 accumulation.
// The weight rows are the MFMA A operand and the token rows of e the B
// operand: each lane then holds four runs of 4 consecutive features of one
// token, so v stores are 16-byte vectors and h loads 8-byte vectors.
// Workgroup tile: TF features x 256 tokens (TF = 128, or 256 when there are
// enough tiles to give every CU two) with eight wavefronts (two per SIMD, so
// one wavefront's matrix work overlaps another's LDS traffic); K advances 64
// per step through double-buffered LDS with the 16-byte chunk c of row r
// stored at chunk c ^ ((r >> 1) & 7).  Slices go from memory straight into
// LDS (global_load_lds_dwordx4, one slice in flight while the other buffer
// is multiplied; ragged token rows re-read the last valid row); an MXFP8
// slice is 128 codes per row, the same 128 bytes, and its per-row scale
// words follow with 4-byte direct loads.  The epilogue stages a key tile's h rows and a value tile's v
// through LDS, so that both move as whole rows.  Tiles are ordered XCD by XCD
// (workgroup i runs on XCD i % 8) with the feature tile fastest, so the
// workgroups that read the same e rows share an L2.
#include <algorithm>
#include <atomic>

#include "device_util.h"
#include "engram_internal.h"
#include "hash_device.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16-byte staging type: a native vector (HIP's uint4 struct copies through memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
// The same, as one vector shuffle (the halves can land in place).
__device__ __forceinline__ i32x8_t cat16(u32x4_t lo, u32x4_t hi) {
  return __builtin_bit_cast(i32x8_t, static_cast<u32x8_t>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
}

// Two 16-byte chunks as the 32-byte MXFP8 operand of one lane.
__device__ __forceinline__ i32x8_t join16(u32x4_t lo, u32x4_t hi) {
  return i32x8_t{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                 static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

constexpr int TK = 256;        // tokens per workgroup
constexpr int BK = 64;         // K slice
constexpr int WF = 2;          // wavefronts along features (wavefronts along tokens: WT, 4 or 2)
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// Main loop: slices go straight into LDS (global_load_lds_dwordx4), NBUF - 1
// of them in flight while the oldest landed one is multiplied.  With one
// slice in flight (NBUF = 2) the loop waits about as long for each slice as
// it multiplies (matrix cores busy 27 % at 4096 tokens, waves waiting on
// their loads 40 % of their cycles); three buffers (144 KiB of LDS at 128
// columns) keep two slices in flight.
//
// MIXED (single-branch layers): a tile's W rows are TF/2 rows of W_V and the
// same TF/2 rows of W_K, so the feature wavefront wf = 0 holds v and wf = 1
// holds k for the same columns.  Every tile then stores half a tile of v and
// reads half a tile of h, instead of value tiles storing whole v tiles while
// key tiles only read h, and each token's statistics tile carries all four
// sums (h.h, k.k, h.k of the key half, v.v of the value half).
template <int TF, bool MX, int WT, int NBUF, bool MIXED>
__global__ void __launch_bounds__(64 * WF * WT) __attribute__((amdgpu_waves_per_eu(WF * WT / 4, WF * WT / 4)))
proj_gate_kernel(ProjGateArgs a) {
  static_assert(NBUF == 2 || NBUF == 3, "two or three slice buffers");
  constexpr int kThreads = 64 * WF * WT;
  // a K slice is 128 bytes of every row: 64 bf16 values, or 128 MXFP8 codes
  // (four 32-value scale blocks)
  constexpr int ESZ = MX ? 1 : 2;          // bytes per element
  constexpr int BKE = 128 / ESZ;           // elements per K slice
  constexpr int kWChunks = TF * 8;         // 16-byte chunks of a W slice
  constexpr int kEChunks = TK * 8;         // 16-byte chunks of an e slice
  constexpr int NW = kWChunks / kThreads;  // W chunks loaded per thread and slice
  constexpr int NE = kEChunks / kThreads;  // e chunks loaded per thread and slice
  constexpr int I = TF / WF / 32;          // 32-row feature blocks per wavefront
  constexpr int J = TK / WT / 32;          // 32-row token blocks per wavefront
  constexpr int kScaleWaves = (TF + TK) / 64;   // MXFP8: wavefronts that load a slice's scale words
  extern __shared__ u32x4_t lds[];
  u32x4_t* Ws = lds;                     // [NBUF][kWChunks]
  u32x4_t* Es = lds + NBUF * kWChunks;   // [NBUF][kEChunks]
  // MXFP8: the slice's scale bytes, one 32-bit word (4 blocks) per W row, then per e row
  uint32_t* Ss = reinterpret_cast<uint32_t*>(lds + NBUF * (kWChunks + kEChunks));   // [NBUF][TF + TK]

  const int n_tiles = a.tiles_f * a.tiles_t;
  const int L = blockIdx.x;
  const int tile = (n_tiles % kXcds == 0) ? (L % kXcds) * (n_tiles / kXcds) + L / kXcds : L;
  const int tf = tile % a.tiles_f;
  const int tt = tile / a.tiles_f;
  const int d = a.d;
  const int f0 = MIXED ? tf * (TF / 2) : tf * TF;   // first feature (MIXED: first v and k column)
  // W row of LDS row r of this tile's slices, counted from row f0
  auto wrow = [&](int r) { return MIXED && r >= TF / 2 ? r + (d - TF / 2) : r; };
  const int64_t t0 = static_cast<int64_t>(tt) * TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave % WF;
  const int wt = wave / WF;
  const int K = a.K;
  const int ksteps = K / BKE;

  f32x16_t acc[I][J];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const char* wbase = reinterpret_cast<const char*>(a.w) + static_cast<int64_t>(f0) * K * ESZ;
  const char* ebase = reinterpret_cast<const char*>(a.e);
  // bf16: K16 steps, lane half h holds K elements 8h..8h+7 (one chunk).
  // MXFP8: K64 steps; lane r (< 32) holds bytes 0-15 and 32-47 of its row's
  // 64-byte run and the scale of its first 32-value block, lane r + 32 bytes
  // 16-31 and 48-63 and the second block's scale (the layout of
  // v_mfma_scale_f32_32x32x64_f8f6f4, checked by a probe against exact sums).
#define ENGRAM_COMPUTE(buf)                                                                        \
  {                                                                                                \
    __builtin_amdgcn_iglp_opt(0);                                                                  \
    if constexpr (!MX) {                                                                           \
      _Pragma("unroll") for (int ks = 0; ks < BKE / 16; ++ks) {                                    \
        const int kc = ks * 2 + (lane >> 5);                                                       \
        bf16x8_t fa[I], fb[J];                                                                     \
        _Pragma("unroll") for (int i = 0; i < I; ++i) fa[i] = __builtin_bit_cast(                  \
            bf16x8_t, Ws[(buf) * kWChunks + swz(wf * (TF / WF) + i * 32 + (lane & 31), kc)]);      \
        _Pragma("unroll") for (int j = 0; j < J; ++j) fb[j] = __builtin_bit_cast(                  \
            bf16x8_t, Es[(buf) * kEChunks + swz(wt * (TK / WT) + j * 32 + (lane & 31), kc)]);      \
        _Pragma("unroll") for (int i = 0; i < I; ++i) _Pragma("unroll") for (int j = 0; j < J; ++j) \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0); \
      }                                                                                            \
    } else {                                                                                       \
      const int h = lane >> 5;                                                                     \
      _Pragma("unroll") for (int ks = 0; ks < 2; ++ks) {                                           \
        i32x8_t fa[I], fb[J];                                                                      \
        int sa[I], sb[J];                                                                          \
        _Pragma("unroll") for (int i = 0; i < I; ++i) {                                            \
          const int row = wf * (TF / WF) + i * 32 + (lane & 31);                                   \
          fa[i] = join16(Ws[(buf) * kWChunks + swz(row, 4 * ks + h)],                              \
                         Ws[(buf) * kWChunks + swz(row, 4 * ks + 2 + h)]);                         \
          sa[i] = static_cast<int>((Ss[(buf) * (TF + TK) + row] >> (8 * (2 * ks + h))) & 0xffu);    \
        }                                                                                          \
        _Pragma("unroll") for (int j = 0; j < J; ++j) {                                            \
          const int row = wt * (TK / WT) + j * 32 + (lane & 31);                                   \
          fb[j] = join16(Es[(buf) * kEChunks + swz(row, 4 * ks + h)],                              \
                         Es[(buf) * kEChunks + swz(row, 4 * ks + 2 + h)]);                         \
          sb[j] = static_cast<int>((Ss[(buf) * (TF + TK) + TF + row] >> (8 * (2 * ks + h))) & 0xffu); \
        }                                                                                          \
        _Pragma("unroll") for (int i = 0; i < I; ++i) _Pragma("unroll") for (int j = 0; j < J; ++j) \
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, \
                                                                        0, sa[i], 0, sb[j]);       \
      }                                                                                            \
    }                                                                                              \
  }

  {
    // Each wavefront instruction fills 64 consecutive 16-byte LDS slots (8
    // rows of a slice).  Slot s of row r holds chunk s ^ ((r >> 1) & 7), so
    // lane l, landing in slot c = l & 7 of row l >> 3, fetches that chunk
    // (the layout that swz() reads).  Token rows past the end re-read the
    // last row; their results are never stored.
    auto issue = [&](int kt, int buf) {
      const int64_t kb = static_cast<int64_t>(kt) * 128;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const int c = tid + i * kThreads;
        const int r = c >> 3;
        const char* src = wbase + static_cast<int64_t>(wrow(r)) * K * ESZ + kb + (((c & 7) ^ ((r >> 1) & 7)) * 16);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                         (__attribute__((address_space(3))) void*)(Ws + buf * kWChunks + i * kThreads + wave * 64),
                                         16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int c = tid + i * kThreads;
        const int r = c >> 3;
        const int64_t tok = min(t0 + r, a.n_tok - 1);
        const char* src = ebase + tok * K * ESZ + kb + (((c & 7) ^ ((r >> 1) & 7)) * 16);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                         (__attribute__((address_space(3))) void*)(Es + buf * kEChunks + i * kThreads + wave * 64),
                                         16, 0, 0);
      }
      if constexpr (MX) {
        // the slice's scale word of every row (4 blocks of 32 codes): W rows,
        // then e rows, 64 rows per wavefront instruction, one instruction
        // for each of the first (TF + TK) / 64 wavefronts
        static_assert(kScaleWaves * 64 == TF + TK && kScaleWaves <= WF * WT, "one scale instruction per wavefront");
        if (wave < kScaleWaves) {
          const int r = wave * 64 + lane;
          const uint8_t* src = r < TF ? a.w_scale + static_cast<int64_t>(f0 + wrow(r)) * (K / 32) + kt * 4
                                      : a.e_scale + min(t0 + (r - TF), a.n_tok - 1) * (K / 32) + kt * 4;
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                           (__attribute__((address_space(3))) void*)(Ss + buf * (TF + TK) + wave * 64),
                                           4, 0, 0);
        }
      }
    };
    // Wait until this wavefront's loads of slice kt have landed while the
    // younger slices stay in flight (vmcnt counts this wavefront's loads:
    // NW + NE per slice, one more for the scale words of an MXFP8 slice).
    auto wait_slice = [&](int younger) {
      if constexpr (NBUF == 3) {
        if (younger > 0) {
          if (MX && wave < kScaleWaves)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NW + NE + 1) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NW + NE) : "memory");
          return;
        }
      }
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    if constexpr (NBUF == 2) {
      // one slice in flight (the form the compiler allocates best for two
      // buffers: 210 rather than 256 VGPRs at 256 columns)
      issue(0, 0);
      for (int kt0 = 0; kt0 < ksteps; kt0 += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kt = kt0 + u;
          if (kt < ksteps) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (kt + 1 < ksteps) issue(kt + 1, u ^ 1);
            ENGRAM_COMPUTE(u);
          }
        }
      }
    } else {
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p)
      if (p < ksteps) issue(p, p);
    // unrolled by NBUF so that the buffer indices are constants
    for (int kt0 = 0; kt0 < ksteps; kt0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int kt = kt0 + u;
        if (kt < ksteps) {
          // this lane's loads of slice kt have landed and its fragment reads
          // of slice kt - 1 have returned; after the barrier, every lane's
          // have.  (A fence in place of the bare barrier would do the same,
          // but the compiler then also waits for all outstanding loads.)
          wait_slice(min(NBUF - 2, ksteps - 1 - kt));
          // into the buffer of slice kt - 1, which every wavefront has read
          if (kt + NBUF - 1 < ksteps) issue(kt + NBUF - 1, (u + NBUF - 1) % NBUF);
          ENGRAM_COMPUTE(u);
        }
      }
    }
    }
    // the epilogue reuses the LDS: all fragment reads done, no load in flight
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
#undef ENGRAM_COMPUTE

  // ---- epilogue: acc[i][j][4g + r] is feature wf*TF/WF + i*32 + g*8 + (lane>>5)*4 + r
  // of the tile's LDS rows, token wt*TK/WT + j*32 + (lane & 31) ----
  // value or key columns: per wavefront (MIXED) or per tile
  const bool is_v = MIXED ? wf == 0 : f0 < d;
  const int m = MIXED ? 0 : (is_v ? 0 : f0 / d - 1);
  // the main loop's LDS is free now: a value wavefront turns its v block
  // around in a private region, a key tile (or key wavefront) holds its h
  // rows; the per-token partials go after them
  float4* red = reinterpret_cast<float4*>(lds + TK * TF / 8);   // [TK][WF] partials of the feature wavefronts
  // first column of this wavefront's block: within v, or within branch m's h
  const int fcol = MIXED ? f0 : (is_v ? f0 + wf * (TF / WF) : f0 - (1 + m) * d);
  if (is_v) {
    // Each wavefront turns its 32-token x TF/WF-feature block of v around in
    // a private LDS region ([32][VC] 16-byte chunks, chunk c of row r at
    // c ^ (r & 15), so that both the accumulator-layout writes and the row
    // reads spread over all banks) and stores whole rows: half a wavefront
    // writes 4*TF/WF contiguous bytes of one token.
    constexpr int VC = TF / WF / 4;                      // 16-byte chunks per row of the block
    float4* Vs = reinterpret_cast<float4*>(lds) + wave * 32 * VC;
    float* vrow0 = a.v + t0 * d + fcol;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = lane & 31;
      const int tl = wt * (TK / WT) + j * 32 + r;
      float s3 = 0.f;
#pragma unroll
      for (int i = 0; i < I; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float x0 = acc[i][j][4 * g], x1 = acc[i][j][4 * g + 1];
          const float x2 = acc[i][j][4 * g + 2], x3 = acc[i][j][4 * g + 3];
          // features i*32 + g*8 + (lane>>5)*4 .. +3 of the block: chunk i*8 + g*2 + (lane>>5)
          Vs[r * VC + ((i * 8 + g * 2 + (lane >> 5)) ^ (r & 15))] = make_float4(x0, x1, x2, x3);
          s3 += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
        }
      }
      s3 += __shfl_xor(s3, 32, 64);
      if ((lane >> 5) == 0) red[tl * WF + wf] = make_float4(0.f, 0.f, 0.f, s3);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wavefront's block is in LDS
      // every LDS read first, then the (ragged-guarded) stores: a read inside
      // each guarded store would go out and be waited for one at a time
      // (native vectors: an array of HIP's float4 structs stays in scratch)
      constexpr int NIT = 32 * VC / 64;
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      f32x4_t xs[NIT];
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int u = it * 64 + lane;
        const int rr = u / VC, c = u % VC;
        xs[it] = reinterpret_cast<const f32x4_t*>(Vs)[rr * VC + (c ^ (rr & 15))];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next block's writes
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int u = it * 64 + lane;
        const int rr = u / VC, c = u % VC;
        const int64_t trow = wt * (TK / WT) + j * 32 + rr;
        if (t0 + trow < a.n_tok) *reinterpret_cast<f32x4_t*>(vrow0 + trow * d + c * 4) = xs[it];
      }
    }
  } else {
    // The h values of this block go into LDS with 16-byte direct loads, a
    // wavefront instruction covering whole row runs; the chunks of a row are
    // rotated by its row number, so that the reads below (32 rows, one
    // chunk each) spread over the banks.  MIXED: each key wavefront loads its own
    // TK/WT tokens x TF/2 columns into a private region and waits for its
    // own loads only; otherwise the workgroup loads the tile's [TK][TF] h
    // rows together (chunk c of row r in slot c ^ (r & HSW), HSW < HC).
    // Token rows past the end re-read the last valid row.
    // Sum k^2 meanwhile.
    constexpr int HC = MIXED ? TF / 16 : TF / 8;                // 16-byte chunks per staged h row
    constexpr int HROWS = MIXED ? TK / WT : TK;                 // rows staged by one loader
    constexpr int HLOADERS = MIXED ? 64 : kThreads;             // threads sharing the loads
    constexpr int NH = HROWS * HC / HLOADERS;                   // loads per thread
    constexpr int HSW = HC < 16 ? HC - 1 : 15;                  // row bits in the chunk swizzle (< HC)
    static_assert(NH * HLOADERS == HROWS * HC && (HC & (HC - 1)) == 0, "whole loads, power-of-two rows");
    u32x4_t* Hs = MIXED ? lds + wave * (HROWS * HC) : lds;
    const int hl_tid = MIXED ? lane : tid;
    const int64_t hrow0 = MIXED ? t0 + wt * (TK / WT) : t0;
#pragma unroll
    for (int q = 0; q < NH; ++q) {
      const int u = q * HLOADERS + hl_tid;   // LDS slot this lane fills (64 consecutive per instruction)
      const int r = u / HC, sl = u % HC;
      const int64_t tok = min(hrow0 + r, a.n_tok - 1);
      const uint16_t* src = a.H + (tok * a.M + m) * d + fcol + (sl ^ (r & HSW)) * 8;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(Hs + q * HLOADERS + (MIXED ? 0 : wave * 64)),
                                       16, 0, 0);
    }
    float s1[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      s1[j] = 0.f;
#pragma unroll
      for (int i = 0; i < I; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          s1[j] += acc[i][j][4 * g] * acc[i][j][4 * g] + acc[i][j][4 * g + 1] * acc[i][j][4 * g + 1] +
                   acc[i][j][4 * g + 2] * acc[i][j][4 * g + 2] + acc[i][j][4 * g + 3] * acc[i][j][4 * g + 3];
    }
    if constexpr (MIXED)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");              // this wavefront's own h block
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");   // every wavefront's part of the tile
    const uint2* Hs2 = reinterpret_cast<const uint2*>(Hs);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int tl = wt * (TK / WT) + j * 32 + (lane & 31);
      const int hr = MIXED ? j * 32 + (lane & 31) : tl;    // row in the staged h block
      float s0 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < I; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // features i*32 + g*8 + (lane>>5)*4 .. +3 of the block: half (lane>>5) of one chunk
          const int c = (MIXED ? 0 : wf * (TF / WF) / 8) + i * 4 + g;
          const uint2 q = Hs2[(hr * HC + (c ^ (hr & HSW))) * 2 + (lane >> 5)];
          const float x0 = acc[i][j][4 * g], x1 = acc[i][j][4 * g + 1];
          const float x2 = acc[i][j][4 * g + 2], x3 = acc[i][j][4 * g + 3];
          const float h0 = __uint_as_float(q.x << 16), h1 = __uint_as_float(q.x & 0xffff0000u);
          const float h2 = __uint_as_float(q.y << 16), h3 = __uint_as_float(q.y & 0xffff0000u);
          s0 += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
          s2 += h0 * x0 + h1 * x1 + h2 * x2 + h3 * x3;
        }
      }
      float s1j = s1[j];
      s0 += __shfl_xor(s0, 32, 64);
      s1j += __shfl_xor(s1j, 32, 64);
      s2 += __shfl_xor(s2, 32, 64);
      if ((lane >> 5) == 0) red[tl * WF + wf] = make_float4(s0, s1j, s2, 0.f);
    }
  }
  // the partials are in LDS; the v stores need not have landed (a full
  // __syncthreads would also wait for them)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  for (int tl = tid; tl < TK; tl += kThreads) {
    const int64_t tok = t0 + tl;
    if (tok < a.n_tok) {
      float4 p = red[tl * WF];
#pragma unroll
      for (int w = 1; w < WF; ++w) {
        const float4 q = red[tl * WF + w];
        p = make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
      }
      a.stats[tok * a.tiles_f + tf] = p;
    }
  }
  advance_state(a, blockIdx.x);
}

// Small batches (decode): a 64-feature x 32-token tile per workgroup, so that
// a few hundred tokens still give hundreds of workgroups.  The four
// wavefronts split K four ways.  Each stages its operands for four K16 steps
// (a 128-byte run of every W and e row) in a private pair of LDS buffers with
// 16-byte direct loads, a wavefront instruction covering 8 whole runs, the
// next batch in flight while the current one is multiplied; the MFMA
// fragments are read from LDS.  (Loading fragments straight from memory, each
// load instruction touches 32 rows at 32 bytes apiece, and the kernel took
// twice as long.)  Only the wavefront itself writes and reads its buffers, so
// the loop needs memory-counter waits but no barrier.  The partial tiles are
// summed through LDS and the epilogue (v store, gate sums per 64 columns)
// follows the large kernel's.
constexpr int kSmallTF = 64;
constexpr int kSmallTK = 32;
constexpr int kSmallWaves = 4;
constexpr int kSmallBatch = 4;   // K16 steps per load batch

// one wavefront's staging buffer: 64 W rows and STK (32, or 64 for the
// float32-output launch of two layers) e rows of a batch's 128-byte run,
// chunk c of row r at slot c ^ (r & 7)
template <int STK>
constexpr int small_rows() { return kSmallTF + STK; }
// (MXFP8: the 128-byte run is 128 codes, and the rows' scale words of the
// batch follow, 128 words, re-reading a valid row past the last)
template <bool MX, int STK = kSmallTK>
constexpr int small_stage() { return small_rows<STK>() * 8 + (MX ? 128 / 4 : 0); }   // 16-byte slots per buffer
template <bool MX, int STK = kSmallTK>
constexpr int small_lds_bytes() { return kSmallWaves * 2 * small_stage<MX, STK>() * 16; }   // staging bytes (reused for the partial sums)

template <bool MX, int STK = kSmallTK>
__device__ __forceinline__ void proj_gate_small_body(const ProjGateArgs& a, uint32_t bid) {
  static_assert(STK == kSmallTK || STK == 2 * kSmallTK, "32 or 64 tokens per tile");
  constexpr int kSmallRows = small_rows<STK>();
  constexpr int JB = STK / 32;                 // 32-token blocks of the tile
  constexpr int kSmallStage = small_stage<MX, STK>();
  extern __shared__ u32x4_t small_lds_buf[];
  u32x4_t* small_lds = small_lds_buf;
  // after the main loop: the partial tiles, +1 column so that the sums are conflict free
  auto part = reinterpret_cast<float (*)[kSmallTF][STK + 1]>(small_lds);
  static_assert(kSmallWaves * kSmallTF * (STK + 1) * 4 <= small_lds_bytes<MX, STK>(), "partial sums fit the staging LDS");
  const int tf = bid % a.tiles_f;
  const int tt = bid / a.tiles_f;
  const int f0 = tf * kSmallTF;
  const int64_t t0 = static_cast<int64_t>(tt) * STK;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = a.K;
  const int kq = K / kSmallWaves;             // this wavefront's K range: [wave*kq, (wave+1)*kq)
  // bf16: K16 steps (K a multiple of 64: at least one), 4 per batch; MXFP8:
  // K64 steps, 2 per batch (K a multiple of 512: whole batches only)
  const int nsteps = MX ? kq / 64 : kq / 16;
  const int half = lane >> 5;                 // lanes 32-63 hold the second half of each step's run

  // epilogue thread (token tl, feature eighth fq; the 8 threads of a token are
  // consecutive lanes, so that v stores and h loads move whole row runs): a
  // key tile's 8 h values are loaded now, alongside the first operand batch
  const int tl = threadIdx.x >> 3;
  const int fq = threadIdx.x & 7;             // 8 features each
  const int64_t gt = t0 + tl;
  const bool valid = gt < a.n_tok;
  const int64_t ct = valid ? gt : a.n_tok - 1;
  const int d = a.d;
  const bool is_v = f0 < d;
  const int m = is_v ? 0 : f0 / d - 1;
  const int c0 = (is_v ? f0 : f0 - (1 + m) * d) + fq * 8;
  uint4 hq = make_uint4(0u, 0u, 0u, 0u);
  if (!is_v && a.kv_out == nullptr) hq = *reinterpret_cast<const uint4*>(a.H + (ct * a.M + m) * d + c0);

  f32x16_t acc0[JB], acc1[JB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[jb][r] = acc1[jb][r] = 0.f;

  // Batch b covers K elements [b*64, b*64 + 64) of this wavefront's range:
  // 12 instructions, 8 rows each (lane l: row 8i + (l >> 3), slot l & 7,
  // which fetches chunk (l & 7) ^ (row & 7)).  Chunks past the range (K/4 not
  // a multiple of 64) re-read the range's last chunk and are never used.
  u32x4_t* stg = small_lds + wave * 2 * kSmallStage;
  constexpr int ESZ = MX ? 1 : 2;             // bytes per element
  constexpr int SPB = MX ? 2 : kSmallBatch;   // steps per batch (a 128-byte run)
  const char* wbase = reinterpret_cast<const char*>(a.w) + (static_cast<int64_t>(f0) * K + wave * kq) * ESZ;
  const char* ebase = reinterpret_cast<const char*>(a.e) + static_cast<int64_t>(wave) * kq * ESZ;
  const int nb = (nsteps + SPB - 1) / SPB;
  auto issue = [&](int b, int buf) {
#pragma unroll
    for (int i = 0; i < kSmallRows / 8; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ (r & 7);
      const int kb = min(b * 128 + ch * 16, kq * ESZ - 16);   // byte offset in the range
      const int64_t row = r < kSmallTF ? static_cast<int64_t>(r) : min(t0 + (r - kSmallTF), a.n_tok - 1);
      const char* src = (r < kSmallTF ? wbase : ebase) + row * K * ESZ + kb;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(stg + buf * kSmallStage + i * 64),
                                       16, 0, 0);
    }
    if constexpr (MX) {
      // the batch's scale word of every row (blocks 4b .. 4b+3 of the range)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(i * 64 + lane, kSmallRows - 1);
        const int64_t col = (static_cast<int64_t>(wave) * kq) / 32 + b * 4;
        const uint8_t* src = r < kSmallTF ? a.w_scale + static_cast<int64_t>(f0 + r) * (K / 32) + col
                                          : a.e_scale + min(t0 + (r - kSmallTF), a.n_tok - 1) * (K / 32) + col;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                         (__attribute__((address_space(3))) void*)(reinterpret_cast<uint32_t*>(
                                             stg + buf * kSmallStage + kSmallRows * 8) + i * 64),
                                         4, 0, 0);
      }
    }
  };
  issue(0, 0);
  for (int b0 = 0; b0 < nb; b0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int b = b0 + u;
      if (b < nb) {
        // this wavefront's fragment reads of buffer u ^ 1 (batch b - 1) are done
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (b + 1 < nb) {
          issue(b + 1, u ^ 1);
          // batch b has landed, b + 1 (a load per 8 rows, two more for the
          // scale words) in flight
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kSmallRows / 8 + (MX ? 2 : 0)) : "memory");
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const u32x4_t* sb = stg + u * kSmallStage;
        const int r = lane & 31;
        if constexpr (!MX) {
#pragma unroll
          for (int j = 0; j < kSmallBatch; ++j) {
            if (b * kSmallBatch + j < nsteps) {
              const int c = 2 * j + half;          // this lane's chunk of the run
              const bf16x8_t fa0 = __builtin_bit_cast(bf16x8_t, sb[r * 8 + (c ^ (r & 7))]);
              const bf16x8_t fa1 = __builtin_bit_cast(bf16x8_t, sb[(32 + r) * 8 + (c ^ (r & 7))]);
#pragma unroll
              for (int jb = 0; jb < JB; ++jb) {
                const int er = kSmallTF + jb * 32 + r;
                const bf16x8_t fb = __builtin_bit_cast(bf16x8_t, sb[er * 8 + (c ^ (er & 7))]);
                acc0[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0, fb, acc0[jb], 0, 0, 0);
                acc1[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1, fb, acc1[jb], 0, 0, 0);
              }
            }
          }
        } else {
          // K64 step ks: lane r holds bytes 0-15 and 32-47 of its row's 64-byte
          // run and block 2ks's scale, lane r + 32 bytes 16-31 and 48-63 and
          // block 2ks+1's (the large kernel's MXFP8 operand layout)
          const uint32_t* sw = reinterpret_cast<const uint32_t*>(sb + kSmallRows * 8);
          const uint32_t wa0 = sw[r], wa1 = sw[32 + r];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int c0c = 4 * ks + half, c1c = 4 * ks + 2 + half;
            const i32x8_t fa0 = join16(sb[r * 8 + (c0c ^ (r & 7))], sb[r * 8 + (c1c ^ (r & 7))]);
            const i32x8_t fa1 = join16(sb[(32 + r) * 8 + (c0c ^ (r & 7))], sb[(32 + r) * 8 + (c1c ^ (r & 7))]);
            const int sh = 8 * (2 * ks + half);
            const int sa0 = static_cast<int>((wa0 >> sh) & 0xffu), sa1 = static_cast<int>((wa1 >> sh) & 0xffu);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
              const int er = kSmallTF + jb * 32 + r;
              const i32x8_t fb = join16(sb[er * 8 + (c0c ^ (er & 7))], sb[er * 8 + (c1c ^ (er & 7))]);
              const int sbb = static_cast<int>((sw[er] >> sh) & 0xffu);
              acc0[jb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa0, fb, acc0[jb], 0, 0, 0, sa0, 0, sbb);
              acc1[jb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa1, fb, acc1[jb], 0, 0, 0, sa1, 0, sbb);
            }
          }
        }
      }
    }
  }
  // every wavefront's fragment reads are done before the partial sums reuse the LDS
  __syncthreads();

  // acc_i[jb][4g + r]: feature i*32 + g*8 + half*4 + r of the tile, token jb*32 + (lane & 31)
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        part[wave][g * 8 + half * 4 + r][jb * 32 + (lane & 31)] = acc0[jb][4 * g + r];
        part[wave][32 + g * 8 + half * 4 + r][jb * 32 + (lane & 31)] = acc1[jb][4 * g + r];
      }
  __syncthreads();

  if constexpr (JB == 2) {
    // the float32 product only (engram_project_ahead): two tokens per thread
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int tk = tl + 32 * tp;
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sacc = 0.f;
#pragma unroll
        for (int w = 0; w < kSmallWaves; ++w) sacc += part[w][fq * 8 + i][tk];
        y[i] = sacc;
      }
      if (t0 + tk < a.n_tok) {
        float4* kp = reinterpret_cast<float4*>(a.kv_out + (t0 + tk) * a.N + f0 + fq * 8);
        kp[0] = make_float4(y[0], y[1], y[2], y[3]);
        kp[1] = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
    advance_state(a, bid);
    return;
  }

  // thread (token tl, feature eighth fq): 8 features of one token, summed over the waves
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float sacc = 0.f;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) sacc += part[w][fq * 8 + i][tl];
    x[i] = sacc;
  }
  if (a.kv_out != nullptr) {
    // the product's columns f0 + fq*8 .. +7 of this token, as they are
    if (valid) {
      float4* kp = reinterpret_cast<float4*>(a.kv_out + gt * a.N + f0 + fq * 8);
      kp[0] = make_float4(x[0], x[1], x[2], x[3]);
      kp[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    advance_state(a, bid);
    return;
  }
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if (is_v) {
    if (valid) {
      float4* vp = reinterpret_cast<float4*>(a.v + gt * d + c0);
      vp[0] = make_float4(x[0], x[1], x[2], x[3]);
      vp[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s3 += x[i] * x[i];
  } else {
    const uint32_t hw[4] = {hq.x, hq.y, hq.z, hq.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float h = __uint_as_float(i & 1 ? (hw[i >> 1] & 0xffff0000u) : (hw[i >> 1] << 16));
      s0 += h * h;
      s1 += x[i] * x[i];
      s2 += h * x[i];
    }
  }
  // the 8 feature groups of a token are lanes 8k .. 8k+7 of one wavefront
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    s0 += __shfl_xor(s0, off, 64);
    s1 += __shfl_xor(s1, off, 64);
    s2 += __shfl_xor(s2, off, 64);
    s3 += __shfl_xor(s3, off, 64);
  }
  if (fq == 0 && valid) a.stats[gt * a.tiles_f + tf] = make_float4(s0, s1, s2, s3);
  advance_state(a, bid);
}

template <bool MX>
__global__ void __launch_bounds__(64 * kSmallWaves)
proj_gate_small_kernel(ProjGateArgs a) {
  proj_gate_small_body<MX>(a, blockIdx.x);
}

// Two layers' small-batch products in one launch: workgroups below split
// serve a, the rest b (each layer's first workgroup advances its decode
// state).
template <bool MX, int STK>
__global__ void __launch_bounds__(64 * kSmallWaves)
proj_gate_small2_kernel(ProjGateArgs a, ProjGateArgs b, uint32_t split) {
  if (blockIdx.x < split)
    proj_gate_small_body<MX, STK>(a, blockIdx.x);
  else
    proj_gate_small_body<MX, STK>(b, blockIdx.x - split);
}

// Many tokens of a multi-branch FP8 product, with W in fragment order
// (engram_pack_mxfp8): a workgroup keeps the e codes of 128 tokens resident
// in LDS for the whole launch (128 KiB at K = 1024) and sweeps the feature
// columns in passes of 256, one 32-column block per wavefront.  A
// wavefront's W operand comes straight from memory into registers, two
// coalesced 16-byte loads per K64 step, kResDepth steps ahead and across pass
// boundaries, so the main loop has no barrier at all; the four token blocks
// of its 32 x 128 output tile reuse each W operand four times.  Per
// multiply-accumulate the L2-to-CU traffic is then W's alone, 1/128 byte,
// against 3/256 for the 128 x 256 tiles that stream both operands.  A key
// pass loads its h values into registers before its K loop, so their latency
// hides behind the matrix work; the per-token partial sums of each 128-column
// statistics tile (four wavefronts) meet in LDS at the end of the pass.
constexpr int kResTK = 128;                // tokens per workgroup, resident in LDS
constexpr int kResWaves = 8;               // wavefront w: 32 features x 128 tokens
constexpr int kResPass = 32 * kResWaves;   // features per pass
constexpr int kResDepth = 4;               // K64 W operands in flight per wavefront
constexpr int kVmcnt0 = 0x0f70;            // s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt unbounded

// LDS: e codes [K/16][128] 16-byte chunks, e scale words [K/128][128], and
// a pass's partial sums: per statistics tile and 64-column half, the first
// wavefront's per-lane sums [4][64] and the per-token sums [128]
constexpr int kResRed = 2 * 2 * 4 * 64 + 2 * 2 * kResTK;   // float4 slots
size_t res_lds_bytes(int K) {
  return static_cast<size_t>(kResTK) * K + static_cast<size_t>(kResTK) * (K / 32) +
         static_cast<size_t>(kResRed) * sizeof(float4);
}

template <int KK>   // K64 steps: K = 64 * KK, a multiple of 256 up to 1024
__global__ void __launch_bounds__(64 * kResWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
proj_gate_mx_resident_kernel(ProjGateArgs a) {
  static_assert(KK % 4 == 0 && KK <= 16, "K a multiple of 256 up to 1024");
  extern __shared__ u32x4_t res_lds[];
  constexpr int K = KK * 64;
  constexpr int nch = K / 16;   // 16-byte chunks of an e row
  u32x4_t* Ec = res_lds;                                                // chunk c of token t at c * 128 + t
  uint32_t* Es = reinterpret_cast<uint32_t*>(res_lds + nch * kResTK);   // scale word w of token t at w * 128 + t
  float4* red = reinterpret_cast<float4*>(Es + (K / 128) * kResTK);     // kResRed partial sums

  const int groups = static_cast<int>(gridDim.x) / a.tiles_t;   // workgroups sharing a token tile
  const int tt = blockIdx.x / groups;
  const int grp = blockIdx.x % groups;
  const int passes = a.N / kResPass;
  const int p0 = grp * passes / groups, p1 = (grp + 1) * passes / groups;
  const int64_t t0 = static_cast<int64_t>(tt) * kResTK;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int r = lane & 31;
  const int d = a.d;

  // e codes and scale words of the tile: one wavefront instruction fills 64
  // consecutive LDS slots, chunk c (or word w) of 64 consecutive tokens;
  // token rows past the end re-read the last valid row
  {
    const uint8_t* ecodes = reinterpret_cast<const uint8_t*>(a.e);
    for (int q = wave; q < 2 * nch; q += kResWaves) {
      const int c = q >> 1;
      const int64_t tok = min(t0 + ((q & 1) << 6) + lane, a.n_tok - 1);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ecodes + tok * K + c * 16),
                                       (__attribute__((address_space(3))) void*)(Ec + c * kResTK + (q & 1) * 64),
                                       16, 0, 0);
    }
    for (int q = wave; q < 2 * (K / 128); q += kResWaves) {
      const int w = q >> 1;
      const int64_t tok = min(t0 + ((q & 1) << 6) + lane, a.n_tok - 1);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.e_scale + tok * (K / 32) + 4 * w),
                                       (__attribute__((address_space(3))) void*)(Es + w * kResTK + (q & 1) * 64),
                                       4, 0, 0);
    }
  }

  // Pass order: the eight XCDs start at passes np/8 apart, so that the
  // chip's h loads (key passes) and v stores (value passes) do not all fall
  // on HBM at once; the workgroups of one XCD keep one order and share W in
  // their L2.
  const int np = p1 - p0;
  const int off = ((blockIdx.x & (kXcds - 1)) * np) / kXcds;
  auto pass_at = [&](int i) { return p0 + (i + off) % np; };

  // this wavefront's W operands: (block b, step kk) is lane slot
  // (b*KK + kk)*64 + lane, its scale word (b*KK/4 + kk/4)*64 + lane; the
  // wavefront's block of pass p is p*8 + wave.  kResDepth steps are in
  // flight, the first ones of the next pass while a pass ends (after the
  // last pass the loads repeat the last block's first steps, unused).  Each
  // ring slot is refilled right after the multiplies that read it, and the
  // e operands of a step are read one step ahead, two register sets in turn.
  const i32x8_t* wop = reinterpret_cast<const i32x8_t*>(a.w_packed);
  const uint32_t* wword = reinterpret_cast<const uint32_t*>(a.w_packed + static_cast<int64_t>(a.N) * K);
  i32x8_t wring[kResDepth];
  {
    const int64_t slot0 = static_cast<int64_t>(pass_at(0) * kResWaves + wave) * KK * 64;
#pragma unroll
    for (int u = 0; u < kResDepth; ++u) wring[u] = wop[slot0 + u * 64 + lane];   // KK >= kResDepth
  }
  uint32_t wsc_next = wword[static_cast<int64_t>(pass_at(0) * kResWaves + wave) * (KK / 4) * 64 + lane];
  // the e tile has landed (every wavefront's part); a wait the compiler
  // sees, so that it counts the operand loads after it exactly
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __builtin_amdgcn_s_barrier();

  auto read_e = [&](int kk, i32x8_t (&fb)[4], int (&sb)[4]) {
    // (the lane index through an empty asm, so that the addresses are formed
    // where they are used: hoisted out of the pass loop, they stay live
    // across it and spill)
    int rr = r;
    asm volatile("" : "+v"(rr));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tr = j * 32 + rr;
      fb[j] = cat16(Ec[(4 * kk + hh) * kResTK + tr], Ec[(4 * kk + 2 + hh) * kResTK + tr]);
      sb[j] = static_cast<int>((Es[(kk >> 1) * kResTK + tr] >> (8 * (2 * (kk & 1) + hh))) & 0xffu);
    }
  };
  i32x8_t fbA[4], fbB[4];
  int sbA[4], sbB[4];
  read_e(0, fbA, sbA);

  // A key pass's 16 h loads per lane are spread over its first kHSteps
  // steps, each after that step's operand loads.  The memory counter
  // retires loads in order, so a wait for an operand load also waits for
  // every load issued before it: an h load issued at step s is waited for
  // at step s + kResDepth + 1 at the latest, and the whole set arrives by the
  // epilogue, instead of the first operand wait of the pass waiting for all
  // of them.
  constexpr int kHSteps = KK < 8 ? KK : 8;
  constexpr int kHPerStep = 8 / kHSteps;
  for (int i = 0; i < np; ++i) {
    const int p = pass_at(i);
    const int fp = p * kResPass;
    const bool is_v = fp < d;
    const int m = is_v ? 0 : fp / d - 1;
    const int fcol = (is_v ? fp : fp - (1 + m) * d) + wave * 32;   // this block's first column of v or of h
    // A key block's h values.  Lane half hh loads columns 16hh .. 16hh+15
    // of its token's 32 (two 16-byte loads, half as many instructions as
    // the accumulator layout's 8-byte pieces), and the epilogue trades half
    // of them with the partner lane (v_permlane32_swap) to reach that
    // layout.  The loads are unconditional (a branch around them inside the
    // unrolled loop costs registers); a value pass reads the first 64 bytes
    // of H instead, unused.  Byte offsets of H fit 32 bits (checked by the
    // launcher).
    u32x4_t hA[4], hB[4];
    uint32_t hoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      hoff[j] = static_cast<uint32_t>(hh * 32) +
                (is_v ? 0u : static_cast<uint32_t>(((min(t0 + j * 32 + r, a.n_tok - 1) * a.M + m) * d + fcol) * 2));
    f32x16_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[j][c] = 0.f;

    const int64_t blk = static_cast<int64_t>(p) * kResWaves + wave;
    const int64_t nblk = i + 1 < np ? static_cast<int64_t>(pass_at(i + 1)) * kResWaves + wave : blk;
    // the whole K loop of a pass unrolled: every wait on an operand load is
    // then counted exactly (through a loop back-edge the compiler waits for
    // all loads)
#pragma unroll
    for (int kk0 = 0; kk0 < KK; kk0 += kResDepth) {
      const uint32_t wsc = wsc_next;   // scale bytes of this group of four steps
      // where the operands kResDepth steps ahead come from: later steps of
      // this block, or the first steps of the next pass's block
      const bool in_pass = kk0 + kResDepth < KK;
      // (uniform bases; the lane offset is added per load)
      const i32x8_t* tslot = wop + (in_pass ? blk * KK + kk0 + kResDepth : nblk * KK) * 64;
      const uint32_t* tword = wword + (in_pass ? blk * (KK / 4) + kk0 / 4 + 1 : nblk * (KK / 4)) * 64;
      const int kn = in_pass ? kk0 + kResDepth : 0;   // the step after this group
#pragma unroll
      for (int u = 0; u < kResDepth; ++u) {
        const int kk = kk0 + u;
        const int sa = static_cast<int>((wsc >> (8 * u)) & 0xffu);
        i32x8_t (&fc)[4] = (u & 1) ? fbB : fbA;   // this step's e operands
        int (&sc)[4] = (u & 1) ? sbB : sbA;
        i32x8_t (&fn)[4] = (u & 1) ? fbA : fbB;   // the next step's
        int (&sn)[4] = (u & 1) ? sbA : sbB;
        read_e(u + 1 < kResDepth ? kk + 1 : kn, fn, sn);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wring[u], fc[j], acc[j], 0, 0, 0, sa, 0, sc[j]);
        __builtin_amdgcn_sched_barrier(0);
        wring[u] = tslot[u * 64 + lane];
        if (u == 0) wsc_next = tword[lane];
        if (kk < kHSteps) {
#pragma unroll
          for (int c = 0; c < kHPerStep; ++c) {
            const int idx = kk * kHPerStep + c;
            const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(a.H) +
                                                                 hoff[idx >> 1] + (idx & 1) * 16);
            if (idx & 1)
              hB[idx >> 1] = hv;
            else
              hA[idx >> 1] = hv;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // epilogue: acc[j][4g + i] is feature g*8 + hh*4 + i of the block, token
    // j*32 + r.  The gate sums of each 128-column statistics tile are formed
    // in exactly the order of the 128 x 256 tile kernel (whose wavefront
    // holds 64 columns): the first 32-column wavefront of each 64-column
    // half leaves its per-lane running sums in LDS, the second continues
    // them and halves them across the lane halves, and the two halves are
    // added last.  The results are then identical bit for bit.
    const int qd = wave >> 2;          // 128-column statistics tile of the pass
    const int half64 = (wave >> 1) & 1;   // 64-column half of the tile
    const bool first = (wave & 1) == 0;   // first 32-column block of the half
    float4* lane_part = red + ((qd * 2 + half64) * 4) * 64;   // [4 token blocks][64 lanes]
    float4* tok_part = red + 2 * 2 * 4 * 64 + (qd * 2 + half64) * kResTK;   // [128 tokens]
    // the previous pass's partial sums have been read (LDS only: the operand
    // loads in flight stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // h in the accumulator layout: after the swaps (in place), lane (hh, r)
    // holds columns g*8 + hh*4 .. +3 in hA[j].xy (g = 0), hB[j].xy (g = 1),
    // hA[j].zw (g = 2) and hB[j].zw (g = 3)
    if (!is_v) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto a0 = __builtin_amdgcn_permlane32_swap(hA[j].x, hA[j].z, false, false);
        const auto a1 = __builtin_amdgcn_permlane32_swap(hA[j].y, hA[j].w, false, false);
        const auto b0 = __builtin_amdgcn_permlane32_swap(hB[j].x, hB[j].z, false, false);
        const auto b1 = __builtin_amdgcn_permlane32_swap(hB[j].y, hB[j].w, false, false);
        hA[j] = u32x4_t{a0[0], a1[0], a0[1], a1[1]};
        hB[j] = u32x4_t{b0[0], b1[0], b0[1], b1[1]};
      }
    }
    auto hq = [&](int j, int g) {
      const u32x4_t& v = (g & 1) ? hB[j] : hA[j];
      return g < 2 ? make_uint2(v.x, v.y) : make_uint2(v.z, v.w);
    };
    float4 part[4];
    if (is_v) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = t0 + j * 32 + r;
        float s3 = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
          if (tok < a.n_tok) *reinterpret_cast<float4*>(a.v + tok * d + fcol + g * 8 + hh * 4) = make_float4(x0, x1, x2, x3);
        }
        if (first) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            s3 += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          }
        }
        part[j] = make_float4(0.f, 0.f, 0.f, s3);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s0 = 0.f, s1 = 0.f, s2 = 0.f;
        if (first) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            s1 += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint2 q = hq(j, g);
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            const float h0 = __uint_as_float(q.x << 16), h1 = __uint_as_float(q.x & 0xffff0000u);
            const float h2 = __uint_as_float(q.y << 16), h3 = __uint_as_float(q.y & 0xffff0000u);
            s0 += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
            s2 += h0 * x0 + h1 * x1 + h2 * x2 + h3 * x3;
          }
        }
        part[j] = make_float4(s0, s1, s2, 0.f);
      }
    }
    if (first) {
#pragma unroll
      for (int j = 0; j < 4; ++j) lane_part[j * 64 + lane] = part[j];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (!first) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 c = lane_part[j * 64 + lane];
        float s0 = c.x, s1 = c.y, s2 = c.z, s3 = c.w;
        if (is_v) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            s3 += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          }
          s3 += __shfl_xor(s3, 32, 64);
          if (hh == 0) tok_part[j * 32 + r] = make_float4(0.f, 0.f, 0.f, s3);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            s1 += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint2 q = hq(j, g);
            const float x0 = acc[j][4 * g], x1 = acc[j][4 * g + 1], x2 = acc[j][4 * g + 2], x3 = acc[j][4 * g + 3];
            const float h0 = __uint_as_float(q.x << 16), h1 = __uint_as_float(q.x & 0xffff0000u);
            const float h2 = __uint_as_float(q.y << 16), h3 = __uint_as_float(q.y & 0xffff0000u);
            s0 += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
            s2 += h0 * x0 + h1 * x1 + h2 * x2 + h3 * x3;
          }
          s0 += __shfl_xor(s0, 32, 64);
          s1 += __shfl_xor(s1, 32, 64);
          s2 += __shfl_xor(s2, 32, 64);
          if (hh == 0) tok_part[j * 32 + r] = make_float4(s0, s1, s2, 0.f);
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tid < 2 * kResTK) {
      const int q2 = tid >> 7, t = tid & (kResTK - 1);
      const int64_t tok = t0 + t;
      if (tok < a.n_tok) {
        const float4* tp = red + 2 * 2 * 4 * 64 + q2 * 2 * kResTK;
        const float4 x = tp[t], y = tp[kResTK + t];
        a.stats[tok * a.tiles_f + p * 2 + q2] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
      }
    }
    // Drain this pass's stores here.  The memory counter mixes loads and
    // stores, which do not finish in order, so with stores in flight every
    // later wait on an operand load would be a wait for all memory work,
    // the next pass's h loads included.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
  }
  advance_state(a, blockIdx.x);
}

// Workgroups per token tile for the resident-token FP8 kernel, or 0 where it
// does not apply: multi-branch layers (whose statistics tiles are plain
// 128-column ones), d a multiple of 256, K a multiple of 256 up to 1024 (the
// e tile in LDS), H below 4 GiB, and enough token tiles that at most
// passes / 4 workgroups per tile fill the 256 CUs.
int res_groups(int64_t n_tok, int N, int d, int K, int M) {
  if (M < 2 || d % kResPass != 0 || N % kResPass != 0 || K % 256 != 0 || K > 1024) return 0;
  if (n_tok * M * d * 2 > int64_t{0xffffffff}) return 0;   // byte offsets of H in 32 bits
  const int64_t tiles_t = (n_tok + kResTK - 1) / kResTK;
  const int passes = N / kResPass;
  for (int g = 1; g <= passes / 4; ++g)
    if (tiles_t * g >= 256) return g;
  return 0;
}

template <int KK>
hipError_t launch_resident_k(const ProjGateArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  static std::atomic<uint64_t> attr_set{0};   // > 64 KiB of dynamic LDS, raised once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(proj_gate_mx_resident_kernel<KK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  launch_k(proj_gate_mx_resident_kernel<KK>, grid, dim3(64 * kResWaves), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_resident(const ProjGateArgs& in, int groups, hipStream_t s) {
  ProjGateArgs a = in;
  a.tiles_f = a.N / 128;
  a.tiles_t = static_cast<int>((a.n_tok + kResTK - 1) / kResTK);
  const size_t lds = res_lds_bytes(a.K);
  const dim3 grid(static_cast<unsigned>(a.tiles_t * groups));
  switch (a.K) {
    case 256: return launch_resident_k<4>(a, grid, lds, s);
    case 512: return launch_resident_k<8>(a, grid, lds, s);
    case 768: return launch_resident_k<12>(a, grid, lds, s);
    case 1024: return launch_resident_k<16>(a, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

template <int TF, bool MX, int NBUF, bool MIXED, int WT = 4>
hipError_t launch_tf(ProjGateArgs a, hipStream_t s) {
  a.tiles_f = a.N / TF;
  a.tiles_t = static_cast<int>((a.n_tok + TK - 1) / TK);
  // main loop: NBUF slices (and MXFP8 scale words); epilogue: the h tile and
  // the per-token partials
  const size_t lds = std::max(static_cast<size_t>(NBUF * (TF + TK) * 8) * sizeof(u32x4_t) +
                                  (MX ? static_cast<size_t>(NBUF * (TF + TK)) * sizeof(uint32_t) : 0),
                              static_cast<size_t>(TK * TF) * 2 + static_cast<size_t>(TK * WF) * sizeof(float4));
  static_assert(NBUF * (TF + TK) * 8 * 16 + (MX ? NBUF * (TF + TK) * 4 : 0) <= 160 * 1024, "fits gfx950's LDS");
  // more than 64 KiB of dynamic LDS exceeds the default per-workgroup limit;
  // raise it once per device and instantiation (gfx950 has 160 KiB per CU)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(proj_gate_kernel<TF, MX, WT, NBUF, MIXED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  launch_k((proj_gate_kernel<TF, MX, WT, NBUF, MIXED>), dim3(a.tiles_f * a.tiles_t), dim3(64 * WF * WT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Few tokens: the small kernel (64-column statistics tiles); otherwise the
// large one with 256-column tiles when there are enough of them.  The MXFP8
// product always takes the large kernel with 128-column tiles.
//
// The small kernel's time grows with tokens x features; the large one costs
// about the same (its K loop's latency) until its tiles fill the chip.
// Measured on gfx950 at K = 1024 (small / large, us): N = 2048, 768 tokens
// 14.4 / 17.5 and 1,024 tokens 18.3 / 17.7; N = 5120, 256 tokens 13.3 / 16.8
// and 384 tokens 17.7 / 17.3.  The two meet near 1.9 M token-features.
//
// The small kernel's statistics come in 64-column tiles, 2d/64 per token and
// branch (one value tile set and one key tile set); the conv takes at most
// kConvMaxStats of them per row, so the small kernel serves d <= 2048 only.
bool proj_gate_small(int64_t n_tok, int N, int d) {
  return 2 * d / kSmallTF <= kConvMaxStats && n_tok * static_cast<int64_t>(N) <= (int64_t{7} << 18);
}

// The FP8 product takes the small kernel only with whole 128-code batches per
// wavefront (K a multiple of 512), and only up to 3 * 2^19 token-features: its
// large kernel is faster than the bf16 one (12.3-13.5 us from 256 to 2,048
// tokens at N = 2048), so the two meet earlier (small / large at K = 1024:
// N = 2048, 768 tokens 12.4 / 12.8 us, 1,024 tokens 16.2 / 12.7; N = 5120,
// 256 tokens 11.3 / 12.3, 384 tokens 14.9 / 12.7).
bool proj_gate_small_for(int64_t n_tok, int N, int d, int K, bool mx) {
  if (!mx) return proj_gate_small(n_tok, N, d);
  return 2 * d / kSmallTF <= kConvMaxStats && K % 512 == 0 && n_tok * static_cast<int64_t>(N) <= (int64_t{3} << 19);
}

// The statistics layout of the launch that launch_proj_gate makes.  The
// large kernel on a single-branch layer pairs value and key columns in each
// tile (MIXED), so that every token's statistics tile holds all four sums.
ProjGateLayout proj_gate_layout(int64_t n_tok, int N, int d, int K, int M, bool mx) {
  ProjGateLayout l;
  l.tf = proj_gate_tile_f(n_tok, N, d, K, mx);
  l.small = l.tf == kSmallTF;
  l.mixed = !l.small && M == 1;
  l.qv = l.mixed ? 2 * d / l.tf : d / l.tf;
  l.qk = l.mixed ? 0 : d / l.tf;
  return l;
}

int proj_gate_tile_f(int64_t n_tok, int N, int d, int K, bool mx) {
  if (proj_gate_small_for(n_tok, N, d, K, mx)) return kSmallTF;
  if (mx) return 128;
  // 256-feature tiles halve the LDS traffic per matrix operation but need at
  // least two tiles per CU (512) to keep the chip busy
  const int64_t tiles256 = ((n_tok + TK - 1) / TK) * (N / 256);
  return (d % 256 == 0 && tiles256 >= 512) ? 256 : 128;
}

template <bool MX>
hipError_t launch_small(const ProjGateArgs& in, hipStream_t s) {
  ProjGateArgs a = in;
  a.tiles_f = a.N / kSmallTF;
  a.tiles_t = static_cast<int>((a.n_tok + kSmallTK - 1) / kSmallTK);
  static std::atomic<uint64_t> attr_set{0};   // > 64 KiB of dynamic LDS, raised once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(proj_gate_small_kernel<MX>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, small_lds_bytes<MX>());
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  launch_k(proj_gate_small_kernel<MX>, dim3(static_cast<unsigned>(a.tiles_f * a.tiles_t)), dim3(64 * kSmallWaves),
           small_lds_bytes<MX>(), s, a);
  return hipGetLastError();
}

// a and b shaped for STK-token tiles (tiles_t counted in STK)
template <bool MX, int STK>
hipError_t launch_small2(const ProjGateArgs& a, const ProjGateArgs& b, hipStream_t s) {
  static std::atomic<uint64_t> attr_set{0};   // > 64 KiB of dynamic LDS, raised once per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(proj_gate_small2_kernel<MX, STK>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, small_lds_bytes<MX, STK>());
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  const uint32_t na = static_cast<uint32_t>(a.tiles_f * a.tiles_t), nb = static_cast<uint32_t>(b.tiles_f * b.tiles_t);
  launch_k((proj_gate_small2_kernel<MX, STK>), dim3(na + nb), dim3(64 * kSmallWaves), small_lds_bytes<MX, STK>(), s,
           a, b, na);
  return hipGetLastError();
}

hipError_t launch_project_layers(const ProjGateArgs& in_a, const ProjGateArgs* in_b, hipStream_t s) {
  if (in_a.w_frag != nullptr) return launch_project_frag(in_a, in_b, s);
  if (in_b != nullptr && in_b->w_frag != nullptr) return hipErrorNotSupported;
  const bool mx = in_a.e_scale != nullptr;
  auto fits = [&](const ProjGateArgs& x) {
    return x.kv_out != nullptr && (x.e_scale != nullptr) == mx && x.N % kSmallTF == 0 &&
           x.K % (mx ? 512 : BK) == 0 && proj_gate_small_for(x.n_tok, x.N, x.d, x.K, mx);
  };
  if (!fits(in_a) || (in_b != nullptr && !fits(*in_b))) return hipErrorNotSupported;
  auto shaped = [](const ProjGateArgs& x, int tk) {
    ProjGateArgs y = x;
    y.tiles_f = y.N / kSmallTF;
    y.tiles_t = static_cast<int>((y.n_tok + tk - 1) / tk);
    return y;
  };
  if (in_b == nullptr || in_b->n_tok == 0 || in_a.n_tok == 0) {
    const ProjGateArgs a = shaped(in_a.n_tok == 0 && in_b != nullptr ? *in_b : in_a, kSmallTK);
    if (a.n_tok == 0) return hipSuccess;
    return mx ? launch_small<true>(a, s) : launch_small<false>(a, s);
  }
  // Two layers: 64-token tiles while the two layers' tiles still fill the
  // chip once (one workgroup of 128 KiB of LDS per CU), so that the launch
  // runs in one round; otherwise the single layer's 32-token tiles.
  const int64_t wg64 = shaped(in_a, 2 * kSmallTK).tiles_f * static_cast<int64_t>(shaped(in_a, 2 * kSmallTK).tiles_t) +
                       shaped(*in_b, 2 * kSmallTK).tiles_f * static_cast<int64_t>(shaped(*in_b, 2 * kSmallTK).tiles_t);
  if (wg64 <= 256) {
    const ProjGateArgs a = shaped(in_a, 2 * kSmallTK), b = shaped(*in_b, 2 * kSmallTK);
    return mx ? launch_small2<true, 2 * kSmallTK>(a, b, s) : launch_small2<false, 2 * kSmallTK>(a, b, s);
  }
  const ProjGateArgs a = shaped(in_a, kSmallTK), b = shaped(*in_b, kSmallTK);
  return mx ? launch_small2<true, kSmallTK>(a, b, s) : launch_small2<false, kSmallTK>(a, b, s);
}

hipError_t launch_proj_gate(const ProjGateArgs& in, hipStream_t s) {
  if (in.n_tok == 0) return hipSuccess;
  if (in.N % 128 != 0) return hipErrorInvalidValue;
  const bool mx = in.e_scale != nullptr;
  if (mx) {
    if (in.K % 128 != 0 || in.w_scale == nullptr) return hipErrorInvalidValue;
    if (proj_gate_small_for(in.n_tok, in.N, in.d, in.K, true)) return launch_small<true>(in, s);
    if (in.w_packed != nullptr) {
      const int g = res_groups(in.n_tok, in.N, in.d, in.K, in.M);
      if (g > 0) return launch_resident(in, g, s);
    }
    // 128-feature tiles, slices straight into LDS like the bf16 product
    // (the 256-feature tile's accumulators and FP8 operands spill registers)
    return in.M == 1 ? launch_tf<128, true, 3, true>(in, s) : launch_tf<128, true, 3, false>(in, s);
  }
  if (in.K % BK != 0) return hipErrorInvalidValue;
  if (proj_gate_small(in.n_tok, in.N, in.d)) return launch_small<false>(in, s);
  if (proj_gate_tile_f(in.n_tok, in.N, in.d, in.K, false) == 256)
    return in.M == 1 ? launch_tf<256, false, 2, true>(in, s) : launch_tf<256, false, 2, false>(in, s);
  return in.M == 1 ? launch_tf<128, false, 3, true>(in, s) : launch_tf<128, false, 3, false>(in, s);
}

}  // namespace engram
