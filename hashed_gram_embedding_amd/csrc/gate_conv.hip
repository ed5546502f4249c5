// Steps 6-8 of "DeepSeek Engram series guide", section "Engram working
// principle", per branch m of the multi-branch variant:
//   alpha = sigmoid(RMSNorm(h) . RMSNorm(k) / sqrt(d)),  v~ = alpha v
//   u = RMSNorm(v~),  c_t = sum_j w[j] u_{t-(w-1-j)*dilation}   (depthwise, causal)
//   Y = SiLU(c) + v~,  H <- H + Y
//
// The gate needs four sums per (token, branch): h.h, k.k, h.k and v.v.  They
// arrive as partial sums over column tiles ("gate statistics", one float4 per
// token and tile: x = sum h^2, y = sum k^2, z = sum h.k, w = sum v^2) from the
// fused projection kernel, or as whole-row sums from gate_stats_kernel when
// the projections are given.  With RMSNorm(alpha v) = gamma v,
//   gamma = alpha / sqrt(alpha^2 mean(v^2) + eps),
// the conv input u is gamma * v.
//
// conv_kernel: a workgroup owns 32 tokens x 256 channels (fewer when d is not
// a multiple of 256) of one branch of one
// sequence.  It forms alpha and gamma for its rows and the (w-1)*dilation halo
// rows before them, stages v of all those rows in LDS (the halo rows before a
// continued sequence come from the decode state, already as u), then each
// thread produces 4 channels of 8 tokens: the conv taps read LDS, SiLU and the
// residual follow, and H is read and written only at the thread's own
// positions.  All gate inputs were read (by the projection kernel or
// gate_stats_kernel) before this kernel writes H, so the in-place update
// cannot feed another token's gate.
#include "device_util.h"
#include "engram_internal.h"
#include "gather_device.h"

namespace engram {
namespace {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int TT = 32;   // output tokens per conv workgroup

// Channels per conv workgroup: the largest of 256, 128, 64 that divides d.
int conv_channels(int d) { return d % 256 == 0 ? 256 : (d % 128 == 0 ? 128 : 64); }

template <int DT>
__device__ __forceinline__ float4 load4(const void* base, int64_t off) {
  if constexpr (DT == ENGRAM_BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                       __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
  }
}

template <int DT>
__device__ __forceinline__ void store4(void* base, int64_t off, float4 f) {
  if constexpr (DT == ENGRAM_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) =
        make_uint2(pack_bf16x2(f.x, f.y), pack_bf16x2(f.z, f.w));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = f;
  }
}

// CPT (2 or 4) consecutive elements, starting at column col of a row, as
// floats.  The row pointer is uniform across the workgroup and col is 32-bit,
// so the access is a scalar base plus a per-lane 32-bit offset.  Four bf16
// values move as one 8-byte nontemporal access: the strip conv reads and
// rewrites each H row once, and with streaming accesses it ran 10 % faster at
// 4096 tokens (and the next projection, which reads H, about 1 us faster);
// with two values per thread the hint measured no better.
template <int DT, int CPT>
__device__ __forceinline__ void loadc(const void* row, uint32_t col, float (&f)[CPT]) {
  static_assert(CPT == 2 || CPT == 4, "2 or 4 channels per thread");
  if constexpr (DT == ENGRAM_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + col;
    if constexpr (CPT == 4) {
      const u32x2_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
      f[0] = __uint_as_float(q.x << 16);
      f[1] = __uint_as_float(q.x & 0xffff0000u);
      f[2] = __uint_as_float(q.y << 16);
      f[3] = __uint_as_float(q.y & 0xffff0000u);
    } else {
      const uint32_t q = *reinterpret_cast<const uint32_t*>(p);
      f[0] = __uint_as_float(q << 16);
      f[1] = __uint_as_float(q & 0xffff0000u);
    }
  } else {
    const float* p = static_cast<const float*>(row) + col;
    if constexpr (CPT == 4) {
      const float4 q = *reinterpret_cast<const float4*>(p);
      f[0] = q.x; f[1] = q.y; f[2] = q.z; f[3] = q.w;
    } else {
      const float2 q = *reinterpret_cast<const float2*>(p);
      f[0] = q.x; f[1] = q.y;
    }
  }
}

template <int DT, int CPT>
__device__ __forceinline__ void storec(void* row, uint32_t col, const float (&f)[CPT]) {
  if constexpr (DT == ENGRAM_BF16) {
    uint16_t* p = static_cast<uint16_t*>(row) + col;
    if constexpr (CPT == 4)
      __builtin_nontemporal_store(u32x2_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])}, reinterpret_cast<u32x2_t*>(p));
    else
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(f[0], f[1]);
  } else {
    float* p = static_cast<float*>(row) + col;
    if constexpr (CPT == 4)
      *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    else
      *reinterpret_cast<float2*>(p) = make_float2(f[0], f[1]);
  }
}

// Gate statistics from given projections: one wavefront per (token, branch).
// stats[t][0].w = sum v^2 (written by the m = 0 wavefront), stats[t][1+m].xyz.
template <int HT, int KT>
__global__ void __launch_bounds__(256)
gate_stats_kernel(const void* __restrict__ H, const void* __restrict__ kv, int64_t n_tok, int M, int d,
                  float4* __restrict__ stats) {
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= n_tok * M) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = pair / M;
  const int m = static_cast<int>(pair - t * M);
  const int64_t h_off = pair * d;
  const int64_t v_off = t * (1 + M) * d;
  const int64_t k_off = v_off + static_cast<int64_t>(1 + m) * d;
  float shh = 0.f, skk = 0.f, shk = 0.f, svv = 0.f;
#pragma unroll 4
  for (int c = lane * 4; c < d; c += 256) {
    const float4 h = load4<HT>(H, h_off + c);
    const float4 k = load4<KT>(kv, k_off + c);
    const float4 v = load4<KT>(kv, v_off + c);
    shh += h.x * h.x + h.y * h.y + h.z * h.z + h.w * h.w;
    skk += k.x * k.x + k.y * k.y + k.z * k.z + k.w * k.w;
    shk += h.x * k.x + h.y * k.y + h.z * k.z + h.w * k.w;
    svv += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  shh = wave_sum(shh);
  skk = wave_sum(skk);
  shk = wave_sum(shk);
  svv = wave_sum(svv);
  if (lane == 0) {
    stats[t * (1 + M) + 1 + m] = make_float4(shh, skk, shk, 0.f);
    if (m == 0) stats[t * (1 + M)] = make_float4(0.f, 0.f, 0.f, svv);
  }
}

template <int HT, int VT, int CG>
__global__ void __launch_bounds__(256)
conv_kernel(ConvArgs a) {
  constexpr int TPT = TT * CG / 256;  // output tokens per thread
  extern __shared__ float4 lds[];     // [R][CG] staged v (or state u), then [R][qv+qk] statistics
  __shared__ float alpha_s[TT + ENGRAM_MAX_CONV_SPAN];
  __shared__ float scale_s[TT + ENGRAM_MAX_CONV_SPAN];
  const GateConvArgs& g = a.g;
  const int M = g.branches;
  const int d = g.d;
  const int kw = g.kernel_w;
  const int span = (kw - 1) * g.dilation;
  const int R = TT + span;
  const int64_t T = a.T;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TT;
  const int b = blockIdx.y / M;
  const int m = blockIdx.y - b * M;
  const int c_base = blockIdx.z * CG * 4;
  const int tid = threadIdx.x;
  const int32_t pos0 = a.has_state ? a.st.pos[b] : 0;
  float4* tile = lds;
  float4* sstat = lds + R * CG;
  const int nqb = a.qv + a.qk;  // statistics this branch needs per row

  // phase 1: stage v rows (or state u rows) and the rows' gate statistics in
  // LDS.  The loops have fixed trip counts (bounded by the largest halo) and
  // are unrolled, so every load is in flight before the first one is waited on.
  constexpr int kMaxRows = TT + ENGRAM_MAX_CONV_SPAN;
  constexpr int kTileIters = (kMaxRows * CG + 255) / 256;
  constexpr int kStatIters = (kMaxRows * kConvMaxStats + 255) / 256;  // up to kConvMaxStats per row (launch_conv checks)
  const int64_t row0 = static_cast<int64_t>(b) * T;
  {
    // v rows of this chunk: the address is clamped into the chunk (always a
    // valid load) and the value replaced by 0 outside it, so there is no
    // branch around the loads
    float4 val[kTileIters];
#pragma unroll
    for (int n = 0; n < kTileIters; ++n) {
      const int idx = tid + n * 256;
      const int r = idx / CG;
      const int q = idx - r * CG;
      const int64_t t = t0 - span + r;
      const int64_t tc = t < 0 ? 0 : (t >= T ? T - 1 : t);
      val[n] = load4<VT>(a.v, (row0 + tc) * a.v_stride + c_base + q * 4);
    }
#pragma unroll
    for (int n = 0; n < kTileIters; ++n) {
      const int idx = tid + n * 256;
      const int r = idx / CG;
      const int64_t t = t0 - span + r;
      const bool inside = t >= 0 && t < T;
      if (r < R && (inside || !(t < 0 && a.has_state)))
        tile[idx] = inside ? val[n] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if (a.has_state && t0 < span) {
    // rows before the chunk start come from the decode state (already u)
    for (int idx = tid; idx < span * CG; idx += 256) {
      const int r = idx / CG;
      const int q = idx - r * CG;
      const int64_t t = t0 - span + r;
      if (t < 0) {
        int slot = static_cast<int>((static_cast<int64_t>(pos0) + t) % span);
        if (slot < 0) slot += span;
        tile[idx] = *reinterpret_cast<const float4*>(a.st.conv + ((static_cast<int64_t>(b) * M + m) * span + slot) * d +
                                                     c_base + q * 4);
      }
    }
  }
  {
    float4 val[kStatIters];
#pragma unroll
    for (int n = 0; n < kStatIters; ++n) {
      const int idx = tid + n * 256;
      const int r = idx / nqb;
      const int q = idx - r * nqb;
      const int64_t t = t0 - span + r;
      const int64_t tc = t < 0 ? 0 : (t >= T ? T - 1 : t);
      const int qc = q < nqb ? q : 0;
      const int src = qc < a.qv ? qc : a.qv + m * a.qk + (qc - a.qv);
      val[n] = a.stats[(row0 + tc) * a.nq + src];
    }
#pragma unroll
    for (int n = 0; n < kStatIters; ++n) {
      const int idx = tid + n * 256;
      const int r = idx / nqb;
      const int64_t t = t0 - span + r;
      if (idx < R * nqb) sstat[idx] = (t >= 0 && t < T) ? val[n] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();

  // phase 0: alpha and gamma of every staged row
  if (tid < R) {
    const int64_t t = t0 - span + tid;
    float al = 0.f, sc = 0.f;
    if (t >= 0 && t < T) {
      const float4* st = sstat + tid * nqb;
      float svv = 0.f, shh = 0.f, skk = 0.f, shk = 0.f;
      for (int q = 0; q < a.qv; ++q) svv += st[q].w;
      for (int q = a.kq0; q < nqb; ++q) {
        shh += st[q].x;
        skk += st[q].y;
        shk += st[q].z;
      }
      const float inv_d = 1.0f / static_cast<float>(d);
      const float rh = 1.0f / sqrtf(shh * inv_d + g.eps);
      const float rk = 1.0f / sqrtf(skk * inv_d + g.eps);
      const float logit = shk * rh * rk / sqrtf(static_cast<float>(d));
      al = 1.0f / (1.0f + expf(-logit));
      sc = al / sqrtf(al * al * (svv * inv_d) + g.eps);
      if (blockIdx.z == 0 && tid >= span) {
        const int64_t o = (static_cast<int64_t>(b) * T + t) * M + m;
        if (a.alpha_out != nullptr) a.alpha_out[o] = al;
        if (a.gamma_out != nullptr) a.gamma_out[o] = sc;
      }
    } else if (t < 0 && a.has_state) {
      sc = 1.0f;  // the state holds u itself
    }
    alpha_s[tid] = al;
    scale_s[tid] = sc;
  }

  // conv weights of this thread's 4 channels, and its H values (loads issued
  // before the barrier so that they overlap the gate arithmetic)
  const int q = tid % CG;
  const int k0 = tid / CG;
  const int c = c_base + q * 4;
  float wt[4][ENGRAM_MAX_KERNEL_W];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < ENGRAM_MAX_KERNEL_W; ++j)
      wt[i][j] = j < kw ? g.conv_w[(static_cast<int64_t>(m) * d + c + i) * kw + j] : 0.f;
  float4 h[TPT];
#pragma unroll
  for (int n = 0; n < TPT; ++n) {
    // clamped (always valid) address, no branch: positions past the end are
    // loaded but never stored
    int64_t t = t0 + k0 + n * (256 / CG);
    t = t < T ? t : T - 1;
    h[n] = load4<HT>(a.H, ((static_cast<int64_t>(b) * T + t) * M + m) * d + c);
  }
  __syncthreads();

  // phase 2: conv taps, SiLU, residual for 4 channels x TPT tokens per thread
#pragma unroll
  for (int n = 0; n < TPT; ++n) {
    const int k = k0 + n * (256 / CG);
    const int64_t t = t0 + k;
    if (t >= T) break;
    const int r = span + k;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < ENGRAM_MAX_KERNEL_W; ++j) {
      if (j < kw) {
        const int rs = r - (kw - 1 - j) * g.dilation;
        const float s = scale_s[rs];
        const float4 u = tile[rs * CG + q];
        acc.x += wt[0][j] * (s * u.x);
        acc.y += wt[1][j] * (s * u.y);
        acc.z += wt[2][j] * (s * u.z);
        acc.w += wt[3][j] * (s * u.w);
      }
    }
    const float al = alpha_s[r];
    const float4 v = tile[r * CG + q];
    float4 y;
    y.x = silu(acc.x) + al * v.x;
    y.y = silu(acc.y) + al * v.y;
    y.z = silu(acc.z) + al * v.z;
    y.w = silu(acc.w) + al * v.w;
    const int64_t ho = ((static_cast<int64_t>(b) * T + t) * M + m) * d + c;
    float4 hn = h[n];
    hn.x += y.x;
    hn.y += y.y;
    hn.z += y.z;
    hn.w += y.w;
    store4<HT>(a.H, ho, hn);
    if (a.y_out != nullptr) *reinterpret_cast<float4*>(a.y_out + ho) = y;
  }
}

// Strip conv for a compile-time kernel width and dilation (the pages' w = 4,
// dilation N = 3).  A workgroup owns TS consecutive tokens x 256*CPT channels
// (CPT per thread) of one branch of one sequence.  Every load is issued up
// front: the TS + (KW-1)*DIL rows of v this strip needs (halo rows before the
// chunk come from the decode state, already as u), the thread's H values and
// the rows' gate statistics.  The statistics are reduced by 16 lanes per row
// into alpha and gamma in LDS (the only barrier); the dilated taps then read
// registers whose indices are fixed at compile time.
//
// Workgroup order: with spx > 0, workgroup i runs on XCD i % 8 (the hardware
// dispatches round robin) and XCD x owns strips [x*spx, (x+1)*spx), branches
// innermost, so the halo rows shared by neighbouring strips and the v rows
// shared by a strip's M branches are read through one L2.  spx == 0 (fewer
// strips than XCDs) keeps the plain order.
template <int HT, int VT, int KW, int DIL, int TS, int CPT>
__device__ __forceinline__ void conv_strip_body(const ConvArgs& a, int spx, int bx, int by, int bz) {
  constexpr int SPAN = (KW - 1) * DIL;
  constexpr int R = TS + SPAN;                 // rows this strip reads
  constexpr int kStatLanes = 16;               // lanes reducing one row's statistics
  constexpr int kStatRows = 256 / kStatLanes;  // rows reduced per pass
  __shared__ float alpha_s[R];
  __shared__ float gamma_s[R];
  const GateConvArgs& g = a.g;
  // Every scalar argument read in one batch with one wait (the asm
  // statements take them as operands, so all their loads are issued before
  // them); left to itself the compiler issues each where it is first needed
  // and waits there, three or four round trips before the first row read.
  {
    const void* const p0 = a.H;
    const void* const p1 = a.v;
    const void* const p2 = a.stats;
    const void* const p3 = g.conv_w;
    const void* const p4 = a.st.conv;
    const void* const p5 = a.st.pos;
    const void* const p6 = a.alpha_out;
    const void* const p7 = a.gamma_out;
    const void* const p8 = a.y_out;
    const int64_t l0 = a.v_stride, l1 = a.T;
    const int32_t i0 = a.qv, i1 = a.qk, i2 = a.nq, i3 = a.kq0, i4 = g.d, i5 = g.branches, i6 = a.has_state,
                  i7 = a.pos_advanced, i8 = a.commit_u, i9 = a.sums_from_kv;
    const float f0 = g.eps;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(p5), "s"(p6), "s"(p7), "s"(p8));
    asm volatile("" ::"s"(l0), "s"(l1), "s"(i0), "s"(i1), "s"(i2), "s"(i3), "s"(i4), "s"(i5), "s"(i6), "s"(i7),
                 "s"(i8), "s"(i9), "s"(f0));
    __builtin_amdgcn_sched_barrier(0);
  }
  const int M = g.branches;
  const int d = g.d;
  const int64_t T = a.T;
  int strip, m;
  {
    const int L = bx;
    if (spx > 0) {
      const int k = L >> 3;
      m = k % M;
      strip = (L & 7) * spx + k / M;
      if (static_cast<int64_t>(strip) * TS >= T) return;   // padding workgroup: no barrier reached yet
    } else {
      m = L % M;
      strip = L / M;
    }
  }
  // Sequences are shorter than 2^31 tokens and rows shorter than 2^31 bytes
  // (checked by the host), so positions and row strides are 32-bit; each row's
  // address is one uniform 64-bit base plus a 32 x 32-bit product.
  constexpr int kVB = VT == ENGRAM_BF16 ? 2 : 4;
  constexpr int kHB = HT == ENGRAM_BF16 ? 2 : 4;
  const int Ti = static_cast<int>(T);
  const int t0 = strip * TS;
  const int b = by;
  const int tid = threadIdx.x;
  const uint32_t c = (bz * 256 + tid) * CPT;  // this thread's CPT channels
  const bool active = c < static_cast<uint32_t>(d);
  const uint32_t cc = active ? c : 0;                 // a valid column for idle threads' loads
  const int64_t row0 = static_cast<int64_t>(b) * T;
  const char* vseq = static_cast<const char*>(a.v) + row0 * a.v_stride * kVB;
  const int vrow = static_cast<int>(a.v_stride) * kVB;
  char* hseq = static_cast<char*>(a.H) + (row0 * M + m) * d * kHB;
  const int hrow = M * d * kHB;
  const int nqb = a.qv + a.qk;

  // ---- issue every load ----
  // A strip that starts the chunk with a decode state reads its halo from
  // the state's ring slots, which depend on pos: pos is read first (reads
  // retire in order, so waiting for it waits for nothing else), as a
  // per-lane value (the compiler moves a uniform load's value to a scalar
  // register at the load and waits for it there), and the halo reads are
  // issued after the strip's own rows, H and the weights.
  const bool ring_halo = a.has_state && t0 < SPAN;
  int32_t pos_ld = 0;
  if (ring_halo) {
    int32_t lane0;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lane0));
    pos_ld = a.st.pos[b + lane0];
  }
  __builtin_amdgcn_sched_barrier(0);
  float v[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 - SPAN + r;
    if (!(r < SPAN && t < 0 && ring_halo)) {
      const int tc = t < 0 ? 0 : (t >= Ti ? Ti - 1 : t);
      loadc<VT, CPT>(vseq + static_cast<int64_t>(tc) * vrow, cc, v[r]);
    }
  }
  float h[TS][CPT];
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    const int t = t0 + k < Ti ? t0 + k : Ti - 1;
    loadc<HT, CPT>(hseq + static_cast<int64_t>(t) * hrow, cc, h[k]);
  }
  float wt[CPT][KW];
  {
    const float* wm = g.conv_w + static_cast<int64_t>(m) * d * KW;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if constexpr (KW == 4) {
        const float4 q = *reinterpret_cast<const float4*>(wm + (cc + i) * KW);
        wt[i][0] = q.x; wt[i][1] = q.y; wt[i][2] = q.z; wt[i][3] = q.w;
      } else {
#pragma unroll
        for (int j = 0; j < KW; ++j) wt[i][j] = wm[(cc + i) * KW + j];
      }
    }
  }
  // the halo before the chunk: the state's ring slot of position pos + t
  int p0 = 0;   // pos at the chunk's start, mod SPAN
  if (ring_halo) {
    p0 = (pos_ld - (a.pos_advanced ? Ti : 0)) % SPAN;
    if (p0 < 0) p0 += SPAN;
    const float* ring = a.st.conv + (static_cast<int64_t>(b) * M + m) * SPAN * d;
#pragma unroll
    for (int r = 0; r < SPAN; ++r) {
      const int t = t0 - SPAN + r;
      if (t < 0) {
        int slot = (p0 + t) % SPAN;
        if (slot < 0) slot += SPAN;
        loadc<ENGRAM_F32, CPT>(ring + static_cast<int64_t>(slot) * d, cc, v[r]);
      }
    }
  }

  bool from_kv = false;
  if constexpr (TS == 1) from_kv = a.sums_from_kv != 0;
  if (from_kv) {
    // ---- a single-token chunk on given float32 projections (v, then the M
    // keys, in one row): the workgroup holds its token's whole row (d <=
    // 256 * CPT, checked by the launcher), so it forms the gate's four sums
    // itself, by a block reduction, instead of reading per-tile statistics.
    // The halo rows are the state's conv inputs (gamma 1) or padding. ----
    __shared__ float4 wsum[4];
    float kk[CPT];
    loadc<VT, CPT>(vseq, static_cast<uint32_t>((1 + m) * d) + cc, kk);
    float s_hh = 0.f, s_kk = 0.f, s_hk = 0.f, s_vv = 0.f;
    if (active) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        s_hh += h[0][i] * h[0][i];
        s_kk += kk[i] * kk[i];
        s_hk += h[0][i] * kk[i];
        s_vv += v[SPAN][i] * v[SPAN][i];
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      s_hh += __shfl_xor(s_hh, off, 64);
      s_kk += __shfl_xor(s_kk, off, 64);
      s_hk += __shfl_xor(s_hk, off, 64);
      s_vv += __shfl_xor(s_vv, off, 64);
    }
    if ((tid & 63) == 0) wsum[tid >> 6] = make_float4(s_hh, s_kk, s_hk, s_vv);
    __syncthreads();
    if (tid < R) {
      float al = 0.f, gm = 0.f;
      if (tid == SPAN) {
        float4 q = wsum[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) q = make_float4(q.x + wsum[w].x, q.y + wsum[w].y, q.z + wsum[w].z, q.w + wsum[w].w);
        const float inv_d = 1.0f / static_cast<float>(d);
        const float rh = 1.0f / sqrtf(q.x * inv_d + g.eps);
        const float rk = 1.0f / sqrtf(q.y * inv_d + g.eps);
        const float logit = q.z * rh * rk / sqrtf(static_cast<float>(d));
        al = 1.0f / (1.0f + expf(-logit));
        gm = al / sqrtf(al * al * (q.w * inv_d) + g.eps);
        const int64_t o = row0 * M + m;
        if (a.alpha_out != nullptr) a.alpha_out[o] = al;
        if (a.gamma_out != nullptr) a.gamma_out[o] = gm;
      } else if (a.has_state) {
        gm = 1.0f;  // the state holds u itself
      }
      alpha_s[tid] = al;
      gamma_s[tid] = gm;
    }
  } else {
  // ---- alpha and gamma of the R rows: 16 lanes per row, shuffle reduction.
  // A lane loads up to kMaxQ statistics per pass (nqb <= 16 * kMaxQ = 64); all
  // passes' loads are issued before any is used. ----
  constexpr int kPasses = (R + kStatRows - 1) / kStatRows;
  constexpr int kMaxQ = 4;
  const int q0 = tid % kStatLanes;
  float4 sp[kPasses][kMaxQ];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int r = pass * kStatRows + tid / kStatLanes;
    const int t = t0 - SPAN + r;
    const int tc = t < 0 ? 0 : (t >= Ti ? Ti - 1 : t);
    const float4* st = a.stats + (row0 + tc) * a.nq;
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
      const int q = q0 + i * kStatLanes;
      const int qc = q < nqb ? q : 0;
      sp[pass][i] = st[qc < a.qv ? qc : a.qv + m * a.qk + (qc - a.qv)];
    }
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int r = pass * kStatRows + tid / kStatLanes;
    const int t = t0 - SPAN + r;
    const bool in_chunk = r < R && t >= 0 && t < Ti;
    float svv = 0.f, shh = 0.f, skk = 0.f, shk = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
      const int q = q0 + i * kStatLanes;
      const float4 p = sp[pass][i];
      // a.kq0 = 0 (mixed statistics): the value statistics carry the key sums too
      const bool key = q < a.qv ? q >= a.kq0 : q < nqb;
      if (q < a.qv) svv += p.w;
      shh += key ? p.x : 0.f;
      skk += key ? p.y : 0.f;
      shk += key ? p.z : 0.f;
    }
#pragma unroll
    for (int off = 1; off < kStatLanes; off <<= 1) {
      svv += __shfl_xor(svv, off, 64);
      shh += __shfl_xor(shh, off, 64);
      skk += __shfl_xor(skk, off, 64);
      shk += __shfl_xor(shk, off, 64);
    }
    if (q0 == 0 && r < R) {
      float al = 0.f, gm = 0.f;
      if (in_chunk) {
        const float inv_d = 1.0f / static_cast<float>(d);
        const float rh = 1.0f / sqrtf(shh * inv_d + g.eps);
        const float rk = 1.0f / sqrtf(skk * inv_d + g.eps);
        const float logit = shk * rh * rk / sqrtf(static_cast<float>(d));
        al = 1.0f / (1.0f + expf(-logit));
        gm = al / sqrtf(al * al * (svv * inv_d) + g.eps);
        if (bz == 0 && r >= SPAN) {
          const int64_t o = (row0 + t) * M + m;
          if (a.alpha_out != nullptr) a.alpha_out[o] = al;
          if (a.gamma_out != nullptr) a.gamma_out[o] = gm;
        }
      } else if (t < 0 && a.has_state) {
        gm = 1.0f;  // the state holds u itself
      }
      alpha_s[r] = al;
      gamma_s[r] = gm;
    }
  }
  }
  __syncthreads();

  // ---- u = gamma v, dilated causal taps, SiLU, residual ----
  float u[R][CPT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float gm = gamma_s[r];
#pragma unroll
    for (int i = 0; i < CPT; ++i) u[r][i] = gm * v[r][i];
  }
#pragma unroll
  for (int k = 0; k < TS; ++k) {
    const int t = t0 + k;
    const int r = SPAN + k;
    const float al = alpha_s[r];
    float y[CPT], hn[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) acc += wt[i][j] * u[r - (KW - 1 - j) * DIL][i];
      y[i] = silu(acc) + al * v[r][i];
      hn[i] = h[k][i] + y[i];
    }
    if (active && t < Ti) {
      storec<HT, CPT>(hseq + static_cast<int64_t>(t) * hrow, c, hn);
      if (a.y_out != nullptr) storec<ENGRAM_F32, CPT>(a.y_out + ((row0 + t) * M + m) * d, c, y);
    }
  }
  // Decode (T = 1 strips): the new position's conv input u goes to its ring
  // slot (pos % SPAN, which held position pos - SPAN: this workgroup read that
  // row for its oldest tap above and owns these channels, so no other
  // workgroup reads the slot).
  if constexpr (TS == 1) {
    if (a.commit_u && active) {
      const int slot = p0;   // T = 1: the chunk's one position
      float uc[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) uc[i] = u[SPAN][i];
      storec<ENGRAM_F32, CPT>(a.st.conv + ((static_cast<int64_t>(b) * M + m) * SPAN + slot) * d, c, uc);
    }
  }
}

// Steps 6-8 of one decode token (T = 1) on its float32 [v | k^(0..M-1)] row
// (ConvArgs.sums_from_kv), for the pages' conv (w = 4, dilation 3) and d <=
// 1024: workgroup (b, m) holds the token's whole row, 4 channels a thread.
// The same arithmetic as the single-token strip conv, laid out for latency:
// every argument is read up front in one batch, then pos (which the state's
// halo slots depend on), the row, H and the conv weights are read together,
// so that the chain is arguments -> (pos, row) -> state rows, with the gate's
// block reduction inside the last latency.
template <int HT>
__global__ void __launch_bounds__(256)
conv_decode_kernel(ConvArgs a) {
  constexpr int KW = 4, DIL = 3, SPAN = (KW - 1) * DIL, CPT = 4;
  const int b = blockIdx.x, m = blockIdx.y, tid = threadIdx.x;
  void* const Hp = a.H;
  const float* const vp = static_cast<const float*>(a.v);
  const int64_t v_stride = a.v_stride;
  const float* const conv_w = a.g.conv_w;
  const int d = a.g.d, M = a.g.branches;
  const float eps = a.g.eps;
  float* const st_conv = a.st.conv;
  const int32_t* const st_pos = a.st.pos;
  const int has_state = a.has_state, pos_adv = a.pos_advanced, commit_u = a.commit_u;
  float* const alpha_out = a.alpha_out;
  float* const gamma_out = a.gamma_out;
  float* const y_out = a.y_out;
  // one batch of argument loads, then one wait (the compiler would otherwise
  // issue each where it is first needed and wait for it there)
  asm volatile("" ::"s"(Hp), "s"(vp), "s"(v_stride), "s"(conv_w), "s"(d), "s"(M), "s"(eps), "s"(st_conv),
               "s"(st_pos), "s"(has_state), "s"(pos_adv), "s"(commit_u));
  asm volatile("" ::"s"(alpha_out), "s"(gamma_out), "s"(y_out));
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t c = tid * CPT;
  const bool active = c < static_cast<uint32_t>(d);
  const uint32_t cc = active ? c : 0;
  const int64_t row = b;   // T = 1: token b of the batch
  const float* vrow = vp + row * v_stride;
  char* hrow = static_cast<char*>(Hp) + (row * M + m) * d * (HT == ENGRAM_BF16 ? 2 : 4);
  // pos first in the memory queue, from a valid address either way, so that
  // waiting for it (reads retire in order) waits for nothing else.  The
  // offset is a zero the compiler cannot see through: as a per-lane value,
  // pos is not moved to a scalar register at the load, which would wait for
  // it there, before the row's reads are issued.
  int32_t lane0;
  asm volatile("v_mov_b32 %0, 0" : "=v"(lane0));
  const int32_t* const pos_p = has_state ? st_pos + b : reinterpret_cast<const int32_t*>(vp);
  const int32_t pos_ld = pos_p[lane0];
  __builtin_amdgcn_sched_barrier(0);
  float v[CPT], kk[CPT], h[CPT];
  loadc<ENGRAM_F32, CPT>(vrow, cc, v);
  loadc<ENGRAM_F32, CPT>(vrow, static_cast<uint32_t>((1 + m) * d) + cc, kk);
  loadc<HT, CPT>(hrow, cc, h);
  float wt[CPT][KW];
  {
    const float* wm = conv_w + static_cast<int64_t>(m) * d * KW;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const float4 q = *reinterpret_cast<const float4*>(wm + (cc + i) * KW);
      wt[i][0] = q.x; wt[i][1] = q.y; wt[i][2] = q.z; wt[i][3] = q.w;
    }
  }
  // the taps' halo rows r = 0, 3, 6 (positions pos - 9, - 6, - 3): the
  // state's ring slots (pos + 3 r) % 9, which already hold u (gamma 1).
  // Without a state the chunk starts here and they are padding; as zeros
  // they add +0 to a sum that starts at +0, as gamma 0 times the clamped row
  // does in the strip conv, so both give the same bits.  (Padding taken from
  // v would make the state's reads wait for v's.)
  __builtin_amdgcn_sched_barrier(0);
  int p9 = 0;
  float hv[KW - 1][CPT];
  if (has_state) {
    p9 = (pos_ld - (pos_adv ? 1 : 0)) % SPAN;
    if (p9 < 0) p9 += SPAN;
    const float* ring = st_conv + (static_cast<int64_t>(b) * M + m) * SPAN * d;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) {
      int slot = p9 + j * DIL;
      if (slot >= SPAN) slot -= SPAN;
      loadc<ENGRAM_F32, CPT>(ring + static_cast<int64_t>(slot) * d, cc, hv[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KW - 1; ++j)
#pragma unroll
      for (int i = 0; i < CPT; ++i) hv[j][i] = 0.f;
  }

  // the gate's four sums over the row (the strip conv's order)
  __shared__ float4 wsum[4];
  __shared__ float ag[2];
  float s_hh = 0.f, s_kk = 0.f, s_hk = 0.f, s_vv = 0.f;
  if (active) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      s_hh += h[i] * h[i];
      s_kk += kk[i] * kk[i];
      s_hk += h[i] * kk[i];
      s_vv += v[i] * v[i];
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    s_hh += __shfl_xor(s_hh, off, 64);
    s_kk += __shfl_xor(s_kk, off, 64);
    s_hk += __shfl_xor(s_hk, off, 64);
    s_vv += __shfl_xor(s_vv, off, 64);
  }
  if ((tid & 63) == 0) wsum[tid >> 6] = make_float4(s_hh, s_kk, s_hk, s_vv);
  __syncthreads();
  if (tid == 0) {
    float4 q = wsum[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) q = make_float4(q.x + wsum[w].x, q.y + wsum[w].y, q.z + wsum[w].z, q.w + wsum[w].w);
    const float inv_d = 1.0f / static_cast<float>(d);
    const float rh = 1.0f / sqrtf(q.x * inv_d + eps);
    const float rk = 1.0f / sqrtf(q.y * inv_d + eps);
    const float logit = q.z * rh * rk / sqrtf(static_cast<float>(d));
    const float al = 1.0f / (1.0f + expf(-logit));
    const float gm = al / sqrtf(al * al * (q.w * inv_d) + eps);
    const int64_t o = row * M + m;
    if (alpha_out != nullptr) alpha_out[o] = al;
    if (gamma_out != nullptr) gamma_out[o] = gm;
    ag[0] = al;
    ag[1] = gm;
  }
  __syncthreads();
  const float al = ag[0], gm = ag[1];

  // u = gamma v, the dilated causal taps, SiLU, residual
  float u[CPT], y[CPT], hn[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    u[i] = gm * v[i];
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) acc += wt[i][j] * hv[j][i];
    acc += wt[i][KW - 1] * u[i];
    y[i] = silu(acc) + al * v[i];
    hn[i] = h[i] + y[i];
  }
  if (active) {
    storec<HT, CPT>(hrow, c, hn);
    if (y_out != nullptr) storec<ENGRAM_F32, CPT>(y_out + (row * M + m) * d, c, y);
    // the new position's conv input goes to its ring slot (pos % SPAN, which
    // held position pos - SPAN: read above as the oldest tap, by this thread)
    if (commit_u && has_state)
      storec<ENGRAM_F32, CPT>(st_conv + ((static_cast<int64_t>(b) * M + m) * SPAN + p9) * d, c, u);
  }
}

template <int HT, int VT, int KW, int DIL, int TS, int CPT>
__global__ void __launch_bounds__(256)
conv_strip_kernel(ConvArgs a, int spx) {
  conv_strip_body<HT, VT, KW, DIL, TS, CPT>(a, spx, blockIdx.x, blockIdx.y, blockIdx.z);
}

// One launch with two kinds of workgroups: the first n_conv run this call's
// strip conv (the 3-D grid flattened x fastest, so workgroup i still runs on
// XCD i % 8 and keeps the strips' XCD order), the rest run the next
// retrieval's hashed gather (Steps 1-4 from token ids and, in decode, the next
// layer's id history).  The two share no data; both are bound by memory
// latency at these sizes, so each fills the other's wait cycles on the same
// CUs -- the pages' prefetch of the next retrieval behind the current
// computation, without a second stream.
template <int KW, int DIL, int TS, int CPT, int GIN, int GOUT, int ITEMS>
__global__ void __launch_bounds__(256)
conv_gather_kernel(ConvArgs a, int spx, uint32_t n_conv, uint32_t gx, GatherJob gj) {
  const uint32_t flat = blockIdx.x;
  if (flat < n_conv) {
    const uint32_t plane = gx * static_cast<uint32_t>(a.B);
    const uint32_t bz = flat / plane;
    const uint32_t rem = flat - bz * plane;
    const uint32_t by = rem / gx;
    conv_strip_body<ENGRAM_BF16, ENGRAM_F32, KW, DIL, TS, CPT>(a, spx, static_cast<int>(rem - by * gx),
                                                                static_cast<int>(by), static_cast<int>(bz));
  } else {
    hashed_gather_body<GIN, GOUT, false, ITEMS>((flat - n_conv) * 256 + threadIdx.x, gj.n_tok, gj.ta, gj.e,
                                                 gj.hs);
  }
}

// After the conv: the chunk's last (w-1)*dilation conv inputs go to their
// circular slots, the last N-1 compressed ids shift into the history, and pos
// advances.  One workgroup per sequence; pos is written after the block has
// read it everywhere.
template <int VT>
__global__ void __launch_bounds__(256)
state_commit_kernel(const void* __restrict__ v, int64_t v_stride, int64_t T, GateConvArgs g,
                    const float* __restrict__ gamma, StateArgs st, const int32_t* __restrict__ tokens,
                    const int32_t* __restrict__ proj, int32_t max_n, int32_t vocab, uint32_t* err) {
  const int64_t b = blockIdx.x;
  const int M = g.branches;
  const int d = g.d;
  const int span = (g.kernel_w - 1) * g.dilation;
  const int32_t pos0 = st.pos[b];
  const int L = static_cast<int>(T < span ? T : span);
  const int c4 = d / 4;
  const int total = M * L * c4;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int cq = idx % c4;
    const int mq = idx / c4;
    const int q = mq % L;
    const int m = mq / L;
    const int64_t p = T - L + q;
    const int slot = static_cast<int>((static_cast<int64_t>(pos0) + p) % span);
    const int64_t bs = b * T + p;
    float4 u = load4<VT>(v, bs * v_stride + cq * 4);
    const float gm = gamma[bs * M + m];
    u.x *= gm;
    u.y *= gm;
    u.z *= gm;
    u.w *= gm;
    *reinterpret_cast<float4*>(st.conv + ((b * M + m) * span + slot) * static_cast<int64_t>(d) + cq * 4) = u;
  }
  if (threadIdx.x == 0 && st.ids != nullptr && tokens != nullptr) {
    const int hl = max_n - 1;
    int32_t next[ENGRAM_MAX_ORDER];
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER - 1; ++i) {
      if (i < hl) {
        const int64_t idx = T + i;  // index in (old ids ++ chunk ids)
        next[i] = idx < hl ? st.ids[b * hl + idx] : proj[token_in_vocab(tokens[b * T + idx - hl], vocab, err)];
      }
    }
#pragma unroll
    for (int i = 0; i < ENGRAM_MAX_ORDER - 1; ++i)
      if (i < hl) st.ids[b * hl + i] = next[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) st.pos[b] = pos0 + static_cast<int32_t>(T);
}

}  // namespace

hipError_t launch_gate_stats(const void* H, const void* kv, int64_t n_tok, const GateConvArgs& g, float4* stats,
                             hipStream_t s) {
  const int64_t pairs = n_tok * g.branches;
  if (pairs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4));
  if (g.hdtype == ENGRAM_BF16 && g.kvdtype == ENGRAM_BF16)
    launch_k((gate_stats_kernel<ENGRAM_BF16, ENGRAM_BF16>), grid, dim3(256), 0, s, H, kv, n_tok,
                       g.branches, g.d, stats);
  else if (g.hdtype == ENGRAM_BF16)
    launch_k((gate_stats_kernel<ENGRAM_BF16, ENGRAM_F32>), grid, dim3(256), 0, s, H, kv, n_tok,
                       g.branches, g.d, stats);
  else
    launch_k((gate_stats_kernel<ENGRAM_F32, ENGRAM_F32>), grid, dim3(256), 0, s, H, kv, n_tok,
                       g.branches, g.d, stats);
  return hipGetLastError();
}

template <int CG>
hipError_t launch_conv_cg(const ConvArgs& a, int vdtype, hipStream_t s) {
  const int span = (a.g.kernel_w - 1) * a.g.dilation;
  const size_t lds = static_cast<size_t>(TT + span) * (CG + a.qv + a.qk) * sizeof(float4);
  const dim3 grid(static_cast<unsigned>((a.T + TT - 1) / TT), static_cast<unsigned>(a.B * a.g.branches),
                  static_cast<unsigned>(a.g.d / (CG * 4)));
  const void* fn;
  if (a.g.hdtype == ENGRAM_BF16 && vdtype == ENGRAM_BF16)
    fn = reinterpret_cast<const void*>(conv_kernel<ENGRAM_BF16, ENGRAM_BF16, CG>);
  else if (a.g.hdtype == ENGRAM_BF16)
    fn = reinterpret_cast<const void*>(conv_kernel<ENGRAM_BF16, ENGRAM_F32, CG>);
  else
    fn = reinterpret_cast<const void*>(conv_kernel<ENGRAM_F32, ENGRAM_F32, CG>);
  if (lds > 48 * 1024) {
    // large statistics tiles (wide d) need more than the default dynamic LDS
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  if (a.g.hdtype == ENGRAM_BF16 && vdtype == ENGRAM_BF16)
    launch_k((conv_kernel<ENGRAM_BF16, ENGRAM_BF16, CG>), grid, dim3(256), lds, s, a);
  else if (a.g.hdtype == ENGRAM_BF16)
    launch_k((conv_kernel<ENGRAM_BF16, ENGRAM_F32, CG>), grid, dim3(256), lds, s, a);
  else
    launch_k((conv_kernel<ENGRAM_F32, ENGRAM_F32, CG>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int KW, int DIL, int TS, int CPT>
hipError_t launch_conv_strip(const ConvArgs& a, int vdtype, hipStream_t s) {
  const int64_t n_strips = (a.T + TS - 1) / TS;
  const int spx = n_strips >= 8 ? static_cast<int>((n_strips + 7) / 8) : 0;
  const int64_t gx = (spx > 0 ? 8 * static_cast<int64_t>(spx) : n_strips) * a.g.branches;
  if (gx > 0x7fffffff || a.B > 65535) return hipErrorInvalidConfiguration;   // grid limits
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(a.B),
                  static_cast<unsigned>((a.g.d + 256 * CPT - 1) / (256 * CPT)));
  if (a.g.hdtype == ENGRAM_BF16 && vdtype == ENGRAM_BF16)
    launch_k((conv_strip_kernel<ENGRAM_BF16, ENGRAM_BF16, KW, DIL, TS, CPT>), grid, dim3(256), 0, s, a, spx);
  else if (a.g.hdtype == ENGRAM_BF16)
    launch_k((conv_strip_kernel<ENGRAM_BF16, ENGRAM_F32, KW, DIL, TS, CPT>), grid, dim3(256), 0, s, a, spx);
  else
    launch_k((conv_strip_kernel<ENGRAM_F32, ENGRAM_F32, KW, DIL, TS, CPT>), grid, dim3(256), 0, s, a, spx);
  return hipGetLastError();
}

// Strip shape of the pages' conv (w = 4, dilation 3): decode steps get
// 1-token strips; otherwise 16-token strips of 512 channels when that gives
// at least 4 workgroups per CU, else 4-token strips of 1024 channels (4x the
// workgroups, more halo re-reads, which hit L2).  Returns TS (CPT = 4 for
// TS <= 4, else 2), or 0 when the strip kernel does not apply.
int conv_strip_ts(const ConvArgs& a) {
  if (a.g.kernel_w != 4 || a.g.dilation != 3 || a.qv + a.qk > kConvMaxStats) return 0;
  if (a.T == 1) return 1;
  const int64_t wg16 = a.B * a.g.branches * ((a.T + 15) / 16) * ((a.g.d + 511) / 512);
  return wg16 < 1024 ? 4 : 16;
}

template <int TS, int CPT, int GIN>
hipError_t launch_conv_gather_ts(const ConvArgs& a, const GatherJob& gj, hipStream_t s) {
  // the strip grid of launch_conv_strip: XCD order from 8 strips up, else plain
  const int64_t n_strips = (a.T + TS - 1) / TS;
  const int spx = n_strips >= 8 ? static_cast<int>((n_strips + 7) / 8) : 0;
  const int64_t gx = (spx > 0 ? 8 * static_cast<int64_t>(spx) : n_strips) * a.g.branches;
  const int64_t gz = (a.g.d + 256 * CPT - 1) / (256 * CPT);
  const int64_t n_conv = gx * a.B * gz;
  const int64_t per_group = static_cast<int64_t>(gj.ta.n_tables) * (gj.ta.dim / 8);
  // 4 tokens per gather thread: the fewest wavefronts, so that the gather and
  // the conv fit on the CUs together
  constexpr int items = 4;
  const int64_t g_threads = (static_cast<int64_t>(gj.n_tok) + items - 1) / items * per_group;
  const int64_t n_blocks = n_conv + (g_threads + 255) / 256;
  if (n_blocks >= (1ll << 31) || g_threads >= (1ll << 31)) return hipErrorNotSupported;
  const dim3 grid(static_cast<unsigned>(n_blocks));
  const uint32_t nc = static_cast<uint32_t>(n_conv), ux = static_cast<uint32_t>(gx);
  if (gj.out_dtype == kGatherOutMXFP8)
    launch_k((conv_gather_kernel<4, 3, TS, CPT, GIN, kGatherOutMXFP8, items>), grid, dim3(256), 0, s, a, spx, nc, ux,
             gj);
  else
    launch_k((conv_gather_kernel<4, 3, TS, CPT, GIN, ENGRAM_BF16, items>), grid, dim3(256), 0, s, a, spx, nc, ux, gj);
  return hipGetLastError();
}

template <int GIN>
hipError_t launch_conv_gather_in(int ts, const ConvArgs& a, const GatherJob& gj, hipStream_t s) {
  switch (ts) {
    case 1: return launch_conv_gather_ts<1, 4, GIN>(a, gj, s);
    case 4: return launch_conv_gather_ts<4, 4, GIN>(a, gj, s);
    default: return launch_conv_gather_ts<16, 2, GIN>(a, gj, s);
  }
}

// The strip conv of this call with the next retrieval's gather in the same
// launch, the conv in exactly the shape launch_conv would give it (so the
// results are bit-identical to the two launches), with or without a decode
// state.  Only for the layer forward's own case: bf16 H and float32 v from
// the fused projection, the strip conv (w = 4, dilation 3), bf16 or int8
// tables without a hot tier, bf16 or MXFP8 rows out; anything else returns
// hipErrorNotSupported before launching, and the caller launches the two
// kernels one after the other.
hipError_t launch_conv_gather(const ConvArgs& a, int vdtype, const GatherJob& gj, hipStream_t s) {
  if (a.g.hdtype != ENGRAM_BF16 || vdtype != ENGRAM_F32 || gj.hot ||
      (gj.ta.dtype != ENGRAM_BF16 && gj.ta.dtype != ENGRAM_I8) ||
      (gj.out_dtype != ENGRAM_BF16 && gj.out_dtype != kGatherOutMXFP8) || a.B * a.T == 0 || gj.n_tok == 0)
    return hipErrorNotSupported;
  const int ts = conv_strip_ts(a);
  if (ts == 0) return hipErrorNotSupported;
  return gj.ta.dtype == ENGRAM_I8 ? launch_conv_gather_in<ENGRAM_I8>(ts, a, gj, s)
                                  : launch_conv_gather_in<ENGRAM_BF16>(ts, a, gj, s);
}

hipError_t launch_conv(const ConvArgs& a, int vdtype, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  if (a.sums_from_kv) {
    // a single token per sequence with the whole row in one workgroup
    if (conv_strip_ts(a) != 1 || a.g.d > 256 * 4 || vdtype != ENGRAM_F32 || a.B > 0x7fffffff ||
        a.g.branches > 65535)
      return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(a.B), static_cast<unsigned>(a.g.branches));
    if (a.g.hdtype == ENGRAM_BF16)
      launch_k(conv_decode_kernel<ENGRAM_BF16>, grid, dim3(256), 0, s, a);
    else
      launch_k(conv_decode_kernel<ENGRAM_F32>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  // both conv kernels stage at most kConvMaxStats statistics per row (the
  // projection launchers never produce more)
  if (a.qv < 1 || (a.qk < 1 && !a.mixed) || (a.mixed && a.qk != 0) || a.qv + a.qk > kConvMaxStats)
    return hipErrorInvalidValue;
  switch (conv_strip_ts(a)) {   // the pages' conv (w = 4, dilation 3): strip kernel
    case 1: return launch_conv_strip<4, 3, 1, 4>(a, vdtype, s);
    case 4: return launch_conv_strip<4, 3, 4, 4>(a, vdtype, s);
    case 16: return launch_conv_strip<4, 3, 16, 2>(a, vdtype, s);
    default: break;
  }
  switch (conv_channels(a.g.d)) {
    case 256: return launch_conv_cg<64>(a, vdtype, s);
    case 128: return launch_conv_cg<32>(a, vdtype, s);
    default: return launch_conv_cg<16>(a, vdtype, s);
  }
}

hipError_t launch_state_commit(const void* v, int64_t v_stride, int vdtype, int64_t B, int64_t T,
                               const GateConvArgs& g, const float* gamma, const StateArgs& st,
                               const int32_t* tokens, const int32_t* proj, int32_t max_n, int32_t vocab,
                               uint32_t* err, hipStream_t s) {
  if (B == 0 || T == 0) return hipSuccess;
  if (vdtype == ENGRAM_BF16)
    launch_k(state_commit_kernel<ENGRAM_BF16>, dim3(static_cast<unsigned>(B)), dim3(256), 0, s,
                       v, v_stride, T, g, gamma, st, tokens, proj, max_n, vocab, err);
  else
    launch_k(state_commit_kernel<ENGRAM_F32>, dim3(static_cast<unsigned>(B)), dim3(256), 0, s,
                       v, v_stride, T, g, gamma, st, tokens, proj, max_n, vocab, err);
  return hipGetLastError();
}

}  // namespace engram
