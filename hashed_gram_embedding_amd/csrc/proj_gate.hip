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
// gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16), float32 accumulation.
// The weight rows are the MFMA A operand and the token rows of e the B
// operand: each lane then holds 4 consecutive features of one token per
// 16x16 block, so v stores are 16-byte vectors and h loads 8-byte vectors.
// Workgroup tile: 128 features x 256 tokens, four wavefronts of 64 x 128;
// K advances 64 per step through double-buffered LDS (96 KiB) with the 16-byte
// chunk c of row r stored at chunk c ^ (r & 7); the next K slice is fetched to
// registers while the current one is multiplied.  Tiles are ordered XCD by
// XCD (workgroup i runs on XCD i % 8) with the feature tile fastest, so the
// workgroups that read the same e rows share an L2.
#include <atomic>

#include "device_util.h"
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int TF = 128;  // features per workgroup
constexpr int TK = 256;  // tokens per workgroup
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kWChunks = TF * BK / 8;  // 16-byte chunks of a W slice
constexpr int kEChunks = TK * BK / 8;  // 16-byte chunks of an e slice

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
proj_gate_kernel(ProjGateArgs a) {
  extern __shared__ uint4 lds[];
  uint4* Ws = lds;                    // [2][kWChunks]
  uint4* Es = lds + 2 * kWChunks;     // [2][kEChunks]

  const int n_tiles = a.tiles_f * a.tiles_t;
  const int L = blockIdx.x;
  const int tile = (n_tiles % kXcds == 0) ? (L % kXcds) * (n_tiles / kXcds) + L / kXcds : L;
  const int tf = tile % a.tiles_f;
  const int tt = tile / a.tiles_f;
  const int f0 = tf * TF;
  const int64_t t0 = static_cast<int64_t>(tt) * TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wf = wave & 1;   // feature half
  const int wt = wave >> 1;  // token half
  const int K = a.K;

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // global -> register staging of one K slice: 4 chunks of W and 8 of e per thread
  uint4 rw0, rw1, rw2, rw3, re[8];
  const uint16_t* wbase = a.w + static_cast<int64_t>(f0) * K;
#define ENGRAM_LOAD_SLICE(k0)                                                                   \
  {                                                                                             \
    rw0 = *reinterpret_cast<const uint4*>(wbase + (tid >> 3) * K + (k0) + (tid & 7) * 8);          \
    rw1 = *reinterpret_cast<const uint4*>(wbase + ((tid >> 3) + 32) * K + (k0) + (tid & 7) * 8);   \
    rw2 = *reinterpret_cast<const uint4*>(wbase + ((tid >> 3) + 64) * K + (k0) + (tid & 7) * 8);   \
    rw3 = *reinterpret_cast<const uint4*>(wbase + ((tid >> 3) + 96) * K + (k0) + (tid & 7) * 8);   \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                             \
      const int64_t tok = t0 + (tid >> 3) + i * 32;                                             \
      re[i] = tok < a.n_tok ? *reinterpret_cast<const uint4*>(a.e + tok * K + (k0) + (tid & 7) * 8) \
                            : make_uint4(0, 0, 0, 0);                                           \
    }                                                                                           \
  }
#define ENGRAM_STORE_SLICE(buf)                                                                 \
  {                                                                                             \
    uint4* ws_ = Ws + (buf) * kWChunks;                                                         \
    uint4* es_ = Es + (buf) * kEChunks;                                                         \
    ws_[swz((tid >> 3), tid & 7)] = rw0;                                                        \
    ws_[swz((tid >> 3) + 32, tid & 7)] = rw1;                                                   \
    ws_[swz((tid >> 3) + 64, tid & 7)] = rw2;                                                   \
    ws_[swz((tid >> 3) + 96, tid & 7)] = rw3;                                                   \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) es_[swz((tid >> 3) + i * 32, tid & 7)] = re[i]; \
  }

  const int ksteps = K / BK;
  ENGRAM_LOAD_SLICE(0);
  ENGRAM_STORE_SLICE(0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ksteps) ENGRAM_LOAD_SLICE((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kc = ks * 4 + (lane >> 4);
      bf16x8_t fa[4], fb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = __builtin_bit_cast(bf16x8_t, Ws[cur * kWChunks + swz(wf * 64 + i * 16 + (lane & 15), kc)]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        fb[j] = __builtin_bit_cast(bf16x8_t, Es[cur * kEChunks + swz(wt * 128 + j * 16 + (lane & 15), kc)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ksteps) ENGRAM_STORE_SLICE(cur ^ 1);
    __syncthreads();
  }
#undef ENGRAM_LOAD_SLICE
#undef ENGRAM_STORE_SLICE

  // ---- epilogue: lane holds features f0 + wf*64 + i*16 + (lane>>4)*4 + r of
  // token t0 + wt*128 + j*16 + (lane & 15) ----
  const int d = a.d;
  const bool is_v = f0 < d;
  const int m = is_v ? 0 : f0 / d - 1;
  const int c0 = is_v ? f0 : f0 - (1 + m) * d;   // column inside v or inside k^(m)
  float4* red = reinterpret_cast<float4*>(lds);   // [TK][2] partials of the two feature halves
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tl = wt * 128 + j * 16 + (lane & 15);
    const int64_t tok = t0 + tl;
    const bool valid = tok < a.n_tok;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = c0 + wf * 64 + i * 16 + (lane >> 4) * 4;
      const f32x4_t x = acc[i][j];
      if (is_v) {
        if (valid) *reinterpret_cast<float4*>(a.v + tok * d + col) = make_float4(x[0], x[1], x[2], x[3]);
        s3 += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
      } else if (valid) {
        const uint2 hq = *reinterpret_cast<const uint2*>(a.H + (tok * a.M + m) * d + col);
        const float h0 = __uint_as_float(hq.x << 16), h1 = __uint_as_float(hq.x & 0xffff0000u);
        const float h2 = __uint_as_float(hq.y << 16), h3 = __uint_as_float(hq.y & 0xffff0000u);
        s0 += h0 * h0 + h1 * h1 + h2 * h2 + h3 * h3;
        s1 += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        s2 += h0 * x[0] + h1 * x[1] + h2 * x[2] + h3 * x[3];
      }
    }
    s0 += __shfl_xor(s0, 16, 64); s0 += __shfl_xor(s0, 32, 64);
    s1 += __shfl_xor(s1, 16, 64); s1 += __shfl_xor(s1, 32, 64);
    s2 += __shfl_xor(s2, 16, 64); s2 += __shfl_xor(s2, 32, 64);
    s3 += __shfl_xor(s3, 16, 64); s3 += __shfl_xor(s3, 32, 64);
    if ((lane >> 4) == 0) red[tl * 2 + wf] = make_float4(s0, s1, s2, s3);
  }
  __syncthreads();
  {
    const int64_t tok = t0 + tid;
    if (tok < a.n_tok) {
      const float4 p = red[tid * 2], q = red[tid * 2 + 1];
      a.stats[tok * a.tiles_f + tf] = make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
    }
  }
}

}  // namespace

size_t proj_gate_lds_bytes() { return static_cast<size_t>(2 * (kWChunks + kEChunks)) * sizeof(uint4); }

hipError_t launch_proj_gate(const ProjGateArgs& in, hipStream_t s) {
  if (in.n_tok == 0) return hipSuccess;
  ProjGateArgs a = in;
  a.tiles_f = a.N / TF;
  a.tiles_t = static_cast<int>((a.n_tok + TK - 1) / TK);
  const size_t lds = proj_gate_lds_bytes();
  // 96 KiB of dynamic LDS exceeds the default per-workgroup limit; raise it
  // once per device (gfx950 has 160 KiB of LDS per CU).
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if ((attr_set.load() & bit) == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(proj_gate_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  hipLaunchKernelGGL(proj_gate_kernel, dim3(a.tiles_f * a.tiles_t), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace engram
