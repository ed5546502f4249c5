// Step 5 of "DeepSeek Engram series guide", section "Engram working
// principle" (k_t = W_K e_t, v_t = W_V e_t), done as one dense product with
// the value and all branch keys stacked, as the multi-branch variant on the
// same page suggests:  kv[t][o] = sum_c e[t][c] * W[o][c].
//
// bf16 path: gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), float32
// accumulation.  A 256-thread workgroup computes a 128 x 128 tile of kv with
// four wavefronts of 64 x 64 each; K advances 64 at a time through LDS.  Both
// operands are K-contiguous (e rows, W rows), so every lane's 8-element MFMA
// fragment is one 16-byte LDS read.  LDS rows are 128 bytes; the 16-byte
// chunk c of row r is stored at chunk c ^ (r & 7) so that the 16 rows a
// fragment read touches spread over the banks.  The next K slice is fetched
// into registers while the current one is multiplied.
//
// Tiles are handed out XCD by XCD: workgroup i runs on XCD i % 8, so tile
// numbers are remapped such that each XCD walks a contiguous range, n
// fastest; the tiles that share an e row block then share one L2.
//
// The bf16 path can write kv as bf16 (the standalone projection entry point)
// or keep the float32 accumulators (inside the layer forward, where v feeds a
// normalisation and the conv and bf16 rounding would cost accuracy).
//
// f32 path: plain per-output dot products (small shapes only).
#include "device_util.h"
#include "engram_internal.h"

namespace engram {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <typename OutT>
__global__ void __launch_bounds__(kThreads)
gemm_bf16_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                 OutT* __restrict__ C, int64_t M, int N, int K, int tiles_m, int tiles_n) {
  __shared__ uint4 As[BM * BK / 8];
  __shared__ uint4 Bs[BN * BK / 8];

  // XCD-aware tile order.
  const int n_tiles = tiles_m * tiles_n;
  const int L = blockIdx.x;
  int tile;
  if (n_tiles % kXcds == 0) {
    tile = (L % kXcds) * (n_tiles / kXcds) + L / kXcds;
  } else {
    tile = L;
  }
  const int tm = tile / tiles_n;
  const int tn = tile - tm * tiles_n;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // global -> register staging: 4 chunks of A and 4 of W per thread
  uint4 ra[4], rb[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3;
      const int kc = c & 7;
      const int64_t gm = m0 + row;
      ra[i] = gm < M ? *reinterpret_cast<const uint4*>(A + gm * K + k0 + kc * 8)
                     : make_uint4(0, 0, 0, 0);
      rb[i] = n0 + row < N
                  ? *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(n0 + row) * K + k0 + kc * 8)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3;
      const int kc = c & 7;
      As[swz(row, kc)] = ra[i];
      Bs[swz(row, kc)] = rb[i];
    }
  };

  const int kt_count = K / BK;
  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kt = 0; kt < kt_count; ++kt) {
    if (kt + 1 < kt_count) load_tile((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kchunk = ks * 4 + (lane >> 4);
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_row = wm * 64 + i * 16 + (lane & 15);
        const uint4 q = As[swz(ra_row, kchunk)];
        a[i] = __builtin_bit_cast(bf16x8_t, q);
        const int rb_row = wn * 64 + i * 16 + (lane & 15);
        const uint4 p = Bs[swz(rb_row, kchunk)];
        b[i] = __builtin_bit_cast(bf16x8_t, p);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (kt + 1 < kt_count) {
      store_tile();
      __syncthreads();
    }
  }

  // epilogue: lane holds rows (lane>>4)*4 + r of column (lane & 15) of each 16x16 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t gm = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
      if (gm >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gn = n0 + wn * 64 + j * 16 + (lane & 15);
        if (gn < N) {
          if constexpr (sizeof(OutT) == 2) C[gm * N + gn] = f32_to_bf16(acc[i][j][r]);
          else C[gm * N + gn] = acc[i][j][r];
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256)
gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W, float* __restrict__ C,
                int64_t M, int N, int K) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= M * N) return;
  const int64_t m = gid / N;
  const int n = static_cast<int>(gid - m * N);
  const float* a = A + m * K;
  const float* w = W + static_cast<int64_t>(n) * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(a[k], w[k], s);
  C[gid] = s;
}

}  // namespace

hipError_t launch_project_kv(const void* e, const void* w, int64_t n_tok, int64_t d_mem,
                             int64_t n_out, int in_dtype, int out_dtype, void* kv, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  if (in_dtype == ENGRAM_BF16) {
    const int tiles_m = static_cast<int>((n_tok + BM - 1) / BM);
    const int tiles_n = static_cast<int>((n_out + BN - 1) / BN);
    const dim3 grid(tiles_m * tiles_n);
    const auto* A = static_cast<const uint16_t*>(e);
    const auto* W = static_cast<const uint16_t*>(w);
    if (out_dtype == ENGRAM_BF16)
      launch_k(gemm_bf16_kernel<uint16_t>, grid, dim3(kThreads), 0, s, A, W,
                         static_cast<uint16_t*>(kv), n_tok, static_cast<int>(n_out),
                         static_cast<int>(d_mem), tiles_m, tiles_n);
    else
      launch_k(gemm_bf16_kernel<float>, grid, dim3(kThreads), 0, s, A, W,
                         static_cast<float*>(kv), n_tok, static_cast<int>(n_out),
                         static_cast<int>(d_mem), tiles_m, tiles_n);
  } else {
    const int64_t total = n_tok * n_out;
    launch_k(gemm_f32_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(e), static_cast<const float*>(w),
                       static_cast<float*>(kv), n_tok, static_cast<int>(n_out), static_cast<int>(d_mem));
  }
  return hipGetLastError();
}

}  // namespace engram
