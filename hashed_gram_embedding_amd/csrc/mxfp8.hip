// MXFP8 quantisation of a matrix (the W of the FP8 projection).  Format and
// rounding as in device_util.h: E4M3 codes, one power-of-two scale per 32
// consecutive values of a row.  One thread quantises 8 values; the 4 threads
// of a block share its largest magnitude through lane shuffles.
#include "device_util.h"
#include "engram_internal.h"

namespace engram {
namespace {

template <int DT>
__global__ void __launch_bounds__(256)
mx_quantize_kernel(const void* __restrict__ x, int64_t n8, uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n8) return;   // n8 is a multiple of 4: whole blocks exit together
  float f[8];
  if constexpr (DT == ENGRAM_BF16) {
    unpack8(reinterpret_cast<const uint4*>(x)[gid], f);
  } else {
    const float4* p = reinterpret_cast<const float4*>(x) + gid * 2;
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  uint32_t sb;
  const uint2 w = mx_quantize8(f, &sb);
  reinterpret_cast<uint2*>(q)[gid] = w;
  if ((gid & 3) == 0) scale[gid >> 2] = static_cast<uint8_t>(sb);
}

// Fragment order of a 32-row block of W for v_mfma_scale_f32_32x32x64_f8f6f4
// (the A-operand layout the projection kernels read out of LDS): for K64
// step kk, lane l = 32h + r holds bytes 16h..16h+15 and 32+16h..32+16h+15 of
// row r's 64-byte run, and its operand scale is that of block 2kk + h.  The
// packed copy stores, per (block, step), the 64 lanes' 32 bytes one after the
// other, then per (block, group of four steps) one 32-bit word per lane with
// the lane's four scale bytes (byte s for step 4kq + s).  A wavefront then
// loads its operand for a step with two fully coalesced 16-byte loads.
// One thread per (block, step, lane) and, in the scale part, per (block,
// step group, lane).
__global__ void __launch_bounds__(256)
mx_pack_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ scale, int64_t rows, int cols,
               uint8_t* __restrict__ packed) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int kk_n = cols / 64;
  const int64_t n_frag = rows / 32 * kk_n * 64;   // fragment-lane slots
  const int64_t n_word = rows / 32 * (kk_n / 4) * 64;
  if (gid < n_frag) {
    const int lane = static_cast<int>(gid & 63);
    const int64_t rest = gid >> 6;
    const int kk = static_cast<int>(rest % kk_n);
    const int64_t row = rest / kk_n * 32 + (lane & 31);
    const int hh = lane >> 5;
    const uint8_t* src = q + row * cols + kk * 64 + hh * 16;
    uint4* dst = reinterpret_cast<uint4*>(packed + gid * 32);
    dst[0] = *reinterpret_cast<const uint4*>(src);
    dst[1] = *reinterpret_cast<const uint4*>(src + 32);
  } else if (gid < n_frag + n_word) {
    const int64_t w = gid - n_frag;
    const int lane = static_cast<int>(w & 63);
    const int64_t rest = w >> 6;
    const int kq = static_cast<int>(rest % (kk_n / 4));
    const int64_t row = rest / (kk_n / 4) * 32 + (lane & 31);
    const int hh = lane >> 5;
    const uint8_t* src = scale + row * (cols / 32) + kq * 8 + hh;   // block 2 * (4kq + s) + hh
    const uint32_t word = static_cast<uint32_t>(src[0]) | static_cast<uint32_t>(src[2]) << 8 |
                          static_cast<uint32_t>(src[4]) << 16 | static_cast<uint32_t>(src[6]) << 24;
    reinterpret_cast<uint32_t*>(packed + rows * cols)[w] = word;
  }
}

// bf16 W as A operands of v_mfma_f32_32x32x16_bf16: for 32-row block b and
// K16 step ks, lane l = 32h + r holds the 8 values of row 32b + r at columns
// 32(ks/2) + 16h + 8(ks%2) .. +7 (the halves of each 32-column group taken
// crosswise, as the gathered rows are).  One thread per (block, step, lane).
__global__ void __launch_bounds__(256)
bf16_pack_kernel(const uint16_t* __restrict__ w, int64_t rows, int cols, uint16_t* __restrict__ packed) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int ks_n = cols / 16;
  if (gid >= rows / 32 * ks_n * 64) return;
  const int lane = static_cast<int>(gid & 63);
  const int64_t rest = gid >> 6;
  const int ks = static_cast<int>(rest % ks_n);
  const int64_t row = rest / ks_n * 32 + (lane & 31);
  const int col = (ks >> 1) * 32 + (lane >> 5) * 16 + (ks & 1) * 8;
  reinterpret_cast<uint4*>(packed)[gid] = *reinterpret_cast<const uint4*>(w + row * cols + col);
}

}  // namespace

hipError_t launch_bf16_pack(const uint16_t* w, int64_t rows, int64_t cols, uint16_t* packed, hipStream_t s) {
  if (rows % 32 != 0 || cols % 32 != 0) return hipErrorInvalidValue;
  const int64_t n = rows / 32 * (cols / 16) * 64;
  if (n == 0) return hipSuccess;
  launch_k(bf16_pack_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, w, rows,
           static_cast<int>(cols), packed);
  return hipGetLastError();
}

hipError_t launch_mx_pack(const uint8_t* q, const uint8_t* scale, int64_t rows, int64_t cols, uint8_t* packed,
                          hipStream_t s) {
  if (rows % 32 != 0 || cols % 256 != 0) return hipErrorInvalidValue;
  const int64_t n = rows / 32 * (cols / 64) * 64 + rows / 32 * (cols / 256) * 64;
  if (n == 0) return hipSuccess;
  launch_k(mx_pack_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, q, scale, rows,
           static_cast<int>(cols), packed);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale,
                              hipStream_t s) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n8 + 255) / 256));
  if (dtype == ENGRAM_BF16)
    launch_k(mx_quantize_kernel<ENGRAM_BF16>, grid, dim3(256), 0, s, x, n8, q, scale);
  else
    launch_k(mx_quantize_kernel<ENGRAM_F32>, grid, dim3(256), 0, s, x, n8, q, scale);
  return hipGetLastError();
}

}  // namespace engram
