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

}  // namespace

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
