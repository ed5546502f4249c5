// Steps 6-8 of "DeepSeek Engram series guide", section "Engram working
// principle", per branch m of the multi-branch variant:
//   alpha = sigmoid(RMSNorm(h) . RMSNorm(k) / sqrt(d)),  v~ = alpha v
//   u = RMSNorm(v~),  c_t = sum_j w[j] u_{t-(w-1-j)*dilation}   (depthwise, causal)
//   Y = SiLU(c) + v~,  H <- H + Y
//
// Two kernels, because H is updated in place while the conv of token t needs
// quantities of tokens up to (w-1)*dilation positions back:
//  * gate_kernel reads h, k and v of every token and writes two scalars per
//    (token, branch): alpha and gamma = alpha / sqrt(alpha^2 mean(v^2) + eps),
//    so that u = gamma * v.  One wavefront per (token, branch); lanes
//    accumulate sum h^2, k^2, h.k and v^2 over d and reduce by shuffles.
//  * conv_kernel rebuilds u at the taps from gamma and v, applies the conv,
//    SiLU and residual, and writes H.  It reads H only at the position it
//    writes, so the in-place update cannot race with another token's gate.
// A decode state supplies u for taps before the chunk (circular slots);
// state_commit_kernel writes the chunk's last conv inputs back afterwards.
#include "device_util.h"
#include "engram_internal.h"

namespace engram {
namespace {

template <int HT>
__device__ __forceinline__ void load8h(const void* base, int64_t off, float* f) {
  if constexpr (HT == ENGRAM_BF16) {
    unpack8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off), f);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

template <int HT>
__device__ __forceinline__ void store8h(void* base, int64_t off, const float* f) {
  if constexpr (HT == ENGRAM_BF16) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = pack8(f);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(f[0], f[1], f[2], f[3]);
    p[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
}

__device__ __forceinline__ void store8f(float* base, int64_t off, const float* f) {
  float4* p = reinterpret_cast<float4*>(base + off);
  p[0] = make_float4(f[0], f[1], f[2], f[3]);
  p[1] = make_float4(f[4], f[5], f[6], f[7]);
}

__device__ __forceinline__ void load8f(const float* base, int64_t off, float* f) {
  const float4* p = reinterpret_cast<const float4*>(base + off);
  const float4 a = p[0], b = p[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

template <int HT, int KT>
__global__ void __launch_bounds__(256)
gate_kernel(const void* __restrict__ H, const void* __restrict__ kv, int64_t n_tok, GateConvArgs g,
            float* __restrict__ alpha, float* __restrict__ gamma) {
  const int M = g.branches;
  const int d = g.d;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= n_tok * M) return;
  const int lane = threadIdx.x & 63;
  const int64_t t = pair / M;
  const int m = static_cast<int>(pair - t * M);
  const int64_t h_off = pair * d;
  const int64_t v_off = t * (1 + M) * d;
  const int64_t k_off = v_off + static_cast<int64_t>(1 + m) * d;
  float shh = 0.f, skk = 0.f, shk = 0.f, svv = 0.f;
  for (int c = lane; c < (d >> 3); c += 64) {
    float h[8], k[8], v[8];
    load8h<HT>(H, h_off + c * 8, h);
    load8h<KT>(kv, k_off + c * 8, k);
    load8h<KT>(kv, v_off + c * 8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      shh += h[i] * h[i];
      skk += k[i] * k[i];
      shk += h[i] * k[i];
      svv += v[i] * v[i];
    }
  }
  shh = wave_sum(shh);
  skk = wave_sum(skk);
  shk = wave_sum(shk);
  svv = wave_sum(svv);
  if (lane == 0) {
    const float inv_d = 1.0f / static_cast<float>(d);
    const float rh = 1.0f / sqrtf(shh * inv_d + g.eps);
    const float rk = 1.0f / sqrtf(skk * inv_d + g.eps);
    const float logit = shk * rh * rk / sqrtf(static_cast<float>(d));
    const float a = 1.0f / (1.0f + expf(-logit));
    alpha[pair] = a;
    gamma[pair] = a / sqrtf(a * a * (svv * inv_d) + g.eps);
  }
}

template <int HT, int KT>
__global__ void __launch_bounds__(256)
conv_kernel(void* __restrict__ H, const void* __restrict__ kv, int64_t B, int64_t T, GateConvArgs g,
            const float* __restrict__ alpha, const float* __restrict__ gamma, StateArgs st,
            int has_state, float* __restrict__ y_out) {
  const int M = g.branches;
  const int d = g.d;
  const int chunks = d >> 3;
  const int64_t total = B * T * M * chunks;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int c8 = static_cast<int>(gid % chunks);
  const int64_t pm = gid / chunks;
  const int m = static_cast<int>(pm % M);
  const int64_t bt = pm / M;
  const int64_t b = bt / T;
  const int64_t t = bt - b * T;
  const int span = (g.kernel_w - 1) * g.dilation;
  const int64_t row_kv = static_cast<int64_t>(1 + M) * d;
  const int ch0 = c8 * 8;
  const int32_t pos0 = has_state ? st.pos[b] : 0;

  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = 0.f;
  float vt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vt[i] = 0.f;
  for (int j = 0; j < g.kernel_w; ++j) {
    const int back = (g.kernel_w - 1 - j) * g.dilation;
    const int64_t s = t - back;
    float u[8];
    if (s >= 0) {
      const int64_t bs = b * T + s;
      load8h<KT>(kv, bs * row_kv + ch0, u);
      if (back == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) vt[i] = u[i];
      }
      const float gm = gamma[bs * M + m];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] *= gm;
    } else if (has_state) {
      int slot = static_cast<int>((static_cast<int64_t>(pos0) + s) % span);
      if (slot < 0) slot += span;
      load8f(st.conv, ((b * M + m) * span + slot) * static_cast<int64_t>(d) + ch0, u);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] += g.conv_w[(static_cast<int64_t>(m) * d + ch0 + i) * g.kernel_w + j] * u[i];
  }
  const float a = alpha[bt * M + m];
  float y[8], h[8];
  const int64_t h_off = pm * d + ch0;
  load8h<HT>(H, h_off, h);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[i] = c[i] / (1.0f + expf(-c[i])) + a * vt[i];
    h[i] += y[i];
  }
  store8h<HT>(H, h_off, h);
  if (y_out != nullptr) store8f(y_out, h_off, y);
}

template <int KT>
__global__ void __launch_bounds__(256)
state_commit_kernel(const void* __restrict__ kv, int64_t T, GateConvArgs g,
                    const float* __restrict__ gamma, StateArgs st, const int32_t* __restrict__ tokens,
                    const int32_t* __restrict__ proj, int32_t max_n) {
  const int64_t b = blockIdx.x;
  const int M = g.branches;
  const int d = g.d;
  const int chunks = d >> 3;
  const int span = (g.kernel_w - 1) * g.dilation;
  const int32_t pos0 = st.pos[b];
  const int L = static_cast<int>(T < span ? T : span);
  const int64_t row_kv = static_cast<int64_t>(1 + M) * d;
  const int total = M * L * chunks;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int c8 = idx % chunks;
    const int mq = idx / chunks;
    const int q = mq % L;
    const int m = mq / L;
    const int64_t p = T - L + q;
    const int slot = static_cast<int>((static_cast<int64_t>(pos0) + p) % span);
    const int64_t bs = b * T + p;
    float u[8];
    load8h<KT>(kv, bs * row_kv + c8 * 8, u);
    const float gm = gamma[bs * M + m];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] *= gm;
    store8f(st.conv, ((b * M + m) * span + slot) * static_cast<int64_t>(d) + c8 * 8, u);
  }
  if (threadIdx.x == 0 && st.ids != nullptr && tokens != nullptr) {
    const int hl = max_n - 1;
    int32_t old[ENGRAM_MAX_ORDER];
    for (int i = 0; i < hl; ++i) old[i] = st.ids[b * hl + i];
    for (int i = 0; i < hl; ++i) {
      const int64_t idx = T + i;  // index in (old ids ++ chunk ids)
      st.ids[b * hl + i] = idx < hl ? old[idx] : proj[tokens[b * T + idx - hl]];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) st.pos[b] = pos0 + static_cast<int32_t>(T);
}

}  // namespace

hipError_t launch_gate(const void* H, const void* kv, int64_t n_tok, const GateConvArgs& g,
                       float* alpha, float* gamma, hipStream_t s) {
  const int64_t pairs = n_tok * g.branches;
  if (pairs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((pairs + 3) / 4));
  const dim3 block(256);
  if (g.hdtype == ENGRAM_BF16 && g.kvdtype == ENGRAM_BF16)
    hipLaunchKernelGGL((gate_kernel<ENGRAM_BF16, ENGRAM_BF16>), grid, block, 0, s, H, kv, n_tok, g, alpha, gamma);
  else if (g.hdtype == ENGRAM_BF16)
    hipLaunchKernelGGL((gate_kernel<ENGRAM_BF16, ENGRAM_F32>), grid, block, 0, s, H, kv, n_tok, g, alpha, gamma);
  else
    hipLaunchKernelGGL((gate_kernel<ENGRAM_F32, ENGRAM_F32>), grid, block, 0, s, H, kv, n_tok, g, alpha, gamma);
  return hipGetLastError();
}

hipError_t launch_conv(void* H, const void* kv, int64_t B, int64_t T, const GateConvArgs& g,
                       const float* alpha, const float* gamma, const StateArgs* st,
                       float* y_out, hipStream_t s) {
  const int64_t total = B * T * g.branches * (g.d / 8);
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  const dim3 block(256);
  StateArgs sa{};
  if (st != nullptr) sa = *st;
  const int has = st != nullptr;
  if (g.hdtype == ENGRAM_BF16 && g.kvdtype == ENGRAM_BF16)
    hipLaunchKernelGGL((conv_kernel<ENGRAM_BF16, ENGRAM_BF16>), grid, block, 0, s, H, kv, B, T, g, alpha, gamma, sa,
                       has, y_out);
  else if (g.hdtype == ENGRAM_BF16)
    hipLaunchKernelGGL((conv_kernel<ENGRAM_BF16, ENGRAM_F32>), grid, block, 0, s, H, kv, B, T, g, alpha, gamma, sa,
                       has, y_out);
  else
    hipLaunchKernelGGL((conv_kernel<ENGRAM_F32, ENGRAM_F32>), grid, block, 0, s, H, kv, B, T, g, alpha, gamma, sa,
                       has, y_out);
  return hipGetLastError();
}

hipError_t launch_state_commit(const void* kv, int64_t B, int64_t T, const GateConvArgs& g,
                               const float* gamma, const StateArgs& st, const int32_t* tokens,
                               const int32_t* proj, int32_t max_n, hipStream_t s) {
  if (B == 0 || T == 0) return hipSuccess;
  if (g.kvdtype == ENGRAM_BF16)
    hipLaunchKernelGGL(state_commit_kernel<ENGRAM_BF16>, dim3(static_cast<unsigned>(B)), dim3(256), 0, s,
                       kv, T, g, gamma, st, tokens, proj, max_n);
  else
    hipLaunchKernelGGL(state_commit_kernel<ENGRAM_F32>, dim3(static_cast<unsigned>(B)), dim3(256), 0, s,
                       kv, T, g, gamma, st, tokens, proj, max_n);
  return hipGetLastError();
}

}  // namespace engram
