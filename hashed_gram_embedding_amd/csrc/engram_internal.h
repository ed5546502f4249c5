// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libengram.so.  Not installed; the public interface is include/engram.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "engram.h"

namespace engram {

// Hash parameters by value: they travel in the kernel-argument segment.
struct HashArgs {
  uint64_t mult[ENGRAM_MAX_TABLES][ENGRAM_MAX_ORDER];  // per table j: m_{n,k,i}
  uint32_t prime[ENGRAM_MAX_TABLES];
  int32_t order[ENGRAM_MAX_TABLES];                    // n of table j
  int32_t n_tables;
  int32_t max_n;
};

struct TableArgs {
  int64_t row_offset[ENGRAM_MAX_TABLES];
  const void* rows;
  const float* scale;
  const int32_t* cache_slot;
  const void* cache_rows;
  const float* cache_scale;
  int32_t n_tables;
  int32_t dim;
  int32_t dtype;  // engram_dtype
};

struct GateConvArgs {
  int32_t d;
  int32_t branches;
  int32_t kernel_w;
  int32_t dilation;
  float eps;
  int32_t hdtype;   // storage of H
  int32_t kvdtype;  // storage of kv (F32 or BF16)
  const float* conv_w;
};

struct StateArgs {
  int32_t* ids;   // may be null (gate/conv-only call does not touch ids)
  float* conv;
  int32_t* pos;
};

hipError_t launch_hash(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                       const int32_t* proj, const HashArgs& a, int32_t* z, hipStream_t s);

hipError_t launch_gather(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype,
                         void* e, hipStream_t s);

hipError_t launch_project_kv(const void* e, const void* w, int64_t n_tok, int64_t d_mem,
                             int64_t n_out, int in_dtype, int out_dtype, void* kv, hipStream_t s);

// alpha[t][m] and gamma[t][m] = alpha / sqrt(alpha^2 mean(v^2) + eps) for every token.
hipError_t launch_gate(const void* H, const void* kv, int64_t n_tok, const GateConvArgs& g,
                       float* alpha, float* gamma, hipStream_t s);

// c = conv(gamma * v), Y = SiLU(c) + alpha v, H += Y.
hipError_t launch_conv(void* H, const void* kv, int64_t B, int64_t T, const GateConvArgs& g,
                       const float* alpha, const float* gamma, const StateArgs* st,
                       float* y_out, hipStream_t s);

// Writes the last conv inputs into the circular state, shifts ids (when
// tokens/proj are given) and advances pos.
hipError_t launch_state_commit(const void* kv, int64_t B, int64_t T, const GateConvArgs& g,
                               const float* gamma, const StateArgs& st, const int32_t* tokens,
                               const int32_t* proj, int32_t max_n, hipStream_t s);

}  // namespace engram
