// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libengram.so.  Not installed; the public interface is include/engram.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "debug_checks.h"
#include "engram.h"

namespace engram {

// Hash parameters by value: they travel in the kernel-argument segment.
struct HashArgs {
  uint64_t mult[ENGRAM_MAX_TABLES][ENGRAM_MAX_ORDER];  // per table j: m_{n,k,i}; 0 for i >= n
  uint64_t inv[ENGRAM_MAX_TABLES];                     // floor((2^64-1) / p_j)
  uint32_t prime[ENGRAM_MAX_TABLES];
  int32_t order[ENGRAM_MAX_TABLES];                    // n of table j
  int32_t n_tables;
  int32_t max_n;
  int32_t vocab;                                       // raw ids are clamped into [0, vocab)
  uint32_t* err;                                       // debug build: the caller's error word, or null
};


struct TableArgs {
  int64_t row_offset[ENGRAM_MAX_TABLES];
  int32_t n_rows[ENGRAM_MAX_TABLES];   // rows of table j (debug build: row indices are checked against it)
  int64_t cache_n;                     // slots in the cache (debug build: slots are checked against it)
  uint32_t* err;                       // debug build: the caller's error word, or null
  const void* rows;
  const float* scale;
  const int32_t* cache_slot;
  const void* cache_rows;
  const float* cache_scale;
  uint32_t* counts;  // optional per-row access counts
  int32_t n_tables;
  int32_t dim;
  int32_t dtype;  // engram_dtype
};

// Engram-Nine hot tier of one order on the device.  A slot is 32 bytes:
// ids[4] with ids[i] = x'_{t-i} for i < n and 0 above, then the hot row,
// then padding.
struct HotOrderArgs {
  const uint32_t* pilots;  // [n_buckets]
  const uint4* slots;      // [n_hot][2]
  const void* rows;        // [n_hot][width]
  uint64_t seed;
  uint64_t n_hot;          // 0 = no hot tier for this order
  uint64_t n_buckets;
};

struct HotArgs {
  HotOrderArgs o[ENGRAM_MAX_ORDER - 1];  // order n at [n-2]
  int32_t width;                         // K * dim: columns of a hot row
  int32_t heads;                         // K
};

// Where the fused hash+gather reads its ids.
// What Steps 1-2 read: the token ids, P, the decode history (null = pad 0)
// and the window's shape, in one 48-byte block.
struct WindowSrc {
  const int32_t* tokens;
  const int32_t* proj;
  const int32_t* hist;
  uint32_t* err;   // debug build: the caller's error word, or null
  int32_t T;       // tokens per sequence (the batch below 2^31 tokens)
  int32_t max_n;
  int32_t vocab;
};

struct HashSrc {
  const int32_t* tokens;
  const int32_t* proj;
  const int32_t* hist;
  int64_t T;
  HashArgs a;
  HotArgs hot;  // used by the hot-tier variant only
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

hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q, uint8_t* scale,
                              hipStream_t s);
// MXFP8 W (codes [rows][cols], scales [rows][cols/32]) in the fragment order
// of the FP8 matrix cores; rows a multiple of 32, cols of 256.
hipError_t launch_mx_pack(const uint8_t* q, const uint8_t* scale, int64_t rows, int64_t cols, uint8_t* packed,
                          hipStream_t s);
// bf16 W [rows][cols] as A operands of v_mfma_f32_32x32x16_bf16, in the
// kGatherOutFrag16 order with row blocks for token blocks; rows a multiple of
// 32, cols of 32.
hipError_t launch_bf16_pack(const uint16_t* w, int64_t rows, int64_t cols, uint16_t* packed, hipStream_t s);

// Gather output in MXFP8: [n_tok][n_tables*dim] E4M3 codes followed by
// [n_tok][n_tables*dim/32] scale bytes (dim a multiple of 32).
constexpr int kGatherOutMXFP8 = 3;
// Gather output in bf16 as operands of v_mfma_f32_32x32x16_bf16 (the B
// side): for token block tb (32 tokens), K16 step ks and lane l = 32h + r,
// 16 bytes at lane slot (tb * K/16 + ks) * 64 + l hold the 8 values of token
// 32tb + r at columns 32(ks/2) + 16h + 8(ks%2) .. +7.  Within every 32-column
// group the two steps take the group's halves crosswise, so that one lane's
// two steps read 16 consecutive values of a row; W packs the same way
// (launch_bf16_pack), and the product is the same sum in another order.  K a
// multiple of 32; the last block is whole, its rows past the last token left
// unwritten.
constexpr int kGatherOutFrag16 = 4;

hipError_t launch_gather(const int32_t* z, int64_t n_tok, const TableArgs& ta, int out_dtype,
                         void* e, hipStream_t s);

// Steps 1-4 in one kernel: rows are addressed by indices hashed in-thread.
// hot: the Engram-Nine hot tier, or null for the cold lookup alone.
hipError_t launch_hash_gather(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                              const int32_t* proj, const HashArgs& a, const TableArgs& ta,
                              const HotArgs* hot, int out_dtype, void* e, hipStream_t s);

hipError_t launch_hot_lookup(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                             const int32_t* proj, int max_n, int32_t vocab, const HotArgs& h, int32_t* out,
                             uint32_t* err, hipStream_t s);

// Host build of one order's minimal perfect hash (pilots, and 8 int32 per
// slot: ids newest first, row, padding).  a, b name the n-grams behind a
// duplicate or a retry.
struct HotBuild {
  enum Status { kOk, kDuplicate, kRetry } status;
  uint32_t a, b;
};
HotBuild hot_build(const int32_t* keys, int64_t n_hot, int n, uint64_t seed, uint32_t* pilots, int32_t* slots);

hipError_t launch_project_kv(const void* e, const void* w, int64_t n_tok, int64_t d_mem,
                             int64_t n_out, int in_dtype, int out_dtype, void* kv, hipStream_t s);

// Fused bf16 projection + gate statistics (see proj_gate.hip).
struct ProjGateArgs {
  const uint16_t* e;  // [n_tok][K] bf16
  const uint16_t* w;  // [N][K] bf16, N = (1+M)*d
  const uint16_t* H;  // [n_tok][M][d] bf16 (read only)
  float* v;           // [n_tok][d]
  float4* stats;      // [n_tok][N/TF], TF = proj_gate_tile_f(n_tok, N, d, K, mx)
  int64_t n_tok;
  int K;
  int N;
  int d;
  int M;
  int tiles_f;  // set by the launcher
  int tiles_t;  // set by the launcher
  // MXFP8 product when non-NULL: e and w hold E4M3 codes ([n_tok][K], [N][K]
  // bytes) and these their block scale bytes ([n_tok][K/32], [N][K/32])
  const uint8_t* e_scale;
  const uint8_t* w_scale;
  // optional MXFP8 W in matrix-core fragment order (engram_pack_mxfp8): the
  // resident-token kernel streams it straight into registers
  const uint8_t* w_packed;
  // small-batch kernel only: store every column of the product here
  // ([n_tok][N] float32: v, then the keys) instead of v and the gate sums; H
  // is then not read
  float* kv_out;
  // with kv_out: W and e both in fragment order (launch_bf16_pack,
  // kGatherOutFrag16), for the register-operand decode product
  const uint16_t* w_frag;
  // Decode-state advance folded into this launch (adv_B > 0): workgroup 0
  // shifts the last N-1 compressed ids of every sequence's T = adv_T new
  // tokens into st_ids and adds adv_T to st_pos.  Nothing in the launch reads
  // them; the conv that follows knows pos has moved (ConvArgs.pos_advanced).
  int32_t* st_ids;        // [adv_B][max_n-1]
  int32_t* st_pos;        // [adv_B]
  const int32_t* tokens;  // [adv_B][adv_T] raw ids
  const int32_t* proj;    // P
  int32_t vocab;          // raw ids are clamped into [0, vocab)
  uint32_t* err;          // debug build: the caller's error word, or null
  int32_t max_n;
  int32_t adv_T;
  int32_t adv_B;
};
constexpr int kProjGateTileF = 64;   // narrowest feature tile (bounds the statistics buffer)
// Gate statistics per (token, branch) that the conv kernels take: the value
// tiles plus one branch's key tiles, qv + qk <= kConvMaxStats.
constexpr int kConvMaxStats = 64;
int proj_gate_tile_f(int64_t n_tok, int N, int d, int K, bool mx);   // feature columns per gate-statistics tile
bool proj_gate_small_for(int64_t n_tok, int N, int d, int K, bool mx);   // the small-batch kernel serves this product
// Gate statistics of a projection launch: qv tiles feed v.v; qk tiles per
// branch feed h.h, k.k, h.k (after the qv ones); mixed = every one of the
// qv tiles feeds all four sums (qk = 0).
struct ProjGateLayout {
  int tf;
  bool small;
  bool mixed;
  int qv;
  int qk;
};
ProjGateLayout proj_gate_layout(int64_t n_tok, int N, int d, int K, int M, bool mx);
hipError_t launch_proj_gate(const ProjGateArgs& a, hipStream_t s);
// Step 5 of up to two layers into float32 rows (ProjGateArgs.kv_out set on
// both) with the small-batch kernel, in one launch; hipErrorNotSupported
// (nothing launched) when a layer's size or format does not take that kernel
// or the two differ in format.  b may be null.  Layers with w_frag set take
// the fragment-operand kernel (both or neither of the two).
hipError_t launch_project_layers(const ProjGateArgs& a, const ProjGateArgs* b, hipStream_t s);
// Whether a float32 product of this size takes the fragment-operand kernel
// (bf16, K a multiple of 128 up to 1024, in the small-batch range).
bool proj_frag_for(int64_t n_tok, int N, int d, int K);
// The fragment-operand product of one or two layers of the same K
// (hipErrorNotSupported when a layer does not fit proj_frag_for).
hipError_t launch_project_frag(const ProjGateArgs& a, const ProjGateArgs* b, hipStream_t s);


// Whole-row gate statistics from given projections: stats [n_tok][1+M].
hipError_t launch_gate_stats(const void* H, const void* kv, int64_t n_tok, const GateConvArgs& g, float4* stats,
                             hipStream_t s);

struct ConvArgs {
  void* H;              // [B][T][M][d]
  const void* v;        // v rows, row stride v_stride elements
  int64_t v_stride;
  const float4* stats;  // [B*T][nq]: qv v tiles, then qk tiles per branch
  int qv;
  int qk;
  int nq;
  int mixed;            // each of the qv statistics also carries the key sums (qk = 0)
  int kq0;              // first statistic of a row that carries key sums: 0 when mixed, else qv
  int64_t B;
  int64_t T;
  GateConvArgs g;
  StateArgs st;
  int has_state;
  int pos_advanced;     // st.pos already holds pos + T (advanced by the projection launch)
  int commit_u;         // T = 1 strip conv: also write the new conv input u into the ring
  int sums_from_kv;     // T = 1 strip conv on float32 [v | k^(0..M-1)] rows (v_stride = (1+M)d, d <= 1024):
                        // the gate sums come from the rows themselves, stats is unused
  float* alpha_out;     // [B*T][M] or null
  float* gamma_out;     // [B*T][M] or null
  float* y_out;         // [B][T][M][d] or null
};
hipError_t launch_conv(const ConvArgs& a, int vdtype, hipStream_t s);
// Token strip of the conv launch_conv runs for a (1, 4 or 16), or 0 when it
// runs the LDS-tiled conv kernel instead.
int conv_strip_ts(const ConvArgs& a);

// A hashed gather (Steps 1-4) to run inside another launch.
struct GatherJob {
  TableArgs ta;
  HashSrc hs;
  void* e;
  uint32_t n_tok;
  int out_dtype;
  bool hot;  // a hot tier is attached (hs.hot)
};
// The strip conv of a with gj's gather in one launch; hipErrorNotSupported
// (nothing launched) when the pair has no fused form.
hipError_t launch_conv_gather(const ConvArgs& a, int vdtype, const GatherJob& gj, hipStream_t s);
// Two hashed gathers (no hot tier, one table and row format) in one launch;
// hipErrorNotSupported (nothing launched) otherwise.  The two jobs travel in
// the kernel-argument segment (about 4.4 KiB).
hipError_t launch_hash_gather2(const GatherJob& a, const GatherJob& b, hipStream_t s);

// Steps 1-5 of one layer in one launch: the fragment-operand product whose
// wavefronts hash and read their own table rows (g.out_dtype unused; no hot
// tier, cache or access counts).  p.e is unused.
struct AheadJob {
  // everything a workgroup reads, in the first 128 bytes (two scalar
  // loads, in flight together): copies of fields of g and p
  struct Head {
    const int32_t* tokens;
    const int32_t* proj;
    const int32_t* hist;
    const uint16_t* w_frag;
    const void* rows;
    const float* scale;
    float* kv_out;
    int32_t* st_ids;
    int32_t* st_pos;
    uint32_t* err;
    int32_t T;
    int32_t max_n;
    int32_t vocab;
    int32_t n_tok;
    int32_t N;
    int32_t tiles_f;
    int32_t has_state;   // advance the decode state (T = 1)
    uint32_t slot;       // the layer's first arrival count
    int64_t pad[2];
  } head;
  GatherJob g;
  ProjGateArgs p;
};
// Whether layer products with these tables take launch_ahead_fused: a
// fragment-operand product with K = 512 or 1024, table dim 32, 64 or 128,
// int8 or bf16 rows.
bool ahead_fused_for(const TableArgs& ta, int64_t n_tok, int N, int d, int K);
// One or two layers (same K and table dtype; b may be null).  A launch that
// advances decode states (T = 1, up to 2048 sequences) has the last
// workgroup of each token tile to finish its reads do that tile's advance,
// counted in device-global arrival slots; calls that run concurrently on one
// device take different slots (blocks of a ring of kAheadSlots, taken in
// turn: 64 launches may be in flight at once).
constexpr int kAheadSlots = 4096;
hipError_t launch_ahead_fused(const AheadJob& a, const AheadJob* b, hipStream_t s);

// Writes the chunk's last conv inputs into the circular state, shifts ids
// (when tokens/proj are given) and advances pos.
hipError_t launch_state_commit(const void* v, int64_t v_stride, int vdtype, int64_t B, int64_t T,
                               const GateConvArgs& g, const float* gamma, const StateArgs& st,
                               const int32_t* tokens, const int32_t* proj, int32_t max_n, int32_t vocab,
                               uint32_t* err, hipStream_t s);

size_t cache_build_workspace(int64_t total_rows);
size_t cache_update_workspace(int64_t total_rows, int64_t cache_n);
hipError_t launch_cache_update(const TableArgs& ta, int64_t total_rows, int row_bytes, int64_t cache_n,
                               int32_t* cache_slot, void* cache_rows, float* cache_scale, uint32_t* counts,
                               int decay_shift, void* ws, hipStream_t s);
hipError_t launch_cache_build(const int32_t* tokens, int64_t B, int64_t T, const int32_t* proj, const HashArgs& ha,
                              const TableArgs& ta, int64_t total_rows, int row_bytes, int64_t cache_n,
                              int32_t* cache_slot, void* cache_rows, float* cache_scale, void* ws, hipStream_t s);

// Benchmark stage timing: after the library opens a named stage, the next
// kernel launched through launch_k records start and stop events in its own
// dispatch packet (hipExtLaunchKernel), so a stage's time is that kernel's
// execution and not the gaps around it.  prof_take hands out the open stage's
// events (false when no stage is open).
bool prof_take(hipEvent_t* start, hipEvent_t* stop);

template <typename F, typename... Args>
inline void launch_k(F kernel, const dim3& grid, const dim3& block, uint32_t lds, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  if (prof_take(&e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

}  // namespace engram
