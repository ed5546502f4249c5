/*
 * engram.h -- C ABI of libengram.so: the Engram conditional-memory layer
 * (hashed n-gram embeddings) on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "DeepSeek Engram series guide" (foosynaptic
 * deepseek-tech-notes), section "Engram working principle", Steps 1-8, and
 * its multi-branch variant.  Per token position t:
 *   x'_t = P(x_t)                                     (Step 1)
 *   g_{t,n} = (x'_{t-n+1}, ..., x'_t), n = 2..N       (Step 2)
 *   z_{t,n,k} = (XOR_i x'_{t-i} m_{n,k,i} mod 2^64) mod p_{n,k}   (Step 3)
 *   e_t = concat_{n outer, k inner} E_{n,k}[z_{t,n,k}]            (Step 4)
 *   v_t = W_V e_t, k_t^(m) = W_K^(m) e_t              (Step 5, variant)
 *   alpha_t^(m) = sigmoid(RMSNorm(h_t^(m)) . RMSNorm(k_t^(m)) / sqrt(d))  (Step 6)
 *   Y^(m) = SiLU(Conv1D(RMSNorm(alpha^(m) V))) + alpha^(m) V   (Step 7)
 *   H^(m) <- H^(m) + Y^(m)                            (Step 8)
 * The pages leave the hash function open; this library fixes the
 * multiplicative-XOR form above, with ids before the sequence start read as
 * 0 (or from the decode history).
 *
 * Conventions shared by every call:
 *  - "device" pointers are HIP device memory (or, where stated, the device
 *    alias of mapped pinned host memory); "host" pointers are read on the
 *    host during the call only.  The caller owns every buffer; the library
 *    keeps no pointer after a call returns and allocates no device memory
 *    (scratch comes in through `ws`; engram_forward_noalloc uses a scratch
 *    array of the library's code instead).
 *  - Every compute call is asynchronous on `stream` (0 = the null stream)
 *    and never synchronises.  Calls are reentrant; calls that write the same
 *    buffers must be ordered by the caller.
 *  - All argument checks that need only host-visible values run before any
 *    launch; on failure nothing is launched and a message is kept for
 *    engram_last_error() (per calling thread).  Device-resident values are
 *    the caller's contract: 0 <= token < vocab, 0 <= z < n_rows[j],
 *    -1 <= cache slots < cache_n (the debug build checks them; see
 *    engram_debug_checks).
 *  - Status codes: ENGRAM_OK, ENGRAM_EINVAL (null or misaligned pointer, bad
 *    size, inconsistent descriptors, workspace too small),
 *    ENGRAM_EUNSUPPORTED (dtype combination or shape outside the supported
 *    set), ENGRAM_EHIP (a HIP runtime or launch error; its text is in
 *    engram_last_error()).
 *  - bf16 is IEEE bfloat16; every rounding to it is to nearest, ties to even.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENGRAM_ABI_VERSION 6
#define ENGRAM_MAX_TABLES 32 /* (N-1)*K */
#define ENGRAM_MAX_ORDER 4   /* N */
#define ENGRAM_MAX_KERNEL_W 8
#define ENGRAM_MAX_CONV_SPAN 24 /* (kernel_w - 1) * dilation */
#define ENGRAM_MAX_D 65536      /* d, hidden width per branch */
#define ENGRAM_MAX_BRANCHES 64  /* M */

typedef enum engram_status {
  ENGRAM_OK = 0,
  ENGRAM_EINVAL = -1,
  ENGRAM_EUNSUPPORTED = -2,
  ENGRAM_EHIP = -3
} engram_status;

typedef enum engram_dtype {
  ENGRAM_F32 = 0,
  ENGRAM_BF16 = 1,
  ENGRAM_I8 = 2 /* table rows only: int8 with one float32 scale per row */
} engram_dtype;

/* Steps 1-3: vocabulary projection and the multi-head hash. */
typedef struct engram_hash_params {
  const int32_t* proj;    /* device [vocab]: P, raw id -> compressed id        */
  int64_t vocab;          /* raw vocabulary size                               */
  int32_t max_n;          /* N: n-gram orders 2..N, 2 <= N <= ENGRAM_MAX_ORDER */
  int32_t heads;          /* K heads per order, (N-1)*K <= ENGRAM_MAX_TABLES   */
  const uint64_t* mult;   /* host [N-1][K][N]: m_{n,k,i} at [n-2][k][i]; i = 0
                             multiplies the current token; entries i >= n are
                             unused                                            */
  const uint32_t* prime;  /* host [(N-1)*K]: table size p_{n,k} of table
                             j = (n-2)*K + k, 2 <= p < 2^31                     */
} engram_hash_params;

/* Steps 3-4: the prime-sized tables E_j, j = (n-2)*K + k, stored back to back
 * in one row array.  Low-precision storage with dequantisation inside the
 * gather follows the mixed-precision direction of "Engram module: ..."
 * (section 8) and the single select-and-dequantise kernel that reads either
 * HBM or pinned host memory ("Engram embedding expansion: co-design for
 * DRAM/SSD offload", section on DRAM offload). */
typedef struct engram_tables {
  int32_t n_tables;          /* = (N-1)*K                                        */
  int32_t dim;               /* columns per row (d_head), a multiple of 8        */
  engram_dtype dtype;        /* ENGRAM_F32, ENGRAM_BF16 or ENGRAM_I8             */
  const void* rows;          /* [total_rows][dim], 16-byte aligned: device memory
                                or the device alias of mapped pinned host memory
                                (engram_host_alloc)                              */
  const int64_t* row_offset; /* host [n_tables]: first row of table j in `rows`  */
  const int64_t* n_rows;     /* host [n_tables]: rows of table j; must equal p_j */
  int64_t total_rows;        /* rows in `rows`; every table must fit inside      */
  const float* row_scale;    /* [total_rows], same memory kind as rows; I8 only  */
  /* optional hot cache in HBM, checked first (NULL cache_slot = none): */
  const int32_t* cache_slot; /* device [total_rows]: cache slot of a row, or -1  */
  const void* cache_rows;    /* device [cache_n][dim], same dtype as rows        */
  const float* cache_scale;  /* device [cache_n]; I8 only                        */
  int64_t cache_n;           /* slots in the cache                               */
  /* optional access statistics for the real-time LFU cache (NULL = none):
     every gather through these tables adds 1 to the count of each row it
     reads (global row, before the cache probe; one atomic add per access) */
  uint32_t* access_counts;   /* device [total_rows]                              */
} engram_tables;

/* Steps 6-8: gate, short conv and residual. */
typedef struct engram_gate_conv_params {
  int32_t d;              /* hidden width per branch, a multiple of 64, <= ENGRAM_MAX_D */
  int32_t branches;       /* M residual branches, 1..ENGRAM_MAX_BRANCHES            */
  int32_t kernel_w;       /* conv taps w, 1..ENGRAM_MAX_KERNEL_W (pages: 4)         */
  int32_t dilation;       /* conv dilation (pages: N); (w-1)*dilation <= 24         */
  float eps;              /* RMSNorm epsilon                                       */
  engram_dtype hdtype;    /* ENGRAM_F32 or ENGRAM_BF16: storage type of H, kv, the
                             projection weights and the gathered rows              */
  const float* conv_w;    /* device [M][d][kernel_w]; tap kernel_w-1 multiplies the
                             current position, tap j the position
                             (kernel_w-1-j)*dilation steps back                     */
} engram_gate_conv_params;

/* Engram-Nine hot tier ("DeepSeek Engram series guide", experiment 3
 * "Engram-Nine", Figure 1: two-tier retrieval).  Per order n an optional set
 * of hot n-grams (the most frequent ones), each with a row of its own of
 * width K*dim.  A hot n-gram g_{t,n} takes its row for the K heads of order
 * n, columns (n-2)*K*dim .. (n-1)*K*dim - 1 of e_t; every other n-gram keeps
 * the K-head cold lookup of Steps 3-4.  The set is indexed by a minimal
 * perfect hash and every slot keeps its whole n-gram as the fingerprint, so
 * a lookup is exact: an n-gram outside the set is never taken for a hot one.
 *
 * The hash (hash-and-displace with one pilot per bucket, after PTHash,
 * Pibiri and Trani, SIGIR 2021), for an n-gram with ids x_i = x'_{t-i}:
 *   mix(v)  = the SplitMix64 finaliser: v ^= v >> 30; v *= 0xbf58476d1ce4e5b9;
 *             v ^= v >> 27; v *= 0x94d049bb133111eb; v ^= v >> 31
 *   h       = mix(seed ^ n), then h = mix(h ^ x_i) for i = 0, 1, .., n-1
 *   range(a, r) = floor(a * r / 2^64)
 *   bucket  = range(h, engram_hot_buckets(n_hot))
 *   slot    = range(mix(h ^ mix(pilots[bucket] + 1)), n_hot)
 * and g_{t,n} is hot, with row slots[slot].row, iff slots[slot].ids equals
 * (x_0, .., x_{n-1}, 0, ..). */
typedef struct engram_hot_slot {
  int32_t ids[ENGRAM_MAX_ORDER]; /* ids[i] = x'_{t-i} for i < n (newest first), 0 above */
  int32_t row;                   /* the n-gram's row in engram_hot_tier.rows             */
  int32_t reserved[3];           /* 0                                                    */
} engram_hot_slot;               /* 32 bytes                                             */

typedef struct engram_hot_tier {
  int64_t n_hot[ENGRAM_MAX_ORDER - 1];                /* hot n-grams of order n at [n-2],
                                                         0..2^31-1; 0 = no hot tier for n */
  uint64_t seed[ENGRAM_MAX_ORDER - 1];                /* seed_used of engram_hot_build     */
  const uint32_t* pilots[ENGRAM_MAX_ORDER - 1];       /* device [engram_hot_buckets(n_hot)]*/
  const engram_hot_slot* slots[ENGRAM_MAX_ORDER - 1]; /* device [n_hot], 32-byte aligned   */
  const void* rows[ENGRAM_MAX_ORDER - 1];             /* device [*][K*dim] of the cold
                                                         tables' dtype (F32 or BF16),
                                                         16-byte aligned                  */
} engram_hot_tier;

/* One Engram layer. */
typedef struct engram_layer {
  engram_hash_params hash;
  engram_tables tables;
  const void* w;          /* device [(1+M)*d][n_tables*dim], hdtype, row-major:
                             rows 0..d-1 are W_V, rows (1+m)*d .. (2+m)*d-1 are
                             W_K^(m) (Step 5; the multi-branch variant fuses the
                             shared W_V with the M keys into one product)          */
  engram_gate_conv_params gc;
  /* optional MXFP8 Step 5 (the Guide's multi-branch variant suggests one FP8
     dense GEMM for W_V and the M keys): W in MXFP8 from engram_quantize_mxfp8
     of w.  When both are set (bf16 layers, tables with dim a multiple of 32,
     n_tables*dim a multiple of 128), the gathered rows are quantised to
     MXFP8 in the gather and the product runs on the FP8 matrix cores with
     per-block scales; NULL = bf16 product.                                      */
  const uint8_t* w_mx;        /* device [(1+M)*d][n_tables*dim] E4M3 codes        */
  const uint8_t* w_mx_scale;  /* device [(1+M)*d][n_tables*dim/32] scale bytes    */
  /* optional (NULL = none; needs w_mx): the same MXFP8 W in matrix-core
     fragment order from engram_pack_mxfp8, 16-byte aligned.  Multi-branch
     layers (M >= 2) with d a multiple of 256 and n_tables*dim a multiple of
     256 up to 1024 then run the product, at enough tokens, with each
     workgroup's token rows held on chip while W streams past them; results
     are identical to those without it.                                       */
  const uint8_t* w_mx_packed;
  /* optional (NULL = none; bf16 layers): w in matrix-core fragment order from
     engram_pack_bf16, 16-byte aligned.  Read only by engram_project_ahead,
     whose bf16 products with n_tables*dim a multiple of 128 up to 1024 then
     load both operands straight into registers; the float32 results agree
     with those without it to rounding (the sums run in another order).        */
  const void* w_packed;
  /* optional Engram-Nine hot tier (read on the host during each call; NULL =
     none): used by engram_forward and engram_retrieve.  Needs F32 or BF16
     tables; a hot hit reads no cold row and counts no access.                  */
  const engram_hot_tier* hot;
} engram_layer;

/* Decode / chunked-prefill state of S sequences (not on the pages; it is
 * what the causal n-gram window and conv need to continue a sequence). */
typedef struct engram_decode_state {
  int32_t* ids;   /* device [S][N-1]: compressed ids of the last N-1 tokens,
                     oldest first (0 = pad before the start)                   */
  float* conv;    /* device [S][M][span][d], span = (kernel_w-1)*dilation: the
                     conv inputs u = RMSNorm(alpha v) of the last span
                     positions; absolute position p lives in slot p % span;
                     zero-initialised for a new sequence                       */
  int32_t* pos;   /* device [S]: tokens consumed so far                        */
} engram_decode_state;

/* Library identity and per-thread error text. */
int32_t engram_abi_version(void);
const char* engram_last_error(void);

/* Steps 1-3.  tokens: device int32 [B][T] raw ids.  hist: device int32
 * [B][N-1] compressed ids preceding t = 0 (oldest first) or NULL for pad 0.
 * z: device int32 [B][T][(N-1)*K], z[b][t][j] = local row in table j.
 * B*T = 0 is a no-op. */
engram_status engram_hash_indices(const int32_t* tokens, int64_t B, int64_t T,
                                  const int32_t* hist, const engram_hash_params* hp,
                                  int32_t* z, hipStream_t stream);

/* Steps 3-4.  z: device int32 [n_tok][n_tables].  e: device
 * [n_tok][n_tables*dim] of out_dtype (F32 or BF16).  Rows are copied exactly
 * (f32 -> bf16 rounds to nearest even); I8 rows become
 * float32(q) * float32(scale), then rounded when out_dtype is BF16.  With a
 * cache, a row whose cache_slot is >= 0 is read from cache_rows, otherwise
 * from rows; the result is identical either way. */
engram_status engram_gather(const int32_t* z, int64_t n_tok, const engram_tables* tab,
                            engram_dtype out_dtype, void* e, hipStream_t stream);

/* Step 5.  kv[t][o] = sum_c e[t][c] * w[o][c] with float32 accumulation.
 * e: device [n_tok][d_mem], w: device [n_out][d_mem], kv: device
 * [n_tok][n_out], all of `dtype` (F32, or BF16 with d_mem and n_out
 * multiples of 64). */
engram_status engram_project_kv(const void* e, const void* w, int64_t n_tok, int64_t d_mem,
                                int64_t n_out, engram_dtype dtype, void* kv,
                                hipStream_t stream);

/* Steps 6-8 on precomputed projections.  H: device [B][T][M][d] (hdtype),
 * read as h and overwritten with h + Y (T < 2^31, B <= 65535).  kv: device [B][T][(1+M)*d]
 * (hdtype): v, then k^(0..M-1).  st: NULL for independent sequences starting
 * at t = 0; otherwise B = S sequences continuing from st, which is advanced
 * by T tokens (its ids are left for engram_forward to update: here no tokens
 * are seen, so st->ids and st->pos are read-only).  alpha_out: device float
 * [B][T][M] or NULL.  y_out: device float [B][T][M][d] or NULL.  ws: device
 * scratch of at least engram_gate_conv_workspace() bytes, 256-byte aligned. */
size_t engram_gate_conv_workspace(int64_t B, int64_t T, const engram_gate_conv_params* p);
engram_status engram_gate_conv_forward(void* H, const void* kv, int64_t B, int64_t T,
                                       const engram_gate_conv_params* p,
                                       engram_decode_state* st, float* alpha_out,
                                       float* y_out, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Steps 1-8 for one layer.  tokens: device int32 [B][T]; H: device
 * [B][T][M][d] updated in place (T < 2^31, B <= 65535, and B*T < 2^31 for
 * the hashed gather: ENGRAM_EUNSUPPORTED otherwise).  st: as for engram_gate_conv_forward; when
 * given, the hash reads st->ids as the history and the state (ids, conv,
 * pos) is advanced by T tokens.  alpha_out / y_out as above.  ws: device
 * scratch of at least engram_forward_workspace() bytes, 256-byte aligned. */
size_t engram_forward_workspace(int64_t B, int64_t T, const engram_layer* L);
engram_status engram_forward(const int32_t* tokens, void* H, int64_t B, int64_t T,
                             const engram_layer* L, engram_decode_state* st,
                             float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* engram_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same layer, the same kernels and the same results bit for bit, with
 * the workspace taken from scratch memory that the library holds, one array
 * of ENGRAM_NOALLOC_SCRATCH_BYTES per GPU, created with the library's code on
 * that GPU and kept until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); the caller still passes
 * tokens, H, the layer's memory and the optional outputs.  Nothing in the
 * scratch needs to start at zero: every call writes what it reads there.
 * Calls that overlap on one GPU (on different streams, or from several
 * threads without ordering) share that GPU's scratch and race; order them.
 * EINVAL when the call needs more than ENGRAM_NOALLOC_SCRATCH_BYTES of
 * workspace (engram_forward_workspace(B, T, L) above it: 4,096 tokens of a
 * single-branch d = 1024 layer need 26 MiB); other arguments as for
 * engram_forward. */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (32u << 20)
engram_status engram_forward_noalloc(const int32_t* tokens, void* H, int64_t B, int64_t T,
                                     const engram_layer* L, engram_decode_state* st,
                                     float* alpha_out, float* y_out, hipStream_t stream);

/* The layer in two halves, so that retrieval can run ahead of the hidden
 * states.  Steps 1-4 depend on the token ids alone (and, in decode, on the
 * state's id history), which is why the RecSDK article runs this sparse
 * retrieval asynchronously as an embedding prefetch that hides the lookup
 * (cache prefetch section) and the DRAM offload study fetches the rows while
 * the preceding layers compute (DRAM offload section).
 *
 * engram_retrieve: Steps 1-4 into e (B*T < 2^31), device [B*T][n_tables*dim] of the
 * layer's hdtype, 16-byte aligned, owned by the caller (for an MXFP8 layer:
 * [B*T][n_tables*dim] E4M3 codes followed by [B*T][n_tables*dim/32] scale
 * bytes).  st: NULL, or the
 * decode state whose ids are the history (read only; with a state, call it
 * after the previous forward on those sequences has committed).
 *
 * engram_forward_retrieved: Steps 5-8 on e from engram_retrieve with the same
 * tokens, B, T and state; arguments otherwise as engram_forward (tokens may be
 * NULL when st is NULL).  ws: at least engram_forward_retrieved_workspace()
 * bytes, 256-byte aligned.  engram_forward equals engram_retrieve followed by
 * engram_forward_retrieved on one stream. */
engram_status engram_retrieve(const int32_t* tokens, int64_t B, int64_t T, const engram_layer* L,
                              const engram_decode_state* st, void* e, hipStream_t stream);
size_t engram_forward_retrieved_workspace(int64_t B, int64_t T, const engram_layer* L);
engram_status engram_forward_retrieved(const int32_t* tokens, const void* e, void* H, int64_t B,
                                       int64_t T, const engram_layer* L, engram_decode_state* st,
                                       float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Steps 5-8 of one layer call and the next retrieval (Steps 1-4) in the same
 * launches: the prefetch of the next embeddings behind the current
 * computation that the RecSDK article (cache prefetch section) and the DRAM
 * offload study (DRAM offload section) describe.  The next retrieval is that
 * of next_L (NULL = L) over next_tokens [next_B][next_T], with next_st's ids
 * as its history (NULL = pad 0): the same layer's next batch, or the next
 * layer's rows of the same tokens (in decode, with that layer's state).  The
 * results are those of engram_forward_retrieved(tokens, e, H, B, T, L, st,
 * alpha_out, y_out, ws, ws_bytes) followed by engram_retrieve(next_tokens,
 * next_B, next_T, next_L, next_st, next_e), bit for bit; where the layers
 * allow it (L: bf16 H with the fused projection, w = 4 and dilation 3;
 * next_L: bf16 or int8 tables, no hot tier) the next gather runs inside this
 * call's conv launch, so that the two memory-latency-bound kernels share the
 * CUs.  st: as for engram_forward_retrieved (advanced by T tokens).  next_st:
 * read only, must not be st.  next_e: device, laid out as e of
 * engram_retrieve for next_L, 16-byte aligned, not overlapping e;
 * next_B * next_T = 0 skips the prefetch, B * T = 0 leaves only it.  ws as for
 * engram_forward_retrieved. */
engram_status engram_forward_retrieved_prefetch(const int32_t* tokens, const void* e, void* H, int64_t B,
                                                int64_t T, const engram_layer* L, engram_decode_state* st,
                                                float* alpha_out, float* y_out, void* ws, size_t ws_bytes,
                                                const engram_layer* next_L, const engram_decode_state* next_st,
                                                const int32_t* next_tokens, int64_t next_B, int64_t next_T,
                                                void* next_e, hipStream_t stream);

/* Step 5 ahead of the hidden states as well.  Steps 1-5 read the token ids
 * (and the decode history) alone: v = W_V e and k^(m) = W_K^(m) e ("DeepSeek
 * Engram series guide", Step 5 and its multi-branch variant) do not depend on
 * h, which first enters at Step 6's gate.  So a caller can run Steps 1-5 of
 * several layers together as soon as the tokens are known (a decode step's
 * sampled token), as the retrieval-ahead calls above do for Steps 1-4, and
 * run each layer's Steps 6-8 when its hidden state arrives.
 *
 * engram_project_ahead: Steps 1-5 of n_layers layers (1 <= n_layers <=
 * ENGRAM_MAX_AHEAD_LAYERS) over the same tokens [B][T] into kv[l], device
 * float32 [B*T][(1+M_l)*d_l], 16-byte aligned, owned by the caller: v, then
 * k^(0..M-1) (the product in float32, unrounded).  layers[l]: bf16 H layers
 * with the fused projection (d a multiple of 128 up to 4096); with states
 * (states[l] non-NULL for every layer, with ids), T must be 1 and each
 * state's ids and pos advance by that token here, so that the matching
 * engram_forward_projected reads them as advanced.  Layers go in pairs, in
 * the small-batch range (n_tok*(1+M)*d within it, which a decode batch of a
 * few hundred sequences is): with w_packed, int8 or bf16 tables of dim 32, 64
 * or 128 (n_tables*dim = 512 or 1024), no HBM cache and no access counts,
 * and at most 2048 sequences when states advance, one launch does both
 * layers' Steps 1-5; otherwise one launch gathers both layers' rows and one
 * multiplies both.  Larger bf16 products without states run the general
 * product per layer; larger ones with states, or MXFP8 ones, are
 * ENGRAM_EUNSUPPORTED.  The one-launch form advances states through
 * arrival counts in a device-global ring: calls with states may overlap on
 * one device (other streams, several graphs) up to 32 at a time.  ws: at
 * least engram_project_ahead_workspace() bytes, 256-byte aligned (the
 * gathered rows).
 *
 * engram_forward_projected: Steps 6-8 of layer L on kv from
 * engram_project_ahead with the same B, T and state; H as for engram_forward
 * (updated in place), alpha_out / y_out as there.  With st (T = 1) the conv
 * reads the state's ring at the advanced pos and writes the new conv input
 * into it.  For T = 1 and d <= 1024 one launch forms the gate's sums and runs
 * the conv; otherwise (no state) a gate-statistics launch comes first.  The
 * gate's sums are then formed over whole rows, so results agree with
 * engram_forward's to rounding, not bit for bit.  ws: at least
 * engram_forward_projected_workspace() bytes, 256-byte aligned. */
#define ENGRAM_MAX_AHEAD_LAYERS 8
size_t engram_project_ahead_workspace(int64_t B, int64_t T, int32_t n_layers, const engram_layer* const* layers);
engram_status engram_project_ahead(const int32_t* tokens, int64_t B, int64_t T, int32_t n_layers,
                                   const engram_layer* const* layers, engram_decode_state* const* states,
                                   float* const* kv, void* ws, size_t ws_bytes, hipStream_t stream);
size_t engram_forward_projected_workspace(int64_t B, int64_t T, const engram_layer* L);
engram_status engram_forward_projected(const float* kv, void* H, int64_t B, int64_t T, const engram_layer* L,
                                       engram_decode_state* st, float* alpha_out, float* y_out, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/* Static LFU admission for the HBM hot-row cache (Ascend RecSDK Engram
 * article, multi-level cache: hot rows by access frequency in fast memory,
 * the full table in host DRAM).  Counts how often each row of `tab` is
 * addressed by the warm-up tokens (device int32 [B][T], hashed like the
 * layer with pad-0 starts), admits the cache_n most frequently addressed rows
 * (ties: lower global row first) and writes
 *   cache_slot  device int32 [total_rows]: slot of an admitted row, else -1;
 *               admitted rows take slots 0..cache_n-1 in ascending row order
 *   cache_rows  device [cache_n][dim] of tab->dtype: copies of those rows
 *   cache_scale device float [cache_n] (I8 only): their scales.
 * tab->rows may be mapped host memory; tab's own cache fields are ignored.
 * Asynchronous.  The ranking is exact while the admission threshold count is
 * below 2^20 - 1 (rows counted 2^20 - 1 times or more rank as equals).
 * ws: engram_cache_build_workspace() bytes, 256-byte aligned. */
size_t engram_cache_build_workspace(int64_t total_rows);
engram_status engram_cache_build(const int32_t* warm_tokens, int64_t B, int64_t T,
                                 const engram_hash_params* hp, const engram_tables* tab,
                                 int64_t cache_n, int32_t* cache_slot, void* cache_rows,
                                 float* cache_scale, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Real-time LFU update of the hot cache between steps: the RecSDK article
 * keeps the hot cache current from access-frequency statistics, with LFU
 * admission and eviction (multi-level cache section, real-time update).
 * counts: device [total_rows], the access_counts the gathers accumulated.
 * The cache_n rows with the highest counts are admitted (ties: lower global
 * row first; exact while the threshold count is below 2^20 - 1).  Cached rows
 * that stay keep their slots; cached rows that are no longer admitted get
 * slot -1; newly admitted rows, in ascending row order, take the free slots
 * in ascending slot order, and only their rows (and int8 scales) are copied
 * from tab->rows (HBM or mapped host memory).  Afterwards every count is
 * shifted right by decay_shift (0..31; 0 keeps the counts).  cache_slot,
 * cache_rows and cache_scale are the cache being updated (as returned by
 * engram_cache_build or a previous update; tab's own cache fields are
 * ignored).  Asynchronous; must not overlap a gather that reads the cache.
 * ws: engram_cache_update_workspace() bytes, 256-byte aligned. */
size_t engram_cache_update_workspace(int64_t total_rows, int64_t cache_n);
engram_status engram_cache_update(const engram_tables* tab, int64_t cache_n, int32_t* cache_slot,
                                  void* cache_rows, float* cache_scale, uint32_t* counts,
                                  int32_t decay_shift, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* MXFP8 quantisation (used for W of the FP8 product): x [rows][cols] (F32 or
 * BF16 on the device, cols a multiple of 32) -> q [rows][cols] E4M3 codes and
 * scale [rows][cols/32] biased-exponent bytes.  Blocks are 32 consecutive
 * values of a row; the scale is the smallest power of two keeping the block's
 * largest magnitude within 448 (E4M3's largest finite value), elements are
 * x / scale rounded to nearest-even E4M3, an all-zero block has scale byte 0. */
engram_status engram_quantize_mxfp8(const void* x, engram_dtype dtype, int64_t rows, int64_t cols,
                                    uint8_t* q, uint8_t* scale, hipStream_t stream);

/* The MXFP8 W of engram_quantize_mxfp8 (q [rows][cols] codes, scale
 * [rows][cols/32] bytes, device) rearranged into the operand order of the FP8
 * matrix cores, for engram_layer.w_mx_packed: packed (device, 16-byte
 * aligned, rows*cols + rows*cols/32 bytes, owned by the caller) holds, for
 * each 32-row block b and K64 step kk, 64 lane slots of 32 bytes (lane
 * l = 32h + r: bytes 64kk+16h .. +15 and 64kk+32+16h .. +15 of row 32b + r),
 * then, for each block b and group kq of four steps, 64 lane words whose
 * byte s is the scale of block 2(4kq+s)+h of row 32b + r.  rows a multiple
 * of 32, cols a multiple of 256 (EINVAL otherwise); rows*cols = 0 is a
 * no-op. */
engram_status engram_pack_mxfp8(const uint8_t* q, const uint8_t* scale, int64_t rows, int64_t cols,
                                uint8_t* packed, hipStream_t stream);

/* The bf16 W of a layer (w [rows][cols], device, 16-byte aligned) in the
 * operand order of the bf16 matrix cores, for engram_layer.w_packed: packed
 * (device, 16-byte aligned, rows*cols*2 bytes, owned by the caller) holds,
 * for each 32-row block b and 16-column step s, 64 lane slots of 16 bytes
 * (lane l = 32h + r: columns 16s + 8h .. +7 of row 32b + r).  rows a multiple
 * of 32, cols of 16 (EINVAL otherwise); rows*cols = 0 is a no-op. */
engram_status engram_pack_bf16(const void* w, int64_t rows, int64_t cols, void* packed, hipStream_t stream);

/* Engram-Nine hot tier set-up and lookup (see engram_hot_tier).
 *
 * engram_hot_buckets: pilots of a hot set of n_hot n-grams, ceil(n_hot / 4)
 * (1 for 1 <= n_hot <= 4, 0 for n_hot <= 0).
 *
 * engram_hot_build (host only, touches no device): the minimal perfect hash
 * of one order's hot set.  keys: host int32 [n_hot][n], n-gram r oldest id
 * first (as in Step 2), ids >= 0, no n-gram twice; 1 <= n_hot < 2^31,
 * 2 <= n <= ENGRAM_MAX_ORDER.  Writes host pilots [engram_hot_buckets(n_hot)]
 * and host slots [n_hot], where n-gram r sits in the slot the hash gives it,
 * with row = r (so the tier's rows are in the caller's key order), and
 * *seed_used: the first of seed, seed+1, .., seed+15 for which every bucket
 * got a pilot.  Pilots are searched per bucket, largest bucket first, from 0
 * upward.  EINVAL: bad arguments or a repeated n-gram; EUNSUPPORTED: no seed
 * of the 16 worked (two n-grams with one 64-bit hash, or a bucket with no
 * pilot below max(2^24, 16 n_hot)).  Deterministic.
 *
 * engram_hot_lookup: hot_row device int32 [B][T][N-1], hot_row[b][t][n-2] =
 * the hot row of g_{t,n} (n-grams formed as in engram_hash_indices, with
 * hist or pad 0 before the start), or -1 when g_{t,n} is not hot or order n
 * has no hot tier.  hot: host-read descriptor as in engram_layer. */
size_t engram_hot_buckets(int64_t n_hot);
engram_status engram_hot_build(const int32_t* keys, int64_t n_hot, int32_t n, uint64_t seed,
                               uint32_t* pilots, engram_hot_slot* slots, uint64_t* seed_used);
engram_status engram_hot_lookup(const int32_t* tokens, int64_t B, int64_t T, const int32_t* hist,
                                const engram_hash_params* hp, const engram_hot_tier* hot,
                                int32_t* hot_row, hipStream_t stream);

/* Stage timing, for benchmarks.  While profiling is on, calls of
 * engram_forward (and engram_forward_noalloc), engram_retrieve,
 * engram_forward_retrieved(_prefetch), engram_gate_conv_forward and
 * engram_hot_lookup on the calling thread time each kernel they launch: the start and stop events are recorded by the kernel's own
 * dispatch (hipExtLaunchKernel), so a stage is the kernel's execution
 * interval (events owned by the library and reused).
 *   on = 1: engram_profile_read returns the stages of the most recent call
 *           (at most 12).
 *   on = 2: stages accumulate over calls until engram_profile_read, which
 *           returns all of them (at most 2048) and starts a new series, so
 *           calls can run back to back without a host wait between them.
 *           Stages beyond 2048 are not recorded; the read then fails with
 *           ENGRAM_EINVAL and starts a new series.
 *   on = 0: stops recording.
 * engram_profile_read waits for the last recorded event, writes up to `cap`
 * stage durations in milliseconds to ms[] and their kernel names to names[]
 * (static strings; names may be NULL), and returns the stage count in
 * *n_stages.  Other values of `on` return ENGRAM_EINVAL. */
engram_status engram_profile_enable(int32_t on);
engram_status engram_profile_read(float* ms, const char** names, int32_t cap, int32_t* n_stages);

/* Debug build (libengram_debug.so, compiled with ENGRAM_DEBUG_CHECKS): the
 * device-resident preconditions of the conventions above are checked by the
 * kernels before the load that uses each value.  A raw token id outside
 * [0, vocab), a row index outside [0, rows of its table) (engram_gather's z;
 * hashed indices are in range by construction and are checked too), a cache
 * slot outside [-1, cache_n) or a hot-tier row outside [0, n_hot) sets its
 * bit in the error word and is replaced by an in-range value (a token or
 * index clamped into its range, a bad slot or hot row read as a miss), so
 * that no access leaves its buffer.  Raw token ids are clamped into the
 * vocabulary in the release build too, without the report.
 *
 * engram_debug_checks: 1 in the debug build, 0 in the release build.
 * engram_debug_set_error_word: word is a device uint32, 4-byte aligned, that
 * later calls (from any thread) OR their violation bits into with one global
 * atomic each; NULL stops recording.  The caller zeroes it first and keeps it
 * allocated while kernels may write it.  EUNSUPPORTED in the release build.
 * engram_debug_read_errors: waits for the device, returns the word's bits and
 * clears it (synchronous).  EINVAL when no word is set; EUNSUPPORTED in the
 * release build. */
#define ENGRAM_ERR_TOKEN 1u    /* raw token id outside [0, vocab)             */
#define ENGRAM_ERR_ROW 2u      /* row index outside its table                 */
#define ENGRAM_ERR_SLOT 4u     /* cache slot outside [-1, cache_n)            */
#define ENGRAM_ERR_HOT_ROW 8u  /* hot-tier row outside [0, n_hot)             */
int32_t engram_debug_checks(void);
engram_status engram_debug_set_error_word(uint32_t* word);
engram_status engram_debug_read_errors(uint32_t* bits);

/* Pinned host memory that kernels read directly over PCIe (tables kept in
 * host DRAM; the DRAM-offload study reads them through unified addressing).
 * engram_host_alloc returns the host pointer and its device alias; the
 * memory must stay allocated until every stream that reads it has drained.
 * engram_host_free releases memory from engram_host_alloc (synchronous). */
engram_status engram_host_alloc(size_t bytes, void** host_ptr, void** device_alias);
engram_status engram_host_free(void* host_ptr);

#ifdef __cplusplus
}
#endif

#endif /* ENGRAM_H */
