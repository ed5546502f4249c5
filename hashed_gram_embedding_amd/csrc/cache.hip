// Static LFU admission for the HBM hot-row cache.  The Ascend RecSDK Engram
// article (multi-level cache) keeps the frequently accessed embedding rows in
// fast device memory and the full table in host DRAM, choosing them by access
// counts (LFU).  Here the counts come from a warm-up token stream hashed
// exactly like the layer (Steps 1-3 of the Engram series guide); the cache_n
// most frequently addressed rows are admitted (ties: lower global row first)
// and get slots in ascending row order.
//
// Kernels, all on the caller's stream:
//   count      one thread per (token, table): atomic increment of the row count
//   histogram  counts clamped to kBins-1 into a histogram
//   threshold  one workgroup finds the admission count c* and how many rows of
//              count c* still fit
//   scan x2    rank of each count-c* row among equals, then the slot of each
//              admitted row (block scans + a scan of the block sums)
//   copy       admitted rows (and int8 scales) into the cache
//
// Real-time LFU (the same article's hot cache kept up to date from access
// statistics, with admission and eviction): the gathers add 1 per access to a
// per-row count, and an update between steps re-ranks the rows by their
// current counts with the same rule.  Rows that stay keep their slots; rows
// that fall out free theirs; newcomers, in ascending row order, take the free
// slots in ascending slot order and only their rows are copied.  Counts may
// then be aged by a right shift.
//   mark       stayers claim their slot, leavers drop theirs
//   scan x2    rank of each newcomer (rows) and of each free slot (slots)
//   assign     newcomer k -> k-th free slot; the newcomer list
//   copy       newcomer rows (and int8 scales) into their slots
//   age        counts >>= shift
#include "device_util.h"
#include "engram_internal.h"
#include "hash_device.h"

namespace engram {
namespace {

constexpr int kBins = 1 << 20;           // exact while the threshold count is below kBins - 1
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanBlock = kScanThreads * kScanItems;

__global__ void __launch_bounds__(256) fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void __launch_bounds__(256)
count_kernel(const int32_t* __restrict__ tokens, int64_t B, int64_t T, const int32_t* __restrict__ proj, HashArgs a,
             TableArgs ta, uint32_t* __restrict__ counts) {
  const int nt = a.n_tables;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= B * T * nt) return;
  const int j = static_cast<int>(gid % nt);
  const int64_t bt = gid / nt;
  const int64_t b = bt / T;
  const int32_t z = hash_index(tokens, proj, nullptr, a, j, b, bt - b * T, T);
  atomicAdd(counts + ta.row_offset[j] + z, 1u);
}

// Count histogram.  Most rows have tiny counts (almost all zero in a large
// table), so one global bin would take millions of contended atomics: each
// workgroup keeps the bins below kLocalBins in LDS, zeros are counted with a
// wavefront ballot (one LDS add per wavefront), and the workgroup adds its
// non-empty bins to the global histogram at the end.
constexpr int kLocalBins = 4096;

__global__ void __launch_bounds__(256)
histogram_kernel(const uint32_t* __restrict__ counts, int64_t n, uint32_t* __restrict__ bins) {
  __shared__ uint32_t local[kLocalBins];
  for (int i = threadIdx.x; i < kLocalBins; i += blockDim.x) local[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t start = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // every lane of a wavefront runs the same number of iterations (the bound
  // is rounded up to whole strides), so the ballot sees all 64 lanes
  const int64_t wave_start = start - lane;
  for (int64_t base = wave_start; base < n; base += stride) {
    const int64_t i = base + lane;
    const bool valid = i < n;
    const uint32_t c = valid ? counts[i] : 0u;
    const uint64_t zeros = __ballot(valid && c == 0);
    if (lane == 0 && zeros != 0) atomicAdd(&local[0], static_cast<uint32_t>(__popcll(zeros)));
    if (valid && c != 0) {
      if (c < kLocalBins) atomicAdd(&local[c], 1u);
      else atomicAdd(bins + (c < kBins - 1 ? c : kBins - 1), 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kLocalBins; i += blockDim.x)
    if (local[i] != 0) atomicAdd(bins + i, local[i]);
}

// params[0] = c*, params[1] = rows of count c* that are admitted.
__global__ void __launch_bounds__(1024)
threshold_kernel(const uint32_t* __restrict__ bins, int64_t cap, int64_t* __restrict__ params) {
  constexpr int kChunk = kBins / 1024;
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  int64_t s = 0;
  for (int i = 0; i < kChunk; ++i) s += bins[tid * kChunk + i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t above = 0;  // rows with a count above the current chunk / bin
    int64_t cstar = 0, need = 0;
    bool found = false;
    for (int ch = 1023; ch >= 0 && !found; --ch) {
      if (above + part[ch] < cap) {
        above += part[ch];
        continue;
      }
      for (int c = (ch + 1) * kChunk - 1; c >= ch * kChunk; --c) {
        if (above + bins[c] >= cap) {
          cstar = c;
          need = cap - above;
          found = true;
          break;
        }
        above += bins[c];
      }
    }
    if (!found) {  // cap exceeds the row count: everything is admitted
      cstar = 0;
      need = cap;
    }
    params[0] = cstar;
    params[1] = need;
  }
}

// Inputs of the scan flags.
struct FlagSrc {
  const uint32_t* counts;
  const int32_t* eq_rank;
  const int64_t* params;
  const int32_t* slot;    // row -> slot map (mode 2)
  const int32_t* owned;   // slot -> 1 when a staying row holds it (mode 3)
};

__device__ __forceinline__ bool admitted(const FlagSrc& f, int64_t i) {
  const uint32_t c = f.counts[i];
  const uint32_t cs = static_cast<uint32_t>(f.params[0]);
  const uint32_t cc = c < kBins - 1 ? c : kBins - 1;
  return cc > cs || (cc == cs && f.eq_rank[i] < f.params[1]);
}

// mode 0: row count == c*;  mode 1: row admitted (eq_rank from mode 0);
// mode 2: row admitted and not cached (a newcomer);  mode 3: slot free.
__device__ __forceinline__ int32_t scan_flag(int mode, const FlagSrc& f, int64_t i) {
  if (mode == 0) {
    const uint32_t c = f.counts[i];
    return (c < kBins - 1 ? c : kBins - 1) == static_cast<uint32_t>(f.params[0]) ? 1 : 0;
  }
  if (mode == 1) return admitted(f, i) ? 1 : 0;
  if (mode == 2) return (f.slot[i] < 0 && admitted(f, i)) ? 1 : 0;
  return f.owned[i] == 0 ? 1 : 0;
}

// Per-block exclusive scan of the flags, block totals to sums[].
__global__ void __launch_bounds__(kScanThreads)
scan_local_kernel(int mode, FlagSrc f, int64_t n, int32_t* __restrict__ out, int32_t* __restrict__ sums) {
  __shared__ int32_t warp_tot[kScanThreads / 64];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kScanBlock + threadIdx.x * kScanItems;
  int32_t v[kScanItems];
  int32_t run = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    v[k] = i < n ? scan_flag(mode, f, i) : 0;
    run += v[k];
  }
  // exclusive scan of the per-thread totals across the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) warp_tot[wave] = x;
  __syncthreads();
  int32_t wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += warp_tot[w];
  int32_t acc = wave_base + x - run;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t i = base + k;
    if (i < n) out[i] = acc;
    acc += v[k];
  }
  if (threadIdx.x == kScanThreads - 1) sums[blockIdx.x] = wave_base + x;
}

// Exclusive scan of the block totals in one workgroup (serial over chunks).
__global__ void __launch_bounds__(1024) scan_sums_kernel(int32_t* __restrict__ sums, int64_t nb) {
  __shared__ int64_t part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (nb + 1023) / 1024;
  int64_t s = 0;
  for (int64_t i = tid * per; i < (tid + 1) * per && i < nb; ++i) s += sums[i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int64_t acc = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t t = part[i];
      part[i] = acc;
      acc += t;
    }
  }
  __syncthreads();
  int64_t acc = part[tid];
  for (int64_t i = tid * per; i < (tid + 1) * per && i < nb; ++i) {
    const int32_t t = sums[i];
    sums[i] = static_cast<int32_t>(acc);
    acc += t;
  }
}

// mode 0: eq_rank[i] = global exclusive rank among equals.
// mode 1: cache_slot[i] = slot of an admitted row, else -1.
// modes 2, 3: rank of a flagged row / slot, else -1.
__global__ void __launch_bounds__(256)
scan_finish_kernel(int mode, FlagSrc f, int64_t n, int32_t* __restrict__ out, const int32_t* __restrict__ sums) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t r = out[i] + sums[i / kScanBlock];
    out[i] = (mode == 0 || scan_flag(mode, f, i)) ? r : -1;
  }
}

// Stayers claim their slot in owned[]; cached rows that are no longer
// admitted leave the cache (slot -1).
__global__ void __launch_bounds__(256)
mark_kernel(FlagSrc f, int64_t n, int32_t* __restrict__ slot, int32_t* __restrict__ owned) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t s = slot[i];
    if (s < 0) continue;
    if (admitted(f, i)) owned[s] = 1;
    else slot[i] = -1;
  }
}

__global__ void __launch_bounds__(256)
free_list_kernel(const int32_t* __restrict__ free_rank, int64_t n_slots, int32_t* __restrict__ free_list) {
  for (int64_t s = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; s < n_slots;
       s += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t r = free_rank[s];
    if (r >= 0) free_list[r] = static_cast<int32_t>(s);
  }
}

// Newcomer k (ascending row order) takes the k-th free slot (ascending slot
// order); there are never more newcomers than free slots.
__global__ void __launch_bounds__(256)
assign_kernel(const int32_t* __restrict__ new_rank, int64_t n, const int32_t* __restrict__ free_list,
              int32_t* __restrict__ slot, int32_t* __restrict__ new_list) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t r = new_rank[i];
    if (r < 0) continue;
    slot[i] = free_list[r];
    new_list[r] = static_cast<int32_t>(i);
  }
}

// One thread per (newcomer, 8-byte chunk); unused list entries hold -1.
__global__ void __launch_bounds__(256)
copy_new_kernel(const int32_t* __restrict__ new_list, int64_t n_slots, const int32_t* __restrict__ slot,
                const uint8_t* __restrict__ rows, const float* __restrict__ scale, int row_bytes,
                uint8_t* __restrict__ cache, float* __restrict__ cache_scale) {
  const int chunks = row_bytes / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n_slots * chunks) return;
  const int64_t k = gid / chunks;
  const int c = static_cast<int>(gid - k * chunks);
  const int32_t r = new_list[k];
  if (r < 0) return;
  const int32_t s = slot[r];
  *reinterpret_cast<uint2*>(cache + static_cast<int64_t>(s) * row_bytes + c * 8) =
      *reinterpret_cast<const uint2*>(rows + static_cast<int64_t>(r) * row_bytes + c * 8);
  if (c == 0 && scale != nullptr) cache_scale[s] = scale[r];
}

__global__ void __launch_bounds__(256) age_kernel(uint32_t* __restrict__ counts, int64_t n, int shift) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    counts[i] >>= shift;
}

// One thread per (row, 16-byte chunk) of an admitted row.
__global__ void __launch_bounds__(256)
copy_rows_kernel(const int32_t* __restrict__ slot, int64_t n, const uint8_t* __restrict__ rows,
                 const float* __restrict__ scale, int row_bytes, uint8_t* __restrict__ cache,
                 float* __restrict__ cache_scale) {
  const int chunks = row_bytes / 8;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= n * chunks) return;
  const int64_t r = gid / chunks;
  const int c = static_cast<int>(gid - r * chunks);
  const int32_t s = slot[r];
  if (s < 0) return;
  *reinterpret_cast<uint2*>(cache + static_cast<int64_t>(s) * row_bytes + c * 8) =
      *reinterpret_cast<const uint2*>(rows + r * row_bytes + c * 8);
  if (c == 0 && scale != nullptr) cache_scale[s] = scale[r];
}

unsigned grid_for(int64_t n, int threads) {
  const int64_t b = (n + threads - 1) / threads;
  return static_cast<unsigned>(b < 65535 * 64 ? b : 65535 * 64);
}

// Exclusive ranks of the flagged items of [0, n) into out (scan_finish_kernel).
void scan(int mode, const FlagSrc& f, int64_t n, int32_t* out, int32_t* sums, hipStream_t s) {
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  launch_k(scan_local_kernel, dim3(static_cast<unsigned>(nb)), dim3(kScanThreads), 0, s, mode, f, n, out, sums);
  launch_k(scan_sums_kernel, dim3(1), dim3(1024), 0, s, sums, nb);
  launch_k(scan_finish_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, mode, f, n, out, sums);
}

// Histogram of the counts and the admission threshold into params.
void rank_threshold(const uint32_t* counts, int64_t total_rows, int64_t cache_n, uint32_t* bins, int64_t* params,
                    hipStream_t s) {
  launch_k(fill_u32, dim3(grid_for(kBins, 256)), dim3(256), 0, s, bins, static_cast<int64_t>(kBins), 0u);
  const int64_t hist_blocks = (total_rows + 256 * 64 - 1) / (256 * 64);   // ~64 items per thread
  launch_k(histogram_kernel, dim3(static_cast<unsigned>(hist_blocks < 2048 ? hist_blocks : 2048)), dim3(256), 0, s,
           counts, total_rows, bins);
  launch_k(threshold_kernel, dim3(1), dim3(1024), 0, s, bins, cache_n, params);
}

}  // namespace

size_t cache_build_workspace(int64_t total_rows) {
  const int64_t nb = (total_rows + kScanBlock - 1) / kScanBlock;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return al(total_rows * 4) /*counts*/ + al(kBins * 4) /*bins*/ + al(total_rows * 4) /*eq rank*/ +
         al(nb * 4) /*block sums*/ + al(16) /*params*/;
}

hipError_t launch_cache_build(const int32_t* tokens, int64_t B, int64_t T, const int32_t* proj, const HashArgs& ha,
                              const TableArgs& ta, int64_t total_rows, int row_bytes, int64_t cache_n,
                              int32_t* cache_slot, void* cache_rows, float* cache_scale, void* ws, hipStream_t s) {
  const int64_t nb = (total_rows + kScanBlock - 1) / kScanBlock;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* p = static_cast<char*>(ws);
  uint32_t* counts = reinterpret_cast<uint32_t*>(p);
  p += al(total_rows * 4);
  uint32_t* bins = reinterpret_cast<uint32_t*>(p);
  p += al(kBins * 4);
  int32_t* eq_rank = reinterpret_cast<int32_t*>(p);
  p += al(total_rows * 4);
  int32_t* sums = reinterpret_cast<int32_t*>(p);
  p += al(nb * 4);
  int64_t* params = reinterpret_cast<int64_t*>(p);

  launch_k(fill_u32, dim3(grid_for(total_rows, 256)), dim3(256), 0, s, counts, total_rows, 0u);
  const int64_t pairs = B * T * ha.n_tables;
  if (pairs > 0)
    launch_k(count_kernel, dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, s, tokens, B, T,
                       proj, ha, ta, counts);
  rank_threshold(counts, total_rows, cache_n, bins, params, s);
  const FlagSrc f{counts, eq_rank, params, nullptr, nullptr};
  for (int mode = 0; mode < 2; ++mode) scan(mode, f, total_rows, mode == 0 ? eq_rank : cache_slot, sums, s);
  const int64_t work = total_rows * (row_bytes / 8);
  launch_k(copy_rows_kernel, dim3(static_cast<unsigned>((work + 255) / 256)), dim3(256), 0, s, cache_slot,
                     total_rows, static_cast<const uint8_t*>(ta.rows), ta.scale, row_bytes,
                     static_cast<uint8_t*>(cache_rows), cache_scale);
  return hipGetLastError();
}

size_t cache_update_workspace(int64_t total_rows, int64_t cache_n) {
  const int64_t nb = (total_rows + kScanBlock - 1) / kScanBlock;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  return al(kBins * 4) /*bins*/ + 2 * al(total_rows * 4) /*eq rank, newcomer rank*/ + al(nb * 4) /*block sums*/ +
         4 * al(cache_n * 4) /*owned, free rank, free list, newcomer list*/ + al(16) /*params*/;
}

hipError_t launch_cache_update(const TableArgs& ta, int64_t total_rows, int row_bytes, int64_t cache_n,
                               int32_t* cache_slot, void* cache_rows, float* cache_scale, uint32_t* counts,
                               int decay_shift, void* ws, hipStream_t s) {
  const int64_t nb = (total_rows + kScanBlock - 1) / kScanBlock;
  auto al = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  char* p = static_cast<char*>(ws);
  uint32_t* bins = reinterpret_cast<uint32_t*>(p);
  p += al(kBins * 4);
  int32_t* eq_rank = reinterpret_cast<int32_t*>(p);
  p += al(total_rows * 4);
  int32_t* new_rank = reinterpret_cast<int32_t*>(p);
  p += al(total_rows * 4);
  int32_t* sums = reinterpret_cast<int32_t*>(p);
  p += al(nb * 4);
  int32_t* owned = reinterpret_cast<int32_t*>(p);
  p += al(cache_n * 4);
  int32_t* free_rank = reinterpret_cast<int32_t*>(p);
  p += al(cache_n * 4);
  int32_t* free_list = reinterpret_cast<int32_t*>(p);
  p += al(cache_n * 4);
  int32_t* new_list = reinterpret_cast<int32_t*>(p);
  p += al(cache_n * 4);
  int64_t* params = reinterpret_cast<int64_t*>(p);

  rank_threshold(counts, total_rows, cache_n, bins, params, s);
  FlagSrc f{counts, eq_rank, params, cache_slot, owned};
  scan(0, f, total_rows, eq_rank, sums, s);
  if (cache_n > 0) {
    launch_k(fill_u32, dim3(grid_for(cache_n, 256)), dim3(256), 0, s, reinterpret_cast<uint32_t*>(owned), cache_n, 0u);
    launch_k(fill_u32, dim3(grid_for(cache_n, 256)), dim3(256), 0, s, reinterpret_cast<uint32_t*>(new_list), cache_n,
             0xffffffffu);
  }
  launch_k(mark_kernel, dim3(grid_for(total_rows, 256)), dim3(256), 0, s, f, total_rows, cache_slot, owned);
  scan(2, f, total_rows, new_rank, sums, s);
  if (cache_n > 0) {
    scan(3, f, cache_n, free_rank, sums, s);
    launch_k(free_list_kernel, dim3(grid_for(cache_n, 256)), dim3(256), 0, s, free_rank, cache_n, free_list);
    launch_k(assign_kernel, dim3(grid_for(total_rows, 256)), dim3(256), 0, s, new_rank, total_rows, free_list,
             cache_slot, new_list);
    const int64_t work = cache_n * (row_bytes / 8);
    launch_k(copy_new_kernel, dim3(static_cast<unsigned>((work + 255) / 256)), dim3(256), 0, s, new_list, cache_n,
             cache_slot, static_cast<const uint8_t*>(ta.rows), ta.scale, row_bytes, static_cast<uint8_t*>(cache_rows),
             cache_scale);
  }
  if (decay_shift > 0)
    launch_k(age_kernel, dim3(grid_for(total_rows, 256)), dim3(256), 0, s, counts, total_rows, decay_shift);
  return hipGetLastError();
}

}  // namespace engram
