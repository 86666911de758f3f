// Dispatch tables on the device (the contract of Tutorial Example 07:
// group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx, plus
// the stable expert-major permutation).
//
// Three launches over chunks of 1024 (token, slot) pairs, each linear in the
// number of pairs (inputs of at most 2 chunks take one launch instead,
// align_small_kernel):
//   1. count: per-chunk expert histogram counts[c][e] (LDS atomics; counts
//             are order-free).
//   2. scan:  per expert, the exclusive prefix of counts over chunks, in
//             place, and the total (group_sizes). A workgroup takes 64
//             experts (one per lane, so a chunk's row is one coalesced
//             256-byte read) and its 16 waves take consecutive ranges of
//             chunks; the range sums meet in LDS. Every histogram entry is
//             read twice and written once.
//   3. rank:  every chunk reads the totals and its own row of prefixes, scans
//             the totals over experts (wavefront inclusive scans + a
//             cross-wave pass), and ranks its pairs: lanes with the same
//             expert are found with ballots over the bits of the expert id,
//             the rank inside a wave is a popcount below the lane, and waves
//             are ordered through a per-wave count table. Positions therefore
//             follow pair order, never the order in which atomics complete.
// Chunk 0 also writes group_offsets, group_padded_offsets and
// group_idx_for_bx.
#include <mutex>

#include "moe_common.h"

namespace {

constexpr int kChunk = 1024;  // pairs per workgroup = threads per workgroup
constexpr int kWaves = kChunk / 64;
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kChunk) void align_count_kernel(const int32_t* __restrict__ ids, int numel, int E,
                                                             int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p < numel) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) counts[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

constexpr int kScanWaves = 16;

// counts[c][e] <- sum of counts[c'][e] over c' < c; group_sizes[e] <- the sum
// over every chunk. Grid: ceil(E / 64) workgroups of kScanWaves waves.
__global__ __launch_bounds__(64 * kScanWaves) void align_scan_kernel(int32_t* __restrict__ counts, int nchunks, int E,
                                                                    int32_t* __restrict__ group_sizes) {
  __shared__ int s_part[kScanWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const bool live = e < E;
  const int per = (nchunks + kScanWaves - 1) / kScanWaves;
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);
  int32_t* col = counts + e;
  // this wave's range sum, eight loads in flight at a time
  int sum = 0;
  if (live) {
    int c = c0;
    for (; c + 8 <= c1; c += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = col[static_cast<int64_t>(c + u) * E];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += x[u];
    }
    for (; c < c1; ++c) sum += col[static_cast<int64_t>(c) * E];
  }
  s_part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_part[w][lane];
  if (wave == kScanWaves - 1 && live) group_sizes[e] = run + sum;
  if (!live) return;
  // exclusive prefixes over this wave's range, in place
  int c = c0;
  for (; c + 8 <= c1; c += 8) {
    int x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = col[static_cast<int64_t>(c + u) * E];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      col[static_cast<int64_t>(c + u) * E] = run;
      run += x[u];
    }
  }
  for (; c < c1; ++c) {
    const int x = col[static_cast<int64_t>(c) * E];
    col[static_cast<int64_t>(c) * E] = run;
    run += x;
  }
}

__global__ __launch_bounds__(kChunk) void align_rank_kernel(
    const int32_t* __restrict__ ids, int numel, int E, int id_bits, int padding_m, int block_m,
    int m_blocks, const int32_t* __restrict__ prefix, const int32_t* __restrict__ group_sizes,
    int32_t* __restrict__ group_offsets, int32_t* __restrict__ group_padded_offsets,
    int32_t* __restrict__ group_idx_for_bx, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_to_row) {
  __shared__ int s_base[kMaxE];           // compact start of this chunk's pairs of expert e
  __shared__ int s_gpo[kMaxE];            // group_padded_offsets
  __shared__ int s_wave_cnt[kWaves][kMaxE];
  __shared__ int s_wsum[2][kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x;

  for (int i = tid; i < kWaves * E; i += kChunk) s_wave_cnt[i / E][i % E] = 0;

  // totals and this chunk's prefix (from the scan), one expert per thread
  // (E <= 1024 = threads)
  int total = 0, before = 0;
  if (tid < E) {
    total = group_sizes[tid];
    before = prefix[static_cast<int64_t>(chunk) * E + tid];
  }
  const int padded = ((total + padding_m - 1) / padding_m) * padding_m;
  // block-wide exclusive scans of total and padded over experts
  const int inc_t = wave_inclusive_scan(total, lane);
  const int inc_p = wave_inclusive_scan(padded, lane);
  if (lane == 63) {
    s_wsum[0][wave] = inc_t;
    s_wsum[1][wave] = inc_p;
  }
  __syncthreads();
  int pre_t = 0, pre_p = 0;
  for (int w = 0; w < wave; ++w) {
    pre_t += s_wsum[0][w];
    pre_p += s_wsum[1][w];
  }
  const int go = pre_t + inc_t - total;
  const int gpo = pre_p + inc_p - padded;
  if (tid < E) {
    s_base[tid] = go + before;
    s_gpo[tid] = gpo;
    if (chunk == 0) {
      group_offsets[tid] = go;
      group_padded_offsets[tid] = gpo;
    }
  }
  __syncthreads();

  if (chunk == 0) {
    // owner of padded block bx: last expert whose padded offset <= bx*block_m
    for (int bx = tid; bx < m_blocks; bx += kChunk) {
      const int64_t x = static_cast<int64_t>(bx) * block_m;
      int lo = 0, hi = E;  // invariant: s_gpo[lo] <= x (s_gpo[0] == 0)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_gpo[mid] <= x) lo = mid; else hi = mid;
      }
      group_idx_for_bx[bx] = lo;
    }
  }

  // ranks of this chunk's pairs
  const int p = chunk * kChunk + tid;
  int e = (p < numel) ? ids[p] : 0;
  const bool valid = (p < numel) && e >= 0 && e < E;
  if (!valid) e = 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const uint64_t below = peers & ((1ull << lane) - 1ull);
  const int rank_in_wave = __popcll(below);
  if (valid && below == 0) s_wave_cnt[wave][e] = __popcll(peers);
  __syncthreads();
  for (int x = tid; x < E; x += kChunk) {  // exclusive prefix over waves, per expert
    int run = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int c = s_wave_cnt[w][x];
      s_wave_cnt[w][x] = run;
      run += c;
    }
  }
  __syncthreads();
  if (valid) {
    const int pos = s_base[e] + s_wave_cnt[wave][e] + rank_in_wave;
    sorted_pair[pos] = p;
    pair_to_row[p] = pos;
  }
}

// Inputs of at most kSmallChunks chunks: the same tables from one workgroup,
// in one launch (the three launches' cost at a decode batch is their launch
// and latency, not their work). Histogram with LDS atomics, the block-wide
// scans of the rank kernel, then the chunks in order, each ranked as in the
// rank kernel with a running per-expert base, so positions follow pair order
// exactly as there. Measured against the three launches (interleaved, whole
// forwards, same bytes): Kimi-K2-shaped T = 1 0.270 -> 0.262 ms, T = 32
// unchanged; at four chunks (the Qwen3-shaped decode, 4096 pairs) the chunks
// ranked one after another cost as much as the launches (0.2500 -> 0.2514
// ms), so the one-launch form stops at two.
constexpr int kSmallChunks = 2;

__global__ __launch_bounds__(kChunk) void align_small_kernel(
    const int32_t* __restrict__ ids, int numel, int E, int id_bits, int padding_m, int block_m, int m_blocks,
    int32_t* __restrict__ group_sizes, int32_t* __restrict__ group_offsets,
    int32_t* __restrict__ group_padded_offsets, int32_t* __restrict__ group_idx_for_bx,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row) {
  __shared__ int s_hist[kMaxE];
  __shared__ int s_base[kMaxE];           // compact start of the next chunk's pairs of expert e
  __shared__ int s_gpo[kMaxE];
  __shared__ int s_wave_cnt[kWaves][kMaxE];
  __shared__ int s_wsum[2][kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunks = (numel + kChunk - 1) / kChunk;
  if (tid < E) s_hist[tid] = 0;
  for (int i = tid; i < kWaves * E; i += kChunk) s_wave_cnt[i / E][i % E] = 0;
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int p = c * kChunk + tid;
    if (p < numel) {
      const int e = ids[p];
      if (e >= 0 && e < E) atomicAdd(&s_hist[e], 1);
    }
  }
  __syncthreads();

  const int total = tid < E ? s_hist[tid] : 0;
  const int padded = ((total + padding_m - 1) / padding_m) * padding_m;
  const int inc_t = wave_inclusive_scan(total, lane);
  const int inc_p = wave_inclusive_scan(padded, lane);
  if (lane == 63) {
    s_wsum[0][wave] = inc_t;
    s_wsum[1][wave] = inc_p;
  }
  __syncthreads();
  int pre_t = 0, pre_p = 0;
  for (int w = 0; w < wave; ++w) {
    pre_t += s_wsum[0][w];
    pre_p += s_wsum[1][w];
  }
  if (tid < E) {
    const int go = pre_t + inc_t - total;
    const int gpo = pre_p + inc_p - padded;
    s_base[tid] = go;
    s_gpo[tid] = gpo;
    group_sizes[tid] = total;
    group_offsets[tid] = go;
    group_padded_offsets[tid] = gpo;
  }
  __syncthreads();
  for (int bx = tid; bx < m_blocks; bx += kChunk) {
    const int64_t x = static_cast<int64_t>(bx) * block_m;
    int lo = 0, hi = E;  // invariant: s_gpo[lo] <= x (s_gpo[0] == 0)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_gpo[mid] <= x) lo = mid; else hi = mid;
    }
    group_idx_for_bx[bx] = lo;
  }

  for (int c = 0; c < nchunks; ++c) {
    const int p = c * kChunk + tid;
    int e = (p < numel) ? ids[p] : 0;
    const bool valid = (p < numel) && e >= 0 && e < E;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint64_t below = peers & ((1ull << lane) - 1ull);
    if (valid && below == 0) s_wave_cnt[wave][e] = __popcll(peers);
    __syncthreads();
    int chunk_total = 0;  // this chunk's pairs of expert tid
    if (tid < E) {
      for (int w = 0; w < kWaves; ++w) {
        const int cnt = s_wave_cnt[w][tid];
        s_wave_cnt[w][tid] = chunk_total;
        chunk_total += cnt;
      }
    }
    __syncthreads();
    if (valid) {
      const int pos = s_base[e] + s_wave_cnt[wave][e] + __popcll(below);
      sorted_pair[pos] = p;
      pair_to_row[p] = pos;
    }
    __syncthreads();
    if (tid < E) {
      s_base[tid] += chunk_total;
      for (int w = 0; w < kWaves; ++w) s_wave_cnt[w][tid] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

extern "C" size_t moe_align_workspace_bytes(int64_t numel, int E) {
  if (numel < 0 || E < 1) return 0;
  const int64_t nchunks = numel > 0 ? moe::ceil_div(numel, kChunk) : 1;
  return static_cast<size_t>(nchunks) * static_cast<size_t>(E) * sizeof(int32_t);
}

namespace {

// The three launches on `counts` (nchunks x E int32, fully written by the
// count kernel before the scan reads it). Arguments checked by the caller.
int align_launch(const int32_t* topk_ids, int64_t numel, int E, int padding_m, int block_m, int32_t* group_sizes,
                 int32_t* group_offsets, int32_t* group_padded_offsets, int32_t* group_idx_for_bx,
                 int32_t* sorted_pair, int32_t* pair_to_row, int32_t* counts, hipStream_t stream) {
  using namespace moe;
  const int64_t m_blocks = moe_num_blocks(numel, E, block_m, padding_m);
  const int nchunks = numel > 0 ? static_cast<int>(ceil_div(numel, kChunk)) : 1;
  int id_bits = 1;
  while ((1 << id_bits) < E) ++id_bits;
  if (nchunks <= kSmallChunks) {
    align_small_kernel<<<1, kChunk, 0, stream>>>(topk_ids, static_cast<int>(numel), E, id_bits, padding_m, block_m,
                                                 static_cast<int>(m_blocks), group_sizes, group_offsets,
                                                 group_padded_offsets, group_idx_for_bx, sorted_pair, pair_to_row);
    return check_launch("moe_align(small)");
  }
  align_count_kernel<<<nchunks, kChunk, 0, stream>>>(topk_ids, static_cast<int>(numel), E, counts);
  int rc = check_launch("moe_align(count)");
  if (rc) return rc;
  align_scan_kernel<<<static_cast<unsigned>(ceil_div(E, 64)), 64 * kScanWaves, 0, stream>>>(counts, nchunks, E,
                                                                                          group_sizes);
  rc = check_launch("moe_align(scan)");
  if (rc) return rc;
  align_rank_kernel<<<nchunks, kChunk, 0, stream>>>(
      topk_ids, static_cast<int>(numel), E, id_bits, padding_m, block_m, static_cast<int>(m_blocks), counts,
      group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx, sorted_pair, pair_to_row);
  return check_launch("moe_align(rank)");
}

// Argument checks shared by both entry points (nothing is enqueued on failure).
int align_check(const char* name, const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
                int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
                int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row) {
  using namespace moe;
  if (T < 0 || top_k < 1) return fail(MOE_ERR_INVALID_ARG, "%s: T=%lld top_k=%d", name, (long long)T, top_k);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d not in [1,%d]", name, E, kMaxE);
  if (block_m <= 0 || padding_m <= 0 || padding_m % block_m != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: padding_m=%d must be a positive multiple of block_m=%d", name, padding_m,
                block_m);
  const int64_t numel = T * top_k;
  if (numel >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: T*top_k >= 2^31", name);
  const int64_t m_blocks = moe_num_blocks(numel, E, block_m, padding_m);
  if (m_blocks * static_cast<int64_t>(block_m) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: padded row space >= 2^31", name);
  if (!group_sizes || !group_offsets || !group_padded_offsets || !group_idx_for_bx)
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if (numel > 0 && (!topk_ids || !sorted_pair || !pair_to_row))
    return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  return MOE_OK;
}

}  // namespace

extern "C" int moe_align(const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
                         int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
                         int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace moe;
  int rc = align_check("moe_align", topk_ids, T, top_k, E, padding_m, block_m, group_sizes, group_offsets,
                       group_padded_offsets, group_idx_for_bx, sorted_pair, pair_to_row);
  if (rc) return rc;
  const int64_t numel = T * top_k;
  if (!workspace) return fail(MOE_ERR_INVALID_ARG, "moe_align: null workspace");
  if (workspace_bytes < moe_align_workspace_bytes(numel, E))
    return fail(MOE_ERR_INVALID_ARG, "moe_align: workspace %zu < %zu bytes", workspace_bytes,
                moe_align_workspace_bytes(numel, E));
  return align_launch(topk_ids, numel, E, padding_m, block_m, group_sizes, group_offsets, group_padded_offsets,
                      group_idx_for_bx, sorted_pair, pair_to_row, static_cast<int32_t*>(workspace), stream);
}

// ---------------------------------------------------------------------------
// moe_align_noalloc: moe_align with its histogram in a file-scope device
// array instead of a caller workspace, for callers that cannot allocate.
// Every GPU holds its own copy of the array (for as long as the process
// runs); host code reaches it only through the address hipGetSymbolAddress
// returns for that device, looked up once per device on its first call (the
// array's name in host code is a host-side stand-in, not a device address).
// The count launch writes every entry the later launches read, so nothing
// needs clearing between calls; concurrent calls on one GPU share the array
// and race.
namespace {

constexpr size_t kAlignScratchBytes = size_t(4) << 20;
static __device__ __align__(256) int32_t scratch[kAlignScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the stream's device (the current device).
int scratch_for_stream(hipStream_t stream, int32_t** out) {
  using namespace moe;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "moe_align_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "moe_align_noalloc: device %d", dev);
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess)
      return fail(MOE_ERR_INVALID_ARG, "moe_align_noalloc: hipStreamGetDevice failed");
    if (sdev != dev)
      return fail(MOE_ERR_INVALID_ARG, "moe_align_noalloc: the stream is on device %d, the current device is %d",
                  static_cast<int>(sdev), dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "moe_align_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" size_t moe_align_noalloc_max_scratch_bytes(void) { return kAlignScratchBytes; }

extern "C" int moe_align_noalloc(const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
                                 int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
                                 int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row,
                                 hipStream_t stream) {
  using namespace moe;
  int rc = align_check("moe_align_noalloc", topk_ids, T, top_k, E, padding_m, block_m, group_sizes, group_offsets,
                       group_padded_offsets, group_idx_for_bx, sorted_pair, pair_to_row);
  if (rc) return rc;
  const int64_t numel = T * top_k;
  const size_t need = moe_align_workspace_bytes(numel, E);
  if (need > kAlignScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_align_noalloc: T*top_k=%lld pairs over E=%d experts need %zu bytes of scratch, the static "
                "array holds %zu (use moe_align with a workspace)",
                static_cast<long long>(numel), E, need, kAlignScratchBytes);
  int32_t* counts = nullptr;
  rc = scratch_for_stream(stream, &counts);
  if (rc) return rc;
  return align_launch(topk_ids, numel, E, padding_m, block_m, group_sizes, group_offsets, group_padded_offsets,
                      group_idx_for_bx, sorted_pair, pair_to_row, counts, stream);
}
