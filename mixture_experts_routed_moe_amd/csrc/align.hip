// Dispatch tables on the device (the contract of Tutorial Example 07:
// group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx, plus
// the stable expert-major permutation).
//
// Two launches over chunks of 1024 (token, slot) pairs:
//   1. count: per-chunk expert histogram (LDS atomics; counts are order-free).
//   2. rank:  every chunk re-reads the small [nchunks, E] histogram to get
//             the global totals and its own chunk prefix, scans the totals
//             over experts (wavefront inclusive scans + a cross-wave pass),
//             and ranks its pairs: lanes with the same expert are found with
//             ballots over the bits of the expert id, the rank inside a wave
//             is a popcount below the lane, and waves are ordered through a
//             per-wave count table. Positions therefore follow pair order,
//             never the order in which atomics complete.
// Chunk 0 also writes the E-sized tables and group_idx_for_bx.
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

__global__ __launch_bounds__(kChunk) void align_rank_kernel(
    const int32_t* __restrict__ ids, int numel, int E, int id_bits, int padding_m, int block_m,
    int m_blocks, const int32_t* __restrict__ counts, int nchunks, int32_t* __restrict__ group_sizes,
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

  // totals and this chunk's prefix, one expert per thread (E <= 1024 = threads)
  // (eight loads in flight at a time: one at a time, each waited for, the
  // 32 chunks of a 32768-pair launch cost 32 round trips)
  int total = 0, before = 0;
  if (tid < E) {
    int c = 0;
    for (; c + 8 <= nchunks; c += 8) {
      int x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = counts[static_cast<int64_t>(c + u) * E + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        before += (c + u < chunk) ? x[u] : 0;
        total += x[u];
      }
    }
    for (; c < nchunks; ++c) {
      const int x = counts[static_cast<int64_t>(c) * E + tid];
      before += (c < chunk) ? x : 0;
      total += x;
    }
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
      group_sizes[tid] = total;
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

}  // namespace

extern "C" size_t moe_align_workspace_bytes(int64_t numel, int E) {
  if (numel < 0 || E < 1) return 0;
  const int64_t nchunks = numel > 0 ? moe::ceil_div(numel, kChunk) : 1;
  return static_cast<size_t>(nchunks) * static_cast<size_t>(E) * sizeof(int32_t);
}

extern "C" int moe_align(const int32_t* topk_ids, int64_t T, int top_k, int E, int padding_m, int block_m,
                         int32_t* group_sizes, int32_t* group_offsets, int32_t* group_padded_offsets,
                         int32_t* group_idx_for_bx, int32_t* sorted_pair, int32_t* pair_to_row,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace moe;
  if (T < 0 || top_k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_align: T=%lld top_k=%d", (long long)T, top_k);
  if (E < 1 || E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, "moe_align: E=%d not in [1,%d]", E, kMaxE);
  if (block_m <= 0 || padding_m <= 0 || padding_m % block_m != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_align: padding_m=%d must be a positive multiple of block_m=%d",
                padding_m, block_m);
  const int64_t numel = T * top_k;
  if (numel >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "moe_align: T*top_k >= 2^31");
  const int64_t m_blocks = moe_num_blocks(numel, E, block_m, padding_m);
  if (m_blocks * static_cast<int64_t>(block_m) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_align: padded row space >= 2^31");
  if (!group_sizes || !group_offsets || !group_padded_offsets || !group_idx_for_bx || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_align: null pointer");
  if (numel > 0 && (!topk_ids || !sorted_pair || !pair_to_row))
    return fail(MOE_ERR_INVALID_ARG, "moe_align: null pointer");
  if (workspace_bytes < moe_align_workspace_bytes(numel, E))
    return fail(MOE_ERR_INVALID_ARG, "moe_align: workspace %zu < %zu bytes", workspace_bytes,
                moe_align_workspace_bytes(numel, E));
  const int nchunks = numel > 0 ? static_cast<int>(ceil_div(numel, kChunk)) : 1;
  int id_bits = 1;
  while ((1 << id_bits) < E) ++id_bits;
  int32_t* counts = static_cast<int32_t*>(workspace);
  align_count_kernel<<<nchunks, kChunk, 0, stream>>>(topk_ids, static_cast<int>(numel), E, counts);
  int rc = check_launch("moe_align(count)");
  if (rc) return rc;
  align_rank_kernel<<<nchunks, kChunk, 0, stream>>>(
      topk_ids, static_cast<int>(numel), E, id_bits, padding_m, block_m, static_cast<int>(m_blocks), counts,
      nchunks, group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx, sorted_pair, pair_to_row);
  return check_launch("moe_align(rank)");
}
