// Tile order of the wide grouped GEMMs (bf16 and block-scaled FP8): which
// 256-row tile of which expert, and which column tile, workgroup w computes.
//
// The row space is the compact expert-major row space of the dispatch tables
// (group_sizes / group_offsets): expert e owns rows go[e] .. go[e] + gs[e], cut
// into ceil(gs[e] / 256) row tiles, the last one partial. The row tiles of all
// experts, in expert order, form the list that both mappings below walk; the
// hardware hands workgroup w to XCD w % 8, and both mappings place tiles that
// share operands on one XCD at about the same time.
#pragma once

#include "moe_common.h"

namespace moe {

constexpr int kWideRows = 256;        // rows of a wide tile
constexpr int kWideGmax = 4;          // row tiles of an expert block (expert-aware mapping)
constexpr int kWideEgMinCols = 16;    // expert-aware mapping from this many column tiles ...
constexpr int kWideEgMinRowTiles = 32;  // ... and this many row tiles
constexpr int kWideGroup = 16;        // tiles of a fixed group (the other mapping)
constexpr int kWideGnMax = 8;         // column tiles of a fixed group, at most

// Expert g, tile q inside it and the expert's row count n of the p-th 256-row
// tile, counting ceil(gs[e] / 256) tiles per expert in expert order. The
// group sizes of up to kFindBatch * 64 experts are loaded at once (one load
// latency before the search, which every workgroup pays before its first
// weight load), then scanned 64 at a time. Returns false past the last tile.
constexpr int kFindBatch = 8;
__device__ __forceinline__ bool find_wide_tile(const int32_t* __restrict__ gs, int E, int p, int& g, int& q, int& n) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int base0 = 0; base0 < E; base0 += 64 * kFindBatch) {
    int cnt[kFindBatch];
#pragma unroll
    for (int b = 0; b < kFindBatch; ++b) {
      const int e = base0 + b * 64 + lane;
      cnt[b] = e < E ? gs[e] : 0;
    }
#pragma unroll
    for (int b = 0; b < kFindBatch; ++b) {
      if (base0 + b * 64 >= E) break;
      const int pc = (cnt[b] + (kWideRows - 1)) / kWideRows;
      const int incl = wave_incl_sum(pc);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (p < before + total) {
        const int j = __builtin_ctzll(__ballot(before + incl > p));
        g = base0 + b * 64 + j;
        q = p - before - (__builtin_amdgcn_readlane(incl, j) - __builtin_amdgcn_readlane(pc, j));
        n = __builtin_amdgcn_readlane(cnt[b], j);
        return true;
      }
      before += total;
    }
  }
  return false;
}

// Launch geometry of a wide GEMM (host-computed, passed to the kernel).
struct WideGrid {
  int m_tiles;   // row tiles, an upper bound: ceil(numel / 256), plus E with tables
  int n_tiles;   // column tiles
  int gm, gn;    // fixed-group shape (the other mapping)
  int eg;        // 1: the expert-aware mapping
};

// Workgroup slots of the mapping (tiles past the last row tile included) for
// m_tiles row tiles; a multiple of 8.
__host__ __device__ inline int64_t wide_blocks(const WideGrid& wg, int64_t m_tiles) {
  if (wg.eg) return (m_tiles + 7) / 8 * 8 * wg.n_tiles;
  const int64_t groups = (m_tiles + wg.gm - 1) / wg.gm * (wg.n_tiles / wg.gn);
  return (groups + 7) / 8 * 8 * wg.gm * wg.gn;
}

// Row tiles of the grouped row space, sum over e of ceil(gs[e] / 256),
// computed by each wave on its own (same batched loads as find_wide_tile).
__device__ __forceinline__ int wide_row_tiles(const int32_t* __restrict__ gs, int E) {
  const int lane = threadIdx.x & 63;
  int t = 0;
  for (int base0 = 0; base0 < E; base0 += 64 * kFindBatch) {
    int cnt[kFindBatch];
#pragma unroll
    for (int b = 0; b < kFindBatch; ++b) {
      const int e = base0 + b * 64 + lane;
      cnt[b] = e < E ? gs[e] : 0;
    }
#pragma unroll
    for (int b = 0; b < kFindBatch; ++b) t += (cnt[b] + (kWideRows - 1)) / kWideRows;
  }
  return __builtin_amdgcn_readlane(wave_incl_sum(t), 63);
}

// Geometry and grid size for numel compact rows over E groups (grouped: with
// dispatch tables) and n_tiles column tiles; false if the grid is too large.
inline bool wide_grid(int64_t numel, int E, bool grouped, int n_tiles, WideGrid& wg, int64_t& blocks) {
  // every non-empty expert ends in at most one partial tile
  const int64_t m_tiles = ceil_div(numel, kWideRows) + (grouped ? E : 0);
  int gn = 1;
  for (int d = kWideGnMax; d >= 1; --d)
    if (n_tiles % d == 0) {
      gn = d;
      break;
    }
  const int gm = kWideGroup / gn > 0 ? kWideGroup / gn : 1;
  // expert-aware groups when a row tile has many column tiles: on the
  // DeepSeek-V3-shaped routing (16 and 28 column tiles) bf16 gate_up 2.46 ->
  // 2.44 ms and down 1.31 -> 1.28 ms (interleaved A/B); with 6 or 8 (the Qwen3
  // shapes) the fixed 16-tile groups are as fast or faster
  const int eg = n_tiles >= kWideEgMinCols && m_tiles >= kWideEgMinRowTiles;
  if (m_tiles > 0x7FFFFFFF) return false;
  wg = WideGrid{static_cast<int>(m_tiles), n_tiles, gm, gn, eg};
  blocks = wide_blocks(wg, m_tiles);
  return blocks <= 0x7FFFFFFF;
}

// The tile of workgroup w: expert g, column tile nt, first row m_off inside
// the expert's rows and the rows left from there, r (the tile holds min(r,
// 256) rows); false for a workgroup past the last tile. Without tables
// (tb.gs NULL) the numel rows form one group.
//
// Expert-aware mapping: groups of n_tiles workgroups, one per row tile of the
// expert-ordered list, group k on XCD k % 8 (consecutive row tiles on
// consecutive XCDs: grouping an XCD's tiles by expert, or by cost, measured
// slower). An expert with mt tiles splits into blocks of gx tiles (gx the
// largest divisor of n_tiles that is at most min(mt, kWideGmax)); each
// block's gx groups cover its gx row tiles by n_tiles / gx column tiles, so a
// group reuses its weight slices gx times and its activation rows n_tiles /
// gx times from L2; the rows a block leaves over take one group each (one
// row tile by every column tile).
//
// Fixed groups: gm row tiles by gn column tiles, group k on XCD k % 8.
__device__ __forceinline__ bool wide_tile_at(const Tables& tb, int E, int64_t numel, const WideGrid& wg, int w,
                                             int& g, int& nt, int64_t& m_off, int64_t& r) {
  const int n_tiles = wg.n_tiles;
  const int xcd = w & 7, j = w >> 3;
  if (wg.eg) {
    const int jg = j / n_tiles;
    const int t = j - jg * n_tiles;
    const int k = jg * 8 + xcd;
    if (k >= wg.m_tiles) return false;
    int q, mt, n = 0;
    if (tb.gs == nullptr) {
      g = 0;
      q = k;
      mt = static_cast<int>((numel + kWideRows - 1) / kWideRows);
    } else {
      if (!find_wide_tile(tb.gs, E, k, g, q, n)) return false;
      mt = (n + kWideRows - 1) / kWideRows;
    }
    int gx = 1;
    for (int d = min(mt, kWideGmax); d > 1; --d)
      if (n_tiles % d == 0) {
        gx = d;
        break;
      }
    int mq;
    if (q < (mt / gx) * gx) {
      const int gi = q % gx;
      mq = q - gi + t % gx;
      nt = gi * (n_tiles / gx) + t / gx;
    } else {
      mq = q;
      nt = t;
    }
    m_off = static_cast<int64_t>(mq) * kWideRows;
    r = (tb.gs == nullptr ? numel : static_cast<int64_t>(n)) - m_off;
  } else {
    const int gsz = wg.gm * wg.gn;
    const int jg = j / gsz;
    const int t = j - jg * gsz;
    const int group = jg * 8 + xcd;
    const int super_cols = n_tiles / wg.gn;
    const int sr = group / super_cols;
    const int sc = group - sr * super_cols;
    const int tm_ = t % wg.gm;
    const int p = sr * wg.gm + tm_;  // 256-row tile index
    nt = sc * wg.gn + (t - tm_) / wg.gm;
    if (p >= wg.m_tiles) return false;
    if (tb.gs == nullptr) {
      g = 0;
      m_off = static_cast<int64_t>(p) * kWideRows;
      r = numel - m_off;
    } else {
      int q, n;
      if (!find_wide_tile(tb.gs, E, p, g, q, n)) return false;
      m_off = static_cast<int64_t>(q) * kWideRows;
      r = static_cast<int64_t>(n) - m_off;
    }
  }
  return r > 0;
}

}  // namespace moe
