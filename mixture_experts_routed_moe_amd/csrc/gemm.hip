// Grouped GEMM C[e] = A[e] @ W[e]^T for the routed experts on bf16 MFMA.
//
// Work decomposition: one workgroup per (padded row block bx, column tile nt).
// The row block is decoded from the dispatch tables (row recovery of the
// tutorial's contract); blocks past an expert's rows, or past the last
// expert, have no rows and return at once. A is the compact [numel, K]
// layout: rows past the block's valid count are never stored, so an expert's
// last, partial tile needs no padding copy.
//
// Two kernels:
//  * grouped_gemm_pipe_kernel, 128-row blocks (the production path): a
//    128 x 256 tile fed by direct-to-LDS loads through a multi-stage ring, see
//    the comment above it;
//  * grouped_gemm_kernel, any block_m in {64, 128} and narrow outputs: a
//    simpler register-staged double buffer, 128 x 128 tile, four wave64s in a
//    2x2 arrangement each accumulating (BM/2) x 64 with
//    v_mfma_f32_32x32x16_bf16. A and W tiles are K-contiguous in LDS, 128
//    bytes per row, with the eight 16-byte chunks of row r stored at chunk
//    position c ^ g(r) (see row_xor) so the fragment reads are free of LDS bank
//    conflicts.
//
// Fused SwiGLU: the W rows of a tile are gate rows and the matching up rows F
// positions further; each wave holds gate columns and the matching up columns
// in separate accumulators, so the epilogue pairs them in registers:
// h = bf16(silu(bf16(g)) * bf16(u)).
#include <algorithm>

#include "moe_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kBN = 128;
constexpr int kThreads = 256;

using moe::Tables;
using moe::decode_block;

// LDS position of 16-byte chunk c in a 128-byte row r: c ^ g(r) with
// g(r) = (r ^ (r >> 3)) & 7. A ds_read_b128 of an MFMA fragment reads one
// chunk from each of 32 consecutive rows; g makes every 8 consecutive rows
// hit 8 different chunk positions (one 128-byte bank sweep) and every 16
// consecutive rows cover each (row parity, position) pair once (one 256-byte
// sweep), so the read is conflict-free whether the LDS serves it in 8-lane or
// 16-lane phases.
__device__ __forceinline__ int row_xor(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ row_xor(row)) << 3); }

template <int BM, bool FUSED>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, Tables tb, int64_t numel, int n_tiles,
    int K, int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C) {
  constexpr int TM = BM / 64;  // 32-row MFMA tiles per wave
  constexpr int A_CH = BM * 8 / kThreads;
  constexpr int B_CH = kBN * 8 / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kBK];

  const int bx = blockIdx.x / n_tiles;
  const int nt = blockIdx.x - bx * n_tiles;
  int g, rows;
  int64_t m_start;
  decode_block(tb, bx, BM, numel, g, m_start, rows);
  if (rows == 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;

  const uint16_t* a_src[A_CH];
  bool a_ok[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = tid + kThreads * i, r = q >> 3, c = q & 7;
    a_ok[i] = r < rows;
    a_src[i] = A + moe::a_row(tb, m_start + (a_ok[i] ? r : 0)) * K + c * 8;
    a_dst[i] = swz(r, c);
  }
  const uint16_t* b_src[B_CH];
  int b_dst[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int q = tid + kThreads * i, r = q >> 3, c = q & 7;
    int64_t wrow;
    if (FUSED) {
      constexpr int half = kBN / 2;
      wrow = r < half ? static_cast<int64_t>(nt) * half + r : static_cast<int64_t>(up_row) + nt * half + (r - half);
    } else {
      wrow = static_cast<int64_t>(nt) * kBN + r;
    }
    b_src[i] = Wb + wrow * K + c * 8;
    b_dst[i] = swz(r, c);
  }

  uint4 ra[A_CH], rb[B_CH];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<uint4*>(&sA[buf][a_dst[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) *reinterpret_cast<uint4*>(&sB[buf][b_dst[i]]) = rb[i];
  };

  floatx16 acc[TM][2];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

  // B rows of this wave's two 32-column MFMA tiles
  int b_row0[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) b_row0[tn] = FUSED ? tn * (kBN / 2) + wn * 32 : wn * 64 + tn * 32;

  const int nk = K / kBK;
  load(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8_t af[TM], bfr[2];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = wm * (BM / 2) + tm * 32 + (lane & 31);
        af[tm] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][swz(r, chunk)]);
      }
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const int r = b_row0[tn] + (lane & 31);
        bfr[tn] = *reinterpret_cast<const bf16x8_t*>(&sB[cur][swz(r, chunk)]);
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
    }
    if (kt + 1 < nk) stash(cur ^ 1);
    __syncthreads();
  }

  // epilogue: 32x32 accumulator element r of lane l sits at
  // row (r & 3) + 4*(l >> 5) + 8*(r >> 2), column l & 31
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * (BM / 2) + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
      if (row >= rows) continue;
      uint16_t* crow = C + (m_start + row) * ldc;
      const int col = lane & 31;
      if (FUSED) {
        const uint16_t gb = moe::f32_to_bf16(acc[tm][0][r]);
        const uint16_t ub = moe::f32_to_bf16(acc[tm][1][r]);
        crow[nt * (kBN / 2) + wn * 32 + col] = moe::swiglu_bf16(gb, ub);
      } else {
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) crow[nt * kBN + wn * 64 + tn * 32 + col] = moe::f32_to_bf16(acc[tm][tn][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for 128-row blocks: 128 x 256 tile (256 W rows: for the
// fused gate_up, 128 gate rows and the matching 128 up rows, i.e. 128 output
// columns), K step BK, a ring of STAGES LDS stages filled by direct-to-LDS
// 16-byte loads (global_load_lds_dwordx4), so no VGPRs are spent staging
// tiles. Four waves in a 2x2 arrangement each accumulate 64 x 128 with
// v_mfma_f32_32x32x16_bf16 (8 accumulator tiles: 6 fragment reads per 8
// MFMAs). What bounds it is the rate at which bytes reach the CU, not the
// MFMAs (without its global loads the same kernel runs above 2 PFLOP/s), so:
//  * the loads of step kt+STAGES-1 are issued in pieces after each sub-step's
//    MFMAs, never as one burst that would block MFMA issue;
//  * fragments are double-buffered across the 16-wide sub-steps (the LDS
//    reads of sub-step s+1 are in flight during sub-step s's MFMAs);
//  * one barrier per K step, which both publishes the new stage and frees the
//    slot read in the previous step.
//
// A direct-to-LDS load writes lane i's 16 bytes at (wave-uniform base + 16*i),
// so the XOR swizzle is applied on the global side: the lane that fills LDS
// chunk position p of row r fetches global chunk p ^ f(r), where f spreads
// the rows read together by a ds_read_b128 over distinct banks
// (see row_swz). Rows of A past the block's valid count are fetched from the
// last valid row (in bounds); they only feed output rows that are never
// stored.
//
// Tile order: the hardware hands workgroup w to XCD w % 8. Logical tiles are
// grouped GM row blocks x GN column tiles and group g runs on XCD g % 8, so
// tiles that share A rows or W columns run together behind one L2.
// Consecutive groups go to different XCDs, which keeps the active (non-empty)
// blocks spread over all eight.
#ifndef MOE_PIPE_BK
#define MOE_PIPE_BK 64
#endif
#ifndef MOE_PIPE_STAGES
#define MOE_PIPE_STAGES 3
#endif
#ifndef MOE_PIPE_OCC
#define MOE_PIPE_OCC 1
#endif
#ifndef MOE_PIPE_GROUP
#define MOE_PIPE_GROUP 16
#endif
#ifndef MOE_PIPE_GN_MAX
#define MOE_PIPE_GN_MAX 8
#endif

constexpr int kPipeBM = 128;
constexpr int kPipeBNW = 256;

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(lds), 16, 0, 0);
}

// Wait until at most N DMA loads of this wave are outstanding and its LDS
// reads have returned, then barrier: after it, every wave's loads up to that
// point have landed in LDS and every wave is done reading the slots it read
// before, so one barrier per K step both publishes the new stage and frees
// the old slot for the next loads.
template <int N>
__device__ __forceinline__ void wait_dma_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Same, with N = stages_left * L chosen at run time (stages_left < S).
template <int L, int S>
__device__ __forceinline__ void wait_dma_barrier_dyn(int stages_left) {
  if constexpr (S <= 0) {
    wait_dma_barrier<0>();
  } else {
    if (stages_left >= S) wait_dma_barrier<S * L>();
    else wait_dma_barrier_dyn<L, S - 1>(stages_left);
  }
}

// Chunk-position XOR for an LDS row of CPR 16-byte chunks: conflict-free
// ds_read_b128 of 32 consecutive rows in 8- and in 16-lane phases.
template <int CPR>
__device__ __forceinline__ int row_swz(int r) {
  return CPR == 8 ? row_xor(r) : (((r >> 1) ^ (r >> 3)) & 3);
}

template <bool FUSED, int BK, int STAGES, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void grouped_gemm_pipe_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, Tables tb, int64_t numel, int m_blocks,
    int n_tiles, int K, int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C, int gm, int gn) {
  constexpr int CPR = BK / 8;                 // 16-byte chunks per LDS row
  constexpr int ROWB = BK * 2;                // bytes per LDS row
  constexpr int RPL = 64 / CPR;               // rows filled by one wave-wide DMA load
  constexpr int A_BYTES = kPipeBM * ROWB;
  constexpr int STAGE_BYTES = (kPipeBM + kPipeBNW) * ROWB;
  constexpr int A_LOADS = kPipeBM / (4 * RPL);   // per wave (and per lane) per stage
  constexpr int B_LOADS = kPipeBNW / (4 * RPL);
  constexpr int L = A_LOADS + B_LOADS;
  static_assert(STAGES >= 3, "the spread issue needs a free slot");
  static_assert(OCC * STAGES * STAGE_BYTES <= 160 * 1024, "LDS ring too large");
  static_assert((STAGES - 2) * L <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t smem[STAGES * STAGE_BYTES];

  // logical tile of this workgroup (see "Tile order" above)
  const int w = blockIdx.x;
  const int xcd = w & 7, j = w >> 3;
  const int gsz = gm * gn;
  const int jg = j / gsz;
  const int t = j - jg * gsz;
  const int group = jg * 8 + xcd;
  const int super_cols = n_tiles / gn;
  const int sr = group / super_cols;
  const int sc = group - sr * super_cols;
  const int tm_ = t % gm;
  const int bx = sr * gm + tm_;
  const int nt = sc * gn + (t - tm_) / gm;
  if (bx >= m_blocks) return;
  int g, rows;
  int64_t m_start;
  decode_block(tb, bx, kPipeBM, numel, g, m_start, rows);
  if (rows == 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane / CPR;                // row inside one DMA load
  const int lpos = lane % CPR;                // LDS chunk position this lane fills

  // per-lane global sources at k = 0 and wave-uniform LDS offsets
  const uint16_t* a_src[A_LOADS];
  int a_lds[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int rb = (wave * A_LOADS + i) * RPL;
    const int r = rb + lrow;
    const int rr = min(r, rows - 1);
    a_src[i] = A + moe::a_row(tb, m_start + rr) * K + (lpos ^ row_swz<CPR>(r)) * 8;
    a_lds[i] = rb * ROWB;
  }
  const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;
  const uint16_t* b_src[B_LOADS];
  int b_lds[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int rb = (wave * B_LOADS + i) * RPL;
    const int r = rb + lrow;
    int64_t wrow;
    if (FUSED)
      wrow = r < kPipeBNW / 2 ? static_cast<int64_t>(nt) * (kPipeBNW / 2) + r
                              : static_cast<int64_t>(up_row) + static_cast<int64_t>(nt) * (kPipeBNW / 2) + (r - kPipeBNW / 2);
    else
      wrow = static_cast<int64_t>(nt) * kPipeBNW + r;
    b_src[i] = Wb + wrow * K + (lpos ^ row_swz<CPR>(r)) * 8;
    b_lds[i] = A_BYTES + rb * ROWB;
  }

  // DMA loads of step kt, load indices [first, first + count): A loads
  // first, then B loads. A step's L loads are spread over the MFMA sub-steps
  // of the previous step so the load queue never blocks MFMA issue for long.
  auto issue = [&](int kt, int first, int count) __attribute__((always_inline)) {
    uint8_t* st = smem + (kt % STAGES) * STAGE_BYTES;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < first || i >= first + count) continue;
      if (i < A_LOADS) dma16(a_src[i] + k0, st + a_lds[i]);
      else dma16(b_src[i - A_LOADS] + k0, st + b_lds[i - A_LOADS]);
    }
  };
  constexpr int NS = BK / 16;                     // MFMA sub-steps per step
  constexpr int PER = (L + NS - 1) / NS;          // loads issued per sub-step

  floatx16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // LDS byte offsets (inside a stage) of this lane's fragment rows
  int a_row[2], b_row[4];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) a_row[tm] = wm * 64 + tm * 32 + (lane & 31);
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
    b_row[tn] = (FUSED ? (tn < 2 ? wn * 64 + tn * 32 : kPipeBNW / 2 + wn * 64 + (tn - 2) * 32)
                       : wn * 128 + tn * 32) + (lane & 31);
  const int khalf = lane >> 5;

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s, 0, L);

  // fragments of one 16-wide sub-step, double-buffered: the LDS reads of
  // sub-step s+1 are issued before the MFMAs of sub-step s, so the MFMA pipe
  // does not sit idle for an LDS round trip between sub-steps
  bf16x8_t af[2][2], bfr[2][4];
  auto read_frags = [&](const uint8_t* st, int ks, int buf) __attribute__((always_inline)) {
    const int chunk = ks * 2 + khalf;
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int r = a_row[tm];
      af[buf][tm] = *reinterpret_cast<const bf16x8_t*>(st + r * ROWB + ((chunk ^ row_swz<CPR>(r)) << 4));
    }
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int r = b_row[tn];
      bfr[buf][tn] = *reinterpret_cast<const bf16x8_t*>(st + A_BYTES + r * ROWB + ((chunk ^ row_swz<CPR>(r)) << 4));
    }
  };
  for (int kt = 0; kt < nk; ++kt) {
    // steps kt+1 .. kt+STAGES-2 may still be in flight; step kt+STAGES-1 is
    // issued during this step's MFMAs into the slot freed by step kt-1
    if (kt + STAGES - 2 < nk) wait_dma_barrier<(STAGES - 2) * L>();
    else wait_dma_barrier_dyn<L, STAGES - 3>(nk - 1 - kt);
    const bool ahead = kt + STAGES - 1 < nk;
    const uint8_t* st = smem + (kt % STAGES) * STAGE_BYTES;
    read_frags(st, 0, 0);
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {
      if (ks + 1 < NS) read_frags(st, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][tm], bfr[ks & 1][tn], acc[tm][tn], 0, 0, 0);
      // the loads set M0, which makes the compiler drain outstanding LDS
      // reads: issue them after this sub-step's MFMAs are queued
      if (ahead) issue(kt + STAGES - 1, ks * PER, PER);
    }
  }

  // epilogue (accumulator element r of lane l: row (r&3) + 4*(l>>5) + 8*(r>>2), column l&31)
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
      if (row >= rows) continue;
      uint16_t* crow = C + (m_start + row) * ldc;
      const int col = lane & 31;
      if (FUSED) {
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          const uint16_t gb = moe::f32_to_bf16(acc[tm][tn][r]);
          const uint16_t ub = moe::f32_to_bf16(acc[tm][tn + 2][r]);
          crow[nt * (kPipeBNW / 2) + wn * 64 + tn * 32 + col] = moe::swiglu_bf16(gb, ub);
        }
      } else {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          crow[nt * kPipeBNW + wn * 128 + tn * 32 + col] = moe::f32_to_bf16(acc[tm][tn][r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel for 128-row blocks: 256 x 256 tiles. A workgroup takes two
// consecutive 128-row blocks of one expert (blocks 2q and 2q+1 of the
// expert's padded range, i.e. its compact rows 256q .. 256q+255), so every
// weight byte brought to the CU feeds 256 rows instead of 128: 128 FLOP per
// staged byte against 85 for the 128 x 256 tile, which is what counts when
// the CUs are fed at a fixed rate. The grid enumerates these 256-row tiles
// directly (find_wide_tile), so no workgroup is launched for the odd blocks:
// launching and retiring one per odd block lines the working workgroups up
// with the hardware's workgroup-to-CU rotation and leaves half of the CUs
// idle.
//
// Eight waves (two per SIMD) in a 4x2 arrangement, each 64 rows x 128 weight
// rows (8 accumulator tiles), so while one wave of a SIMD waits on a load
// issue, a barrier or an LDS read, the other keeps the matrix core busy
// (measured on the DeepSeek-V3-shaped routed gate_up: 2.83 ms against 3.02
// ms with four 128 x 128 waves). A wave whose rows are all past the tile's
// valid rows skips its MFMAs.
//
// An expert's last tile often has 128 rows or fewer (an odd block count).
// Such a "half" tile loads only 128 A rows and splits K between the wave
// rows: wave rows wm and wm + 2 cover the same 64 rows, the first over the
// even 16-wide sub-steps, the second over the odd ones, and the two partial
// sums meet in LDS at the end. A half tile therefore costs about half a full
// one, and the padding overhead stays that of 128-row blocks.
//
// Loads, fragments and barriers work as in grouped_gemm_pipe_kernel, over
// the ring described at wide_ring_tile.
constexpr int kWideRows = 256;
constexpr int kWideW = 256;

// The wide tile's K loop, K step 64 (whole 128-byte rows, so every L1 -> L2
// request moves a full line). The A part and the W part of a step are 32 KiB
// each; A(kt) goes to A slot kt % 3 and W(kt) to W slot kt % 2 (LDS: three A
// slots, then two W slots, 160 KiB). During step kt the loads of W(kt+1) and
// A(kt+2) go into the slots steps kt-1 used, and the wait at the top of step
// kt+1 leaves A(kt+2) in flight: between one and three 32 KiB parts are in
// flight at any time and the ring never drains.
//
// The loop is unrolled over the six steps after which both slot sequences
// repeat, so every slot index is a compile-time constant: the LDS fragment
// reads take per-lane offsets computed once (opaque to the optimizer, so the
// slot base stays in the instruction's immediate offset) and the
// direct-to-LDS loads take an SGPR destination (M0) and a uniform global base
// plus a per-lane offset that does not change over K. The inner loop then
// issues almost nothing besides MFMAs, LDS reads and loads.
// Chunk position XOR of the wide tile's LDS rows: (r & 7) ^ ((r >> 3) & 1).
// Any 8 consecutive rows from a multiple of 8 take 8 different positions (one
// 128-byte bank sweep), and the 8 rows of one parity among 16 consecutive rows
// from a multiple of 16 take 8 different positions (one 256-byte sweep), so
// the fragment reads are conflict-free in 8- and in 16-lane phases. Rows 16
// apart share the XOR, so every fragment of a sub-step sits at a constant
// offset from the first one (32 rows = 4 KiB apart) and one per-lane offset
// serves all of them.
__device__ __forceinline__ int wide_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

#ifndef MOE_WIDE_SKIP
#define MOE_WIDE_SKIP 1
#endif
constexpr int kWideSlotBytes = kWideRows * 128;
constexpr int kWideASlots = 3;
constexpr int kWideWSlots = 2;
constexpr int kWideWRing = kWideASlots * kWideSlotBytes;  // first W slot
constexpr int kWideLds = (kWideASlots + kWideWSlots) * kWideSlotBytes;

// SiLU table of the fused gate_up epilogue: entry i is silu_spec of the bf16
// gate moe::silu_table_entry(i) decodes (|g| in [2^-25, 128), both signs),
// 32 KiB. gemm_silu_table_kernel writes it before each fused wide launch on
// the same stream (constants: a concurrent call on another stream writes the
// same bits).
__device__ float g_gemm_silu_tab[moe::kSiluTabMid];

__global__ __launch_bounds__(256) void gemm_silu_table_kernel() {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < moe::kSiluTabMid) g_gemm_silu_tab[i] = moe::silu_table_entry(i);
}

// silu_spec of a bf16 gate (bits gb) from the 8192-entry table, or the
// closed forms outside its range: g/2 for |g| below 2^-25 and g for g at or
// above 128 (the same bits as moe::silu_lookup). Negative gates of magnitude
// at least 128 are not covered (silu_tab_misses); the caller evaluates those
// directly.
__device__ __forceinline__ float silu_tab(const float* tab, uint32_t gb) {
  const uint32_t e = (gb >> 7) & 0xFFu;
  const uint32_t k = e - static_cast<uint32_t>(moe::kSiluTabE0);  // wraps for e < kSiluTabE0
  const float t = tab[((gb >> 3) & 0x1000u) | ((k & 31u) << 7) | (gb & 127u)];
  const float g = __uint_as_float(gb << 16);
  const float out = e < static_cast<uint32_t>(moe::kSiluTabE0) ? g * 0.5f : g;
  return k < 32u ? t : out;
}

__device__ __forceinline__ bool silu_tab_misses(uint32_t gb) {
  return (gb & 0x8000u) && ((gb >> 7) & 0xFFu) >= static_cast<uint32_t>(moe::kSiluTabE0 + 32);
}

template <int V>
struct Ic {
  static constexpr int value = V;
};

template <bool FUSED, bool HALF, int NW>
__device__ __forceinline__ void wide_ring_tile(uint8_t* smem, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ Wb, int64_t m_start, int rows, int nt,
                                               int K, int up_row, int ldc, uint16_t* __restrict__ C,
                                               const int32_t* __restrict__ gather, int gather_k) {
  constexpr int BK = 64, CPR = 8, ROWB = 128, RPL = 8;
  constexpr int AROWS = HALF ? kWideRows / 2 : kWideRows;
  constexpr int WM = NW / 2;                         // wave rows (two wave columns)
  constexpr int TM = kWideRows / WM / 32;            // 32-row MFMA tiles per wave
  constexpr int A_LOADS = AROWS / (NW * RPL);        // per wave per step
  constexpr int B_LOADS = kWideW / (NW * RPL);
  constexpr int NS = BK / 16;
  constexpr int MY_NS = HALF ? NS / 2 : NS;
  constexpr int L = A_LOADS + B_LOADS;               // loads issued per step
  constexpr int PER = (L + MY_NS - 1) / MY_NS;
  static_assert(kWideSlotBytes == kWideW * ROWB, "a slot holds one 256-row part");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane / CPR;
  const int lpos = lane % CPR;

  // direct-to-LDS sources: a uniform base per step plus fixed per-lane
  // offsets (with a gather table, from the start of A: the host checks that
  // A's rows fit 32-bit byte offsets)
  const char* a_base = reinterpret_cast<const char*>(gather ? A : A + m_start * K);
  const char* w_base = reinterpret_cast<const char*>(Wb + static_cast<int64_t>(nt) * (FUSED ? kWideW / 2 : kWideW) * K);
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = (wave * A_LOADS + i) * RPL + lrow;
    const int rr = min(r, rows - 1);
    const uint32_t ar = gather ? static_cast<uint32_t>(gather[m_start + rr] / gather_k) : static_cast<uint32_t>(rr);
    a_off[i] = ar * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>((lpos ^ wide_swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = (wave * B_LOADS + i) * RPL + lrow;
    const int lr = (FUSED && r >= kWideW / 2) ? up_row + (r - kWideW / 2) : r;
    b_off[i] = static_cast<uint32_t>(lr) * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>((lpos ^ wide_swz(r)) << 4);
  }
  const int a_lds0 = wave * A_LOADS * RPL * ROWB;
  const int b_lds0 = kWideWRing + wave * B_LOADS * RPL * ROWB;

  floatx16 acc[TM][4];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // half tiles: wave rows wm and wm + WM/2 cover the same rows, the first
  // the even sub-steps, the second the odd ones
  const int kpar = HALF ? (wm >= WM / 2) : 0;
  const int row0 = (HALF ? wm % (WM / 2) : wm) * TM * 32;
#if MOE_WIDE_SKIP
  // 32-row MFMA tiles of this wave that hold valid rows (the others are
  // skipped: with two waves per SIMD the partner wave gets the matrix core)
  const int live_tm = __builtin_amdgcn_readfirstlane(min(TM, max(0, (rows - row0 + 31) / 32)));
#endif
  const int khalf = lane >> 5;
  // per-lane LDS byte offset of this wave's first A and first W fragment in
  // each sub-step; the other fragments sit at constant offsets from them
  const int a_r0 = row0 + (lane & 31);
  const int b_r0 = (FUSED ? wn * 64 : wn * 128) + (lane & 31);
  uint32_t a_rd[MY_NS], b_rd[MY_NS];
#pragma unroll
  for (int i = 0; i < MY_NS; ++i) {
    const int chunk = (HALF ? 2 * i + kpar : i) * 2 + khalf;
    a_rd[i] = static_cast<uint32_t>(a_r0 * ROWB + ((chunk ^ wide_swz(a_r0)) << 4));
    b_rd[i] = static_cast<uint32_t>(kWideWRing + b_r0 * ROWB + ((chunk ^ wide_swz(b_r0)) << 4));
    asm volatile("" : "+v"(a_rd[i]), "+v"(b_rd[i]));
  }
  // W fragment tn: rows b_r0 + b_frag_row(tn)
  constexpr int kBFragRow[4] = {0, 32, FUSED ? kWideW / 2 : 64, FUSED ? kWideW / 2 + 32 : 96};

  const int nk = K / BK;
  // prologue: A(0), W(0), A(1)
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) dma16(a_base + a_off[i], smem + a_lds0 + i * RPL * ROWB);
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) dma16(w_base + b_off[i], smem + b_lds0 + i * RPL * ROWB);
  if (nk > 1) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      dma16(a_base + BK * 2 + a_off[i], smem + kWideSlotBytes + a_lds0 + i * RPL * ROWB);
  }

  bf16x8_t af[2][TM], bfr[2][4];
  auto step = [&](auto sa, auto sw, int kt) __attribute__((always_inline)) {
    constexpr int SA = decltype(sa)::value, SW = decltype(sw)::value;
    constexpr int A_NEXT = (SA + 2) % kWideASlots, W_NEXT = (SW + 1) % kWideWSlots;
    // every load except A(kt+1) (the last issued) must have landed
    if (kt + 1 < nk) wait_dma_barrier<A_LOADS>();
    else wait_dma_barrier<0>();
    auto read_frags = [&](int i, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[buf][tm] = *reinterpret_cast<const bf16x8_t*>(smem + a_rd[i] + SA * kWideSlotBytes + tm * 32 * ROWB);
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
        bfr[buf][tn] =
            *reinterpret_cast<const bf16x8_t*>(smem + b_rd[i] + SW * kWideSlotBytes + kBFragRow[tn] * ROWB);
    };
    const char* w_src = w_base + (kt + 1) * BK * 2;
    const char* a_src = a_base + (kt + 2) * BK * 2;
    read_frags(0, 0);
#pragma unroll
    for (int i = 0; i < MY_NS; ++i) {
      // a sub-step is: the reads of the next sub-step's fragments, this
      // sub-step's MFMAs, its share of the loads; the scheduler keeps them in
      // that order (left free, it hoists every read of a step and spills)
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < MY_NS) read_frags(i + 1, (i + 1) & 1);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
#if MOE_WIDE_SKIP
        if (tm >= live_tm) break;  // wave-uniform: this and later row tiles hold no valid rows
#endif
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i & 1][tm], bfr[i & 1][tn], acc[tm][tn], 0, 0, 0);
      }
      // this sub-step's share of the loads for W(kt+1), then A(kt+2)
#pragma unroll
      for (int j = i * PER; j < i * PER + PER && j < L; ++j) {
        if (j < B_LOADS) {
          if (kt + 1 < nk)
            dma16(w_src + b_off[j], smem + b_lds0 + W_NEXT * kWideSlotBytes + j * RPL * ROWB);
        } else {
          if (kt + 2 < nk)
            dma16(a_src + a_off[j - B_LOADS],
                  smem + a_lds0 + A_NEXT * kWideSlotBytes + (j - B_LOADS) * RPL * ROWB);
        }
      }
    }
  };
  // six steps per iteration (both slot sequences repeat after six), each
  // guarded, so the loop has a single exit
  for (int kt = 0; kt < nk; kt += 6) {
    step(Ic<0>{}, Ic<0>{}, kt);
    if (kt + 1 < nk) step(Ic<1>{}, Ic<1>{}, kt + 1);
    if (kt + 2 < nk) step(Ic<2>{}, Ic<0>{}, kt + 2);
    if (kt + 3 < nk) step(Ic<0>{}, Ic<1>{}, kt + 3);
    if (kt + 4 < nk) step(Ic<1>{}, Ic<0>{}, kt + 4);
    if (kt + 5 < nk) step(Ic<2>{}, Ic<1>{}, kt + 5);
  }

  // FUSED: the SiLU table goes into the ring's last 32 KiB (the second W slot,
  // above the half-tile exchange) once every wave is past its last fragment
  // read; it lands while the halves meet
  constexpr int kTabOff = kWideLds - moe::kSiluTabMid * 4;
  if constexpr (FUSED) {
    static_assert(kTabOff >= 128 * 1024, "the table sits above the exchange");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < moe::kSiluTabMid / 4 / (64 * NW); ++i) {
      const int c = (i * NW + wave) * 64;  // a wave-wide load fills 64 consecutive 16-byte pieces
      dma16(reinterpret_cast<const float4*>(g_gemm_silu_tab) + c + lane, smem + kTabOff + c * 16);
    }
  }

  if constexpr (HALF) {
    // the two K halves meet in LDS (the ring is idle: every load has landed
    // at the last step's wait): the odd-sub-step waves hand over their sums
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    constexpr int XCH = TM * 4 * 4 * 64;                 // floatx4 per wave
    static_assert(NW / 2 * XCH * 16 <= kWideLds, "exchange fits the ring");
    floatx4* xch = reinterpret_cast<floatx4*>(smem) + ((wm % (WM / 2)) * 2 + wn) * XCH;
    if (kpar) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            floatx4 v = {acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2], acc[tm][tn][4 * q + 3]};
            xch[((tm * 4 + tn) * 4 + q) * 64 + lane] = v;
          }
    }
    // (and for this wave's table pieces: after it the table is whole)
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kpar) return;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      // one row tile's partial sums at a time, added here (not sunk into the
      // conditional stores below, which would keep every read live at once)
      asm volatile("" ::: "memory");
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 v = xch[((tm * 4 + tn) * 4 + q) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tm][tn][4 * q + e] += v[e];
        }
        asm volatile("" : "+v"(acc[tm][tn]));
      }
    }
  }

  // FUSED without the halves: wait for the table (every wave's pieces)
  if constexpr (FUSED && !HALF) asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  const float* tab = reinterpret_cast<const float*>(smem + kTabOff);
  // the SiLUs come from the table unless a gate of this wave needs the direct
  // evaluation (a negative one of magnitude at least 128): one vote per wave,
  // and one loop for each case
  auto store = [&](auto use_tab) __attribute__((always_inline)) {
    constexpr bool TAB = decltype(use_tab)::value != 0;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
        if (row >= rows) continue;
        uint16_t* crow = C + (m_start + row) * ldc;
        const int col = lane & 31;
        if (FUSED) {
#pragma unroll
          for (int tn = 0; tn < 2; ++tn) {
            const uint16_t gb = moe::f32_to_bf16(acc[tm][tn][r]);
            const uint16_t ub = moe::f32_to_bf16(acc[tm][tn + 2][r]);
            crow[nt * (kWideW / 2) + wn * 64 + tn * 32 + col] =
                TAB ? moe::f32_to_bf16(silu_tab(tab, gb) * moe::bf16_to_f32(ub)) : moe::swiglu_bf16(gb, ub);
          }
        } else {
#pragma unroll
          for (int tn = 0; tn < 4; ++tn)
            crow[nt * kWideW + wn * 128 + tn * 32 + col] = moe::f32_to_bf16(acc[tm][tn][r]);
        }
      }
    }
  };
  if constexpr (FUSED) {
    bool miss = false;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int r = 0; r < 16; ++r) miss |= silu_tab_misses(moe::f32_to_bf16(acc[tm][tn][r]));
    if (__builtin_amdgcn_readfirstlane(static_cast<int>(__ballot(miss) != 0)))
      store(Ic<0>{});
    else
      store(Ic<1>{});
  } else {
    store(Ic<0>{});
  }
}

// Expert g and tile q inside it of the p-th 256-row tile, counting
// ceil(gs[e] / 256) tiles per expert in expert order (a wave-wide scan over
// the group sizes, 64 experts at a time). Returns false past the last tile.
__device__ __forceinline__ bool find_wide_tile(const int32_t* __restrict__ gs, int E, int p, int& g, int& q) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int pc = e < E ? (gs[e] + (kWideRows - 1)) / kWideRows : 0;
    int incl = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int total = __shfl(incl, 63);
    if (p < before + total) {
      const int j = __builtin_ctzll(__ballot(before + incl > p));
      g = __builtin_amdgcn_readfirstlane(base + j);
      q = __builtin_amdgcn_readfirstlane(p - before - (__shfl(incl, j) - __shfl(pc, j)));
      return true;
    }
    before += total;
  }
  return false;
}

#ifndef MOE_WIDE_GMAX
#define MOE_WIDE_GMAX 4
#endif
#ifndef MOE_WIDE_EG_MIN_COLS
#define MOE_WIDE_EG_MIN_COLS 16
#endif
#ifndef MOE_WIDE_EG_MIN_ROW_TILES
#define MOE_WIDE_EG_MIN_ROW_TILES 32
#endif

template <bool FUSED, int NW>
__global__ __launch_bounds__(64 * NW, 1) void grouped_gemm_wide_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, Tables tb, int E, int64_t numel, int m_tiles,
    int n_tiles, int K, int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C, int gm, int gn,
    int expert_groups) {
  constexpr int SMEM = kWideLds;
  static_assert(SMEM <= 160 * 1024, "LDS ring too large");
  static_assert(SMEM >= 128 * 1024, "the half-tile exchange needs 128 KiB");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int w = blockIdx.x;
  const int xcd = w & 7, j = w >> 3;
  int g, nt;
  int64_t m_start, r;
  if (expert_groups) {
    // Groups of n_tiles tiles, one per 256-row tile of the expert-ordered list
    // (group k runs on XCD k % 8). An expert with mt tiles splits into blocks
    // of gx tiles (gx the largest divisor of n_tiles that is at most
    // min(mt, MOE_WIDE_GMAX)); each block's gx groups cover its gx row tiles by
    // n_tiles / gx column tiles, so a group reuses its weight slice gx times and
    // its activation rows n_tiles / gx times from L2; the rows a block leaves
    // over take one group each (one row tile by every column tile).
    const int jg = j / n_tiles;
    const int t = j - jg * n_tiles;
    const int k = jg * 8 + xcd;
    if (k >= m_tiles) return;
    int q, mt;
    if (tb.gs == nullptr) {
      g = 0;
      q = k;
      mt = static_cast<int>((numel + kWideRows - 1) / kWideRows);
    } else {
      if (!find_wide_tile(tb.gs, E, k, g, q)) return;
      mt = (tb.gs[g] + kWideRows - 1) / kWideRows;
    }
    int gx = 1;
    for (int d = min(mt, MOE_WIDE_GMAX); d > 1; --d)
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
    if (tb.gs == nullptr) {
      m_start = static_cast<int64_t>(mq) * kWideRows;
      r = numel - m_start;
    } else {
      m_start = static_cast<int64_t>(tb.go[g]) + static_cast<int64_t>(mq) * kWideRows;
      r = static_cast<int64_t>(tb.gs[g]) - static_cast<int64_t>(mq) * kWideRows;
    }
  } else {
    const int gsz = gm * gn;
    const int jg = j / gsz;
    const int t = j - jg * gsz;
    const int group = jg * 8 + xcd;
    const int super_cols = n_tiles / gn;
    const int sr = group / super_cols;
    const int sc = group - sr * super_cols;
    const int tm_ = t % gm;
    const int p = sr * gm + tm_;  // 256-row tile index
    nt = sc * gn + (t - tm_) / gm;
    if (p >= m_tiles) return;
    if (tb.gs == nullptr) {
      g = 0;
      m_start = static_cast<int64_t>(p) * kWideRows;
      r = numel - m_start;
    } else {
      int q;
      if (!find_wide_tile(tb.gs, E, p, g, q)) return;
      m_start = static_cast<int64_t>(tb.go[g]) + static_cast<int64_t>(q) * kWideRows;
      r = static_cast<int64_t>(tb.gs[g]) - static_cast<int64_t>(q) * kWideRows;
    }
  }
  if (r <= 0) return;
  const int rows = r >= kWideRows ? kWideRows : static_cast<int>(r);
  const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;
  if (rows <= kWideRows / 2)
    wide_ring_tile<FUSED, true, NW>(smem, A, Wb, m_start, rows, nt, K, up_row, ldc, C, tb.gather, tb.gather_k);
  else
    wide_ring_tile<FUSED, false, NW>(smem, A, Wb, m_start, rows, nt, K, up_row, ldc, C, tb.gather, tb.gather_k);
}

// Group shape for the tile order: GN column tiles (a divisor of n_tiles, at
// most MOE_PIPE_GN_MAX) by GM row blocks, about MOE_PIPE_GROUP tiles.
void pipe_groups(int n_tiles, int& gm, int& gn) {
  gn = 1;
  for (int d = MOE_PIPE_GN_MAX; d >= 1; --d)
    if (n_tiles % d == 0) {
      gn = d;
      break;
    }
  gm = MOE_PIPE_GROUP / gn > 0 ? MOE_PIPE_GROUP / gn : 1;
}

template <bool FUSED>
int launch_pipe(const uint16_t* A, const uint16_t* W, Tables tb, int64_t numel, int64_t m_blocks, int n_tiles, int K,
                int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  int gm, gn;
  pipe_groups(n_tiles, gm, gn);
  const int64_t groups = moe::ceil_div(m_blocks, gm) * (n_tiles / gn);
  const int64_t blocks = moe::ceil_div(groups, 8) * 8 * gm * gn;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  grouped_gemm_pipe_kernel<FUSED, MOE_PIPE_BK, MOE_PIPE_STAGES, MOE_PIPE_OCC><<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
      A, W, tb, numel, static_cast<int>(m_blocks), n_tiles, K, w_stride, up_row, ldc, C, gm, gn);
  return moe::check_launch(name);
}

#ifndef MOE_WIDE_GROUP
#define MOE_WIDE_GROUP 16
#endif
#ifndef MOE_WIDE_WAVES
#define MOE_WIDE_WAVES 8
#endif

template <bool FUSED>
int launch_wide(const uint16_t* A, const uint16_t* W, Tables tb, int E, int64_t numel, int n_tiles, int K,
                int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  // every non-empty expert ends in at most one partial tile
  const int64_t m_tiles = moe::ceil_div(numel, kWideRows) + (tb.gs ? E : 0);
  int gn = 1;
  for (int d = MOE_PIPE_GN_MAX; d >= 1; --d)
    if (n_tiles % d == 0) {
      gn = d;
      break;
    }
  const int gm = MOE_WIDE_GROUP / gn > 0 ? MOE_WIDE_GROUP / gn : 1;
  // expert-aware groups (see the kernel) when a row tile has many column
  // tiles: on the DeepSeek-V3-shaped routing (16 and 28 column tiles) gate_up
  // 2.46 -> 2.44 ms and down 1.31 -> 1.28 ms (interleaved A/B); with 6 or 8
  // (the Qwen3 shapes) the fixed 16-tile groups are as fast or faster
  const int eg = n_tiles >= MOE_WIDE_EG_MIN_COLS && m_tiles >= MOE_WIDE_EG_MIN_ROW_TILES;
  const int64_t groups = moe::ceil_div(m_tiles, gm) * (n_tiles / gn);
  const int64_t blocks = eg ? moe::ceil_div(m_tiles, 8) * 8 * n_tiles : moe::ceil_div(groups, 8) * 8 * gm * gn;
  if (blocks > 0x7FFFFFFF || m_tiles > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  if (FUSED) {
    gemm_silu_table_kernel<<<moe::kSiluTabMid / 256, 256, 0, stream>>>();
    const int rc = moe::check_launch("gemm_silu_table_kernel");
    if (rc) return rc;
  }
  grouped_gemm_wide_kernel<FUSED, MOE_WIDE_WAVES><<<static_cast<unsigned>(blocks), 64 * MOE_WIDE_WAVES, 0, stream>>>(
      A, W, tb, E, numel, static_cast<int>(m_tiles), n_tiles, K, w_stride, up_row, ldc, C, gm, gn, eg);
  return moe::check_launch(name);
}

// ---------------------------------------------------------------------------
// Few-row kernel (decode). When the groups hold a handful of rows (a one-token
// shared expert, a few tokens spread over many experts) the time is the weight
// stream, and 128- or 256-row tiles split the output into too few workgroups
// to reach HBM bandwidth (28 for a 7168 x 18432 down projection). One
// 256-thread workgroup per (group, 32 output columns): 8 lanes per weight row
// each read 16 bytes a step, so a row's lanes cover 128 contiguous bytes, with
// kGemvUnroll steps in flight per lane, and fp32 dot products against the
// group's rows, kGemvRows at a time (the rows are few: read from L2).
constexpr int kGemvCols = 32;
constexpr int kGemvRows = 4;
constexpr int kGemvUnroll = 4;

__device__ __forceinline__ void bf16x8_to_f32(uint4 v, float* f) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// The k-th expert with rows (a wave-wide scan over the group sizes, 64 at a
// time); false past the last one.
__device__ __forceinline__ bool find_nonempty(const int32_t* __restrict__ gs, int E, int k, int& g) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const uint64_t live = __ballot(e < E && gs[e] > 0);
    const int total = __popcll(live);
    if (k < before + total) {
      // the (k - before)-th set bit of live
      uint64_t m = live;
      for (int i = 0; i < k - before; ++i) m &= m - 1;
      g = __builtin_amdgcn_readfirstlane(base + __builtin_ctzll(m));
      return true;
    }
    before += total;
  }
  return false;
}

template <bool FUSED>
__global__ __launch_bounds__(256) void grouped_gemv_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W, Tables tb, int E,
                                                           int64_t numel, int n_tiles, int K, int64_t w_stride,
                                                           int up_row, int ldc, uint16_t* __restrict__ C) {
  // grid: min(numel, E) expert slots (at most that many experts have rows)
  // by the column tiles; slot k takes the k-th expert with rows
  const int k = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  int g;
  int64_t m0;
  int rows;
  if (tb.gs == nullptr) {
    g = 0;
    m0 = 0;
    rows = static_cast<int>(numel);
  } else {
    if (!find_nonempty(tb.gs, E, k, g)) return;
    m0 = tb.go[g];
    rows = tb.gs[g];
  }
  if (rows <= 0) return;
  const int t = threadIdx.x, wr = t >> 3, kc = t & 7;
  const int col = nt * kGemvCols + wr;
  const uint16_t* wg = W + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(col) * K;
  const uint16_t* wu = W + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(FUSED ? up_row + col : col) * K;
  for (int r0 = 0; r0 < rows; r0 += kGemvRows) {
    const int nr = min(kGemvRows, rows - r0);
    const uint16_t* arow[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) arow[r] = A + moe::a_row(tb, m0 + r0 + min(r, nr - 1)) * K;
    float acc_g[kGemvRows], acc_u[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) acc_g[r] = acc_u[r] = 0.0f;
    // K in steps of 64 (8 lanes x 8 values): whole blocks of kGemvUnroll
    // steps with every weight load, then every activation load (L1/L2 hits),
    // issued before the arithmetic; then the remaining steps one at a time
    auto block = [&](int kb, auto unroll) __attribute__((always_inline)) {
      constexpr int U = decltype(unroll)::value;
      uint4 vg[U], vu[U], va[U][kGemvRows];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kb + u * 64 + kc * 8;
        vg[u] = *reinterpret_cast<const uint4*>(wg + k);
        if (FUSED) vu[u] = *reinterpret_cast<const uint4*>(wu + k);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r)
          va[u][r] = *reinterpret_cast<const uint4*>(arow[r] + kb + u * 64 + kc * 8);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float fg[8], fu[8];
        bf16x8_to_f32(vg[u], fg);
        if (FUSED) bf16x8_to_f32(vu[u], fu);
#pragma unroll
        for (int r = 0; r < kGemvRows; ++r) {
          float fa[8];
          bf16x8_to_f32(va[u][r], fa);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            acc_g[r] += fa[i] * fg[i];
            if (FUSED) acc_u[r] += fa[i] * fu[i];
          }
        }
      }
    };
    int kb = 0;
    for (; kb + 64 * kGemvUnroll <= K; kb += 64 * kGemvUnroll) block(kb, Ic<kGemvUnroll>{});
    for (; kb < K; kb += 64) block(kb, Ic<1>{});
    // the 8 lanes of a weight row are consecutive: reduce over lanes 1, 2, 4 apart
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
      for (int d = 1; d < 8; d <<= 1) {
        acc_g[r] += __shfl_xor(acc_g[r], d);
        if (FUSED) acc_u[r] += __shfl_xor(acc_u[r], d);
      }
    if (kc == 0) {
#pragma unroll
      for (int r = 0; r < kGemvRows; ++r) {
        if (r >= nr) break;
        uint16_t* crow = C + (m0 + r0 + r) * ldc;
        if (FUSED)
          crow[col] = moe::swiglu_bf16(moe::f32_to_bf16(acc_g[r]), moe::f32_to_bf16(acc_u[r]));
        else
          crow[col] = moe::f32_to_bf16(acc_g[r]);
      }
    }
  }
}

template <bool FUSED>
int launch_gemv(const uint16_t* A, const uint16_t* W, Tables tb, int E, int64_t numel, int K, int64_t w_stride,
                int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  const int n_tiles = ldc / kGemvCols;
  const int64_t slots = tb.gs ? std::min<int64_t>(numel, E) : 1;
  const int64_t blocks = slots * n_tiles;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  grouped_gemv_kernel<FUSED><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(A, W, tb, E, numel, n_tiles, K,
                                                                                w_stride, up_row, ldc, C);
  return moe::check_launch(name);
}

// ---------------------------------------------------------------------------
// Skinny dense kernel: one group of 5..32 rows (a shared expert at a decode
// batch). The row-tile kernels give such a launch one workgroup per 256
// output columns (28 for a 7168-wide down projection), and the few-row kernel
// re-reads the weights once per 4 rows. Here one 512-thread workgroup takes
// 32 output columns (fused: 32 gate and the matching 32 up weight rows) and
// its eight waves split K (wave w takes the 64-wide steps w, w + 8, ...), so a
// 7168 x 18432 down projection runs 224 workgroups. Operands go from global
// memory straight to the MFMA registers: lane l reads 64 contiguous bytes
// (32 k values) of activation row l & 31 and of weight row l & 31 at k
// offset 32 (l >> 5) of each step, and MFMA i of the step takes the lane's
// i-th 16 bytes of both, so every k of the step is summed once. Each wave
// keeps kSkinnyDepth steps of loads in flight; the eight partial sums meet in
// LDS and are added in wave order (the result does not depend on timing).
constexpr int kSkinnyCols = 32;
constexpr int kSkinnyWaves = 8;
#ifndef MOE_SKINNY_DEPTH
#define MOE_SKINNY_DEPTH 2
#endif
#ifndef MOE_SKINNY_OCC
#define MOE_SKINNY_OCC 2
#endif
constexpr int kSkinnyDepth = MOE_SKINNY_DEPTH;
#ifndef MOE_SKINNY_MAX_ROWS
#define MOE_SKINNY_MAX_ROWS 32
#endif

template <bool FUSED>
__global__ __launch_bounds__(64 * kSkinnyWaves, MOE_SKINNY_OCC) void dense_skinny_kernel(const uint16_t* __restrict__ A,
                                                                            const uint16_t* __restrict__ W, int rows,
                                                                            int K, int up_row, int ldc,
                                                                            uint16_t* __restrict__ C) {
  constexpr int NB = FUSED ? 2 : 1;   // 32-column weight blocks per wave (gate, up)
  constexpr int D = kSkinnyDepth;
  __shared__ float red[kSkinnyWaves][NB][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int l32 = lane & 31, h = lane >> 5;
  const int nt = blockIdx.x;
  const uint16_t* w0 = W + (static_cast<int64_t>(nt) * kSkinnyCols + l32) * K + h * 32;
  const uint16_t* w1 = W + (static_cast<int64_t>(FUSED ? up_row : 0) + static_cast<int64_t>(nt) * kSkinnyCols + l32) * K +
                       h * 32;
  // activation row l32; rows past the last read the last row (never stored)
  const uint16_t* ap = A + static_cast<int64_t>(min(l32, rows - 1)) * K + h * 32;

  floatx16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.0f;
  const int nk = K / 64;
  const int n_my = wave < nk ? (nk - wave + kSkinnyWaves - 1) / kSkinnyWaves : 0;
  if (n_my > 0) {
    uint4 bw[D][NB][4], ba[D][4];
    // loads of this wave's step s into slot d (steps past the last reload it
    // and add zero); site: a distinct empty asm statement after each call
    // site's loads keeps the optimizer from merging the prologue's loads
    // with the loop's into one block
    auto issue = [&](auto dd, int s, auto site) __attribute__((always_inline)) {
      constexpr int d = decltype(dd)::value;
      const int ko = (min(s, n_my - 1) * kSkinnyWaves + wave) * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bw[d][0][j] = *reinterpret_cast<const uint4*>(w0 + ko + j * 8);
        if (FUSED) bw[d][NB - 1][j] = *reinterpret_cast<const uint4*>(w1 + ko + j * 8);
        ba[d][j] = *reinterpret_cast<const uint4*>(ap + ko + j * 8);
      }
      asm volatile("; skinny loads %0" ::"n"(decltype(site)::value * 8 + d));
    };
    auto mfmas = [&](auto dd, bool live) __attribute__((always_inline)) {
      constexpr int d = decltype(dd)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, live ? ba[d][i] : make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bw[d][b][i]), acc[b], 0, 0, 0);
      }
    };
    static_assert(D >= 1 && D <= 4, "depth 1..4");
    issue(Ic<0>{}, 0, Ic<0>{});
    if constexpr (D > 1) issue(Ic<1>{}, 1, Ic<0>{});
    if constexpr (D > 2) issue(Ic<2>{}, 2, Ic<0>{});
    if constexpr (D > 3) issue(Ic<3>{}, 3, Ic<0>{});
    const int n_pad = (n_my + D - 1) / D * D;
    int s0 = 0;
    // whole blocks of D steps, each slot refilled D steps ahead after its
    // MFMAs; the last block refills nothing
    for (; s0 + D < n_pad; s0 += D) {
      __builtin_amdgcn_sched_barrier(0);
      mfmas(Ic<0>{}, true);
      __builtin_amdgcn_sched_barrier(0);
      issue(Ic<0>{}, s0 + D, Ic<1>{});
      if constexpr (D > 1) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(Ic<1>{}, true);
        __builtin_amdgcn_sched_barrier(0);
        issue(Ic<1>{}, s0 + D + 1, Ic<1>{});
      }
      if constexpr (D > 2) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(Ic<2>{}, true);
        __builtin_amdgcn_sched_barrier(0);
        issue(Ic<2>{}, s0 + D + 2, Ic<1>{});
      }
      if constexpr (D > 3) {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(Ic<3>{}, true);
        __builtin_amdgcn_sched_barrier(0);
        issue(Ic<3>{}, s0 + D + 3, Ic<1>{});
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(Ic<0>{}, s0 < n_my);
    if constexpr (D > 1) mfmas(Ic<1>{}, s0 + 1 < n_my);
    if constexpr (D > 2) mfmas(Ic<2>{}, s0 + 2 < n_my);
    if constexpr (D > 3) mfmas(Ic<3>{}, s0 + 3 < n_my);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][b][e][lane] = acc[b][e];
  __syncthreads();
  if (wave != 0) return;
  // result register e of lane l: activation row (e & 3) + 4h + 8(e >> 2), column l & 31
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int row = (e & 3) + 4 * h + 8 * (e >> 2);
    float v[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      v[b] = red[0][b][e][lane];
#pragma unroll
      for (int w = 1; w < kSkinnyWaves; ++w) v[b] += red[w][b][e][lane];
    }
    if (row >= rows) continue;
    uint16_t* crow = C + static_cast<int64_t>(row) * ldc + static_cast<int64_t>(nt) * kSkinnyCols + l32;
    if (FUSED)
      *crow = moe::swiglu_bf16(moe::f32_to_bf16(v[0]), moe::f32_to_bf16(v[NB - 1]));
    else
      *crow = moe::f32_to_bf16(v[0]);
  }
}

template <bool FUSED>
int launch_skinny(const uint16_t* A, const uint16_t* W, int64_t numel, int K, int up_row, int ldc, uint16_t* C,
                  hipStream_t stream, const char* name) {
  dense_skinny_kernel<FUSED><<<static_cast<unsigned>(ldc / kSkinnyCols), 64 * kSkinnyWaves, 0, stream>>>(
      A, W, static_cast<int>(numel), K, up_row, ldc, C);
  return moe::check_launch(name);
}

#ifndef MOE_GEMV_MAX_ROWS
#define MOE_GEMV_MAX_ROWS 4
#endif
#ifndef MOE_GEMV_GROUPED_PCT
#define MOE_GEMV_GROUPED_PCT 10
#endif

template <bool FUSED>
int launch(const uint16_t* A, const uint16_t* W, Tables tb, int64_t numel, int E, int block_m, int padding_m,
           int n_tiles, int K, int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream,
           const char* name, bool a_off32 = true) {
  const int64_t m_blocks = tb.gs ? moe_num_blocks(numel, E, block_m, padding_m) : moe::ceil_div(numel, block_m);
  const int64_t blocks = m_blocks * n_tiles;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  // ldc is the output width: F for the fused gate_up, 2F or H otherwise
  const int pipe_cols = FUSED ? kPipeBNW / 2 : kPipeBNW;
  // 256-row tiles pay off once experts average a full 128-row block (at
  // fewer rows per expert nearly every tile is a half tile and the 128-row
  // kernel, with less fixed cost per tile, is faster)
#ifndef MOE_WIDE_MIN_ROWS
#define MOE_WIDE_MIN_ROWS 128
#endif
  // few rows (at most 4 in one dense group, or numel <= E / 10 over the
  // experts: one decode token's top-k): the weight-streaming kernel (at 256
  // rows over 384 experts the row-tile kernels are faster)
  const bool few_rows = tb.gs ? numel * 100 <= MOE_GEMV_GROUPED_PCT * static_cast<int64_t>(E) : numel <= MOE_GEMV_MAX_ROWS;
  if (few_rows && K % 64 == 0 && ldc % kGemvCols == 0)
    return launch_gemv<FUSED>(A, W, tb, E, numel, K, w_stride, up_row, ldc, C, stream, name);
  // one dense group of up to 32 rows: the K-split skinny kernel
  if (tb.gs == nullptr && tb.gather == nullptr && numel <= MOE_SKINNY_MAX_ROWS && K % 64 == 0 &&
      ldc % kSkinnyCols == 0)
    return launch_skinny<FUSED>(A, W, numel, K, up_row, ldc, C, stream, name);
  // the wide kernel addresses a tile's A and W rows with 32-bit byte offsets
  // (with a gather table, A's offsets count from its first row: a_off32)
  const bool wide_fits = (static_cast<int64_t>(up_row) + kWideW) * K * 2 < (int64_t(1) << 32) && a_off32;
#ifndef MOE_WIDE_DENSE_MIN_TILES
#define MOE_WIDE_DENSE_MIN_TILES 128
#endif
  // a dense launch with few 256-row tiles: the 128-row kernel gives it twice the workgroups
  const bool dense_few = tb.gs == nullptr && moe::ceil_div(numel, kWideRows) * (ldc / pipe_cols) < MOE_WIDE_DENSE_MIN_TILES;
  if (block_m == kPipeBM && ldc % pipe_cols == 0 && K % 64 == 0 && wide_fits && !dense_few &&
      numel >= static_cast<int64_t>(MOE_WIDE_MIN_ROWS) * E)
    return launch_wide<FUSED>(A, W, tb, E, numel, ldc / pipe_cols, K, w_stride, up_row, ldc, C, stream, name);
  if (block_m == kPipeBM && ldc % pipe_cols == 0)
    return launch_pipe<FUSED>(A, W, tb, numel, m_blocks, ldc / pipe_cols, K, w_stride, up_row, ldc, C, stream, name);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  if (block_m == 128)
    grouped_gemm_kernel<128, FUSED><<<grid, block, 0, stream>>>(A, W, tb, numel, n_tiles, K, w_stride, up_row, ldc, C);
  else
    grouped_gemm_kernel<64, FUSED><<<grid, block, 0, stream>>>(A, W, tb, numel, n_tiles, K, w_stride, up_row, ldc, C);
  return moe::check_launch(name);
}

int check_common(const char* name, const uint16_t* A, const uint16_t* W, const int32_t* gs, const int32_t* go,
                 const int32_t* gpo, const int32_t* gidx, int64_t numel, int E, int padding_m, int block_m,
                 const uint16_t* C) {
  using namespace moe;
  if (numel < 0) return fail(MOE_ERR_INVALID_ARG, "%s: numel < 0", name);
  if (block_m != 64 && block_m != 128) return fail(MOE_ERR_UNSUPPORTED, "%s: block_m=%d not in {64,128}", name, block_m);
  const bool dense = gs == nullptr;
  if (dense != (go == nullptr) || dense != (gpo == nullptr) || dense != (gidx == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "%s: tables must be all NULL (dense) or all non-NULL", name);
  if (!dense) {
    if (E < 1) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d", name, E);
    if (padding_m <= 0 || padding_m % block_m != 0)
      return fail(MOE_ERR_INVALID_ARG, "%s: padding_m=%d must be a positive multiple of block_m=%d", name, padding_m,
                  block_m);
  } else if (E != 1) {
    return fail(MOE_ERR_INVALID_ARG, "%s: dense mode (NULL tables) needs E=1", name);
  }
  if (numel >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: numel >= 2^31", name);
  if (numel > 0 && (!A || !W || !C)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if (numel > 0 && (!aligned16(A) || !aligned16(W) || !aligned16(C)))
    return fail(MOE_ERR_INVALID_ARG, "%s: A/W/C not 16-byte aligned", name);
  return MOE_OK;
}

}  // namespace

extern "C" int grouped_gemm_gate_up(const uint16_t* x_perm, const uint16_t* w_gate_up, const int32_t* group_sizes,
                                    const int32_t* group_offsets, const int32_t* group_padded_offsets,
                                    const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                                    int padding_m, int block_m, int fuse_swiglu, uint16_t* out,
                                    hipStream_t stream) {
  const char* name = "grouped_gemm_gate_up";
  int rc = check_common(name, x_perm, w_gate_up, group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx,
                        numel, E, padding_m, block_m, out);
  if (rc) return rc;
  if (H < kBK || H % kBK != 0 || F < 64 || F % 64 != 0)
    return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H=%d must be a multiple of 64, F=%d a multiple of 64", name, H, F);
  if (numel == 0) return MOE_OK;
  const Tables tb{group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx};
  const int64_t w_stride = static_cast<int64_t>(2) * F * H;
  if (fuse_swiglu)
    return launch<true>(x_perm, w_gate_up, tb, numel, E, block_m, padding_m, F / 64, H, w_stride, F, F, out, stream, name);
  return launch<false>(x_perm, w_gate_up, tb, numel, E, block_m, padding_m, (2 * F) / kBN, H, w_stride, 0, 2 * F, out,
                       stream, name);
}

extern "C" int grouped_gemm_gate_up_gather(const uint16_t* hidden, int64_t T, const int32_t* sorted_pair, int top_k,
                                           const uint16_t* w_gate_up, const int32_t* group_sizes,
                                           const int32_t* group_offsets, const int32_t* group_padded_offsets,
                                           const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                                           int padding_m, int block_m, int fuse_swiglu, uint16_t* out,
                                           hipStream_t stream) {
  const char* name = "grouped_gemm_gate_up_gather";
  if (!group_sizes) return moe::fail(MOE_ERR_INVALID_ARG, "%s: the gather needs the dispatch tables", name);
  int rc = check_common(name, hidden, w_gate_up, group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx,
                        numel, E, padding_m, block_m, out);
  if (rc) return rc;
  if (T < 0 || top_k < 1 || numel != T * top_k)
    return moe::fail(MOE_ERR_INVALID_ARG, "%s: numel=%lld must be T=%lld times top_k=%d", name,
                     static_cast<long long>(numel), static_cast<long long>(T), top_k);
  if (numel > 0 && !sorted_pair) return moe::fail(MOE_ERR_INVALID_ARG, "%s: null sorted_pair", name);
  if (H < kBK || H % kBK != 0 || F < 64 || F % 64 != 0)
    return moe::fail(MOE_ERR_UNSUPPORTED, "%s: H=%d must be a multiple of 64, F=%d a multiple of 64", name, H, F);
  if (numel == 0) return MOE_OK;
  Tables tb{group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx};
  tb.gather = sorted_pair;
  tb.gather_k = top_k;
  const bool a_off32 = T * H * 2 < (int64_t(1) << 32);
  const int64_t w_stride = static_cast<int64_t>(2) * F * H;
  if (fuse_swiglu)
    return launch<true>(hidden, w_gate_up, tb, numel, E, block_m, padding_m, F / 64, H, w_stride, F, F, out, stream,
                        name, a_off32);
  return launch<false>(hidden, w_gate_up, tb, numel, E, block_m, padding_m, (2 * F) / kBN, H, w_stride, 0, 2 * F, out,
                       stream, name, a_off32);
}

extern "C" int grouped_gemm_down(const uint16_t* h, const uint16_t* w_down, const int32_t* group_sizes,
                                 const int32_t* group_offsets, const int32_t* group_padded_offsets,
                                 const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F, int padding_m,
                                 int block_m, uint16_t* y, hipStream_t stream) {
  const char* name = "grouped_gemm_down";
  int rc = check_common(name, h, w_down, group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx, numel, E,
                        padding_m, block_m, y);
  if (rc) return rc;
  if (F < kBK || F % kBK != 0 || H < kBN || H % kBN != 0)
    return moe::fail(MOE_ERR_UNSUPPORTED, "%s: F=%d must be a multiple of 64, H=%d a multiple of 128", name, F, H);
  if (numel == 0) return MOE_OK;
  const Tables tb{group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx};
  return launch<false>(h, w_down, tb, numel, E, block_m, padding_m, H / kBN, F, static_cast<int64_t>(H) * F, 0, H, y,
                       stream, name);
}
