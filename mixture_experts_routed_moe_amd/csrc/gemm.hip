// Grouped GEMM C[e] = A[e] @ W[e]^T for the routed experts on bf16 MFMA.
//
// Work decomposition: a workgroup computes one row tile by one column tile
// of one expert at a time (the persistent form of the 256-row kernel walks a
// list of them). Row tiles are found from the dispatch tables (the compact
// expert-major row space that the routing tables define); a tile past an
// expert's rows, or past the last expert, has no rows and returns at once. A
// is the compact [numel, K] layout: rows past a tile's valid count are never
// stored, so an expert's last, partial tile needs no padding copy.
//
// Five kernels, chosen per launch by launch() below:
//  * grouped_gemm_wide_kernel (the production path for 128-row blocks): 256 x
//    256 tiles, eight waves, direct-to-LDS loads through a ring of stages, the
//    tile order of wide_sched.h; see the comment above it. Its persistent
//    form, grouped_gemm_wide_persistent_kernel, runs the same tile bodies on
//    a grid of one workgroup per CU that claims tiles at run time (chosen for
//    small experts, see launch_wide);
//  * grouped_gemm_pipe_kernel: 128 x 256 tiles on the same kind of ring, for
//    dense launches with too few 256-row tiles to fill the chip, K not a
//    multiple of 64, and operands past the wide kernel's 32-bit offsets;
//  * grouped_gemm_kernel, any block_m in {64, 128}: a simpler
//    register-staged double buffer, 128 x 128 tile, four wave64s in a 2x2
//    arrangement each accumulating (BM/2) x 64 with v_mfma_f32_32x32x16_bf16.
//    A and W tiles are K-contiguous in LDS, 128 bytes per row, with the eight
//    16-byte chunks of row r stored at chunk position c ^ g(r) (see row_xor)
//    so the fragment reads are free of LDS bank conflicts;
//  * grouped_gemv_kernel: a handful of rows per expert (decode), streaming
//    the weights with fp32 dot products;
//  * dense_skinny_kernel: one dense group of 5 to 32 rows, K split over the
//    waves of a workgroup.
//
// Fused SwiGLU: the W rows of a tile are gate rows and the matching up rows F
// positions further; each wave holds gate columns and the matching up columns
// in separate accumulators, so the epilogue pairs them in registers:
// h = bf16(silu(bf16(g)) * bf16(u)).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe_common.h"
#include "wide_sched.h"

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
constexpr int kPipeBK = 64;
constexpr int kPipeStages = 3;
constexpr int kPipeOcc = 1;
constexpr int kPipeGroup = 16;
constexpr int kPipeGnMax = 8;

constexpr int kPipeBM = 128;
constexpr int kPipeBNW = 256;

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)(lds), 16, 0, 0);
}

// The buffer form of the direct-to-LDS load (buffer_load_dwordx4 ... lds):
// 16 bytes per lane from the resource's base + voff + soff (voff per lane,
// soff wave-uniform) into lds + 16 * lane. The step offset goes in as a
// scalar, and, not being a FLAT instruction, it leaves the compiler's LDS
// waits exact: while a global_load_lds is in flight the compiler waits for
// every outstanding LDS read (lgkmcnt(0)) before an MFMA, the prefetched
// fragments of the next sub-step included. Resource: stride 0, the largest
// record count (the callers' offsets stay below 2^32), the gfx9 raw-buffer
// word 3.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, static_cast<int>(voff), soff, 0, 0);
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
// ms with four 128 x 128 waves). In the small-row rings a wave whose rows
// are all past the tile's valid rows skips its MFMAs; a full tile has more
// than 128 valid rows, and its waves compute every row tile.
//
// An expert's only or last tile often has 128 rows or fewer (most experts of
// a skewed routing have a few rows): such a tile loads only 64 or 128 A rows
// and runs the ring of wide_stage_tile, whose deeper stages keep more of the
// weight stream in flight; the padding overhead stays that of 64- or
// 128-row blocks.
//
// Loads, fragments and barriers work as in grouped_gemm_pipe_kernel, over
// the rings described at wide_ring_tile and wide_stage_tile.
using moe::kWideRows;
constexpr int kWideW = 256;

// The wide tile's K loop, K step 64 (whole 128-byte rows, so every L1 -> L2
// request moves a full line). The A part and the W part of a step are 32 KiB
// each; the operand with three slots (the weights, see kWideWDeep) is loaded
// two steps ahead and the other, with two slots, one step ahead (LDS: the A
// slots, then the W slots, 160 KiB). During step kt the loads of A(kt+1) and
// W(kt+2) go into the slots steps kt-1 used, and the wait at the top of step
// kt+1 leaves W(kt+2) in flight: between one and three 32 KiB parts are in
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

constexpr int kWideSlotBytes = kWideRows * 128;
// K rotation of the small-row tiles (wide_stage_tile): when rows are a
// multiple of 4 KiB long (K a multiple of 2048), expert g walks its K blocks
// from block (g * kWideKRot) mod nk and wraps around. Tiles that walk K in
// step put all their requests at one offset inside each 4 KiB, and HBM serves
// such a stream at about 4.4 TB/s instead of 6.1 (a load-only stream of the
// Qwen3-shaped decode gate_up's weights, 805 MB: 183 -> 133 us with one start
// per expert); 7 is odd, so 32 consecutive experts start at 32 different
// 128-byte offsets of a 4 KiB row. All tiles of an expert share the start,
// so the ones that share its weights or rows stay in step. Measured
// (interleaved): Qwen3 decode gate_up 0.192 -> 0.153 ms, Kimi-K2 T = 512 down
// 1.945 -> 1.867 ms, Qwen3 prefill gate_up 0.336 -> 0.331 ms, the
// DeepSeek-V3 shapes unchanged. Rotating the full tiles too, or rows of other
// lengths (the 14 KiB rows of K = 7168), made the prefill GEMMs 1-4% slower.
constexpr int kWideKRot = 7;
// The operand with three slots is loaded two steps ahead, the other one step:
// the weights, the stream that comes from HBM (interleaved against three A
// slots: routed gate_up 2.828 -> 2.770 ms on the DeepSeek-V3 routing, Qwen3
// prefill 0.343 -> 0.336 ms, aligned GLM-5 shapes 1-2% faster; same bytes).
constexpr bool kWideWDeep = true;
constexpr int kWideASlots = kWideWDeep ? 2 : 3;
constexpr int kWideWSlots = kWideWDeep ? 3 : 2;
constexpr int kWideWRing = kWideASlots * kWideSlotBytes;  // first W slot
constexpr int kWideLds = (kWideASlots + kWideWSlots) * kWideSlotBytes;

// SiLU table of the fused gate_up epilogue: entry i is silu_spec of the bf16
// gate moe::silu_table_gate(i) (|g| in [2^-25, 128), both signs), 32 KiB,
// computed at compile time (code-object data: no launch writes it).
__device__ const moe::SiluTable<moe::kSiluTabMid> g_gemm_silu_tab = moe::make_silu_table<moe::kSiluTabMid>();

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

// Per-lane A byte offsets of a wide tile's direct-to-LDS loads: row r of
// the tile (clamped to the last valid row) is A row gather[m_start + r] /
// gather_k, or m_start + r without a gather table (then counted from the
// tile's first row). The gather entries are loaded together, so the
// prologue waits for them once.
template <int A_LOADS, int NW, int RPL>
__device__ __forceinline__ void wide_a_offsets(uint32_t* a_off, const int32_t* __restrict__ gather, int gather_k,
                                               int64_t m_start, int rows, int K, int wave, int lrow, int lpos) {
  if (gather) {
    int32_t gv[A_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) gv[i] = gather[m_start + min((wave * A_LOADS + i) * RPL + lrow, rows - 1)];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = (wave * A_LOADS + i) * RPL + lrow;
      a_off[i] = static_cast<uint32_t>(gv[i] / gather_k) * static_cast<uint32_t>(K) * 2u +
                 static_cast<uint32_t>((lpos ^ wide_swz(r)) << 4);
    }
  } else {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int r = (wave * A_LOADS + i) * RPL + lrow;
      a_off[i] = static_cast<uint32_t>(min(r, rows - 1)) * static_cast<uint32_t>(K) * 2u +
                 static_cast<uint32_t>((lpos ^ wide_swz(r)) << 4);
    }
  }
}

template <int V>
struct Ic {
  static constexpr int value = V;
};

template <bool FUSED, int NW, typename KDone>
__device__ __forceinline__ void wide_ring_tile(uint8_t* smem, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ Wb, const int32_t* __restrict__ go_g,
                                               int64_t m_off, int rows, int nt,
                                               int K, int up_row, int ldc, uint16_t* __restrict__ C,
                                               const int32_t* __restrict__ gather, int gather_k, KDone&& k_done) {
  constexpr int BK = 64, CPR = 8, ROWB = 128, RPL = 8;
  constexpr int AROWS = kWideRows;
  constexpr int WM = NW / 2;                         // wave rows (two wave columns)
  constexpr int TM = kWideRows / WM / 32;            // 32-row MFMA tiles per wave
  constexpr int A_LOADS = AROWS / (NW * RPL);        // per wave per step
  constexpr int B_LOADS = kWideW / (NW * RPL);
  constexpr int NS = BK / 16;
  constexpr int MY_NS = NS;
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
  const char* w_base = reinterpret_cast<const char*>(Wb + static_cast<int64_t>(nt) * (FUSED ? kWideW / 2 : kWideW) * K);
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
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

  // every wave computes all of its row tiles: a full tile has more than 128
  // valid rows, and skipping the MFMAs of a row tile past them cost more in
  // branches than it saved (DeepSeek-V3 gate_up 2.736 -> 2.695 ms without the
  // skip, Qwen3 prefill 2% faster, bit-identical)
  const int row0 = wm * TM * 32;
  const int khalf = lane >> 5;
  // per-lane LDS byte offset of this wave's first A and first W fragment in
  // each sub-step; the other fragments sit at constant offsets from them
  const int a_r0 = row0 + (lane & 31);
  const int b_r0 = (FUSED ? wn * 64 : wn * 128) + (lane & 31);
  uint32_t a_rd[MY_NS], b_rd[MY_NS];
#pragma unroll
  for (int i = 0; i < MY_NS; ++i) {
    const int chunk = i * 2 + khalf;
    a_rd[i] = static_cast<uint32_t>(a_r0 * ROWB + ((chunk ^ wide_swz(a_r0)) << 4));
    b_rd[i] = static_cast<uint32_t>(kWideWRing + b_r0 * ROWB + ((chunk ^ wide_swz(b_r0)) << 4));
    asm volatile("" : "+v"(a_rd[i]), "+v"(b_rd[i]));
  }
  // W fragment tn: rows b_r0 + b_frag_row(tn)
  constexpr int kBFragRow[4] = {0, 32, FUSED ? kWideW / 2 : 64, FUSED ? kWideW / 2 + 32 : 96};

  const int nk = K / BK;
  const __amdgpu_buffer_rsrc_t w_rsrc = dma_rsrc(w_base);
  __amdgpu_buffer_rsrc_t a_rsrc = w_rsrc;  // set once the row offset is known (after W(0) is out)
  // the operand with three slots runs two steps ahead (its loads are issued
  // last in a step), the other one step ahead
  constexpr int FIRST = kWideWDeep ? A_LOADS : B_LOADS;   // loads of the one-ahead operand
  constexpr int LAST = kWideWDeep ? B_LOADS : A_LOADS;    // loads of the two-ahead operand
  auto load_a = [&](int kt, int slot, int i) __attribute__((always_inline)) {
    dma16b(a_rsrc, a_off[i], kt * BK * 2, smem + a_lds0 + slot * kWideSlotBytes + i * RPL * ROWB);
  };
  auto load_w = [&](int kt, int slot, int i) __attribute__((always_inline)) {
    dma16b(w_rsrc, b_off[i], kt * BK * 2, smem + b_lds0 + slot * kWideSlotBytes + i * RPL * ROWB);
  };
  // FUSED: the SiLU table (32 KiB, one slot) takes the place of W(nk) in the
  // W slot that step would have used, loaded during step nk - 2 like a W part
  // (same count per wave, so the waits are unchanged); the wait of the last
  // step lands it
  static_assert(moe::kSiluTabMid * 4 == kWideSlotBytes && moe::kSiluTabMid / 4 / (64 * NW) == B_LOADS,
                "the table loads like one W step");
  const __amdgpu_buffer_rsrc_t tab_rsrc = dma_rsrc(g_gemm_silu_tab.v);
  auto load_tab = [&](int slot, int i) __attribute__((always_inline)) {
    const int c = (i * NW + wave) * 64;  // a wave-wide load fills 64 consecutive 16-byte pieces
    dma16b(tab_rsrc, static_cast<uint32_t>((c + lane) * 16), 0, smem + kWideWRing + slot * kWideSlotBytes + c * 16);
  };
  // prologue: W(0), which needs only the expert and the column tile, goes out
  // before the loads the A rows depend on (the group offset, then the
  // gather entries); then A(0), then step 1 of the two-ahead operand
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) load_w(0, 0, i);
  const int64_t m_start = (go_g ? static_cast<int64_t>(*go_g) : 0) + m_off;
  a_rsrc = dma_rsrc(gather ? A : A + m_start * K);
  wide_a_offsets<A_LOADS, NW, RPL>(a_off, gather, gather_k, m_start, rows, K, wave, lrow, lpos);
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) load_a(0, 0, i);
  if (nk > 1) {
    if constexpr (kWideWDeep) {
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) load_w(1, 1, i);
    } else {
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) load_a(1, 1, i);
    }
  }

  bf16x8_t af[2][TM], bfr[2][4];
  auto step = [&](auto sa, auto sw, int kt) __attribute__((always_inline)) {
    constexpr int SA = decltype(sa)::value, SW = decltype(sw)::value;
    constexpr int A_NEXT = (SA + kWideASlots - 1) % kWideASlots, W_NEXT = (SW + kWideWSlots - 1) % kWideWSlots;
    // every load except step kt+1 of the two-ahead operand (the last issued) must have landed
    if (kt + 1 < nk) wait_dma_barrier<LAST>();
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
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
          acc[tm][tn] = FUSED ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[i & 1][tn], af[i & 1][tm], acc[tm][tn], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i & 1][tm], bfr[i & 1][tn], acc[tm][tn], 0, 0, 0);
      }
      // this sub-step's share of the loads: step kt+1 of the one-ahead
      // operand, then step kt+2 of the two-ahead one
#pragma unroll
      for (int j = i * PER; j < i * PER + PER && j < L; ++j) {
        if (j < FIRST) {
          if (kt + 1 < nk) {
            if constexpr (kWideWDeep) load_a(kt + 1, A_NEXT, j);
            else load_w(kt + 1, W_NEXT, j);
          }
        } else {
          if (kt + 2 < nk) {
            if constexpr (kWideWDeep) load_w(kt + 2, W_NEXT, j - FIRST);
            else load_a(kt + 2, A_NEXT, j - FIRST);
          } else if constexpr (FUSED && kWideWDeep) {
            if (kt + 2 == nk) load_tab(W_NEXT, j - FIRST);
          }
        }
      }
    }
  };
  // six steps per iteration (both slot sequences repeat after six), each
  // guarded, so the loop has a single exit
  for (int kt = 0; kt < nk; kt += 6) {
    step(Ic<0>{}, Ic<0>{}, kt);
    if (kt + 1 < nk) step(Ic<1 % kWideASlots>{}, Ic<1 % kWideWSlots>{}, kt + 1);
    if (kt + 2 < nk) step(Ic<2 % kWideASlots>{}, Ic<2 % kWideWSlots>{}, kt + 2);
    if (kt + 3 < nk) step(Ic<3 % kWideASlots>{}, Ic<3 % kWideWSlots>{}, kt + 3);
    if (kt + 4 < nk) step(Ic<4 % kWideASlots>{}, Ic<4 % kWideWSlots>{}, kt + 4);
    if (kt + 5 < nk) step(Ic<5 % kWideASlots>{}, Ic<5 % kWideWSlots>{}, kt + 5);
  }
  k_done();

  // FUSED with a single K step (no step nk - 2): the table goes into the last
  // W slot once every wave is past its last fragment read
  const int tab_slot = nk >= 2 ? nk % kWideWSlots : kWideWSlots - 1;
  if constexpr (FUSED) {
    if (nk < 2) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) load_tab(tab_slot, i);
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  const float* tab = reinterpret_cast<const float*>(smem + kWideWRing + tab_slot * kWideSlotBytes);
  // the SiLUs come from the table unless a gate of this wave needs the direct
  // evaluation (a negative one of magnitude at least 128): one vote per wave,
  // and one loop for each case
  // Output layout. Unfused: lane l holds column l & 31 of each 32-column
  // tile, rows row0 + tm * 32 + (r & 3) + 4 (l >> 5) + 8 (r >> 2) in
  // register r, and each store writes two 64-byte row pieces. Fused: the
  // MFMAs take the W fragment as their first operand, so lane l holds output
  // row row0 + tm * 32 + (l & 31) and, in registers 4q .. 4q + 3, its four
  // consecutive columns 8q + 4 (l >> 5) .. + 3, one 8-byte store of h each.
  // The bits are the same either way. Measured, interleaved: the fused
  // gate_up 1-2% faster (DeepSeek-V3 2.753 -> 2.726 ms, Qwen3 prefill 0.284
  // -> 0.278 ms); the unfused down 2-11% slower (DeepSeek-V3 1.435 -> 1.469
  // ms, Qwen3 prefill 0.166 -> 0.184 ms), whose stores then touch 32 rows
  // at 16 bytes each. Staging the unfused 256 x 256 tile through LDS for
  // whole 16-byte row stores (16 per lane instead of 128 two-byte ones) left
  // the down projection's time unchanged (DeepSeek-V3 1.450 -> 1.448 ms,
  // Kimi-K2 T=4096 and the aligned GLM-5 shapes within 0.3%).
  auto store = [&](auto use_tab) __attribute__((always_inline)) {
    constexpr bool TAB = decltype(use_tab)::value != 0;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if constexpr (FUSED) {
        const int row = row0 + tm * 32 + (lane & 31);
        if (row >= rows) continue;
        uint16_t* crow = C + (m_start + row) * ldc + 4 * (lane >> 5);
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint16_t gb = moe::f32_to_bf16(acc[tm][tn][4 * q + j]);
              const uint16_t ub = moe::f32_to_bf16(acc[tm][tn + 2][4 * q + j]);
              h[j] = TAB ? moe::f32_to_bf16(silu_tab(tab, gb) * moe::bf16_to_f32(ub)) : moe::swiglu_bf16(gb, ub);
            }
            *reinterpret_cast<uint2*>(crow + nt * (kWideW / 2) + wn * 64 + tn * 32 + 8 * q) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
          if (row >= rows) continue;
          uint16_t* crow = C + (m_start + row) * ldc;
#pragma unroll
          for (int tn = 0; tn < 4; ++tn)
            crow[nt * kWideW + wn * 128 + tn * 32 + (lane & 31)] = moe::f32_to_bf16(acc[tm][tn][r]);
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

// Tiles of at most AR = 64 or 128 valid rows (an expert's only or last
// tile; most experts of a skewed routing have a few rows). What such a tile
// waits for is its weight slice (256 rows x K) streaming in from HBM: with
// the full tile's ring (one W step of 32 KiB in flight) a CU pulls about 21
// GB/s of weights. Here the ring is S equal stages, each the step's AR A
// rows and its 256 W rows (AR = 64: 40 KiB, four stages; AR = 128: 48 KiB,
// three stages), and the loads of step kt + S - 1 go into the slot step
// kt - 1 used, so up to S - 1 steps of weights are in flight.
//
// Waves: AR = 64, 2 x 4 (32 rows x 64 W rows each: one MFMA row tile, two
// column tiles); AR = 128, 2 x 2 waves of 64 rows x 128 W rows, with K split
// between wave groups (the even and the odd 16-wide sub-steps) and the two
// partial sums added through LDS at the end (as the full tile's half case
// did), which halves the fragment reads per MFMA. Fused: a wave's column
// tiles are gate tiles and the matching up tiles.
template <int AR>
struct StageShape;
template <>
struct StageShape<64> {
  static constexpr int TMW = 1, WR = 2, TNW = 2, WC = 4, KS = 1;
};
template <>
struct StageShape<128> {
  static constexpr int TMW = 2, WR = 2, TNW = 4, WC = 2, KS = 2;
};

//
// NC column tiles (nt .. nt + NC - 1, unfused tiles of at most 64 rows and
// K / 64 a multiple of the ring depth): the ring runs on over NC x K / 64
// steps, column tile c's weights one tile stride further, and each column
// tile is stored at its last step while the next one's first steps are in
// flight, so a short-K launch pays the tile's setup (the tile search, the
// group offset, the first loads' latency) once per NC tiles.
template <bool FUSED, int AR, int NW, typename KDone, int NC = 1>
__device__ __forceinline__ void wide_stage_tile(uint8_t* smem, const uint16_t* __restrict__ A,
                                                const uint16_t* __restrict__ Wb, const int32_t* __restrict__ go_g,
                                                int64_t m_off, int rows, int nt,
                                                int K, int up_row, int ldc, uint16_t* __restrict__ C,
                                                const int32_t* __restrict__ gather, int gather_k, int k0,
                                                KDone&& k_done, Ic<NC> = {}) {
  using SS = StageShape<AR>;
  constexpr int BK = 64, CPR = 8, ROWB = 128, RPL = 8;
  constexpr int TMW = SS::TMW, TNW = SS::TNW, WR = SS::WR, WC = SS::WC, KS = SS::KS;
  constexpr int A_BYTES = AR * ROWB;
  constexpr int STAGE = A_BYTES + kWideW * ROWB;
  constexpr int S = kWideLds / STAGE;
  constexpr int A_LOADS = AR / (NW * RPL);           // per wave per step
  constexpr int B_LOADS = kWideW / (NW * RPL);
  constexpr int L = A_LOADS + B_LOADS;
  constexpr int NS = BK / 16;
  constexpr int MY_NS = NS / KS;
  constexpr int PER = (L + MY_NS - 1) / MY_NS;
  static_assert(WR * WC * KS == NW && WR * TMW * 32 == AR && WC * TNW * 32 == kWideW, "wave layout");
  static_assert(S >= 3 && S <= 4 && (S - 2) * L <= 63, "ring");
  static_assert(A_LOADS >= 1 && AR % (NW * RPL) == 0, "A loads");
  static_assert(NC == 1 || (!FUSED && KS == 1), "column-tile runs: unfused, one K group");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wc = wave % WC;
  const int wr = (wave / WC) % WR;
  const int kpar = wave / (WC * WR);
  const int lrow = lane / CPR;
  const int lpos = lane % CPR;

  const __amdgpu_buffer_rsrc_t w_rsrc =
      dma_rsrc(Wb + static_cast<int64_t>(nt) * (FUSED ? kWideW / 2 : kWideW) * K);
  __amdgpu_buffer_rsrc_t a_rsrc = w_rsrc;  // set once the row offset is known (after W(0) is out)
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = (wave * B_LOADS + i) * RPL + lrow;
    const int lr = (FUSED && r >= kWideW / 2) ? up_row + (r - kWideW / 2) : r;
    b_off[i] = static_cast<uint32_t>(lr) * static_cast<uint32_t>(K) * 2u + static_cast<uint32_t>((lpos ^ wide_swz(r)) << 4);
  }
  const int a_lds0 = wave * A_LOADS * RPL * ROWB;
  const int b_lds0 = A_BYTES + wave * B_LOADS * RPL * ROWB;

  floatx16 acc[TMW][TNW];
#pragma unroll
  for (int a = 0; a < TMW; ++a)
#pragma unroll
    for (int b = 0; b < TNW; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  const int row0 = wr * TMW * 32;
  // 32-row MFMA tiles of this wave that hold valid rows (the others are skipped)
  const int live_tm = __builtin_amdgcn_readfirstlane(min(TMW, max(0, (rows - row0 + 31) / 32)));
  const int khalf = lane >> 5;
  const int a_r0 = row0 + (lane & 31);
  const int b_r0 = wc * (FUSED ? TNW / 2 : TNW) * 32 + (lane & 31);
  uint32_t a_rd[MY_NS], b_rd[MY_NS];
#pragma unroll
  for (int i = 0; i < MY_NS; ++i) {
    const int chunk = (KS == 2 ? 2 * i + kpar : i) * 2 + khalf;
    a_rd[i] = static_cast<uint32_t>(a_r0 * ROWB + ((chunk ^ wide_swz(a_r0)) << 4));
    b_rd[i] = static_cast<uint32_t>(A_BYTES + b_r0 * ROWB + ((chunk ^ wide_swz(b_r0)) << 4));
    asm volatile("" : "+v"(a_rd[i]), "+v"(b_rd[i]));
  }
  // W fragment tn: rows b_r0 + b_frag_row(tn) (fused: the gate tiles, then the matching up tiles)
  auto b_frag_row = [](int tn) constexpr {
    return FUSED ? (tn < TNW / 2 ? tn * 32 : kWideW / 2 + (tn - TNW / 2) * 32) : tn * 32;
  };

  const int nk = K / BK;
  const int nkv = nk * NC;  // steps over all NC column tiles
  const int w_col = kWideW * K * 2;  // bytes of one column tile's weight rows
  auto issue = [&](int kv, int slot_base, int first, int count) __attribute__((always_inline)) {
    // step kv reads K block (kt + k0) mod nk of column tile c (kv = c nk + kt)
    const int c = NC == 1 ? 0 : kv / nk;
    const int kr = kv - c * nk + k0;
    const int ko = (kr >= nk ? kr - nk : kr) * BK * 2;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      if (j < first || j >= first + count) continue;
      if (j < B_LOADS)
        dma16b(w_rsrc, b_off[j], ko + c * w_col, smem + slot_base + b_lds0 + j * RPL * ROWB);
      else
        dma16b(a_rsrc, a_off[j - B_LOADS], ko, smem + slot_base + a_lds0 + (j - B_LOADS) * RPL * ROWB);
    }
  };
  // prologue: steps 0 .. S-2, W(0) first: it needs only the expert and the
  // column tile, and goes out before the loads the A rows depend on (the
  // group offset, then the gather entries); the order of the DMA loads is
  // that of issue(), so the waits are unchanged
  issue(0, 0, 0, B_LOADS);
  const int64_t m_start = (go_g ? static_cast<int64_t>(*go_g) : 0) + m_off;
  a_rsrc = dma_rsrc(gather ? A : A + m_start * K);
  wide_a_offsets<A_LOADS, NW, RPL>(a_off, gather, gather_k, m_start, rows, K, wave, lrow, lpos);
  issue(0, 0, B_LOADS, A_LOADS);
  if (nkv > 1) issue(1, STAGE, 0, L);
  if constexpr (S > 3) {
    if (nkv > 2) issue(2, 2 * STAGE, 0, L);
  }

  bf16x8_t af[2][TMW], bfr[2][TNW];
  auto step = [&](auto slot_c, int kt) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int SL_NEXT = (SL + S - 1) % S;  // step kt + S - 1 reuses the slot of step kt - 1
    // steps kt+1 .. kt+S-2 (those that exist) may still be in flight
    const int later = nkv - 1 - kt;
    if (later >= S - 2) wait_dma_barrier<(S - 2) * L>();
    else wait_dma_barrier_dyn<L, S - 3>(later);
    auto read_frags = [&](int i, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int tm = 0; tm < TMW; ++tm)
        af[buf][tm] = *reinterpret_cast<const bf16x8_t*>(smem + a_rd[i] + SL * STAGE + tm * 32 * ROWB);
#pragma unroll
      for (int tn = 0; tn < TNW; ++tn)
        bfr[buf][tn] = *reinterpret_cast<const bf16x8_t*>(smem + b_rd[i] + SL * STAGE + b_frag_row(tn) * ROWB);
    };
    const bool ahead = kt + S - 1 < nkv;
    read_frags(0, 0);
#pragma unroll
    for (int i = 0; i < MY_NS; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < MY_NS) read_frags(i + 1, (i + 1) & 1);
#pragma unroll
      for (int tm = 0; tm < TMW; ++tm) {
        if (tm >= live_tm) break;  // wave-uniform: this and later row tiles hold no valid rows
#pragma unroll
        for (int tn = 0; tn < TNW; ++tn)
          acc[tm][tn] = FUSED ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[i & 1][tn], af[i & 1][tm], acc[tm][tn], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i & 1][tm], bfr[i & 1][tn], acc[tm][tn], 0, 0, 0);
      }
      if (ahead) issue(kt + S - 1, SL_NEXT * STAGE, i * PER, PER);
    }
  };
  // column tile c, then (NC > 1) its store while the next one's loads fly;
  // the slots follow kt mod S because nk is then a multiple of S
  for (int c = 0; c < NC; ++c) {
    const int kb = c * nk;
    for (int kt = 0; kt < nk; kt += S) {
      step(Ic<0>{}, kb + kt);
      if (kt + 1 < nk) step(Ic<1>{}, kb + kt + 1);
      if (kt + 2 < nk) step(Ic<2>{}, kb + kt + 2);
      if constexpr (S > 3) {
        if (kt + 3 < nk) step(Ic<3>{}, kb + kt + 3);
      }
    }
    if constexpr (NC > 1) {
      if (c + 1 < NC) {
        const int row_a = wr * TMW * 32;
#pragma unroll
        for (int tm = 0; tm < TMW; ++tm) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = row_a + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
            if (row < rows) {
              uint16_t* crow = C + (m_start + row) * ldc;
#pragma unroll
              for (int tn = 0; tn < TNW; ++tn)
                crow[(nt + c) * kWideW + wc * TNW * 32 + tn * 32 + (lane & 31)] = moe::f32_to_bf16(acc[tm][tn][r]);
            }
#pragma unroll
            for (int tn = 0; tn < TNW; ++tn) acc[tm][tn][r] = 0.0f;
          }
        }
      }
    }
  }
  k_done();

  // FUSED: the SiLU table goes into the ring's last 32 KiB once every wave is
  // past its last fragment read (above the K-split exchange)
  constexpr int kTabOff = kWideLds - moe::kSiluTabMid * 4;
  if constexpr (FUSED) {
    static_assert(KS == 1 || kTabOff >= 128 * 1024, "the table sits above the exchange");
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int i = 0; i < moe::kSiluTabMid / 4 / (64 * NW); ++i) {
      const int c = (i * NW + wave) * 64;
      dma16b(dma_rsrc(g_gemm_silu_tab.v), static_cast<uint32_t>((c + lane) * 16), 0, smem + kTabOff + c * 16);
    }
  }
  if constexpr (KS == 2) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    typedef float floatx4 __attribute__((ext_vector_type(4)));
    constexpr int XCH = TMW * TNW * 4 * 64;          // floatx4 per wave
    static_assert(NW / 2 * XCH * 16 <= 128 * 1024, "exchange fits below the table");
    floatx4* xch = reinterpret_cast<floatx4*>(smem) + (wr * WC + wc) * XCH;
    if (kpar) {
#pragma unroll
      for (int tm = 0; tm < TMW; ++tm)
#pragma unroll
        for (int tn = 0; tn < TNW; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            floatx4 v = {acc[tm][tn][4 * q], acc[tm][tn][4 * q + 1], acc[tm][tn][4 * q + 2], acc[tm][tn][4 * q + 3]};
            xch[((tm * TNW + tn) * 4 + q) * 64 + lane] = v;
          }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kpar) return;
#pragma unroll
    for (int tm = 0; tm < TMW; ++tm) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int tn = 0; tn < TNW; ++tn) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 v = xch[((tm * TNW + tn) * 4 + q) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[tm][tn][4 * q + e] += v[e];
        }
        asm volatile("" : "+v"(acc[tm][tn]));
      }
    }
  } else if constexpr (FUSED) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
  const float* tab = reinterpret_cast<const float*>(smem + kTabOff);
  // output layout as in wide_ring_tile (fused: a row per lane, 8-byte stores)
  auto store = [&](auto use_tab) __attribute__((always_inline)) {
    constexpr bool TAB = decltype(use_tab)::value != 0;
#pragma unroll
    for (int tm = 0; tm < TMW; ++tm) {
      if constexpr (FUSED) {
        const int row = row0 + tm * 32 + (lane & 31);
        if (row >= rows) continue;
        uint16_t* crow = C + (m_start + row) * ldc + 4 * (lane >> 5);
#pragma unroll
        for (int tn = 0; tn < TNW / 2; ++tn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint16_t gb = moe::f32_to_bf16(acc[tm][tn][4 * q + j]);
              const uint16_t ub = moe::f32_to_bf16(acc[tm][tn + TNW / 2][4 * q + j]);
              h[j] = TAB ? moe::f32_to_bf16(silu_tab(tab, gb) * moe::bf16_to_f32(ub)) : moe::swiglu_bf16(gb, ub);
            }
            *reinterpret_cast<uint2*>(crow + nt * (kWideW / 2) + wc * (TNW / 2) * 32 + tn * 32 + 8 * q) =
                make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
          }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + tm * 32 + (r & 3) + 4 * (lane >> 5) + 8 * (r >> 2);
          if (row >= rows) continue;
          uint16_t* crow = C + (m_start + row) * ldc;
#pragma unroll
          for (int tn = 0; tn < TNW; ++tn)
            crow[(nt + NC - 1) * kWideW + wc * TNW * 32 + tn * 32 + (lane & 31)] = moe::f32_to_bf16(acc[tm][tn][r]);
        }
      }
    }
  };
  if constexpr (FUSED) {
    bool miss = false;
#pragma unroll
    for (int tm = 0; tm < TMW; ++tm)
#pragma unroll
      for (int tn = 0; tn < TNW / 2; ++tn)
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

// The tile of expert g, rows m_off .. m_off + min(r, 256) of its group, by
// column tile nt: the tile body for its row count. k_done() runs once: after
// the tile's last MFMA step, before its epilogue.
template <bool FUSED, int NW, typename KDone>
__device__ __forceinline__ void wide_tile_body(uint8_t* smem, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ W, const Tables& tb, int K,
                                               int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C, int g,
                                               int nt, int64_t m_off, int64_t r, KDone&& k_done) {
  const int rows = r >= kWideRows ? kWideRows : static_cast<int>(r);
  const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;
  // the group's offset is read by the tile after its first weight loads are out
  const int32_t* go_g = tb.gs == nullptr ? nullptr : tb.go + g;
  // the small-row tiles' first K block (see kWideKRot)
  const int k0 = K % 2048 == 0 ? (g * kWideKRot) % (K / 64) : 0;
  if (rows <= 64)
    wide_stage_tile<FUSED, 64, NW>(smem, A, Wb, go_g, m_off, rows, nt, K, up_row, ldc, C, tb.gather, tb.gather_k, k0,
                                   k_done);
  else if (rows <= kWideRows / 2)
    wide_stage_tile<FUSED, 128, NW>(smem, A, Wb, go_g, m_off, rows, nt, K, up_row, ldc, C, tb.gather, tb.gather_k,
                                    k0, k_done);
  else
    wide_ring_tile<FUSED, NW>(smem, A, Wb, go_g, m_off, rows, nt, K, up_row, ldc, C, tb.gather, tb.gather_k, k_done);
}

// ring depth of the 64-row stage tiles (four 40 KiB stages)
constexpr int kSmallRowStages = kWideLds / (64 * 128 + kWideW * 128);
static_assert(kSmallRowStages == 4, "64-row stage ring");

// Slot w of the wide mapping: the tile body for its row count (nothing for a
// slot past the last tile). With NC == 2 (unfused only) the slot covers
// column tiles 2 nt and 2 nt + 1: one continued ring (wide_stage_tile's NC) for an unfused
// tile of at most 64 rows when K / 64 is a multiple of its depth, else the
// two tiles one after the other.
//
// k_done() runs once per call: after the slot's last MFMA step, before its
// epilogue (or at once for an empty slot).
template <bool FUSED, int NW, int NC = 1, typename KDone>
__device__ __forceinline__ void wide_tile(uint8_t* smem, const uint16_t* __restrict__ A,
                                          const uint16_t* __restrict__ W, const Tables& tb, int E, int64_t numel,
                                          const moe::WideGrid& wg, int K, int64_t w_stride, int up_row, int ldc,
                                          uint16_t* __restrict__ C, int w, KDone&& k_done) {
  int g, nt;
  int64_t m_off, r;  // the tile's first row inside its group, rows left from there
  if (!moe::wide_tile_at(tb, E, numel, wg, w, g, nt, m_off, r)) {
    k_done();
    return;
  }
  static_assert(NC == 1 || (NC == 2 && !FUSED), "column-tile pairs: unfused");
  if constexpr (NC == 2) {
    {
      if (r <= 64 && (K / 64) % kSmallRowStages == 0) {
        const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;
        const int32_t* go_g = tb.gs == nullptr ? nullptr : tb.go + g;
        const int k0 = K % 2048 == 0 ? (g * kWideKRot) % (K / 64) : 0;
        wide_stage_tile<false, 64, NW>(smem, A, Wb, go_g, m_off, static_cast<int>(r), 2 * nt, K, up_row, ldc, C,
                                       tb.gather, tb.gather_k, k0, k_done, Ic<2>{});
        return;
      }
    }
    wide_tile_body<FUSED, NW>(smem, A, W, tb, K, w_stride, up_row, ldc, C, g, 2 * nt, m_off, r, [] {});
    // every wave is past its LDS reads before the second tile's loads land
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    wide_tile_body<FUSED, NW>(smem, A, W, tb, K, w_stride, up_row, ldc, C, g, 2 * nt + 1, m_off, r, k_done);
    return;
  }
  wide_tile_body<FUSED, NW>(smem, A, W, tb, K, w_stride, up_row, ldc, C, g, nt, m_off, r, k_done);
}

constexpr int kWideLdsUsed = kWideLds;
static_assert(kWideLdsUsed <= 160 * 1024, "LDS ring too large");
static_assert(kWideLdsUsed >= 128 * 1024, "the half-tile exchange needs 128 KiB");

// One workgroup per slot of the mapping (the hardware places workgroup w on
// XCD w % 8, as the mapping assumes); NC column tiles per slot.
template <bool FUSED, int NW, int NC>
__global__ __launch_bounds__(64 * NW, 1) void grouped_gemm_wide_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, Tables tb, int E, int64_t numel,
    moe::WideGrid wg, int K, int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWideLdsUsed];
  wide_tile<FUSED, NW, NC>(smem, A, W, tb, E, numel, wg, K, w_stride, up_row, ldc, C, static_cast<int>(blockIdx.x),
                           [] {});
}

// Persistent form: a fixed grid of one workgroup per CU (the ring takes the
// CU's whole LDS) walks the same slots. The slots w = 8 j + x of XCD x are
// handed out in the order of j, as the hardware hands out a one-tile-per-
// workgroup grid: workgroup b (on XCD x = b % 8) starts with j = b / 8 and
// then takes j = G / 8 + c, where c is its claim on XCD x's counter (G the
// grid, a multiple of 8), until j passes the last slot. A workgroup claims
// its next slot after the last MFMA step of its current tile, so the atomic's
// round trip is hidden behind the tile's epilogue, and the result goes to the
// other waves through LDS once the tile is done. (Claiming when a tile starts
// reserves the next slot a whole tile early and broke the order's timing:
// 2% slower; claiming after the epilogue was no faster.)
//
// Counters: kClaimSlots x 8 in device memory, zero when the code object is
// loaded. A workgroup that starts inside the slot range claims until a claim
// fails, so a launch makes exactly nx claims on each of its counters (nx the
// slots per XCD: the successful ones, nx - G / 8 if positive, plus one failed
// claim per such workgroup, min(G / 8, nx)); the claim that returns nx - 1 is
// the last and puts the counter back to zero. Every launch thus finds and
// leaves its counters at zero, with no reset launch (also under graph
// replay). Launches that run at the same time need different counters: the
// host gives each stream its own slot, and launches on one stream run in
// order.
constexpr int kClaimSlots = 64;
__device__ uint32_t g_wide_claims[kClaimSlots * 8];

template <bool FUSED, int NW>
__global__ __launch_bounds__(64 * NW, 1) void grouped_gemm_wide_persistent_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W, Tables tb, int E, int64_t numel,
    moe::WideGrid wg, int K, int64_t w_stride, int up_row, int ldc, uint16_t* __restrict__ C, int slot) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kWideLdsUsed];
  // the slots of the actual row tiles (the host's m_tiles is an upper bound)
  if (tb.gs != nullptr) wg.m_tiles = moe::wide_row_tiles(tb.gs, E);
  const int x = static_cast<int>(blockIdx.x & 7);
  const int nx = static_cast<int>(moe::wide_blocks(wg, wg.m_tiles) >> 3);
  uint32_t* claim = g_wide_claims + slot * 8 + x;
  const int g8 = static_cast<int>(gridDim.x >> 3);
  int j = static_cast<int>(blockIdx.x >> 3);
  while (j < nx) {
    uint32_t c = 0;
    wide_tile<FUSED, NW>(smem, A, W, tb, E, numel, wg, K, w_stride, up_row, ldc, C, j * 8 + x, [&] {
      if (threadIdx.x == 0) c = atomicAdd(claim, 1u);
    });
    // every wave is past its LDS reads of the tile (no DMA load is in flight
    // at a tile's end)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (threadIdx.x == 0) {
      if (c == static_cast<uint32_t>(nx - 1)) atomicExch(claim, 0u);
      *reinterpret_cast<volatile int*>(smem) = g8 + static_cast<int>(c);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    j = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(smem));
    // read before the next tile's loads overwrite it
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Group shape for the tile order: GN column tiles (a divisor of n_tiles, at
// most kPipeGnMax) by GM row blocks, about kPipeGroup tiles.
void pipe_groups(int n_tiles, int& gm, int& gn) {
  gn = 1;
  for (int d = kPipeGnMax; d >= 1; --d)
    if (n_tiles % d == 0) {
      gn = d;
      break;
    }
  gm = kPipeGroup / gn > 0 ? kPipeGroup / gn : 1;
}

template <bool FUSED>
int launch_pipe(const uint16_t* A, const uint16_t* W, Tables tb, int64_t numel, int64_t m_blocks, int n_tiles, int K,
                int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  int gm, gn;
  pipe_groups(n_tiles, gm, gn);
  const int64_t groups = moe::ceil_div(m_blocks, gm) * (n_tiles / gn);
  const int64_t blocks = moe::ceil_div(groups, 8) * 8 * gm * gn;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  grouped_gemm_pipe_kernel<FUSED, kPipeBK, kPipeStages, kPipeOcc><<<static_cast<unsigned>(blocks), kThreads, 0, stream>>>(
      A, W, tb, numel, static_cast<int>(m_blocks), n_tiles, K, w_stride, up_row, ldc, C, gm, gn);
  return moe::check_launch(name);
}

constexpr int kWideWaves = 8;

// The claim counters of the streams seen so far: stream i (in order of
// first use, on any device) owns slot i. -1 once every slot is taken, and
// for hipStreamPerThread, whose one handle names a different stream in each
// host thread.
int claim_slot(hipStream_t stream) {
  static std::mutex mu;
  static hipStream_t seen[kClaimSlots];
  static int n = 0;
  if (stream == hipStreamPerThread) return -1;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (seen[i] == stream) return i;
  if (n == kClaimSlots) return -1;
  seen[n] = stream;
  return n++;
}

// Compute units of the current device (0 if unknown), cached per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The wide GEMMs run persistent when an expert's weight matrix (K x the
// output columns, bf16) is at most kPersistentMaxExpertBytes and the experts
// hold at least kPersistentMinRows rows on average (numel / E), the mapping
// has more slots than the grid of one workgroup per CU and the stream has a
// claim slot; otherwise one workgroup per slot. Measured against one
// workgroup per slot (interleaved runs, bit-identical outputs):
//  * Qwen3-shaped prefill (6 MiB experts of 256 rows on average): gate_up
//    0.300 -> 0.293 ms, down 0.172 -> 0.168 ms, the forward 0.520 -> 0.499 ms;
//  * slower: the DeepSeek-V3 and Kimi-K2 shapes (29 to 59 MiB experts), 1 to
//    3% (DeepSeek-V3 gate_up 2.737 -> 2.779 ms, down 1.433 -> 1.449 ms); the
//    Qwen3-shaped decode (32 rows per expert) 2%; the aligned 16 MiB experts
//    of 1024 rows (K = 4096, N = 2048) 3%; the 8 MiB ones (K = 1024, N =
//    4096) even.
// Claiming from one counter for all XCDs instead, which loses the order's
// L2 sharing, was slower on every shape.
constexpr int64_t kPersistentMaxExpertBytes = int64_t(8) << 20;
constexpr int64_t kPersistentMinRows = 128;
constexpr int kPairMaxK = 1024;
constexpr int64_t kPairMaxRows = 64;

template <bool FUSED>
int launch_wide(const uint16_t* A, const uint16_t* W, Tables tb, int E, int64_t numel, int n_tiles, int K,
                int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  // column-tile pairs: unfused grouped launches of short K (at most 16 steps)
  // whose experts average at most 64 rows, so most slots are small-row tiles
  // whose setup is a large part of their time
  const int nc = !FUSED && tb.gs != nullptr && K <= kPairMaxK && n_tiles % 2 == 0 &&
                         numel <= kPairMaxRows * static_cast<int64_t>(E)
                     ? 2
                     : 1;
  moe::WideGrid wg;
  int64_t blocks;
  if (!moe::wide_grid(numel, E, tb.gs != nullptr, n_tiles / nc, wg, blocks))
    return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  const int grid = device_cus() / 8 * 8;
  const bool persistent = static_cast<int64_t>(K) * n_tiles * kWideW * 2 <= kPersistentMaxExpertBytes &&
                          numel >= kPersistentMinRows * E;
  const int slot = nc == 1 && persistent && grid > 0 && blocks > grid ? claim_slot(stream) : -1;
  if (slot >= 0)
    grouped_gemm_wide_persistent_kernel<FUSED, kWideWaves><<<static_cast<unsigned>(grid), 64 * kWideWaves, 0, stream>>>(
        A, W, tb, E, numel, wg, K, w_stride, up_row, ldc, C, slot);
  else if (nc == 2)
    grouped_gemm_wide_kernel<false, kWideWaves, 2><<<static_cast<unsigned>(blocks), 64 * kWideWaves, 0, stream>>>(
        A, W, tb, E, numel, wg, K, w_stride, up_row, ldc, C);
  else
    grouped_gemm_wide_kernel<FUSED, kWideWaves, 1><<<static_cast<unsigned>(blocks), 64 * kWideWaves, 0, stream>>>(
        A, W, tb, E, numel, wg, K, w_stride, up_row, ldc, C);
  return moe::check_launch(name);
}

// ---------------------------------------------------------------------------
// Few-row kernel (decode). When the groups hold a handful of rows (a one-token
// shared expert, a few tokens spread over many experts) the time is the weight
// stream, and 128- or 256-row tiles split the output into too few workgroups
// to reach HBM bandwidth (28 for a 7168 x 18432 down projection). One
// 256-thread workgroup per (group, 256 / LPR output columns): LPR lanes per
// weight row each read 16 bytes a step, so a row's lanes cover LPR * 16
// contiguous bytes, with kGemvUnroll steps in flight per lane, and fp32 dot
// products against the group's rows, kGemvRows at a time (the rows are few:
// read from L2).
constexpr int kGemvCols = 32;   // output columns of a workgroup at 8 lanes per row
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

// The passes of a few-row workgroup over its group's rows, RP rows a pass
// (the weights are streamed once per pass).
template <bool FUSED, int LPR, int RP>
__device__ __forceinline__ void gemv_rows(const uint16_t* __restrict__ A, const uint16_t* __restrict__ wg,
                                          const uint16_t* __restrict__ wu, const Tables& tb, int64_t m0, int rows,
                                          int K, int k_rot, int kc, int col, int ldc, uint16_t* __restrict__ C) {
  constexpr int STEP = LPR * 8;
  constexpr int BLOCK = STEP * kGemvUnroll;
  for (int r0 = 0; r0 < rows; r0 += RP) {
    const int nr = min(RP, rows - r0);
    const uint16_t* arow[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) arow[r] = A + moe::a_row(tb, m0 + r0 + min(r, nr - 1)) * K;
    float acc_g[RP], acc_u[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) acc_g[r] = acc_u[r] = 0.0f;
    // K in steps of STEP (LPR lanes x 8 values): whole blocks of kGemvUnroll
    // steps with every weight load, then every activation load (L1/L2 hits),
    // issued before the arithmetic; then the remaining steps one at a time
    auto block = [&](int kb, auto unroll) __attribute__((always_inline)) {
      constexpr int U = decltype(unroll)::value;
      uint4 vg[U], vu[U], va[U][RP];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kb + u * STEP + kc * 8;
        vg[u] = *reinterpret_cast<const uint4*>(wg + k);
        if (FUSED) vu[u] = *reinterpret_cast<const uint4*>(wu + k);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < RP; ++r)
          va[u][r] = *reinterpret_cast<const uint4*>(arow[r] + kb + u * STEP + kc * 8);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float fg[8], fu[8];
        bf16x8_to_f32(vg[u], fg);
        if (FUSED) bf16x8_to_f32(vu[u], fu);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
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
    auto run = [&](int kb, int k_end) __attribute__((always_inline)) {
      for (; kb + BLOCK <= k_end; kb += BLOCK) block(kb, Ic<kGemvUnroll>{});
      for (; kb < k_end; kb += STEP) block(kb, Ic<1>{});
    };
    run(k_rot, K);
    run(0, k_rot);
    // the LPR lanes of a weight row are consecutive: reduce over lanes 1, 2, 4, ... apart
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int d = 1; d < LPR; d <<= 1) {
        acc_g[r] += __shfl_xor(acc_g[r], d);
        if (FUSED) acc_u[r] += __shfl_xor(acc_u[r], d);
      }
    if (kc == 0) {
#pragma unroll
      for (int r = 0; r < RP; ++r) {
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

template <bool FUSED, int LPR>
__global__ __launch_bounds__(256) void grouped_gemv_kernel(const uint16_t* __restrict__ A,
                                                           const uint16_t* __restrict__ W, Tables tb, int E,
                                                           int64_t numel, int n_tiles, int K, int64_t w_stride,
                                                           int up_row, int ldc, uint16_t* __restrict__ C) {
  constexpr int COLS = 256 / LPR;        // output columns (weight rows) of a workgroup
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
  const int t = threadIdx.x, wr = t / LPR, kc = t % LPR;
  const int col = nt * COLS + wr;
  const uint16_t* wg = W + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(col) * K;
  const uint16_t* wu = W + static_cast<int64_t>(g) * w_stride + static_cast<int64_t>(FUSED ? up_row + col : col) * K;
  // K rotation as in the wide kernel's small-row tiles (kWideKRot): with rows
  // a multiple of 4 KiB long the weight rows are read from element k_rot (a
  // whole unrolled block) to the end, then from 0; a gate column and its up
  // column take the same start, so the fused result is the SwiGLU of the
  // unfused one
  constexpr int BLOCK = LPR * 8 * kGemvUnroll;   // K elements of an unrolled block
  int k_rot = 0;
  if (K % 2048 == 0 && K % BLOCK == 0) {
    const int pair = FUSED ? nt : nt % max(1, ldc / 2 / COLS);
    k_rot = (g * kWideKRot + pair) % (K / BLOCK) * BLOCK;
  }
  // one row (a decode token's expert, or a one-token dense group): the
  // single-row passes, with a quarter of the activation loads
  if (rows == 1)
    gemv_rows<FUSED, LPR, 1>(A, wg, wu, tb, m0, rows, K, k_rot, kc, col, ldc, C);
  else
    gemv_rows<FUSED, LPR, kGemvRows>(A, wg, wu, tb, m0, rows, K, k_rot, kc, col, ldc, C);
}

// Lanes per weight row: 32 (8 rows a workgroup) when K is a multiple of 256,
// else 8 (32 rows). The bytes in flight are the launch's weight rows times
// the lanes per row times 64, which at 8 lanes left a one-token dense down
// projection (7168 rows) far short of what HBM needs; on the one-token
// Kimi-K2 shapes, with the single-row passes (interleaved, ms): shared
// gate_up 0.120 -> 0.088, shared down 0.088 -> 0.053, routed gate_up 0.092
// -> 0.080, routed down 0.061 -> 0.049.
template <bool FUSED>
int launch_gemv(const uint16_t* A, const uint16_t* W, Tables tb, int E, int64_t numel, int K, int64_t w_stride,
                int up_row, int ldc, uint16_t* C, hipStream_t stream, const char* name) {
  const bool wide_rows = K % (32 * 8) == 0 && ldc % (256 / 32) == 0;
  const int n_tiles = ldc / (wide_rows ? 256 / 32 : 256 / 8);
  const int64_t slots = tb.gs ? std::min<int64_t>(numel, E) : 1;
  const int64_t blocks = slots * n_tiles;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  if (wide_rows)
    grouped_gemv_kernel<FUSED, 32><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(A, W, tb, E, numel, n_tiles, K,
                                                                                      w_stride, up_row, ldc, C);
  else
    grouped_gemv_kernel<FUSED, 8><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(A, W, tb, E, numel, n_tiles, K,
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
constexpr int kSkinnyOcc = 2;
constexpr int kSkinnyDepth = 2;
constexpr int kSkinnyMaxRows = 32;

template <bool FUSED>
__global__ __launch_bounds__(64 * kSkinnyWaves, kSkinnyOcc) void dense_skinny_kernel(const uint16_t* __restrict__ A,
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
  // K rotation as in the wide kernel's small-row tiles (kWideKRot): with rows
  // a multiple of 4 KiB long the steps start at k_rot, a multiple of the wave
  // count (every wave keeps its steps, and the partial sums their order), the
  // same for a gate column and its up column
  int k_rot = 0;
  if (K % 2048 == 0) k_rot = (FUSED ? nt : nt % max(1, ldc / 2 / kSkinnyCols)) * kSkinnyWaves % nk;
  if (n_my > 0) {
    uint4 bw[D][NB][4], ba[D][4];
    // loads of this wave's step s into slot d (steps past the last reload it
    // and add zero); site: a distinct empty asm statement after each call
    // site's loads keeps the optimizer from merging the prologue's loads
    // with the loop's into one block
    auto issue = [&](auto dd, int s, auto site) __attribute__((always_inline)) {
      constexpr int d = decltype(dd)::value;
      const int kr = min(s, n_my - 1) * kSkinnyWaves + wave + k_rot;
      const int ko = (kr >= nk ? kr - nk : kr) * 64;
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

constexpr int kGemvMaxRows = 4;
constexpr int kGemvGroupedPct = 10;

template <bool FUSED>
int launch(const uint16_t* A, const uint16_t* W, Tables tb, int64_t numel, int E, int block_m, int padding_m,
           int n_tiles, int K, int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream,
           const char* name, bool a_off32 = true) {
  const int64_t m_blocks = tb.gs ? moe_num_blocks(numel, E, block_m, padding_m) : moe::ceil_div(numel, block_m);
  const int64_t blocks = m_blocks * n_tiles;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  // ldc is the output width: F for the fused gate_up, 2F or H otherwise
  const int pipe_cols = FUSED ? kPipeBNW / 2 : kPipeBNW;
  // Grouped launches take the 256-row kernel whatever the rows per expert:
  // an expert's tile of at most 64 or 128 rows runs a ring of deeper stages
  // (wide_stage_tile), which beat the 128-row kernel on the decode-like
  // shapes too (interleaved: Kimi-K2 T = 512 gate_up 3.64 -> 3.59 ms, down
  // 2.09 -> 1.97 ms; Qwen3 decode 0.201 -> 0.189 / 0.094 -> 0.089 ms).
  //
  // Few rows (at most 4 in one dense group, or numel <= E / 10 over the
  // experts: one decode token's top-k): the weight-streaming kernel (at 256
  // rows over 384 experts the row-tile kernels are faster)
  const bool few_rows = tb.gs ? numel * 100 <= kGemvGroupedPct * static_cast<int64_t>(E) : numel <= kGemvMaxRows;
  if (few_rows && K % 64 == 0 && ldc % kGemvCols == 0)
    return launch_gemv<FUSED>(A, W, tb, E, numel, K, w_stride, up_row, ldc, C, stream, name);
  // one dense group of up to 32 rows: the K-split skinny kernel
  if (tb.gs == nullptr && tb.gather == nullptr && numel <= kSkinnyMaxRows && K % 64 == 0 &&
      ldc % kSkinnyCols == 0)
    return launch_skinny<FUSED>(A, W, numel, K, up_row, ldc, C, stream, name);
  // the wide kernel addresses a tile's A and W rows with 32-bit byte offsets
  // (with a gather table, A's offsets count from its first row: a_off32)
  const bool wide_fits = (static_cast<int64_t>(up_row) + kWideW) * K * 2 < (int64_t(1) << 32) && a_off32;
  constexpr int kWideDenseMinTiles = 128;
  // a dense launch with few 256-row tiles: the 128-row kernel gives it twice the workgroups
  const bool dense_few = tb.gs == nullptr && moe::ceil_div(numel, kWideRows) * (ldc / pipe_cols) < kWideDenseMinTiles;
  if (block_m == kPipeBM && ldc % pipe_cols == 0 && K % 64 == 0 && wide_fits && !dense_few)
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
