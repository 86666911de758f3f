// SwiGLU and the fused SwiGLU + FP8 (OCP e4m3) activation quantizer.
//
// Both take every SiLU from a lookup table in LDS (a lookup and a few selects
// instead of an exp polynomial and a divide), which moves them from ALU-bound
// towards the HBM bound. The 8320 exact silu_spec values of moe_common.h's
// table are computed at compile time into the constant array g_silu_tab (part
// of the code object: no launch writes it), and each workgroup copies it into
// LDS.
//
// swiglu_quant_fp8: one 512-thread workgroup per 128x128 block of
// h = SiLU(gate) * up. Thread (rg, cg) of 32x16 owns rows rg*4..rg*4+3 and
// columns cg*8..cg*8+7 of the block, so
//   * gate/up loads are 16-byte vectors and a row's 16 threads read 256
//     contiguous bytes of each half;
//   * the 1x128 row amax is a reduction over the 16 lanes of a row (xor 1..8),
//     on the bf16 magnitude bits with packed 16-bit max;
//   * the 128x128 block amax adds a reduction over row groups and one LDS
//     exchange between the eight waves;
//   * the row-layout store is 8 bytes per thread (a row's 128 bytes come
//     from 16 consecutive lanes); the transposed codes are gathered in LDS
//     (in the table's space, free once the SiLUs are done) and written as
//     16-byte pieces, eight lanes per 128-byte line of q_t;
//   * codes are packed with the converter's half-word select, four per word
//     without masks or shifts.
// Measured: the block-per-workgroup shape with many workgroups in flight
// beats persistent or multi-block workgroups that load the table once (their
// lockstep phases leave HBM idle while they compute).
// h never leaves registers. code = e4m3(RN32(h / s)): the quotient is taken
// as RN32(h * RN64(1/s)) in fp64. That is the correctly rounded fp32
// quotient: the fp64 product is within 2^-52 (relative) of h/s, while h/s
// (h with 8 significant bits, s with 24) is either exact in fp64 or at least
// 2^-47 away from every fp32 rounding boundary, and it is never exactly a
// boundary because that would need a 25-bit odd factor dividing an 8-bit one.
#include <algorithm>

#include "moe_common.h"

namespace {

constexpr int kTile = 128;

__device__ __forceinline__ uint32_t wave_umax_xor(uint32_t v, int first, int last) {
  for (int off = first; off <= last; off <<= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}

// Two fp32 values -> two e4m3 bytes written into half `hi` of `old` (the
// other half is kept).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2(float a, float b, uint32_t old) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// Elementwise max of two packed 16-bit halves over lanes first, 2*first, ..., last apart.
__device__ __forceinline__ uint32_t wave_pkmax_xor(uint32_t v, int first, int last) {
  for (int off = first; off <= last; off <<= 1)
    v = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(as_u16x2(v), as_u16x2(static_cast<uint32_t>(
                                                                                 __shfl_xor(static_cast<int>(v), off)))));
  return v;
}

// Two fp32 products rounded to bf16 (nearest even), packed low | high << 16.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return static_cast<uint32_t>(moe::f32_to_bf16(lo)) | (static_cast<uint32_t>(moe::f32_to_bf16(hi)) << 16);
}

// The 8320 silu_spec values, evaluated at compile time (code-object data).
__device__ const moe::SiluTable<moe::kSiluTabSize> g_silu_tab = moe::make_silu_table<moe::kSiluTabSize>();

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kSiluTabPieces = moe::kSiluTabSize / 4;                   // 16-byte pieces
constexpr int kSiluTabLds = (kSiluTabPieces + 63) / 64 * 64 * 4;        // floats: whole 64-piece loads
static_assert(moe::kSiluTabSize % 4 == 0, "16-byte pieces");

// Starts copying g_silu_tab into tab[kSiluTabLds] with direct-to-LDS loads
// (no VGPRs); thread t of n, n a multiple of 64. A wave-wide load fills 64
// consecutive pieces; in the last one, lanes past the table re-read its last
// piece into the padding. The caller waits for the loads and barriers.
__device__ __forceinline__ void load_silu_table(float* tab, int t, int n) {
  const int lane = t & 63;
  for (int c = (t >> 6) * 64; c < kSiluTabPieces; c += n) {
    const int src = min(c + lane, kSiluTabPieces - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const float4*>(g_silu_tab.v) + src,
                                     (lds_void_t*)(reinterpret_cast<float4*>(tab) + c), 16, 0, 0);
  }
}

constexpr int kSwigluChunks = 4;   // 16-byte chunks per thread

__global__ __launch_bounds__(256) void swiglu_kernel(const uint4* __restrict__ gu, uint32_t total, uint32_t f8,
                                                     uint4* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) float tab[kSiluTabLds];
  load_silu_table(tab, threadIdx.x, 256);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const uint32_t base = blockIdx.x * (256u * kSwigluChunks) + threadIdx.x;
  uint4 g[kSwigluChunks], u[kSwigluChunks];
#pragma unroll
  for (int q = 0; q < kSwigluChunks; ++q) {
    const uint32_t i = min(base + q * 256u, total - 1u);
    const uint32_t m = i / f8, c = i - m * f8;
    g[q] = gu[static_cast<uint64_t>(m) * 2 * f8 + c];
    u[q] = gu[static_cast<uint64_t>(m) * 2 * f8 + f8 + c];
  }
#pragma unroll
  for (int q = 0; q < kSwigluChunks; ++q) {
    const uint32_t i = base + q * 256u;
    if (i >= total) break;
    const uint32_t gw[4] = {g[q].x, g[q].y, g[q].z, g[q].w};
    const uint32_t uw[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = moe::swiglu_bf16_tab(tab, gw[k] & 0xFFFFu, uw[k] & 0xFFFFu);
      const uint32_t hi = moe::swiglu_bf16_tab(tab, gw[k] >> 16, uw[k] >> 16);
      o[k] = lo | (hi << 16);
    }
    h[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

constexpr int kQuantThreads = 512;   // per 128x128 block: 32 row groups of 4 x 16 column groups of 8

// The rows of padded 128-row block pb of the expanded layout: groups are
// consecutive row ranges of gs[0..E), each taking ceil(gs[e]/128) blocks.
// Wave-wide prefix sums over the group sizes, 64 at a time, find the group
// and the block inside it; the sizes of up to kGroupScanBatch * 64 groups are
// loaded at once. The sums are DPP row shifts and broadcasts: with
// __shfl_up, whose data goes through the LDS permute path, the scan before a
// workgroup's first load made the 131072 x 6144 per-block form over 256
// groups 9% slower. Returns false past the groups' last block.
constexpr int kGroupScanBatch = 8;
__device__ __forceinline__ bool find_group_block(const int32_t* __restrict__ gs, int E, int pb, int& r0, int& rows) {
  const int lane = threadIdx.x & 63;
  int before_b = 0, before_r = 0;
  for (int base0 = 0; base0 < E; base0 += 64 * kGroupScanBatch) {
    int cnt[kGroupScanBatch];
#pragma unroll
    for (int b = 0; b < kGroupScanBatch; ++b) {
      const int e = base0 + b * 64 + lane;
      cnt[b] = e < E ? gs[e] : 0;
    }
#pragma unroll
    for (int b = 0; b < kGroupScanBatch; ++b) {
      if (base0 + b * 64 >= E) break;
      const int n = cnt[b];
      const int nb = (n + kTile - 1) / kTile;
      const int incl_b = moe::wave_incl_sum(nb), incl_r = moe::wave_incl_sum(n);
      const int total_b = __builtin_amdgcn_readlane(incl_b, 63), total_r = __builtin_amdgcn_readlane(incl_r, 63);
      if (pb < before_b + total_b) {
        const int j = __builtin_ctzll(__ballot(before_b + incl_b > pb));
        const int n_j = __builtin_amdgcn_readlane(n, j);
        const int first_b = before_b + __builtin_amdgcn_readlane(incl_b, j) - __builtin_amdgcn_readlane(nb, j);
        const int first_r = before_r + __builtin_amdgcn_readlane(incl_r, j) - n_j;
        const int q = pb - first_b;
        r0 = first_r + q * kTile;
        rows = min(kTile, n_j - q * kTile);
        return true;
      }
      before_b += total_b;
      before_r += total_r;
    }
  }
  return false;
}

// One 512-thread workgroup per (padded 128-row block pb, 128-column tile fb).
// SWIGLU: x is [M, 2K] (gate | up) and the value quantized is
// bf16(SiLU(gate) * up); otherwise x is the bf16 [M, K] activation itself.
// PER_TILE: the transposed scales are per column and 128-row tile (one per
// q_t row of the block) instead of one per 128x128 block. gs == nullptr: one
// group of M rows (GROUPED = false). Blocks past the groups' padded total
// write zero codes and scales into their q_t columns.
template <bool SWIGLU, bool PER_TILE, bool GROUPED, bool TRANS = true, int NB = 1>
__global__ __launch_bounds__(kQuantThreads) void tile_quant_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                   const int32_t* __restrict__ gs, int E, int m_pad,
                                                                   int n_fb, uint8_t* __restrict__ q_row,
                                                                   float* __restrict__ s_row,
                                                                   uint8_t* __restrict__ q_t,
                                                                   float* __restrict__ s_t) {
  // the SiLU table, and once the SiLUs are done the transposed codes of the
  // block; with two SwiGLU blocks a workgroup the second block still needs
  // the table, so the codes get a 16 KiB area of their own
  constexpr int kLds = SWIGLU ? kSiluTabLds : kTile * kTile / 4;
  constexpr bool kOwnStage = SWIGLU && NB > 1;
  __shared__ __attribute__((aligned(16))) float tab[kLds];
  __shared__ __attribute__((aligned(16))) uint8_t stage[kOwnStage ? kTile * kTile : 16];
  __shared__ uint32_t s_wmax[kQuantThreads / 64][PER_TILE ? kTile / 2 : 1];
  static_assert(kLds * 4 >= kTile * kTile, "the transposed block fits in the table's space");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 15, rg = tid >> 4;
  // NB adjacent column blocks per workgroup (their loads in flight together)
  const int n_fbw = n_fb / NB;
  const int fb0 = (blockIdx.x % n_fbw) * NB;
  const int pb = blockIdx.x / n_fbw;
  const int n_pb = m_pad / kTile;

  int r0, rows;
  bool live;
  if (!GROUPED) {
    r0 = pb * kTile;
    rows = min(kTile, M - r0);
    live = rows > 0;
  } else {
    live = find_group_block(gs, E, pb, r0, rows);
    // sizes that are negative or sum past M (a caller error) must not move a
    // block outside [0, M): such rows are dropped
    rows = min(rows, M - r0);
    live = live && r0 >= 0 && rows > 0;
  }
  if (!live) {
    if constexpr (!TRANS) return;
    // past the last group: zero codes and scales in these blocks' q_t columns
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int fb = fb0 + cb;
#pragma unroll
      for (int r = 0; r < (kTile * kTile / 16) / kQuantThreads; ++r) {
        const int piece = tid + kQuantThreads * r;
        const int c = piece >> 3, part = piece & 7;
        *reinterpret_cast<uint4*>(q_t + static_cast<int64_t>(fb * kTile + c) * m_pad + pb * kTile + part * 16) =
            make_uint4(0u, 0u, 0u, 0u);
      }
      if (PER_TILE) {
        if (tid < kTile) s_t[static_cast<int64_t>(fb * kTile + tid) * n_pb + pb] = 0.0f;
      } else if (tid == 0) {
        s_t[static_cast<int64_t>(fb) * n_pb + pb] = 0.0f;
      }
    }
    return;
  }
  const int lrow0 = rg * 4;   // this thread's first row inside the block

  // all 8 (SWIGLU) or 4 loads first; rows past the block's valid rows read
  // its last row (in bounds) and are masked. The input is read once, so the
  // loads are non-temporal (same bytes; interleaved, MALL flushed: 131072 x
  // 6144 over 256 groups 696.7 -> 690.0 us per block, 906 -> 899 us per tile,
  // SwiGLU 131072 x 8192 708.7 -> 690.1 us; M = 32768 unchanged, 89.8 -> 89.7 us)
  uint4 gb[NB][4], ub[SWIGLU ? NB : 1][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = r0 + min(lrow0 + i, rows - 1);
    const uint16_t* rp = x + m * (SWIGLU ? 2 : 1) * K;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) gb[cb][i] = moe::load_stream16(rp + (fb0 + cb) * kTile + cg * 8);
    if (SWIGLU) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) ub[cb][i] = moe::load_stream16(rp + K + (fb0 + cb) * kTile + cg * 8);
    }
  }
  if (SWIGLU) load_silu_table(tab, tid, kQuantThreads);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (SWIGLU) __syncthreads();

  // each block in turn: fb, its first column col0 and its loaded rows g (the
  // row-layout-only form, which returns at the end of its block, has NB = 1)
  static_assert(NB == 1 || TRANS, "one block without the transposed layout");
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
  if (cb > 0) __syncthreads();  // the previous block is done with the LDS staging and s_wmax
  const int fb = fb0 + cb;
  const uint4 (&g)[4] = gb[cb];
  const uint4 (&u)[4] = ub[SWIGLU ? cb : 0];
  const int col0 = fb * kTile + cg * 8;
  uint32_t hp[4][4];  // h as bf16 pairs: hp[i][k] holds columns 2k, 2k+1 of row i
  if constexpr (SWIGLU) {
    // Fast path: every gate of the wave is in the table's range (bf16
    // magnitude bits in [0x3300, 0x4300), checked two at a time with packed
    // 16-bit subtract and max), so a SiLU is one lookup at
    // sign * 4096 + (magnitude - 0x3300). Otherwise the wave takes the general
    // lookup (closed forms outside the range).
    u16x2 worst = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) worst = __builtin_elementwise_max(worst, as_u16x2(gw[k] & 0x7FFF7FFFu) - u16x2{0x3300, 0x3300});
    }
    const bool fast = __ballot(max(worst.x, worst.y) >= 0x1000) == 0;
    if (fast) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
        const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float s_lo = tab[((gw[k] >> 3) & 0x1000u) | ((gw[k] & 0x7FFFu) - 0x3300u)];
          const float s_hi = tab[((gw[k] >> 19) & 0x1000u) | (((gw[k] >> 16) & 0x7FFFu) - 0x3300u)];
          hp[i][k] = bf16_pair(s_lo * __uint_as_float(uw[k] << 16), s_hi * __uint_as_float(uw[k] & 0xFFFF0000u));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t gw[4] = {g[i].x, g[i].y, g[i].z, g[i].w};
        const uint32_t uw[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          hp[i][k] = bf16_pair(moe::silu_lookup(tab, gw[k] & 0xFFFFu) * __uint_as_float(uw[k] << 16),
                               moe::silu_lookup(tab, gw[k] >> 16) * __uint_as_float(uw[k] & 0xFFFF0000u));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hp[i][0] = g[i].x;
      hp[i][1] = g[i].y;
      hp[i][2] = g[i].z;
      hp[i][3] = g[i].w;
    }
  }
  if (rows < kTile) {
    // rows past the block's valid rows (a group's or the array's last block) are zero
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) hp[i][k] = lrow0 + i < rows ? hp[i][k] : 0u;
  }
  auto hv = [&](int i, int j) __attribute__((always_inline)) {
    return __uint_as_float((j & 1) ? (hp[i][j >> 1] & 0xFFFF0000u) : (hp[i][j >> 1] << 16));
  };

  // 1x128 row amax (16 lanes per row), and the 128x128 block amax or the
  // per-column amax, on the bf16 magnitude bits (their integer order is the
  // order of |h|)
  float amax_row[4];
  uint32_t blk_bits = 0u;
  u16x2 colm[4] = {};   // PER_TILE: magnitude maxima of this thread's 8 columns over its 4 rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u16x2 mag = as_u16x2(hp[i][k] & 0x7FFF7FFFu);
      m2 = __builtin_elementwise_max(m2, mag);
      if (PER_TILE) colm[k] = __builtin_elementwise_max(colm[k], mag);
    }
    const uint32_t a = wave_umax_xor(max(static_cast<uint32_t>(m2.x), static_cast<uint32_t>(m2.y)), 1, 8);
    amax_row[i] = __uint_as_float(a << 16);
    blk_bits = max(blk_bits, a);
  }
  // the transposed scales: per block, or per column (s_col[j] for this
  // thread's column col0 + j)
  float sb = 0.0f, s_col[8];
  double inv_sb = 0.0, inv_col[8];
  if constexpr (!TRANS) {
    // row layout only: no transposed scales
  } else if constexpr (PER_TILE) {
    // columns: over the wave's 4 row groups (lanes 16 apart), then the 8 waves through LDS
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t v = wave_pkmax_xor(__builtin_bit_cast(uint32_t, colm[k]), 16, 32);
      if (lane < 16) s_wmax[wave][cg * 4 + k] = v;
    }
    __syncthreads();  // also: every SiLU lookup is done, the table's space is free
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u16x2 c2 = as_u16x2(s_wmax[0][cg * 4 + k]);
#pragma unroll
      for (int w = 1; w < kQuantThreads / 64; ++w) c2 = __builtin_elementwise_max(c2, as_u16x2(s_wmax[w][cg * 4 + k]));
      s_col[2 * k] = __uint_as_float(static_cast<uint32_t>(c2.x) << 16) / 448.0f;
      s_col[2 * k + 1] = __uint_as_float(static_cast<uint32_t>(c2.y) << 16) / 448.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) inv_col[j] = s_col[j] > 0.0f ? 1.0 / static_cast<double>(s_col[j]) : 0.0;
    if (rg == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) s_t[static_cast<int64_t>(col0 + j) * n_pb + pb] = s_col[j];
    }
  } else {
    blk_bits = wave_umax_xor(blk_bits, 16, 32);
    if (lane == 0) s_wmax[wave][0] = blk_bits;
    __syncthreads();  // also: every SiLU lookup is done, the table's space is free
    uint32_t bb = s_wmax[0][0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) bb = max(bb, s_wmax[w][0]);
    const float blk = __uint_as_float(bb << 16);
    sb = blk / 448.0f;
    inv_sb = sb > 0.0f ? 1.0 / static_cast<double>(sb) : 0.0;
    if (tid == 0) s_t[static_cast<int64_t>(fb) * n_pb + pb] = sb;
  }

  // codes: two rows at a time; each h is widened to fp64 once and divided
  // by both scales. Row codes pack four per word; a column's four transposed
  // codes (rows 0-3) fill its word, rows (0,1) in the low half, (2,3) high.
  uint32_t qt[8];
#pragma unroll
  for (int i = 0; i < 4; i += 2) {
    float sr[2];
    double inv_r[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      sr[r] = amax_row[i + r] / 448.0f;
      inv_r[r] = sr[r] > 0.0f ? 1.0 / static_cast<double>(sr[r]) : 0.0;
    }
    float qr[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double d0 = static_cast<double>(hv(i, j)), d1 = static_cast<double>(hv(i + 1, j));
      qr[0][j] = static_cast<float>(d0 * inv_r[0]);
      qr[1][j] = static_cast<float>(d1 * inv_r[1]);
      if constexpr (TRANS) {
        const double inv_t = PER_TILE ? inv_col[j] : inv_sb;
        float b0 = static_cast<float>(d0 * inv_t), b1 = static_cast<float>(d1 * inv_t);
        if (PER_TILE && !(s_col[j] > 0.0f)) b0 = b1 = 0.0f;   // an all-zero column tile: codes 0
        if (i == 0)
          qt[j] = fp8x2<false>(b0, b1, 0u);
        else
          qt[j] = fp8x2<true>(b0, b1, qt[j]);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int lr = lrow0 + i + r;
      uint32_t w0 = fp8x2<true>(qr[r][2], qr[r][3], fp8x2<false>(qr[r][0], qr[r][1], 0u));
      uint32_t w1 = fp8x2<true>(qr[r][6], qr[r][7], fp8x2<false>(qr[r][4], qr[r][5], 0u));
      // an all-zero row has scale 0 and codes 0 (a -0.0 would otherwise encode as 0x80)
      w0 = sr[r] > 0.0f ? w0 : 0u;
      w1 = sr[r] > 0.0f ? w1 : 0u;
      if (lr < rows) {
        const int64_t m = r0 + lr;
        *reinterpret_cast<uint2*>(q_row + m * K + col0) = make_uint2(w0, w1);
        if (cg == 0) s_row[m * n_fb + fb] = sr[r];
      }
    }
  }
  if constexpr (!TRANS) return;
  if (!PER_TILE && !(sb > 0.0f)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) qt[j] = 0u;
  }
  // transposed layout through LDS: the block's column c is 128 bytes (its
  // rows) of q_t row fb*128 + c; this thread's 4 rows of a column are 4 of
  // them. Rows past the valid ones hold code 0, which is the required padding.
  uint8_t* tq = kOwnStage ? stage : reinterpret_cast<uint8_t*>(tab);
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t*>(tq + (cg * 8 + j) * kTile + rg * 4) = qt[j];
  __syncthreads();
  // then 16-byte pieces, eight lanes per q_t row: whole 128-byte lines
#pragma unroll
  for (int r = 0; r < (kTile * kTile / 16) / kQuantThreads; ++r) {
    const int piece = tid + kQuantThreads * r;
    const int c = piece >> 3, part = piece & 7;
    *reinterpret_cast<uint4*>(q_t + static_cast<int64_t>(fb * kTile + c) * m_pad + pb * kTile + part * 16) =
        *reinterpret_cast<const uint4*>(tq + c * kTile + part * 16);
  }
  }
}

}  // namespace

extern "C" int swiglu(const uint16_t* gate_up, int64_t M, int F, uint16_t* h, hipStream_t stream) {
  using namespace moe;
  if (M < 0 || F < 8 || F % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "swiglu: M=%lld F=%d (F must be a positive multiple of 8)", (long long)M, F);
  if (M == 0) return MOE_OK;
  const int64_t total = M * (F / 8);
  if (total >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "swiglu: M*F too large");
  if (!gate_up || !h) return fail(MOE_ERR_INVALID_ARG, "swiglu: null pointer");
  if (!aligned16(gate_up) || !aligned16(h)) return fail(MOE_ERR_INVALID_ARG, "swiglu: pointers not 16-byte aligned");
  const int64_t blocks = ceil_div(total, 256 * kSwigluChunks);
  swiglu_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(reinterpret_cast<const uint4*>(gate_up),
                                                                   static_cast<uint32_t>(total),
                                                                   static_cast<uint32_t>(F / 8),
                                                                   reinterpret_cast<uint4*>(h));
  return check_launch("swiglu");
}

namespace {

template <bool SWIGLU>
int launch_tile_quant(const uint16_t* x, int64_t M, int K, const int32_t* gs, int E, int per_tile, int64_t m_pad,
                      uint8_t* q_row, float* s_row, uint8_t* q_t, float* s_t, hipStream_t stream, const char* name) {
  const int n_fb = K / kTile;
  const int64_t blocks = (m_pad / kTile) * n_fb;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: too many blocks", name);
  const unsigned grid = static_cast<unsigned>(blocks);
  const int Mi = static_cast<int>(M), mp = static_cast<int>(m_pad);
  constexpr int kTqPairMinWgs = 1024;
  // Grouped launches: two adjacent column blocks per workgroup, their loads in
  // flight together (with the SwiGLU the second block's transposed codes take
  // their own LDS, the table staying for it): measured faster on every
  // grouped shape tried. Ungrouped launches were slower paired (SwiGLU,
  // M x 2048: 0.094 -> 0.105 ms) and keep one block per workgroup, as does a
  // small launch, where halving the grid would leave compute units idle
  // (1024 paired workgroups = 4 per CU).
  const bool pair = gs != nullptr && n_fb % 2 == 0 && blocks >= 2 * kTqPairMinWgs;
  const unsigned grid2 = static_cast<unsigned>(blocks / 2);
  // (the per-tile SwiGLU form is unpaired: two of its blocks need more than
  // 128 VGPRs, one workgroup per CU)
#define MOE_TQ(PT, GR)                                                                                            \
  do {                                                                                                            \
    constexpr int kNB = (GR && !(SWIGLU && PT)) ? 2 : 1;                                                         \
    if (pair && kNB == 2)                                                                                         \
      tile_quant_kernel<SWIGLU, PT, GR, true, kNB><<<grid2, kQuantThreads, 0, stream>>>(                         \
          x, Mi, K, gs, E, mp, n_fb, q_row, s_row, q_t, s_t);                                                     \
    else                                                                                                          \
      tile_quant_kernel<SWIGLU, PT, GR><<<grid, kQuantThreads, 0, stream>>>(x, Mi, K, gs, E, mp, n_fb, q_row,     \
                                                                            s_row, q_t, s_t);                     \
  } while (0)
  if (q_t == nullptr) {
    // row layout only (no transposed outputs): one pass over ceil(M/128) blocks
    tile_quant_kernel<SWIGLU, false, false, false><<<grid, kQuantThreads, 0, stream>>>(
        x, Mi, K, nullptr, 0, mp, n_fb, q_row, s_row, nullptr, nullptr);
  } else if (gs == nullptr) {
    if (per_tile) MOE_TQ(true, false);
    else MOE_TQ(false, false);
  } else {
    if (per_tile) MOE_TQ(true, true);
    else MOE_TQ(false, true);
  }
#undef MOE_TQ
  return moe::check_launch(name);
}

}  // namespace

extern "C" int swiglu_quant_fp8(const uint16_t* gate_up, int64_t M, int F, uint8_t* q_row, float* s_row,
                                uint8_t* q_t, float* s_t, hipStream_t stream) {
  using namespace moe;
  if (M < 0 || F < kTile || F % kTile != 0)
    return fail(MOE_ERR_INVALID_ARG, "swiglu_quant_fp8: M=%lld F=%d (F must be a positive multiple of 128)",
                (long long)M, F);
  if (M == 0) return MOE_OK;
  const int64_t m_pad = ceil_div(M, kTile) * kTile;
  if (m_pad >= (int64_t(1) << 31) || m_pad * static_cast<int64_t>(F) >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "swiglu_quant_fp8: M too large");
  if (!gate_up || !q_row || !s_row || !q_t || !s_t) return fail(MOE_ERR_INVALID_ARG, "swiglu_quant_fp8: null pointer");
  if (!aligned16(gate_up) || !aligned16(q_row) || !aligned16(q_t))
    return fail(MOE_ERR_INVALID_ARG, "swiglu_quant_fp8: gate_up/q_row/q_t not 16-byte aligned");
  return launch_tile_quant<true>(gate_up, M, F, nullptr, 0, 0, m_pad, q_row, s_row, q_t, s_t, stream,
                                 "swiglu_quant_fp8");
}

extern "C" int64_t tile_quant_fp8_m_pad_bound(int64_t M, int E) {
  if (M < 0 || E < 0) return -1;
  return (moe::ceil_div(M, kTile) + E) * kTile;
}

extern "C" int tile_quant_fp8(const uint16_t* x, int64_t M, int K, int swiglu, const int32_t* group_sizes, int E,
                              int per_tile, int64_t m_pad, uint8_t* q_row, float* s_row, uint8_t* q_t, float* s_t,
                              hipStream_t stream) {
  using namespace moe;
  const char* name = "tile_quant_fp8";
  if (M < 0 || K < kTile || K % kTile != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: M=%lld K=%d (K must be a positive multiple of 128)", name, (long long)M, K);
  if (swiglu != 0 && swiglu != 1) return fail(MOE_ERR_INVALID_ARG, "%s: swiglu=%d", name, swiglu);
  if (per_tile != 0 && per_tile != 1) return fail(MOE_ERR_INVALID_ARG, "%s: per_tile=%d", name, per_tile);
  if ((q_t == nullptr) != (s_t == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "%s: q_t and s_t must both be given or both be NULL", name);
  if (q_t == nullptr) {
    // row layout only: group sizes, per_tile and m_pad play no part
    if (M == 0) return MOE_OK;
    if (M >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: M too large", name);
    if (!x || !q_row || !s_row) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
    if (!aligned16(x) || !aligned16(q_row)) return fail(MOE_ERR_INVALID_ARG, "%s: x/q_row not 16-byte aligned", name);
    const int64_t rows_pad = ceil_div(M, kTile) * kTile;
    if (swiglu)
      return launch_tile_quant<true>(x, M, K, nullptr, 0, 0, rows_pad, q_row, s_row, nullptr, nullptr, stream, name);
    return launch_tile_quant<false>(x, M, K, nullptr, 0, 0, rows_pad, q_row, s_row, nullptr, nullptr, stream, name);
  }
  if (m_pad < 0 || m_pad % kTile != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: m_pad=%lld must be a non-negative multiple of 128", name, (long long)m_pad);
  if (group_sizes == nullptr && m_pad < ceil_div(M, kTile) * kTile)
    return fail(MOE_ERR_INVALID_ARG, "%s: m_pad=%lld < %lld padded rows", name, (long long)m_pad,
                (long long)(ceil_div(M, kTile) * kTile));
  if (group_sizes != nullptr && (E < 1 || E > 65536)) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d", name, E);
  if (m_pad >= (int64_t(1) << 31) || M >= (int64_t(1) << 31) || m_pad * static_cast<int64_t>(K) >= (int64_t(1) << 40))
    return fail(MOE_ERR_UNSUPPORTED, "%s: M or m_pad too large", name);
  if (m_pad == 0) return MOE_OK;
  if (M > 0 && (!x || !q_row || !s_row)) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if ((x && !aligned16(x)) || (q_row && !aligned16(q_row)) || !aligned16(q_t))
    return fail(MOE_ERR_INVALID_ARG, "%s: x/q_row/q_t not 16-byte aligned", name);
  if (swiglu)
    return launch_tile_quant<true>(x, M, K, group_sizes, E, per_tile, m_pad, q_row, s_row, q_t, s_t, stream, name);
  return launch_tile_quant<false>(x, M, K, group_sizes, E, per_tile, m_pad, q_row, s_row, q_t, s_t, stream, name);
}
