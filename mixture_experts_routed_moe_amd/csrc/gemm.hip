// Grouped GEMM C[e] = A[e] @ W[e]^T for the routed experts on bf16 MFMA.
//
// Work decomposition: one workgroup per (padded row block bx, column tile nt).
// The row block is decoded from the dispatch tables (row recovery of the
// tutorial's contract); blocks past an expert's rows, or past the last
// expert, have no rows and return at once. A is the compact [numel, K]
// layout: rows past the block's valid count are loaded as zero and never
// stored, so an expert's last, partial tile needs no padding copy.
//
// Tile: BM x 128 outputs, K step 64, four wave64s in a 2x2 arrangement; each
// wave accumulates (BM/2) x 64 with v_mfma_f32_32x32x16_bf16. A and W tiles
// are K-contiguous in LDS, 128 bytes per row, with the eight 16-byte chunks
// of row r stored at chunk position (c ^ (r & 7)) so the ds_read_b128 of
// eight consecutive rows hits eight different chunk positions. Global loads
// of the next K step are issued into registers before the MFMAs of the
// current step (LDS double buffer, one barrier per step).
//
// Fused SwiGLU: the 128 W rows of a tile are 64 gate rows and the 64 up rows
// F positions further; wave column wn holds gate columns wn*32..+32 and the
// matching up columns in two accumulators, so the epilogue pairs them in
// registers: h = bf16(silu(bf16(g)) * bf16(u)).
#include "moe_common.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kBN = 128;
constexpr int kThreads = 256;

struct Tables {
  const int32_t* gs;
  const int32_t* go;
  const int32_t* gpo;
  const int32_t* gidx;
};

// Row recovery of padded block bx: expert g, first compact row and valid rows.
__device__ __forceinline__ void decode_block(const Tables& tb, int bx, int bm, int64_t numel, int& g,
                                             int64_t& m_start, int& rows) {
  int64_t r;
  if (tb.gs == nullptr) {
    g = 0;
    m_start = static_cast<int64_t>(bx) * bm;
    r = numel - m_start;
  } else {
    g = tb.gidx[bx];
    m_start = static_cast<int64_t>(bx) * bm - tb.gpo[g] + tb.go[g];
    r = static_cast<int64_t>(tb.go[g]) + tb.gs[g] - m_start;
  }
  rows = r <= 0 ? 0 : (r >= bm ? bm : static_cast<int>(r));
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

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
  const uint16_t* Ab = A + m_start * K;
  const uint16_t* Wb = W + static_cast<int64_t>(g) * w_stride;

  const uint16_t* a_src[A_CH];
  bool a_ok[A_CH];
  int a_dst[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int q = tid + kThreads * i, r = q >> 3, c = q & 7;
    a_ok[i] = r < rows;
    a_src[i] = Ab + static_cast<int64_t>(a_ok[i] ? r : 0) * K + c * 8;
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

template <bool FUSED>
int launch(const uint16_t* A, const uint16_t* W, Tables tb, int64_t numel, int E, int block_m, int padding_m,
           int n_tiles, int K, int64_t w_stride, int up_row, int ldc, uint16_t* C, hipStream_t stream,
           const char* name) {
  const int64_t m_blocks = tb.gs ? moe_num_blocks(numel, E, block_m, padding_m) : moe::ceil_div(numel, block_m);
  const int64_t blocks = m_blocks * n_tiles;
  if (blocks > 0x7FFFFFFF) return moe::fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
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
