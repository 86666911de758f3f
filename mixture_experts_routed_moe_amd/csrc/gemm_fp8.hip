// Block-scaled FP8 (OCP e4m3) grouped GEMM for the down projection, and the
// 128x128-block weight quantizer it takes its weights from.
//
// Operands: the activation codes qa [numel, K] with one fp32 scale per row and
// 128-column tile, sa [numel, K/128] (the FP8 quantizer's row layout), and
// expert weights qw [E, N, K] with one scale per 128x128 block,
// sw [E, N/128, K/128]. y[m, n] = bf16(sum over 128-wide K blocks kb of
// sa[m, kb] * sw[e, n/128, kb] * sum_{k in kb} qa[m, k] * qw[e, n, k]).
//
// gfx950's fp8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 takes its
// own per-32-element power-of-two scales; the fp32 scales here are not powers
// of two, so it runs with unit scales and each 128-wide K block's two products
// are scaled into the fp32 accumulator in registers. The instruction's A
// operand is the weight and its B operand the activation: a lane of the
// 32 x 32 result then holds one activation row (its column index), whose
// scale is one register, against 16 weight rows of one 128-row scale block,
// whose scale is one wave-uniform value.
#include "moe_common.h"

namespace {

constexpr int kT = 128;                                  // tile edge and scale block
constexpr int kF8Threads = 256;                          // four waves, 2 x 2, each 64 x 64

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// Chunk-position XOR of a 128-byte LDS row (eight 16-byte chunks): the 32
// rows of a fragment read are conflict-free in 8- and 16-lane phases.
__device__ __forceinline__ int f8_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// direct-to-LDS loads: lane i writes lds + 16 i (or + 4 i)
// The buffer form of the direct-to-LDS load (buffer_load_dword[x4] ... lds):
// bytes from the resource's base + voff + soff into lds + size * lane. Unlike
// the FLAT form it leaves the compiler's LDS waits exact while loads are in
// flight, and takes the K step as a scalar offset; per-lane offsets are 32
// bits (the hosts check that the A codes and one group's weight codes stay
// below 4 GiB).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f8_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void dmab16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, static_cast<int>(voff), soff, 0, 0);
}
__device__ __forceinline__ void dmab4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, static_cast<int>(voff), soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// One 256-thread workgroup per 128x128 block of w [rows, K]; thread t holds
// row t/2, columns (t%2)*64 .. +64. s = fl32(amax/448); code = e4m3 of the
// fp32 quotient RN32(w * RN64(1/s)), which is the correctly rounded fp32 w/s
// (w has 8 significant bits: the argument made for the activation quantizer).
__global__ __launch_bounds__(256) void block_quant_kernel(const uint16_t* __restrict__ w, int K, int n_kb,
                                                           uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ uint32_t s_max[4];
  const int kb = blockIdx.x % n_kb;
  const int64_t nb = blockIdx.x / n_kb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t row = nb * kT + (t >> 1);
  const int64_t off = row * K + kb * kT + (t & 1) * 64;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = reinterpret_cast<const uint4*>(w + off)[i];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ws[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(ws[k] & 0x7FFFu, (ws[k] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), d)));
  if (lane == 0) s_max[wave] = m;
  __syncthreads();
  const uint32_t bb = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const float sc = __uint_as_float(bb << 16) / 448.0f;
  const double inv = sc > 0.0f ? 1.0 / static_cast<double>(sc) : 0.0;
  if (t == 0) s[nb * n_kb + kb] = sc;
  uint32_t out[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ws[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
      const float a0 = static_cast<float>(static_cast<double>(__uint_as_float(ws[k] << 16)) * inv);
      const float a1 = static_cast<float>(static_cast<double>(__uint_as_float(ws[k] & 0xFFFF0000u)) * inv);
      const float b0 = static_cast<float>(static_cast<double>(__uint_as_float(ws[k + 1] << 16)) * inv);
      const float b1 = static_cast<float>(static_cast<double>(__uint_as_float(ws[k + 1] & 0xFFFF0000u)) * inv);
      uint32_t word = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false));
      word = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(b0, b1, static_cast<int>(word), true));
      out[i * 2 + k / 2] = sc > 0.0f ? word : 0u;   // an all-zero block: codes 0 (no -0.0 codes)
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(q + off);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

// One workgroup per (128-row block bx of the padded expert-major row space,
// 128-row weight tile nt). K advances 128 bytes (one scale block) per step;
// the A rows, the W rows and the A row scales of a step load direct-to-LDS
// into a ring of S stages. A block with more than 64 valid rows (AR = 128)
// has two stages of 33 KiB: step kb+1 loads while step kb computes. A block
// of at most 64 rows (an expert's only or last block; most experts of a
// skewed routing have a few rows) only streams its weights, so it takes the
// ring for 64 A rows: three stages of 24 KiB, two steps of weights in flight
// (two workgroups per CU: 73 KiB of LDS each). A rows past the block's valid
// rows are read from its last row and never stored. With a gather table
// (tb.gather) compact row r of A and of its scales is row gather[r] /
// gather_k of qa and sa (the token's codes).
// FUSED (gate_up with SwiGLU): the tile's weight rows are 64 gate rows
// nt*64.. and the matching 64 up rows up_row + nt*64..; a wave's first
// 32-row MFMA block is gate, its second the matching up block, so one lane
// holds both halves of each output and the epilogue stores
// SwiGLU(bf16(gate), bf16(up)) into the 64 output columns nt*64.. of y.
template <int AR>
struct F8Ring {
  static constexpr int S = AR == 128 ? 2 : 3;                      // stages
  static constexpr int A_BYTES = AR * kT;
  static constexpr int STAGE = A_BYTES + kT * kT + AR * 4;         // A rows, W rows, A row scales
};
// every wave issues one 4-byte scale load per step (so every wave's count of
// loads per step is the same); the waves past the scales load a copy of the
// first scales into a scratch area of their own
constexpr int kF8Scratch = 4 * 64 * 4;
constexpr int kF8Lds = (2 * F8Ring<128>::STAGE > 3 * F8Ring<64>::STAGE ? 2 * F8Ring<128>::STAGE
                                                                        : 3 * F8Ring<64>::STAGE) + kF8Scratch;
static_assert(2 * kF8Lds <= 160 * 1024, "two workgroups per CU");

template <bool FUSED, int AR>
__device__ __forceinline__ void fp8_tile(uint8_t* smem, const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                         const uint8_t* __restrict__ qw, const float* __restrict__ sw,
                                         const moe::Tables& tb, int g, int64_t m_start, int rows, int nt, int N,
                                         int K, int up_row, int ldc, uint16_t* __restrict__ y) {
  using R = F8Ring<AR>;
  constexpr int S = R::S, STAGE = R::STAGE;
  constexpr int A_LD = AR / 32;          // A loads (8 rows each) per wave and step
  constexpr int TM = AR / 64;            // 32-row MFMA blocks per wave
  constexpr int L = A_LD + 4 + 1;        // loads per wave and step: A, W, one scale load
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nkb = K / kT;
  const int lrow = lane >> 3, lpos = lane & 7;

  // this wave's A rows (A_LD x 8) and 32 W rows of every step
  uint32_t a_src[A_LD], w_src[4];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = wave * (AR / 4) + i * 8 + lrow;
    const int rr = min(r, rows - 1);
    a_src[i] = static_cast<uint32_t>(moe::a_row(tb, m_start + rr) * K) + static_cast<uint32_t>((lpos ^ f8_swz(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + lrow;
    // weight row of LDS row r: fused, rows 0-63 gate nt*64 + r, rows 64-127 up
    const int64_t wr = FUSED ? (r < kT / 2 ? static_cast<int64_t>(nt) * (kT / 2) + r
                                           : static_cast<int64_t>(up_row) + nt * (kT / 2) + (r - kT / 2))
                             : static_cast<int64_t>(nt) * kT + r;
    w_src[i] = static_cast<uint32_t>(wr * K) + static_cast<uint32_t>((lpos ^ f8_swz(r)) * 16);
  }
  // the AR A row scales of a step, 64 a wave: waves past them reload the
  // first 64 into their own scratch slot
  const bool real_scale = wave * 64 < AR;
  const uint32_t sa_src =
      static_cast<uint32_t>(moe::a_row(tb, m_start + min((real_scale ? wave * 64 : 0) + lane, rows - 1)) * nkb * 4);
  const __amdgpu_buffer_rsrc_t a_rsrc = f8_rsrc(qa), sa_rsrc = f8_rsrc(sa);
  const __amdgpu_buffer_rsrc_t w_rsrc = f8_rsrc(qw + static_cast<int64_t>(g) * N * K);
  const int sa_dst = real_scale ? R::A_BYTES + kT * kT + wave * 64 * 4 : -1;
  uint8_t* const scratch = smem + kF8Lds - kF8Scratch + wave * 64 * 4;
  // the weight scale block of each of the wave's two 32-row MFMA blocks (128-row
  // blocks: fused, the gate rows nt*64.. sit in block nt/2, the up rows in
  // block up_row/128 + nt/2; otherwise both in block nt)
  const float* sw_blk[2];
  sw_blk[0] = sw + (static_cast<int64_t>(g) * (N / kT) + (FUSED ? nt / 2 : nt)) * nkb;
  sw_blk[1] = sw + (static_cast<int64_t>(g) * (N / kT) + (FUSED ? up_row / kT + nt / 2 : nt)) * nkb;

  auto issue = [&](int kb, int st) __attribute__((always_inline)) {
    uint8_t* base = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) dmab16(a_rsrc, a_src[i], kb * kT, base + (wave * (AR / 4) + i * 8) * kT);
#pragma unroll
    for (int i = 0; i < 4; ++i) dmab16(w_rsrc, w_src[i], kb * kT, base + R::A_BYTES + (wave * 32 + i * 8) * kT);
    dmab4(sa_rsrc, sa_src, kb * 4, sa_dst >= 0 ? base + sa_dst : scratch);
  };

  floatx16 acc[TM][2];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

  // fragment rows and the two 16-byte chunks of each 64-wide K half: lane
  // half h of half j takes chunks 4j + 2h and 4j + 2h + 1 (the same mapping
  // for both operands, which is all the dot products need)
  const int h = lane >> 5;
  const int a_row0 = wm * (AR / 2) + (lane & 31);
  // 32-row MFMA blocks of this wave that hold valid rows (the others skip their MFMAs)
  const int live_tm = __builtin_amdgcn_readfirstlane(min(TM, max(0, (rows - wm * (AR / 2) + 31) / 32)));
  // LDS row of the wave's MFMA block tn: fused, tn 0 gate rows wn*32.., tn 1
  // up rows 64 + wn*32..; otherwise rows wn*64 + tn*32..
  const int w_row0 = (FUSED ? wn * 32 : wn * 64) + (lane & 31);
  constexpr int kWBlk1 = FUSED ? kT / 2 : 32;
  auto frag = [&](const uint8_t* rows_base, int r, int j) __attribute__((always_inline)) {
    const int c0 = 4 * j + 2 * h;
    const v4i lo = *reinterpret_cast<const v4i*>(rows_base + r * kT + ((c0 ^ f8_swz(r)) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(rows_base + r * kT + (((c0 + 1) ^ f8_swz(r)) << 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };

  // prologue: steps 0 .. S-2
  issue(0, 0);
  if (S > 2 && nkb > 1) issue(1, 1);
  for (int kb = 0; kb < nkb; ++kb) {
    // stage kb has landed for every wave (the S-2 later steps may still be in
    // flight), and every wave is done with stage kb-1, whose slot takes step kb+S-1
    if constexpr (S == 2) {
      wait_vm_barrier<0>();
    } else {
      if (kb + 1 < nkb) wait_vm_barrier<L>();
      else wait_vm_barrier<0>();
    }
    if (kb + S - 1 < nkb) issue(kb + S - 1, (kb + S - 1) % S);
    const uint8_t* st = smem + (kb % S) * STAGE;
    const float* s_rows = reinterpret_cast<const float*>(st + R::A_BYTES + kT * kT);
    const float w_scale[2] = {sw_blk[0][kb], sw_blk[1][kb]};
    v8i af[TM][2], wf[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) af[tm][j] = frag(st, a_row0 + tm * 32, j);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) wf[tn][j] = frag(st + R::A_BYTES, w_row0 + tn * kWBlk1, j);
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (tm >= live_tm) break;  // wave-uniform: no valid rows from here on
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const float sc = s_rows[a_row0 + tm * 32] * w_scale[tn];
        floatx16 p = {};
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[tn][0], af[tm][0], p, 0, 0, 0, 127, 0, 127);
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[tn][1], af[tm][1], p, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][tn][r] += p[r] * sc;
      }
    }
  }

  // lane (h, c): activation row a_row0 + tm*32; result element r is weight
  // row w_row0-relative (r & 3) + 4h + 8(r >> 2), four consecutive columns per
  // quad of registers
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int lr = a_row0 + tm * 32;
    if (lr >= rows) continue;
    if constexpr (FUSED) {
      uint16_t* yrow = y + (m_start + lr) * ldc + static_cast<int64_t>(nt) * (kT / 2) + wn * 32;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = moe::swiglu_bf16(moe::f32_to_bf16(acc[tm][0][4 * q4 + e]), moe::f32_to_bf16(acc[tm][1][4 * q4 + e]));
        *reinterpret_cast<uint2*>(yrow + 8 * q4 + 4 * h) =
            make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      }
    } else {
      uint16_t* yrow = y + (m_start + lr) * ldc + static_cast<int64_t>(nt) * kT + wn * 64;
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int n = tn * 32 + 8 * q4 + 4 * h;
          const uint32_t lo = moe::pack_bf16x2(acc[tm][tn][4 * q4], acc[tm][tn][4 * q4 + 1]);
          const uint32_t hi = moe::pack_bf16x2(acc[tm][tn][4 * q4 + 2], acc[tm][tn][4 * q4 + 3]);
          *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
        }
    }
  }
}

template <bool FUSED>
__global__ __launch_bounds__(kF8Threads, 2) void grouped_gemm_fp8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ qw,
    const float* __restrict__ sw, moe::Tables tb, int64_t numel, int n_tiles, int N, int K,
    int up_row, int ldc, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kF8Lds];
  // Row-major tile order. The hardware hands workgroup w to XCD w % 8, so with
  // n_tiles a multiple of 8 (56 and 32 on the DeepSeek-V3 shapes) column tile
  // nt of every row block lands on XCD nt % 8: each XCD's L2 holds one eighth
  // of every expert's weights, which are most of the bytes, while the much
  // smaller activation codes are read by all eight.
  const int bx = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  int g, rows;
  int64_t m_start;
  moe::decode_block(tb, bx, kT, numel, g, m_start, rows);
  if (rows == 0) return;
  if (rows <= 64)
    fp8_tile<FUSED, 64>(smem, qa, sa, qw, sw, tb, g, m_start, rows, nt, N, K, up_row, ldc, y);
  else
    fp8_tile<FUSED, 128>(smem, qa, sa, qw, sw, tb, g, m_start, rows, nt, N, K, up_row, ldc, y);
}

}  // namespace

extern "C" int fp8_block_quant_weights(const uint16_t* w, int64_t rows, int K, uint8_t* q, float* s,
                                       hipStream_t stream) {
  using namespace moe;
  const char* name = "fp8_block_quant_weights";
  if (rows < 0 || rows % kT != 0 || K < kT || K % kT != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: rows=%lld K=%d (both multiples of 128)", name, (long long)rows, K);
  if (rows == 0) return MOE_OK;
  if (!w || !q || !s) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if (!aligned16(w) || !aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "%s: w/q not 16-byte aligned", name);
  const int64_t blocks = (rows / kT) * (K / kT);
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "%s: too many blocks", name);
  block_quant_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(w, K, K / kT, q, s);
  return check_launch(name);
}

extern "C" int grouped_gemm_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                                const int32_t* group_sizes, const int32_t* group_offsets,
                                const int32_t* group_padded_offsets, const int32_t* group_idx_for_bx, int64_t numel,
                                int E, int N, int K, int padding_m, int block_m, uint16_t* y, hipStream_t stream) {
  using namespace moe;
  const char* name = "grouped_gemm_fp8";
  if (numel < 0 || N < kT || N % kT != 0 || K < kT || K % kT != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: numel=%lld N=%d K=%d (N, K multiples of 128)", name, (long long)numel, N,
                K);
  if (block_m != kT) return fail(MOE_ERR_UNSUPPORTED, "%s: block_m=%d (only 128)", name, block_m);
  const bool dense = group_sizes == nullptr;
  if (dense != (group_offsets == nullptr) || dense != (group_padded_offsets == nullptr) ||
      dense != (group_idx_for_bx == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "%s: tables must be all NULL (dense) or all non-NULL", name);
  if (dense && E != 1) return fail(MOE_ERR_INVALID_ARG, "%s: dense mode (NULL tables) needs E=1", name);
  if (!dense && (E < 1 || padding_m <= 0 || padding_m % kT != 0))
    return fail(MOE_ERR_INVALID_ARG, "%s: E=%d padding_m=%d (a positive multiple of 128)", name, E, padding_m);
  if (numel >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: numel >= 2^31", name);
  if (numel * K >= (int64_t(1) << 32) || static_cast<int64_t>(N) * K >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "%s: the A codes or one group's weight codes reach 4 GiB", name);
  if (numel == 0) return MOE_OK;
  if (!qa || !sa || !qw || !sw || !y) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(y))
    return fail(MOE_ERR_INVALID_ARG, "%s: qa/qw/y not 16-byte aligned", name);
  const int64_t m_blocks = dense ? ceil_div(numel, kT) : moe_num_blocks(numel, E, kT, padding_m);
  const int n_tiles = N / kT;
  const int64_t blocks = m_blocks * n_tiles;
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  const Tables tb{group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx};
  grouped_gemm_fp8_kernel<false><<<static_cast<unsigned>(blocks), kF8Threads, 0, stream>>>(qa, sa, qw, sw, tb, numel,
                                                                                          n_tiles, N, K, 0, N, y);
  return check_launch(name);
}

extern "C" int grouped_gemm_gate_up_fp8(const uint8_t* qa, const float* sa, int64_t a_rows, const int32_t* sorted_pair,
                                        int top_k, const uint8_t* qw, const float* sw, const int32_t* group_sizes,
                                        const int32_t* group_offsets, const int32_t* group_padded_offsets,
                                        const int32_t* group_idx_for_bx, int64_t numel, int E, int H, int F,
                                        int padding_m, int block_m, int fuse_swiglu, uint16_t* out,
                                        hipStream_t stream) {
  using namespace moe;
  const char* name = "grouped_gemm_gate_up_fp8";
  if (numel < 0 || a_rows < 0 || H < kT || H % kT != 0 || F < kT || F % kT != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: numel=%lld a_rows=%lld H=%d F=%d (H, F multiples of 128)", name,
                (long long)numel, (long long)a_rows, H, F);
  if (block_m != kT) return fail(MOE_ERR_UNSUPPORTED, "%s: block_m=%d (only 128)", name, block_m);
  if (fuse_swiglu != 0 && fuse_swiglu != 1) return fail(MOE_ERR_INVALID_ARG, "%s: fuse_swiglu=%d", name, fuse_swiglu);
  const bool dense = group_sizes == nullptr;
  if (dense != (group_offsets == nullptr) || dense != (group_padded_offsets == nullptr) ||
      dense != (group_idx_for_bx == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "%s: tables must be all NULL (dense) or all non-NULL", name);
  if (dense && (E != 1 || sorted_pair))
    return fail(MOE_ERR_INVALID_ARG, "%s: dense mode (NULL tables) needs E=1 and no sorted_pair", name);
  if (!dense && (E < 1 || padding_m <= 0 || padding_m % kT != 0))
    return fail(MOE_ERR_INVALID_ARG, "%s: E=%d padding_m=%d (a positive multiple of 128)", name, E, padding_m);
  if (sorted_pair ? (top_k < 1 || numel != a_rows * top_k) : a_rows != numel)
    return fail(MOE_ERR_INVALID_ARG, "%s: a_rows=%lld must be numel (compact rows) or numel/top_k (gather)", name,
                (long long)a_rows);
  if (numel >= (int64_t(1) << 31)) return fail(MOE_ERR_UNSUPPORTED, "%s: numel >= 2^31", name);
  if (a_rows * H >= (int64_t(1) << 32) || int64_t(2) * F * H >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "%s: the A codes or one group's weight codes reach 4 GiB", name);
  if (numel == 0) return MOE_OK;
  if (!qa || !sa || !qw || !sw || !out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", name);
  if (!aligned16(qa) || !aligned16(qw) || !aligned16(out))
    return fail(MOE_ERR_INVALID_ARG, "%s: qa/qw/out not 16-byte aligned", name);
  const int64_t m_blocks = dense ? ceil_div(numel, kT) : moe_num_blocks(numel, E, kT, padding_m);
  const int n_tiles = fuse_swiglu ? F / (kT / 2) : (2 * F) / kT;
  const int64_t blocks = m_blocks * n_tiles;
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "%s: grid too large", name);
  Tables tb{group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx};
  tb.gather = sorted_pair;
  tb.gather_k = sorted_pair ? top_k : 1;
  if (fuse_swiglu)
    grouped_gemm_fp8_kernel<true><<<static_cast<unsigned>(blocks), kF8Threads, 0, stream>>>(
        qa, sa, qw, sw, tb, numel, n_tiles, 2 * F, H, F, F, out);
  else
    grouped_gemm_fp8_kernel<false><<<static_cast<unsigned>(blocks), kF8Threads, 0, stream>>>(
        qa, sa, qw, sw, tb, numel, n_tiles, 2 * F, H, 0, 2 * F, out);
  return check_launch(name);
}
