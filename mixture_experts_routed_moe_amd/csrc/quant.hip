// SwiGLU and the fused SwiGLU + FP8 (OCP e4m3) activation quantizer.
//
// swiglu_quant_fp8: one workgroup per 128x128 block of h = SiLU(gate) * up.
// Thread (rg, cg) of 16x16 owns rows rg*8..rg*8+7 and columns cg*8..cg*8+7
// of the block, so
//   * gate/up loads are 16-byte vectors and a row's 16 threads read 256
//     contiguous bytes of each half;
//   * the 1x128 row amax is a reduction over the 16 lanes of a row (xor 1..8);
//   * the 128x128 block amax adds a reduction over row groups and one LDS
//     exchange between the four waves;
//   * the row-layout store is 8 bytes per thread (a row's 128 bytes come
//     from 16 consecutive lanes) and the transposed store is also 8 bytes
//     per thread: a thread's 8 consecutive rows of one column are 8
//     consecutive bytes of q_t, no LDS transpose needed.
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

__device__ __forceinline__ float wave_max_xor(float v, int first, int last) {
  for (int off = first; off <= last; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Two fp32 values -> two e4m3 bytes in the low half of the result.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Correctly rounded fp32 quotient h / s from a per-tile RN64(1/s).
__device__ __forceinline__ float quotient(float h, double inv_s) {
  return static_cast<float>(static_cast<double>(h) * inv_s);
}

__global__ __launch_bounds__(256) void swiglu_kernel(const uint4* __restrict__ gu, uint32_t total, uint32_t f8,
                                                     uint4* __restrict__ h) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
    const uint32_t m = i / f8, c = i - m * f8;
    const uint4 g = gu[static_cast<uint64_t>(m) * 2 * f8 + c];
    const uint4 u = gu[static_cast<uint64_t>(m) * 2 * f8 + f8 + c];
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = moe::swiglu_bf16(static_cast<uint16_t>(gw[k] & 0xFFFFu), static_cast<uint16_t>(uw[k] & 0xFFFFu));
      const uint16_t hi = moe::swiglu_bf16(static_cast<uint16_t>(gw[k] >> 16), static_cast<uint16_t>(uw[k] >> 16));
      o[k] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
    }
    h[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ __launch_bounds__(256) void swiglu_quant_kernel(const uint16_t* __restrict__ x, int M, int F,
                                                           int m_pad, int n_fb, uint8_t* __restrict__ q_row,
                                                           float* __restrict__ s_row, uint8_t* __restrict__ q_t,
                                                           float* __restrict__ s_t) {
  __shared__ float s_wmax[4];
  const int fb = blockIdx.x % n_fb;
  const int mb = blockIdx.x / n_fb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid & 15, rg = tid >> 4;
  const int col0 = fb * kTile + cg * 8;
  const int row0 = mb * kTile + rg * 8;

  float h[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = row0 + i;
    if (m < M) {
      const uint16_t* rp = x + static_cast<int64_t>(m) * 2 * F;
      const uint4 g = *reinterpret_cast<const uint4*>(rp + col0);
      const uint4 u = *reinterpret_cast<const uint4*>(rp + F + col0);
      const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        h[i][2 * k] = moe::bf16_to_f32(moe::swiglu_bf16(static_cast<uint16_t>(gw[k] & 0xFFFFu),
                                                        static_cast<uint16_t>(uw[k] & 0xFFFFu)));
        h[i][2 * k + 1] = moe::bf16_to_f32(moe::swiglu_bf16(static_cast<uint16_t>(gw[k] >> 16),
                                                            static_cast<uint16_t>(uw[k] >> 16)));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[i][j] = 0.0f;
    }
  }

  // 1x128 row amax (16 lanes per row) and the 128x128 block amax
  float amax_row[8];
  float blk = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(h[i][j]));
    a = wave_max_xor(a, 1, 8);
    amax_row[i] = a;
    blk = fmaxf(blk, a);
  }
  blk = wave_max_xor(blk, 16, 32);
  if (lane == 0) s_wmax[wave] = blk;
  __syncthreads();
  blk = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));

  // block (transposed) scale
  const float sb = blk / 448.0f;
  const double inv_sb = sb > 0.0f ? 1.0 / static_cast<double>(sb) : 0.0;
  if (tid == 0) s_t[static_cast<int64_t>(fb) * (m_pad / kTile) + mb] = sb;

  // row layout: codes and scales
  uint32_t qt[8][2];  // transposed codes: [column j][rows 0-3 | rows 4-7]
#pragma unroll
  for (int j = 0; j < 8; ++j) qt[j][0] = qt[j][1] = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = row0 + i;
    const float s = amax_row[i] / 448.0f;
    const double inv_s = s > 0.0f ? 1.0 / static_cast<double>(s) : 0.0;
    uint32_t w0 = 0u, w1 = 0u;
    if (s > 0.0f) {
      w0 = e4m3x2(quotient(h[i][0], inv_s), quotient(h[i][1], inv_s)) |
           (e4m3x2(quotient(h[i][2], inv_s), quotient(h[i][3], inv_s)) << 16);
      w1 = e4m3x2(quotient(h[i][4], inv_s), quotient(h[i][5], inv_s)) |
           (e4m3x2(quotient(h[i][6], inv_s), quotient(h[i][7], inv_s)) << 16);
    }
    if (m < M) {
      *reinterpret_cast<uint2*>(q_row + static_cast<int64_t>(m) * F + col0) = make_uint2(w0, w1);
      if (cg == 0) s_row[static_cast<int64_t>(m) * n_fb + fb] = s;
    }
    if (sb > 0.0f) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const uint32_t pr = e4m3x2(quotient(h[i][j], inv_sb), quotient(h[i][j + 1], inv_sb));
        const int sh = (i & 3) * 8;
        qt[j][i >> 2] |= (pr & 0xFFu) << sh;
        qt[j + 1][i >> 2] |= (pr >> 8) << sh;
      }
    }
  }
  // transposed layout: column f = col0 + j, rows row0..row0+7 are 8 bytes
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint2*>(q_t + static_cast<int64_t>(col0 + j) * m_pad + row0) = make_uint2(qt[j][0], qt[j][1]);
}

}  // namespace

extern "C" int swiglu(const uint16_t* gate_up, int64_t M, int F, uint16_t* h, hipStream_t stream) {
  using namespace moe;
  if (M < 0 || F < 8 || F % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "swiglu: M=%lld F=%d (F must be a positive multiple of 8)", (long long)M, F);
  if (M == 0) return MOE_OK;
  const int64_t total = M * (F / 8);
  if (total >= (int64_t(1) << 32)) return fail(MOE_ERR_UNSUPPORTED, "swiglu: M*F too large");
  if (!gate_up || !h) return fail(MOE_ERR_INVALID_ARG, "swiglu: null pointer");
  if (!aligned16(gate_up) || !aligned16(h)) return fail(MOE_ERR_INVALID_ARG, "swiglu: pointers not 16-byte aligned");
  const int64_t blocks = std::min<int64_t>(ceil_div(total, 256), 256 * 64);
  swiglu_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(reinterpret_cast<const uint4*>(gate_up),
                                                                   static_cast<uint32_t>(total),
                                                                   static_cast<uint32_t>(F / 8),
                                                                   reinterpret_cast<uint4*>(h));
  return check_launch("swiglu");
}

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
  const int n_fb = F / kTile;
  const int64_t blocks = (m_pad / kTile) * n_fb;
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "swiglu_quant_fp8: too many blocks");
  swiglu_quant_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      gate_up, static_cast<int>(M), F, static_cast<int>(m_pad), n_fb, q_row, s_row, q_t, s_t);
  return check_launch("swiglu_quant_fp8");
}
