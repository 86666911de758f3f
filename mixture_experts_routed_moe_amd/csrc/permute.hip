// Token permute (gather into the compact expert-major layout) and unpermute
// (per-token gather-reduce over the k expert outputs). Both are HBM-bound
// row copies: one workgroup per output row, 16-byte vector accesses, so a
// wave moves 1 KiB per instruction.
#include "moe_common.h"

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void permute_kernel(const uint4* __restrict__ hidden,
                                                           const int32_t* __restrict__ sorted_pair, int top_k,
                                                           int h8, uint4* __restrict__ x_perm) {
  const int64_t r = blockIdx.x;
  const int64_t src = sorted_pair[r] / top_k;
  const uint4* in = hidden + src * h8;
  uint4* out = x_perm + r * h8;
#pragma unroll 4
  for (int c = threadIdx.x; c < h8; c += kThreads) out[c] = in[c];
}

template <int MAXK>
__global__ __launch_bounds__(kThreads) void unpermute_kernel(const uint4* __restrict__ y,
                                                             const int32_t* __restrict__ pair_to_row,
                                                             const float* __restrict__ weights, int top_k, int h8,
                                                             float rsf, const uint4* __restrict__ addend,
                                                             uint4* __restrict__ out) {
  const int64_t t = blockIdx.x;
  int64_t row[MAXK];
  float w[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    row[j] = j < top_k ? static_cast<int64_t>(pair_to_row[t * top_k + j]) * h8 : 0;
    w[j] = j < top_k ? weights[t * top_k + j] : 0.0f;
  }
  for (int c = threadIdx.x; c < h8; c += kThreads) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
      if (j < top_k) {
        const uint4 v = y[row[j] + c];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w[j] * moe::bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
          acc[2 * i + 1] += w[j] * moe::bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
        }
      }
    }
    float add[8];
    if (addend != nullptr) {
      const uint4 a = addend[t * h8 + c];
      const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        add[2 * i] = moe::bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
        add[2 * i + 1] = moe::bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) add[i] = 0.0f;
    }
    uint4 o;
    o.x = moe::pack_bf16x2(rsf * acc[0] + add[0], rsf * acc[1] + add[1]);
    o.y = moe::pack_bf16x2(rsf * acc[2] + add[2], rsf * acc[3] + add[3]);
    o.z = moe::pack_bf16x2(rsf * acc[4] + add[4], rsf * acc[5] + add[5]);
    o.w = moe::pack_bf16x2(rsf * acc[6] + add[6], rsf * acc[7] + add[7]);
    out[t * h8 + c] = o;
  }
}

}  // namespace

extern "C" int moe_permute(const uint16_t* hidden, const int32_t* sorted_pair, int64_t T, int top_k, int H,
                           uint16_t* x_perm, hipStream_t stream) {
  using namespace moe;
  if (T < 0 || top_k < 1 || H < 8 || H % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: T=%lld top_k=%d H=%d (H must be a positive multiple of 8)",
                (long long)T, top_k, H);
  const int64_t numel = T * top_k;
  if (numel == 0) return MOE_OK;
  if (numel > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: T*top_k too large");
  if (!hidden || !sorted_pair || !x_perm) return fail(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  if (!aligned16(hidden) || !aligned16(x_perm))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: hidden/x_perm not 16-byte aligned");
  permute_kernel<<<static_cast<unsigned>(numel), kThreads, 0, stream>>>(
      reinterpret_cast<const uint4*>(hidden), sorted_pair, top_k, H / 8, reinterpret_cast<uint4*>(x_perm));
  return check_launch("moe_permute");
}

extern "C" int moe_unpermute(const uint16_t* y, const int32_t* pair_to_row, const float* topk_weights, int64_t T,
                             int top_k, int H, float routed_scaling_factor, const uint16_t* addend,
                             uint16_t* out, hipStream_t stream) {
  using namespace moe;
  if (T < 0 || top_k < 1 || H < 8 || H % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_unpermute: T=%lld top_k=%d H=%d (H must be a positive multiple of 8)",
                (long long)T, top_k, H);
  if (top_k > 16) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute: top_k=%d > 16", top_k);
  if (T == 0) return MOE_OK;
  if (T > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute: T too large");
  if (!y || !pair_to_row || !topk_weights || !out) return fail(MOE_ERR_INVALID_ARG, "moe_unpermute: null pointer");
  if (!aligned16(y) || !aligned16(out) || (addend && !aligned16(addend)))
    return fail(MOE_ERR_INVALID_ARG, "moe_unpermute: y/out/addend not 16-byte aligned");
  if (static_cast<const void*>(out) == static_cast<const void*>(y))
    return fail(MOE_ERR_INVALID_ARG, "moe_unpermute: out aliases y");
  const unsigned grid = static_cast<unsigned>(T);
  const uint4* y4 = reinterpret_cast<const uint4*>(y);
  const uint4* a4 = reinterpret_cast<const uint4*>(addend);
  uint4* o4 = reinterpret_cast<uint4*>(out);
  if (top_k <= 2)
    unpermute_kernel<2><<<grid, kThreads, 0, stream>>>(y4, pair_to_row, topk_weights, top_k, H / 8,
                                                       routed_scaling_factor, a4, o4);
  else if (top_k <= 4)
    unpermute_kernel<4><<<grid, kThreads, 0, stream>>>(y4, pair_to_row, topk_weights, top_k, H / 8,
                                                       routed_scaling_factor, a4, o4);
  else if (top_k <= 8)
    unpermute_kernel<8><<<grid, kThreads, 0, stream>>>(y4, pair_to_row, topk_weights, top_k, H / 8,
                                                       routed_scaling_factor, a4, o4);
  else
    unpermute_kernel<16><<<grid, kThreads, 0, stream>>>(y4, pair_to_row, topk_weights, top_k, H / 8,
                                                        routed_scaling_factor, a4, o4);
  return check_launch("moe_unpermute");
}
