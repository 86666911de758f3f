// Top-k softmax routing: one wavefront per token.
//
// Each lane holds ceil(E/64) logits in registers. k rounds of a wave-wide
// argmax (value, then lower expert id) pick the experts in descending order;
// the selected logits stay in the lane that equals their slot, and the
// renormalised weights are a softmax over those k logits, which equals the
// full softmax divided by its top-k mass.
#include "moe_common.h"

namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ void better(float& bv, int& be, float ov, int oe) {
  if (ov > bv || (ov == bv && oe < be)) {
    bv = ov;
    be = oe;
  }
}

template <int VPT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + t * E;

  float v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_e = 0;
  float top_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) better(bv, be, v[i], e);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      better(bv, be, ov, oe);
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) top_v = bv;
  }
  // softmax over the k selected logits (max is the first one)
  const float ex = lane < k ? expf(my_v - top_v) : 0.0f;
  float s = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane < k) {
    ids[t * k + lane] = my_e;
    weights[t * k + lane] = ex / s;
  }
}

}  // namespace

extern "C" int moe_topk_softmax(const float* logits, int64_t T, int E, int top_k, int32_t* topk_ids,
                                float* topk_weights, hipStream_t stream) {
  using namespace moe;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: T < 0");
  if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: E=%d not in [1,1024]", E);
  if (top_k < 1 || top_k > 16 || top_k > E)
    return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: top_k=%d not in [1,min(E,16)]", top_k);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: null pointer");
  const int64_t blocks = ceil_div(T, kWavesPerBlock);
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: T too large");
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWavesPerBlock);
  const int vpt = (E + 63) / 64;
  if (vpt <= 1)
    topk_softmax_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, top_k, topk_ids, topk_weights);
  else if (vpt <= 2)
    topk_softmax_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, top_k, topk_ids, topk_weights);
  else if (vpt <= 4)
    topk_softmax_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, top_k, topk_ids, topk_weights);
  else if (vpt <= 8)
    topk_softmax_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, top_k, topk_ids, topk_weights);
  else
    topk_softmax_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, top_k, topk_ids, topk_weights);
  return check_launch("moe_topk_softmax");
}
