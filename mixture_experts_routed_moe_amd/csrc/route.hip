// Top-k routing: one wavefront per token.
//
// Each lane holds ceil(E/64) routing logits (router score plus the optional
// per-expert bias) in registers. k rounds of a wave-wide argmax (value, then
// lower expert id; DPP max reductions, no LDS permutes) pick the experts in
// descending order; the selected logits
// stay in the lane that equals their slot. Scores: softmax over all E (the
// sum over every lane's logits), or the logistic sigmoid of each logit;
// renormalised weights divide by the selected experts' score sum, which for
// softmax equals a softmax over the k selected logits.
#include "moe_common.h"

namespace {

constexpr int kWavesPerBlock = 4;

// Largest of the 64 lanes' values, in every lane: DPP row shifts by 1, 2, 4
// and 8, then the row broadcasts (as wave_incl_sum, with max; lanes shifted
// in from outside a row give 0, which is at most every value), then lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  uint32_t v = x;
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// Order-preserving code of a logit: for numbers, a > b iff key(a) > key(b)
// as unsigned integers, and a == b (-0 and +0 included) iff the keys are
// equal; every number's code is at least 2, a NaN's is 1 (below every
// number), and 0 marks nothing.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 1u;
  const uint32_t b = __float_as_uint(f) == 0x80000000u ? 0u : __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  return s;
}

template <int VPT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void topk_softmax_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t T, int E, int k, int sigmoid,
    int renormalize, int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + t * E;

  float v[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? (bias ? row[e] + bias[e] : row[e]) : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_e = 0;
  float top_v = 0.0f;
  // each round: the largest remaining logit (a wave max over order-preserving
  // codes), then the lowest expert id holding it (a wave max over 1024 - id),
  // both DPP reductions; the winner's logit is read from its lane
  for (int j = 0; j < k; ++j) {
    uint32_t mk = 0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) mk = max(mk, order_key(v[i]));
    }
    const uint32_t top = wave_max_u32(mk);
    uint32_t lid = 0;  // 1024 - the lowest id of this lane whose logit has the top code
#pragma unroll
    for (int i = VPT - 1; i >= 0; --i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && order_key(v[i]) == top) lid = 1024u - static_cast<uint32_t>(e);
    }
    const int be = 1024 - static_cast<int>(wave_max_u32(lid));
    const int bi = be >> 6;
    float sel = v[0];
#pragma unroll
    for (int i = 1; i < VPT; ++i)
      if (i == bi) sel = v[i];
    const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel), be & 63));
    if ((be & 63) == lane) taken |= 1u << bi;
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
    if (j == 0) top_v = bv;
  }
  float score, denom;
  if (sigmoid) {
    score = lane < k ? 1.0f / (1.0f + expf(-my_v)) : 0.0f;
    denom = renormalize ? wave_sum(score) : 1.0f;
  } else {
    // the first selected logit is the maximum over all E
    score = lane < k ? expf(my_v - top_v) : 0.0f;
    if (renormalize) {
      denom = wave_sum(score);
    } else {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (lane + 64 * i < E) s += expf(v[i] - top_v);
      denom = wave_sum(s);
    }
  }
  if (lane < k) {
    ids[t * k + lane] = my_e;
    weights[t * k + lane] = score / denom;
  }
}

}  // namespace

extern "C" int moe_topk_softmax(const float* logits, const float* expert_bias, int64_t T, int E, int top_k,
                                int scoring, int renormalize, int32_t* topk_ids, float* topk_weights,
                                hipStream_t stream) {
  using namespace moe;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: T < 0");
  if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: E=%d not in [1,1024]", E);
  if (top_k < 1 || top_k > 16 || top_k > E)
    return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: top_k=%d not in [1,min(E,16)]", top_k);
  if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: scoring=%d", scoring);
  if (renormalize != 0 && renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: renormalize=%d not 0 or 1", renormalize);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return fail(MOE_ERR_INVALID_ARG, "moe_topk_softmax: null pointer");
  const int64_t blocks = ceil_div(T, kWavesPerBlock);
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_topk_softmax: T too large");
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kWavesPerBlock);
  const int vpt = (E + 63) / 64;
  const int sig = scoring == MOE_SCORING_SIGMOID;
#define MOE_ROUTE_LAUNCH(V)                                                                                   \
  topk_softmax_kernel<V><<<grid, block, 0, stream>>>(logits, expert_bias, T, E, top_k, sig, renormalize, topk_ids, \
                                                     topk_weights)
  if (vpt <= 1)
    MOE_ROUTE_LAUNCH(1);
  else if (vpt <= 2)
    MOE_ROUTE_LAUNCH(2);
  else if (vpt <= 4)
    MOE_ROUTE_LAUNCH(4);
  else if (vpt <= 8)
    MOE_ROUTE_LAUNCH(8);
  else
    MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
  return check_launch("moe_topk_softmax");
}
