// Token permute (gather into the compact expert-major layout) and unpermute
// (per-token gather-reduce over the k expert outputs). Both are HBM-bound
// row copies with 16-byte vector accesses (a wave moves 1 KiB per
// instruction); each thread keeps about 16 loads in flight.
#include "moe_common.h"

namespace {

constexpr int kThreads = 256;

// Rows that are read once (hidden in the permute, y and the addend in the
// unpermute) are loaded non-temporally: measured on the DeepSeek-V3-shaped
// workload, the unpermute goes from 0.112 to 0.102 ms and the permute gains
// about 1%; non-temporal stores made the permute 35% slower, so stores are
// plain.

// R rows per workgroup, CPT 16-byte chunks per thread per row and pass (a
// row wider than 256*CPT chunks takes several passes): the R source-row
// indices are read first, then every load of a pass is issued before its
// first store, so each thread has R*CPT loads in flight.
template <int R, int CPT>
__global__ __launch_bounds__(kThreads) void permute_kernel(const uint4* __restrict__ hidden,
                                                           const int32_t* __restrict__ sorted_pair, int64_t numel,
                                                           int top_k, int h8, uint4* __restrict__ x_perm) {
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * R;
  const int tid = threadIdx.x;
  // rows past numel and chunks past the row end are clamped to the last row
  // and chunk: they load and store (again) that element's correct value, so
  // every load and store is unconditional and the loads all go out first
  int64_t src[R], dst[R];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int64_t r = min(r0 + q, numel - 1);
    src[q] = static_cast<int64_t>(sorted_pair[r] / top_k) * h8;
    dst[q] = r * h8;
  }
  for (int cb = 0; cb < h8; cb += CPT * kThreads) {
    uint4 v[R][CPT];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int i = 0; i < CPT; ++i) v[q][i] = hidden[src[q] + min(cb + tid + i * kThreads, h8 - 1)];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int i = 0; i < CPT; ++i) x_perm[dst[q] + min(cb + tid + i * kThreads, h8 - 1)] = v[q][i];
  }
}

// Token-major form of the same permutation, x_perm[pair_to_row[p]] =
// hidden[p / k]: R tokens per workgroup, each source row read once and
// written to its k destination rows. The gather form reads every hidden row k
// times in expert order; the streaming x_perm writes evict hidden from the
// MALL between those reads, so they come from HBM again (measured: about 0.13
// ms against about 0.09 ms for this form on the DeepSeek-V3-shaped workload).
template <int R, int CPT, int MAXK>
__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(const uint4* __restrict__ hidden,
                                                                   const int32_t* __restrict__ pair_to_row,
                                                                   int64_t T, int top_k, int h8,
                                                                   uint4* __restrict__ x_perm) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * R;
  const int tid = threadIdx.x;
  // tokens past T are clamped to the last token (their loads and stores
  // repeat its correct values); so are chunks past the row end
  int64_t src[R], dst[R][MAXK];
#pragma unroll
  for (int q = 0; q < R; ++q) {
    const int64_t t = min(t0 + q, T - 1);
    src[q] = t * h8;
#pragma unroll
    for (int j = 0; j < MAXK; ++j) dst[q][j] = static_cast<int64_t>(pair_to_row[t * top_k + (j < top_k ? j : 0)]) * h8;
  }
  for (int cb = 0; cb < h8; cb += CPT * kThreads) {
    uint4 v[R][CPT];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int i = 0; i < CPT; ++i) v[q][i] = moe::load_stream16(hidden + src[q] + min(cb + tid + i * kThreads, h8 - 1));
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
      for (int j = 0; j < MAXK; ++j)
#pragma unroll
        for (int i = 0; i < CPT; ++i) x_perm[dst[q][j] + min(cb + tid + i * kThreads, h8 - 1)] = v[q][i];
  }
}

// Work is cut into wave-sized items: one item is one token's output chunks
// [128*b, 128*b + 128) (16 bytes each), two per lane, so a 7168-wide row is
// seven items and every item ends with the loads it issued; each workgroup
// runs four independent items, one per wave, and there are no barriers. The
// token's k row indices and weights are wave-uniform (scalar loads); then all
// 2k gathers are issued before they are reduced (fp32, slots in ascending
// order), scaled, added to the addend and rounded once.
constexpr int kUnpermuteCpl = 2;                          // 16-byte chunks per lane and row
constexpr int kUnpermuteChunks = 64 * kUnpermuteCpl;      // chunks per item
constexpr int kUnpermuteWaves = 4;

template <int MAXK>
__global__ __launch_bounds__(64 * kUnpermuteWaves) void unpermute_kernel(
    const uint4* __restrict__ y, const int32_t* __restrict__ pair_to_row, const float* __restrict__ weights,
    int64_t T, int top_k, int h8, int items_per_token, float rsf, const uint4* __restrict__ addend,
    uint4* __restrict__ out) {
  constexpr int CPL = kUnpermuteCpl;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kUnpermuteWaves +
                       __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int64_t t = item / items_per_token;
  if (t >= T) return;  // the whole wave leaves together
  const int lane = threadIdx.x & 63;
  const int cb = static_cast<int>(item - t * items_per_token) * kUnpermuteChunks;
  int64_t row[MAXK];
  float w[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    row[j] = static_cast<int64_t>(pair_to_row[t * top_k + (j < top_k ? j : 0)]) * h8;
    w[j] = j < top_k ? weights[t * top_k + j] : 0.0f;
  }
  // slots past top_k read their token's first slot and weigh 0; chunks past
  // the row end are clamped to its last chunk and not stored: every load is in
  // bounds and used, so all of them go out before the reduction
  int c[CPL], cr[CPL];
#pragma unroll
  for (int h = 0; h < CPL; ++h) {
    c[h] = cb + h * 64 + lane;
    cr[h] = min(c[h], h8 - 1);
  }
  uint4 v[CPL][MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j)
#pragma unroll
    for (int h = 0; h < CPL; ++h) v[h][j] = moe::load_stream16(y + row[j] + cr[h]);
  uint4 a[CPL] = {};
  if (addend != nullptr) {
#pragma unroll
    for (int h = 0; h < CPL; ++h) a[h] = moe::load_stream16(addend + t * h8 + cr[h]);
  }
#pragma unroll
  for (int h = 0; h < CPL; ++h) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXK; ++j) {
      const uint32_t u[4] = {v[h][j].x, v[h][j].y, v[h][j].z, v[h][j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += w[j] * moe::bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
        acc[2 * i + 1] += w[j] * moe::bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
      }
    }
    float add[8];
    const uint32_t u[4] = {a[h].x, a[h].y, a[h].z, a[h].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      add[2 * i] = moe::bf16_to_f32(static_cast<uint16_t>(u[i] & 0xFFFFu));
      add[2 * i + 1] = moe::bf16_to_f32(static_cast<uint16_t>(u[i] >> 16));
    }
    uint4 o;
    o.x = moe::pack_bf16x2(rsf * acc[0] + add[0], rsf * acc[1] + add[1]);
    o.y = moe::pack_bf16x2(rsf * acc[2] + add[2], rsf * acc[3] + add[3]);
    o.z = moe::pack_bf16x2(rsf * acc[4] + add[4], rsf * acc[5] + add[5]);
    o.w = moe::pack_bf16x2(rsf * acc[6] + add[6], rsf * acc[7] + add[7]);
    if (c[h] < h8) out[t * h8 + c[h]] = o;
  }
}

}  // namespace

template <int MAXK>
void launch_scatter(const uint4* h4, const int32_t* p2r, int64_t T, int top_k, int h8, uint4* x4, hipStream_t stream) {
  using moe::ceil_div;
  // two tokens per workgroup, about 8 loads in flight per thread
  if (h8 <= kThreads)
    permute_scatter_kernel<4, 1, MAXK><<<static_cast<unsigned>(ceil_div(T, 4)), kThreads, 0, stream>>>(h4, p2r, T, top_k, h8, x4);
  else if (h8 <= 2 * kThreads)
    permute_scatter_kernel<2, 2, MAXK><<<static_cast<unsigned>(ceil_div(T, 2)), kThreads, 0, stream>>>(h4, p2r, T, top_k, h8, x4);
  else
    permute_scatter_kernel<1, 4, MAXK><<<static_cast<unsigned>(T), kThreads, 0, stream>>>(h4, p2r, T, top_k, h8, x4);
}

extern "C" int moe_permute(const uint16_t* hidden, const int32_t* sorted_pair, const int32_t* pair_to_row, int64_t T,
                           int top_k, int H, uint16_t* x_perm, hipStream_t stream) {
  using namespace moe;
  if (T < 0 || top_k < 1 || H < 8 || H % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: T=%lld top_k=%d H=%d (H must be a positive multiple of 8)",
                (long long)T, top_k, H);
  const int64_t numel = T * top_k;
  if (numel == 0) return MOE_OK;
  if (numel > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: T*top_k too large");
  if (!hidden || !x_perm || (!sorted_pair && !pair_to_row))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  if (!aligned16(hidden) || !aligned16(x_perm))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: hidden/x_perm not 16-byte aligned");
  const int h8 = H / 8;
  const uint4* h4 = reinterpret_cast<const uint4*>(hidden);
  uint4* x4 = reinterpret_cast<uint4*>(x_perm);
  if (pair_to_row && top_k <= 16) {
    if (top_k <= 2) launch_scatter<2>(h4, pair_to_row, T, top_k, h8, x4, stream);
    else if (top_k <= 4) launch_scatter<4>(h4, pair_to_row, T, top_k, h8, x4, stream);
    else if (top_k <= 8) launch_scatter<8>(h4, pair_to_row, T, top_k, h8, x4, stream);
    else launch_scatter<16>(h4, pair_to_row, T, top_k, h8, x4, stream);
    return check_launch("moe_permute");
  }
  if (!sorted_pair) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: top_k=%d > 16 needs sorted_pair", top_k);
  // about 16 loads in flight per thread
  if (h8 <= kThreads)
    permute_kernel<16, 1><<<static_cast<unsigned>(ceil_div(numel, 16)), kThreads, 0, stream>>>(h4, sorted_pair, numel,
                                                                                               top_k, h8, x4);
  else if (h8 <= 2 * kThreads)
    permute_kernel<8, 2><<<static_cast<unsigned>(ceil_div(numel, 8)), kThreads, 0, stream>>>(h4, sorted_pair, numel,
                                                                                             top_k, h8, x4);
  else if (h8 <= 4 * kThreads)
    permute_kernel<4, 4><<<static_cast<unsigned>(ceil_div(numel, 4)), kThreads, 0, stream>>>(h4, sorted_pair, numel,
                                                                                             top_k, h8, x4);
  else
    permute_kernel<2, 8><<<static_cast<unsigned>(ceil_div(numel, 2)), kThreads, 0, stream>>>(h4, sorted_pair, numel,
                                                                                             top_k, h8, x4);
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
  const int h8 = H / 8;
  const int items_per_token = static_cast<int>(ceil_div(h8, kUnpermuteChunks));
  const int64_t blocks = ceil_div(T * items_per_token, kUnpermuteWaves);
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute: T*H too large");
  const unsigned grid = static_cast<unsigned>(blocks);
  const int threads = 64 * kUnpermuteWaves;
  const uint4* y4 = reinterpret_cast<const uint4*>(y);
  const uint4* a4 = reinterpret_cast<const uint4*>(addend);
  uint4* o4 = reinterpret_cast<uint4*>(out);
  const float rsf = routed_scaling_factor;
  if (top_k <= 2)
    unpermute_kernel<2><<<grid, threads, 0, stream>>>(y4, pair_to_row, topk_weights, T, top_k, h8, items_per_token,
                                                      rsf, a4, o4);
  else if (top_k <= 4)
    unpermute_kernel<4><<<grid, threads, 0, stream>>>(y4, pair_to_row, topk_weights, T, top_k, h8, items_per_token,
                                                      rsf, a4, o4);
  else if (top_k <= 8)
    unpermute_kernel<8><<<grid, threads, 0, stream>>>(y4, pair_to_row, topk_weights, T, top_k, h8, items_per_token,
                                                      rsf, a4, o4);
  else
    unpermute_kernel<16><<<grid, threads, 0, stream>>>(y4, pair_to_row, topk_weights, T, top_k, h8, items_per_token,
                                                       rsf, a4, o4);
  return check_launch("moe_unpermute");
}
