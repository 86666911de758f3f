// Shared device helpers and host error plumbing for the MI355X (gfx950)
// routed-expert MoE library. Device code only targets CDNA4: wave64, bf16 and
// fp8 (OCP e4m3) conversions in hardware, MFMA matrix cores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe_mi355x.h"

// ------------------------------------------------------------------ host --
namespace moe {

// Records a message for moe_last_error() and returns `code`.
int fail(int code, const char* fmt, ...);
// Maps a failed HIP launch to MOE_ERR_HIP; returns MOE_OK otherwise.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace moe

// ---------------------------------------------------------------- device --
namespace moe {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1, 2,
// 4 and 8 (lanes shifted in from outside a 16-lane row add 0), then lane 15
// of each row added to the next row and lane 31 to the upper two rows.
__device__ __forceinline__ int wave_incl_sum(int x) {
  int v = x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// The project's fp32 exponential. Every SwiGLU (standalone, fused into the
// gate_up GEMM epilogue, fused into the FP8 quantizer) evaluates exactly this
// sequence of IEEE binary32 operations, so their results agree bit for bit:
//   clamp x to [-86, 88]; n = rint(x * log2 e);
//   r = (x - n*LN2_HI) - n*LN2_LO   (Cody-Waite reduction, LN2_HI has 15
//                                    significant bits so n*LN2_HI is exact);
//   p = degree-7 Taylor polynomial of e^r in Horner form, no fused multiply-add;
//   result = p * 2^n (exact, n in [-124, 127]).
__device__ __forceinline__ float exp_spec(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;   // fp32 nearest to log2(e)
  const float kLn2Hi = 0x1.62e4p-1f;     // leading 15 bits of ln 2
  const float kLn2Lo = 0x1.7f7d1cp-20f;  // ln 2 - kLn2Hi, rounded
  x = fminf(fmaxf(x, -86.0f), 88.0f);
  const float n = __builtin_rintf(x * kLog2e);
  const float r = (x - n * kLn2Hi) - n * kLn2Lo;
  float p = 0x1.a01a02p-13f;             // 1/5040
  p = 0x1.6c16c2p-10f + r * p;           // 1/720
  p = 0x1.111112p-7f + r * p;            // 1/120
  p = 0x1.555556p-5f + r * p;            // 1/24
  p = 0x1.555556p-3f + r * p;            // 1/6
  p = 0.5f + r * p;
  p = 1.0f + r * p;
  p = 1.0f + r * p;
  const float two_n = __uint_as_float(static_cast<uint32_t>(static_cast<int>(n) + 127) << 23);
  return p * two_n;
}

// SiLU(g) = g / (1 + exp(-g)) with the divide correctly rounded (the HIP
// default for fp32 '/').
__device__ __forceinline__ float silu_spec(float g) {
#pragma clang fp contract(off)
  const float d = 1.0f + exp_spec(-g);
  return g / d;
}

// One SwiGLU output: bf16(silu(gate) * up) from bf16 inputs.
__device__ __forceinline__ uint16_t swiglu_bf16(uint16_t gate, uint16_t up) {
#pragma clang fp contract(off)
  const float s = silu_spec(bf16_to_f32(gate));
  return f32_to_bf16(s * bf16_to_f32(up));
}

// ------------------------------------------------- dispatch-table decode --
// The four dispatch tables of the grouped GEMMs (all NULL: one dense group).
struct Tables {
  const int32_t* gs;
  const int32_t* go;
  const int32_t* gpo;
  const int32_t* gidx;
  // optional gather: compact row R of the GEMM's A operand is row
  // gather[R] / gather_k of the A pointer (the token of sorted pair R),
  // so a GEMM reads the unpermuted hidden states directly
  const int32_t* gather = nullptr;
  int gather_k = 1;
};

// The A row that holds compact row R (R itself without a gather table).
__device__ __forceinline__ int64_t a_row(const Tables& tb, int64_t R) {
  return tb.gather ? static_cast<int64_t>(tb.gather[R] / tb.gather_k) : R;
}

// Row recovery of padded block bx (the tutorial's m_start identity): expert
// g, first compact row m_start = bx*bm - gpo[g] + go[g], and the block's
// valid rows, clamped to [0, bm].
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

// ------------------------------------------ streaming (non-temporal) access --
// A 16-byte load of data read once per kernel, marked non-temporal so it
// does not displace reused lines in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------ SiLU lookup in LDS --
// The gate input of every SwiGLU is bf16, so silu_spec(g) has 2^16 possible
// arguments. A table of the 2 * 32 * 128 = 8192 values with |g| in
// [2^-25, 128) (bf16 exponent field 102..133, both signs), plus 128 values for
// the mantissas of g in [-256, -128), gives silu_spec(g) for every finite g:
//   |g| < 2^-25: exp(-g) rounds to exactly 1, so silu = g / 2;
//   g >= 128:    1 + exp(-g) rounds to 1, so silu = g;
//   g <= -128:   the exponent argument saturates at 88, silu = g / D for one
//                constant D, which scales exactly with powers of two of g
//                (the results stay normal), so the [-256, -128) entry times
//                2^(exponent - 134) is exact.
// Every entry is silu_spec's value, computed at compile time (below), so a
// lookup returns the same bits as the direct evaluation.
constexpr int kSiluTabE0 = 102;                          // bf16 exponent field of 2^-25
constexpr int kSiluTabMid = 2 * 32 * 128;
constexpr int kSiluTabSize = kSiluTabMid + 128;

// The bf16 gate (bits) of table entry i.
constexpr uint32_t silu_table_gate(int i) {
  return i < kSiluTabMid ? (static_cast<uint32_t>(i >> 12) << 15) |
                               (static_cast<uint32_t>(((i >> 7) & 31) + kSiluTabE0) << 7) |
                               static_cast<uint32_t>(i & 127)
                         : 0x8000u | (134u << 7) | static_cast<uint32_t>(i - kSiluTabMid);
}

// exp_spec and silu_spec for constant evaluation: the same IEEE binary32
// operations in the same order (a constant expression rounds every
// operation to nearest-even and never contracts), with rint written as the
// 1.5 * 2^23 shift (exact round-half-even for |v| < 2^22; here |v| < 128).
constexpr float exp_spec_cx(float x) {
  x = x < -86.0f ? -86.0f : (x > 88.0f ? 88.0f : x);
  const float v = x * 0x1.715476p+0f;
  const float n = (v + 0x1.8p23f) - 0x1.8p23f;
  const float r = (x - n * 0x1.62e4p-1f) - n * 0x1.7f7d1cp-20f;
  float p = 0x1.a01a02p-13f;
  p = 0x1.6c16c2p-10f + r * p;
  p = 0x1.111112p-7f + r * p;
  p = 0x1.555556p-5f + r * p;
  p = 0x1.555556p-3f + r * p;
  p = 0.5f + r * p;
  p = 1.0f + r * p;
  p = 1.0f + r * p;
  return p * __builtin_bit_cast(float, static_cast<uint32_t>(static_cast<int>(n) + 127) << 23);
}

constexpr float silu_spec_cx(float g) { return g / (1.0f + exp_spec_cx(-g)); }

// The first N entries of the table, as a compile-time constant: a kernel
// reads it from its code object's data (no kernel writes it, so concurrent
// calls on any streams share it without ordering).
template <int N>
struct SiluTable {
  float v[N];
};

template <int N>
constexpr SiluTable<N> make_silu_table() {
  static_assert(N <= kSiluTabSize, "table size");
  SiluTable<N> t{};
  for (int i = 0; i < N; ++i) t.v[i] = silu_spec_cx(__builtin_bit_cast(float, silu_table_gate(i) << 16));
  return t;
}

// silu_spec of a bf16 gate (bits in the low 16 bits of gb), from the table.
// Written with bit masks rather than branches: every lane takes the same
// instructions, and no per-element condition has to stay live.
__device__ __forceinline__ float silu_lookup(const float* tab, uint32_t gb) {
  const uint32_t e = (gb >> 7) & 0xFFu;
  const uint32_t k = e - kSiluTabE0;                                  // wraps for e < kSiluTabE0
  const uint32_t mid = 0u - static_cast<uint32_t>(k < 32u);           // all ones inside the table range
  const uint32_t idx_mid = ((gb >> 3) & 0x1000u) | ((k & 31u) << 7) | (gb & 127u);
  const uint32_t idx = (idx_mid & mid) | ((kSiluTabMid + (gb & 127u)) & ~mid);
  const float t = tab[idx];
  const float g = __uint_as_float(gb << 16);
  const float big = (gb & 0x8000u) ? __builtin_ldexpf(t, static_cast<int>(e) - 134) : g;  // |g| >= 128
  const float out = e < static_cast<uint32_t>(kSiluTabE0) ? g * 0.5f : big;
  return __uint_as_float((__float_as_uint(t) & mid) | (__float_as_uint(out) & ~mid));
}

// bf16(silu(gate) * up), the same bits as swiglu_bf16, with the SiLU from the table.
__device__ __forceinline__ uint16_t swiglu_bf16_tab(const float* tab, uint32_t gate, uint32_t up) {
#pragma clang fp contract(off)
  return f32_to_bf16(silu_lookup(tab, gate) * __uint_as_float(up << 16));
}

}  // namespace moe
