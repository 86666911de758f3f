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

}  // namespace moe
