// Device and host helpers shared by the HIP kernels of libmoe_fp8 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_fp8.h"

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

#define MOE_CHECK_LAUNCH()                                  \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

static inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ------------------------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an fp32 pattern, so widening is exact; narrowing
// rounds to nearest even (NaN stays NaN) with gfx950's conversion instruction, v_cvt_pk_bf16_f32,
// which converts two values at once.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef float bf16_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16_x2 __attribute__((ext_vector_type(2)));
// (lo, hi) -> one word, lo in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((bf16_f32x2){lo, hi}, bf16_x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)pack_bf16x2(f, 0.0f); }

// ------------------------------------------------------------------------------------------
// Block scale of a block whose largest magnitude is amax.  Default: amax / 448 (IEEE fp32 division;
// 1 for an all-zero block).  Power of two (the scale the hardware-scaled MFMA takes as an E8M0
// exponent): the smallest power of two at or above t = amax / 448, at least 2^-127 (the smallest
// E8M0 value), 1 for an all-zero block.  From t's bits: a normal t with a zero mantissa is a power
// of two, otherwise the next one has the exponent field plus one; a subnormal t (or t flushed to 0
// by the division) rounds up to 2^-127 or 2^-126.
__device__ __forceinline__ float block_scale(float amax, bool pow2) {
  if (amax == 0.0f) return 1.0f;
  const float t = amax / 448.0f;
  if (!pow2) return t;
  const uint32_t u = __float_as_uint(t), ex = u >> 23, man = u & 0x7FFFFFu;
  const uint32_t s = ex == 0 ? (u <= 0x00400000u ? 0x00400000u : 0x00800000u) : (man == 0 ? u : (ex + 1) << 23);
  return __uint_as_float(s);
}
// E8M0 code of a power-of-two scale (its fp32 exponent field; 2^-127, an fp32 subnormal, is code 0)
__device__ __forceinline__ uint32_t e8m0_code(float pow2_scale) { return (__float_as_uint(pow2_scale) >> 23) & 0xFFu; }

// ------------------------------------------------------------------------------------------
// OCP FP8 E4M3 encode: round to nearest even, saturating to +-448, sign of zero kept.
// gfx950's v_cvt_pk_fp8_f32 rounds to nearest even on [-448, 448] but returns NaN beyond 464,
// so the value is clamped to the largest finite magnitude first (clamping commutes with
// saturating rounding: every |v| >= 448 maps to 448 either way).  fminf/fmaxf keep -0.
__device__ __forceinline__ float e4m3_clamp(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// two values -> low 16 bits of the result (byte 0 = a, byte 1 = b)
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xFFFFu;
}

// four values -> one 32-bit word (byte i = value i)
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return (uint32_t)w;
}

// ------------------------------------------------------------------------------------------
// Fixed fp32 exponential used by the router (softmax and sigmoid scores), so that scores that
// feed routing decisions are reproducible bit for bit: Cody & Waite (1980) reduction
// x = n*ln2 + r with ln2 = hi + lo (hi has few enough bits that n*hi is exact for |n| <= 127),
// degree-6 Taylor polynomial of e^r by Horner's rule with fused multiply-adds, exact scaling by
// 2^n.  The input is clamped to [-86, 88] so the result is a normal, finite fp32 number.
// Every step is one IEEE fp32 operation; the library is compiled with -ffp-contract=off.
__device__ __forceinline__ float router_exp(float x) {
  x = fminf(fmaxf(x, -86.0f), 88.0f);
  const float n = rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e400p-1f, x);
  r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
  float p = 0x1.6c16c2p-10f;
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return p * __uint_as_float((uint32_t)((int)n + 127) << 23);
}

__device__ __forceinline__ float router_sigmoid(float z) { return 1.0f / (1.0f + router_exp(-z)); }

// ------------------------------------------------------------------------------------------
// wave64 helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }
static inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t i, float (&v)[8]) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ------------------------------------------------------------------------------------------
// The quotients x / s of an encoder, s one block's scale.  With y = 1/s correctly rounded (one IEEE
// division per block), q0 = x*y is within an ulp of x/s, the residual x - q0*s is exact in one FMA
// while it does not underflow, and q0 + residual*y rounded once is then the correctly rounded x/s
// (Markstein's theorem on division by a correctly rounded reciprocal; Markstein, IBM J. Res. Dev.
// 34(1), 1990).  The residual can underflow only for |x| below about 2^-100, where |x/s| is far below
// the smallest e4m3 step for every s >= 2^-60, so the e4m3 code (zero, sign of x) is the same;
// the sign is copied from x so that -0 stays -0.  Scales below 2^-60 or not finite take IEEE
// divisions.  Three VALU operations per value instead of a full division.
__device__ __forceinline__ bool quot_by_recip(float s) { return s >= 0x1p-60f && s <= 0x1.fffffep+127f; }
__device__ __forceinline__ float quot_recip_step(float x, float s, float y) {
  const float q0 = x * y;
  const float r = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, y, q0), x);
}
template <int N>
__device__ __forceinline__ void quotients(const float* v, float s, float* r) {
  if (quot_by_recip(s)) {
    const float y = 1.0f / s;
#pragma unroll
    for (int q = 0; q < N; ++q) r[q] = quot_recip_step(v[q], s, y);
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q) r[q] = v[q] / s;
  }
}

__device__ __forceinline__ uint2 encode8(const float (&v)[8], float s) {
  float r[8];
  quotients<8>(v, s, r);
  return make_uint2(e4m3_pack4(r[0], r[1], r[2], r[3]), e4m3_pack4(r[4], r[5], r[6], r[7]));
}

// ------------------------------------------------------------------------------------------
// Cross-lane moves within a 16-lane row by DPP (no LDS crossbar): lane i reads lane i^1 (quad
// permutation 1,0,3,2), i^2 (2,3,0,1), 7-i within its 8 (half-row mirror) or 15-i within its 16
// (row mirror).  Every source lane is inside the row, so rows are independent of one another.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }
// max over each aligned 16-lane row, in every lane of the row
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, dpp_f32<DPP_XOR1>(m));
  m = fmaxf(m, dpp_f32<DPP_XOR2>(m));
  m = fmaxf(m, dpp_f32<DPP_HALF_MIRROR>(m));
  return fmaxf(m, dpp_f32<DPP_MIRROR>(m));
}


// 1x128 activation block b (x[128 b, 128 b + 128), rows contiguous and cols % 128 == 0): 16 lanes
// per block, lane `sub` holding 8 consecutive values; amax across the 16 lanes, the block scale,
// e4m3 codes (x / s an IEEE division) and, from lane 0, the scale.
template <bool BF16, bool POW2>
__device__ __forceinline__ void quant_1x128_piece(const void* __restrict__ x, int64_t b, int sub,
                                                  uint8_t* __restrict__ q, float* __restrict__ scales) {
  float v[8];
  load8<BF16>(x, b * 128 + sub * 8, v);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = row16_max(m);   // the block's 16 lanes are one aligned DPP row
  const float s = block_scale(m, POW2);
  *reinterpret_cast<uint2*>(q + b * 128 + sub * 8) = encode8(v, s);
  if (sub == 0) scales[b] = s;
}

// U blocks b0, b0 + step, ..., b0 + (U-1) step per 16-lane group (blocks >= nblocks skipped), every
// load issued before the first block is encoded.
template <bool BF16, bool POW2, int U>
__device__ __forceinline__ void quant_1x128_pieces(const void* __restrict__ x, int64_t b0, int64_t step,
                                                   int64_t nblocks, int sub, uint8_t* __restrict__ q,
                                                   float* __restrict__ scales) {
  float v[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (b0 + u * step < nblocks) load8<BF16>(x, (b0 + u * step) * 128 + sub * 8, v[u]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t b = b0 + u * step;
    if (b >= nblocks) break;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
    m = row16_max(m);
    const float s = block_scale(m, POW2);
    *reinterpret_cast<uint2*>(q + b * 128 + sub * 8) = encode8(v[u], s);
    if (sub == 0) scales[b] = s;
  }
}
