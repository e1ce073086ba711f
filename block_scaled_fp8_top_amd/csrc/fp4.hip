// FP4 expert weights: the 4-bit analogue of the block-scaled recipe.  "RL at 1T Scale: prime-rl
// Performance Deep Dive" names NVFP4 as future work; the MI355X matrix cores take the OCP
// microscaling form instead: FP4 E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in 1x32
// blocks along K, each block with a power-of-two scale given as an E8M0 exponent.
//
// Quantisation (per 1x32 block): s = the smallest power of two at or above fl32(amax / 6), at least
// 2^-127, 1 for an all-zero block; q = e2m1(x / s) (x / s an IEEE fp32 division), round to nearest
// with ties to the even code, saturating at 6, sign of zero kept.  Two codes per byte, element 2i in
// the low nibble; the scale is stored as its E8M0 code (the fp32 exponent field).
//
// Packed layout for the grouped GEMM (one 128-wide K step of a 256-row panel): 16 KB of codes in
// MFMA fragment order -- 16-byte piece 64 i + L holds row 16 i + (L % 16) of the panel and K chunk
// L / 16 (32 elements), which is exactly the 16 bytes lane L of a 16x16x128 FP4 operand takes for
// 16-row block i -- and 1 KB of scale codes, [panel row][chunk].  Panel rows as for FP8 weights
// (SwiGLU: gate rows then up rows; rows past N are zero).
#include <algorithm>

#include "common.h"

namespace {

__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 3;
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return sign | c;
}

// smallest power of two at or above t = amax / 6, at least 2^-127 (1 for amax == 0)
__device__ __forceinline__ float fp4_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  const float t = amax / 6.0f;
  const uint32_t u = __float_as_uint(t), ex = u >> 23, man = u & 0x7FFFFFu;
  const uint32_t s = ex == 0 ? (u <= 0x00400000u ? 0x00400000u : 0x00800000u) : (man == 0 ? u : (ex + 1) << 23);
  return __uint_as_float(s);
}

// one thread per 1x32 block
template <bool BF16>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const void* __restrict__ w, int64_t nblocks,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ e8) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(w) + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = p[i];
      const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(ww[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(w) + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float s = fp4_scale(amax);
  uint32_t word[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x |= e2m1_code(v[8 * i + j] / s) << (4 * j);
    word[i] = x;
  }
  *reinterpret_cast<uint4*>(q + b * 16) = make_uint4(word[0], word[1], word[2], word[3]);
  e8[b] = (uint8_t)((__float_as_uint(s) >> 23) & 0xFFu);
}

__device__ __forceinline__ int panel_row4(int epi, int nt, int r, int F) {
  return epi == 1 ? (r < 128 ? nt * 128 + r : F + nt * 128 + (r - 128)) : nt * 256 + r;
}

// one thread per 16-byte code piece of a packed step (1024 per step) and, for the first 64 of
// them, one 16-byte piece of the step's scale image
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ e8,
                                                       int N, int K, int ny, int epi, int64_t steps,
                                                       uint8_t* __restrict__ pq, uint8_t* __restrict__ pe) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= steps * 1024) return;
  const int KB = K / 128;
  const int w = (int)(u & 1023);
  const int64_t step = u >> 10;              // (g, nt, kb)
  const int kb = (int)(step % KB);
  const int64_t gnt = step / KB;
  const int nt = (int)(gnt % ny);
  const int64_t g = gnt / ny;
  {
    const int i = w >> 6, L = w & 63;
    const int r = 16 * i + (L & 15), chunk = L >> 4;
    const int n = panel_row4(epi, nt, r, N / 2);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) v = *reinterpret_cast<const uint4*>(q + ((size_t)g * N + n) * (K / 2) + (size_t)kb * 64 + chunk * 16);
    *reinterpret_cast<uint4*>(pq + (size_t)u * 16) = v;
  }
  if (w < 64) {
    // scale image bytes [16 w, 16 w + 16): rows 4 w .. 4 w + 3, chunks 0..3
    uint32_t word[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * w + j;
      const int n = panel_row4(epi, nt, r, N / 2);
      word[j] = n < N ? *reinterpret_cast<const uint32_t*>(e8 + ((size_t)g * N + n) * (K / 32) + (size_t)kb * 4) : 0u;
    }
    *reinterpret_cast<uint4*>(pe + (size_t)step * 1024 + w * 16) = make_uint4(word[0], word[1], word[2], word[3]);
  }
}

int64_t fp4_panels(int32_t N, int32_t epilogue) { return epilogue == MOE_EPI_STORE ? ceil_div64(N, 256) : N / 256; }

int check_fp4(int32_t groups, int32_t N, int32_t K, int32_t epilogue) {
  if (groups < 1 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (epilogue != MOE_EPI_STORE && epilogue != MOE_EPI_SWIGLU_QUANT) return MOE_ERR_ARG;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && N % 256 != 0) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_quant_mxfp4(const void* w, int w_dtype, int64_t rows, int32_t cols, uint8_t* q, uint8_t* e8,
                               void* stream) {
  if (rows < 0 || cols < 32 || cols % 32 != 0) return MOE_ERR_SHAPE;
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return MOE_OK;
  if (!w || !q || !e8) return MOE_ERR_NULL;
  const int64_t grid = ceil_div64(nblocks, 256);
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  if (w_dtype == MOE_BF16)
    quant_mxfp4_kernel<true><<<(unsigned)grid, 256, 0, as_stream(stream)>>>(w, nblocks, q, e8);
  else
    quant_mxfp4_kernel<false><<<(unsigned)grid, 256, 0, as_stream(stream)>>>(w, nblocks, q, e8);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" size_t moe_packed_fp4_bytes(int32_t groups, int32_t N, int32_t K, int32_t epilogue, size_t* scale_bytes) {
  if (check_fp4(groups, N, K, epilogue) != MOE_OK) return 0;
  const size_t steps = (size_t)groups * (size_t)fp4_panels(N, epilogue) * (size_t)(K / 128);
  if (scale_bytes) *scale_bytes = steps * 1024;
  return steps * 16384;
}

extern "C" int moe_pack_weights_fp4(const uint8_t* q, const uint8_t* e8, int32_t groups, int32_t N, int32_t K,
                                    int32_t epilogue, uint8_t* packed_q, uint8_t* packed_e8, void* stream) {
  int rc = check_fp4(groups, N, K, epilogue);
  if (rc != MOE_OK) return rc;
  if (!q || !e8 || !packed_q || !packed_e8) return MOE_ERR_NULL;
  const int ny = (int)fp4_panels(N, epilogue);
  const int64_t steps = (int64_t)groups * ny * (K / 128);
  const int64_t grid = ceil_div64(steps * 1024, 256);
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  pack_fp4_kernel<<<(unsigned)grid, 256, 0, as_stream(stream)>>>(q, e8, N, K, ny, epilogue == MOE_EPI_SWIGLU_QUANT,
                                                                  steps, packed_q, packed_e8);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
