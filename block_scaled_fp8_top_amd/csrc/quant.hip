// Block-scaled FP8 e4m3 quantisation (1x128 activation blocks, 128x128 weight blocks).
//
// Per block: amax = max |x|; s = amax / 448 (IEEE fp32 division; 1 for an all-zero block), or the
// power-of-two scale of common.h's block_scale;
// q = e4m3(x / s) with x / s an IEEE fp32 division (hipcc emits correctly rounded fp32 division by
// default), rounded to nearest even and saturated at 448 by the clamp-then-convert in common.h.
// HBM-bound: every input byte is read once and every code written once.
#include "common.h"

namespace {

// 1x128: 16 lanes per block, 8 consecutive values per lane.  Blocks are contiguous in memory
// (rows are contiguous and cols % 128 == 0), so block b covers x[128 b, 128 b + 128) and its
// scale is scales[b].  A workgroup (16 lane groups) takes Q1_U * 16 consecutive blocks, group g
// blocks 16 u + g of them, so each step u of the workgroup reads 16 adjacent blocks.
constexpr int Q1_U = 4;
template <bool BF16, bool POW2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x, int64_t nblocks,
                                                          uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int64_t b0 = (int64_t)blockIdx.x * (16 * Q1_U) + threadIdx.x / 16;
  // every lane of a 16-lane group shares its blocks; whole groups are in or out of range
  quant_1x128_pieces<BF16, POW2, Q1_U>(x, b0, 16, nblocks, threadIdx.x & 15, q, scales);
}

// 128x128: one workgroup of 256 threads per block; thread (r16 = tid / 16, c = tid % 16) handles
// rows r16 + 16 p (p < 8), columns 8c .. 8c+7.
template <bool BF16, bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const void* __restrict__ x, int64_t rows, int cols,
                                                            uint8_t* __restrict__ q, float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t rb_n = rows / 128;
  const int cb_n = cols / 128;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / (rb_n * cb_n);
  const int64_t rb = (blk / cb_n) % rb_n;
  const int cb = (int)(blk % cb_n);
  const int tid = threadIdx.x, r16 = tid / 16, c = tid % 16;
  const int64_t base = b * rows * cols + (rb * 128) * (int64_t)cols + cb * 128 + c * 8;
  float v[8][8];
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    load8<BF16>(x, base + (int64_t)(r16 + 16 * p) * cols, v[p]);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[p][i]));
  }
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid / 64] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = block_scale(m, POW2);
#pragma unroll
  for (int p = 0; p < 8; ++p)
    *reinterpret_cast<uint2*>(q + base + (int64_t)(r16 + 16 * p) * cols) = encode8(v[p], s);
  if (tid == 0) scales[blk] = s;
}

}  // namespace

extern "C" int moe_quant_fp8_block(const void* x, int x_dtype, int64_t batch, int64_t rows, int32_t cols,
                                   int32_t block_rows, int32_t scale_mode, uint8_t* q, float* scales, void* stream) {
  if (block_rows != 1 && block_rows != 128) return MOE_ERR_ARG;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (batch < 0 || rows < 0 || cols < 0 || cols % 128 != 0 || rows % block_rows != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  const int64_t nblocks = batch * (rows / block_rows) * (cols / 128);
  if (nblocks == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL;
  hipStream_t st = as_stream(stream);
  const bool bf16 = x_dtype == MOE_BF16, pow2 = scale_mode == MOE_SCALE_POW2;
  if (block_rows == 1) {
    const int64_t grid = ceil_div64(nblocks, 16 * Q1_U);
    if (grid > INT32_MAX) return MOE_ERR_SHAPE;
    auto k = bf16 ? (pow2 ? quant_1x128_kernel<true, true> : quant_1x128_kernel<true, false>)
                  : (pow2 ? quant_1x128_kernel<false, true> : quant_1x128_kernel<false, false>);
    k<<<(unsigned)grid, 256, 0, st>>>(x, nblocks, q, scales);
  } else {
    if (nblocks > INT32_MAX) return MOE_ERR_SHAPE;
    auto k = bf16 ? (pow2 ? quant_128x128_kernel<true, true> : quant_128x128_kernel<true, false>)
                  : (pow2 ? quant_128x128_kernel<false, true> : quant_128x128_kernel<false, false>);
    k<<<(unsigned)nblocks, 256, 0, st>>>(x, rows, cols, q, scales);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
