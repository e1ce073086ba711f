// Combine: out[t,:] = sum_j w[t,j] * y[dest_row[t,j],:] (+ y[shared_first_row + t,:]).
//
// One workgroup per (token, 2048-column slice); each thread owns 8 consecutive columns (16-byte
// bf16 or 2 x 16-byte fp32 loads).  The rows of up to 8 slots are loaded together (all loads in
// flight before the first use), then accumulated in fp32 with fused multiply-adds in slot order,
// the shared row added last, one rounding to the output dtype.  No atomics: each output element
// has one owner.  The residual form (a MoE layer on a residual branch, stacked) also adds the layer
// input: x_next = act(residual + act(sum)), the sum rounded to the activation dtype first, exactly
// as if the layer output were stored and then added in fp32 and rounded again.
#include "common.h"

namespace {

template <bool YBF16>
__device__ __forceinline__ void load8y(const void* y, int64_t off, float (&v)[8]) {
  if (YBF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool OBF16>
__device__ __forceinline__ void store8(void* __restrict__ out, int64_t off, const float (&v)[8]) {
  if (OBF16) {
    uint32_t p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + off) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + off);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// the value a float takes once stored in the output dtype
template <bool OBF16>
__device__ __forceinline__ float as_stored(float v) {
  return OBF16 ? bf16_to_f32(f32_to_bf16(v)) : v;
}

// RES: residual form (out may be NULL; x_next = act(residual + act(sum)), all in the output dtype)
template <bool YBF16, bool OBF16, bool RES = false>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w, int k, int H,
                                                      const int32_t* __restrict__ shared_first_row,
                                                      void* __restrict__ out, const void* residual = nullptr,
                                                      void* x_next = nullptr) {
  const int64_t t = blockIdx.x;
  const int32_t* d = dest + t * k;
  const float* wt = w + t * k;
  const int64_t srow = shared_first_row ? (int64_t)(*shared_first_row) + t : -1;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c < H) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += 8) {
      int32_t row[8];
      float v[8][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        row[j] = j0 + j < k ? d[j0 + j] : -1;
        if (row[j] >= 0) load8y<YBF16>(y, (int64_t)row[j] * H + c, v[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (row[j] < 0) continue;
        const float wj = wt[j0 + j];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(wj, v[j][q], acc[q]);
      }
    }
    if (srow >= 0) {
      float v[8];
      load8y<YBF16>(y, srow * H + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = acc[q] + v[q];
    }
    if (!RES || out) store8<OBF16>(out, t * H + c, acc);
    if (RES) {
      float r[8];
      load8y<OBF16>(residual, t * H + c, r);
#pragma unroll
      for (int q = 0; q < 8; ++q) r[q] = r[q] + as_stored<OBF16>(acc[q]);
      store8<OBF16>(x_next, t * H + c, r);
    }
  }
}

}  // namespace

extern "C" int moe_combine(const void* y, int y_dtype, const int32_t* dest_row, const float* topk_w, int64_t T,
                           int32_t k, int32_t H, const int32_t* shared_first_row, void* out, int out_dtype,
                           void* stream) {
  if (T < 0 || k < 1 || k > 64 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if ((y_dtype != MOE_BF16 && y_dtype != MOE_F32) || (out_dtype != MOE_BF16 && out_dtype != MOE_F32))
    return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!y || !dest_row || !topk_w || !out) return MOE_ERR_NULL;
  if (T > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  const dim3 grid((unsigned)T, (unsigned)ceil_div64(H, 256 * 8));
  const bool yb = y_dtype == MOE_BF16, ob = out_dtype == MOE_BF16;
  if (yb && ob)
    combine_kernel<true, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out);
  else if (yb)
    combine_kernel<true, false><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out);
  else if (ob)
    combine_kernel<false, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out);
  else
    combine_kernel<false, false><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_combine_residual(const void* y, int y_dtype, const int32_t* dest_row, const float* topk_w, int64_t T,
                                    int32_t k, int32_t H, const int32_t* shared_first_row, const void* residual,
                                    void* out, void* x_next, int act_dtype, void* stream) {
  if (T < 0 || k < 1 || k > 64 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if ((y_dtype != MOE_BF16 && y_dtype != MOE_F32) || (act_dtype != MOE_BF16 && act_dtype != MOE_F32))
    return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!y || !dest_row || !topk_w || !residual || !x_next) return MOE_ERR_NULL;
  if (T > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  const dim3 grid((unsigned)T, (unsigned)ceil_div64(H, 256 * 8));
  const bool yb = y_dtype == MOE_BF16, ob = act_dtype == MOE_BF16;
  if (yb && ob)
    combine_kernel<true, true, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out, residual,
                                                           x_next);
  else if (yb)
    combine_kernel<true, false, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out,
                                                            residual, x_next);
  else if (ob)
    combine_kernel<false, true, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out,
                                                            residual, x_next);
  else
    combine_kernel<false, false, true><<<grid, 256, 0, st>>>(y, dest_row, topk_w, k, H, shared_first_row, out,
                                                             residual, x_next);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
