// Backward of the block-scaled FP8 MoE layer: the kernels that are not grouped GEMMs.
//
// "RL at 1T Scale: prime-rl Performance Deep Dive", section "FP8 training": the trainer runs the
// inference recipe (DeepSeek V3's block-scaled FP8), so its backward contracts in FP8 as well;
// section "Router replay": the selection is replayed, so it is a fixed input here and only the
// routing weights carry gradient.  The data-gradient GEMMs are the forward grouped GEMM run on
// transposed weights (a 128x128 block keeps its scale under transposition, so no re-quantisation):
//
//   combine backward   dY[dest(t,j)] = w[t,j] * dout[t] (dY = dout for the shared row), 1x128
//                      quantised along H; dw[t,j] = <dout[t], Y[dest(t,j)]>
//   GEMM (W2^T)        dh = deq(dY) deq(W2)                         [rows, F]   fp32
//   GEMM (W1, store)   G = deq(A) deq(W1)^T, recomputed             [rows, 2F]  fp32
//   SwiGLU backward    dgate = dh up s (1 + gate (1 - s)), dup = dh gate s, s = sigmoid(gate);
//                      1x128 quantised along 2F
//   GEMM (W1^T)        dA = deq(dG) deq(W1)                         [rows, H]
//   combine (w = 1)    dx_experts[t] = sum_j dA[dest(t,j)] + dA_shared[t]
//   router backward    dz from dw with the configured score function and normalisation
//
// All of these kernels are HBM-bound elementwise / row passes; each reads its inputs once.
#include <algorithm>

#include "common.h"

namespace {

template <bool BF16>
__device__ __forceinline__ void load8v(const void* x, int64_t i, float (&v)[8]) {
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

// 1x128 quantisation of 8 values held by each of 16 consecutive lanes (one block): the block's
// scale and the 8 codes of this lane
__device__ __forceinline__ uint2 quant8_block(const float (&v)[8], bool pow2, float& s) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = row16_max(m);   // the 16 lanes are one aligned DPP row
  s = block_scale(m, pow2);
  return encode8(v, s);
}

constexpr int CB_THREADS = 256;      // combine backward: one workgroup per token
constexpr int CB_KMAX = 16;          // slots per token handled by one workgroup

// Combine backward.  Thread i of the workgroup owns columns c = 2048 p + 8 i .. +7 for p = 0, 1,
// ...; 16 consecutive threads cover one 128-column block, so the block maxima are 16-lane
// reductions.  For each slot: dY = w * dout (one fp32 product), quantised and stored at the
// slot's row; the slot's dw partial accumulates dout * Y with fused multiply-adds, and the
// partials are reduced across the workgroup at the end (fixed order: deterministic).
template <bool DBF16, bool YBF16, bool POW2>
__global__ __launch_bounds__(CB_THREADS) void combine_backward_kernel(
    const void* __restrict__ dout, const void* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ w, int k, int H, const int32_t* __restrict__ shared_first_row,
    uint8_t* __restrict__ dyq, float* __restrict__ dys, float* __restrict__ dw, float* __restrict__ row_w) {
  __shared__ float red[CB_THREADS / 64][CB_KMAX];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, sub = tid & 15;
  const int HB = H / 128;
  int32_t row[CB_KMAX];
  float wt[CB_KMAX], acc[CB_KMAX];
#pragma unroll
  for (int j = 0; j < CB_KMAX; ++j) {
    row[j] = j < k ? dest[t * k + j] : -1;
    wt[j] = j < k ? w[t * k + j] : 0.0f;
    acc[j] = 0.0f;
  }
  const int64_t srow = shared_first_row ? (int64_t)(*shared_first_row) + t : -1;
  // each written row's factor, for the weight gradients' dY operand
  if (row_w && tid < k && dest[t * k + tid] >= 0) row_w[dest[t * k + tid]] = w[t * k + tid];
  if (row_w && tid == 64 && srow >= 0) row_w[srow] = 1.0f;
  for (int c = tid * 8; c < H; c += CB_THREADS * 8) {
    // 16-lane groups are whole blocks (H % 128 == 0), so a group is entirely in or out of range
    float d[8];
    load8v<DBF16>(dout, t * H + c, d);
#pragma unroll
    for (int j = 0; j < CB_KMAX; ++j) {
      if (row[j] < 0) continue;   // uniform: the whole workgroup serves one token
      float v[8], s;
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = wt[j] * d[q];
      const uint2 codes = quant8_block(v, POW2, s);
      *reinterpret_cast<uint2*>(dyq + (int64_t)row[j] * H + c) = codes;
      if (sub == 0) dys[(int64_t)row[j] * HB + c / 128] = s;
      float yv[8];
      load8v<YBF16>(y, (int64_t)row[j] * H + c, yv);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[j] = __builtin_fmaf(d[q], yv[q], acc[j]);
    }
    if (srow >= 0) {
      float s;
      const uint2 codes = quant8_block(d, POW2, s);
      *reinterpret_cast<uint2*>(dyq + srow * H + c) = codes;
      if (sub == 0) dys[srow * HB + c / 128] = s;
    }
  }
#pragma unroll
  for (int j = 0; j < CB_KMAX; ++j) {
    float v = acc[j];   // slots j >= k accumulated nothing
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((tid & 63) == 0) red[tid >> 6][j] = v;
  }
  __syncthreads();
  if (tid < k) {
    float v = 0.0f;
#pragma unroll
    for (int wv = 0; wv < CB_THREADS / 64; ++wv) v += red[wv][tid];
    dw[t * k + tid] = v;   // a slot routed nowhere accumulated nothing: 0
  }
}

// SwiGLU backward + 1x128 quantisation.  16 lanes per (row, 128-column block of F); lane owns 8
// consecutive columns f.  dG columns [0, F) are dgate and [F, 2F) dup, so each group writes one
// block of each.
template <bool POW2>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const float* __restrict__ dh, const float* __restrict__ g,
                                                              int64_t rows, int F, uint8_t* __restrict__ dgq,
                                                              float* __restrict__ dgs) {
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int FB = F / 128;
  const int64_t grp = gt >> 4;
  if (grp >= rows * FB) return;   // whole 16-lane groups
  const int sub = threadIdx.x & 15;
  const int64_t r = grp / FB;
  const int fb = (int)(grp % FB);
  const int f = fb * 128 + sub * 8;
  float d[8], gate[8], up[8];
  load8v<false>(dh, r * F + f, d);
  load8v<false>(g, r * 2 * F + f, gate);
  load8v<false>(g, r * 2 * F + F + f, up);
  float dg[8], du[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float s = 1.0f / (1.0f + __expf(-gate[q]));
    dg[q] = d[q] * up[q] * s * (1.0f + gate[q] * (1.0f - s));
    du[q] = d[q] * gate[q] * s;
  }
  float s0, s1;
  const uint2 c0 = quant8_block(dg, POW2, s0);
  const uint2 c1 = quant8_block(du, POW2, s1);
  *reinterpret_cast<uint2*>(dgq + r * 2 * F + f) = c0;
  *reinterpret_cast<uint2*>(dgq + r * 2 * F + F + f) = c1;
  if (sub == 0) {
    dgs[r * 2 * FB + fb] = s0;
    dgs[r * 2 * FB + FB + fb] = s1;
  }
}

// Router backward, one 64-lane workgroup per token (selection held fixed; slots with index -1
// carry nothing).  Scores come from the router's own exp, as in the forward:
//   sigmoid s = 1 / (1 + exp(-z));  softmax p = exp(z - max) / sum (full softmax over E).
//   renormalised, w_j = score_j / sum_l score_l:
//     sigmoid  dz_{i_j} = s_j (1 - s_j) (dw_j - sum_l w_l dw_l) / sum_l s_l
//     softmax  dz_{i_j} = w_j (dw_j - sum_l w_l dw_l)
//   not renormalised, w_j = score_j:
//     sigmoid  dz_{i_j} = dw_j s_j (1 - s_j)
//     softmax  dz_e = [e selected] w_e dw_e - p_e sum_l w_l dw_l  (every expert)
// Each dz element is written once, by the lane that owns its expert.
__global__ __launch_bounds__(64) void route_backward_kernel(const float* __restrict__ z, const int32_t* __restrict__ idx,
                                                            const float* __restrict__ dw, int E, int k, int score_fn,
                                                            int renorm, float* __restrict__ dz) {
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* zt = z + t * E;
  // the selected slots: lane j < k holds slot j
  int e_j = -1;
  float dw_j = 0.0f, sc_j = 0.0f;
  if (lane < k) {
    e_j = idx[t * k + lane];
    dw_j = dw[t * k + lane];
  }
  float m = -INFINITY, S = 0.0f;
  if (score_fn == MOE_SCORE_SOFTMAX) {
    for (int e = lane; e < E; e += 64) m = fmaxf(m, zt[e]);
    m = wave_max(m);
    for (int e = lane; e < E; e += 64) S += router_exp(zt[e] - m);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    if (e_j >= 0) sc_j = router_exp(zt[e_j] - m) / S;
  } else if (e_j >= 0) {
    sc_j = router_sigmoid(zt[e_j]);
  }
  // sums over the valid slots: sum score, and sum w dw
  float ssum = e_j >= 0 ? sc_j : 0.0f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ssum += __shfl_xor(ssum, o, 64);
  const float w_j = e_j < 0 ? 0.0f : (renorm ? sc_j / ssum : sc_j);
  float wdw = w_j * dw_j;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wdw += __shfl_xor(wdw, o, 64);
  float g_j = 0.0f;   // the selected expert's dz contribution (besides the dense softmax term)
  if (e_j >= 0) {
    if (score_fn == MOE_SCORE_SIGMOID)
      g_j = renorm ? sc_j * (1.0f - sc_j) * (dw_j - wdw) / ssum : dw_j * sc_j * (1.0f - sc_j);
    else
      g_j = renorm ? w_j * (dw_j - wdw) : w_j * dw_j;
  }
  const bool dense = score_fn == MOE_SCORE_SOFTMAX && !renorm;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    float v = dense && e < E ? -(router_exp(zt[e] - m) / S) * wdw : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e_j, j, 64);
      const float gj = __shfl(g_j, j, 64);
      if (ej == e) v += gj;
    }
    if (e < E) dz[t * E + e] = v;
  }
}

// Transpose of 128x128-block FP8 weights: qt[g][c][r] = q[g][r][c], st[g][cb][rb] = s[g][rb][cb].
// One workgroup per 128x128 block: 16-byte row pieces into LDS (row pitch 132 bytes), then each
// thread gathers 16 bytes of one output row (16 consecutive source rows of one column).
__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                               int N, int K, uint8_t* __restrict__ qt,
                                                               float* __restrict__ st) {
  constexpr int P = 132;
  __shared__ uint8_t tile[128 * P];
  const int NB = N / 128, KB = K / 128;
  const int64_t blk = blockIdx.x;
  const int64_t g = blk / ((int64_t)NB * KB);
  const int rb = (int)((blk / KB) % NB), cb = (int)(blk % KB);
  const uint8_t* src = q + (g * N + (int64_t)rb * 128) * K + (int64_t)cb * 128;
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int u = tid + 256 * p;          // 1024 pieces: row u / 8, piece u % 8
    const int r = u >> 3, pc = u & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * K + pc * 16);
    uint32_t* d = reinterpret_cast<uint32_t*>(&tile[r * P + pc * 16]);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();
  uint8_t* dst = qt + (g * K + (int64_t)cb * 128) * N + (int64_t)rb * 128;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int u = tid + 256 * p;          // output row c = u / 8 (source column), piece u % 8
    const int c = u >> 3, pc = u & 7;
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) x |= (uint32_t)tile[(pc * 16 + 4 * i + b) * P + c] << (8 * b);
      wv[i] = x;
    }
    *reinterpret_cast<uint4*>(dst + (int64_t)c * N + pc * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
  if (tid == 0) st[(g * KB + cb) * NB + rb] = s[(g * NB + rb) * KB + cb];
}

}  // namespace

extern "C" int moe_combine_backward(const void* dout, int dout_dtype, const void* y, int y_dtype,
                                    const int32_t* dest_row, const float* topk_w, int64_t T, int32_t k, int32_t H,
                                    const int32_t* shared_first_row, int32_t scale_mode, uint8_t* dyq, float* dys,
                                    float* dw, float* row_w, void* stream) {
  if (T < 0 || k < 1 || k > CB_KMAX || H < 128 || H % 128 != 0) return MOE_ERR_SHAPE;
  if ((dout_dtype != MOE_BF16 && dout_dtype != MOE_F32) || (y_dtype != MOE_BF16 && y_dtype != MOE_F32))
    return MOE_ERR_DTYPE;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!dout || !y || !dest_row || !topk_w || !dyq || !dys || !dw) return MOE_ERR_NULL;
  if (T > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  const bool db = dout_dtype == MOE_BF16, yb = y_dtype == MOE_BF16, p2 = scale_mode == MOE_SCALE_POW2;
#define CB_LAUNCH(A, B, C)                                                                                    \
  combine_backward_kernel<A, B, C><<<(unsigned)T, CB_THREADS, 0, st>>>(dout, y, dest_row, topk_w, k, H,     \
                                                                      shared_first_row, dyq, dys, dw, row_w)
  if (db && yb) { if (p2) CB_LAUNCH(true, true, true); else CB_LAUNCH(true, true, false); }
  else if (db) { if (p2) CB_LAUNCH(true, false, true); else CB_LAUNCH(true, false, false); }
  else if (yb) { if (p2) CB_LAUNCH(false, true, true); else CB_LAUNCH(false, true, false); }
  else { if (p2) CB_LAUNCH(false, false, true); else CB_LAUNCH(false, false, false); }
#undef CB_LAUNCH
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_swiglu_backward_quant(const float* dh, const float* g, int64_t rows, int32_t F,
                                         int32_t scale_mode, uint8_t* dgq, float* dgs, void* stream) {
  if (rows < 0 || F < 128 || F % 128 != 0) return MOE_ERR_SHAPE;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (rows == 0) return MOE_OK;
  if (!dh || !g || !dgq || !dgs) return MOE_ERR_NULL;
  const int64_t threads = rows * (F / 128) * 16;
  const int64_t grid = ceil_div64(threads, 256);
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  if (scale_mode == MOE_SCALE_POW2)
    swiglu_backward_kernel<true><<<(unsigned)grid, 256, 0, st>>>(dh, g, rows, F, dgq, dgs);
  else
    swiglu_backward_kernel<false><<<(unsigned)grid, 256, 0, st>>>(dh, g, rows, F, dgq, dgs);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_route_backward(const float* logits, const int32_t* topk_idx, const float* dw, int64_t T,
                                  const moe_router_cfg* cfg, float* dz, void* stream) {
  if (!cfg) return MOE_ERR_NULL;
  const int E = cfg->num_experts, k = cfg->top_k;
  if (T < 0 || E < 1 || k < 1 || k > E || k > 64) return MOE_ERR_SHAPE;
  if (cfg->score_fn != MOE_SCORE_SOFTMAX && cfg->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !dw || !dz) return MOE_ERR_NULL;
  if (T > INT32_MAX) return MOE_ERR_SHAPE;
  route_backward_kernel<<<(unsigned)T, 64, 0, as_stream(stream)>>>(logits, topk_idx, dw, E, k, cfg->score_fn,
                                                                    cfg->renormalize ? 1 : 0, dz);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_transpose_fp8_blocks(const uint8_t* q, const float* scales, int32_t groups, int32_t N, int32_t K,
                                        uint8_t* qt, float* scales_t, void* stream) {
  if (groups < 0 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (groups == 0) return MOE_OK;
  if (!q || !scales || !qt || !scales_t) return MOE_ERR_NULL;
  if (q == qt) return MOE_ERR_ARG;
  const int64_t blocks = (int64_t)groups * (N / 128) * (K / 128);
  if (blocks > INT32_MAX) return MOE_ERR_SHAPE;
  transpose_blocks_kernel<<<(unsigned)blocks, 256, 0, as_stream(stream)>>>(q, scales, N, K, qt, scales_t);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
