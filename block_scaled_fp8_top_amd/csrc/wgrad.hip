// Expert-weight gradients of the block-scaled FP8 MoE layer.
//
// "RL at 1T Scale: prime-rl Performance Deep Dive", section "FP8 training": the trainer runs the
// block-scaled FP8 recipe (DeepSeek V3's), so the weight gradients contract in FP8 as well:
//   dW2[e] = sum over e's rows r of dY[r]^T h[r]      [H, F]
//   dW1[e] = sum over e's rows r of dG[r]^T x[r]      [2F, H]
// Both operands contract over an expert's rows, so they are quantised in 128x1 blocks (128
// consecutive rows of one expert by one column) and stored transposed, one contiguous block per
// expert: expert e's rows fill K_e = 128 * ntiles_e padded rows (zero-padded), and its block
// [C, K_e] (codes; scales [C, ntiles_e]) starts at tile_first[e] * 128 * C bytes (scales at
// tile_first[e] * C), tile_first = exclusive prefix sum of ntiles_e = ceil(rows_e / 128).  A block
// is contiguous so that the GEMM's reads of one expert stay within a few MB.
//
//   moe_wgrad_tiles            tile_first [G+1] from the group offsets
//   moe_colwise_quant_rows     dY = w * dout gathered per row (or x gathered per row), 128x1 codes
//   moe_colwise_quant_swiglu   h = silu(gate) up, or dG = [dgate | dup], from the GEMM1 output G
//   moe_grouped_gemm_wgrad     C_e = A_e B_e^T over e's segment, fp32 out, one matrix per expert
#include <algorithm>

#include "common.h"

namespace {

// ------------------------------------------------------------------------------------------------
// tile_first[g] = sum_{g' < g} ceil(rows_g' / 128); tile_first[G] = total.  One workgroup.
__global__ __launch_bounds__(1024) void wgrad_tiles_kernel(const int32_t* __restrict__ offsets, int groups,
                                                           int32_t* __restrict__ tile_first) {
  __shared__ int part[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int g0 = 0; g0 < groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    const int nt = g < groups ? (offsets[g + 1] - offsets[g] + 127) / 128 : 0;
    part[threadIdx.x] = nt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    if (g < groups) tile_first[g] = carry + part[threadIdx.x] - nt;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_first[groups] = carry;
}

// the group whose tile range holds tile b (tile_first ascending), or -1 past the last tile
__device__ __forceinline__ int group_of_tile(const int32_t* __restrict__ tile_first, int groups, int b) {
  if (b >= tile_first[groups]) return -1;
  int lo = 0, hi = groups - 1;   // largest g with tile_first[g] <= b
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_first[mid] <= b) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------------------------------------
// 128x1 quantisation of one 128-row tile x 64 columns.  Thread (rr = tid / 16, cc = tid % 16) holds
// rows 8 rr .. 8 rr + 7 and columns 4 cc .. 4 cc + 3 of the tile; a column's maximum is reduced over
// the 16 threads that share cc (lanes 16 apart within a wave, then across the 4 waves); each thread
// then stores 8 codes (its 8 rows) per column as one 8-byte piece of the transposed operand.
constexpr int CQ_COLS = 64;

template <bool POW2>
__device__ __forceinline__ void colwise_store(float (&v)[8][4], int tile, int tf0, int ntiles, int C, int c0,
                                              uint8_t* __restrict__ qt, float* __restrict__ st) {
  __shared__ float red[4][CQ_COLS];
  const int tid = threadIdx.x, rr = tid >> 4, cc = tid & 15, lane = tid & 63, wave = tid >> 6;
  __syncthreads();   // a previous call's reads of red are done
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i][j]));
    a = fmaxf(a, __shfl_xor(a, 16, 64));
    a = fmaxf(a, __shfl_xor(a, 32, 64));
    m[j] = a;
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][cc * 4 + j] = m[j];
  }
  __syncthreads();
  // the expert's block: codes [C, 128 ntiles] at 128 C tf0, scales [C, ntiles] at C tf0
  const int64_t kg = (int64_t)ntiles * 128;
  uint8_t* qb = qt + (int64_t)tf0 * 128 * C;
  float* sb = st + (int64_t)tf0 * C;
  const int lt = tile - tf0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = cc * 4 + j;
    const float amax = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
    const float s = block_scale(amax, POW2);
    const float col[8] = {v[0][j], v[1][j], v[2][j], v[3][j], v[4][j], v[5][j], v[6][j], v[7][j]};
    float r[8];
    quotients<8>(col, s, r);
    const uint32_t lo = e4m3_pack4(r[0], r[1], r[2], r[3]);
    const uint32_t hi = e4m3_pack4(r[4], r[5], r[6], r[7]);
    *reinterpret_cast<uint2*>(qb + (int64_t)(c0 + c) * kg + lt * 128 + rr * 8) = make_uint2(lo, hi);
    if (rr == 0) sb[(int64_t)(c0 + c) * ntiles + lt] = s;
  }
}

// rows of x (or of dout) gathered per dispatched row, times an optional per-row factor
template <bool XBF16, bool POW2>
__global__ __launch_bounds__(256) void colquant_rows_kernel(const void* __restrict__ x, const int32_t* __restrict__ src,
                                                            const float* __restrict__ rowf,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ tile_first, int groups, int C,
                                                            uint8_t* __restrict__ qt, float* __restrict__ st) {
  const int tile = blockIdx.x;
  const int g = group_of_tile(tile_first, groups, tile);
  if (g < 0) return;
  const int r0 = offsets[g] + (tile - tile_first[g]) * 128, r1 = offsets[g + 1];
  const int c0 = blockIdx.y * CQ_COLS;
  const int tid = threadIdx.x, rr = tid >> 4, cc = tid & 15;
  float v[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + rr * 8 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[i][j] = 0.0f;
    if (r < r1) {
      const int64_t t = src ? (int64_t)src[r] : (int64_t)r;
      const float f = rowf ? rowf[r] : 1.0f;
      const int64_t off = t * C + c0 + cc * 4;
      if (XBF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
        v[i][0] = __uint_as_float(u.x << 16); v[i][1] = __uint_as_float(u.x & 0xFFFF0000u);
        v[i][2] = __uint_as_float(u.y << 16); v[i][3] = __uint_as_float(u.y & 0xFFFF0000u);
      } else {
        const float4 q = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
        v[i][0] = q.x; v[i][1] = q.y; v[i][2] = q.z; v[i][3] = q.w;
      }
      if (rowf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = f * v[i][j];
      }
    }
  }
  colwise_store<POW2>(v, tile, tile_first[g], tile_first[g + 1] - tile_first[g], C, c0, qt, st);
}

// from the GEMM1 output G = [gate | up] ([rows, 2F] fp32): h = silu(gate) up (C = F), or with dh
// ([rows, F] fp32) dG = [dgate | dup] (C = 2F) in exactly the SwiGLU backward's operations.  A
// workgroup covers features f0 .. f0 + 63; for dG it writes both halves (columns f and F + f) from
// one read of gate, up and dh.
template <bool DG, bool POW2>
__global__ __launch_bounds__(256) void colquant_swiglu_kernel(const float* __restrict__ gm, const float* __restrict__ dh,
                                                              int F, const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ tile_first, int groups,
                                                              uint8_t* __restrict__ qt, float* __restrict__ st) {
  const int tile = blockIdx.x;
  const int g = group_of_tile(tile_first, groups, tile);
  if (g < 0) return;
  const int r0 = offsets[g] + (tile - tile_first[g]) * 128, r1 = offsets[g + 1];
  const int f0 = blockIdx.y * CQ_COLS;
  const int tid = threadIdx.x, rr = tid >> 4, cc = tid & 15;
  const int f = f0 + cc * 4;
  float v[8][4], u[8][4];   // h or dgate; dup
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + rr * 8 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[i][j] = u[i][j] = 0.0f;
    if (r < r1) {
      const float4 ga = *reinterpret_cast<const float4*>(gm + (int64_t)r * 2 * F + f);
      const float4 ua = *reinterpret_cast<const float4*>(gm + (int64_t)r * 2 * F + F + f);
      const float gv[4] = {ga.x, ga.y, ga.z, ga.w}, uv[4] = {ua.x, ua.y, ua.z, ua.w};
      if (!DG) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = (gv[j] * uv[j]) / (1.0f + __expf(-gv[j]));
      } else {
        const float4 da = *reinterpret_cast<const float4*>(dh + (int64_t)r * F + f);
        const float dv[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s = 1.0f / (1.0f + __expf(-gv[j]));
          v[i][j] = dv[j] * uv[j] * s * (1.0f + gv[j] * (1.0f - s));
          u[i][j] = dv[j] * gv[j] * s;
        }
      }
    }
  }
  const int nt = tile_first[g + 1] - tile_first[g];
  colwise_store<POW2>(v, tile, tile_first[g], nt, DG ? 2 * F : F, f0, qt, st);
  if (DG) colwise_store<POW2>(u, tile, tile_first[g], nt, 2 * F, F + f0, qt, st);
}

// ------------------------------------------------------------------------------------------------
// C_e [M, N] = A_e B_e^T over expert e's K_e padded rows, A_e [M, K_e] and B_e [N, K_e] the experts'
// blocks of 128x1-quantised codes (scales [M or N, K_e/128]).  One workgroup
// per 128 x 128 output tile of one expert (grid N/128, M/128, G); four waves of 64 x 64 each
// (4 x 4 MFMA 16x16x128 tiles); k in 128-wide steps, the next step's operands loaded into registers
// during the current step's MFMAs, LDS double-buffered.  An expert with no rows gets zeros.
// amax scales: each 128-wide step's product is promoted with its scale products s_A[m] s_B[n]
// (the weights side of a lane's 4 outputs has 4 different scales); power-of-two scales: the matrix
// cores apply both as E8M0 exponents.
constexpr int WG_T = 128;

__device__ __forceinline__ int wswz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
}

template <bool POW2>
__global__ __launch_bounds__(256) void wgrad_gemm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                         const uint8_t* __restrict__ b, const float* __restrict__ bs,
                                                         int M, int N, const int32_t* __restrict__ tile_first,
                                                         float* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) uint8_t la[2][WG_T * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][WG_T * 128];
  __shared__ __attribute__((aligned(16))) float lsa[2][WG_T];
  __shared__ __attribute__((aligned(16))) float lsb[2][WG_T];
  const int n0 = blockIdx.x * WG_T, m0 = blockIdx.y * WG_T, g = blockIdx.z;
  const int t0 = tile_first[g], t1 = tile_first[g + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kt = t1 - t0;                     // the expert's 128-row tiles
  const int64_t kg = (int64_t)kt * 128;        // row length of its blocks
  // staging: 1024 16-byte pieces per operand per step; thread takes pieces tid + 256 p
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  float rsv = 0.0f;   // this thread's scale: A rows for tid < 128, B rows above
  const int srow_ = tid & 127;
  const float* sp_ = tid < 128 ? as + (int64_t)t0 * M + (int64_t)(m0 + srow_) * kt
                                : bs + (int64_t)t0 * N + (int64_t)(n0 + srow_) * kt;
  // piece p of a thread: row (tid + 256 p) / 8 = tid / 8 + 32 p, 16-byte chunk tid % 8
  const int prow = tid >> 3, pch = tid & 7;
  const uint8_t* pa_ = a + (int64_t)t0 * 128 * M + (int64_t)(m0 + prow) * kg + pch * 16;
  const uint8_t* pb_ = b + (int64_t)t0 * 128 * N + (int64_t)(n0 + prow) * kg + pch * 16;
  const int64_t pstep = 32 * kg;
#define WG_LOAD(TILE)                                                                       \
  do {                                                                                      \
    const int64_t k0_ = (int64_t)((TILE) - t0) * 128;                                       \
    ra0 = *reinterpret_cast<const uint4*>(pa_ + k0_);                                       \
    ra1 = *reinterpret_cast<const uint4*>(pa_ + pstep + k0_);                               \
    ra2 = *reinterpret_cast<const uint4*>(pa_ + 2 * pstep + k0_);                           \
    ra3 = *reinterpret_cast<const uint4*>(pa_ + 3 * pstep + k0_);                           \
    rb0 = *reinterpret_cast<const uint4*>(pb_ + k0_);                                       \
    rb1 = *reinterpret_cast<const uint4*>(pb_ + pstep + k0_);                               \
    rb2 = *reinterpret_cast<const uint4*>(pb_ + 2 * pstep + k0_);                           \
    rb3 = *reinterpret_cast<const uint4*>(pb_ + 3 * pstep + k0_);                           \
    rsv = sp_[(TILE) - t0];                                                                 \
  } while (0)
#define WG_STORE(BUF)                                                                       \
  do {                                                                                      \
    *reinterpret_cast<uint4*>(&la[BUF][wswz(prow, pch)]) = ra0;                             \
    *reinterpret_cast<uint4*>(&la[BUF][wswz(prow + 32, pch)]) = ra1;                        \
    *reinterpret_cast<uint4*>(&la[BUF][wswz(prow + 64, pch)]) = ra2;                        \
    *reinterpret_cast<uint4*>(&la[BUF][wswz(prow + 96, pch)]) = ra3;                        \
    *reinterpret_cast<uint4*>(&lb[BUF][wswz(prow, pch)]) = rb0;                             \
    *reinterpret_cast<uint4*>(&lb[BUF][wswz(prow + 32, pch)]) = rb1;                        \
    *reinterpret_cast<uint4*>(&lb[BUF][wswz(prow + 64, pch)]) = rb2;                        \
    *reinterpret_cast<uint4*>(&lb[BUF][wswz(prow + 96, pch)]) = rb3;                        \
    if (tid < 128) lsa[BUF][srow_] = rsv;                                                   \
    else lsb[BUF][srow_] = rsv;                                                             \
  } while (0)
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int lr = lane & 15, lq = lane >> 4;
  if (t0 < t1) {
    WG_LOAD(t0);
    WG_STORE(0);
  }
  __syncthreads();
  int buf = 0;
  for (int tile = t0; tile < t1; ++tile) {
    const bool more = tile + 1 < t1;
    if (more) WG_LOAD(tile + 1);
    // B fragments of the step stay in registers; A fragments and the amax path's products are
    // taken one 16-row block at a time, which keeps the kernel at two waves per SIMD
    intx8 bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rb_ = wn * 64 + i * 16 + lr;
      const intx4 blo = *reinterpret_cast<const intx4*>(&lb[buf][wswz(rb_, 2 * lq)]);
      const intx4 bhi = *reinterpret_cast<const intx4*>(&lb[buf][wswz(rb_, 2 * lq + 1)]);
      bf[i] = intx8{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
    }
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const int ra_ = wm * 64 + ms * 16 + lr;
      const intx4 alo = *reinterpret_cast<const intx4*>(&la[buf][wswz(ra_, 2 * lq)]);
      const intx4 ahi = *reinterpret_cast<const intx4*>(&la[buf][wswz(ra_, 2 * lq + 1)]);
      const intx8 af = intx8{alo[0], alo[1], alo[2], alo[3], ahi[0], ahi[1], ahi[2], ahi[3]};
      if (POW2) {
        const uint32_t ea = e8m0_code(lsa[buf][ra_]);
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          acc[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[ns], af, acc[ms][ns], 0, 0, 0, e8m0_code(lsb[buf][wn * 64 + ns * 16 + lr]), 0, ea);
      } else {
        floatx4 p[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          p[ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ns], af, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                   0, 0, 0);
        const float sa = lsa[buf][ra_];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const float4 sb = *reinterpret_cast<const float4*>(&lsb[buf][wn * 64 + ns * 16 + 4 * lq]);
          const float sbv[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ms][ns][r] = __builtin_fmaf(p[ns][r], sa * sbv[r], acc[ms][ns][r]);
        }
      }
    }
    if (more) WG_STORE(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  // lane: output row m = m0 + wm*64 + ms*16 + lr, columns n0 + wn*64 + ns*16 + 4 lq .. +3
  float* cg = c + (int64_t)g * M * N;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int64_t m = m0 + wm * 64 + ms * 16 + lr;
      const int n = n0 + wn * 64 + ns * 16 + 4 * lq;
      *reinterpret_cast<float4*>(cg + m * N + n) =
          make_float4(acc[ms][ns][0], acc[ms][ns][1], acc[ms][ns][2], acc[ms][ns][3]);
    }
#undef WG_LOAD
#undef WG_STORE
}

int check_seg(int32_t groups, int64_t max_tiles, int32_t C) {
  if (groups < 1 || groups > 4096 || max_tiles < 0 || max_tiles > INT32_MAX / 128 || C < 128 || C % 128 != 0)
    return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" int64_t moe_wgrad_max_tiles(int64_t max_rows, int32_t groups) {
  if (max_rows < 0 || groups < 1) return 0;
  return ceil_div64(max_rows, 128) + groups;
}

extern "C" int moe_wgrad_tiles(const int32_t* offsets, int32_t groups, int32_t* tile_first, void* stream) {
  if (groups < 1 || groups > 4096) return MOE_ERR_SHAPE;
  if (!offsets || !tile_first) return MOE_ERR_NULL;
  wgrad_tiles_kernel<<<1, 1024, 0, as_stream(stream)>>>(offsets, groups, tile_first);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_colwise_quant_rows(const void* x, int x_dtype, const int32_t* src_row, const float* row_scale,
                                      const int32_t* offsets, const int32_t* tile_first, int32_t groups,
                                      int64_t max_tiles, int32_t C, int32_t scale_mode, uint8_t* qt, float* st,
                                      void* stream) {
  int rc = check_seg(groups, max_tiles, C);
  if (rc != MOE_OK) return rc;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (max_tiles == 0) return MOE_OK;
  if (!x || !offsets || !tile_first || !qt || !st) return MOE_ERR_NULL;
  const dim3 grid((unsigned)max_tiles, (unsigned)(C / CQ_COLS));
  hipStream_t s = as_stream(stream);
  const bool bf = x_dtype == MOE_BF16, p2 = scale_mode == MOE_SCALE_POW2;
  auto k = bf ? (p2 ? colquant_rows_kernel<true, true> : colquant_rows_kernel<true, false>)
              : (p2 ? colquant_rows_kernel<false, true> : colquant_rows_kernel<false, false>);
  k<<<grid, 256, 0, s>>>(x, src_row, row_scale, offsets, tile_first, groups, C, qt, st);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_colwise_quant_swiglu(const float* g, const float* dh, int32_t F, const int32_t* offsets,
                                        const int32_t* tile_first, int32_t groups, int64_t max_tiles,
                                        int32_t scale_mode, uint8_t* qt, float* st, void* stream) {
  int rc = check_seg(groups, max_tiles, F);
  if (rc != MOE_OK) return rc;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (max_tiles == 0) return MOE_OK;
  if (!g || !offsets || !tile_first || !qt || !st) return MOE_ERR_NULL;
  const dim3 grid((unsigned)max_tiles, (unsigned)(F / CQ_COLS));
  hipStream_t s = as_stream(stream);
  const bool p2 = scale_mode == MOE_SCALE_POW2;
  if (dh) {
    auto k = p2 ? colquant_swiglu_kernel<true, true> : colquant_swiglu_kernel<true, false>;
    k<<<grid, 256, 0, s>>>(g, dh, F, offsets, tile_first, groups, qt, st);
  } else {
    auto k = p2 ? colquant_swiglu_kernel<false, true> : colquant_swiglu_kernel<false, false>;
    k<<<grid, 256, 0, s>>>(g, dh, F, offsets, tile_first, groups, qt, st);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_grouped_gemm_wgrad(const uint8_t* a, const float* as, int32_t M, const uint8_t* b, const float* bs,
                                      int32_t N, const int32_t* tile_first, int32_t groups, int64_t max_tiles,
                                      int32_t scale_mode, float* c, void* stream) {
  if (groups < 1 || groups > 65535 || max_tiles < 0 || max_tiles > INT32_MAX / 128) return MOE_ERR_SHAPE;
  if (M < 128 || N < 128 || M % 128 != 0 || N % 128 != 0 || M / 128 > 65535) return MOE_ERR_SHAPE;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (!a || !as || !b || !bs || !tile_first || !c) return MOE_ERR_NULL;
  const dim3 grid((unsigned)(N / WG_T), (unsigned)(M / WG_T), (unsigned)groups);
  if (scale_mode == MOE_SCALE_POW2)
    wgrad_gemm_kernel<true><<<grid, 256, 0, as_stream(stream)>>>(a, as, b, bs, M, N, tile_first, c);
  else
    wgrad_gemm_kernel<false><<<grid, 256, 0, as_stream(stream)>>>(a, as, b, bs, M, N, tile_first, c);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
