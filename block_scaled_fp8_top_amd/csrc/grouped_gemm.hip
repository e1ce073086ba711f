// Grouped block-scaled FP8 GEMM on gfx950 matrix cores.
//
// out[r, n] = sum_kb (as[r,kb] * bs[g, n/128, kb]) * sum_{k in kb} a[r,k] * b[g,n,k]   for rows r of group g.
//
// One K block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3, fp32 result), so
// every MFMA produces a fresh 128-wide partial P that is promoted into the fp32 accumulator with
// its scale product: acc = fma(P, as * bs, acc).
//
// Workgroup tile: BM = 128 rows x BN = 256 (virtual) columns, 8 wavefronts in a 2 x 4 grid, each
// computing 64 x 64 as 4 x 4 MFMA tiles of 16 x 16.  A and B K-slices (128 bytes per row) are
// double-buffered in LDS with a 16-byte-chunk XOR swizzle (chunk c of row r at c ^ (r & 7)) so
// that the 16 rows read by one MFMA operand fetch spread over the banks.
//
// Epilogue STORE writes out in bf16 or fp32.  Epilogue SWIGLU_QUANT maps the 256 virtual columns
// of a tile to 128 gate columns [f0, f0+128) and the matching 128 up columns [F+f0, F+f0+128); each
// wave holds gate and up of the same 32 h columns in the same lanes, forms h = silu(gate) * up in
// fp32, and the tile's 128 h columns are one 1x128 quantisation block (amax across the 4 waves of
// a row through LDS).
//
// Row tiles never straddle groups: a small kernel turns `offsets` into a list of (group, first row)
// tiles in the workspace; surplus workgroups of the fixed-size grid exit at once.
#include <algorithm>

#include "common.h"

namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NTHREADS = 512;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 4); }

// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int groups,
                                                        int2* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                        int max_tiles) {
  __shared__ int part[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int g0 = 0; g0 < groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int nt = 0;
    if (g < groups) nt = (offsets[g + 1] - offsets[g] + BM - 1) / BM;
    part[threadIdx.x] = nt;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int start = carry + part[threadIdx.x] - nt;
    if (g < groups)
      for (int i = 0; i < nt && start + i < max_tiles; ++i) tiles[start + i] = make_int2(g, offsets[g] + i * BM);
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) *ntiles = min(carry, max_tiles);
}

// ------------------------------------------------------------------------------------------------
template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const int32_t* __restrict__ offsets,
    const int2* __restrict__ tiles, const int32_t* __restrict__ ntiles, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, int N, int K, void* __restrict__ out, float* __restrict__ out_scales) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][BN * BK];
  __shared__ float as_lds[2][BM];
  __shared__ float red[2][4][64];

  if ((int)blockIdx.x >= *ntiles) return;
  const int2 tile = tiles[blockIdx.x];
  const int g = tile.x;
  const int row0 = tile.y;
  const int row_end = min(row0 + BM, offsets[g + 1]);
  const int KB = K / BK;
  const int F = N / 2;                         // SwiGLU only
  const int n0 = blockIdx.y * (EPI == 1 ? 128 : BN);   // first h column (SwiGLU) or output column
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  const uint8_t* bg = b + (size_t)g * N * K;
  const float* bsg = bs + (size_t)g * (N / 128) * KB;

  // ---- global -> register staging assignments
  // A: 128 rows x 8 chunks = 1024 chunks, 2 per thread; B: 256 rows x 8 chunks, 4 per thread.
  int a_row[2], a_chk[2];
  const uint8_t* a_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * NTHREADS;
    a_row[i] = c >> 3;
    a_chk[i] = c & 7;
    const int r = min(row0 + a_row[i], row_end - 1);   // rows past the group end: any valid row
    a_src[i] = a + (size_t)r * K + a_chk[i] * 16;
  }
  int b_row[4], b_chk[4];
  const uint8_t* b_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * NTHREADS;
    b_row[i] = c >> 3;
    b_chk[i] = c & 7;
    int n;
    if (EPI == 1) n = b_row[i] < 128 ? n0 + b_row[i] : F + n0 + (b_row[i] - 128);
    else n = min(n0 + b_row[i], N - 1);
    b_src[i] = bg + (size_t)n * K + b_chk[i] * 16;
  }
  const float* as_src = as + (size_t)min(row0 + (tid & 127), row_end - 1) * KB;

  // ---- wave's B rows in the LDS tile and its B scale row-blocks
  int b_lrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (EPI == 1) b_lrow[ns] = ns < 2 ? wn * 32 + ns * 16 : 128 + wn * 32 + (ns - 2) * 16;
    else b_lrow[ns] = wn * 64 + ns * 16;
  }
  const int nb_lo = EPI == 1 ? n0 / 128 : (n0 + wn * 64) / 128;
  const int nb_hi = EPI == 1 ? (F + n0) / 128 : nb_lo;
  const bool wave_active = EPI == 1 ? true : (n0 + wn * 64 < N);

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[2], rb[4];
  float ras = 0.f;
  auto gload = [&](int kb) {
    const size_t ko = (size_t)kb * BK;
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + ko);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + ko);
    if (tid < BM) ras = as_src[kb];
  };
  auto lstore = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&a_lds[s][swz(a_row[i], a_chk[i])]) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&b_lds[s][swz(b_row[i], b_chk[i])]) = rb[i];
    if (tid < BM) as_lds[s][tid] = ras;
  };

  gload(0);
  lstore(0);
  __syncthreads();

  const int lr = lane & 15;         // row within a 16-row operand tile
  const int kc = (lane >> 4) * 2;   // first of the two 16-byte K chunks this lane supplies
  for (int kb = 0; kb < KB; ++kb) {
    const int s = kb & 1;
    if (kb + 1 < KB) gload(kb + 1);
    if (wave_active) {
      const float sb_lo = bsg[nb_lo * KB + kb];
      const float sb_hi = bsg[nb_hi * KB + kb];
      intx8 af[4], bf[4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const int r = wm * 64 + ms * 16 + lr;
        const intx4 lo = *reinterpret_cast<const intx4*>(&a_lds[s][swz(r, kc)]);
        const intx4 hi = *reinterpret_cast<const intx4*>(&a_lds[s][swz(r, kc + 1)]);
        af[ms] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const int r = b_lrow[ns] + lr;
        const intx4 lo = *reinterpret_cast<const intx4*>(&b_lds[s][swz(r, kc)]);
        const intx4 hi = *reinterpret_cast<const intx4*>(&b_lds[s][swz(r, kc + 1)]);
        bf[ns] = intx8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      float sa[4][4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[ms][i] = as_lds[s][wm * 64 + ms * 16 + (lane >> 4) * 4 + i];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        float c_lo[4], c_hi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c_lo[i] = sa[ms][i] * sb_lo;
          c_hi[i] = sa[ms][i] * sb_hi;
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const floatx4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[ms], bf[ns], floatx4{0.f, 0.f, 0.f, 0.f},
                                                                             0, 0, 0, 0, 0, 0);
          const bool hi = EPI == 1 && ns >= 2;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[ms][ns][i] = __builtin_fmaf(p[i], hi ? c_hi[i] : c_lo[i], acc[ms][ns][i]);
        }
      }
    }
    if (kb + 1 < KB) lstore(s ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if (EPI == 0) {
    if (!wave_active) return;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + wm * 64 + ms * 16 + (lane >> 4) * 4 + i;
        if (r >= row_end) continue;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const int col = n0 + wn * 64 + ns * 16 + lr;
          if (OUT_BF16)
            reinterpret_cast<uint16_t*>(out)[(size_t)r * N + col] = f32_to_bf16(acc[ms][ns][i]);
          else
            reinterpret_cast<float*>(out)[(size_t)r * N + col] = acc[ms][ns][i];
        }
      }
  } else {
    // h for this lane: rows (ms, i), columns wn*32 + hs*16 + lr (hs = 0, 1)
    float h[4][2][4];
    float m[4][4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.0f;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const float gt = acc[ms][hs][i], up = acc[ms][hs + 2][i];
          const float v = (gt * up) / (1.0f + __expf(-gt));
          h[ms][hs][i] = v;
          mx = fmaxf(mx, fabsf(v));
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        m[ms][i] = mx;
      }
    // cross-wave amax over the 4 waves (wn) that share these rows
    if (lr == 0) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wm][wn][ms * 16 + (lane >> 4) * 4 + i] = m[ms][i];
    }
    __syncthreads();
    uint8_t* hq = reinterpret_cast<uint8_t*>(out);
    const int FB = F / 128;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lrow = ms * 16 + (lane >> 4) * 4 + i;
        const float amax = fmaxf(fmaxf(red[wm][0][lrow], red[wm][1][lrow]), fmaxf(red[wm][2][lrow], red[wm][3][lrow]));
        const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
        const int r = row0 + wm * 64 + lrow;
        if (r >= row_end) continue;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int col = n0 + wn * 32 + hs * 16 + lr;
          hq[(size_t)r * F + col] = (uint8_t)(e4m3_pack2(h[ms][hs][i] / sc, 0.0f) & 0xFF);
        }
        if (wn == 0 && lr == 0) out_scales[(size_t)r * FB + n0 / 128] = sc;
      }
  }
}

int max_tiles_for(int64_t max_rows, int groups) { return (int)(ceil_div64(max_rows, BM) + groups); }

}  // namespace

size_t moe_gemm_workspace(int64_t max_rows, int32_t groups) {
  return (size_t)max_tiles_for(max_rows, groups) * sizeof(int2) + 256;
}

extern "C" int moe_grouped_gemm_fp8(const uint8_t* a, const float* as, const int32_t* offsets, int32_t groups,
                                    int64_t max_rows, const uint8_t* b, const float* bs, int32_t N, int32_t K,
                                    int32_t epilogue, void* out, int out_dtype, float* out_scales, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (groups < 1 || groups > 4096 || max_rows < 0 || max_rows > INT32_MAX - 2 * BM) return MOE_ERR_SHAPE;
  if (N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (epilogue == MOE_EPI_STORE) {
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  } else if (epilogue == MOE_EPI_SWIGLU_QUANT) {
    if (out_dtype != MOE_FP8_E4M3) return MOE_ERR_DTYPE;
    if (N % 256 != 0) return MOE_ERR_SHAPE;   // F = N/2 must be a multiple of 128
  } else {
    return MOE_ERR_ARG;
  }
  if (max_rows == 0) return MOE_OK;
  if (!a || !as || !offsets || !b || !bs || !out) return MOE_ERR_NULL;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && !out_scales) return MOE_ERR_NULL;
  if (!workspace || workspace_bytes < moe_gemm_workspace(max_rows, groups)) return MOE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  const int mt = max_tiles_for(max_rows, groups);
  int2* tiles = reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(workspace) + 256);
  int32_t* ntiles = reinterpret_cast<int32_t*>(workspace);
  tile_map_kernel<<<1, 1024, 0, st>>>(offsets, groups, tiles, ntiles, mt);
  MOE_CHECK_LAUNCH();
  if (epilogue == MOE_EPI_STORE) {
    dim3 grid((unsigned)mt, (unsigned)ceil_div64(N, BN));
    if (out_dtype == MOE_BF16)
      grouped_gemm_kernel<0, true><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, b, bs, N, K, out, nullptr);
    else
      grouped_gemm_kernel<0, false><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, b, bs, N, K, out, nullptr);
  } else {
    dim3 grid((unsigned)mt, (unsigned)(N / 256));
    grouped_gemm_kernel<1, false><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, b, bs, N, K, out,
                                                             out_scales);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
