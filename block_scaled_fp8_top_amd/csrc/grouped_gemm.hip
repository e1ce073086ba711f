// Grouped block-scaled FP8 GEMM on gfx950 matrix cores.
//
// out[r, n] = sum_kb (as[r,kb] * bs[g, n/128, kb]) * sum_{k in kb} a[r,k] * b[g,n,k]   for rows r of group g.
//
// One K block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3, fp32 result), so
// every MFMA produces a fresh 128-wide partial P that is promoted into the fp32 accumulator with
// its scale product: acc = fma(P, as * bs, acc).
//
// Workgroup tile: BM = 128 rows x BN = 256 (virtual) columns, 8 wavefronts in a 2 x 4 grid, each
// computing 64 x 64 as 4 x 4 MFMA tiles of 16 x 16.
//
// Data movement: the A and B K-slices (128 bytes per row) and the tile's activation scales go
// straight from global memory into a 3-stage LDS ring with global_load_lds (no registers in
// between), issued two K steps ahead; each wavefront waits for its own loads with an explicit
// vmcnt and a bare s_barrier publishes the stage (a __syncthreads fence would drain every load in
// flight).  Rows are stored with a 16-byte-chunk XOR swizzle (chunk c of row r at slot
// c ^ ((r >> 1) & 7): the 16 rows one MFMA operand read touches then hit 16 distinct bank groups),
// applied on the global side: lane L of a DMA instruction writes LDS slot L, so it
// fetches the chunk that belongs there.  Weight scales travel through scalar loads in a 3-deep ring.
//
// Tile order: a one-workgroup kernel turns `offsets` into the list of 128-row tiles (never
// straddling a group).  The grid is one-dimensional; hardware workgroup ids are dealt to the 8
// XCDs round-robin, so they are renumbered to make each XCD's ids contiguous, and logical tiles
// run expert by expert, N-tile-major, so the workgroups alive on one XCD share the same A rows and
// B columns in that XCD's L2.
//
// Epilogue STORE writes out in bf16 or fp32.  Epilogue SWIGLU_QUANT maps the 256 virtual columns
// of a tile to 128 gate columns [f0, f0+128) and the matching 128 up columns [F+f0, F+f0+128); each
// wave holds gate and up of the same 32 h columns in the same lanes, forms h = silu(gate) * up in
// fp32, and the tile's 128 h columns are one 1x128 quantisation block (amax across the 4 waves of
// a row through LDS).
#include <algorithm>

#include "common.h"

namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NTHREADS = 512;
constexpr int NSTAGE = 3;
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane L's bytes land at lds_addr + 16 L (4 L).
// Issued through inline assembly so that the compiler's conservative wait insertion (it cannot tell
// which LDS stage an in-flight DMA targets) does not drain the pipeline; every wait on these loads
// is explicit.  M0 holds the wave-uniform LDS address and has no other user in these kernels.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// ------------------------------------------------------------------------------------------------
// tiles[i] = {group, first row, index of the group's first tile, number of tiles of the group}
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int groups,
                                                        int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
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
      for (int i = 0; i < nt && start + i < max_tiles; ++i) tiles[start + i] = make_int4(g, offsets[g] + i * BM, start, nt);
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) *ntiles = min(carry, max_tiles);
}

// wait until at most n of this wave's vector memory instructions are outstanding (immediate operand)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
  }
}

// ------------------------------------------------------------------------------------------------
template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const float* __restrict__ as, const int32_t* __restrict__ offsets,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, int ny, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, int N, int K, void* __restrict__ out, float* __restrict__ out_scales) {
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds[NSTAGE][A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b_lds[NSTAGE][B_BYTES];
  __shared__ __attribute__((aligned(16))) float as_lds[4][BM];   // scale ring: slot kb & 3
  __shared__ float red[2][4][64];

  // ---- logical tile: XCD-contiguous renumbering, then expert-major, N-tile-major order
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int L = xcd * (nwg >> 3) + min(xcd, nwg & 7) + slot;
  const int q = L / ny;
  if (q >= *ntiles) return;
  const int4 tq = tiles[q];
  const int local = L - tq.z * ny;
  const int nt_idx = local / tq.w;
  const int mt_idx = local - nt_idx * tq.w;
  const int g = tq.x;
  const int row0 = offsets[g] + mt_idx * BM;
  const int row_end = min(row0 + BM, offsets[g + 1]);
  const int KB = K / BK;
  const int F = N / 2;                                   // SwiGLU only
  const int n0 = nt_idx * (EPI == 1 ? 128 : BN);         // first h column (SwiGLU) or output column
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;

  const uint8_t* bg = b + (size_t)g * N * K;
  const float* bsg = bs + (size_t)g * (N / 128) * KB;

  // ---- this lane's DMA sources: A rows j*8 + lane/8 for j = 2*wave + {0,1}; B rows for j = 4*wave + {0..3}
  const int drow = lane >> 3, dslot = lane & 7;
  // 32-bit byte offsets from a / from this group's weights (both < 2^32 for every supported shape)
  uint32_t aoff0, aoff1, boff[4];
  {
    const int r0 = (2 * wave) * 8 + drow, r1 = r0 + 8;
    aoff0 = (uint32_t)min(row0 + r0, row_end - 1) * (uint32_t)K + ((dslot ^ ((r0 >> 1) & 7)) << 4);   // rows past the
    aoff1 = (uint32_t)min(row0 + r1, row_end - 1) * (uint32_t)K + ((dslot ^ ((r1 >> 1) & 7)) << 4);   // group end: any row
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (4 * wave + i) * 8 + drow;
    int n;
    if (EPI == 1) n = r < 128 ? n0 + r : F + n0 + (r - 128);
    else n = min(n0 + r, N - 1);
    boff[i] = (uint32_t)n * (uint32_t)K + ((dslot ^ ((r >> 1) & 7)) << 4);
  }
  const float* ssrc = as + (size_t)min(row0 + (wave & 1) * 64 + lane, row_end - 1) * KB;   // waves 0, 1
  const bool scale_loader = wave < 2;
  const int per_stage = scale_loader ? 7 : 6;   // vector memory instructions per stage for this wave

  // ---- wave's B rows in the LDS tile and its B scale row-blocks
  int b_lrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    if (EPI == 1) b_lrow[ns] = ns < 2 ? wn * 32 + ns * 16 : 128 + wn * 32 + (ns - 2) * 16;
    else b_lrow[ns] = wn * 64 + ns * 16;
  }
  const int nb_lo = EPI == 1 ? n0 / 128 : min(n0 + wn * 64, N - 1) / 128;
  const int nb_hi = EPI == 1 ? (F + n0) / 128 : nb_lo;
  const bool wave_active = EPI == 1 ? true : (n0 + wn * 64 < N);

  // wave-uniform LDS destinations of this wave's DMA instructions, stage 0; stage s adds s * stride
  const uint32_t a_dst = lds_u32(&a_lds[0][(2 * wave) * 1024]);
  const uint32_t b_dst = lds_u32(&b_lds[0][(4 * wave) * 1024]);
  const uint32_t s_dst = lds_u32(&as_lds[0][(wave & 1) * 64]);
#define GEMM_ISSUE(KBV, ST)                                                   \
  do {                                                                        \
    const uint32_t ko_ = (uint32_t)(KBV) * BK;                                \
    const uint32_t ao_ = a_dst + (uint32_t)(ST) * A_BYTES;                    \
    const uint32_t bo_ = b_dst + (uint32_t)(ST) * B_BYTES;                    \
    dma16(a + (aoff0 + ko_), ao_);                                            \
    dma16(a + (aoff1 + ko_), ao_ + 1024);                                     \
    dma16(bg + (boff[0] + ko_), bo_);                                         \
    dma16(bg + (boff[1] + ko_), bo_ + 1024);                                  \
    dma16(bg + (boff[2] + ko_), bo_ + 2048);                                  \
    dma16(bg + (boff[3] + ko_), bo_ + 3072);                                  \
    if (scale_loader) dma4(ssrc + (KBV), s_dst + (uint32_t)((KBV) & 3) * BM * 4); \
  } while (0)

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;         // row within a 16-row operand tile
  const int kc = (lane >> 4) * 2;   // first of the two 16-byte K chunks this lane supplies
  // operand fragments of one K step, read from LDS stage ST
  intx8 af[4], bf[4];
#define GEMM_READ(ST)                                                                                   \
  do {                                                                                                  \
    _Pragma("unroll") for (int ms = 0; ms < 4; ++ms) {                                                  \
      const int r_ = wm * 64 + ms * 16 + lr;                                                            \
      const intx4 lo_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, kc)]);                       \
      const intx4 hi_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, kc + 1)]);                   \
      af[ms] = intx8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};                   \
    }                                                                                                   \
    _Pragma("unroll") for (int ns = 0; ns < 4; ++ns) {                                                  \
      const int r_ = b_lrow[ns] + lr;                                                                   \
      const intx4 lo_ = *reinterpret_cast<const intx4*>(&b_lds[ST][swz(r_, kc)]);                       \
      const intx4 hi_ = *reinterpret_cast<const intx4*>(&b_lds[ST][swz(r_, kc + 1)]);                   \
      bf[ns] = intx8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};                   \
    }                                                                                                   \
  } while (0)

  GEMM_ISSUE(0, 0);
  if (KB > 1) GEMM_ISSUE(1, 1);
  float sbl0 = bsg[nb_lo * KB], sbh0 = bsg[nb_hi * KB];
  float sbl1 = KB > 1 ? bsg[nb_lo * KB + 1] : 0.f, sbh1 = KB > 1 ? bsg[nb_hi * KB + 1] : 0.f;
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb % NSTAGE;
    wait_vm(kb + 1 < KB ? per_stage : 0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    float sbl2 = 0.f, sbh2 = 0.f;
    if (kb + 2 < KB) {
      GEMM_ISSUE(kb + 2, (kb + 2) % NSTAGE);
      sbl2 = bsg[nb_lo * KB + kb + 2];
      sbh2 = bsg[nb_hi * KB + kb + 2];
    }
    if (wave_active) {
      GEMM_READ(st);
      const float* srow = &as_lds[kb & 3][wm * 64 + (lane >> 4) * 4];
      floatx4 p[4][4];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          p[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[ms], bf[ns], floatx4{0.f, 0.f, 0.f, 0.f},
                                                                       0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        const floatx4 sa = *reinterpret_cast<const floatx4*>(srow + ms * 16);
        floatx4 c_lo, c_hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c_lo[i] = sa[i] * sbl0;
          c_hi[i] = sa[i] * sbh0;
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const bool hi = EPI == 1 && ns >= 2;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[ms][ns][i] = __builtin_fmaf(p[ms][ns][i], hi ? c_hi[i] : c_lo[i], acc[ms][ns][i]);
        }
      }
    }
    sbl0 = sbl1;
    sbh0 = sbh1;
    sbl1 = sbl2;
    sbh1 = sbh2;
  }
#undef GEMM_READ
#undef GEMM_ISSUE

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
        if (lr == 0) red[wm][wn][ms * 16 + (lane >> 4) * 4 + i] = mx;
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
  return (size_t)max_tiles_for(max_rows, groups) * sizeof(int4) + 256;
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
  int4* tiles = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(workspace) + 256);
  int32_t* ntiles = reinterpret_cast<int32_t*>(workspace);
  tile_map_kernel<<<1, 1024, 0, st>>>(offsets, groups, tiles, ntiles, mt);
  MOE_CHECK_LAUNCH();
  const int ny = (int)(epilogue == MOE_EPI_STORE ? ceil_div64(N, BN) : N / 256);
  const int64_t nwg = (int64_t)mt * ny;
  if (nwg > INT32_MAX) return MOE_ERR_SHAPE;
  const unsigned grid = (unsigned)nwg;
  if (epilogue == MOE_EPI_STORE) {
    if (out_dtype == MOE_BF16)
      grouped_gemm_kernel<0, true><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
                                                              nullptr);
    else
      grouped_gemm_kernel<0, false><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
                                                               nullptr);
  } else {
    grouped_gemm_kernel<1, false><<<grid, NTHREADS, 0, st>>>(a, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
                                                             out_scales);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
