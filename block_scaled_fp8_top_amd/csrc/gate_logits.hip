// Router gate projection: logits[t,e] = fp32 fma chain over h ascending (+ bias).
//
// The chain order is part of the contract (it makes routing reproducible bit for bit), so the
// contraction cannot use matrix cores or split K: it is fp32 VALU work.  Each thread owns a
// TT x TE register tile of outputs and walks h in order; x and Wg are staged through two LDS
// buffers in chunks of HC columns (x converted to fp32 on the way; the next chunk's global loads
// are in flight during the current chunk's chain), padded so that the 16-byte LDS reads of
// different rows fall in different banks.
#include "common.h"

namespace {

constexpr int HC = 32;        // h columns per LDS chunk
constexpr int PAD = HC + 4;   // padded LDS row (floats)
constexpr int NT = 256;       // threads per workgroup: 16 (experts) x 16 (tokens)

template <int TT, int TE, bool BF16>
__global__ __launch_bounds__(NT) void gate_logits_kernel(const void* __restrict__ xv, const float* __restrict__ wg,
                                                         const float* __restrict__ bias, int64_t T, int H, int E,
                                                         float* __restrict__ z) {
  constexpr int BT = 16 * TT, BE = 16 * TE;
  constexpr int XI = BT * (HC / 8), WI = BE * (HC / 8);   // 8-column staging items per chunk
  constexpr int XPT = (XI + NT - 1) / NT, WPT = (WI + NT - 1) / NT;
  // two LDS buffers: chunk c is read from buffer c & 1 while chunk c + 1 is written to the other
  __shared__ __attribute__((aligned(16))) float xs[2][BT * PAD];
  __shared__ __attribute__((aligned(16))) float ws[2][BE * PAD];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int e0 = blockIdx.y * BE;

  float acc[TT][TE];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

  // this thread's staging items of one chunk, held in registers between the global loads (issued
  // before the previous chunk's chain) and the LDS stores (after it)
  uint4 rxb[XPT];          // bf16 x: 8 values
  float4 rxf[XPT][2];      // fp32 x
  float4 rw[WPT][2];
  auto load = [&](int h0) {
    const int hc = min(HC, H - h0);
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int it = tid + q * NT;
      const int r = it / (HC / 8), c8 = (it % (HC / 8)) * 8;
      const int64_t t = t0 + r;
      const bool ok = it < XI && t < T && c8 < hc;
      if (BF16) {
        rxb[q] = ok ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(xv) + t * H + h0 + c8)
                    : make_uint4(0u, 0u, 0u, 0u);
      } else {
        const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xv) + t * H + h0 + c8);
        rxf[q][0] = ok ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        rxf[q][1] = ok ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int it = tid + q * NT;
      const int r = it / (HC / 8), c8 = (it % (HC / 8)) * 8;
      const int e = e0 + r;
      const bool ok = it < WI && e < E && c8 < hc;
      const float4* p = reinterpret_cast<const float4*>(wg + (int64_t)e * H + h0 + c8);
      rw[q][0] = ok ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      rw[q][1] = ok ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int it = tid + q * NT;
      if (it >= XI) continue;
      const int r = it / (HC / 8), c8 = (it % (HC / 8)) * 8;
      float4* d = reinterpret_cast<float4*>(&xs[buf][r * PAD + c8]);
      if (BF16) {
        const uint4 u = rxb[q];
        d[0] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                           __uint_as_float(u.y & 0xFFFF0000u));
        d[1] = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u), __uint_as_float(u.w << 16),
                           __uint_as_float(u.w & 0xFFFF0000u));
      } else {
        d[0] = rxf[q][0];
        d[1] = rxf[q][1];
      }
    }
#pragma unroll
    for (int q = 0; q < WPT; ++q) {
      const int it = tid + q * NT;
      if (it >= WI) continue;
      const int r = it / (HC / 8), c8 = (it % (HC / 8)) * 8;
      float4* d = reinterpret_cast<float4*>(&ws[buf][r * PAD + c8]);
      d[0] = rw[q][0];
      d[1] = rw[q][1];
    }
  };

  const int nchunk = (H + HC - 1) / HC;
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunk) load((c + 1) * HC);   // in flight during this chunk's chain
    const int hc = min(HC, H - c * HC);        // a multiple of 8
    // ---- the chain, 4 h at a time, strictly ascending
    for (int hh = 0; hh < hc; hh += 4) {
      float4 xr[TT], wr[TE];
#pragma unroll
      for (int i = 0; i < TT; ++i) xr[i] = *reinterpret_cast<const float4*>(&xs[buf][(ty * TT + i) * PAD + hh]);
#pragma unroll
      for (int j = 0; j < TE; ++j) wr[j] = *reinterpret_cast<const float4*>(&ws[buf][(tx * TE + j) * PAD + hh]);
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TE; ++j) {
          float a = acc[i][j];
          a = __builtin_fmaf(xr[i].x, wr[j].x, a);
          a = __builtin_fmaf(xr[i].y, wr[j].y, a);
          a = __builtin_fmaf(xr[i].z, wr[j].z, a);
          a = __builtin_fmaf(xr[i].w, wr[j].w, a);
          acc[i][j] = a;
        }
    }
    // the other buffer was last read during chunk c - 1, before the barrier that ended it
    if (c + 1 < nchunk) store(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int64_t t = t0 + ty * TT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = e0 + tx * TE + j;
      if (e >= E) continue;
      float v = acc[i][j];
      if (bias) v = v + bias[e];
      z[t * E + e] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Small problems (decode-sized T*E): one wavefront per 8 tokens x 8 experts, one logit per lane.
// Each output is a chain of H dependent fmas, so the launch is latency-bound and the per-lane
// instruction count per fma decides the time.  Chunks of 256 columns of x and Wg are copied
// global -> LDS by DMA (global_load_lds) into a ring of NSLOT slots, NSLOT-1 chunks ahead of the
// chain (as deep as the 6-bit vmcnt allows: five chunks for bf16 x, three for fp32); bf16 x
// is widened to fp32 once per chunk into a separate LDS block (each of the 64 lanes converts 32
// values, instead of every lane converting its whole row), so the chain loop is one 16-byte LDS
// read of x, one of Wg and four fmas per 4 columns.  LDS rows are padded by 16 bytes (bank spread).
constexpr int CH = 256;                       // columns per chunk
constexpr int WROW = CH * 4 + 16;             // padded fp32 row in LDS (bytes): Wg and widened x

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}

template <bool BF16>
__global__ __launch_bounds__(64) void gate_logits_chain_kernel(const void* __restrict__ xv, const float* __restrict__ wg,
                                                               const float* __restrict__ bias, int64_t T, int H,
                                                               int E, float* __restrict__ z) {
  constexpr int XB = BF16 ? 2 : 4;                       // bytes per x element
  constexpr int NSLOT = BF16 ? 6 : 4;
  constexpr int XROW = BF16 ? CH * 2 : WROW;             // raw x row in the ring (bytes)
  constexpr int XSLOT = 8 * XROW, WSLOT = 8 * WROW;
  constexpr int XINST = CH * XB / 1024;                  // DMA instructions per x row (1 KB each)
  __shared__ __attribute__((aligned(16))) uint8_t xs[NSLOT][XSLOT];
  __shared__ __attribute__((aligned(16))) uint8_t ws[NSLOT][WSLOT];
  __shared__ __attribute__((aligned(16))) uint8_t xf[BF16 ? 8 * WROW : 16];   // widened x of the current chunk
  const int lane = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 8;
  const int e0 = blockIdx.y * 8;
  const int tt = lane >> 3, ee = lane & 7;
  const int nchunk = (H + CH - 1) / CH;

  // DMA sources (rows clamped into range; columns past H fetch column 0 of the same row).
  //  bf16 x: one instruction per pair of rows (lanes 0-31: row 2p, lanes 32-63: row 2p+1; 8 columns
  //  per lane), landing as two consecutive 512-byte rows; fp32 x and Wg: one instruction per row.
  const uint32_t xbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&xs[0][0]);
  const uint32_t wbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&ws[0][0]);
  const char* wrow[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) wrow[r] = reinterpret_cast<const char*>(wg + (int64_t)min(e0 + r, E - 1) * H);

  auto issue = [&](int c, int slot) {
    const int h0 = c * CH;
    if (BF16) {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const int col = (lane & 31) * 8;
        const int h = h0 + col < H ? h0 + col : 0;
        const int64_t t = min(t0 + 2 * pr + (lane >> 5), T - 1);
        dma16(reinterpret_cast<const char*>(xv) + (t * H + h) * 2, xbase + slot * XSLOT + pr * 2 * XROW);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int h = h0 + lane * 4 < H ? h0 + lane * 4 : 0;
        const int64_t t = min(t0 + r, T - 1);
        dma16(reinterpret_cast<const char*>(xv) + (t * H + h) * 4, xbase + slot * XSLOT + r * XROW);
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int h = h0 + lane * 4 < H ? h0 + lane * 4 : 0;
      dma16(wrow[r] + (int64_t)h * 4, wbase + slot * WSLOT + r * WROW);
    }
  };
  constexpr int PER_CHUNK = (BF16 ? 4 : 8) + 8;          // DMA instructions per chunk
  static_assert(XINST <= 1, "x row chunk fits one DMA instruction");
  static_assert((NSLOT - 1) * PER_CHUNK <= 63 && NSLOT <= 6, "in-flight DMA fits vmcnt");

  for (int c = 0; c < NSLOT - 1 && c < nchunk; ++c) issue(c, c);
  float acc = 0.0f;
  for (int c = 0; c < nchunk; ++c) {
    const int left = min(nchunk - 1 - c, NSLOT - 2);   // chunks issued after c that may stay in flight
    switch (left) {
      case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER_CHUNK) : "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER_CHUNK) : "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER_CHUNK) : "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER_CHUNK) : "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + NSLOT - 1 < nchunk) issue(c + NSLOT - 1, (c + NSLOT - 1) % NSLOT);
    const int slot = c % NSLOT;
    const uint8_t* xr;
    if (BF16) {
      // widen: lane L converts row L/8, columns 32 (L%8) .. +32
      const int r = lane >> 3, c0 = (lane & 7) * 32;
      const uint8_t* src = &xs[slot][r * XROW + c0 * 2];
      uint8_t* dst = &xf[r * WROW + c0 * 4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 u = *reinterpret_cast<const uint4*>(src + q * 16);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
        float4 lo, hi;
        lo.x = __uint_as_float(w4[0] << 16); lo.y = __uint_as_float(w4[0] & 0xFFFF0000u);
        lo.z = __uint_as_float(w4[1] << 16); lo.w = __uint_as_float(w4[1] & 0xFFFF0000u);
        hi.x = __uint_as_float(w4[2] << 16); hi.y = __uint_as_float(w4[2] & 0xFFFF0000u);
        hi.z = __uint_as_float(w4[3] << 16); hi.w = __uint_as_float(w4[3] & 0xFFFF0000u);
        *reinterpret_cast<float4*>(dst + q * 32) = lo;
        *reinterpret_cast<float4*>(dst + q * 32 + 16) = hi;
      }
      xr = &xf[tt * WROW];   // one wavefront: its LDS writes land before its later LDS reads
    } else {
      xr = &xs[slot][tt * XROW];
    }
    const uint8_t* wr = &ws[slot][ee * WROW];
    const int hc = min(CH, H - c * CH);   // a multiple of 8
    if (hc == CH) {
      // full chunk: 8 batches of 32 columns, fully unrolled; the next batch's LDS reads are issued
      // before this batch's fmas so their latency overlaps the chain
      constexpr int U = 8, NB = CH / (4 * U);
      float4 xb[2][U], wb[2][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        xb[0][u] = *reinterpret_cast<const float4*>(xr + u * 16);
        wb[0][u] = *reinterpret_cast<const float4*>(wr + u * 16);
      }
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        if (bt + 1 < NB) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            xb[(bt + 1) & 1][u] = *reinterpret_cast<const float4*>(xr + ((bt + 1) * 4 * U + 4 * u) * 4);
            wb[(bt + 1) & 1][u] = *reinterpret_cast<const float4*>(wr + ((bt + 1) * 4 * U + 4 * u) * 4);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float4 xv4 = xb[bt & 1][u], wv4 = wb[bt & 1][u];
          acc = __builtin_fmaf(xv4.x, wv4.x, acc);
          acc = __builtin_fmaf(xv4.y, wv4.y, acc);
          acc = __builtin_fmaf(xv4.z, wv4.z, acc);
          acc = __builtin_fmaf(xv4.w, wv4.w, acc);
        }
      }
    } else {
      for (int hh = 0; hh < hc; hh += 4) {   // the last, partial chunk
        const float4 xv4 = *reinterpret_cast<const float4*>(xr + hh * 4);
        const float4 wv4 = *reinterpret_cast<const float4*>(wr + hh * 4);
        acc = __builtin_fmaf(xv4.x, wv4.x, acc);
        acc = __builtin_fmaf(xv4.y, wv4.y, acc);
        acc = __builtin_fmaf(xv4.z, wv4.z, acc);
        acc = __builtin_fmaf(xv4.w, wv4.w, acc);
      }
    }
  }
  const int64_t t = t0 + tt;
  const int e = e0 + ee;
  if (t < T && e < E) {
    float v = acc;
    if (bias) v = v + bias[e];
    z[t * E + e] = v;
  }
}

template <int TT, int TE>
int launch(const void* x, bool bf16, const float* wg, const float* bias, int64_t T, int H, int E, float* z,
           hipStream_t st) {
  dim3 grid((unsigned)ceil_div64(T, 16 * TT), (unsigned)ceil_div64(E, 16 * TE));
  if (bf16)
    gate_logits_kernel<TT, TE, true><<<grid, NT, 0, st>>>(x, wg, bias, T, H, E, z);
  else
    gate_logits_kernel<TT, TE, false><<<grid, NT, 0, st>>>(x, wg, bias, T, H, E, z);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

}  // namespace

extern "C" int moe_gate_logits(const void* x, int x_dtype, const float* wg, const float* bias, int64_t T, int32_t H,
                               int32_t E, float* logits, void* stream) {
  if (T < 0 || H < 1 || E < 1 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!x || !wg || !logits) return MOE_ERR_NULL;
  if (E > 65535 * 16 || T > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  const bool bf16 = x_dtype == MOE_BF16;
  hipStream_t st = as_stream(stream);
  if (T * (int64_t)E <= 131072) {
    dim3 grid((unsigned)ceil_div64(T, 8), (unsigned)ceil_div64(E, 8));
    if (bf16)
      gate_logits_chain_kernel<true><<<grid, 64, 0, st>>>(x, wg, bias, T, H, E, logits);
    else
      gate_logits_chain_kernel<false><<<grid, 64, 0, st>>>(x, wg, bias, T, H, E, logits);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  // Larger register tiles amortise LDS reads; use them only when they still give >= 512
  // workgroups (two per CU), because each output is one long dependent chain.
  const int64_t wg84 = ceil_div64(T, 128) * ceil_div64(E, 64);
  const int64_t wg44 = ceil_div64(T, 64) * ceil_div64(E, 64);
  const int64_t wg22 = ceil_div64(T, 32) * ceil_div64(E, 32);
  if (wg84 >= 512) return launch<8, 4>(x, bf16, wg, bias, T, H, E, logits, st);
  if (wg44 >= 512) return launch<4, 4>(x, bf16, wg, bias, T, H, E, logits, st);
  if (wg22 >= 512) return launch<2, 2>(x, bf16, wg, bias, T, H, E, logits, st);
  return launch<1, 1>(x, bf16, wg, bias, T, H, E, logits, st);
}
