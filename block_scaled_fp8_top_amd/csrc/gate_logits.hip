// Router gate projection: logits[t,e] = fp32 fma chain over h ascending (+ bias).
//
// The chain order is part of the contract (it makes routing reproducible bit for bit), so the
// contraction cannot use matrix cores or split K: it is fp32 VALU work.  Three kernels, chosen by
// size (moe_gate_logits): register tiles, the x-broadcast kernel and a one-logit-per-lane chain.
// Tiles: each thread owns a TT x TE register tile of outputs and walks h in order; x and Wg are
// staged through two LDS buffers in chunks of HC columns (x converted to fp32 on the way; the next
// chunk's global loads are in flight during the current chunk's chain), padded so that the 16-byte
// LDS reads of different rows fall in different banks.
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

// ------------------------------------------------------------------------------------------------
// Many tokens, E of 64, 128 or 256, H a multiple of 32: x broadcast within 16-lane rows.
// A wavefront owns TT tokens and a slice of 64 TE experts (workgroup column blockIdx.y: experts
// e0 = 64 TE blockIdx.y onwards; lane l: experts e0 + l, e0 + l + 64, ...), so a Wg value read from
// LDS serves TT fmas (the tile kernel above reads an x value and a Wg value from LDS for every
// TT x TE tile, twice the LDS bytes per fma at TT = TE = 4).  The x of a 32-column
// chunk sits in two registers per token, lane 16 r + k holding columns 2k and 2k + 1, and the fma of
// column h takes it from lane h / 2 of the lane's own row through a DPP row broadcast
// (row_newbcast) fused into the fma, v_fmac_f32_dpp.  Chunks of Wg (E rows of 128 bytes, 16-byte
// pieces XOR-swizzled by row so that eight rows' reads of one piece hit distinct banks) and of raw x
// are copied global -> LDS by DMA (global_load_lds) into two buffers, one chunk ahead of the chain
// (a deeper ring for x, which is read once from HBM, measured no faster).  Workgroup: NW wavefronts,
// NW TT tokens, one expert slice.  Slices of 128 experts (TE = 2) rather than all 256 keep the
// workgroup's LDS at 34 KB, so four workgroups (16 wavefronts) share a CU; at 8192 tokens, H 6144,
// 256 experts and bf16 x that measured 420 us against 446 us for whole-E workgroups (TE = 4), and
// 423-438 us for 8 or 16 tokens per wavefront over 128 or 64 experts.
//
// A DPP source register needs two wait states after a VALU instruction writes it, which the
// compiler does not insert for inline assembly: the widened x registers pass through an s_nop 1
// that takes them as operands, so every DPP read of them comes after it.
constexpr int BC_HC = 32;   // h columns per chunk

template <int K>
__device__ __forceinline__ void fmac_row_bcast(float& acc, float x, float w) {
  asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(x), "v"(w), "i"(K));
}

__device__ __forceinline__ void bc_dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}

// columns HL .. 31 of a chunk, four at a time: per expert of the lane one 16-byte LDS read (the
// row's piece HL / 4, at its swizzled slot woff[HL / 4]) gives four columns; the reads of the next
// piece are issued before the fmas of this one
template <int TT, int TE>
__device__ __forceinline__ void bc_read(float4 (&w4)[TE], const uint8_t* __restrict__ wbuf, int off) {
#pragma unroll
  for (int j = 0; j < TE; ++j) w4[j] = *reinterpret_cast<const float4*>(wbuf + j * 64 * 128 + off);
}
template <int HL, int TT, int TE>
__device__ __forceinline__ void bcast_chunk(float (&acc)[TT][TE], const float (&xa)[TT], const float (&xb)[TT],
                                            const uint8_t* __restrict__ wbuf, const int (&woff)[8],
                                            const float4 (&w4)[TE]) {
  float4 nx[TE];
  if constexpr (HL + 4 < BC_HC) bc_read<TT, TE>(nx, wbuf, woff[HL / 4 + 1]);
#define BC_COL(M, C)                                                                        \
  _Pragma("unroll") for (int i = 0; i < TT; ++i)                                            \
    _Pragma("unroll") for (int j = 0; j < TE; ++j)                                          \
      fmac_row_bcast<(HL + M) / 2>(acc[i][j], (M) % 2 == 0 ? xa[i] : xb[i], w4[j].C);
  BC_COL(0, x)
  BC_COL(1, y)
  BC_COL(2, z)
  BC_COL(3, w)
#undef BC_COL
  if constexpr (HL + 4 < BC_HC) bcast_chunk<HL + 4, TT, TE>(acc, xa, xb, wbuf, woff, nx);
}

template <int TT, int TE, int NW, bool BF16>
__global__ __launch_bounds__(NW * 64) void gate_logits_bcast_kernel(const void* __restrict__ xv,
                                                                  const float* __restrict__ wg,
                                                                  const float* __restrict__ bias, int64_t T, int H,
                                                                  int EALL, float* __restrict__ z) {
  constexpr int E = 64 * TE, BT = NW * TT;   // E: experts of this workgroup's slice (of EALL)
  const int e0 = blockIdx.y * E;
  wg += (int64_t)e0 * H;
  constexpr int XB = BF16 ? 2 : 4;                    // bytes per x value
  constexpr int WBUF = E * BC_HC * 4;                 // bytes of a Wg chunk
  constexpr int XBUF = BT * BC_HC * XB;               // bytes of an x chunk
  constexpr int WI = WBUF / 1024 / NW;                // Wg DMA instructions per wavefront and chunk
  constexpr int XI = XBUF / 1024;                     // x DMA instructions per chunk (waves 0 .. XI-1)
  constexpr int XROWS = 1024 / (BC_HC * XB);          // tokens per x DMA instruction
  static_assert(XI >= 1 && XI <= NW && WI >= 1 && WI * NW * 1024 == WBUF, "DMA split");
  static_assert(2 * (WBUF + XBUF) <= 80 * 1024, "LDS: two workgroups per CU");
  __shared__ __attribute__((aligned(1024))) uint8_t ws[2][WBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t xs[2][XBUF];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tb = (int64_t)blockIdx.x * BT;
  const int nchunk = H / BC_HC;

  // DMA sources.  Wg instruction i = wave WI + q holds rows 8i .. 8i + 7: lane L writes LDS word L,
  // row 8i + L / 8, slot L % 8, which holds the row's piece (L % 8) ^ (row % 8) = (L % 8) ^ (L / 8).
  // x instruction wave (waves 0 .. XI-1): tokens XROWS wave .. + XROWS - 1, row-major (clamped to T-1).
  const char* wsrc[WI];
#pragma unroll
  for (int q = 0; q < WI; ++q) {
    const int row = 8 * (wave * WI + q) + (lane >> 3);
    wsrc[q] = reinterpret_cast<const char*>(wg) + ((int64_t)row * H) * 4 + (((lane & 7) ^ (lane >> 3)) << 4);
  }
  const int xper = 64 / XROWS;   // lanes per token row
  const int64_t xrow = min(tb + XROWS * min(wave, XI - 1) + lane / xper, T - 1);
  const char* xsrc = reinterpret_cast<const char*>(xv) + xrow * H * XB + (lane % xper) * 16;
  const uint32_t wdst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&ws[0][wave * WI * 1024]);
  const uint32_t xdst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&xs[0][min(wave, XI - 1) * 1024]);
  const bool x_dma = wave < XI;
  auto issue = [&](int c) {   // chunk c into buffer c & 1
    const int64_t h0 = (int64_t)c * BC_HC;
#pragma unroll
    for (int q = 0; q < WI; ++q) bc_dma16(wsrc[q] + h0 * 4, wdst + (c & 1) * WBUF + q * 1024);
    if (x_dma) bc_dma16(xsrc + h0 * XB, xdst + (c & 1) * XBUF);
  };

  // this lane's swizzled slot of piece q in its rows (row % 8 = lane % 8 for every expert l + 64 j)
  int woff[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) woff[q] = lane * 128 + ((q ^ (lane & 7)) << 4);

  float acc[TT][TE];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TE; ++j) acc[i][j] = 0.0f;

  issue(0);
  for (int c = 0; c < nchunk; ++c) {
    const int b = c & 1;
    // this wave's DMA of chunk c has landed; after the barrier every wave's has, and every wave is
    // done with chunk c - 1, whose buffers take chunk c + 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c + 1 < nchunk) issue(c + 1);
    // this wave's tokens: lane 16 r + k takes columns 2k and 2k + 1
    float xa[TT], xb[TT];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const uint8_t* row = &xs[b][(wave * TT + i) * BC_HC * XB];
      if constexpr (BF16) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(row + (lane & 15) * 4);
        xa[i] = __uint_as_float(u << 16);
        xb[i] = __uint_as_float(u & 0xFFFF0000u);
      } else {
        const float2 p = *reinterpret_cast<const float2*>(row + (lane & 15) * 8);
        xa[i] = p.x;
        xb[i] = p.y;
      }
    }
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < TT; ++i) asm volatile("s_nop 1" : "+v"(xa[i]), "+v"(xb[i]));
    }
    float4 w4[TE];
    bc_read<TT, TE>(w4, &ws[b][0], woff[0]);
    bcast_chunk<0, TT, TE>(acc, xa, xb, &ws[b][0], woff, w4);
  }
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int64_t t = tb + wave * TT + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TE; ++j) {
      const int e = e0 + lane + 64 * j;
      float v = acc[i][j];
      if (bias) v = v + bias[e];
      z[t * EALL + e] = v;
    }
  }
}

template <int TT, int TE, int NW>
int launch_bcast(const void* x, bool bf16, const float* wg, const float* bias, int64_t T, int H, int E, float* z,
                 hipStream_t st) {
  const dim3 grid((unsigned)ceil_div64(T, NW * TT), (unsigned)(E / (64 * TE)));
  if (bf16)
    gate_logits_bcast_kernel<TT, TE, NW, true><<<grid, NW * 64, 0, st>>>(x, wg, bias, T, H, E, z);
  else
    gate_logits_bcast_kernel<TT, TE, NW, false><<<grid, NW * 64, 0, st>>>(x, wg, bias, T, H, E, z);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <int TT, int NW>
int launch_bcast_e(const void* x, bool bf16, const float* wg, const float* bias, int64_t T, int H, int E, float* z,
                   hipStream_t st) {
  // slices of 128 experts where E allows (E = 128 or 256), else one slice of 64
  if (E == 64) return launch_bcast<TT, 1, NW>(x, bf16, wg, bias, T, H, E, z, st);
  return launch_bcast<TT, 2, NW>(x, bf16, wg, bias, T, H, E, z, st);
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
  // Below that, the x-broadcast kernel (4 tokens per wavefront, 4 wavefronts and a ring of two
  // chunks per workgroup, expert slices of 128, so four workgroups share a CU) where its shape rules
  // allow.  Measured at 8192 tokens, H 6144, 256 experts, bf16 x: 420 us against 481 us for the
  // 4 x 4 tiles and 571 us for the 8 x 4 tiles.  The 8 x 4 tiles above stay ahead where they fill
  // the chip (732 us against 799 us at 16384 tokens): their plain fmas issue faster than the
  // DPP-fused ones, and 32 accumulators per thread hide more.
  if (E % 64 == 0 && E <= 256 && H % BC_HC == 0 && T >= 8192)
    return launch_bcast_e<4, 4>(x, bf16, wg, bias, T, H, E, logits, st);
  if (wg44 >= 512) return launch<4, 4>(x, bf16, wg, bias, T, H, E, logits, st);
  if (wg22 >= 512) return launch<2, 2>(x, bf16, wg, bias, T, H, E, logits, st);
  return launch<1, 1>(x, bf16, wg, bias, T, H, E, logits, st);
}
