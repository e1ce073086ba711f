// Grouped block-scaled FP8 GEMM on gfx950 matrix cores.
//
// out[r, n] = sum_kb (as[r,kb] * bs[g, n/128, kb]) * sum_{k in kb} a[r,k] * b[g,n,k]   for rows r of group g.
//
// One K block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4 (e4m3 x e4m3, fp32 result), so
// every MFMA produces a fresh 128-wide partial P that is promoted into the fp32 accumulator with
// its scale product: acc = fma(P, as * bs, acc).  The weight slice is the instruction's first
// operand and the activations its second, so a lane's four results are four consecutive output
// columns of one row: one scale product per lane and tile, and no transpose before the stores.
// (fp32 VALU work does not overlap with the fp8 MFMAs on gfx950, so every VALU instruction in the
// K loop costs MFMA time; the loop keeps only the promotion FMAs and scalar address arithmetic.)
//
// Workgroup tile: BM rows x BN = 256 (virtual) columns, 8 wavefronts.  Row-tile heights:
//   BM = 256: waves in a 2 x 4 grid, each 128 x 64 (8 x 4 MFMA tiles), 2-stage LDS ring (64 KB per
//             stage) - for groups of many hundreds of rows: per flop it moves half the global->LDS
//             bytes of the 128-row tile and reads a quarter fewer LDS bytes, and the per-CU vector
//             memory path, not the matrix cores, is what a narrower tile runs into;
//   BM = 128: waves in a 2 x 4 grid, each 64 x 64 (4 x 4 MFMA tiles of 16 x 16), 3-stage LDS ring
//             (48 KB per stage) - for groups of a few hundred rows;
//   BM = 32, 48, 64: waves in a 1 x 8 grid, each BM x 32 (BM/16 x 2 MFMA tiles), a 4-stage ring
//             for 32 and 48 rows (36 / 38 KB per stage), 3 stages for 64 - for groups of a few
//             dozen rows (decode), where the kernel streams the weights: a 128-row tile would spend
//             most of its DMA and LDS on rows past the group end, and the deeper ring keeps more
//             weight bytes in flight per CU.
//
// Data movement: the A and B K-slices (128 bytes per row) and the tile's activation scales go
// straight from global memory into the LDS ring with global_load_lds (no registers in between),
// issued NSTAGE-1 K steps ahead; each wavefront waits for its own loads with an explicit vmcnt and
// a bare s_barrier publishes the stage (a __syncthreads fence would drain every load in flight).
// Packed weights sit in LDS in the order the MFMA operand reads them: lane l of an operand needs
// row l%16 and K bytes 32(l/16) .. +32, so each 16-row block (2 KB) stores every lane's first 16
// bytes in lane order, then every lane's second 16 bytes; both reads of a fragment are 64
// consecutive 16-byte words, the conflict-free pattern, and each DMA instruction copies 1 KB of
// consecutive packed bytes.  Row-major operands (activations, unpacked weights) are stored as
// swizzled 128-byte rows instead (swz below), which keeps their global reads to whole cache lines.
// Either way the layout is made on the global side: lane L of a DMA instruction writes LDS word L,
// so it fetches the bytes that belong there.  Weights may come pre-packed
// (moe_pack_weights_fp8): each K step of a 256-row panel is then one contiguous 32 KB block holding
// exactly that LDS image, and every DMA instruction reads 1 KB of consecutive bytes instead of
// eight 128-byte row pieces K bytes apart, which keeps HBM streaming near its peak.  The weight
// scales of each step travel by DMA too, through a small LDS ring beside the operand ring.
//
// Tile order: a one-workgroup kernel turns `offsets` into the list of BM-row tiles (never
// straddling a group); a unit is one (tile, 256-column panel) pair, logical units run expert by
// expert, panel-major.  One persistent workgroup per CU takes every G-th unit; each round of G
// units is renumbered XCD-contiguously (hardware ids are dealt to the 8 XCDs round-robin) so that
// neighbouring units, which share A rows or B panels, share an L2.
//
// Epilogue STORE writes out in bf16 or fp32.  Epilogue SWIGLU_QUANT maps the 256 virtual columns
// of a tile to 128 gate columns [f0, f0+128) and the matching 128 up columns [F+f0, F+f0+128); each
// wave holds gate and up of the same h columns in the same lanes, forms h = silu(gate) * up in
// fp32, and the tile's 128 h columns are one 1x128 quantisation block (amax across the waves of a
// row through LDS).
#include <algorithm>
#include <atomic>

#include "common.h"

namespace {

constexpr int BN = 256, BK = 128;
constexpr int NTHREADS = 512;
constexpr int MIN_BM = 32;
constexpr int SPLIT_BM = 128;   // tile height of the third list (short tiles of 256-row plans)

template <int BM_, bool FP4 = false>
struct Tile {
  static constexpr int BM = BM_;
  static constexpr int WM = BM_ >= 128 ? 2 : 1;             // wave grid WM x WN
  static constexpr int WN = 8 / WM;
  static constexpr int MS = BM_ / WM / 16;                   // 16 x 16 MFMA tiles per wave along M
  static constexpr int NS = BN / WN / 16;                    // ... along N
  static constexpr int A_BYTES = BM_ * BK, B_BYTES = FP4 ? BN * BK / 2 : BN * BK;   // FP4: two codes per byte
  // ring within 160 KB of LDS
  static constexpr int NSTAGE = 4 * (A_BYTES + B_BYTES) <= 155 * 1024 ? 4 : 3 * (A_BYTES + B_BYTES) <= 150 * 1024 ? 3 : 2;
  // A fragments read AH 16-row blocks at a time (keeps a 128-row wave within its registers)
  static constexpr int AH = MS > 4 ? MS / 4 : MS;
  static constexpr int A_INSTR = BM_ / 8;                    // 1 KB DMA instructions per A slice
  static constexpr int B_INSTR = B_BYTES / 1024;             // ... per B slice
  // waves that issue the DMA: all 8.  (Leaving waves 0-3 free of DMA issue, so that each SIMD keeps
  // one wave that never stalls on issuing global->LDS copies, measured slower: 5.28 against 5.18 ms
  // for the prefill GEMM1 with 256-row tiles, 5.60 against 5.46 with 128-row tiles.)
  static constexpr int DW = 8;
  static constexpr int A_PW = A_INSTR >= DW ? A_INSTR / DW : 1;   // A instructions per DMA wave
  static constexpr int B_PW = B_INSTR / DW;                        // B instructions per DMA wave
  static constexpr int S_INSTR = BM_ >= 64 ? BM_ / 64 : 1;   // 256-byte scale DMA instructions
  static constexpr int AS_W = BM_ >= 64 ? BM_ : 64;          // floats per scale-ring slot
  static_assert(WM * WN == 8 && MS >= 1 && NS >= 2 && NS % 2 == 0, "tile shape");
  static_assert(A_INSTR % DW == 0 || A_INSTR < DW, "A slice split");
  static_assert(B_INSTR % DW == 0 && B_PW % 2 == 0 && S_INSTR <= DW, "B slice split");
};

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane L's bytes land at lds_addr + 16 L (4 L).
// Issued through inline assembly so that the compiler's conservative wait insertion (it cannot tell
// which LDS stage an in-flight DMA targets) does not drain the pipeline; every wait on these loads
// is explicit.  M0 holds the wave-uniform LDS address and has no other user in these kernels.
// dma16s: wave-uniform 64-bit base in SGPRs (so the per-step K advance is scalar work), 32-bit
// per-lane offset and an immediate offset IMM, which the hardware adds to both the global and the
// LDS address (lane L's bytes land at lds_addr + IMM + 16 L).
template <int IMM>
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3" ::"s"(lds_addr), "v"(voff), "s"(base),
               "i"(IMM) : "memory", "m0");
}
// The weight operand's DMA: with NT the loads carry the non-temporal hint.  Short tiles (decode)
// read each weight panel for about one tile, so the stream should not displace reusable lines;
// measured on the decode layer: GEMM1 138 -> 128 us, GEMM2 82 -> 78 us.  Taller tiles reuse a panel
// across a group's tiles through the L2, where the hint measured 1-4% slower.
template <int IMM, bool NT>
__device__ __forceinline__ void dma16s_w(const void* base, uint32_t voff, uint32_t lds_addr) {
  if (NT)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3 nt" ::"s"(lds_addr), "v"(voff),
                 "s"(base), "i"(IMM) : "memory", "m0");
  else
    dma16s<IMM>(base, voff, lds_addr);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// DMA instruction i (1 KB of a stage) and lane L: the row of the K slice and the 16-byte chunk of
// its 128 bytes that land at LDS word 64 i + L (16-row block i/2, operand half i%2)
__device__ __forceinline__ int dma_row(int i, int L) { return 16 * (i >> 1) + (L & 15); }
__device__ __forceinline__ int dma_chunk(int i, int L) { return ((L >> 4) << 1) | (i & 1); }
// Row-major operands (activations; weights that are not packed) keep whole 128-byte rows per DMA
// instruction, which keeps the global reads to one full cache line per 8 lanes: instruction i holds
// rows 8i .. 8i+7, lane L row 8i + L/8, its 16-byte chunk L%8 stored at slot (L%8) ^ f(row) with
// f(row) = (row & 7) ^ ((row >> 3) & 1).  Of the XOR swizzles measured on gfx950 for the operand
// read pattern this one is the fastest (175 B/clk/CU against 180 for linear reads; (row & 7) or
// ((row >> 1) & 7) alone reach 123).
__device__ __forceinline__ int swz_mask(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ swz_mask(row)) << 4); }

typedef uint32_t uint32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t uint32x4 __attribute__((ext_vector_type(4)));

// Weight row held by virtual row r (0..255) of panel nt: SwiGLU panels pair gate rows
// [128 nt, 128 nt + 128) with up rows [F + 128 nt, ...); STORE panels are rows [256 nt, 256 nt + 256).
__device__ __forceinline__ int panel_row(int epi, int nt, int r, int F) {
  return epi == 1 ? (r < 128 ? nt * 128 + r : F + nt * 128 + (r - 128)) : nt * BN + r;
}

// ------------------------------------------------------------------------------------------------
// Packed weights: packed[g][nt][kb] is the 32 KB LDS image of K step kb of panel nt: 16-byte unit
// u = 64 i + L (DMA instruction i, lane L) holds chunk dma_chunk(i, L) of virtual row dma_row(i, L).
// One thread per 16-byte unit; rows past N (STORE panels) are zero.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ b, int N, int K, int ny, int epi,
                                                           int64_t units, uint8_t* __restrict__ packed) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int KB = K / BK;
  const int w = (int)(u & 2047);                // unit within the 32 KB block
  const int64_t blk = u >> 11;                  // (g, nt, kb) block index
  const int kb = (int)(blk % KB);
  const int64_t gnt = blk / KB;
  const int nt = (int)(gnt % ny);
  const int64_t g = gnt / ny;
  const int r = dma_row(w >> 6, w & 63);
  const int chunk = dma_chunk(w >> 6, w & 63);
  const int n = panel_row(epi, nt, r, N / 2);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n < N) v = *reinterpret_cast<const uint4*>(b + ((size_t)g * N + n) * K + (size_t)kb * BK + chunk * 16);
  *reinterpret_cast<uint4*>(packed + (size_t)u * 16) = v;
}

// ------------------------------------------------------------------------------------------------
// tiles[i] = {group, first row, index of the group's first tile, number of tiles of the group}.
// A block scan gives each group's first tile; then every thread writes tiles (each finds its group
// by binary search over the first tiles), so a long group's tiles are not written by one thread.
constexpr int TILE_MAP_MAXG = 4096;
// exclusive prefix over the groups of cnt(g) into dst[0 .. groups] (dst[groups] = total), in
// chunks of 1024 groups; every thread of the workgroup calls it
template <typename F>
__device__ __forceinline__ void group_prefix(int groups, F cnt, int* dst, int* part, int* carry) {
  if (threadIdx.x == 0) *carry = 0;
  __syncthreads();
  for (int g0 = 0; g0 < groups; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    const int n = g < groups ? cnt(g) : 0;
    part[threadIdx.x] = n;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
      const int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    if (g < groups) dst[g] = *carry + part[threadIdx.x] - n;
    __syncthreads();
    if (threadIdx.x == 1023) *carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) dst[groups] = *carry;
  __syncthreads();
}

// the group owning list position t: the last group whose first position is at or before t (a
// group with no positions shares its first position with the next, so the last one owns t)
__device__ __forceinline__ int owner(const int* first, int groups, int t) {
  int lo = 0, hi = groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// The tile list: group g's ceil(rows_g / bm) tiles, groups in order; entry {group, first row, first
// tile of the unit-order block, tiles in the block}, the block being the group's tiles; its length
// goes to ntiles[0].  With second != 0 a second list at tiles + second holds the same tiles with
// every group's full tiles first (block: the group's full tiles) and then each group's short last
// tile (a block of its own); its length goes to ntiles[1].  With third != 0 as well (256-row
// plans), the second list keeps only the short tiles of more than SPLIT_BM rows, and a third list
// at tiles + third holds one SPLIT_BM-row tile for each group whose short remainder has 1 ..
// SPLIT_BM rows; its length goes to ntiles[2].  run_planned picks the lists.
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t* __restrict__ offsets, int groups, int bm,
                                                        int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                        int max_tiles, int second, int third) {
  __shared__ int part[1024];
  __shared__ int first[TILE_MAP_MAXG + 1];   // first[g] = tiles before group g; first[groups] = all
  __shared__ int carry;
  group_prefix(groups, [&](int g) { return (offsets[g + 1] - offsets[g] + bm - 1) / bm; }, first, part, &carry);
  const int total = min(first[groups], max_tiles);
  for (int t = threadIdx.x; t < total; t += 1024) {
    const int lo = owner(first, groups, t);
    const int i = t - first[lo];
    tiles[t] = make_int4(lo, offsets[lo] + i * bm, first[lo], first[lo + 1] - first[lo]);
  }
  if (threadIdx.x == 0) *ntiles = total;
  if (!second) return;
  __syncthreads();
  // full tiles: first[] becomes the full-tile prefix; short tiles follow all of them
  group_prefix(groups, [&](int g) { return (offsets[g + 1] - offsets[g]) / bm; }, first, part, &carry);
  const int nfull = first[groups];
  for (int t = threadIdx.x; t < min(nfull, total); t += 1024) {
    const int lo = owner(first, groups, t);
    const int i = t - first[lo];
    tiles[second + t] = make_int4(lo, offsets[lo] + i * bm, first[lo], first[lo + 1] - first[lo]);
  }
  __syncthreads();
  auto short_rows = [&](int g) { return (offsets[g + 1] - offsets[g]) % bm; };
  group_prefix(groups, [&](int g) { return short_rows(g) > (third ? SPLIT_BM : 0) ? 1 : 0; }, first, part, &carry);
  const int n2 = min(nfull + first[groups], total);
  for (int t = nfull + threadIdx.x; t < n2; t += 1024) {
    const int lo = owner(first, groups, t - nfull);
    const int nf = (offsets[lo + 1] - offsets[lo]) / bm;
    tiles[second + t] = make_int4(lo, offsets[lo] + nf * bm, t, 1);
  }
  if (threadIdx.x == 0) ntiles[1] = n2;
  if (!third) return;
  __syncthreads();
  group_prefix(groups, [&](int g) { return short_rows(g) > 0 && short_rows(g) <= SPLIT_BM ? 1 : 0; }, first, part,
               &carry);
  const int n3 = first[groups];   // at most groups: the host reserves that many entries
  for (int t = threadIdx.x; t < n3; t += 1024) {
    const int lo = owner(first, groups, t);
    const int nf = (offsets[lo + 1] - offsets[lo]) / bm;
    tiles[third + t] = make_int4(lo, offsets[lo] + nf * bm, t, 1);
  }
  if (threadIdx.x == 0) ntiles[2] = n3;
}

// wait until M * v of this wave's vector memory instructions are outstanding, v one of LO .. HI:
// a short chain of compares for the few counts a loop meets in its steady state
template <int M, int LO, int HI>
__device__ __forceinline__ void wait_vm_steady(int v) {
  if constexpr (M == 0 || LO >= HI) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(M * LO < 63 ? M * LO : 63) : "memory");
  } else {
    if (v == LO) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(M * LO < 63 ? M * LO : 63) : "memory");
      return;
    }
    wait_vm_steady<M, LO + 1, HI>(v);
  }
}

// wait until at most n of this wave's vector memory instructions are outstanding (n is
// wave-uniform; s_waitcnt takes an immediate)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define WAIT_CASE(N) \
  case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
#define WAIT_CASE8(B) WAIT_CASE(B) WAIT_CASE(B + 1) WAIT_CASE(B + 2) WAIT_CASE(B + 3) WAIT_CASE(B + 4) \
  WAIT_CASE(B + 5) WAIT_CASE(B + 6) WAIT_CASE(B + 7)
    WAIT_CASE(1) WAIT_CASE(2) WAIT_CASE(3) WAIT_CASE(4) WAIT_CASE(5) WAIT_CASE(6) WAIT_CASE(7)
    WAIT_CASE8(8) WAIT_CASE8(16) WAIT_CASE8(24) WAIT_CASE8(32) WAIT_CASE8(40) WAIT_CASE8(48) WAIT_CASE8(56)
#undef WAIT_CASE8
#undef WAIT_CASE
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// ------------------------------------------------------------------------------------------------
// Where unit u (a tile-row block x panel pair, in logical order) sits: group, rows, panel.  A group's
// w tiles x ny panels run in blocks of PB panels: every tile of the group on panels 0 .. PB-1, then
// on panels PB .. 2PB-1, and so on (the last block takes the remaining ny % PB panels).  Consecutive
// units, which run at the same time on one XCD, then share a few weight panels and a few activation
// tiles, so a large group's activation rows are fetched once per PB panels rather than once per
// panel (panel-major order) and each panel once per XCD's worth of tiles.
constexpr int PB = 4;
struct Unit {
  int g, row0, row_end, nt;
};
__device__ __forceinline__ Unit unit_at(int u, int ny, const int4* __restrict__ tiles, const int32_t* __restrict__ offsets,
                                        int bm) {
  const int q = u / ny;
  const int4 tq = tiles[q];
  const int local = u - tq.z * ny;   // unit within the group: [0, w * ny)
  const int w = tq.w;
  const int nfull = ny / PB;         // full panel blocks
  const int pb = local / (w * PB);
  int tile, nt;
  if (pb < nfull) {
    const int rem = local - pb * w * PB;
    tile = rem / PB;
    nt = pb * PB + (rem - tile * PB);
  } else {
    const int r = ny - nfull * PB;   // panels in the last block (>= 1 here)
    const int rem = local - nfull * w * PB;
    tile = rem / r;
    nt = nfull * PB + (rem - tile * r);
  }
  Unit res;
  res.nt = nt;
  res.g = tq.x;
  res.row0 = tq.y + (tile - (q - tq.z)) * bm;   // tq.y: tile q's own first row
  res.row_end = min(res.row0 + bm, offsets[res.g + 1]);
  return res;
}

// Persistent workgroups: workgroup w takes units me(w), me(w) + G, me(w) + 2G, ... (G = grid size),
// and its K steps over all of them form one stream: the DMA lookahead runs into the next unit while
// the current unit's last steps and epilogue execute, so no unit pays the pipeline fill again.
template <int BM, int EPI, bool OUT_BF16, bool PACKED, bool POW2, bool FP4 = false, bool WNT = false>
__global__ __launch_bounds__(NTHREADS) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a, const int32_t* __restrict__ a_rows, int a_count, const float* __restrict__ as,
    const int32_t* __restrict__ offsets,
    const int4* __restrict__ tiles, const int32_t* __restrict__ ntiles, int ny, const uint8_t* __restrict__ b,
    const float* __restrict__ bs, int N, int K, void* __restrict__ out, float* __restrict__ out_scales,
    float* __restrict__ g_out) {
  static_assert(!FP4 || (PACKED && POW2), "FP4 weights come packed, with power-of-two activation scales");
  using T = Tile<BM, FP4>;
  constexpr int WM = T::WM, WN = T::WN, MS = T::MS, NS = T::NS, HS = NS / 2, NSTAGE = T::NSTAGE;
  constexpr int B_PW = T::B_PW;      // B DMA instructions per DMA wave and step
  constexpr int BQ = PACKED ? (B_PW + 3) / 4 : B_PW;   // B offsets kept per DMA wave
  constexpr int A_BYTES = T::A_BYTES, B_BYTES = T::B_BYTES, AS_W = T::AS_W;
  constexpr int WROWS = MS * 16;   // rows per wave
  constexpr int D = NSTAGE - 1;    // DMA lookahead in K steps
  // non-temporal weight loads for the short (weight-streaming) tiles, and for every tile of a launch
  // whose weight panels are each read by one tile (WNT: the short remainders of a 256-row plan)
  constexpr bool W_NT = BM <= 64 || WNT;
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds[NSTAGE][A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b_lds[NSTAGE][B_BYTES];
  __shared__ __attribute__((aligned(16))) float as_lds[4][AS_W];   // activation-scale ring: slot (step & 3)
  __shared__ __attribute__((aligned(16))) float bsc_lds[4][64];    // weight-scale ring: [0] low, [1] high block
  // FP4 weights: E8M0 scale codes of each step, [panel row][32-wide K chunk] (ring slot step & 3)
  __shared__ __attribute__((aligned(16))) uint8_t bsc4_lds[4][FP4 ? 1024 : 16];
  __shared__ float red[WM][WN][WROWS];

  // ---- this workgroup's units: each round of G consecutive logical units is split into
  // XCD-contiguous equal shares (hardware ids are dealt to the 8 XCDs round-robin)
  const int real = *ntiles * ny;
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  // each round's units XCD-contiguous: neighbouring units share A rows or B panels (a group's
  // tiles of one panel are adjacent), and so share an L2
  const int me = xcd * (G >> 3) + min(xcd, G & 7) + slot;
  if (me >= real) return;
  const int nunits = (real - me + G - 1) / G;
  const int KB = K / BK;
  const int total = nunits * KB;   // K steps of this workgroup
  const int F = N / 2;             // SwiGLU only
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const size_t gstride = (PACKED ? (size_t)ny * BN : (size_t)N) * K / (FP4 ? 2 : 1);   // bytes of one group's weights

  // ---- DMA roles.  DMA wave d (wave 8 - DW + d) issues A instructions d*A_PW + j (or just d, for
  // slices of fewer than DW instructions) and B instructions d*B_PW + j.  Row-major operands:
  // instruction i holds rows 8i .. 8i+7, lane L row 8i + L/8 and chunk L%8 (stored at its swizzled
  // slot); packed weights: lane L's 16 bytes sit at 1024 i + 16 L of the K step's block.
  const bool dma_wave = wave >= 8 - T::DW;
  const int dw = max(wave - (8 - T::DW), 0);
  const bool has_a = dma_wave && (T::A_INSTR >= T::DW || dw < T::A_INSTR);
  const int a_i0 = T::A_INSTR >= T::DW ? dw * T::A_PW : dw;
  const bool scale_loader = wave >= 8 - T::S_INSTR;   // the last S_INSTR waves bring 64 rows' scales each
  const int sidx = max(wave - (8 - T::S_INSTR), 0);
  // the first DMA wave also brings the step's two weight scales (lane 0: low 128-column block, lane 1: high)
  const bool bscale_loader = wave == 8 - T::DW;
  const int per_stage =
      dma_wave ? (has_a ? T::A_PW : 0) + B_PW + (scale_loader ? 1 : 0) + (bscale_loader ? 1 : 0) : 0;
  // the outstanding count of a steady-state step, per_stage * (D - 1), and the range of per_stage
  // over the waves (every wave issues DMA; A only when the slice has an instruction for it; one
  // scale load each for some waves)
  const int steady = per_stage * (D - 1);
  constexpr int PS_LO = (T::A_INSTR >= T::DW ? T::A_PW : 0) + B_PW, PS_HI = T::A_PW + B_PW + 2;
  static_assert(T::DW == 8, "every wave issues DMA");

  // issue-side context of the unit whose steps are being issued: 32-bit byte offsets from a and
  // from the unit's group weights (both < 2^32 for every accepted shape); rows past the tile's end
  // read the tile's last row (any valid row would do)
  uint32_t aoff[T::A_PW], boff[BQ];
  const uint8_t* bg = b;
  const float* ssrc = as;
  const float* bsrc = bs;   // this lane's weight-scale row (low block for lane != 1)
  const uint8_t* bsrc4 = reinterpret_cast<const uint8_t*>(bs);   // FP4: the unit's panel scale images
  int ii = 0, ik = 0;   // unit index and K step of the next step to issue
#define GEMM_ISSUE_CTX(I)                                                                           \
  do {                                                                                              \
    const Unit un_ = unit_at(me + (I) * G, ny, tiles, offsets, BM);                                 \
    _Pragma("unroll") for (int j_ = 0; j_ < T::A_PW; ++j_) {                                        \
      const int r_ = (a_i0 + j_) * 8 + (lane >> 3);                                                \
      int src_ = min(un_.row0 + r_, un_.row_end - 1);                                               \
      if (a_rows) {                                                                                 \
        /* gathered rows: the 8 rows of instruction j_ are wave-uniform, so their row ids come */  \
        /* through the scalar cache (a vector load here would make the compiler drain the DMA */   \
        /* in flight before using it); each lane then selects its own, clamped to a's rows */      \
        int g8_[8];                                                                                 \
        _Pragma("unroll") for (int q_ = 0; q_ < 8; ++q_)                                            \
          g8_[q_] = a_rows[min(un_.row0 + (a_i0 + j_) * 8 + q_, un_.row_end - 1)];                  \
        int t_ = g8_[0];                                                                            \
        _Pragma("unroll") for (int q_ = 1; q_ < 8; ++q_) t_ = (lane >> 3) == q_ ? g8_[q_] : t_;     \
        src_ = min(max(t_, 0), a_count - 1);                                                        \
      }                                                                                             \
      aoff[j_] = (uint32_t)src_ * (uint32_t)K + (((lane & 7) ^ swz_mask(r_)) << 4);                 \
    }                                                                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < BQ; ++i_) {                                             \
      if (PACKED) {                                                                                 \
        /* one base per 4 instructions (the immediate offset reaches 4095) */                      \
        boff[i_] = (uint32_t)un_.nt * (uint32_t)(BN * K / (FP4 ? 2 : 1)) +                           \
                   (uint32_t)((B_PW * dw + 4 * i_) * 1024 + lane * 16);                             \
      } else {                                                                                      \
        const int r_ = (B_PW * dw + i_) * 8 + (lane >> 3);                                          \
        const int n_ = min(panel_row(EPI, un_.nt, r_, F), N - 1);                                   \
        boff[i_] = (uint32_t)n_ * (uint32_t)K + (((lane & 7) ^ swz_mask(r_)) << 4);                 \
      }                                                                                             \
    }                                                                                               \
    bg = b + (size_t)un_.g * gstride;                                                               \
    ssrc = as + (size_t)min(un_.row0 + sidx * 64 + lane, un_.row_end - 1) * KB;                     \
    const int nlo_ = EPI == 1 ? un_.nt : min(un_.nt * BN, N - 1) / 128;                             \
    const int nhi_ = EPI == 1 ? (F / 128) + un_.nt : min(un_.nt * BN + 128, N - 1) / 128;           \
    bsrc = bs + ((size_t)un_.g * (N / 128) + (lane == 1 ? nhi_ : nlo_)) * KB;                       \
    bsrc4 = reinterpret_cast<const uint8_t*>(bs) + ((size_t)un_.g * ny + un_.nt) * (size_t)KB * 1024; \
  } while (0)

  // wave-uniform LDS destinations of this wave's DMA instructions, stage 0; stage s adds s * stride
  const uint32_t a_dst = lds_u32(&a_lds[0][a_i0 * 1024]);
  const uint32_t b_dst = lds_u32(&b_lds[0][(B_PW * dw) * 1024]);
  const uint32_t bsc4_dst = lds_u32(&bsc4_lds[0][0]);
  const uint32_t s_dst = lds_u32(&as_lds[0][sidx * 64]);
  const uint32_t bsc_dst = lds_u32(&bsc_lds[0][0]);
  // issue K step ik of unit ii (global step SV) into LDS stage ST, then advance (ii, ik)
#define GEMM_ISSUE(SV, ST)                                                                \
  do {                                                                                    \
    const uint32_t ko_ = (uint32_t)ik * BK;                                               \
    const uint32_t kob_ = PACKED ? (uint32_t)ik * B_BYTES : ko_;                          \
    if (has_a) {                                                                          \
      const uint32_t ao_ = a_dst + (uint32_t)(ST) * A_BYTES;                              \
      _Pragma("unroll") for (int j_ = 0; j_ < T::A_PW; ++j_)                               \
        dma16s<0>(a + ko_, aoff[j_], ao_ + 1024 * j_);                                    \
    }                                                                                     \
    const uint32_t bo_ = b_dst + (uint32_t)(ST) * B_BYTES;                                \
    if (dma_wave) {                                                                       \
      if (PACKED) {                                                                       \
        _Pragma("unroll") for (int q_ = 0; q_ < BQ; ++q_) {                                \
          dma16s_w<0, W_NT>(bg + kob_, boff[q_], bo_ + 4096 * q_);                        \
          dma16s_w<1024, W_NT>(bg + kob_, boff[q_], bo_ + 4096 * q_);                     \
          if (B_PW - 4 * q_ > 2) {                                                        \
            dma16s_w<2048, W_NT>(bg + kob_, boff[q_], bo_ + 4096 * q_);                   \
            dma16s_w<3072, W_NT>(bg + kob_, boff[q_], bo_ + 4096 * q_);                   \
          }                                                                               \
        }                                                                                 \
      } else {                                                                            \
        _Pragma("unroll") for (int q_ = 0; q_ < B_PW; ++q_)                                \
          dma16s_w<0, W_NT>(bg + kob_, boff[q_], bo_ + 1024 * q_);                        \
      }                                                                                   \
    }                                                                                     \
    if (scale_loader) dma4(ssrc + ik, s_dst + (uint32_t)((SV) & 3) * AS_W * 4);           \
    if (FP4) {                                                                            \
      if (bscale_loader)                                                                  \
        dma16s<0>(bsrc4 + (size_t)ik * 1024, (uint32_t)(lane * 16),                       \
                  bsc4_dst + (uint32_t)((SV) & 3) * 1024);                                \
    } else if (bscale_loader) {                                                           \
      dma4(bsrc + ik, bsc_dst + (uint32_t)((SV) & 3) * 256);                              \
    }                                                                                     \
    if (++ik == KB) {                                                                     \
      ik = 0;                                                                             \
      if (++ii < nunits) GEMM_ISSUE_CTX(ii);                                              \
    }                                                                                     \
  } while (0)

  // ---- compute-side context of the unit being accumulated
  int ci = 0, ck = 0;   // unit index and K step being computed
  Unit cu = unit_at(me, ny, tiles, offsets, BM);
  int b_lrow[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    if (EPI == 1) b_lrow[ns] = ns < HS ? wn * HS * 16 + ns * 16 : 128 + wn * HS * 16 + (ns - HS) * 16;
    else b_lrow[ns] = wn * NS * 16 + ns * 16;
  }

  floatx4 acc[MS][NS];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15;         // row within a 16-row operand tile
  // operand fragments of one K step, read from LDS stage ST: the 16-row block starting at row R
  // is 2 KB at 128 R; lane l's 32 bytes are words l and 64 + l of it.  With FP8 on both sides the
  // K order inside a lane is immaterial as long as both operands share it, so lane group c takes
  // the 16-byte chunks 2c, 2c + 1.  An FP4 operand holds K 32c .. 32c + 31 in lane group c while an
  // FP8 operand holds K 16c .. 16c + 15 in its low and 64 + 16c .. 64 + 16c + 15 in its high 16
  // bytes, so against FP4 weights the activation fragment takes chunks c and 4 + c.
  intx8 af[T::AH], bf[NS];
  const int a_c0 = FP4 ? (lane >> 4) : (lane >> 4) * 2, a_c1 = FP4 ? 4 + (lane >> 4) : (lane >> 4) * 2 + 1;
  // A fragments of 16-row blocks MS0 .. MS0 + AH - 1 (of this wave's rows) from LDS stage ST
#define GEMM_READ_A_INTO(DST, ST, MS0)                                                                  \
  do {                                                                                                  \
    _Pragma("unroll") for (int ms = 0; ms < T::AH; ++ms) {                                              \
      const int r_ = wm * WROWS + ((MS0) + ms) * 16 + lr;                                               \
      const intx4 lo_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, a_c0)]);                     \
      const intx4 hi_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, a_c1)]);                     \
      DST[ms] = intx8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};                  \
    }                                                                                                   \
  } while (0)
#define GEMM_READ_A(ST, MS0) GEMM_READ_A_INTO(af, ST, MS0)
#define GEMM_READ_A1(DST, ST, M_)                                                                       \
  do {                                                                                                  \
    const int r_ = wm * WROWS + (M_) * 16 + lr;                                                         \
    const intx4 lo_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, a_c0)]);                       \
    const intx4 hi_ = *reinterpret_cast<const intx4*>(&a_lds[ST][swz(r_, a_c1)]);                       \
    DST = intx8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};                        \
  } while (0)
#define GEMM_READ_B(ST)                                                                                 \
  do {                                                                                                  \
    _Pragma("unroll") for (int ns = 0; ns < NS; ++ns) {                                                 \
      /* packed weights: operand order; row-major weights: swizzled rows; FP4: one 1 KB */              \
      /* block per 16 rows, lane l's 16 bytes at 16 l */                                                \
      const int r_ = b_lrow[ns] + lr;                                                                   \
      if (FP4) {                                                                                        \
        const intx4 q_ = *reinterpret_cast<const intx4*>(&b_lds[ST][b_lrow[ns] * 64 + lane * 16]);      \
        bf[ns] = intx8{q_[0], q_[1], q_[2], q_[3], 0, 0, 0, 0};                                         \
        continue;                                                                                       \
      }                                                                                                 \
      const int o_ = PACKED ? b_lrow[ns] * BK + lane * 16 : swz(r_, (lane >> 4) * 2);                   \
      const int o2_ = PACKED ? o_ + 1024 : swz(r_, (lane >> 4) * 2 + 1);                                \
      const intx4 lo_ = *reinterpret_cast<const intx4*>(&b_lds[ST][o_]);                                \
      const intx4 hi_ = *reinterpret_cast<const intx4*>(&b_lds[ST][o2_]);                               \
      bf[ns] = intx8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};                   \
    }                                                                                                   \
  } while (0)

  // ---- prologue: steps 0 .. D-1 in flight
  GEMM_ISSUE_CTX(0);
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < total) GEMM_ISSUE(s, s);

  int st = 0;         // LDS stage of step s
  int recent[D];       // epilogue store instructions issued at the end of steps s-D .. s-1
#pragma unroll
  for (int j = 0; j < D; ++j) recent[j] = 0;
  for (int s = 0; s < total; ++s) {
    // Wait for this wave's DMA of step s.  vmcnt retires vector memory instructions in issue
    // order, so the ones allowed to stay outstanding are exactly those issued after step s's
    // DMA: the DMA of steps s+1 .. s+D-1 and the epilogue stores of the last D steps (each
    // epilogue issues a fixed, wave-uniform number of stores; no store is skipped by a branch).
    int later = per_stage * min(D - 1, total - 1 - s);
#pragma unroll
    for (int j = 0; j < D; ++j) later += recent[j];
    // the steady state (no epilogue stores in flight, not the last steps) meets one count per
    // wave, per_stage * (D - 1): a short path for it; the 64-way switch compiles to a tree of
    // compares and branches that every step would otherwise walk
    if (later == steady && steady <= 63) wait_vm_steady<D - 1, PS_LO, PS_HI>(per_stage);
    else wait_vm(min(later, 63));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + D < total) {
      const int ist = st == 0 ? NSTAGE - 1 : st - 1;   // (s + D) % NSTAGE: the stage read last step
      GEMM_ISSUE(s + D, ist);
    }
    // a wave whose rows all lie past the unit's last row (a group's short last tile) or whose
    // columns lie past N does no fragment reads and no MFMAs
    const bool wave_active =
        (EPI == 1 ? true : (cu.nt * BN + wn * NS * 16 < N)) && wm * WROWS < cu.row_end - cu.row0;
    if (wave_active) {
      GEMM_READ_B(st);
      const float* srow = &as_lds[s & 3][wm * WROWS + lr];
      // weight scales of this step: SwiGLU gate columns use the low block and up columns the high
      // one; a STORE wave's 16*NS columns lie in block (wn * NS * 16) / 128 of the panel
      const float sb_lo = bsc_lds[s & 3][EPI == 1 ? 0 : (wn * NS * 16) / 128];
      const float sb_hi = bsc_lds[s & 3][1];
      // FP4 weights: each lane's operand row has its own scale per 32-wide K chunk (lane / 16)
      uint32_t eb4[NS];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
        eb4[ns] = FP4 ? (uint32_t)bsc4_lds[s & 3][(b_lrow[ns] + lr) * 4 + (lane >> 4)] : 0u;
      // one 16-row block of MFMAs with A fragment AF: pow2 accumulates in place; amax takes fresh
      // partials of the block and promotes them with the block's scale products
#define GEMM_ROW(M_, AF)                                                                                   \
  do {                                                                                                     \
    if (POW2) {                                                                                            \
      const uint32_t eb_lo_ = e8m0_code(sb_lo), eb_hi_ = e8m0_code(sb_hi);                                 \
      const uint32_t ea_ = e8m0_code(srow[(M_) * 16]);                                                     \
      _Pragma("unroll") for (int ns = 0; ns < NS; ++ns)                                                    \
        acc[M_][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(                                   \
            bf[ns], AF, acc[M_][ns], FP4 ? 4 : 0, 0, 0, FP4 ? eb4[ns] : ((EPI == 1 && ns >= HS) ? eb_hi_ : eb_lo_), \
            0, ea_);                                                                                       \
    } else {                                                                                               \
      floatx4 p_[NS];                                                                                      \
      _Pragma("unroll") for (int ns = 0; ns < NS; ++ns)                                                    \
        p_[ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ns], AF, floatx4{0.f, 0.f, 0.f, 0.f}, \
                                                                  0, 0, 0, 0, 0, 0);                       \
      const float sa_ = srow[(M_) * 16];                                                                   \
      const float c_lo_ = sa_ * sb_lo, c_hi_ = EPI == 1 ? sa_ * sb_hi : c_lo_;                             \
      _Pragma("unroll") for (int ns = 0; ns < NS; ++ns) {                                                  \
        const bool hi_ = EPI == 1 && ns >= HS;                                                             \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                      \
          acc[M_][ns][i] = __builtin_fmaf(p_[ns][i], hi_ ? c_hi_ : c_lo_, acc[M_][ns][i]);                 \
      }                                                                                                    \
    }                                                                                                      \
  } while (0)
      if constexpr (T::AH == MS && (POW2 || EPI == 1)) {
        GEMM_READ_A(st, 0);
        if (POW2) {
          // power-of-two scales: the matrix cores apply them (E8M0 exponents; each lane gives the
          // scale of its operand row for its 32-wide K piece, here the same for the whole 128-wide
          // step) and accumulate straight into acc - no promotion
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) GEMM_ROW(ms, af[ms]);
        } else {
          // every fresh partial of the step first, then the promotion
          floatx4 p[MS][NS];
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns)
              p[ms][ns] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ns], af[ms],
                                                                           floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0,
                                                                           0, 0);
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) {
            const float sa = srow[ms * 16];
            const float c_lo = sa * sb_lo, c_hi = EPI == 1 ? sa * sb_hi : c_lo;
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
              const bool hi = EPI == 1 && ns >= HS;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[ms][ns][i] = __builtin_fmaf(p[ms][ns][i], hi ? c_hi : c_lo, acc[ms][ns][i]);
            }
          }
        }
      } else if constexpr (POW2) {
        // tall wave tile, power-of-two scales: the rows in groups of AH 16-row blocks (a
        // read-ahead ring as below measured no faster here: the MFMAs accumulate in place and the
        // two waves of a SIMD already overlap one's reads with the other's MFMAs)
#pragma unroll
        for (int h = 0; h < MS / T::AH; ++h) {
          GEMM_READ_A(st, h * T::AH);
#pragma unroll
          for (int ms = 0; ms < T::AH; ++ms) GEMM_ROW(h * T::AH + ms, af[ms]);
        }
      } else {
        // amax scales, tall wave tiles and the plain (no SwiGLU) epilogue: A fragments one 16-row
        // block at a time through a ring of two register sets, block m + 1 read before the MFMAs
        // and promotion of block m, so a read's LDS latency hides behind the work on the block
        // before it.  Measured on the prefill GEMMs: 4% faster than reading groups of blocks into
        // one set for 256-row tiles, 2% for the plain epilogue at 128 rows, 2% slower for the
        // SwiGLU epilogue at 128 rows (which therefore keeps the branch above).
        intx8 ar[2];
        GEMM_READ_A1(ar[0], st, 0);
#pragma unroll
        for (int m = 0; m < MS; ++m) {
          if (m + 1 < MS) GEMM_READ_A1(ar[(m + 1) % 2], st, m + 1);
          GEMM_ROW(m, ar[m % 2]);
        }
      }
#undef GEMM_ROW
    }
    st = st + 1 == NSTAGE ? 0 : st + 1;
#pragma unroll
    for (int j = 0; j + 1 < D; ++j) recent[j] = recent[j + 1];
    recent[D - 1] = 0;

    if (++ck < KB) continue;
    // ---- epilogue of unit ci, then move on.  Lane l holds row l%16 and columns 4(l/16) .. +3 of
    // each 16 x 16 result tile.  Stores go through a buffer resource bounded by the unit's valid
    // rows, so rows past the group end are dropped by the hardware instead of by a branch, and
    // every wave issues a fixed number of stores.
    const int row0 = cu.row0, nrows = cu.row_end - cu.row0;
    const int tr = lr;                 // this lane's row within a 16-row tile
    const int tc = (lane >> 4) * 4;    // first of the lane's 4 consecutive columns
    if (EPI == 0) {
      if (wave_active) {
        constexpr int EB = OUT_BF16 ? 2 : 4;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<uint8_t*>(out) + (size_t)row0 * N * EB, 0, nrows * N * EB, 0x00020000);
        if (OUT_BF16) {
          // bf16: the tiles ns = 2p and 2p + 1 of a row block go out together.  A lane's packed
          // pairs (4 columns of one row each) pass through v_permlane16_swap, which exchanges lane
          // rows 1 and 3 of the first operand with lane rows 0 and 2 of the second; afterwards lane
          // rows 0 and 2 hold columns 0-7 and 8-15 of tile 2p, rows 1 and 3 those of tile 2p + 1,
          // 16 bytes per lane.  One 16-byte store per lane and tile pair then writes 64 contiguous
          // bytes per output row, against two 8-byte stores of 32 bytes per row: measured on the
          // long-context stream's store GEMM 21.9 -> 20.4 ms per 16-chunk step, prefill 2.71 ->
          // 2.49 ms (non-temporal stores, 8 or 16 bytes, were slower).
          const int g = lane >> 4;
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int p = 0; p < NS / 2; ++p) {
              const uint32_t a0 = pack_bf16x2(acc[ms][2 * p][0], acc[ms][2 * p][1]);
              const uint32_t a1 = pack_bf16x2(acc[ms][2 * p][2], acc[ms][2 * p][3]);
              const uint32_t b0 = pack_bf16x2(acc[ms][2 * p + 1][0], acc[ms][2 * p + 1][1]);
              const uint32_t b1 = pack_bf16x2(acc[ms][2 * p + 1][2], acc[ms][2 * p + 1][3]);
              const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
              const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
              uint32x4 w;
              w[0] = s0[0];
              w[1] = s1[0];
              w[2] = s0[1];
              w[3] = s1[1];
              const int col = cu.nt * BN + wn * NS * 16 + (2 * p + (g & 1)) * 16 + 8 * (g >> 1);
              __builtin_amdgcn_raw_buffer_store_b128(w, rs, ((wm * WROWS + ms * 16 + tr) * N + col) * EB, 0, 0);
            }
          recent[D - 1] = MS * NS / 2;
        } else {
          const int c0 = cu.nt * BN + wn * NS * 16 + tc;
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
              uint32x4 w;
#pragma unroll
              for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(acc[ms][ns][i]);
              __builtin_amdgcn_raw_buffer_store_b128(w, rs, ((wm * WROWS + ms * 16 + tr) * N + c0 + ns * 16) * EB, 0,
                                                     0);
            }
          recent[D - 1] = MS * NS;
        }
      }
    } else {
      // training forward: also store the fp32 GEMM output G = [gate | up] ([rows, N], N = 2F), which
      // the backward's SwiGLU derivative needs (uniform branch; rows past the group are dropped)
      if (g_out) {
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            g_out + (size_t)row0 * N, 0, nrows * N * 4, 0x00020000);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            const int col = (ns < HS ? 0 : F) + cu.nt * 128 + wn * HS * 16 + (ns % HS) * 16 + tc;
            uint32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[ms][ns][i]);
            __builtin_amdgcn_raw_buffer_store_b128(v, rg, ((wm * WROWS + ms * 16 + tr) * N + col) * 4, 0, 0);
          }
      }
      // h for this lane, formed in place in acc[ms][hs < HS]: rows (ms, i), columns
      // wn*HS*16 + hs*16 + tc + i of the 128-wide block
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int hs = 0; hs < HS; ++hs) {
            const float gt = acc[ms][hs][i], up = acc[ms][hs + HS][i];
            // silu(gate) * up with the hardware reciprocal (about 1 ulp; h is compared within a
            // tolerance, never bitwise): a full IEEE division here cost ~10 VALU instructions per value
            const float v = (gt * up) * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
            acc[ms][hs][i] = v;
            mx = fmaxf(mx, fabsf(v));
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (lane < 16) red[wm][wn][ms * 16 + lr] = mx;
      }
      // publish the row maxima (LDS only: a __syncthreads fence would also drain the DMA in flight)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int FB = F / 128;
      const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint8_t*>(out) + (size_t)row0 * F, 0, nrows * F, 0x00020000);
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
          out_scales + (size_t)row0 * FB, 0, nrows * FB * 4, 0x00020000);
      const int f0 = cu.nt * 128 + wn * HS * 16 + tc;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int lrow = ms * 16 + tr;   // this lane's row within the wave's rows
        float amax = red[wm][0][lrow];
#pragma unroll
        for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[wm][w][lrow]);
        const float sc = block_scale(amax, POW2);
        const int row = wm * WROWS + lrow;
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
          const float v[4] = {acc[ms][hs][0], acc[ms][hs][1], acc[ms][hs][2], acc[ms][hs][3]};
          float r[4];
          quotients<4>(v, sc, r);
          const uint32_t codes = e4m3_pack4(r[0], r[1], r[2], r[3]);
          __builtin_amdgcn_raw_buffer_store_b32(codes, rq, row * F + f0 + hs * 16, 0, 0);
        }
        // the row's scale: one lane per row (column group 0) of wave column 0; other lanes aim past
        // the buffer's end, which the hardware drops
        if (wn == 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), rsc,
                                                (lane >> 4) == 0 ? (row * FB + cu.nt) * 4 : 0x7FFFFFF0, 0, 0);
      }
      recent[D - 1] = MS * HS + (wn == 0 ? MS : 0) + (g_out ? MS * NS : 0);
    }
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    ck = 0;
    if (++ci < nunits) cu = unit_at(me + ci * G, ny, tiles, offsets, BM);
  }
#undef GEMM_READ_A
#undef GEMM_READ_A_INTO
#undef GEMM_READ_A1
#undef GEMM_READ_B
#undef GEMM_ISSUE
#undef GEMM_ISSUE_CTX
}

int64_t max_tiles_for(int64_t max_rows, int groups, int bm) { return ceil_div64(max_rows, bm) + groups; }

}  // namespace

// Where the plan's second tile list (full tiles first) starts, in tiles from the first list, or 0
// when there is none.  It is written for tiles of 128 and 256 rows, when it fits in the plan
// workspace beside the first list.  A group's short last tile skips its padded wave rows and ends
// early; in group order, the workgroups that share its weight panels then drift apart by more K
// steps than an XCD's L2 holds, and the panels come again from beyond the L2.  With every full
// tile first, the units of a round take equal time.  Measured on the SwiGLU GEMM: beyond-L2 fetch
// at prefill 18.4 -> 14.4 GB, time -2% at prefill and -4% on the long-context chunk.  The store
// GEMM (shorter K) measured 2-3% slower in that order and keeps the first list.
int64_t moe_plan_second_list(int64_t max_rows, int groups, int bm) {
  const int64_t mt = max_tiles_for(max_rows, groups, bm);
  return bm >= 128 && 2 * mt <= max_tiles_for(max_rows, groups, MIN_BM) ? mt : 0;
}

// Where the plan's third tile list starts, in tiles from the first list, or 0 when there is none:
// for 256-row plans whose workspace holds `groups` more entries after the second list.  Such a
// GEMM runs as two launches: the second list (full tiles, then short tiles of more than SPLIT_BM
// rows) with 256-row tiles, then the third (the short remainders of 1 .. SPLIT_BM rows) with
// SPLIT_BM-row tiles.  A remainder of a few rows mostly streams its weight panel, and as a 256-row
// tile at the end of the one launch it took longer than as a 128-row tile of a launch of its own.
// Measured on the long-context chunk (65536 rows over 194 experts, 167 remainders of <= 128 rows):
// SwiGLU GEMM 2700 -> 2492 us, store GEMM 1527 -> 1421 us; on the prefill routing (about 512 rows
// per expert) the remainders over 128 rows stay in the first launch, where a 128-row tile would
// stream their panel twice.
int64_t moe_plan_third_list(int64_t max_rows, int groups, int bm) {
  const int64_t second = moe_plan_second_list(max_rows, groups, bm);
  return bm == 256 && second != 0 && 2 * second + groups <= max_tiles_for(max_rows, groups, MIN_BM) ? 2 * second : 0;
}

namespace {

// Row-tile height when the caller leaves it open: the smallest height that holds twice the
// average group, so that few groups need a second tile (which streams the same weight panel
// again); short groups then stream weights through 32- or 64-row tiles, long ones use 128.
// Groups averaging more than 256 rows take 256-row tiles (per flop, half the global->LDS bytes of
// a 128-row tile; measured on the prefill layer: GEMM1 5.46 -> 5.18 ms, GEMM2 2.99 -> 2.73 ms).
int auto_tile_rows(int64_t max_rows, int groups) {
  const int64_t avg2 = 2 * ceil_div64(max_rows, groups);
  return avg2 <= 32 ? 32 : avg2 <= 48 ? 48 : avg2 <= 64 ? 64 : avg2 < 512 ? 128 : 256;
}
bool valid_tile_rows(int bm) { return bm == 32 || bm == 48 || bm == 64 || bm == 128 || bm == 256; }

template <int BM, bool PACKED, bool POW2, bool FP4 = false, bool WNT = false>
void launch3(unsigned grid, hipStream_t st, int epilogue, int out_dtype, const uint8_t* a, const int32_t* a_rows,
             int a_count, const float* as,
             const int32_t* offsets, const int4* tiles, const int32_t* ntiles, int ny, const uint8_t* b,
             const float* bs, int N, int K, void* out, float* out_scales, float* g_out) {
  if (epilogue == MOE_EPI_STORE) {
    if (out_dtype == MOE_BF16)
      grouped_gemm_kernel<BM, 0, true, PACKED, POW2, FP4, WNT><<<grid, NTHREADS, 0, st>>>(
          a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out, nullptr, nullptr);
    else
      grouped_gemm_kernel<BM, 0, false, PACKED, POW2, FP4, WNT><<<grid, NTHREADS, 0, st>>>(
          a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out, nullptr, nullptr);
  } else {
    grouped_gemm_kernel<BM, 1, false, PACKED, POW2, FP4, WNT><<<grid, NTHREADS, 0, st>>>(
        a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out, out_scales, g_out);
  }
}

// b_layout: 0 row-major, 1 packed FP8, 2 packed FP4 (power-of-two scales only).  WNT: every weight
// panel of the launch is read by one tile (non-temporal weight loads; packed weights only).
template <int BM, bool WNT = false>
void launch(unsigned grid, hipStream_t st, int b_layout, int epilogue, int scale_mode, int out_dtype,
            const uint8_t* a, const int32_t* a_rows, int a_count, const float* as, const int32_t* offsets, const int4* tiles, const int32_t* ntiles,
            int ny, const uint8_t* b, const float* bs, int N, int K, void* out, float* out_scales, float* g_out) {
  const bool p2 = scale_mode == MOE_SCALE_POW2;
  if constexpr (BM == 256 || WNT) {
    // 256-row tiles, and the short remainders of a 256-row plan, stream packed weights only (the
    // host rejects row-major weights for 256-row plans)
    if (b_layout == MOE_B_PACKED_FP4)
      launch3<BM, true, true, true, WNT>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny,
                                         b, bs, N, K, out, out_scales, g_out);
    else if (p2)
      launch3<BM, true, true, false, WNT>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny,
                                          b, bs, N, K, out, out_scales, g_out);
    else
      launch3<BM, true, false, false, WNT>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles,
                                           ny, b, bs, N, K, out, out_scales, g_out);
  } else {
    if (b_layout == MOE_B_PACKED_FP4)
      launch3<BM, true, true, true>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs,
                                    N, K, out, out_scales, g_out);
    else if (b_layout == MOE_B_PACKED && p2)
      launch3<BM, true, true>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K,
                              out, out_scales, g_out);
    else if (b_layout == MOE_B_PACKED)
      launch3<BM, true, false>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N,
                               K, out, out_scales, g_out);
    else if (p2)
      launch3<BM, false, true>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N,
                               K, out, out_scales, g_out);
    else
      launch3<BM, false, false>(grid, st, epilogue, out_dtype, a, a_rows, a_count, as, offsets, tiles, ntiles, ny, b, bs, N,
                                K, out, out_scales, g_out);
  }
}

// compute units of the current device, queried once per device (atomics: calls may come from
// several host threads at once)
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// panels per group: ceil(N / 256) for STORE, N / 256 for SwiGLU (N % 256 == 0 there)
int64_t panels(int32_t N, int32_t epilogue) { return epilogue == MOE_EPI_STORE ? ceil_div64(N, BN) : N / BN; }

}  // namespace

size_t moe_gemm_workspace(int64_t max_rows, int32_t groups) {
  return (size_t)max_tiles_for(max_rows, groups, MIN_BM) * sizeof(int4) + 256;
}

extern "C" size_t moe_packed_weight_bytes(int32_t groups, int32_t N, int32_t K, int32_t epilogue) {
  if (groups < 1 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return 0;
  if (epilogue != MOE_EPI_STORE && epilogue != MOE_EPI_SWIGLU_QUANT) return 0;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && N % 256 != 0) return 0;
  return (size_t)groups * (size_t)panels(N, epilogue) * BN * (size_t)K;
}

extern "C" int moe_pack_weights_fp8(const uint8_t* b, int32_t groups, int32_t N, int32_t K, int32_t epilogue,
                                    uint8_t* packed, void* stream) {
  if (epilogue != MOE_EPI_STORE && epilogue != MOE_EPI_SWIGLU_QUANT) return MOE_ERR_ARG;
  if (groups < 1 || N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && N % 256 != 0) return MOE_ERR_SHAPE;
  const int64_t ny = panels(N, epilogue);
  if (ny * BN * (int64_t)K > (int64_t)UINT32_MAX) return MOE_ERR_SHAPE;
  if (!b || !packed) return MOE_ERR_NULL;
  const int64_t units = (int64_t)groups * ny * BN * K / 16;
  const int64_t blocks = (units + 255) / 256;
  if (blocks > INT32_MAX) return MOE_ERR_SHAPE;
  pack_weights_kernel<<<(unsigned)blocks, 256, 0, as_stream(stream)>>>(b, N, K, (int)ny, epilogue, units, packed);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

namespace {

// argument checks shared by the one-call and the planned entry points
int check_gemm_args(int64_t max_rows, int32_t groups, int32_t N, int32_t K, int32_t epilogue, int32_t scale_mode,
                    int out_dtype, int32_t b_layout) {
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (groups < 1 || groups > 4096 || max_rows < 0 || max_rows > INT32_MAX - 256) return MOE_ERR_SHAPE;
  if (N < 128 || K < 128 || N % 128 != 0 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (epilogue == MOE_EPI_STORE) {
    if (out_dtype != MOE_BF16 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  } else if (epilogue == MOE_EPI_SWIGLU_QUANT) {
    if (out_dtype != MOE_FP8_E4M3) return MOE_ERR_DTYPE;
    if (N % 256 != 0) return MOE_ERR_SHAPE;   // F = N/2 must be a multiple of 128
  } else {
    return MOE_ERR_ARG;
  }
  // byte offsets inside a and inside one group's weights are 32-bit in the kernel
  if ((max_rows + 1) * (int64_t)K > (int64_t)UINT32_MAX || panels(N, epilogue) * BN * (int64_t)K > (int64_t)UINT32_MAX)
    return MOE_ERR_SHAPE;
  if (b_layout != MOE_B_ROWMAJOR && b_layout != MOE_B_PACKED && b_layout != MOE_B_PACKED_FP4) return MOE_ERR_ARG;
  if (b_layout == MOE_B_PACKED_FP4 && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  return MOE_OK;
}

}  // namespace

// The host half of a plan: checks, tile height, sizes (no launch).  *max_tiles receives the length
// of the tile list the workspace holds (0 when max_rows is 0).  Shared with the dispatch, whose
// one-workgroup path writes the tile list itself.
int moe_plan_host(int32_t groups, int64_t max_rows, int32_t tile_rows, void* workspace, size_t workspace_bytes,
                  moe_gemm_plan* plan, int64_t* max_tiles) {
  if (!plan) return MOE_ERR_NULL;
  if (groups < 1 || groups > 4096 || max_rows < 0 || max_rows > INT32_MAX - 256) return MOE_ERR_SHAPE;
  if (tile_rows != 0 && !valid_tile_rows(tile_rows)) return MOE_ERR_ARG;
  const int bm = tile_rows != 0 ? tile_rows : auto_tile_rows(max_rows, groups);
  plan->tile_rows = bm;
  plan->groups = groups;
  plan->max_rows = max_rows;
  plan->workspace = workspace;
  *max_tiles = 0;
  if (max_rows == 0) return MOE_OK;
  if (!workspace || workspace_bytes < moe_gemm_workspace(max_rows, groups)) return MOE_ERR_WORKSPACE;
  *max_tiles = max_tiles_for(max_rows, groups, bm);
  return MOE_OK;
}

extern "C" int moe_grouped_gemm_plan(const int32_t* offsets, int32_t groups, int64_t max_rows, int32_t tile_rows,
                                     void* workspace, size_t workspace_bytes, moe_gemm_plan* plan, void* stream) {
  if (!plan) return MOE_ERR_NULL;
  if (max_rows > 0 && !offsets) return MOE_ERR_NULL;
  int64_t mt = 0;
  const int rc = moe_plan_host(groups, max_rows, tile_rows, workspace, workspace_bytes, plan, &mt);
  if (rc != MOE_OK || max_rows == 0) return rc;
  const int bm = plan->tile_rows;
  int4* tiles = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(workspace) + 256);
  int32_t* ntiles = reinterpret_cast<int32_t*>(workspace);
  tile_map_kernel<<<1, 1024, 0, as_stream(stream)>>>(offsets, groups, bm, tiles, ntiles, (int)mt,
                                                    (int)moe_plan_second_list(max_rows, groups, bm),
                                                    (int)moe_plan_third_list(max_rows, groups, bm));
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

namespace {
int run_planned(const moe_gemm_plan* plan, const uint8_t* a, const int32_t* a_rows, int64_t a_count, const float* as,
                const int32_t* offsets,
                const uint8_t* b, int32_t b_layout, const float* bs, int32_t N, int32_t K, int32_t epilogue,
                int32_t scale_mode, void* out, int out_dtype, float* out_scales, float* g_out, void* stream) {
  if (!plan) return MOE_ERR_NULL;
  const int64_t max_rows = plan->max_rows;
  const int32_t groups = plan->groups;
  const int bm = plan->tile_rows;
  int rc = check_gemm_args(max_rows, groups, N, K, epilogue, scale_mode, out_dtype, b_layout);
  if (rc != MOE_OK) return rc;
  if (!valid_tile_rows(bm)) return MOE_ERR_ARG;
  if (bm == 256 && b_layout == MOE_B_ROWMAJOR) return MOE_ERR_ARG;   // 256-row tiles need packed weights
  if (max_rows == 0) return MOE_OK;
  // gathered rows: a holds a_count rows; every byte offset into it must fit 32 bits like a's own
  if (a_rows && (a_count < 1 || (a_count + 1) * (int64_t)K >= ((int64_t)1 << 32))) return MOE_ERR_SHAPE;
  if (!a || !as || !offsets || !b || !bs || !out || !plan->workspace) return MOE_ERR_NULL;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && !out_scales) return MOE_ERR_NULL;
  hipStream_t st = as_stream(stream);
  const int64_t mt = max_tiles_for(max_rows, groups, bm);
  const int ny = (int)panels(N, epilogue);
  const int64_t nwg = mt * ny;
  if (nwg > INT32_MAX) return MOE_ERR_SHAPE;
  const int4* tiles = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(plan->workspace) + 256);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(plan->workspace);
  const int cus = compute_units();
  if (cus <= 0) return MOE_ERR_HIP;
  const int64_t second = moe_plan_second_list(max_rows, groups, bm);
  const int64_t third = moe_plan_third_list(max_rows, groups, bm);
  if (third) {
    // two launches: the second list with 256-row tiles, then the third with SPLIT_BM-row tiles
    // (one persistent workgroup per compute unit each, never more than the list can hold)
    launch<256>((unsigned)std::min<int64_t>(nwg, cus), st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows,
                (int)a_count, as, offsets, tiles + second, ntiles + 1, ny, b, bs, N, K, out, out_scales, g_out);
    MOE_CHECK_LAUNCH();
    // each remainder is one tile, so each of its weight panels is read once: non-temporal weight
    // loads (same box: store GEMM -2% on the long-context stream and at prefill)
    launch<SPLIT_BM, true>((unsigned)std::min<int64_t>((int64_t)groups * ny, cus), st, b_layout, epilogue, scale_mode,
                           out_dtype, a, a_rows, (int)a_count, as, offsets, tiles + third, ntiles + 2, ny, b, bs, N, K,
                           out, out_scales, g_out);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  if (epilogue == MOE_EPI_SWIGLU_QUANT && second) {   // full tiles first
    tiles += second;
    ntiles += 1;
  }
  // one persistent workgroup per compute unit (the LDS ring admits one per CU), never more than
  // the worst-case number of units
  const unsigned grid = (unsigned)std::min<int64_t>(nwg, cus);
  if (bm == 32)
    launch<32>(grid, st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows, (int)a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
               out_scales, g_out);
  else if (bm == 48)
    launch<48>(grid, st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows, (int)a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
               out_scales, g_out);
  else if (bm == 64)
    launch<64>(grid, st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows, (int)a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K, out,
               out_scales, g_out);
  else if (bm == 128)
    launch<128>(grid, st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows, (int)a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K,
                out, out_scales, g_out);
  else
    launch<256>(grid, st, b_layout, epilogue, scale_mode, out_dtype, a, a_rows, (int)a_count, as, offsets, tiles, ntiles, ny, b, bs, N, K,
                out, out_scales, g_out);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
}  // namespace

extern "C" int moe_grouped_gemm_fp8_planned(const moe_gemm_plan* plan, const uint8_t* a, const float* as,
                                            const int32_t* offsets, const uint8_t* b, int32_t b_layout,
                                            const float* bs, int32_t N, int32_t K, int32_t epilogue,
                                            int32_t scale_mode, void* out, int out_dtype, float* out_scales,
                                            void* stream) {
  return run_planned(plan, a, nullptr, 0, as, offsets, b, b_layout, bs, N, K, epilogue, scale_mode, out, out_dtype,
                     out_scales, nullptr, stream);
}

extern "C" int moe_grouped_gemm_fp8_gather(const moe_gemm_plan* plan, const uint8_t* a, int64_t a_count,
                                           const int32_t* a_rows, const float* as, const int32_t* offsets,
                                           const uint8_t* b, int32_t b_layout, const float* bs, int32_t N, int32_t K,
                                           int32_t epilogue, int32_t scale_mode, void* out, int out_dtype,
                                           float* out_scales, float* g_out, void* stream) {
  if (!a_rows && plan && plan->max_rows > 0) return MOE_ERR_NULL;
  if (g_out && epilogue != MOE_EPI_SWIGLU_QUANT) return MOE_ERR_ARG;
  return run_planned(plan, a, a_rows, a_count, as, offsets, b, b_layout, bs, N, K, epilogue, scale_mode, out,
                     out_dtype, out_scales, g_out, stream);
}

extern "C" int moe_grouped_gemm_fp8_swiglu_save(const moe_gemm_plan* plan, const uint8_t* a, const float* as,
                                                const int32_t* offsets, const uint8_t* b, int32_t b_layout,
                                                const float* bs, int32_t N, int32_t K, int32_t scale_mode,
                                                uint8_t* h, float* h_scales, float* g_out, void* stream) {
  if (!g_out && plan && plan->max_rows > 0) return MOE_ERR_NULL;
  return run_planned(plan, a, nullptr, 0, as, offsets, b, b_layout, bs, N, K, MOE_EPI_SWIGLU_QUANT, scale_mode, h, MOE_FP8_E4M3,
                     h_scales, g_out, stream);
}

extern "C" int moe_grouped_gemm_fp8(const uint8_t* a, const float* as, const int32_t* offsets, int32_t groups,
                                    int64_t max_rows, const uint8_t* b, int32_t b_layout, const float* bs, int32_t N,
                                    int32_t K, int32_t epilogue, int32_t scale_mode, int32_t tile_rows, void* out,
                                    int out_dtype, float* out_scales, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  int rc = check_gemm_args(max_rows, groups, N, K, epilogue, scale_mode, out_dtype, b_layout);
  if (rc != MOE_OK) return rc;
  if (tile_rows != 0 && !valid_tile_rows(tile_rows)) return MOE_ERR_ARG;
  if (tile_rows == 256 && b_layout == MOE_B_ROWMAJOR) return MOE_ERR_ARG;
  if (max_rows == 0) return MOE_OK;
  if (!a || !as || !offsets || !b || !bs || !out) return MOE_ERR_NULL;
  if (epilogue == MOE_EPI_SWIGLU_QUANT && !out_scales) return MOE_ERR_NULL;
  if (!workspace || workspace_bytes < moe_gemm_workspace(max_rows, groups)) return MOE_ERR_WORKSPACE;
  if (compute_units() <= 0) return MOE_ERR_HIP;
  // the automatic height never picks 256-row tiles for row-major weights (packed weights only)
  if (tile_rows == 0 && b_layout == MOE_B_ROWMAJOR) tile_rows = std::min(auto_tile_rows(max_rows, groups), 128);
  moe_gemm_plan plan;
  rc = moe_grouped_gemm_plan(offsets, groups, max_rows, tile_rows, workspace, workspace_bytes, &plan, stream);
  if (rc != MOE_OK) return rc;
  return moe_grouped_gemm_fp8_planned(&plan, a, as, offsets, b, b_layout, bs, N, K, epilogue, scale_mode, out,
                                      out_dtype, out_scales, stream);
}

// ------------------------------------------------------------------------------------------------
// No-allocation variant: the tile plan lives in this file-scope device array (one copy per GPU).
// Host code never passes `scratch` itself (its host-side name is not a device address): the
// device address of each GPU's copy is looked up once, with that device current, and cached.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
// device address of this device's scratch (nullptr on a HIP error)
void* scratch_address() {
  static std::atomic<void*> cached[MAX_DEVICES];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  cached[dev].store(q, std::memory_order_release);   // concurrent first calls store the same value
  return q;
}
}  // namespace

extern "C" int moe_grouped_gemm_fp8_noalloc(const uint8_t* a, const float* as, const int32_t* offsets, int32_t groups,
                                            int64_t max_rows, const uint8_t* b, int32_t b_layout, const float* bs,
                                            int32_t N, int32_t K, int32_t epilogue, int32_t scale_mode,
                                            int32_t tile_rows, void* out, int out_dtype, float* out_scales,
                                            void* stream) {
  int rc = check_gemm_args(max_rows, groups, N, K, epilogue, scale_mode, out_dtype, b_layout);
  if (rc != MOE_OK) return rc;
  if (max_rows == 0) return MOE_OK;
  if (moe_gemm_workspace(max_rows, groups) > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_HIP;
  return moe_grouped_gemm_fp8(a, as, offsets, groups, max_rows, b, b_layout, bs, N, K, epilogue, scale_mode, tile_rows,
                              out, out_dtype, out_scales, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}
