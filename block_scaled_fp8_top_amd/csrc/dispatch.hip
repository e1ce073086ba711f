// Dispatch: a stable counting sort of the flattened [T,k] expert ids into expert-contiguous
// groups, then the permutation of the quantised activation rows and their scales.
//
//   1. count:   the T*k slots are cut into chunks of CHUNK; each chunk's expert histogram goes to
//               the workspace (LDS integer atomics: exact counts, order-free).
//   2. scan:    one workgroup turns the per-chunk histograms into expert totals, the exclusive
//               prefix `offsets`, and each chunk's starting row per expert (and, when asked, the
//               grouped GEMM's tile lists).
//   3. scatter: one wavefront per chunk walks its slots in order, 64 at a time; lanes holding the
//               same expert find each other with ballots over the bits of the expert id, so each
//               slot's row is (chunk base) + (earlier slots of the chunk with that expert) --
//               exactly the stable order.  Also fills the shared expert's rows.
//   4. permute: rows [0, offsets[G]) copy xq[src_token[row]] and xs[src_token[row]] (the scales
//               alone when the codes are gathered by the GEMM).
//
// Small batches (decode: up to SMALL_MAX slots) run steps 1-3 in one workgroup instead
// (small_dispatch_kernel), which gives the same stable order.
#include <algorithm>

#include "common.h"

namespace {

constexpr int CHUNK = 1024;   // slots per chunk
constexpr int MAXE = 1024;

// Inclusive scan of v over the 1024 threads of the workgroup (integers: the order of the additions
// does not matter): a shuffle scan within each wavefront, then each wavefront adds the totals of
// the wavefronts before it.  wsum: 16 ints of LDS.  Every thread calls it.
__device__ __forceinline__ int block_scan_1024(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += wsum[w];
  __syncthreads();   // wsum may be written again by the next call
  return x + add;
}

// The grouped GEMM's tile lists for row tiles of bm, written by one workgroup of 1024 threads that
// has the expert totals: thread e < E holds total = expert e's rows, part[] the inclusive block scan
// of the totals over e, routed = part[E - 1]; the shared expert (append_shared) is group E with T
// rows.  The entries are those the plan kernel of the grouped GEMM writes: {group, first row, the
// block's first tile, the block's tile count}, at most max_tiles of them, and their number into
// ntiles[0]; with second != 0 the second list at tiles + second (every group's full tiles first,
// then the groups' short last tiles; with third != 0 only those over 128 rows) into ntiles[1], and
// with third != 0 the third list at tiles + third (one 128-row tile per short remainder of 1 .. 128
// rows) into ntiles[2].  Needs E + append_shared <= 1024.  tpart[16] and first[1025] are LDS
// scratch.
__device__ __forceinline__ void write_tile_lists(int tid, int E, int T, int append_shared, int total,
                                                 const int* part, int routed, int bm, int4* __restrict__ tiles,
                                                 int32_t* __restrict__ ntiles, int max_tiles, int second, int third,
                                                 int* tpart, int* first) {
  // tile plan: group g has ceil(rows / bm) tiles; a block scan gives each group's first tile, then
  // every thread writes tiles, finding a tile's group by binary search over the first tiles
  const int G = E + (append_shared ? 1 : 0);
  const int rows_g = tid < E ? total : (tid == E && append_shared ? T : 0);
  // first[0 .. G]: exclusive block scan over the groups of v (this thread's group's count)
  auto scan_first = [&](int v) {
    const int incl = block_scan_1024(v, tpart);
    if (tid < G) first[tid] = incl - v;
    if (tid == G - 1) first[G] = incl;
    __syncthreads();
  };
  // the group owning position t: the last group whose first position is at or before t
  auto owner = [&](int t) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  auto row_of = [&](int g) { return g < E ? (g == 0 ? 0 : part[g - 1]) : routed; };
  scan_first((rows_g + bm - 1) / bm);
  const int ntot = min(first[G], max_tiles);
  for (int t = tid; t < ntot; t += 1024) {
    const int lo = owner(t);
    tiles[t] = make_int4(lo, row_of(lo) + (t - first[lo]) * bm, first[lo], first[lo + 1] - first[lo]);
  }
  if (tid == 0) *ntiles = ntot;
  if (!second) return;
  __syncthreads();
  scan_first(rows_g / bm);                       // full tiles first
  const int nfull = first[G];
  for (int t = tid; t < min(nfull, ntot); t += 1024) {
    const int lo = owner(t);
    tiles[second + t] = make_int4(lo, row_of(lo) + (t - first[lo]) * bm, first[lo], first[lo + 1] - first[lo]);
  }
  __syncthreads();
  // then every group's short last tile (with a third list, only those over 128 rows)
  scan_first(rows_g % bm > (third ? 128 : 0) ? 1 : 0);
  const int n2 = min(nfull + first[G], ntot);
  for (int t = nfull + tid; t < n2; t += 1024) {
    const int lo = owner(t - nfull);
    const int g_rows = lo < E ? row_of(lo + 1) - row_of(lo) : T;
    tiles[second + t] = make_int4(lo, row_of(lo) + (g_rows / bm) * bm, t, 1);
  }
  if (tid == 0) ntiles[1] = n2;
  if (!third) return;
  __syncthreads();
  scan_first(rows_g % bm > 0 && rows_g % bm <= 128 ? 1 : 0);   // the third list: short remainders
  const int n3 = first[G];
  for (int t = tid; t < n3; t += 1024) {
    const int lo = owner(t);
    const int g_rows = lo < E ? row_of(lo + 1) - row_of(lo) : T;
    tiles[third + t] = make_int4(lo, row_of(lo) + (g_rows / bm) * bm, t, 1);
  }
  if (tid == 0) ntiles[2] = n3;
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int64_t nslots, int E,
                                                    int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[MAXE];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * CHUNK;
  for (int i = threadIdx.x; i < CHUNK; i += 256) {
    const int64_t s = s0 + i;
    if (s < nslots) {
      const int e = idx[s];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// one workgroup of 1024 threads; thread e owns expert e.  With tiles != NULL it also writes the
// grouped GEMM's tile lists (write_tile_lists), so no plan kernel has to read the offsets back.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                    int append_shared, int64_t T, int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int bm, int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                    int max_tiles, int second, int third) {
  __shared__ int part[1024];
  __shared__ int tpart[16];
  __shared__ int first[1025];
  const int e = threadIdx.x;
  // expert e's total over the chunks: 16 independent loads in flight per step (a load-add chain
  // over 128 chunks would cost 128 memory round trips)
  int total = 0;
  if (e < E) {
    int c = 0;
    for (; c + 16 <= nchunks; c += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = chunk_counts[(int64_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) total += v[i];
    }
    for (; c < nchunks; ++c) total += chunk_counts[(int64_t)c * E + e];
  }
  // inclusive block scan of totals over e
  part[e] = block_scan_1024(total, tpart);
  __syncthreads();
  const int excl = part[e] - total;
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    // each chunk's base row for expert e: the expert's offset plus its counts in earlier chunks
    int run = excl, c = 0;
    for (; c + 16 <= nchunks; c += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = chunk_counts[(int64_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        chunk_base[(int64_t)(c + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; c < nchunks; ++c) {
      const int v = chunk_counts[(int64_t)c * E + e];
      chunk_base[(int64_t)c * E + e] = run;
      run += v;
    }
  }
  const int routed = part[E - 1];
  if (e == 0) {
    offsets[E] = routed;
    if (append_shared) {
      counts[E] = (int32_t)T;
      offsets[E + 1] = routed + (int32_t)T;
    }
  }
  if (tiles)
    write_tile_lists(e, E, (int)T, append_shared, total, part, routed, bm, tiles, ntiles, max_tiles, second, third,
                     tpart, first);
}

template <int BITS>
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ idx, int64_t nslots, int k, int E,
                                                     int64_t T, int append_shared,
                                                     const int32_t* __restrict__ chunk_base,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ dest_row, int32_t* __restrict__ src_token) {
  __shared__ int running[MAXE];
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  for (int e = lane; e < E; e += 64) running[e] = chunk_base[(int64_t)chunk * E + e];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t s0 = (int64_t)chunk * CHUNK;
  for (int i = 0; i < CHUNK; i += 64) {
    const int64_t s = s0 + i + lane;
    const bool in = s < nslots;
    const int e = in ? idx[s] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
      const uint64_t m = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    int pos = -1;
    if (valid) {
      const int rank = __popcll(peers & lt);
      pos = running[e] + rank;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (valid && (peers & lt) == 0) running[e] += __popcll(peers);  // group leader advances the base
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (in) dest_row[s] = pos;
    if (valid) src_token[pos] = (int32_t)(s / k);
    if (s0 + i + 64 >= nslots) break;
  }
  if (append_shared) {
    const int32_t base = offsets[E];
    for (int64_t t = (int64_t)chunk * 64 + lane; t < T; t += (int64_t)gridDim.x * 64) src_token[base + t] = (int32_t)t;
  }
}

// rows [0, offsets[G]): one row per 64-lane group, 16-byte copies
__global__ __launch_bounds__(256) void permute_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ xs,
                                                      int H, const int32_t* __restrict__ src_token,
                                                      const int32_t* __restrict__ total_rows, int64_t max_rows,
                                                      uint8_t* __restrict__ aq, float* __restrict__ as) {
  const int64_t rows = *total_rows;
  const int lane = threadIdx.x & 63;
  for (int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / 64; row < rows && row < max_rows;
       row += (int64_t)gridDim.x * 4) {
    const int64_t t = src_token[row];
    if (aq) {   // codes too (without them a grouped GEMM gathers the rows through src_token)
      const uint4* src = reinterpret_cast<const uint4*>(xq + t * H);
      uint4* dst = reinterpret_cast<uint4*>(aq + row * H);
      for (int c = lane; c < H / 16; c += 64) dst[c] = src[c];
    }
    const int nsc = H / 128;
    for (int c = lane; c < nsc; c += 64) as[row * nsc + c] = xs[t * nsc + c];
  }
}

// Scales only (the grouped GEMM gathers the codes through src_token): one thread per (row, 16-byte
// piece of the row's H/128 scales; H % 512 == 0), a row's pieces on consecutive threads.  Measured
// at 65536 rows, H 6144: 4.5 us, against 18.3 us with 16 lanes per row and 4 rows per lane group.
__global__ __launch_bounds__(256) void permute_scales_kernel(const float* __restrict__ xs, int H,
                                                             const int32_t* __restrict__ src_token,
                                                             const int32_t* __restrict__ total_rows, int64_t max_rows,
                                                             float* __restrict__ as) {
  const int64_t rows = min((int64_t)*total_rows, max_rows);
  const int np = H / 512;   // 16-byte pieces per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = i / np;
  if (r >= rows) return;
  const int c = (int)(i - r * np);
  const int64_t t = src_token[r];
  reinterpret_cast<float4*>(as + r * (H / 128))[c] = reinterpret_cast<const float4*>(xs + t * (H / 128))[c];
}

constexpr int SMALL_MAX = 8192;       // slots
constexpr int SMALL_CNT = 16384;      // (64-slot pieces) x experts counters in LDS

// One workgroup for the whole batch.  The slots are cut into pieces of 64 (one wavefront step);
// within a piece, lanes holding the same expert find each other with ballots over the expert id
// bits, giving each slot its rank among the piece's earlier slots of that expert, and the group
// leader records the piece's count for the expert.  Thread e then turns its expert's piece counts
// into running bases (pieces in order), a block scan gives the expert offsets, and every slot's
// row is offset + piece base + rank: the stable order.
// With tiles != NULL the same workgroup also writes the grouped GEMM's tile list for row tiles of
// bm (the entries the plan kernel of the grouped GEMM writes: {group, first row, the block's first
// tile, the block's tile count}, at most max_tiles of them, and their number into ntiles[0]), with
// second != 0 the second list at tiles + second (every group's full tiles first, then the groups'
// short last tiles; with third != 0 only those over 128 rows) into ntiles[1], and with third != 0
// the third list at tiles + third (one 128-row tile per short remainder of 1 .. 128 rows) into
// ntiles[2], as the plan kernel does.
template <int BITS>
__global__ __launch_bounds__(1024) void small_dispatch_kernel(const int32_t* __restrict__ idx, int nslots, int k, int E,
                                                              int T, int append_shared, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ dest_row,
                                                              int32_t* __restrict__ src_token, int bm,
                                                              int4* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                              int max_tiles, int second, int third) {
  __shared__ int sidx[SMALL_MAX];
  __shared__ uint8_t srank[SMALL_MAX];
  __shared__ int cnt[SMALL_CNT];      // [piece][e]
  __shared__ int part[1024];
  __shared__ int tpart[16];
  __shared__ int first[1025];         // tile plan: the groups' first tiles, first[G] = all tiles
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npiece = (nslots + 63) / 64;
  for (int i = tid; i < npiece * E; i += 1024) cnt[i] = 0;
  for (int s = tid; s < nslots; s += 1024) sidx[s] = idx[s];
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int q = wave; q < npiece; q += 16) {
    const int s = q * 64 + lane;
    const bool in = s < nslots;
    const int e = in ? sidx[s] : -1;
    const bool valid = in && e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bt = 0; bt < BITS; ++bt) {
      const uint64_t m = __ballot(valid && ((e >> bt) & 1));
      peers &= ((e >> bt) & 1) ? m : ~m;
    }
    if (valid) {
      srank[s] = (uint8_t)__popcll(peers & lt);
      if ((peers & lt) == 0) cnt[q * E + e] = __popcll(peers);   // group leader
    } else if (in) {
      dest_row[s] = -1;
    }
  }
  __syncthreads();
  // expert e: running bases over the pieces, then the block scan of the totals
  int total = 0;
  if (tid < E) {
    for (int q = 0; q < npiece; ++q) {
      const int c = cnt[q * E + tid];
      cnt[q * E + tid] = total;
      total += c;
    }
  }
  part[tid] = block_scan_1024(total, tpart);
  __syncthreads();
  const int routed = part[E - 1];
  if (tid < E) {
    counts[tid] = total;
    offsets[tid] = part[tid] - total;
  }
  if (tid == 0) {
    offsets[E] = routed;
    if (append_shared) {
      counts[E] = T;
      offsets[E + 1] = routed + T;
    }
  }
  __syncthreads();   // part[] now holds inclusive sums: offset of e = part[e] - (its total)
  for (int s = tid; s < nslots; s += 1024) {
    const int e = sidx[s];
    if (e < 0 || e >= E) continue;
    const int first = e == 0 ? 0 : part[e - 1];
    const int row = first + cnt[(s >> 6) * E + e] + srank[s];
    dest_row[s] = row;
    src_token[row] = s / k;
  }
  if (append_shared)
    for (int t = tid; t < T; t += 1024) src_token[routed + t] = t;
  if (tiles)
    write_tile_lists(tid, E, T, append_shared, total, part, routed, bm, tiles, ntiles, max_tiles, second, third,
                     tpart, first);
}

int64_t nchunks_for(int64_t T, int k) { return ceil_div64(T * k, CHUNK); }

}  // namespace

size_t moe_dispatch_workspace(int64_t T, int32_t k, int32_t E) {
  return (size_t)(2 * nchunks_for(T, k) * (int64_t)E * 4 + 256);
}

int64_t moe_plan_second_list(int64_t max_rows, int groups, int bm);
int64_t moe_plan_third_list(int64_t max_rows, int groups, int bm);
int moe_plan_host(int32_t groups, int64_t max_rows, int32_t tile_rows, void* workspace, size_t workspace_bytes,
                  moe_gemm_plan* plan, int64_t* max_tiles);

namespace {

// The dispatch; with plan_ws != NULL (and at most 1024 groups) its one-workgroup kernel -- the small
// path's kernel, else the scan -- also writes the tile lists of plan_bm-row tiles into plan_ws
// (*planned is then set).
int dispatch_impl(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                  const uint8_t* xq, const float* xs, int32_t H, int32_t* counts, int32_t* offsets,
                  int32_t* dest_row, int32_t* src_token, uint8_t* aq, float* as, void* workspace,
                  size_t workspace_bytes, void* stream, int plan_bm, void* plan_ws, int64_t plan_max_tiles,
                  bool* planned) {
  *planned = false;
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > MAXE) return MOE_ERR_SHAPE;
  if (T * (int64_t)k + T > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  // rows: aq given -> codes and scales are permuted; only as given -> only the scales
  const bool copy_rows = aq || as;
  if (copy_rows && (H < 128 || H % 128 != 0)) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !dest_row || !src_token)) return MOE_ERR_NULL;
  if (copy_rows && (!xs || !as || (aq && !xq))) return MOE_ERR_NULL;
  const int64_t nch = nchunks_for(T, k);
  if (!workspace || workspace_bytes < moe_dispatch_workspace(T, k, E)) return MOE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + nch * E;
  const int64_t nslots = T * k;
  int bits = 1;
  while ((1 << bits) < E) ++bits;
  // the tile plan is written by the dispatch's own one-workgroup kernel (the small path's, else
  // the scan) when the groups fit its 1024 threads
  const bool plan_here = plan_ws && E + (append_shared ? 1 : 0) <= 1024 && plan_max_tiles <= INT32_MAX &&
                         nslots + (append_shared ? T : 0) <= INT32_MAX;
  int4* ptiles = plan_here ? reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(plan_ws) + 256) : nullptr;
  int32_t* pntiles = plan_here ? reinterpret_cast<int32_t*>(plan_ws) : nullptr;
  const int64_t second = plan_here ? moe_plan_second_list(nslots + (append_shared ? T : 0),
                                                          E + (append_shared ? 1 : 0), plan_bm) : 0;
  const int64_t third = plan_here ? moe_plan_third_list(nslots + (append_shared ? T : 0),
                                                        E + (append_shared ? 1 : 0), plan_bm) : 0;
  if (nslots <= SMALL_MAX && ceil_div64(nslots, 64) * E <= SMALL_CNT) {
    switch (bits) {
#define CASE_SMALL(B)                                                                                   \
  case B:                                                                                               \
    small_dispatch_kernel<B><<<1, 1024, 0, st>>>(topk_idx, (int)nslots, k, E, (int)T, append_shared, counts, \
                                                 offsets, dest_row, src_token, plan_bm, ptiles, pntiles, \
                                                 (int)plan_max_tiles, (int)second, (int)third);          \
    break;
      CASE_SMALL(1) CASE_SMALL(2) CASE_SMALL(3) CASE_SMALL(4) CASE_SMALL(5)
      CASE_SMALL(6) CASE_SMALL(7) CASE_SMALL(8) CASE_SMALL(9) CASE_SMALL(10)
#undef CASE_SMALL
      default:
        return MOE_ERR_SHAPE;
    }
    MOE_CHECK_LAUNCH();
    *planned = plan_here;
  } else {
  if (nch > 0) {
    count_kernel<<<(unsigned)nch, 256, 0, st>>>(topk_idx, nslots, E, chunk_counts);
    MOE_CHECK_LAUNCH();
  }
  scan_kernel<<<1, 1024, 0, st>>>(chunk_counts, (int)nch, E, append_shared, T, chunk_base, counts, offsets, plan_bm,
                                  ptiles, pntiles, (int)plan_max_tiles, (int)second, (int)third);
  MOE_CHECK_LAUNCH();
  *planned = plan_here;
  if (nch > 0) {
    const unsigned g = (unsigned)nch;
    switch (bits) {
#define CASE_BITS(B)                                                                                                  \
  case B:                                                                                                             \
    scatter_kernel<B><<<g, 64, 0, st>>>(topk_idx, nslots, k, E, T, append_shared, chunk_base, offsets, dest_row,      \
                                        src_token);                                                                   \
    break;
      CASE_BITS(1) CASE_BITS(2) CASE_BITS(3) CASE_BITS(4) CASE_BITS(5)
      CASE_BITS(6) CASE_BITS(7) CASE_BITS(8) CASE_BITS(9) CASE_BITS(10)
#undef CASE_BITS
      default:
        return MOE_ERR_SHAPE;
    }
    MOE_CHECK_LAUNCH();
  }
  }
  if (copy_rows && T > 0) {
    const int G = E + (append_shared ? 1 : 0);
    const int64_t max_rows = nslots + (append_shared ? T : 0);
    if (!aq && H % 512 == 0 && ceil_div64(max_rows * (H / 512), 256) <= INT32_MAX) {
      const int64_t grid = ceil_div64(max_rows * (H / 512), 256);
      permute_scales_kernel<<<(unsigned)grid, 256, 0, st>>>(xs, H, src_token, offsets + G, max_rows, as);
    } else {
      const int64_t grid = std::min<int64_t>(ceil_div64(max_rows, 4), 65536);
      permute_kernel<<<(unsigned)grid, 256, 0, st>>>(xq, xs, H, src_token, offsets + G, max_rows, aq, as);
    }
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}
}  // namespace

extern "C" int moe_dispatch(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                            const uint8_t* xq, const float* xs, int32_t H, int32_t* counts, int32_t* offsets,
                            int32_t* dest_row, int32_t* src_token, uint8_t* aq, float* as, void* workspace,
                            size_t workspace_bytes, void* stream) {
  bool planned = false;
  return dispatch_impl(topk_idx, T, k, E, append_shared, xq, xs, H, counts, offsets, dest_row, src_token, aq, as,
                       workspace, workspace_bytes, stream, 0, nullptr, 0, &planned);
}

extern "C" int moe_dispatch_plan(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                                 const uint8_t* xq, const float* xs, int32_t H, int32_t* counts, int32_t* offsets,
                                 int32_t* dest_row, int32_t* src_token, uint8_t* aq, float* as, void* workspace,
                                 size_t workspace_bytes, int32_t tile_rows, void* gemm_workspace,
                                 size_t gemm_workspace_bytes, moe_gemm_plan* plan, void* stream) {
  if (T < 0 || k < 1 || k > 64 || E < 1 || E > MAXE) return MOE_ERR_SHAPE;
  if (T * (int64_t)k + T > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  const int32_t G = E + (append_shared ? 1 : 0);
  const int64_t max_rows = T * (int64_t)k + (append_shared ? T : 0);
  int64_t mt = 0;
  int rc = moe_plan_host(G, max_rows, tile_rows, gemm_workspace, gemm_workspace_bytes, plan, &mt);
  if (rc != MOE_OK) return rc;
  bool planned = false;
  rc = dispatch_impl(topk_idx, T, k, E, append_shared, xq, xs, H, counts, offsets, dest_row, src_token, aq, as,
                     workspace, workspace_bytes, stream, plan->tile_rows, max_rows > 0 ? gemm_workspace : nullptr, mt,
                     &planned);
  if (rc != MOE_OK || planned || max_rows == 0) return rc;
  // the multi-kernel dispatch path: the plan kernel of the grouped GEMM
  return moe_grouped_gemm_plan(offsets, G, max_rows, plan->tile_rows, gemm_workspace, gemm_workspace_bytes, plan,
                               stream);
}
