// Top-k router and router replay, one wavefront (64 lanes) per token.
//
// Lane l holds experts e = l + 64*j (j < EPL).  Scores (softmax or sigmoid with the fixed
// router_exp), the optional group limit, the top-k selection by (logit desc, expert asc) and the
// weights follow the router contract in moe_fp8.h step for step, so that indices and weights are
// reproducible bit for bit.  Sequential sums (the softmax denominator over experts, the
// renormalisation over slots) are taken in the stated order by a single lane or redundantly by
// every lane, never as a tree.  Logits may be -inf (a masked expert): such an expert still ranks
// by the same rule (below every finite logit, ties to the lower index), so a token with fewer than
// k finite allowed logits takes its remaining slots from the lowest-index allowed -inf experts.
// The "no candidate" placeholder of a lane is (-inf, INT_MAX), which every real expert ranks
// before.  NaN logits are outside the contract.
#include <float.h>

#include "common.h"

namespace {

constexpr int WAVES = 4;  // tokens per workgroup
constexpr int MAX_GROUPS = 64;
// 1x128 blocks quantised by one workgroup of the fused router + quantisation launch (16 lanes per block)
constexpr int QBLK = 64 * WAVES / 16;
static_assert(QBLK * 16 == 64 * WAVES, "whole 16-lane groups per workgroup");

struct Cand {
  float z;
  int e;
};

// strict order: a before b when its logit is larger, or equal with a lower expert index
__device__ __forceinline__ bool before(float za, int ea, float zb, int eb) { return za > zb || (za == zb && ea < eb); }

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float oz = __shfl_xor(c.z, o, 64);
    const int oe = __shfl_xor(c.e, o, 64);
    if (before(oz, oe, c.z, c.e)) {
      c.z = oz;
      c.e = oe;
    }
  }
  return c;
}

// Scores of all experts into sc[] (LDS), keys into key[] (LDS).  Returns nothing; the wave is
// synchronised on exit (LDS visible to every lane).
template <int EPL>
__device__ __forceinline__ void token_scores(const float* __restrict__ zrow, int E, int score_fn, int lane,
                                             float (&z)[EPL], float* key, float* sc) {
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    z[j] = e < E ? zrow[e] : -FLT_MAX;
    if (e < E) key[e] = z[j];
  }
  if (score_fn == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < E) m = fmaxf(m, z[j]);
    m = wave_max(m);
    float p[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      p[j] = router_exp(z[j] - m);
      if (e < E) sc[e] = p[j];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    float S = 0.0f;
    if (lane == 0)
      for (int e = 0; e < E; ++e) S = S + sc[e];
    S = __shfl(S, 0, 64);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E) sc[e] = p[j] / S;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E) sc[e] = router_sigmoid(z[j]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
}

template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int64_t t, const moe_router_cfg& cfg,
                                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                            int32_t* __restrict__ record, int64_t record_ld, int lane, float* key,
                                            float* sc) {
  const int E = cfg.num_experts, k = cfg.top_k;
  float z[EPL];
  token_scores<EPL>(logits + t * E, E, cfg.score_fn, lane, z, key, sc);

  // ---- group limit: lane g < n_group scores group g; lane 0 keeps the best topk_group groups
  uint64_t allowed_groups = ~0ull;
  int gs = E;
  if (cfg.n_group > 1) {
    gs = E / cfg.n_group;
    float gscore = -FLT_MAX;
    if (lane < cfg.n_group) {
      const int base = lane * gs;
      uint64_t taken_lo = 0;  // selection bits for the first 64 members (group_score_topk is small)
      float sum = 0.0f;
      int prev[8];
      for (int r = 0; r < cfg.group_score_topk; ++r) {
        int best = -1;
        float bz = 0.0f;
        for (int i = 0; i < gs; ++i) {
          bool used = false;
          if (i < 64) used = (taken_lo >> i) & 1ull;
          else
            for (int q = 0; q < r; ++q) used |= prev[q] == i;
          if (used) continue;
          const float zi = key[base + i];
          if (best < 0 || before(zi, base + i, bz, base + best)) {
            best = i;
            bz = zi;
          }
        }
        if (best < 64) taken_lo |= 1ull << best;
        prev[r] = best;
        sum = sum + sc[base + best];
      }
      gscore = sum;
    }
    // lane 0 gathers the group scores (ascending group order) and keeps topk_group of them
    uint64_t keep = 0;
    for (int r = 0; r < cfg.topk_group; ++r) {
      int best = -1;
      float bs = 0.0f;
      for (int g = 0; g < cfg.n_group; ++g) {
        const float s = __shfl(gscore, g, 64);
        if ((keep >> g) & 1ull) continue;
        if (best < 0 || s > bs) {
          best = g;
          bs = s;
        }
      }
      keep |= 1ull << best;
    }
    allowed_groups = keep;
  }

  // ---- top-k by (logit desc, expert asc) among allowed experts
  uint32_t taken = 0;  // bit j: expert lane + 64*j already selected
  int my_e = -1;
#pragma unroll 1
  for (int r = 0; r < k; ++r) {
    Cand c{-INFINITY, 0x7FFFFFFF};
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e >= E || ((taken >> j) & 1u)) continue;
      if (!((allowed_groups >> (e / gs)) & 1ull)) continue;
      if (c.e == 0x7FFFFFFF || before(z[j], e, c.z, c.e)) {
        c.z = z[j];
        c.e = e;
      }
    }
    c = wave_best(c);
    if (lane == (c.e & 63)) taken |= 1u << (c.e >> 6);
    if (lane == r) my_e = c.e;
  }
  // ---- weights
  const float my_s = lane < k ? sc[my_e] : 0.0f;
  float w = my_s;
  if (cfg.renormalize) {
    float d = 0.0f;
    for (int r = 0; r < k; ++r) d = d + __shfl(my_s, r, 64);
    w = my_s / d;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = w;
    if (record) record[lane * record_ld + t] = my_e;
  }
}

// one wavefront per token
template <int EPL>
__global__ __launch_bounds__(64 * WAVES) void route_kernel(const float* __restrict__ logits, int64_t T,
                                                           moe_router_cfg cfg, int32_t* __restrict__ topk_idx,
                                                           float* __restrict__ topk_w, int32_t* __restrict__ record,
                                                           int64_t record_ld) {
  __shared__ float key_s[WAVES][64 * EPL];
  __shared__ float sc_s[WAVES][64 * EPL];
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const int64_t t = (int64_t)blockIdx.x * WAVES + wv;
  if (t >= T) return;
  route_token<EPL>(logits, t, cfg, topk_idx, topk_w, record, record_ld, lane, key_s[wv], sc_s[wv]);
}

// The router and the 1x128 quantisation of x in one launch (the quantisation does not depend on
// the routing): workgroups [0, nroute) route 4 tokens each as route_kernel does; the others
// quantise 16 blocks of 128 values each, as the 1x128 quantisation kernel does.
template <int EPL, bool BF16, bool POW2>
__global__ __launch_bounds__(64 * WAVES) void route_quant_kernel(const float* __restrict__ logits, int64_t T,
                                                                 moe_router_cfg cfg, int32_t* __restrict__ topk_idx,
                                                                 float* __restrict__ topk_w,
                                                                 int32_t* __restrict__ record, int64_t record_ld,
                                                                 int64_t nroute, const void* __restrict__ x,
                                                                 int64_t nblocks, uint8_t* __restrict__ xq,
                                                                 float* __restrict__ xs) {
  __shared__ float key_s[WAVES][64 * EPL];
  __shared__ float sc_s[WAVES][64 * EPL];
  if ((int64_t)blockIdx.x < nroute) {
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const int64_t t = (int64_t)blockIdx.x * WAVES + wv;
    if (t >= T) return;
    route_token<EPL>(logits, t, cfg, topk_idx, topk_w, record, record_ld, lane, key_s[wv], sc_s[wv]);
    return;
  }
  const int64_t b = ((int64_t)blockIdx.x - nroute) * QBLK + threadIdx.x / 16;
  if (b >= nblocks) return;   // whole 16-lane groups are in or out of range
  quant_1x128_piece<BF16, POW2>(x, b, threadIdx.x & 15, xq, xs);
}

// ---------------------------------------------------------------------------------------------
// Sixteen lanes per token (four tokens per wavefront, FTOK per workgroup), for E = 16 * EPT
// experts: token-local lane tl holds experts tl*EPT .. tl*EPT + EPT - 1 in registers.  With a group
// limit, a group (E / n_group experts, a multiple of EPT) is LPG = 16 / n_group adjacent lanes, an
// aligned DPP segment.  Every expert carries a 64-bit rank key: the order-preserving bits of its
// logit (-0 taken as +0, since the order compares values) above the complemented expert index,
// so key order is (logit descending, expert ascending) and no real key is 0.  A selection round
// takes the largest key below the previous round's winner: the next expert in that order.  The
// results are those of route_token bit for bit: the same scores (the same fp32 operations on the
// same logits), the same sums in the same order, the same orders.
constexpr int FTOK = 16;

__device__ __forceinline__ uint64_t rank_key(float z, int e) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
// largest key of each aligned segment of n lanes (n = 1, 2, 4, 8 or 16, wave-uniform), in every
// lane of the segment
__device__ __forceinline__ uint64_t seg_max(uint64_t v, int n) {
  if (n >= 2) v = umax64(v, dpp_u64<DPP_XOR1>(v));
  if (n >= 4) v = umax64(v, dpp_u64<DPP_XOR2>(v));
  if (n >= 8) v = umax64(v, dpp_u64<DPP_HALF_MIRROR>(v));
  if (n >= 16) v = umax64(v, dpp_u64<DPP_MIRROR>(v));
  return v;
}
// largest of this lane's keys below thr (0 if none)
template <int EPT>
__device__ __forceinline__ uint64_t lane_best_below(const uint64_t (&key)[EPT], uint64_t thr) {
  uint64_t b = 0;
#pragma unroll
  for (int m = 0; m < EPT; ++m)
    if (key[m] < thr && key[m] > b) b = key[m];
  return b;
}

// token t (live: t < T; a dead token computes on placeholders and writes nothing).  psum: the
// token's E floats of LDS (softmax only).
template <int EPT, bool SOFTMAX>
__device__ __forceinline__ void route_token16(const float* __restrict__ logits, int64_t t, bool live,
                                              const moe_router_cfg& cfg, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w, int32_t* __restrict__ record,
                                              int64_t record_ld, float* psum) {
  constexpr int E = 16 * EPT;
  const int k = cfg.top_k;
  const int lane = threadIdx.x & 63, tl = lane & 15, tokbase = lane & 48;
  const int e0 = tl * EPT;
  float z[EPT];
  if (live) {
    const float4* src = reinterpret_cast<const float4*>(logits + t * E + e0);
#pragma unroll
    for (int m = 0; m < EPT / 4; ++m) {
      const float4 v = src[m];
      z[4 * m] = v.x; z[4 * m + 1] = v.y; z[4 * m + 2] = v.z; z[4 * m + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < EPT; ++m) z[m] = 0.0f;
  }
  uint64_t key[EPT];
#pragma unroll
  for (int m = 0; m < EPT; ++m) key[m] = rank_key(z[m], e0 + m);

  // scores: softmax p_e / S with S summed over e ascending from +0, or the sigmoid
  float mx = 0.0f, S = 1.0f;
  if (SOFTMAX) {
    mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < EPT; ++m) mx = fmaxf(mx, z[m]);
    mx = row16_max(mx);
#pragma unroll
    for (int m = 0; m < EPT; ++m) psum[e0 + m] = router_exp(z[m] - mx);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    float acc = 0.0f;
    if (tl == 0)
      for (int e = 0; e < E; ++e) acc = acc + psum[e];
    S = __shfl(acc, tokbase, 64);
  }
  auto score = [&](float zz) { return SOFTMAX ? router_exp(zz - mx) / S : router_sigmoid(zz); };

  // group limit: each group's score is the sum of the scores of its group_score_topk first
  // experts in key order; the topk_group groups first by (score descending, group ascending) stay
  if (cfg.n_group > 1) {
    const int lpg = 16 / cfg.n_group;
    uint64_t thr = ~0ull;
    float gsum = 0.0f;
    for (int r = 0; r < cfg.group_score_topk; ++r) {
      const uint64_t b = seg_max(lane_best_below<EPT>(key, thr), lpg);
      gsum = gsum + score(key_logit(b));
      thr = b;
    }
    const int G = tl / lpg;
    int rank = 0;
    for (int h = 0; h < cfg.n_group; ++h) {
      const float sh = __shfl(gsum, tokbase + h * lpg, 64);
      rank += (sh > gsum || (sh == gsum && h < G)) ? 1 : 0;
    }
    if (rank >= cfg.topk_group) {
#pragma unroll
      for (int m = 0; m < EPT; ++m) key[m] = 0;
    }
  }

  // top-k: slot r is kept by lane r % 16 in entry r / 16
  uint64_t slot[4] = {0, 0, 0, 0};
  uint64_t thr = ~0ull;
#pragma unroll 1
  for (int r = 0; r < k; ++r) {
    const uint64_t b = seg_max(lane_best_below<EPT>(key, thr), 16);
    if ((r & 15) == tl) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((r >> 4) == q) slot[q] = b;
    }
    thr = b;
  }
  float sw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (16 * q < k && 16 * q + tl < k) sw[q] = score(key_logit(slot[q]));
  float d = 1.0f;
  if (cfg.renormalize) {
    d = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      for (int i = 0; i < 16 && 16 * q + i < k; ++i) d = d + __shfl(sw[q], tokbase + i, 64);
  }
  if (!live) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * q + tl;
    if (r < k) {
      const int e = key_expert(slot[q]);
      topk_idx[t * k + r] = e;
      topk_w[t * k + r] = cfg.renormalize ? sw[q] / d : sw[q];
      if (record) record[r * record_ld + t] = e;
    }
  }
}

template <int EPT, bool SOFTMAX>
__global__ __launch_bounds__(64 * WAVES) void route16_kernel(const float* __restrict__ logits, int64_t T,
                                                             moe_router_cfg cfg, int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ topk_w, int32_t* __restrict__ record,
                                                             int64_t record_ld) {
  __shared__ float psum[SOFTMAX ? FTOK : 1][SOFTMAX ? 16 * EPT : 1];
  const int tok = threadIdx.x / 16;
  const int64_t t = (int64_t)blockIdx.x * FTOK + tok;
  route_token16<EPT, SOFTMAX>(logits, t, t < T, cfg, topk_idx, topk_w, record, record_ld,
                              psum[SOFTMAX ? tok : 0]);
}

// The router (16 tokens per workgroup, as route16_kernel) and the 1x128 quantisation of x (RQ_U * 16
// blocks per workgroup) in one launch: the routing workgroups are spread through the grid, one at
// every rstride-th position, so that the latency-bound routing runs beside the HBM-bound
// quantisation instead of before it.  Two blocks per 16-lane group: per long-context chunk (8192
// tokens, H 6144) the launch measured 37.4 us against 41.0 us with 4 blocks, 39.4 with 8 and 58 with 16.
constexpr int RQ_U = 2;
template <int EPT, bool SOFTMAX, bool BF16, bool POW2>
__global__ __launch_bounds__(64 * WAVES) void route16_quant_kernel(
    const float* __restrict__ logits, int64_t T, moe_router_cfg cfg, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ record, int64_t record_ld, int64_t nroute, int64_t rstride,
    const void* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ xq, float* __restrict__ xs) {
  __shared__ float psum[SOFTMAX ? FTOK : 1][SOFTMAX ? 16 * EPT : 1];
  const int64_t i = blockIdx.x;
  int64_t qw;   // quantisation workgroup index, or -1 for a routing workgroup
  if (i < nroute * rstride) {
    if (i % rstride == 0) {
      const int tok = threadIdx.x / 16;
      const int64_t t = (i / rstride) * FTOK + tok;
      route_token16<EPT, SOFTMAX>(logits, t, t < T, cfg, topk_idx, topk_w, record, record_ld,
                                  psum[SOFTMAX ? tok : 0]);
      return;
    }
    qw = i - i / rstride - 1;
  } else {
    qw = i - nroute;
  }
  quant_1x128_pieces<BF16, POW2, RQ_U>(x, qw * (16 * RQ_U) + threadIdx.x / 16, 16, nblocks, threadIdx.x & 15, xq,
                                        xs);
}

template <int EPL>
__global__ __launch_bounds__(64 * WAVES) void replay_kernel(const float* __restrict__ logits, int64_t T,
                                                            moe_router_cfg cfg, const int32_t* __restrict__ replay,
                                                            int64_t replay_ld, int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w, int32_t* __restrict__ bad) {
  __shared__ float key_s[WAVES][64 * EPL];
  __shared__ float sc_s[WAVES][64 * EPL];
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const int64_t t = (int64_t)blockIdx.x * WAVES + wv;
  if (t >= T) return;
  const int E = cfg.num_experts, k = cfg.top_k;
  const int my_e = lane < k ? replay[lane * replay_ld + t] : 0;
  bool ok = my_e >= 0 && my_e < E;
  for (int q = 0; q < k; ++q) {
    const int oe = __shfl(my_e, q, 64);
    if (q < lane && oe == my_e) ok = false;
  }
  const bool all_ok = __ballot(lane < k && !ok) == 0;
  if (!all_ok) {
    if (lane < k) {
      topk_idx[t * k + lane] = -1;
      topk_w[t * k + lane] = 0.0f;
    }
    if (lane == 0 && bad) atomicAdd(bad, 1);
    return;
  }
  float my_s;
  if (cfg.score_fn == MOE_SCORE_SOFTMAX) {
    float z[EPL];
    token_scores<EPL>(logits + t * E, E, cfg.score_fn, lane, z, key_s[wv], sc_s[wv]);
    my_s = lane < k ? sc_s[wv][my_e] : 0.0f;
  } else {
    my_s = lane < k ? router_sigmoid(logits[t * E + my_e]) : 0.0f;
  }
  float w = my_s;
  if (cfg.renormalize) {
    float d = 0.0f;
    for (int r = 0; r < k; ++r) d = d + __shfl(my_s, r, 64);
    w = my_s / d;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = w;
  }
}

// Replay fused with the gate projection, for sigmoid routers: a token's weights depend only on the
// logits of its k recorded experts, so only those k dot products are computed (k/E of the gate
// work).  Lane (token, slot) walks its own chain: x[t,h] * wg[e,h] fma'd in ascending h from +0,
// then + bias[e] -- the chain of the gate projection, so each logit equals that kernel's output
// bit for bit.  Validation, weights and renormalisation follow the replay kernel.
template <bool BF16>
__global__ __launch_bounds__(256) void replay_gate_kernel(const void* __restrict__ xv, const float* __restrict__ wg,
                                                          const float* __restrict__ bias, int64_t T, int H,
                                                          moe_router_cfg cfg, const int32_t* __restrict__ replay,
                                                          int64_t replay_ld, int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w, int32_t* __restrict__ bad) {
  const int E = cfg.num_experts, k = cfg.top_k;
  const int tpw = 64 / k;   // tokens per wavefront
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tt = lane / k, j = lane - tt * k;
  const int64_t t = ((int64_t)blockIdx.x * 4 + wv) * tpw + tt;
  const bool live = tt < tpw && t < T;
  const int e = live ? replay[j * replay_ld + t] : 0;
  bool ok = e >= 0 && e < E;
  const int base = tt * k;
  for (int q = 0; q < k; ++q) {
    const int oe = __shfl(e, (base + q) & 63, 64);
    if (q < j && oe == e) ok = false;
  }
  const uint64_t badm = __ballot(live && !ok);
  const uint64_t mine = k == 64 ? ~0ull : (((1ull << k) - 1ull) << (base & 63));
  const bool tok_ok = (badm & mine) == 0;
  float z = 0.0f;
  if (live && tok_ok) {
    const float* wr = wg + (int64_t)e * H;
    if (BF16) {
      const uint16_t* xr = reinterpret_cast<const uint16_t*>(xv) + t * H;
#pragma unroll 4
      for (int h = 0; h < H; h += 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(xr + h);
        const float4 w0 = *reinterpret_cast<const float4*>(wr + h);
        const float4 w1 = *reinterpret_cast<const float4*>(wr + h + 4);
        z = __builtin_fmaf(__uint_as_float(u.x << 16), w0.x, z);
        z = __builtin_fmaf(__uint_as_float(u.x & 0xFFFF0000u), w0.y, z);
        z = __builtin_fmaf(__uint_as_float(u.y << 16), w0.z, z);
        z = __builtin_fmaf(__uint_as_float(u.y & 0xFFFF0000u), w0.w, z);
        z = __builtin_fmaf(__uint_as_float(u.z << 16), w1.x, z);
        z = __builtin_fmaf(__uint_as_float(u.z & 0xFFFF0000u), w1.y, z);
        z = __builtin_fmaf(__uint_as_float(u.w << 16), w1.z, z);
        z = __builtin_fmaf(__uint_as_float(u.w & 0xFFFF0000u), w1.w, z);
      }
    } else {
      const float* xr = reinterpret_cast<const float*>(xv) + t * H;
#pragma unroll 4
      for (int h = 0; h < H; h += 4) {
        const float4 a = *reinterpret_cast<const float4*>(xr + h);
        const float4 w = *reinterpret_cast<const float4*>(wr + h);
        z = __builtin_fmaf(a.x, w.x, z);
        z = __builtin_fmaf(a.y, w.y, z);
        z = __builtin_fmaf(a.z, w.z, z);
        z = __builtin_fmaf(a.w, w.w, z);
      }
    }
    if (bias) z = z + bias[e];
  }
  const float my_s = live && tok_ok ? router_sigmoid(z) : 0.0f;
  float w = my_s;
  if (cfg.renormalize) {
    float d = 0.0f;
    for (int q = 0; q < k; ++q) d = d + __shfl(my_s, (base + q) & 63, 64);
    w = my_s / d;
  }
  if (!live) return;
  if (tok_ok) {
    topk_idx[t * k + j] = e;
    topk_w[t * k + j] = w;
  } else {
    topk_idx[t * k + j] = -1;
    topk_w[t * k + j] = 0.0f;
    if (j == 0 && bad) atomicAdd(bad, 1);
  }
}

__global__ __launch_bounds__(256) void score_eval_kernel(const float* __restrict__ x, int64_t n, int score_fn,
                                                        float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  y[i] = score_fn == MOE_SCORE_SOFTMAX ? router_exp(x[i]) : router_sigmoid(x[i]);
}

int check_cfg(const moe_router_cfg* c) {
  if (!c) return MOE_ERR_NULL;
  const int E = c->num_experts, k = c->top_k;
  if (E < 1 || E > 1024 || k < 1 || k > 64 || k > E) return MOE_ERR_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_ARG;
  if (c->n_group > 1) {
    if (c->n_group > MAX_GROUPS || E % c->n_group != 0) return MOE_ERR_ARG;
    const int gs = E / c->n_group;
    if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_ARG;
    if (c->group_score_topk < 1 || c->group_score_topk > gs || c->group_score_topk > 8) return MOE_ERR_ARG;
    if (k > c->topk_group * gs) return MOE_ERR_ARG;
  } else if (c->n_group < 1) {
    return MOE_ERR_ARG;
  }
  return MOE_OK;
}

// experts per lane of the 16-lane router for this call, or 0 where it does not apply: E of 64, 128,
// 256 or 512, a group limit (if any) of 2, 4, 8 or 16 groups, 16-byte aligned logits
int fast_ept(const moe_router_cfg& c, const float* logits) {
  const int E = c.num_experts;
  if (E != 64 && E != 128 && E != 256 && E != 512) return 0;
  if (c.n_group > 1 && (c.n_group > 16 || 16 % c.n_group != 0)) return 0;
  if ((reinterpret_cast<uintptr_t>(logits) & 15) != 0) return 0;
  return E / 16;
}

}  // namespace

#define DISPATCH_EPT(EPT_RT, SOFTMAX_RT, BODY)                   \
  do {                                                           \
    if (SOFTMAX_RT) {                                            \
      constexpr bool SM = true;                                  \
      if ((EPT_RT) == 4) { constexpr int EPT = 4; BODY; }        \
      else if ((EPT_RT) == 8) { constexpr int EPT = 8; BODY; }   \
      else if ((EPT_RT) == 16) { constexpr int EPT = 16; BODY; } \
      else { constexpr int EPT = 32; BODY; }                     \
    } else {                                                     \
      constexpr bool SM = false;                                 \
      if ((EPT_RT) == 4) { constexpr int EPT = 4; BODY; }        \
      else if ((EPT_RT) == 8) { constexpr int EPT = 8; BODY; }   \
      else if ((EPT_RT) == 16) { constexpr int EPT = 16; BODY; } \
      else { constexpr int EPT = 32; BODY; }                     \
    }                                                            \
  } while (0)

#define DISPATCH_EPL(E, BODY)                  \
  do {                                         \
    if ((E) <= 64) {                           \
      constexpr int EPL = 1;                   \
      BODY;                                    \
    } else if ((E) <= 128) {                   \
      constexpr int EPL = 2;                   \
      BODY;                                    \
    } else if ((E) <= 256) {                   \
      constexpr int EPL = 4;                   \
      BODY;                                    \
    } else if ((E) <= 512) {                   \
      constexpr int EPL = 8;                   \
      BODY;                                    \
    } else {                                   \
      constexpr int EPL = 16;                  \
      BODY;                                    \
    }                                          \
  } while (0)

extern "C" int moe_route(const float* logits, int64_t T, const moe_router_cfg* cfg, int32_t* topk_idx, float* topk_w,
                         int32_t* record, int64_t record_ld, void* stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (T < 0 || T > (int64_t)INT32_MAX * WAVES) return MOE_ERR_SHAPE;
  if (record && record_ld < T) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
  const moe_router_cfg c = *cfg;
  hipStream_t st = as_stream(stream);
  const int ept = fast_ept(c, logits);
  if (ept) {
    const unsigned grid = (unsigned)ceil_div64(T, FTOK);
    DISPATCH_EPT(ept, c.score_fn == MOE_SCORE_SOFTMAX,
                 (route16_kernel<EPT, SM><<<grid, 64 * WAVES, 0, st>>>(logits, T, c, topk_idx, topk_w, record,
                                                                       record_ld)));
  } else {
    const unsigned grid = (unsigned)ceil_div64(T, WAVES);
    DISPATCH_EPL(c.num_experts, (route_kernel<EPL><<<grid, 64 * WAVES, 0, st>>>(logits, T, c, topk_idx, topk_w,
                                                                                 record, record_ld)));
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_route_quant(const float* logits, int64_t T, const moe_router_cfg* cfg, int32_t* topk_idx,
                               float* topk_w, int32_t* record, int64_t record_ld, const void* x, int x_dtype,
                               int32_t H, int32_t scale_mode, uint8_t* xq, float* xs, void* stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (T < 0 || T > (int64_t)INT32_MAX * WAVES) return MOE_ERR_SHAPE;
  if (H < 128 || H % 128 != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (scale_mode != MOE_SCALE_AMAX && scale_mode != MOE_SCALE_POW2) return MOE_ERR_ARG;
  if (record && record_ld < T) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w || !x || !xq || !xs) return MOE_ERR_NULL;
  const moe_router_cfg c = *cfg;
  const int64_t nblocks = T * (H / 128);
  hipStream_t st = as_stream(stream);
  const bool bf16 = x_dtype == MOE_BF16, pow2 = scale_mode == MOE_SCALE_POW2;
  const int ept = fast_ept(c, logits);
  if (ept) {
    const int64_t nroute = ceil_div64(T, FTOK), nquant = ceil_div64(nblocks, 16 * RQ_U);
    const int64_t grid = nroute + nquant;
    if (grid > INT32_MAX) return MOE_ERR_SHAPE;
    const int64_t rstride = grid / nroute;   // >= 1; routing workgroups at 0, rstride, 2 rstride, ...
#define RQ16_LAUNCH(B, P)                                                                                       \
  DISPATCH_EPT(ept, c.score_fn == MOE_SCORE_SOFTMAX,                                                            \
               (route16_quant_kernel<EPT, SM, B, P><<<(unsigned)grid, 64 * WAVES, 0, st>>>(                     \
                   logits, T, c, topk_idx, topk_w, record, record_ld, nroute, rstride, x, nblocks, xq, xs)))
    if (bf16 && pow2) RQ16_LAUNCH(true, true);
    else if (bf16) RQ16_LAUNCH(true, false);
    else if (pow2) RQ16_LAUNCH(false, true);
    else RQ16_LAUNCH(false, false);
#undef RQ16_LAUNCH
  } else {
    const int64_t nroute = ceil_div64(T, WAVES);
    const int64_t grid = nroute + ceil_div64(nblocks, QBLK);
    if (grid > INT32_MAX) return MOE_ERR_SHAPE;
#define RQ_LAUNCH(B, P)                                                                                          \
  DISPATCH_EPL(c.num_experts, (route_quant_kernel<EPL, B, P><<<(unsigned)grid, 64 * WAVES, 0, st>>>(             \
                                  logits, T, c, topk_idx, topk_w, record, record_ld, nroute, x, nblocks, xq, xs)))
    if (bf16 && pow2) RQ_LAUNCH(true, true);
    else if (bf16) RQ_LAUNCH(true, false);
    else if (pow2) RQ_LAUNCH(false, true);
    else RQ_LAUNCH(false, false);
#undef RQ_LAUNCH
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_replay_route(const float* logits, int64_t T, const moe_router_cfg* cfg, const int32_t* replay,
                                int64_t replay_ld, int32_t* topk_idx, float* topk_w, int32_t* bad_count,
                                void* stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (T < 0 || T > (int64_t)INT32_MAX * WAVES) return MOE_ERR_SHAPE;
  if (replay_ld < T) return MOE_ERR_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !replay || !topk_idx || !topk_w) return MOE_ERR_NULL;
  const moe_router_cfg c = *cfg;
  const unsigned grid = (unsigned)ceil_div64(T, WAVES);
  hipStream_t st = as_stream(stream);
  DISPATCH_EPL(c.num_experts, (replay_kernel<EPL><<<grid, 64 * WAVES, 0, st>>>(logits, T, c, replay, replay_ld,
                                                                                topk_idx, topk_w, bad_count)));
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_replay_gate(const void* x, int x_dtype, const float* wg, const float* bias, int64_t T, int32_t H,
                               const moe_router_cfg* cfg, const int32_t* replay, int64_t replay_ld, int32_t* topk_idx,
                               float* topk_w, int32_t* bad_count, void* stream) {
  const int rc = check_cfg(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_ARG;   // softmax weights need every logit
  if (T < 0 || H < 8 || H % 8 != 0 || T > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (replay_ld < T) return MOE_ERR_ARG;
  if (!x || !wg || !replay || !topk_idx || !topk_w) return MOE_ERR_NULL;
  const int tpw = 64 / cfg->top_k;
  const int64_t grid = ceil_div64(T, 4 * tpw);
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  if (x_dtype == MOE_BF16)
    replay_gate_kernel<true><<<(unsigned)grid, 256, 0, st>>>(x, wg, bias, T, H, *cfg, replay, replay_ld, topk_idx,
                                                            topk_w, bad_count);
  else
    replay_gate_kernel<false><<<(unsigned)grid, 256, 0, st>>>(x, wg, bias, T, H, *cfg, replay, replay_ld, topk_idx,
                                                             topk_w, bad_count);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" int moe_router_score_eval(const float* x, int64_t n, int score_fn, float* y, void* stream) {
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_ARG;
  if (n < 0 || ceil_div64(n, 256) > INT32_MAX) return MOE_ERR_SHAPE;
  if (n == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_NULL;
  score_eval_kernel<<<(unsigned)ceil_div64(n, 256), 256, 0, as_stream(stream)>>>(x, n, score_fn, y);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
