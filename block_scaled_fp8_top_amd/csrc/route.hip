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

}  // namespace

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
  const unsigned grid = (unsigned)ceil_div64(T, WAVES);
  hipStream_t st = as_stream(stream);
  DISPATCH_EPL(c.num_experts, (route_kernel<EPL><<<grid, 64 * WAVES, 0, st>>>(logits, T, c, topk_idx, topk_w,
                                                                               record, record_ld)));
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
  const int64_t nroute = ceil_div64(T, WAVES);
  const int64_t nblocks = T * (H / 128);
  const int64_t grid = nroute + ceil_div64(nblocks, QBLK);
  if (grid > INT32_MAX) return MOE_ERR_SHAPE;
  hipStream_t st = as_stream(stream);
  const bool bf16 = x_dtype == MOE_BF16, pow2 = scale_mode == MOE_SCALE_POW2;
#define RQ_LAUNCH(B, P)                                                                                          \
  DISPATCH_EPL(c.num_experts, (route_quant_kernel<EPL, B, P><<<(unsigned)grid, 64 * WAVES, 0, st>>>(             \
                                  logits, T, c, topk_idx, topk_w, record, record_ld, nroute, x, nblocks, xq, xs)))
  if (bf16 && pow2) RQ_LAUNCH(true, true);
  else if (bf16) RQ_LAUNCH(true, false);
  else if (pow2) RQ_LAUNCH(false, true);
  else RQ_LAUNCH(false, false);
#undef RQ_LAUNCH
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
