/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for the block-scaled FP8
 * Mixture-of-Experts layer (router or router replay, dispatch, 1x128 / 128x128 FP8 e4m3
 * quantisation, grouped expert GEMMs with SwiGLU, weighted combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header, table or constant generator with the HIP library.
 *
 * Sources.  The method is the MoE layer of "RL at 1T Scale: prime-rl Performance Deep Dive"
 * (Prime Intellect blog): routing decisions recorded at inference and replayed on the trainer
 * (section "Router replay"), tokens dispatched to and combined from their experts (sections
 * "Wide EP" and "Parallelism / EP"), and block-scaled FP8 as proposed by DeepSeek V3 for both
 * inference and training (sections "FP8 inference" and "FP8 training").  The pages give no
 * formula for any step; every numeric detail below is a stated reading (router function,
 * block shapes, scale rule, rounding, summation orders) and is listed with its reason in the
 * repository's design notes.  Each function says which reading it implements.
 *
 * Precision.  Where a floating-point result decides an integer (routing indices, FP8 codes,
 * scales that are compared bit for bit) the oracle computes in fp32 with a pinned operation
 * order, IEEE round-to-nearest-even and no contraction (build with -ffp-contract=off; fused
 * multiply-adds are written as explicit fmaf calls).  Everything that is only compared within
 * a tolerance (GEMMs, SwiGLU, combine) is computed in fp64.
 *
 * Threads: OpenMP over independent tokens / rows / blocks only; no result depends on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------------------------
 * FP8 E4M3 (OCP "E4M3FN"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  No
 * infinities; S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448; the
 * smallest subnormal is 2^-9.  DeepSeek V3's recipe (cited by the blog's FP8 training
 * section) stores activations and weights in this format.
 * ------------------------------------------------------------------------------------- */

/* Exact value of a code, from the format definition. */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);            /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(8.0 + m, e - 10);          /* (1 + m/8) * 2^(e-7)   */
  return sign ? -v : v;
}

/* Round-to-nearest-even encode with saturation to +-448; the sign of zero is kept.
 * Precondition: v is finite. */
uint8_t orc_e4m3_encode(float v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (a >= 448.0) return sign | 0x7E;   /* [448,464) rounds to 448; beyond that saturates */
  if (a < 0.015625) {                   /* below the smallest normal 2^-6: grid step 2^-9  */
    double m = rint(a * 512.0);         /* exact scaling, then round half to even          */
    return sign | (uint8_t)m;           /* m == 8 is code 0x08 = 2^-6, the smallest normal */
  }
  int e;
  double f = frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1)  */
  e -= 1;                               /* a = (2f) * 2^e, 2f in [1, 2) */
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m == 8.0) { m = 0.0; e += 1; }
  return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* ---------------------------------------------------------------------------------------
 * Pinned exponential and sigmoid, built only from IEEE fp32 operations so that two
 * implementations following the same steps agree bit for bit.
 * Method: Cody & Waite (1980) argument reduction x = n ln2 + r with ln2 split into a short
 * high part (exact products n*hi for |n| <= 127) and a low part, a degree-6 Taylor polynomial
 * for e^r on |r| <= ln2/2 evaluated by Horner's rule with fused multiply-adds, and an exact
 * scaling by 2^n.  The input is clamped to [-86, 88] so that the result is always a normal,
 * finite fp32 number.
 * ------------------------------------------------------------------------------------- */
static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

float orc_exp(float x) {
  const float log2e = 0x1.715476p+0f;
  const float ln2_hi = 0x1.62e400p-1f, ln2_lo = 0x1.7f7d1cp-20f;
  if (x < -86.0f) x = -86.0f;
  if (x > 88.0f) x = 88.0f;
  float n = rintf(x * log2e);
  float r = fmaf(-n, ln2_hi, x);
  r = fmaf(-n, ln2_lo, r);
  float p = 0x1.6c16c2p-10f;            /* 1/720 */
  p = fmaf(p, r, 0x1.111112p-7f);       /* 1/120 */
  p = fmaf(p, r, 0x1.555556p-5f);       /* 1/24  */
  p = fmaf(p, r, 0x1.555556p-3f);       /* 1/6   */
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return p * f32_from_bits((uint32_t)((int)n + 127) << 23);
}

float orc_sigmoid(float z) { return 1.0f / (1.0f + orc_exp(-z)); }

void orc_exp_array(const float* x, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_exp(x[i]);
}
void orc_sigmoid_array(const float* x, int64_t n, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoid(x[i]);
}

/* ---------------------------------------------------------------------------------------
 * Gate logits: z[t,e] = sum_h x[t,h] * Wg[e,h] (+ b[e]).  The sum is a single fp32 chain of
 * fused multiply-adds in ascending h starting from +0, then one fp32 add of the bias.  The
 * fixed order is what lets two implementations agree on the routing indices bit for bit.
 * x is given as fp32 (bf16 activations widen to fp32 exactly).
 * ------------------------------------------------------------------------------------- */
void orc_gate_logits(const float* x, const float* wg, const float* bias, int64_t T, int32_t H,
                     int32_t E, float* z) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int32_t h = 0; h < H; ++h) acc = fmaf(x[t * (int64_t)H + h], wg[(int64_t)e * H + h], acc);
      if (bias) acc = acc + bias[e];
      z[t * (int64_t)E + e] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------------------
 * Router.  For one token with logits z[0..E):
 *   scores  softmax: p_e = exp(z_e - max z) / S, S = fp32 sum of exp(z_e - max z) in
 *                    ascending e;   sigmoid: s_e = 1 / (1 + exp(-z_e)).
 *   groups  if n_group > 1 the experts form n_group contiguous groups; a group's score is the
 *           fp32 sum of the scores of its top `group_score_topk` experts taken in selection
 *           order; the `topk_group` best groups are kept (ties: lower group index).
 *   top-k   among kept experts, by key z descending, ties to the lower expert index; slot j
 *           holds the j-th best.
 *   weights w_j = score of slot j; with renormalisation w_j = score_j / sum_j' score_j' with
 *           the denominator summed in slot order.  No extra routed scaling factor.
 * ------------------------------------------------------------------------------------- */
typedef struct {
  int32_t num_experts, top_k, score_fn, renormalize, n_group, topk_group, group_score_topk;
} orc_router_cfg;

enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };

/* strict "a ranks before b" on (key desc, index asc) */
static int ranks_before(float za, int a, float zb, int b) { return za > zb || (za == zb && a < b); }

static void token_scores(const float* z, int E, int score_fn, float* score) {
  if (score_fn == ORC_SOFTMAX) {
    float m = z[0];
    for (int e = 1; e < E; ++e) if (z[e] > m) m = z[e];
    float S = 0.0f;
    for (int e = 0; e < E; ++e) { score[e] = orc_exp(z[e] - m); S = S + score[e]; }
    for (int e = 0; e < E; ++e) score[e] = score[e] / S;
  } else {
    for (int e = 0; e < E; ++e) score[e] = orc_sigmoid(z[e]);
  }
}

static void route_token(const float* z, const orc_router_cfg* c, float* score, unsigned char* allowed,
                        int32_t* idx, float* w) {
  int E = c->num_experts, k = c->top_k;
  token_scores(z, E, c->score_fn, score);
  for (int e = 0; e < E; ++e) allowed[e] = 1;
  if (c->n_group > 1) {
    int G = c->n_group, gs = E / G;
    float gscore[1024];
    unsigned char taken[1024];
    for (int g = 0; g < G; ++g) {
      /* top group_score_topk experts of the group by key, summed in that order */
      for (int e = 0; e < gs; ++e) taken[e] = 0;
      float sum = 0.0f;
      for (int r = 0; r < c->group_score_topk; ++r) {
        int best = -1;
        for (int e = 0; e < gs; ++e) {
          int ge = g * gs + e;
          if (taken[e]) continue;
          if (best < 0 || ranks_before(z[ge], ge, z[g * gs + best], g * gs + best)) best = e;
        }
        taken[best] = 1;
        sum = sum + score[g * gs + best];
      }
      gscore[g] = sum;
    }
    unsigned char keep[1024];
    for (int g = 0; g < G; ++g) keep[g] = 0;
    for (int r = 0; r < c->topk_group; ++r) {
      int best = -1;
      for (int g = 0; g < G; ++g) {
        if (keep[g]) continue;
        if (best < 0 || gscore[g] > gscore[best]) best = g;   /* ties: lower index stays */
      }
      keep[best] = 1;
    }
    for (int e = 0; e < E; ++e) allowed[e] = keep[e / gs];
  }
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (!allowed[e]) continue;
      if (best < 0 || ranks_before(z[e], e, z[best], best)) best = e;
    }
    idx[j] = best;
    allowed[best] = 0;
  }
  float denom = 0.0f;
  for (int j = 0; j < k; ++j) denom = denom + score[idx[j]];
  for (int j = 0; j < k; ++j) w[j] = c->renormalize ? score[idx[j]] / denom : score[idx[j]];
}

/* Route T tokens.  idx, w: [T,k].  If record != NULL, record[j*record_ld + t] = idx[t,j]
 * (one layer of the [num_layers, top_k, seq_len] routing payload). */
void orc_route(const float* z, int64_t T, const orc_router_cfg* c, int32_t* idx, float* w,
               int32_t* record, int64_t record_ld) {
  int E = c->num_experts, k = c->top_k;
#pragma omp parallel
  {
    float* score = (float*)malloc(sizeof(float) * E);
    unsigned char* allowed = (unsigned char*)malloc(E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      route_token(z + t * E, c, score, allowed, idx + t * k, w + t * k);
      if (record)
        for (int j = 0; j < k; ++j) record[j * record_ld + t] = idx[t * k + j];
    }
    free(score);
    free(allowed);
  }
}

/* Replay: indices come from payload[j*replay_ld + t] unchanged; weights are recomputed from
 * the current logits with the configured score function and normalisation.  A token whose
 * recorded indices are out of range or repeated is routed nowhere (index -1, weight 0) and
 * counted.  Returns the number of such tokens. */
int64_t orc_replay_route(const float* z, int64_t T, const orc_router_cfg* c, const int32_t* replay,
                         int64_t replay_ld, int32_t* idx, float* w) {
  int E = c->num_experts, k = c->top_k;
  int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
  {
    float* score = (float*)malloc(sizeof(float) * E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      int ok = 1;
      for (int j = 0; j < k; ++j) {
        int32_t e = replay[j * replay_ld + t];
        if (e < 0 || e >= E) ok = 0;
        for (int j2 = 0; j2 < j; ++j2)
          if (replay[j2 * replay_ld + t] == e) ok = 0;
      }
      if (!ok) {
        for (int j = 0; j < k; ++j) { idx[t * k + j] = -1; w[t * k + j] = 0.0f; }
        bad += 1;
        continue;
      }
      token_scores(z + t * E, E, c->score_fn, score);
      float denom = 0.0f;
      for (int j = 0; j < k; ++j) denom = denom + score[replay[j * replay_ld + t]];
      for (int j = 0; j < k; ++j) {
        int32_t e = replay[j * replay_ld + t];
        idx[t * k + j] = e;
        w[t * k + j] = c->renormalize ? score[e] / denom : score[e];
      }
    }
    free(score);
  }
  return bad;
}

/* ---------------------------------------------------------------------------------------
 * Block quantisation (DeepSeek-V3-style fine-grained scaling): x is [batch][rows][cols] fp32;
 * blocks are block_rows x 128 (1x128 for activations, 128x128 for weights).  Per block:
 * amax = max |x| (exact), s = amax / 448 (IEEE fp32 division; s = 1 for an all-zero block) or, with
 * pow2, orc_pow2_scale(amax); q = e4m3(x / s) with x / s an IEEE fp32 division.
 * scales: [batch][rows/block_rows][cols/128].
 * ------------------------------------------------------------------------------------- */
/* Power-of-two scale (for the hardware-scaled MFMA, whose E8M0 block scales are powers of two):
 * the smallest power of two at or above t = amax / 448 (IEEE fp32 division), and at least 2^-127
 * (the smallest E8M0 value; also the result when t underflows to 0); 1 for an all-zero block.  frexpf writes t = m * 2^e with m in
 * [0.5, 1): t is itself a power of two exactly when m == 0.5. */
float orc_pow2_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float t = amax / 448.0f;
  int e;
  float m = frexpf(t, &e);
  float s = m == 0.5f ? t : m == 0.0f ? 0.0f : ldexpf(1.0f, e);   /* t == 0 when amax/448 underflows */
  float lo = ldexpf(1.0f, -127);
  return s < lo ? lo : s;
}

void orc_quant_block(const float* x, int64_t batch, int64_t rows, int32_t cols, int32_t block_rows,
                     int32_t pow2, uint8_t* q, float* scales) {
  int64_t rb_n = rows / block_rows, cb_n = cols / 128;
  int64_t nblocks = batch * rb_n * cb_n;
#pragma omp parallel for schedule(static)
  for (int64_t blk = 0; blk < nblocks; ++blk) {
    int64_t b = blk / (rb_n * cb_n), rb = (blk / cb_n) % rb_n, cb = blk % cb_n;
    const float* base = x + b * rows * cols;
    uint8_t* qbase = q + b * rows * cols;
    float amax = 0.0f;
    for (int64_t r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
      for (int64_t c = cb * 128; c < cb * 128 + 128; ++c) {
        float a = fabsf(base[r * cols + c]);
        if (a > amax) amax = a;
      }
    float s = pow2 ? orc_pow2_scale(amax) : (amax == 0.0f ? 1.0f : amax / 448.0f);
    for (int64_t r = rb * block_rows; r < (rb + 1) * block_rows; ++r)
      for (int64_t c = cb * 128; c < cb * 128 + 128; ++c)
        qbase[r * cols + c] = orc_e4m3_encode(base[r * cols + c] / s);
    scales[blk] = s;
  }
}

/* ---------------------------------------------------------------------------------------
 * Dispatch: a stable counting sort of the flattened [T,k] expert ids.
 *   counts[e]  = number of (t,j) with idx[t,j] == e   (slots with idx -1 are skipped)
 *   offsets    = exclusive scan of counts; groups = E (+1 shared expert appended last)
 *   dest_row[t,j] = offsets[e] + number of earlier (t',j') (row-major order) with expert e
 *   src_token[row] = token whose copy lands in that row
 * The shared expert (append_shared) is group E with one row per token, in token order.
 * offsets has groups+1 entries.
 * ------------------------------------------------------------------------------------- */
void orc_dispatch(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t append_shared,
                  int32_t* counts, int32_t* offsets, int32_t* dest_row, int32_t* src_token) {
  int32_t G = E + (append_shared ? 1 : 0);
  for (int32_t g = 0; g < G; ++g) counts[g] = 0;
  for (int64_t i = 0; i < T * k; ++i)
    if (idx[i] >= 0) counts[idx[i]] += 1;
  if (append_shared) counts[E] = (int32_t)T;
  offsets[0] = 0;
  for (int32_t g = 0; g < G; ++g) offsets[g + 1] = offsets[g] + counts[g];
  int32_t* fill = (int32_t*)calloc(G, sizeof(int32_t));
  for (int64_t i = 0; i < T * k; ++i) {
    int32_t e = idx[i];
    if (e < 0) { dest_row[i] = -1; continue; }
    int32_t row = offsets[e] + fill[e]++;
    dest_row[i] = row;
    src_token[row] = (int32_t)(i / k);
  }
  if (append_shared)
    for (int64_t t = 0; t < T; ++t) src_token[offsets[E] + t] = (int32_t)t;
  free(fill);
}

/* Row permutation: out[row] = in[src_token[row]] for byte rows of width `row_bytes`. */
void orc_permute_rows(const uint8_t* in, const int32_t* src_token, int64_t rows, int64_t row_bytes,
                      uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    memcpy(out + r * row_bytes, in + (int64_t)src_token[r] * row_bytes, (size_t)row_bytes);
}

/* ---------------------------------------------------------------------------------------
 * Dequantisation to fp64: value(q) * s is exact in fp64 (<= 4 significant bits times 24).
 * a: [M][K] codes with 1x128 scales as [M][K/128];  b: [N][K] codes with 128x128 scales as
 * [N/128][K/128].
 * ------------------------------------------------------------------------------------- */
void orc_dequant_act(const uint8_t* a, const float* as, int64_t M, int32_t K, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int32_t k = 0; k < K; ++k)
      out[m * K + k] = orc_e4m3_value(a[m * K + k]) * (double)as[m * (K / 128) + k / 128];
}

void orc_dequant_weight(const uint8_t* b, const float* bs, int32_t N, int32_t K, double* out) {
#pragma omp parallel for schedule(static)
  for (int32_t n = 0; n < N; ++n)
    for (int32_t k = 0; k < K; ++k)
      out[(int64_t)n * K + k] =
          orc_e4m3_value(b[(int64_t)n * K + k]) * (double)bs[(n / 128) * (K / 128) + k / 128];
}

/* Block-scaled GEMM in its defining form: out[m][n] = sum over 128-wide K blocks kb of
 * (sA[m,kb] * sB[n/128,kb]) * (sum_{k in kb} value(a[m,k]) * value(b[n,k])), all in fp64.
 * Equal to the dequantise-then-multiply product up to fp64 rounding; kept as a self-check. */
void orc_gemm_block_form(const uint8_t* a, const float* as, int64_t M, const uint8_t* b,
                         const float* bs, int32_t N, int32_t K, double* out) {
  int32_t KB = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; ++m)
    for (int32_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int32_t kb = 0; kb < KB; ++kb) {
        double part = 0.0;
        for (int32_t k = kb * 128; k < kb * 128 + 128; ++k)
          part += orc_e4m3_value(a[m * K + k]) * orc_e4m3_value(b[(int64_t)n * K + k]);
        acc += part * ((double)as[m * KB + kb] * (double)bs[(n / 128) * KB + kb]);
      }
      out[m * N + n] = acc;
    }
}

/* ---------------------------------------------------------------------------------------
 * FP4 weights (the 4-bit analogue of the block-scaled recipe; the pages name NVFP4 only as
 * future work, so the format here is the OCP microscaling one the MI355X matrix cores take):
 * OCP FP4 E2M1 elements -- 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
 * 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6 for codes 0..7; no infinities or NaN -- in 1x32
 * blocks along K, each with a power-of-two scale s = the smallest power of two at or above
 * fl32(amax / 6), at least 2^-127 (1 for an all-zero block), stored as its E8M0 exponent code
 * (the fp32 exponent field; 2^-127 is code 0).  q = e2m1(x / s), round to nearest with ties to
 * the even code, saturating at 6, sign of zero kept.  Two codes per byte, element 2i in the low
 * nibble.
 * ------------------------------------------------------------------------------------- */
double orc_e2m1_value(uint8_t code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[code & 7];
  return (code & 8) ? -v : v;
}

/* nearest magnitude, ties to the even code (the midpoints 0.25, 0.75, ... go to codes 0, 2, 2, 4, 4, 6, 6) */
uint8_t orc_e2m1_encode(float v) {
  uint8_t sign = signbit(v) ? 8 : 0;
  double a = fabs((double)v);
  uint8_t c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return sign | c;
}

void orc_e2m1_encode_array(const float* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(v[i]);
}

/* the block scale of a 1x32 FP4 block with largest magnitude amax */
float orc_fp4_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float t = amax / 6.0f;
  int e;
  float m = frexpf(t, &e);
  float s = m == 0.5f ? t : m == 0.0f ? 0.0f : ldexpf(1.0f, e);
  float lo = ldexpf(1.0f, -127);
  return s < lo ? lo : s;
}

/* x [rows][cols] fp32 -> q [rows][cols/2] packed codes, e8 [rows][cols/32] E8M0 scale codes */
void orc_quant_mxfp4(const float* x, int64_t rows, int32_t cols, uint8_t* q, uint8_t* e8) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t b = 0; b < cols / 32; ++b) {
      const float* v = x + r * cols + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      float s = orc_fp4_scale(amax);
      int e;
      frexpf(s, &e);                       /* s = 0.5 * 2^e, i.e. 2^(e-1) */
      e8[r * (cols / 32) + b] = (uint8_t)(e - 1 + 127);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = orc_e2m1_encode(v[i] / s), hi = orc_e2m1_encode(v[i + 1] / s);
        q[r * (cols / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
}

/* fp64 value of packed FP4 weights [N][K/2] with E8M0 scales [N][K/32] */
void orc_dequant_mxfp4(const uint8_t* q, const uint8_t* e8, int64_t N, int32_t K, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int32_t k = 0; k < K; ++k) {
      uint8_t byte = q[n * (K / 2) + k / 2];
      uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
      out[n * K + k] = orc_e2m1_value(code) * ldexp(1.0, (int)e8[n * (K / 32) + k / 32] - 127);
    }
}
