// Backward of the router gate projection z = x Wg^T (+ b), fp32:
//   dx[t,h]  = dx_in[t,h] + sum_e dz[t,e] Wg[e,h]      (then one rounding to the dx dtype)
//   dWg[e,h] = sum_t dz[t,e] x[t,h]
//   db[e]    = sum_t dz[t,e]
// The router runs in fp32 on the vector ALUs in the forward, and so does its backward.  Both
// products are C = op(A) B with B [K,N] N-contiguous (Wg for dx, x for dWg): one kernel, A
// either row-major [M,K] (dz for dx) or stored transposed as [K,M] (dz for dWg).  128 x 128 output
// tiles, 256 threads with 8 x 8 outputs each, K staged through LDS 8 at a time with the next
// slice's global loads in flight.  dWg's long K (the tokens) is split into S fixed slices whose
// partial products land in the caller's workspace and are summed in slice order, so the result
// is deterministic.
#include <algorithm>

#include "common.h"

namespace {

constexpr int TB = 128, KC = 8, NTH = 256;

// C tile (m0, n0) of op(A) B over k in [k0, k1); A_T: A stored [K, M]; out: fp32 partial (OUT 0),
// or dx (OUT 1: + dx_in, stored fp32 or bf16).  asum (OUT 0 only, may be null): the first column
// of workgroups also writes the slice's row sums of op(A) (sum over k of A[m][k], k ascending).
template <bool A_T, bool B_BF16, bool O_BF16, int OUT>
__global__ __launch_bounds__(NTH) void gemm_kn_kernel(const float* __restrict__ a, const void* __restrict__ b,
                                                      int64_t M, int N, int64_t K, int64_t ksplit,
                                                      const float* __restrict__ c_in, void* __restrict__ c,
                                                      float* __restrict__ asum) {
  __shared__ __attribute__((aligned(16))) float as[2][KC][TB];
  __shared__ __attribute__((aligned(16))) float bs[2][KC][TB];
  const int tid = threadIdx.x;
  const int tm = tid / 16, tn = tid % 16;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const int n0 = blockIdx.x * TB;
  const int64_t k0 = (int64_t)blockIdx.z * ksplit;
  const int64_t k1 = std::min<int64_t>(K, k0 + ksplit);
  // staging: each thread brings 4 A values and 4 B values per slice
  float ra[4], rb[4];
  auto load = [&](int64_t kk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + NTH * i;   // 0 .. 1023
      if (A_T) {                     // A[k][m]: 128 consecutive m per k row
        const int kr = e / TB, mc = e % TB;
        const int64_t kg = kk + kr, mg = m0 + mc;
        ra[i] = (kg < k1 && mg < M) ? a[kg * M + mg] : 0.0f;
      } else {                       // A[m][k]: 8 consecutive k per m row
        const int mr = e / KC, kc = e % KC;
        const int64_t kg = kk + kc, mg = m0 + mr;
        ra[i] = (kg < k1 && mg < M) ? a[mg * K + kg] : 0.0f;
      }
      const int kr = e / TB, nc = e % TB;
      const int64_t kg = kk + kr;
      const int ng = n0 + nc;
      if (kg < k1 && ng < N) {
        if (B_BF16) rb[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(b)[kg * N + ng]);
        else rb[i] = reinterpret_cast<const float*>(b)[kg * N + ng];
      } else {
        rb[i] = 0.0f;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + NTH * i;
      if (A_T) as[buf][e / TB][e % TB] = ra[i];
      else as[buf][e % KC][e / KC] = ra[i];
      bs[buf][e / TB][e % TB] = rb[i];
    }
  };
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  float rsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bool sums = OUT == 0 && asum != nullptr && blockIdx.x == 0 && tn == 0;
  int buf = 0;
  if (k0 < k1) {
    load(k0);
    store(0);
  }
  __syncthreads();
  for (int64_t kk = k0; kk < k1; kk += KC) {
    const bool more = kk + KC < k1;
    if (more) load(kk + KC);
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      const float4 a0 = *reinterpret_cast<const float4*>(&as[buf][q][tm * 8]);
      const float4 a1 = *reinterpret_cast<const float4*>(&as[buf][q][tm * 8 + 4]);
      const float4 b0 = *reinterpret_cast<const float4*>(&bs[buf][q][tn * 8]);
      const float4 b1 = *reinterpret_cast<const float4*>(&bs[buf][q][tn * 8 + 4]);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
      if (sums) {
#pragma unroll
        for (int i = 0; i < 8; ++i) rsum[i] = rsum[i] + av[i];
      }
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  if (sums) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (m0 + tm * 8 + i < M) asum[(int64_t)blockIdx.z * M + m0 + tm * 8 + i] = rsum[i];
  }
  // outputs: rows m0 + tm*8 + i, columns n0 + tn*8 .. +7 (N % 8 == 0 is required by the host)
  const int nc = n0 + tn * 8;
  if (nc >= N) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + tm * 8 + i;
    if (m >= M) break;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = acc[i][j];
    if (OUT == 0) {
      float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + ((int64_t)blockIdx.z * M + m) * N + nc);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      if (c_in) {
        const float4* ci = reinterpret_cast<const float4*>(c_in + m * N + nc);
        const float4 p = ci[0], q = ci[1];
        v[0] = p.x + v[0]; v[1] = p.y + v[1]; v[2] = p.z + v[2]; v[3] = p.w + v[3];
        v[4] = q.x + v[4]; v[5] = q.y + v[5]; v[6] = q.z + v[6]; v[7] = q.w + v[7];
      }
      if (O_BF16) {
        uint32_t p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) p[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(c) + m * N + nc) = make_uint4(p[0], p[1], p[2], p[3]);
      } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + m * N + nc);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  }
}

// dWg = sum of the S slice partials in slice order; db[e] = sum of the S slice sums of dz[:, e]
// in slice order (within a slice the tokens were summed in order)
__global__ __launch_bounds__(256) void reduce_slices_kernel(const float* __restrict__ part, int S, int64_t MN,
                                                            float* __restrict__ out, const float* __restrict__ psum,
                                                            int E, float* __restrict__ db) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < MN) {
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(int64_t)s * MN + i];
    out[i] = v;
  }
  if (db && i < E) {
    float v = psum[i];
    for (int s = 1; s < S; ++s) v += psum[(int64_t)s * E + i];
    db[i] = v;
  }
}

// token slices of dWg: about 64 tokens each for short batches (enough workgroups to fill the
// chip), at most 16 (the partials are re-read once by the reduction)
int gate_bwd_slices(int64_t T) { return (int)std::max<int64_t>(1, std::min<int64_t>(16, ceil_div64(T, 64))); }

}  // namespace

extern "C" size_t moe_gate_backward_workspace(int64_t T, int32_t E, int32_t H) {
  if (T < 0 || E < 1 || H < 8) return 0;
  return (size_t)gate_bwd_slices(T) * ((size_t)E * (size_t)H + (size_t)E) * sizeof(float);
}

extern "C" int moe_gate_backward(const float* dz, const void* x, int x_dtype, const float* wg, int64_t T, int32_t H,
                                 int32_t E, const float* dx_in, void* dx, int dx_dtype, float* dwg, float* db,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || E < 1 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if ((x_dtype != MOE_F32 && x_dtype != MOE_BF16) || (dx_dtype != MOE_F32 && dx_dtype != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!dz || !x || !wg || !dx || !dwg) return MOE_ERR_NULL;
  if ((int64_t)E * H > INT32_MAX || T > INT32_MAX) return MOE_ERR_SHAPE;
  const int S = gate_bwd_slices(T);
  const size_t need = moe_gate_backward_workspace(T, E, H);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  // dx = dx_in + dz Wg: M = T, N = H, K = E, A = dz row-major, B = Wg [E, H]
  {
    const dim3 grid((unsigned)ceil_div64(H, TB), (unsigned)ceil_div64(T, TB), 1);
    if (dx_dtype == MOE_BF16)
      gemm_kn_kernel<false, false, true, 1><<<grid, NTH, 0, st>>>(dz, wg, T, H, E, E, dx_in, dx, nullptr);
    else
      gemm_kn_kernel<false, false, false, 1><<<grid, NTH, 0, st>>>(dz, wg, T, H, E, E, dx_in, dx, nullptr);
    MOE_CHECK_LAUNCH();
  }
  // dWg = dz^T x: M = E, N = H, K = T, A = dz stored [T, E], B = x [T, H]; S slices of K
  {
    const int64_t ks = ceil_div64(ceil_div64(T, S), KC) * KC;
    const dim3 grid((unsigned)ceil_div64(H, TB), (unsigned)ceil_div64(E, TB), (unsigned)S);
    const int64_t MN = (int64_t)E * H;
    float* part = reinterpret_cast<float*>(workspace);
    float* psum = part + (int64_t)S * MN;
    if (x_dtype == MOE_BF16)
      gemm_kn_kernel<true, true, false, 0><<<grid, NTH, 0, st>>>(dz, x, E, H, T, ks, nullptr, part, psum);
    else
      gemm_kn_kernel<true, false, false, 0><<<grid, NTH, 0, st>>>(dz, x, E, H, T, ks, nullptr, part, psum);
    MOE_CHECK_LAUNCH();
    reduce_slices_kernel<<<(unsigned)ceil_div64(std::max<int64_t>(MN, E), 256), 256, 0, st>>>(part, S, MN, dwg, psum,
                                                                                              E, db);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}
