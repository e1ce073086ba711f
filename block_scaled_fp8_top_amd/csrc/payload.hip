// Router-replay payload codec: fixed-width bit packing of routing indices, and its transport to and
// from pinned host memory ("RL at 1T Scale: prime-rl Performance Deep Dive", section "Router
// replay": the [num_layers, top_k, seq_len] routing payload runs to tens of Gbps and hundreds of GB
// and is handled as an opaque tensor by tensor operations only).
//
// Format: b = max(1, ceil(log2 E)) bits per index; index i occupies bits [i*b, (i+1)*b) of a
// little-endian bit stream, least significant bit first, zero-padded to whole groups of 32 indices.
// A group of 32 indices is exactly b 32-bit words, so group g is words [g*b, (g+1)*b) and no word
// is shared between groups.
//
// Kernels: pack takes one thread per group of 32 indices (128 bytes of int32 in eight 16-byte
// loads, b packed words out in 16-, 8- or 4-byte pieces); unpack takes one thread per 4 indices so
// that its int32 stores, the larger side, are fully coalesced.  The width is a template parameter,
// so every shift is a constant.  HBM-bound: 4 + b/8 bytes per index.
#include <algorithm>

#include "common.h"

namespace {

constexpr int PW = 256;          // threads per workgroup (one 32-index group each per iteration)

int payload_bits(int32_t E) {
  int b = 1;
  while ((1 << b) < E) ++b;
  return b;
}

// store the B words of one group (16-byte pieces when B is a multiple of 4)
template <int B>
__device__ __forceinline__ void store_words(uint32_t* __restrict__ dst, const uint32_t (&w)[B]) {
  if (B % 4 == 0) {
#pragma unroll
    for (int i = 0; i < B; i += 4) *reinterpret_cast<uint4*>(dst + i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
  } else if (B % 2 == 0) {
#pragma unroll
    for (int i = 0; i < B; i += 2) *reinterpret_cast<uint2*>(dst + i) = make_uint2(w[i], w[i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) dst[i] = w[i];
  }
}

// one thread per group of 32 indices: 128 bytes in (8 x 16-byte loads), B words out
template <int B>
__global__ __launch_bounds__(PW) void payload_pack_kernel(const int32_t* __restrict__ idx, int64_t n, int E,
                                                          uint32_t* __restrict__ out, int32_t* __restrict__ bad) {
  const int64_t ngroups = (n + 31) / 32;
  int nbad = 0;
  for (int64_t g = (int64_t)blockIdx.x * PW + threadIdx.x; g < ngroups; g += (int64_t)gridDim.x * PW) {
    const int64_t first = g * 32;
    int v[32];
    if (first + 32 <= n) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int4 t = *reinterpret_cast<const int4*>(idx + first + 4 * q);
        v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = first + j < n ? idx[first + j] : 0;
    }
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (v[j] < 0 || v[j] >= E) ++nbad;   // padding entries are 0, always in range
      const uint32_t c = (uint32_t)v[j] & ((1u << B) - 1u);
      const int pos = j * B, wi = pos >> 5, sh = pos & 31;
      w[wi] |= c << sh;
      if (sh + B > 32) w[wi + 1] |= c >> (32 - sh);
    }
    store_words<B>(out + g * B, w);
  }
  // one atomic per wavefront that found out-of-range indices
  for (int o = 32; o > 0; o >>= 1) nbad += __shfl_xor(nbad, o, 64);
  if (bad && (threadIdx.x & 63) == 0 && nbad) atomicAdd(bad, nbad);
}

// one thread per 4 consecutive indices, so that each store instruction writes 1 KB of consecutive
// int32 (16 bytes per lane); index i's B bits start at bit i*B, in one word or straddling two
template <int B>
__global__ __launch_bounds__(PW) void payload_unpack_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                            int32_t* __restrict__ idx) {
  const int64_t nq = (n + 3) / 4;
  const int64_t nwords = (n + 31) / 32 * B;
  for (int64_t q = (int64_t)blockIdx.x * PW + threadIdx.x; q < nq; q += (int64_t)gridDim.x * PW) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t pos = (q * 4 + i) * B;
      const int64_t wi = pos >> 5;
      const int sh = (int)(pos & 31);
      uint32_t c = in[wi] >> sh;
      if (sh + B > 32 && wi + 1 < nwords) c |= in[wi + 1] << (32 - sh);
      v[i] = (int)(c & ((1u << B) - 1u));
    }
    const int64_t first = q * 4;
    if (first + 4 <= n) {
      *reinterpret_cast<int4*>(idx + first) = make_int4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (first + i < n) idx[first + i] = v[i];
    }
  }
}

unsigned payload_grid(int64_t n) {
  const int64_t groups = (n + 31) / 32;
  return (unsigned)std::min<int64_t>((groups + PW - 1) / PW, 8192);
}

int launch_pack(const int32_t* idx, int64_t n, int32_t E, uint8_t* packed, int32_t* bad, hipStream_t st) {
  const unsigned grid = payload_grid(n);
  uint32_t* out = reinterpret_cast<uint32_t*>(packed);
  switch (payload_bits(E)) {
#define PACK_CASE(B) \
  case B: payload_pack_kernel<B><<<grid, PW, 0, st>>>(idx, n, E, out, bad); break;
    PACK_CASE(1) PACK_CASE(2) PACK_CASE(3) PACK_CASE(4) PACK_CASE(5) PACK_CASE(6) PACK_CASE(7) PACK_CASE(8)
    PACK_CASE(9) PACK_CASE(10) PACK_CASE(11) PACK_CASE(12) PACK_CASE(13) PACK_CASE(14) PACK_CASE(15) PACK_CASE(16)
#undef PACK_CASE
    default: return MOE_ERR_SHAPE;
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

int launch_unpack(const uint8_t* packed, int64_t n, int32_t E, int32_t* idx, hipStream_t st) {
  const unsigned grid = (unsigned)std::min<int64_t>(((n + 3) / 4 + PW - 1) / PW, 16384);
  const uint32_t* in = reinterpret_cast<const uint32_t*>(packed);
  switch (payload_bits(E)) {
#define UNPACK_CASE(B) \
  case B: payload_unpack_kernel<B><<<grid, PW, 0, st>>>(in, n, idx); break;
    UNPACK_CASE(1) UNPACK_CASE(2) UNPACK_CASE(3) UNPACK_CASE(4) UNPACK_CASE(5) UNPACK_CASE(6) UNPACK_CASE(7)
    UNPACK_CASE(8) UNPACK_CASE(9) UNPACK_CASE(10) UNPACK_CASE(11) UNPACK_CASE(12) UNPACK_CASE(13)
    UNPACK_CASE(14) UNPACK_CASE(15) UNPACK_CASE(16)
#undef UNPACK_CASE
    default: return MOE_ERR_SHAPE;
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

constexpr int64_t PAYLOAD_MAX_N = (int64_t)1 << 40;

int check(int64_t n, int32_t E) {
  if (n < 0 || n > PAYLOAD_MAX_N || E < 1 || E > 65536) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" size_t moe_payload_bytes(int64_t n, int32_t E) {
  if (check(n, E) != MOE_OK) return 0;
  return (size_t)((n + 31) / 32) * 4 * (size_t)payload_bits(E);
}

extern "C" int moe_payload_pack(const int32_t* idx, int64_t n, int32_t E, uint8_t* packed, int32_t* bad_count,
                                void* stream) {
  int rc = check(n, E);
  if (rc != MOE_OK) return rc;
  if (n == 0) return MOE_OK;
  if (!idx || !packed) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(packed)) & 15) return MOE_ERR_ARG;
  return launch_pack(idx, n, E, packed, bad_count, as_stream(stream));
}

extern "C" int moe_payload_unpack(const uint8_t* packed, int64_t n, int32_t E, int32_t* idx, void* stream) {
  int rc = check(n, E);
  if (rc != MOE_OK) return rc;
  if (n == 0) return MOE_OK;
  if (!idx || !packed) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(packed)) & 15) return MOE_ERR_ARG;
  return launch_unpack(packed, n, E, idx, as_stream(stream));
}

extern "C" int moe_payload_to_host(const int32_t* idx, int64_t n, int32_t E, uint8_t* staging, void* host,
                                   int32_t* bad_count, void* stream) {
  int rc = check(n, E);
  if (rc != MOE_OK) return rc;
  if (n == 0) return MOE_OK;
  if (!host) return MOE_ERR_NULL;
  rc = moe_payload_pack(idx, n, E, staging, bad_count, stream);
  if (rc != MOE_OK) return rc;
  if (hipMemcpyAsync(host, staging, moe_payload_bytes(n, E), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

extern "C" int moe_payload_from_host(const void* host, int64_t n, int32_t E, uint8_t* staging, int32_t* idx,
                                     void* stream) {
  int rc = check(n, E);
  if (rc != MOE_OK) return rc;
  if (n == 0) return MOE_OK;
  if (!host || !staging || !idx) return MOE_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(idx) | reinterpret_cast<uintptr_t>(staging)) & 15) return MOE_ERR_ARG;
  if (hipMemcpyAsync(staging, host, moe_payload_bytes(n, E), hipMemcpyHostToDevice, as_stream(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return launch_unpack(staging, n, E, idx, as_stream(stream));
}
