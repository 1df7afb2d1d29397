// q8_kv3.hip -- 3-bit KV-cache codec: rows of D values (a key or value
// head vector) <-> 3-bit Lloyd-Max codes of their Walsh-Hadamard transform
// plus one binary32 scale.
//
// The source engine keeps its 256K-token KV cache in 3 bits with a
// Walsh-Hadamard transform and a Lloyd-Max quantiser, 17 GB -> 3.5 GB
// (news.hada.io topic 29953, "CUDA inference engine for running
// Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)", list of
// non-throttled paths, KV-cache item).  The pages give nothing more; the
// format implemented here is specified in include/q8.h (q8_kv3_encode).
//
// Both kernels are bound by HBM.  One wave owns one row; lane l holds the
// E = D/64 consecutive elements [l*E, l*E + E), loaded or stored with one
// vector access.  The transform's butterfly stages run in order len = 1,
// 2, 4, ...: stages with len < E inside the lane, the others as lane
// exchanges (lane l with lane l ^ (len/E)), every pair (a, b) becoming
// (a + b, a - b) in binary32 -- the order the format fixes, so the results
// are bit-identical to any implementation of it.
#include <float.h>

#include "q8_kernels.h"

// Every product and sum below is its own binary32 operation: no fused
// multiply-add, which would round differently from the format's definition.
#pragma clang fp contract(off)

namespace q8 {
namespace {

constexpr int kRowsPerBlock = 4;   // one wave per row
constexpr int kThreads = kRowsPerBlock * 64;

// The codebook: the 8-level Lloyd-Max quantiser of a unit Gaussian, and the
// decision thresholds, the binary32 midpoints of adjacent levels.
constexpr float kL0 = -2.1520f, kL1 = -1.3440f, kL2 = -0.7560f, kL3 = -0.2451f;
constexpr float kL4 = 0.2451f, kL5 = 0.7560f, kL6 = 1.3440f, kL7 = 2.1520f;
constexpr float kT0 = (kL0 + kL1) * 0.5f, kT1 = (kL1 + kL2) * 0.5f, kT2 = (kL2 + kL3) * 0.5f,
                kT3 = (kL3 + kL4) * 0.5f, kT4 = (kL4 + kL5) * 0.5f, kT5 = (kL5 + kL6) * 0.5f,
                kT6 = (kL6 + kL7) * 0.5f;

__device__ __forceinline__ int code_of(float u) {
  return (kT0 <= u) + (kT1 <= u) + (kT2 <= u) + (kT3 <= u) + (kT4 <= u) + (kT5 <= u) + (kT6 <= u);
}

__device__ __forceinline__ float level_of(int c) {
  float v = kL0;
  v = c == 1 ? kL1 : v;
  v = c == 2 ? kL2 : v;
  v = c == 3 ? kL3 : v;
  v = c == 4 ? kL4 : v;
  v = c == 5 ? kL5 : v;
  v = c == 6 ? kL6 : v;
  v = c == 7 ? kL7 : v;
  return v;
}

// Unnormalised Walsh-Hadamard transform of the wave's row, in place.
template <int E>
__device__ __forceinline__ void fwht(float (&v)[E], int lane) {
#pragma unroll
  for (int len = 1; len < E; len <<= 1)
#pragma unroll
    for (int j = 0; j < E; ++j)
      if ((j & len) == 0) {
        const float a = v[j], b = v[j + len];
        v[j] = a + b;
        v[j + len] = a - b;
      }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {   // len = m * E
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const float other = __shfl_xor(v[j], m);
      v[j] = upper ? other - v[j] : v[j] + other;
    }
  }
}

template <int E, bool kBf16>
__device__ __forceinline__ void load_row(const void* x, int64_t off, float (&v)[E]) {
  if constexpr (kBf16) {
    const uint16_t* p = static_cast<const uint16_t*>(x) + off;
    if constexpr (E == 1) {
      v[0] = __uint_as_float(static_cast<uint32_t>(p[0]) << 16);
    } else if constexpr (E == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
      v[0] = __uint_as_float(w << 16);
      v[1] = __uint_as_float(w & 0xffff0000u);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p);
      v[0] = __uint_as_float(w.x << 16);
      v[1] = __uint_as_float(w.x & 0xffff0000u);
      v[2] = __uint_as_float(w.y << 16);
      v[3] = __uint_as_float(w.y & 0xffff0000u);
    }
  } else {
    const float* p = static_cast<const float*>(x) + off;
    if constexpr (E == 1) {
      v[0] = p[0];
    } else if constexpr (E == 2) {
      const float2 w = *reinterpret_cast<const float2*>(p);
      v[0] = w.x;
      v[1] = w.y;
    } else {
      const float4 w = *reinterpret_cast<const float4*>(p);
      v[0] = w.x;
      v[1] = w.y;
      v[2] = w.z;
      v[3] = w.w;
    }
  }
}

template <int E, bool kBf16>
__global__ __launch_bounds__(kThreads) void kv3_encode_kernel(
    const void* __restrict__ x, int64_t R, int64_t ldx, uint8_t* __restrict__ codes,
    float* __restrict__ scales) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;   // the whole wave
  float y[E];
  load_row<E, kBf16>(x, row * ldx + lane * E, y);
  fwht<E>(y, lane);

  // s^2 * D: sum of squares by the pairwise tree len = D/2, ..., 1 (lane
  // exchanges for len >= E, then inside the lane)
  float q[E];
#pragma unroll
  for (int j = 0; j < E; ++j) q[j] = y[j] * y[j];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
    for (int j = 0; j < E; ++j) q[j] = q[j] + __shfl_xor(q[j], m);
#pragma unroll
  for (int len = E / 2; len >= 1; len >>= 1)
#pragma unroll
    for (int j = 0; j < len; ++j) q[j] = q[j] + q[j + len];

  float s = sqrtf(q[0] / static_cast<float>(D));
  // a zero, binary32-subnormal or NaN scale: s = 0 and every code 4
  const bool flat = !(s >= FLT_MIN);
  const float inv = flat ? 0.0f : 1.0f / s;
  if (flat) s = 0.0f;

  // this lane's codes at bits 3 * ((l*E + j) % 8) of its 24-bit group
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int c = flat ? 4 : code_of(y[j] * inv);
    w |= static_cast<uint32_t>(c) << (3 * ((lane * E + j) & 7));
  }
  constexpr int kLanesPerGroup = 8 / E;
#pragma unroll
  for (int m = 1; m < kLanesPerGroup; m <<= 1) w |= __shfl_xor(w, m);
  const int gq = lane % kLanesPerGroup;   // position of the lane in its group
  uint8_t* out = codes + row * (3 * D / 8) + (lane / kLanesPerGroup) * 3;
#pragma unroll
  for (int b = 0; b < 3; ++b)
    if (b % kLanesPerGroup == gq) out[b] = static_cast<uint8_t>(w >> (8 * b));
  if (lane == 0) scales[row] = s;
}

template <int E, bool kBf16>
__global__ __launch_bounds__(kThreads) void kv3_decode_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales, int64_t R,
    void* __restrict__ out, int64_t ldo) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= R) return;   // the whole wave
  const uint8_t* in = codes + row * (3 * D / 8) + (lane * E / 8) * 3;
  const uint32_t w = in[0] | (static_cast<uint32_t>(in[1]) << 8) | (static_cast<uint32_t>(in[2]) << 16);
  const float s = scales[row];
  float z[E];
#pragma unroll
  for (int j = 0; j < E; ++j) z[j] = s * level_of((w >> (3 * ((lane * E + j) & 7))) & 7u);
  fwht<E>(z, lane);
  constexpr float kInvD = 1.0f / static_cast<float>(D);
#pragma unroll
  for (int j = 0; j < E; ++j) z[j] = z[j] * kInvD;
  const int64_t off = row * ldo + lane * E;
  if constexpr (kBf16) {
    uint16_t b[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {   // round to nearest even (finite values)
      const uint32_t u = __float_as_uint(z[j]);
      b[j] = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
    }
    uint16_t* p = static_cast<uint16_t*>(out) + off;
    if constexpr (E == 1) p[0] = b[0];
    else if constexpr (E == 2) *reinterpret_cast<uint32_t*>(p) = b[0] | (static_cast<uint32_t>(b[1]) << 16);
    else
      *reinterpret_cast<uint2*>(p) = make_uint2(b[0] | (static_cast<uint32_t>(b[1]) << 16),
                                                b[2] | (static_cast<uint32_t>(b[3]) << 16));
  } else {
    float* p = static_cast<float*>(out) + off;
    if constexpr (E == 1) p[0] = z[0];
    else if constexpr (E == 2) *reinterpret_cast<float2*>(p) = make_float2(z[0], z[1]);
    else *reinterpret_cast<float4*>(p) = make_float4(z[0], z[1], z[2], z[3]);
  }
}

template <int E>
hipError_t launch_enc(const void* x, int dtype, int64_t R, int64_t ldx, uint8_t* codes,
                      float* scales, hipStream_t stream) {
  const uint32_t grid = static_cast<uint32_t>((R + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == 1)
    hipLaunchKernelGGL((kv3_encode_kernel<E, true>), dim3(grid), dim3(kThreads), 0, stream, x, R,
                       ldx, codes, scales);
  else
    hipLaunchKernelGGL((kv3_encode_kernel<E, false>), dim3(grid), dim3(kThreads), 0, stream, x,
                       R, ldx, codes, scales);
  return hipGetLastError();
}

template <int E>
hipError_t launch_dec(const uint8_t* codes, const float* scales, int64_t R, int dtype, void* out,
                      int64_t ldo, hipStream_t stream) {
  const uint32_t grid = static_cast<uint32_t>((R + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == 1)
    hipLaunchKernelGGL((kv3_decode_kernel<E, true>), dim3(grid), dim3(kThreads), 0, stream,
                       codes, scales, R, out, ldo);
  else
    hipLaunchKernelGGL((kv3_decode_kernel<E, false>), dim3(grid), dim3(kThreads), 0, stream,
                       codes, scales, R, out, ldo);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv3_encode(const void* x, int dtype, int64_t R, int64_t D, int64_t ldx,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  switch (D) {
    case 64: return launch_enc<1>(x, dtype, R, ldx, codes, scales, stream);
    case 128: return launch_enc<2>(x, dtype, R, ldx, codes, scales, stream);
    case 256: return launch_enc<4>(x, dtype, R, ldx, codes, scales, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv3_decode(const uint8_t* codes, const float* scales, int64_t R, int64_t D,
                             int dtype, void* out, int64_t ldo, hipStream_t stream) {
  switch (D) {
    case 64: return launch_dec<1>(codes, scales, R, dtype, out, ldo, stream);
    case 128: return launch_dec<2>(codes, scales, R, dtype, out, ldo, stream);
    case 256: return launch_dec<4>(codes, scales, R, dtype, out, ldo, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q8
