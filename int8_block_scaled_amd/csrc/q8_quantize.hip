// q8_quantize.hip -- activation rows -> Q8_0 blocks (int8 q + binary16 d).
//
// The Q8_0 quantiser (block of 32 values along K, one binary16 scale
// d = amax/127, q = x/d rounded half away from zero); the source engine
// quantises activations on the fly into this block format so its int8 GEMM
// can run on them (news.hada.io topic 29953, "CUDA inference engine for
// running Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)", GEMM
// item of the list of non-throttled paths; Q8_0 in the limitations list).
//
// HBM-bound: every byte of x is read once, q and d are written once.
// Layout of the work: four lanes own one 32-value block (eight values per
// lane, one 16-byte bfloat16 load or two 16-byte binary32 loads), so a
// wave covers 16 consecutive blocks = 512 contiguous values of a row and
// its loads and stores are fully coalesced.  The block maximum is reduced
// across the four lanes with two DPP-free lane exchanges.
//
// Bit-exactness: d32 = amax/127 and id = 1/d32 use the correctly rounded
// binary32 division (HIP's default; never build this with fast-math or
// -fno-hip-fp32-correctly-rounded-divide-sqrt), v = x*id is a single
// multiply, roundf rounds half away from zero, and the binary16 conversion
// is v_cvt_f16_f32 (round to nearest even, binary16 subnormals kept).
#include <float.h>

#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;

template <bool kBf16>
__device__ __forceinline__ void load8(const void* __restrict__ x, int64_t off, float v[8]) {
  if constexpr (kBf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(
    const void* __restrict__ x, int64_t total_threads, int64_t KB, int64_t ldx,
    int8_t* __restrict__ q, uint16_t* __restrict__ d) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  // Threads past the end still take part in the lane exchange below with
  // zeros; they load and store nothing.
  const bool live = t < total_threads;
  const int64_t blk = t >> 2;            // block index over [M][KB]
  const int sub = static_cast<int>(t & 3);
  const int64_t m = blk / KB;
  const int64_t kb = blk - m * KB;

  float v[8];
  if (live) {
    load8<kBf16>(x, m * ldx + kb * kQK + sub * 8, v);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // The four lanes of a block are consecutive and 4-aligned in the wave.
  amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 4));

  const float d32 = amax / 127.0f;
  uint32_t lo = 0, hi = 0;
  uint16_t dbits = 0;
  if (d32 >= FLT_MIN) {
    const float id = 1.0f / d32;
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int qi = static_cast<int>(roundf(v[i] * id));  // |qi| <= 127
      b[i] = static_cast<uint32_t>(qi) & 0xffu;
    }
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    dbits = f32_to_f16_bits(d32);
  }
  if (live) {
    *reinterpret_cast<uint2*>(q + blk * kQK + sub * 8) = make_uint2(lo, hi);
    if (sub == 0) d[blk] = dbits;
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           int8_t* q, uint16_t* d, hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t total = M * KB * 4;
  const int64_t grid = (total + kThreads - 1) / kThreads;
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_act_kernel<true>, dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream, x, total, KB, ldx, q, d);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, dim3(static_cast<uint32_t>(grid)),
                       dim3(kThreads), 0, stream, x, total, KB, ldx, q, d);
  return hipGetLastError();
}

}  // namespace q8
