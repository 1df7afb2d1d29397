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
// across the four lanes with two lane exchanges (quantize8 in q8_kernels.h,
// which states the bit-exactness conditions).

#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kThreads = 128;   // K/8 items per row: a whole number of workgroups for K % 1024 == 0
constexpr int kMaxGridY = 65535;

// Grid: x covers the K/8 items of a row (four per block), y the rows (each
// y-slice loops over rows y, y + gridDim.y, ... when M exceeds the grid's
// y limit), so no thread divides by the row length.
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void quantize_act_kernel(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    uint16_t* __restrict__ d) {
  const int t = static_cast<int>(blockIdx.x) * kThreads + static_cast<int>(threadIdx.x);
  // Items past the row end still take part in the lane exchange below with
  // zeros; they load and store nothing.
  const bool live = t < static_cast<int>(K / 8);
  const int64_t KB = K / kQK;
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {   // uniform trip count
    float v[8];
    if (live) {
      load8<kBf16>(x, m * ldx + t * 8, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    uint32_t lo, hi;
    uint16_t dbits;
    quantize8(v, lo, hi, dbits);
    if (live) {
      *reinterpret_cast<uint2*>(q + m * K + t * 8) = make_uint2(lo, hi);
      if ((t & 3) == 0) d[m * KB + (t >> 2)] = dbits;
    }
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           int8_t* q, uint16_t* d, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((K / 8 + kThreads - 1) / kThreads),
                  static_cast<uint32_t>(M < kMaxGridY ? M : kMaxGridY));
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_act_kernel<true>, grid, dim3(kThreads), 0, stream, x, M, K, ldx,
                       q, d);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, grid, dim3(kThreads), 0, stream, x, M, K, ldx,
                       q, d);
  return hipGetLastError();
}

}  // namespace q8
