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
// Two layouts of the work, with the same arithmetic per block (so the same
// bits):
//   - four lanes own one 32-value block (eight values per lane, one 16-byte
//     bfloat16 load or two 16-byte binary32 loads), so a wave covers 16
//     consecutive blocks = 512 contiguous values of a row and its loads and
//     stores are fully coalesced; the block maximum is reduced across the
//     four lanes with two lane exchanges (quantize8 in q8_kernels.h, which
//     states the bit-exactness conditions);
//   - for large inputs (2^18 blocks and more, rows of at least 64 blocks),
//     one lane owns a whole block:
//     it loads its 32 values itself, takes the maximum and the scale once
//     and writes its 32 codes with two 16-byte stores.  Fewer vector
//     instructions per byte and no lane exchanges: 10-15 % faster at 2048
//     and 8192 rows of 4096, but slower on small inputs, where the quarter
//     as many lanes hide less of the memory latency.

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

// One lane per block (grid: x over the row's blocks, 64 per workgroup; y
// over rows, looping past the grid's y limit).
template <bool kBf16>
__global__ __launch_bounds__(64) void quantize_blk_kernel(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    uint16_t* __restrict__ d) {
  const int64_t KB = K / kQK;
  const int64_t kb = static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x;
  if (kb >= KB) return;   // no lane exchanges here
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    float v[kQK];
#pragma unroll
    for (int j = 0; j < kQK / 8; ++j) load8<kBf16>(x, m * ldx + kb * kQK + 8 * j, v + 8 * j);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < kQK; ++e) amax = fmaxf(amax, fabsf(v[e]));
    float id;
    uint16_t dbits;
    const bool nz = block_scale(amax, id, dbits);
    uint32_t w[kQK / 4];
#pragma unroll
    for (int c = 0; c < kQK / 4; ++c) {
      w[c] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[c] |= (nz ? static_cast<uint32_t>(block_code(v[4 * c + e], id)) & 0xffu : 0u)
                << (8 * e);
    }
    uint4* const qo = reinterpret_cast<uint4*>(q + m * K + kb * kQK);   // 16-byte aligned
    qo[0] = make_uint4(w[0], w[1], w[2], w[3]);
    qo[1] = make_uint4(w[4], w[5], w[6], w[7]);
    d[m * KB + kb] = dbits;
  }
}

constexpr int64_t kBlockPerLaneMin = int64_t(1) << 18;   // blocks

}  // namespace

hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           int8_t* q, uint16_t* d, hipStream_t stream) {
  const dim3 grid_y(1, static_cast<uint32_t>(M < kMaxGridY ? M : kMaxGridY));
  if (M * (K / kQK) >= kBlockPerLaneMin && K / kQK >= 64) {   // and whole waves of blocks
    const dim3 grid(static_cast<uint32_t>((K / kQK + 63) / 64), grid_y.y);
    if (dtype == 1)
      hipLaunchKernelGGL(quantize_blk_kernel<true>, grid, dim3(64), 0, stream, x, M, K, ldx, q, d);
    else
      hipLaunchKernelGGL(quantize_blk_kernel<false>, grid, dim3(64), 0, stream, x, M, K, ldx, q,
                         d);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<uint32_t>((K / 8 + kThreads - 1) / kThreads), grid_y.y);
  if (dtype == 1)
    hipLaunchKernelGGL(quantize_act_kernel<true>, grid, dim3(kThreads), 0, stream, x, M, K, ldx,
                       q, d);
  else
    hipLaunchKernelGGL(quantize_act_kernel<false>, grid, dim3(kThreads), 0, stream, x, M, K, ldx,
                       q, d);
  return hipGetLastError();
}

}  // namespace q8
