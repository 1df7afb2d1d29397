// q8_pack.hip -- GGUF Q8_0 weight blocks -> the packed layout of include/q8.h.
//
// A pure byte permutation, run once when the weights load.  The source
// engine reads Q8_0 GGUF weights (news.hada.io topic 29953, "CUDA inference
// engine for running Qwen3.5/3.6 hybrid models on mining cards (CMP
// 100-210)", benchmark list: same Q8_0 GGUF as the baseline); this call
// turns its 34-byte blocks into row groups of 64 features in which every
// (group, block, half) piece is 1 KB of 16-byte row slices -- the order in
// which both the matrix-core kernel (one 16-byte slice per lane and per
// 32x32x32 int8 operand) and the decode kernel (one coalesced 1 KB load per
// wave) consume them -- plus a separate plane of binary16 scales.
//
// One thread writes one 16-byte output slice (and, for h == 0, the row's
// scale).  Source blocks are 34 bytes and may sit at any alignment, so they
// are read a byte at a time; the output side is fully coalesced.
#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;

// blocks2 == NULL: row n of the packed weight is row n of blocks.  Else
// (gate/up interleave, N = 2I): row 64g + r is row 32g + r of blocks (the
// gate weight) for r < 32, and row 32g + r - 32 of blocks2 (the up weight).
__global__ __launch_bounds__(kThreads) void pack_weights_kernel(
    const uint8_t* __restrict__ blocks, const uint8_t* __restrict__ blocks2, int64_t N,
    int64_t KB, int64_t slices, uint8_t* __restrict__ qplane, uint16_t* __restrict__ splane) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (s >= slices) return;
  const int r = static_cast<int>(s & 63);         // row within the group
  const int h = static_cast<int>((s >> 6) & 1);   // which 16-byte half of the block
  const int64_t gk = s >> 7;                      // g*KB + kb
  const int64_t g = gk / KB;
  const int64_t kb = gk - g * KB;
  const int64_t n = g * kGroupRows + r;

  uint32_t w[4] = {0u, 0u, 0u, 0u};
  uint16_t scale = 0;
  if (n < N) {
    const uint8_t* src = blocks;
    int64_t sn = n;
    if (blocks2 != nullptr) {
      src = r < 32 ? blocks : blocks2;
      sn = g * 32 + (r & 31);
    }
    const uint8_t* b = src + (sn * KB + kb) * 34;
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 2] |= static_cast<uint32_t>(b[2 + 16 * h + i]) << (8 * (i & 3));
    scale = static_cast<uint16_t>(b[0] | (b[1] << 8));
  }
  reinterpret_cast<uint4*>(qplane)[s] = make_uint4(w[0], w[1], w[2], w[3]);
  if (h == 0) splane[gk * kGroupRows + r] = scale;
}

}  // namespace

hipError_t launch_pack(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* packed,
                       hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int64_t slices = NG * KB * 2 * kGroupRows;
  uint8_t* qplane = packed;
  uint16_t* splane = reinterpret_cast<uint16_t*>(packed + NG * KB * kGroupBlockBytes);
  const int64_t grid = (slices + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, blocks, nullptr, N, KB, slices, qplane, splane);
  return hipGetLastError();
}

hipError_t launch_pack_gateup(const uint8_t* gate, const uint8_t* up, int64_t I, int64_t K,
                              uint8_t* packed, hipStream_t stream) {
  const int64_t N = 2 * I;   // a multiple of 64: no padding rows
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int64_t slices = NG * KB * 2 * kGroupRows;
  uint8_t* qplane = packed;
  uint16_t* splane = reinterpret_cast<uint16_t*>(packed + NG * KB * kGroupBlockBytes);
  const int64_t grid = (slices + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, gate, up, N, KB, slices, qplane, splane);
  return hipGetLastError();
}

}  // namespace q8
