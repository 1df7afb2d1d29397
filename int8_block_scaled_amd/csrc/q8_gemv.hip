// q8_gemv.hip -- decode path of the Q8_0 product, M = 1..8 token rows.
//
// C[m][n] = sum_kb d_a[m][kb] d_w[n][kb] int32(sum_j q_a q_w); the source
// engine's generation step runs this product through its int8 dot-product
// kernel (news.hada.io topic 29953, "CUDA inference engine for running
// Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)": GEMM item of
// the list of non-throttled paths; generation speed in the benchmark list).
//
// At M <= 8 the product is bound by HBM: each weight byte is used M times.
// The kernel therefore streams the packed weights once, with 16-byte loads
// that a wave issues as one contiguous 1 KB piece, and does the int8 dots
// on the vector ALU (v_dot4_i32_i8), not on the matrix cores.
//
// Work split: one workgroup per 64-row group; its waves split the K blocks
// evenly.  Lane l of a wave owns row 64g + l.  In a piece (g, kb, h) lane l
// holds bytes [16h, 16h+16) of its row's block kb, so all 64 lanes need the
// same 16 activation bytes: those are wave-uniform and come from scalar
// loads into SGPRs, which v_dot4 takes as its second operand.  A lane has
// both halves of its block, so the block dot is an exact int32 in one lane
// and is scaled there: acc += float(P) * (d_w * d_a), where the binary16 x
// binary16 product is exact in binary32.  Waves then add their partial
// sums in a fixed order through LDS, so results are reproducible.
#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kThreads = kMaxWaves * 64;

template <int MR>
__global__ __launch_bounds__(kThreads) void gemv_q8_kernel(
    const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    float* __restrict__ C, int64_t N, int64_t K, int64_t KB, int64_t ldc, int kb_per_wave) {
  __shared__ float red[kMaxWaves][MR][64];
  const int64_t g = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int64_t kb0 = static_cast<int64_t>(wave) * kb_per_wave;
  const int64_t kb1 = kb0 + kb_per_wave < KB ? kb0 + kb_per_wave : KB;

  const uint4* wp = reinterpret_cast<const uint4*>(wq + g * KB * kGroupBlockBytes) + lane;
  const uint16_t* sp = ws + g * KB * kGroupRows + lane;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

#pragma unroll 4
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    const uint4 w0 = wp[(kb * 2 + 0) * 64];
    const uint4 w1 = wp[(kb * 2 + 1) * 64];
    const float dw = f16_bits_to_f32(sp[kb * kGroupRows]);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int* a = reinterpret_cast<const int*>(q_a + m * K + kb * kQK);  // wave-uniform
      int p = 0;
      p = __builtin_amdgcn_sdot4(static_cast<int>(w0.x), a[0], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w0.y), a[1], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w0.z), a[2], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w0.w), a[3], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w1.x), a[4], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w1.y), a[5], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w1.z), a[6], p, false);
      p = __builtin_amdgcn_sdot4(static_cast<int>(w1.w), a[7], p, false);
      const float s = dw * f16_bits_to_f32(d_a[m * KB + kb]);  // exact: 11 x 11 bits
      acc[m] = fmaf(static_cast<float>(p), s, acc[m]);
    }
  }

#pragma unroll
  for (int m = 0; m < MR; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  // MR*64 sums; a workgroup may have fewer than MR waves when KB is small.
  for (int t = threadIdx.x; t < MR * 64; t += blockDim.x) {
    const int m = t >> 6, r = t & 63;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += red[w][m][r];
    const int64_t n = g * kGroupRows + r;
    if (n < N) C[m * ldc + n] = sum;
  }
}

template <int MR>
hipError_t launch_m(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                    const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < kMaxWaves ? KB : kMaxWaves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  hipLaunchKernelGGL(gemv_q8_kernel<MR>, dim3(static_cast<uint32_t>(NG)), dim3(waves * 64), 0,
                     stream, q_a, d_a, w_packed, ws, C, N, K, KB, ldc, kb_per_wave);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  switch (M) {
    case 1: return launch_m<1>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 2: return launch_m<2>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 3: return launch_m<3>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 4: return launch_m<4>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 5: return launch_m<5>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 6: return launch_m<6>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 7: return launch_m<7>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 8: return launch_m<8>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q8
