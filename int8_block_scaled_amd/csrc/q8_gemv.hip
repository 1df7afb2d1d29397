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
// that a wave issues as one contiguous 1 KB piece, marked nontemporal (the
// stream has no reuse; measured 7% faster at M = 1 than cached loads), and
// does the int8 dots on the vector ALU (v_dot4_i32_i8), not on the matrix
// cores.
//
// Work split: one workgroup per 64-row group; its (up to 16) waves split the
// K blocks evenly and walk their range in chunks of L blocks, all of a
// chunk's loads in flight together.  Lane l of a wave owns row 64g + l.  In a piece (g, kb, h) lane l
// holds bytes [16h, 16h+16) of its row's block kb, so all 64 lanes need the
// same 16 activation bytes: those are wave-uniform and come from scalar
// loads into SGPRs, which v_dot4 takes as its second operand.  A lane has
// both halves of its block, so the block dot is an exact int32 in one lane
// and is scaled there: acc += float(P) * (d_w * d_a), where the binary16 x
// binary16 product is exact in binary32.  Waves then add their partial
// sums in a fixed order through LDS, so results are reproducible.
#include <cstdlib>

#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kMaxWaves = 16;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int kThreads = kMaxWaves * 64;

// One chunk of L blocks: all weight loads of the chunk are issued first (2 x
// 16 bytes per lane per block, plus the binary16 scales), then the dots.
// Block indices past the wave's range are clamped to its last block (a
// cached re-read) and their contribution is dropped, so the code is
// straight-line and every load of the chunk is in flight together.
template <int MR, int L, bool NT>
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

  const v4u* wp = reinterpret_cast<const v4u*>(wq + g * KB * kGroupBlockBytes) + lane;
  const uint16_t* sp = ws + g * KB * kGroupRows + lane;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

  for (int64_t c = kb0; c < kb1; c += L) {
    v4u w0[L], w1[L];
    float dw[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t kb = (c + i < kb1) ? c + i : kb1 - 1;
      if constexpr (NT) {   // streamed once: no reuse to keep in the caches
        w0[i] = __builtin_nontemporal_load(wp + (kb * 2 + 0) * 64);
        w1[i] = __builtin_nontemporal_load(wp + (kb * 2 + 1) * 64);
      } else {
        w0[i] = wp[(kb * 2 + 0) * 64];
        w1[i] = wp[(kb * 2 + 1) * 64];
      }
      // unconditional load (a branch here would serialise the chunk's loads)
      dw[i] = f16_bits_to_f32(sp[kb * kGroupRows]) * (c + i < kb1 ? 1.0f : 0.0f);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t kb = (c + i < kb1) ? c + i : kb1 - 1;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const int* a = reinterpret_cast<const int*>(q_a + m * K + kb * kQK);  // wave-uniform
        int p = 0;
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].x), a[0], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].y), a[1], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].z), a[2], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].w), a[3], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].x), a[4], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].y), a[5], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].z), a[6], p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].w), a[7], p, false);
        const float s = dw[i] * f16_bits_to_f32(d_a[m * KB + kb]);  // exact: 11 x 11 bits
        acc[m] = fmaf(static_cast<float>(p), s, acc[m]);
      }
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

// Fused decode step: the same product, from unquantised activation rows x
// (binary32 or bfloat16).  Every wave quantises the activation blocks of its
// chunk itself (quantize8, the code of the quantise kernel, so codes and
// scales are bit-identical to it), right after issuing the chunk's weight
// loads so that the two loads overlap, and keeps them in a small LDS slot
// of its own: codes [m][i][32] and scales [m][i] for the L blocks i of the
// chunk.  Lanes then read them back with broadcast LDS loads.  The block
// walk, the dot products and the reduction are those of gemv_q8_kernel, so
// C is bit-identical to quantising first and then running that kernel.
// Workgroup 0 also stores the codes and scales when q_out is not NULL.
template <int MR, int L, bool kBf16>
__global__ __launch_bounds__(kThreads) void gemv_q8_act_kernel(
    const void* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wq,
    const uint16_t* __restrict__ ws, float* __restrict__ C, int64_t N, int64_t K, int64_t KB,
    int64_t ldc, int kb_per_wave, int8_t* __restrict__ q_out, uint16_t* __restrict__ d_out) {
  constexpr int kSlotBytes = MR * L * (kQK + 4);   // per wave: codes, then binary32 scales
  constexpr int kItems = MR * L * 4;               // quantiser lanes per chunk (4 per block)
  constexpr int kPasses = (kItems + 63) / 64;
  __shared__ __align__(16) uint8_t lds[kMaxWaves * (kSlotBytes > MR * 256 ? kSlotBytes : MR * 256)];
  const int64_t g = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int64_t kb0 = static_cast<int64_t>(wave) * kb_per_wave;
  const int64_t kb1 = kb0 + kb_per_wave < KB ? kb0 + kb_per_wave : KB;
  const bool store_q = q_out != nullptr && blockIdx.x == 0;

  uint8_t* const qslot = lds + wave * kSlotBytes;
  float* const dslot = reinterpret_cast<float*>(qslot + MR * L * kQK);

  const v4u* wp = reinterpret_cast<const v4u*>(wq + g * KB * kGroupBlockBytes) + lane;
  const uint16_t* sp = ws + g * KB * kGroupRows + lane;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.0f;

  for (int64_t c = kb0; c < kb1; c += L) {
    v4u w0[L], w1[L];
    float dw[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int64_t kb = (c + i < kb1) ? c + i : kb1 - 1;
      w0[i] = __builtin_nontemporal_load(wp + (kb * 2 + 0) * 64);
      w1[i] = __builtin_nontemporal_load(wp + (kb * 2 + 1) * 64);
      dw[i] = f16_bits_to_f32(sp[kb * kGroupRows]) * (c + i < kb1 ? 1.0f : 0.0f);
    }
    // Quantise the chunk's activation blocks: item t = (m * L + i) * 4 + sub.
    float v[kPasses][8];
#pragma unroll
    for (int u = 0; u < kPasses; ++u) {
      const int t = u * 64 + lane;
      const int m = t / (L * 4), i = (t / 4) % L, sub = t % 4;
      const int64_t kb = (c + i < kb1) ? c + i : kb1 - 1;
      if (t < kItems) {
        load8<kBf16>(x, m * ldx + kb * kQK + sub * 8, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kPasses; ++u) {
      const int t = u * 64 + lane;
      const int m = t / (L * 4), i = (t / 4) % L, sub = t % 4;
      uint32_t lo, hi;
      uint16_t dbits;
      quantize8(v[u], lo, hi, dbits);   // all lanes take part (lane exchanges)
      if (t < kItems) {
        *reinterpret_cast<uint2*>(qslot + (m * L + i) * kQK + sub * 8) = make_uint2(lo, hi);
        if (sub == 0) dslot[m * L + i] = f16_bits_to_f32(dbits);
        if (store_q && c + i < kb1) {
          *reinterpret_cast<uint2*>(q_out + m * K + (c + i) * kQK + sub * 8) = make_uint2(lo, hi);
          if (sub == 0) d_out[m * KB + c + i] = dbits;
        }
      }
    }
    // The slot is this wave's alone and a wave's LDS accesses complete in
    // order: no barrier is needed before reading it back.
#pragma unroll
    for (int i = 0; i < L; ++i) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const v4u* ap = reinterpret_cast<const v4u*>(qslot + (m * L + i) * kQK);
        const v4u a0 = ap[0], a1 = ap[1];
        int p = 0;
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].x), static_cast<int>(a0.x), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].y), static_cast<int>(a0.y), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].z), static_cast<int>(a0.z), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w0[i].w), static_cast<int>(a0.w), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].x), static_cast<int>(a1.x), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].y), static_cast<int>(a1.y), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].z), static_cast<int>(a1.z), p, false);
        p = __builtin_amdgcn_sdot4(static_cast<int>(w1[i].w), static_cast<int>(a1.w), p, false);
        const float s = dw[i] * dslot[m * L + i];   // exact: 11 x 11 bits
        acc[m] = fmaf(static_cast<float>(p), s, acc[m]);
      }
    }
  }

  __syncthreads();   // every wave is done with its slot: reuse LDS for the partials
  float* red = reinterpret_cast<float*>(lds);   // [wave][m][lane]
#pragma unroll
  for (int m = 0; m < MR; ++m) red[(wave * MR + m) * 64 + lane] = acc[m];
  __syncthreads();
  for (int t = threadIdx.x; t < MR * 64; t += blockDim.x) {
    const int m = t >> 6, r = t & 63;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += red[(w * MR + m) * 64 + r];
    const int64_t n = g * kGroupRows + r;
    if (n < N) C[m * ldc + n] = sum;
  }
}

template <int MR, int L, bool NT>
hipError_t launch_m(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                    const uint8_t* w_packed, float* C, int64_t ldc, int max_waves,
                    hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < max_waves ? KB : max_waves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  hipLaunchKernelGGL((gemv_q8_kernel<MR, L, NT>), dim3(static_cast<uint32_t>(NG)), dim3(waves * 64),
                     0, stream, q_a, d_a, w_packed, ws, C, N, K, KB, ldc, kb_per_wave);
  return hipGetLastError();
}

template <int MR>
hipError_t launch_cfg(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                      const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  // Q8_GEMV_CFG=<c> (benchmarking aid): c = 0: 16 waves x chunks of 4
  // blocks, nontemporal weight loads (default); 1: the same with ordinary
  // loads; 2: 16 waves x chunks of 8, nontemporal.
  int cfg = 0;
  if (const char* e = getenv("Q8_GEMV_CFG")) cfg = atoi(e);
  switch (cfg) {
    case 1: return launch_m<MR, 4, false>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
    case 2: return launch_m<MR, 8, true>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
    default: return launch_m<MR, 4, true>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
  }
}

template <int MR>
hipError_t launch_act_m(const void* x, bool bf16, int64_t ldx, int64_t N, int64_t K,
                        const uint8_t* w_packed, float* C, int64_t ldc, int8_t* q_out,
                        uint16_t* d_out, hipStream_t stream) {
  constexpr int L = 4;   // as the default configuration of the unfused kernel
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < kMaxWaves ? KB : kMaxWaves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  if (bf16)
    hipLaunchKernelGGL((gemv_q8_act_kernel<MR, L, true>), dim3(static_cast<uint32_t>(NG)),
                       dim3(waves * 64), 0, stream, x, ldx, w_packed, ws, C, N, K, KB, ldc,
                       kb_per_wave, q_out, d_out);
  else
    hipLaunchKernelGGL((gemv_q8_act_kernel<MR, L, false>), dim3(static_cast<uint32_t>(NG)),
                       dim3(waves * 64), 0, stream, x, ldx, w_packed, ws, C, N, K, KB, ldc,
                       kb_per_wave, q_out, d_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_act(int M, const void* x, int dtype, int64_t ldx, int64_t N, int64_t K,
                           const uint8_t* w_packed, float* C, int64_t ldc, int8_t* q_out,
                           uint16_t* d_out, hipStream_t stream) {
  const bool bf16 = dtype == 1;
  switch (M) {
    case 1: return launch_act_m<1>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 2: return launch_act_m<2>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 3: return launch_act_m<3>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 4: return launch_act_m<4>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 5: return launch_act_m<5>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 6: return launch_act_m<6>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 7: return launch_act_m<7>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    case 8: return launch_act_m<8>(x, bf16, ldx, N, K, w_packed, C, ldc, q_out, d_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(int M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  switch (M) {
    case 1: return launch_cfg<1>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 2: return launch_cfg<2>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 3: return launch_cfg<3>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 4: return launch_cfg<4>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 5: return launch_cfg<5>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 6: return launch_cfg<6>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 7: return launch_cfg<7>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    case 8: return launch_cfg<8>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q8
