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
// Work split: a workgroup owns up to 64 rows (a whole 64-row group in
// gemv_q8_kernel; a slice sized so the grid fills every CU in the default,
// gemv_q8_slice_kernel); its (up to 16) waves split the K blocks evenly and
// walk their range in chunks of L blocks, all of a chunk's loads in flight
// together.  Lane l of a wave owns one row.  In a piece (g, kb, h) a lane
// holds bytes [16h, 16h+16) of its row's block kb, so all lanes need the
// same 16 activation bytes: those are wave-uniform and come from scalar
// loads into SGPRs, which v_dot4 takes as its second operand.  A lane has
// both halves of its block, so the block dot is an exact int32 in one lane
// and is scaled there: acc += float(P) * (d_w * d_a), where the binary16 x
// binary16 product is exact in binary32.  Waves then add their partial
// sums in a fixed order through LDS, so results are reproducible.
#include <cstdio>
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
//
// kSwiglu: the weight is gate/up-packed (64-row group g = gate rows 32g..,
// then up rows 32g..; N = 2I): row r and row r + 32 of the group are the
// gate and up of hidden unit 32g + r, so instead of C the workgroup writes
// the Q8_0 block g of h = silu(gate) * up: q_h [M][I], d_h [M][I/32].
template <int MR, int L, bool NT, bool kSwiglu = false>
__global__ __launch_bounds__(kThreads) void gemv_q8_kernel(
    const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    float* __restrict__ C, int64_t N, int64_t K, int64_t KB, int64_t ldc, int kb_per_wave,
    int8_t* __restrict__ q_h = nullptr, uint16_t* __restrict__ d_h = nullptr) {
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
  if constexpr (kSwiglu) {
    // MR*32 hidden units; each 32 consecutive threads (32-aligned lanes of
    // one wave, since blockDim is a multiple of 64) hold one block.
    const int64_t I = N / 2;
    for (int t = threadIdx.x; t < MR * 32; t += blockDim.x) {
      const int m = t >> 5, r = t & 31;
      float gsum = 0.0f, usum = 0.0f;
      for (int w = 0; w < nwaves; ++w) {
        gsum += red[w][m][r];
        usum += red[w][m][r + 32];
      }
      uint16_t dbits;
      const int q = quantize_lane32(silu_mul(gsum, usum), dbits);
      q_h[m * I + g * 32 + r] = static_cast<int8_t>(q);
      if (r == 0) d_h[m * (I / kQK) + g] = dbits;
    }
    return;
  }
  // MR*64 sums; a workgroup may have fewer than MR waves when KB is small.
  for (int t = threadIdx.x; t < MR * 64; t += blockDim.x) {
    const int m = t >> 6, r = t & 63;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += red[w][m][r];
    const int64_t n = g * kGroupRows + r;
    if (n < N) C[m * ldc + n] = sum;
  }
}

// Row-slice variant: a workgroup owns R <= 64 consecutive rows (a slice that
// may straddle two 64-row groups) instead of one whole group, with R chosen
// so that the grid fills every CU (N = 12288: R = 48, 256 workgroups for
// 256 CUs instead of 192).  Lane l < R owns row R*w + l and computes its
// piece addresses itself; lanes past R (or past N) re-read a row of the
// slice (same lines, no extra HBM traffic) and are dropped.  Everything else is as in
// gemv_q8_kernel: chunks of L blocks, wave-uniform activations in SGPRs,
// exact block dots, waves added in a fixed order.
template <int MR, int L>
__global__ __launch_bounds__(kThreads) void gemv_q8_slice_kernel(
    const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
    float* __restrict__ C, int64_t N, int64_t K, int64_t KB, int64_t ldc, int kb_per_wave,
    int rows) {
  __shared__ float red[kMaxWaves][MR][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int64_t kb0 = static_cast<int64_t>(wave) * kb_per_wave;
  const int64_t kb1 = kb0 + kb_per_wave < KB ? kb0 + kb_per_wave : KB;
  // Slices that share a row group share 128-byte lines of its scale plane:
  // keep neighbours on one XCD (workgroup i runs on XCD i % 8) so that the
  // line comes from HBM once, into that XCD's L2.
  int slice = blockIdx.x;
  if (gridDim.x % 8 == 0) slice = (slice & 7) * (gridDim.x >> 3) + (slice >> 3);
  const int64_t n0 = static_cast<int64_t>(slice) * rows;
  // the row this lane loads: its own, or the slice's last; never past N - 1
  // (when N is a multiple of 64 the packed layout has no padding rows)
  int64_t n = n0 + (lane < rows ? lane : rows - 1);
  n = n < N ? n : N - 1;
  const int64_t g = n >> 6, r = n & 63;

  const v4u* wp = reinterpret_cast<const v4u*>(wq + g * KB * kGroupBlockBytes) + r;
  const uint16_t* sp = ws + g * KB * kGroupRows + r;

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
  for (int t = threadIdx.x; t < MR * 64; t += blockDim.x) {
    const int m = t >> 6, l = t & 63;
    if (l >= rows) continue;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += red[w][m][l];
    const int64_t nn = n0 + l;
    if (nn < N) C[m * ldc + nn] = sum;
  }
}

// Rows per workgroup of the slice kernels: enough workgroups for the 256
// CUs, a multiple of 8, at most one 64-row group.
inline int slice_rows(int64_t N) {
  int64_t rows = (N + 255) / 256;
  rows = ((rows + 7) / 8) * 8;
  return static_cast<int>(rows > kGroupRows ? kGroupRows : rows);
}

template <int MR, int L>
hipError_t launch_slice(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                        const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < kMaxWaves ? KB : kMaxWaves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  const int rows = slice_rows(N);
  const int64_t grid = (N + rows - 1) / rows;
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  hipLaunchKernelGGL((gemv_q8_slice_kernel<MR, L>), dim3(static_cast<uint32_t>(grid)),
                     dim3(waves * 64), 0, stream, q_a, d_a, w_packed, ws, C, N, K, KB, ldc,
                     kb_per_wave, rows);
  return hipGetLastError();
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
    int64_t ldc, int kb_per_wave, int rows, int8_t* __restrict__ q_out,
    uint16_t* __restrict__ d_out) {
  constexpr int kSlotBytes = MR * L * (kQK + 4);   // per wave: codes, then binary32 scales
  constexpr int kItems = MR * L * 4;               // quantiser lanes per chunk (4 per block)
  constexpr int kPasses = (kItems + 63) / 64;
  __shared__ __align__(16) uint8_t lds[kMaxWaves * (kSlotBytes > MR * 256 ? kSlotBytes : MR * 256)];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int64_t kb0 = static_cast<int64_t>(wave) * kb_per_wave;
  const int64_t kb1 = kb0 + kb_per_wave < KB ? kb0 + kb_per_wave : KB;
  const bool store_q = q_out != nullptr && blockIdx.x == 0;
  // rows (and their order over the XCDs) as in gemv_q8_slice_kernel
  int slice = blockIdx.x;
  if (gridDim.x % 8 == 0) slice = (slice & 7) * (gridDim.x >> 3) + (slice >> 3);
  const int64_t n0 = static_cast<int64_t>(slice) * rows;
  int64_t n = n0 + (lane < rows ? lane : rows - 1);
  n = n < N ? n : N - 1;
  const int64_t g = n >> 6, r = n & 63;

  uint8_t* const qslot = lds + wave * kSlotBytes;
  float* const dslot = reinterpret_cast<float*>(qslot + MR * L * kQK);

  const v4u* wp = reinterpret_cast<const v4u*>(wq + g * KB * kGroupBlockBytes) + r;
  const uint16_t* sp = ws + g * KB * kGroupRows + r;

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
    const int m = t >> 6, l = t & 63;
    if (l >= rows) continue;
    float sum = 0.0f;
    for (int w = 0; w < nwaves; ++w) sum += red[(w * MR + m) * 64 + l];
    const int64_t nn = n0 + l;
    if (nn < N) C[m * ldc + nn] = sum;
  }
}

template <int MR, int L, bool NT, bool kSwiglu = false>
hipError_t launch_m(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                    const uint8_t* w_packed, float* C, int64_t ldc, int max_waves,
                    hipStream_t stream, int8_t* q_h = nullptr, uint16_t* d_h = nullptr) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < max_waves ? KB : max_waves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  hipLaunchKernelGGL((gemv_q8_kernel<MR, L, NT, kSwiglu>), dim3(static_cast<uint32_t>(NG)),
                     dim3(waves * 64), 0, stream, q_a, d_a, w_packed, ws, C, N, K, KB, ldc,
                     kb_per_wave, q_h, d_h);
  return hipGetLastError();
}

template <int MR>
hipError_t launch_cfg(int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                      const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  // Q8_GEMV_CFG=<c> (benchmarking aid): c = 0: row slices sized to fill
  // the CUs, 16 waves, nontemporal weight loads, chunks of 8 blocks at M = 1
  // (all of a wave's blocks at K = 4096), 4 at M = 2..3 and 2 from M = 4 on,
  // where the activation operands of a chunk take more scalar registers
  // (measured at N12288 K4096: M1 10.13 vs 10.30 us with chunks of 4, M4
  // 10.69 vs 10.90, M6 12.0 vs 13.0) (default); 1: one workgroup per 64-row
  // group, chunks of 4; 2: as 1 with ordinary loads; 3: as 1 with chunks of
  // 8; 4: row slices with chunks of 4.  The chunk size does not change the
  // order of any sum.
  const int forced = env_index("Q8_GEMV_CFG");
  const int cfg = forced > 4 ? 0 : (forced < 0 ? 0 : forced);
  if (log_enabled())
    fprintf(stderr, "q8: product M=%d N=%lld K=%lld: decode kernel, configuration %d\n", MR,
            static_cast<long long>(N), static_cast<long long>(K), cfg);
  switch (cfg) {
    case 1: return launch_m<MR, 4, true>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
    case 2: return launch_m<MR, 4, false>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
    case 3: return launch_m<MR, 8, true>(N, K, q_a, d_a, w_packed, C, ldc, 16, stream);
    case 4: return launch_slice<MR, 4>(N, K, q_a, d_a, w_packed, C, ldc, stream);
    default:
      return launch_slice<MR, MR == 1 ? 8 : (MR <= 3 ? 4 : 2)>(N, K, q_a, d_a, w_packed, C, ldc,
                                                                stream);
  }
}

template <int MR>
hipError_t launch_act_m(const void* x, bool bf16, int64_t ldx, int64_t N, int64_t K,
                        const uint8_t* w_packed, float* C, int64_t ldc, int8_t* q_out,
                        uint16_t* d_out, hipStream_t stream) {
  // Chunks of 8 blocks at M = 1 (11.1 vs 11.5 us at N12288 K4096), else 4:
  // with the quantisation of each chunk in the loop, smaller chunks did not
  // pay here as they do in the unfused kernel (M4: 13.5 vs 12.2 us).
  constexpr int L = MR == 1 ? 8 : 4;
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const int waves = static_cast<int>(KB < kMaxWaves ? KB : kMaxWaves);
  const int kb_per_wave = static_cast<int>((KB + waves - 1) / waves);
  // Every workgroup quantises the whole activation, so above M = 4 the
  // extra workgroups of row slices cost more than they gain: whole groups.
  const int rows = MR > 4 ? kGroupRows : slice_rows(N);
  const uint32_t grid = static_cast<uint32_t>((N + rows - 1) / rows);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  if (bf16)
    hipLaunchKernelGGL((gemv_q8_act_kernel<MR, L, true>), dim3(grid), dim3(waves * 64), 0,
                       stream, x, ldx, w_packed, ws, C, N, K, KB, ldc, kb_per_wave, rows, q_out,
                       d_out);
  else
    hipLaunchKernelGGL((gemv_q8_act_kernel<MR, L, false>), dim3(grid), dim3(waves * 64), 0,
                       stream, x, ldx, w_packed, ws, C, N, K, KB, ldc, kb_per_wave, rows, q_out,
                       d_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_swiglu(int M, int64_t I, int64_t K, const int8_t* q_a,
                              const uint16_t* d_a, const uint8_t* w_packed, int8_t* q_h,
                              uint16_t* d_h, hipStream_t stream) {
  const int64_t N = 2 * I;
  if (log_enabled())
    fprintf(stderr, "q8: gated step M=%d I=%lld K=%lld: decode kernel, one workgroup per group\n",
            M, static_cast<long long>(I), static_cast<long long>(K));
#define Q8_SWIGLU_M(MR)                                                                     \
  case MR:                                                                                  \
    return launch_m<MR, 4, true, true>(N, K, q_a, d_a, w_packed, nullptr, 0, 16, stream, q_h, \
                                       d_h);
  switch (M) {
    Q8_SWIGLU_M(1)
    Q8_SWIGLU_M(2)
    Q8_SWIGLU_M(3)
    Q8_SWIGLU_M(4)
    Q8_SWIGLU_M(5)
    Q8_SWIGLU_M(6)
    Q8_SWIGLU_M(7)
    Q8_SWIGLU_M(8)
    default: return hipErrorInvalidValue;
  }
#undef Q8_SWIGLU_M
}

hipError_t launch_gemv_act(int M, const void* x, int dtype, int64_t ldx, int64_t N, int64_t K,
                           const uint8_t* w_packed, float* C, int64_t ldc, int8_t* q_out,
                           uint16_t* d_out, hipStream_t stream) {
  const bool bf16 = dtype == 1;
  if (log_enabled())
    fprintf(stderr, "q8: quantise+product M=%d N=%lld K=%lld: fused decode kernel\n", M,
            static_cast<long long>(N), static_cast<long long>(K));
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
