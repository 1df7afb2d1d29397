// q8_gemm.hip -- prefill path of the Q8_0 product on the int8 matrix cores.
//
// C[m][n] = sum_kb d_a[m][kb] d_w[n][kb] int32(sum_j q_a q_w).  The source
// engine runs its prefill GEMMs on int8 dot products because its card's
// matrix units are throttled (news.hada.io topic 29953, "CUDA inference
// engine for running Qwen3.5/3.6 hybrid models on mining cards (CMP
// 100-210)": tensor-core item of the list of what is locked, GEMM item of
// the list of non-throttled paths).  MI355X has full-rate int8 matrix
// cores, so here the block dots run on v_mfma_i32_32x32x32_i8, whose K of
// 32 is exactly one Q8_0 block: one instruction gives the exact int32 dot
// of one block for a 32x32 output tile.
//
// Scale epilogue (the binding cost).  Each 32x32 int32 partial needs its
// two per-block scales applied and must be accumulated in binary32.  The
// accumulator input of the MFMA is preset to the bits of 1.5*2^23, so the
// int32 result, read as binary32, is exactly 1.5*2^23 + P (|P| < 2^22).
// Then
//     y   = fma(Pbits, d_w, -1.5*2^23*d_w)   = RN(P * d_w)     (one rounding)
//     acc = fma(y, d_a, acc)                                     (one rounding)
// i.e. two VALU operations per output and block, with no int->float
// conversion.  d_w is per lane (lane = output column) and -1.5*2^23*d_w is
// exact (d_w has 11 significant bits).  With unpacked binary32 FMAs (16
// lanes per clock per SIMD) against 1024 int8 MACs per clock per SIMD this
// epilogue caps the kernel at 1/4 of the int8 matrix-core peak; the kernel
// is organised to keep the VALU busy and everything else off it.
//
// Tiling.  A workgroup of 4 waves computes a BM x BN = 128 x 128 tile; each
// wave a 64 x 64 sub-tile (2 x 2 MFMA tiles).  K advances in stages of
// KBS = 4 blocks.  Per stage, q_a rows, packed weight pieces and both scale
// vectors are staged HBM -> registers -> LDS, double buffered, so global
// loads of stage s+1 are in flight while stage s computes.  LDS holds each
// operand as 16-byte slices in [block][half][row] order, so a fragment load
// (lane l: row l%32, half l/32) reads 512 contiguous bytes per half-wave.
// Activation scales are widened to binary32 once, when staged.
//
// Workgroup order: tiles run M-fastest so consecutive workgroups share a
// weight tile; when the grid is a multiple of 8 the ids are remapped so
// each of the 8 XCDs (which receive workgroups round-robin) gets one
// contiguous range of tiles and keeps its weight tiles in its own L2.
#include "q8_kernels.h"

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, KBS = 4;
constexpr int kWaves = 4, kThreads = kWaves * 64;
constexpr int WM = 64, WN = 64;                 // per-wave tile
constexpr int TM = WM / 32, TN = WN / 32;       // MFMA tiles per wave
constexpr int kSlots = 2 * KBS;                 // 16-byte slots per row per stage

// LDS per stage (bytes)
constexpr int kAq = KBS * 2 * BM * 16;          // activation quants
constexpr int kBq = KBS * 2 * BN * 16;          // weight quants
constexpr int kAs = KBS * BM * 4;               // activation scales (binary32)
constexpr int kBs = KBS * BN * 4;               // weight scales (binary32)
constexpr int kStage = kAq + kBq + kAs + kBs;

constexpr int kALoads = BM * kSlots / kThreads;         // 16-byte A loads per thread
constexpr int kBLoads = BN * kSlots / kThreads;         // 16-byte B loads per thread
constexpr int kASc = BM * KBS / kThreads;               // A scales per thread
constexpr int kBSc = BN * KBS / kThreads;               // B scales per thread
static_assert(kALoads * kThreads == BM * kSlots, "A staging");
static_assert(kBLoads * kThreads == BN * kSlots, "B staging");
static_assert(kASc * kThreads == BM * KBS && kBSc * kThreads == BN * KBS, "scale staging");

constexpr float kBias = 12582912.0f;            // 1.5 * 2^23
constexpr int kBiasBits = 0x4B400000;

struct Staged {
  uint4 a[kALoads];
  uint4 b[kBLoads];
  float as[kASc];
  float bs[kBSc];
};

__device__ __forceinline__ void load_stage(Staged& st, int tid, int64_t m0, int64_t g0,
                                           int64_t kb0, int64_t M, int64_t K, int64_t KB,
                                           int64_t NG, const int8_t* __restrict__ q_a,
                                           const uint16_t* __restrict__ d_a,
                                           const uint8_t* __restrict__ wq,
                                           const uint16_t* __restrict__ ws) {
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int idx = i * kThreads + tid;
    const int m = (idx & 15) + 16 * (idx >> 7);
    const int s = (idx >> 4) & (kSlots - 1);
    const int64_t row = m0 + m, kb = kb0 + (s >> 1);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < M && kb < KB)
      v = *reinterpret_cast<const uint4*>(q_a + row * K + kb0 * kQK + s * 16);
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int idx = i * kThreads + tid;
    const int piece = idx >> 6, lane = idx & 63;
    const int gl = piece / (2 * KBS);
    const int kbl = (piece >> 1) % KBS;
    const int h = piece & 1;
    const int64_t g = g0 + gl, kb = kb0 + kbl;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (g < NG && kb < KB)
      v = reinterpret_cast<const uint4*>(wq + ((g * KB + kb) * 2 + h) * kPieceBytes)[lane];
    st.b[i] = v;
  }
#pragma unroll
  for (int i = 0; i < kASc; ++i) {
    const int idx = i * kThreads + tid;
    const int m = idx % BM, kbl = idx / BM;
    const int64_t row = m0 + m, kb = kb0 + kbl;
    st.as[i] = (row < M && kb < KB) ? f16_bits_to_f32(d_a[row * KB + kb]) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kBSc; ++i) {
    const int idx = i * kThreads + tid;
    const int n = idx % BN, kbl = idx / BN;
    const int64_t g = g0 + n / kGroupRows, kb = kb0 + kbl;
    st.bs[i] = (g < NG && kb < KB) ? f16_bits_to_f32(ws[(g * KB + kb) * kGroupRows + n % kGroupRows])
                                   : 0.0f;
  }
}

__device__ __forceinline__ void store_stage(const Staged& st, int tid, uint8_t* buf) {
  uint4* aq = reinterpret_cast<uint4*>(buf);
  uint4* bq = reinterpret_cast<uint4*>(buf + kAq);
  float* as = reinterpret_cast<float*>(buf + kAq + kBq);
  float* bs = reinterpret_cast<float*>(buf + kAq + kBq + kAs);
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int idx = i * kThreads + tid;
    const int m = (idx & 15) + 16 * (idx >> 7);
    const int s = (idx >> 4) & (kSlots - 1);
    aq[s * BM + m] = st.a[i];                 // [kb][h][row], s = 2*kb + h
  }
#pragma unroll
  for (int i = 0; i < kBLoads; ++i) {
    const int idx = i * kThreads + tid;
    const int piece = idx >> 6, lane = idx & 63;
    const int gl = piece / (2 * KBS);
    const int kbl = (piece >> 1) % KBS;
    const int h = piece & 1;
    bq[(kbl * 2 + h) * BN + gl * kGroupRows + lane] = st.b[i];
  }
#pragma unroll
  for (int i = 0; i < kASc; ++i) as[i * kThreads + tid] = st.as[i];   // [kb][row]
#pragma unroll
  for (int i = 0; i < kBSc; ++i) bs[i * kThreads + tid] = st.bs[i];   // [kb][col]
}

__global__ __launch_bounds__(kThreads, 2) void gemm_q8_mfma_kernel(
    const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws, float* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t KB, int64_t NG, int64_t ldc, int tiles_m,
    int remap) {
  __shared__ __align__(16) uint8_t smem[2 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware order: hardware id i lands on XCD i % 8; give each XCD a
  // contiguous range of logical tiles.
  int bid = blockIdx.x;
  if (remap) {
    const int per = gridDim.x >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  const int tm = bid % tiles_m, tn = bid / tiles_m;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t g0 = n0 / kGroupRows;

  const int wm0 = (wave & 1) * WM;            // wave's rows within the tile
  const int wn0 = (wave >> 1) * WN;           // wave's columns within the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;

  float acc[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;

  const int64_t nstages = (KB + KBS - 1) / KBS;
  Staged st;
  load_stage(st, tid, m0, g0, 0, M, K, KB, NG, q_a, d_a, wq, ws);
  store_stage(st, tid, smem);
  __syncthreads();

  for (int64_t s = 0; s < nstages; ++s) {
    uint8_t* cur = smem + (s & 1) * kStage;
    uint8_t* nxt = smem + ((s + 1) & 1) * kStage;
    const bool more = s + 1 < nstages;
    if (more) load_stage(st, tid, m0, g0, (s + 1) * KBS, M, K, KB, NG, q_a, d_a, wq, ws);

    const uint4* aq = reinterpret_cast<const uint4*>(cur);
    const uint4* bq = reinterpret_cast<const uint4*>(cur + kAq);
    const float* as = reinterpret_cast<const float*>(cur + kAq + kBq);
    const float* bs = reinterpret_cast<const float*>(cur + kAq + kBq + kAs);

#pragma unroll 1
    for (int kb = 0; kb < KBS; ++kb) {
      v4i af[TM], bf[TN];
      float av[TM][16];
      float wv[TN], nwv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4 u = aq[(kb * 2 + half) * BM + wm0 + 32 * i + l32];
        af[i] = v4i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z),
                    static_cast<int>(u.w)};
        // Rows held by this lane in the MFMA output: 8*(r/4) + 4*half + r%4.
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 f = *reinterpret_cast<const float4*>(
              as + kb * BM + wm0 + 32 * i + 8 * q4 + 4 * half);
          av[i][4 * q4 + 0] = f.x;
          av[i][4 * q4 + 1] = f.y;
          av[i][4 * q4 + 2] = f.z;
          av[i][4 * q4 + 3] = f.w;
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint4 u = bq[(kb * 2 + half) * BN + wn0 + 32 * j + l32];
        bf[j] = v4i{static_cast<int>(u.x), static_cast<int>(u.y), static_cast<int>(u.z),
                    static_cast<int>(u.w)};
        wv[j] = bs[kb * BN + wn0 + 32 * j + l32];
        nwv[j] = -kBias * wv[j];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], bias, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = fmaf(__int_as_float(p[r]), wv[j], nwv[j]);
            acc[i][j][r] = fmaf(y, av[i][r], acc[i][j][r]);
          }
        }
    }

    if (more) store_stage(st, tid, nxt);
    __syncthreads();
  }

  // Output: lane holds column wn0 + 32j + l32 and rows 8*(r/4) + 4*half + r%4.
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn0 + 32 * j + l32;
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < M) C[row * ldc + col] = acc[i][j][r];
      }
  }
}

}  // namespace

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t grid = tiles_m * tiles_n;
  const int remap = (grid % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(gemm_q8_mfma_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0,
                     stream, q_a, d_a, w_packed, ws, C, M, N, K, KB, NG, ldc,
                     static_cast<int>(tiles_m), remap);
  return hipGetLastError();
}

}  // namespace q8
