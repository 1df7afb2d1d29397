// q8_kernels.h -- internal declarations shared by the HIP sources of libq8gemm
// (not installed; the public interface is include/q8.h).
//
// The operation is the Q8_0 weight x activation product described in
// include/q8.h (news.hada.io topic 29953, "CUDA inference engine for running
// Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)": GEMM item of the
// list of non-throttled paths; Q8_0 as the supported format in the benchmark
// and limitations lists).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kQK = 32;            // values per Q8_0 block along K
constexpr int kGroupRows = 64;     // output features per packed row group
constexpr int kPieceBytes = 1024;  // one (group, block, half) piece: 64 rows x 16 B
constexpr int kGroupBlockBytes = 2 * kPieceBytes;  // quant bytes per (group, block)

// Launchers (q8_quantize.hip, q8_pack.hip, q8_gemv.hip, q8_gemm.hip).  Shapes
// are validated by the caller; each returns the launch's hipError_t.
hipError_t launch_quantize(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                           int8_t* q, uint16_t* d, hipStream_t stream);
hipError_t launch_pack(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* packed,
                       hipStream_t stream);
// Gate and up weights ([I][K/32] blocks each) packed as their 2I interleaved
// rows: 64-row group g = gate rows 32g..32g+31, then up rows 32g..32g+31.
hipError_t launch_pack_gateup(const uint8_t* gate, const uint8_t* up, int64_t I, int64_t K,
                              uint8_t* packed, hipStream_t stream);
// Gated FFN step on gate/up-packed weights: q_h/d_h = Q8_0(silu(A Wg^T) * (A Wu^T)).
hipError_t launch_gemm_swiglu(int64_t M, int64_t I, int64_t K, const int8_t* q_a,
                              const uint16_t* d_a, const uint8_t* w_packed, int8_t* q_h,
                              uint16_t* d_h, hipStream_t stream);
hipError_t launch_gemv_swiglu(int M, int64_t I, int64_t K, const int8_t* q_a,
                              const uint16_t* d_a, const uint8_t* w_packed, int8_t* q_h,
                              uint16_t* d_h, hipStream_t stream);
hipError_t launch_gemv(int M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream);
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream);
// Fused decode step (M <= kGemvMaxM): quantise x and multiply; q_out/d_out
// may be NULL, else they receive the quantised rows.
hipError_t launch_gemv_act(int M, const void* x, int dtype, int64_t ldx, int64_t N, int64_t K,
                           const uint8_t* w_packed, float* C, int64_t ldc, int8_t* q_out,
                           uint16_t* d_out, hipStream_t stream);
// Quantise-and-multiply for kGemvMaxM < M <= 64 in one kernel (the small-M
// kernel quantising its own chunks), taken only when Q8_GEMM_ACT_FUSED=1;
// small_act_applies() tells whether a call takes it (otherwise quantise,
// then multiply).
bool small_act_applies(int64_t M, int dtype, int64_t ldx);
hipError_t launch_small_act(int64_t M, const void* x, int dtype, int64_t ldx, int64_t N,
                            int64_t K, const uint8_t* w_packed, float* C, int64_t ldc,
                            int8_t* q_out, uint16_t* d_out, hipStream_t stream);

// Block-sparse causal attention (q8_attn.hip); D in {64, 128}, 64-token blocks.
hipError_t launch_attn_pool(const uint16_t* x, int64_t L, int64_t ldx, int64_t H, int64_t D,
                            float* pooled, hipStream_t stream);
hipError_t launch_attn_select(const float* pq, const float* pk, int64_t Hq, int64_t Hkv, int64_t NB,
                              int64_t D, int k, int kmax, int32_t* idx, int32_t* cnt,
                              hipStream_t stream);
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t L,
                           int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t D,
                           const int32_t* idx, const int32_t* cnt, int kmax, int out_dtype,
                           void* out, int64_t ldo, hipStream_t stream);

// 3-bit KV-cache codec (q8_kv3.hip); D in {64, 128, 256}.
hipError_t launch_kv3_encode(const void* x, int dtype, int64_t R, int64_t D, int64_t ldx,
                             uint8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_kv3_decode(const uint8_t* codes, const float* scales, int64_t R, int64_t D,
                             int dtype, void* out, int64_t ldo, hipStream_t stream);

constexpr int kGemvMaxM = 8;       // M <= kGemvMaxM takes the decode kernel

// Q8_LOG set (and not "0") in the environment: the launchers print their
// dispatch decision (kernel and configuration) to stderr, one line per call.
bool log_enabled();

// A plain non-negative decimal number from the environment (at most 1000),
// or -1 when the variable is unset or anything else.
int env_index(const char* name);

inline int64_t num_groups(int64_t N) { return (N + kGroupRows - 1) / kGroupRows; }

// binary16 bits -> binary32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// binary32 -> binary16 bits, round to nearest even, binary16 subnormals kept
// (v_cvt_f16_f32 under the default rounding and denormal modes).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// ---------------------------------------------------------------------------
// The Q8_0 block quantiser, shared by the quantise kernel and the fused
// decode kernel so that both produce the same bits.  Four consecutive,
// 4-aligned lanes of a wave hold the 32 values of one block, eight each.
//
// Bit-exactness: d32 = amax/127 and id = 1/d32 use the correctly rounded
// binary32 division (HIP's default; never build with fast-math or
// -fno-hip-fp32-correctly-rounded-divide-sqrt), v = x*id is a single
// multiply, roundf rounds half away from zero, and the binary16 conversion
// is v_cvt_f16_f32 (round to nearest even, binary16 subnormals kept).
// ---------------------------------------------------------------------------

// Eight consecutive values of row data x (binary32, or bfloat16 widened
// exactly) starting at element off.
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

// A block's scale from its maximum magnitude: d32 = amax/127; id = 1/d32
// and the binary16 bits of d32.  Returns false (codes 0, d = +0) when
// d32 < FLT_MIN (an all-zero block, or a binary32-subnormal scale).
__device__ __forceinline__ bool block_scale(float amax, float& id, uint16_t& dbits) {
  const float d32 = amax / 127.0f;
  if (!(d32 >= 1.17549435e-38f)) {   // FLT_MIN
    id = 0.0f;
    dbits = 0;
    return false;
  }
  id = 1.0f / d32;
  dbits = f32_to_f16_bits(d32);
  return true;
}

// A value's code: v * id rounded half away from zero (|code| <= 127).
__device__ __forceinline__ int block_code(float v, float id) {
  return static_cast<int>(roundf(v * id));
}

// Quantise the lane's eight values of a block: codes packed little-endian
// into lo (values 0..3) and hi (4..7), and the block's binary16 scale bits.
// All four lanes of every block must be active.
__device__ __forceinline__ void quantize8(const float v[8], uint32_t& lo, uint32_t& hi,
                                          uint16_t& dbits) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
  float id;
  lo = 0;
  hi = 0;
  if (block_scale(amax, id, dbits)) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = static_cast<uint32_t>(block_code(v[i], id)) & 0xffu;
    lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  }
}

// ---------------------------------------------------------------------------
// Gated feed-forward step applied to the gate and up products g, u of one
// hidden unit: h = silu(g) * u, silu(x) = x / (1 + e^-x), in binary32
// (device expf, correctly rounded division, one rounding for the product);
// then h is quantised like an activation, in blocks of 32 hidden units that
// sit in 32 consecutive, 32-aligned lanes of a wave (one value each).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Every lane of the 32-lane group must take part (lane exchanges).  Returns
// the lane's code; dbits receives the block's scale bits.
__device__ __forceinline__ int quantize_lane32(float h, uint16_t& dbits) {
  float amax = fabsf(h);
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 32));
  float id;
  return block_scale(amax, id, dbits) ? block_code(h, id) : 0;
}

}  // namespace q8
