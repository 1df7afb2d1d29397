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
hipError_t launch_gemv(int M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream);
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream);

constexpr int kGemvMaxM = 8;       // M <= kGemvMaxM takes the decode kernel

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

}  // namespace q8
