// q8_api.hip -- the C ABI of libq8gemm (declared and documented in
// include/q8.h): host-side argument checks, the one-time device check,
// dispatch and launch.  No allocation, no synchronisation.
#include <atomic>
#include <mutex>
#include <cstdlib>
#include <cstring>

#include "q8.h"

#include "q8_kernels.h"

namespace q8 {
bool log_enabled() {
  const char* e = getenv("Q8_LOG");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0');
}

int env_index(const char* name) {
  const char* e = getenv(name);
  if (e == nullptr || *e == '\0') return -1;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  if (*end != '\0' || v < 0 || v > 1000) return -1;
  return static_cast<int>(v);
}
}  // namespace q8

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else
std::atomic<int> g_device_ok[kMaxDevices];

q8_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q8_ERR_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return Q8_ERR_DEVICE;
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? Q8_OK : Q8_ERR_DEVICE;
}

// Workspace of q8_gemm_act_noalloc: the quantised rows (int8 q, then the
// binary16 scales at a 256-byte boundary) between its two kernels, for
// callers that cannot allocate.  One copy per GPU, for the life of the
// process; every call on a GPU uses it, so calls that overlap on one GPU
// race.  Host code never uses the array's name as an address: each device's
// copy is looked up once with hipGetSymbolAddress (with that device
// current) and only that address is passed to kernels.
constexpr size_t kScratchBytes = size_t(48) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<uint8_t*> g_scratch[kMaxDevices];

// The current device's copy of the workspace, or nullptr if the lookup
// fails.  Call after check_device().
uint8_t* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return nullptr;
    p = static_cast<uint8_t*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Offset of the scales in the workspace after M x K int8 codes.
size_t scratch_scale_offset(int64_t M, int64_t K) {
  return (static_cast<size_t>(M * K) + 255) & ~size_t(255);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Sizes the kernels index with 32-bit grids and 64-bit offsets: keep every
// launch's workgroup count below 2^31.
constexpr int64_t kMaxDim = int64_t(1) << 31;

// K is bounded so that 32-bit buffer offsets cover a 256-row tile of q_a.
constexpr int64_t kMaxK = int64_t(1) << 24;

bool valid_k(int64_t K) { return K >= 32 && K % 32 == 0 && K <= kMaxK; }

bool valid_head_dim(int64_t D) { return D == 64 || D == 128 || D == 256; }
bool valid_attn_dim(int64_t D) { return D == 64 || D == 128; }
// attention: 64-token blocks, at most 4096 of them (262144 tokens); row
// pitches below 2^24 elements, so that 64 rows of a block fit a 32-bit
// buffer range
constexpr int64_t kMaxAttnBlocks = 4096;
constexpr int64_t kMaxAttnLd = int64_t(1) << 24;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* q8_status_string(q8_status s) {
  switch (s) {
    case Q8_OK: return "ok";
    case Q8_ERR_NULL: return "null pointer argument";
    case Q8_ERR_SHAPE: return "invalid shape (need K % 32 == 0, K >= 32, N >= 1, M >= 0, ld >= row length)";
    case Q8_ERR_ALIGN: return "misaligned pointer or row pitch";
    case Q8_ERR_DTYPE: return "unknown dtype";
    case Q8_ERR_SIZE: return "packed buffer too small, or rows too many for the static workspace";
    case Q8_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case Q8_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

q8_status q8_pack_weights(const void* w_blocks, int64_t N, int64_t K, void* w_packed,
                          size_t* packed_bytes, void* stream) {
  if (packed_bytes == nullptr) return Q8_ERR_NULL;
  if (N < 1 || N >= kMaxDim || !valid_k(K)) return Q8_ERR_SHAPE;
  const int64_t NG = q8::num_groups(N);
  const int64_t KB = K / q8::kQK;
  const size_t need = static_cast<size_t>(NG * KB) * (q8::kGroupBlockBytes + 2 * q8::kGroupRows);
  if (w_packed == nullptr) {
    *packed_bytes = need;
    return Q8_OK;
  }
  if (w_blocks == nullptr) return Q8_ERR_NULL;
  if (!aligned(w_packed, 16)) return Q8_ERR_ALIGN;
  if (*packed_bytes < need) return Q8_ERR_SIZE;
  if (NG * KB * 2 * q8::kGroupRows / 256 >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_pack(static_cast<const uint8_t*>(w_blocks), N, K,
                         static_cast<uint8_t*>(w_packed), as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_quantize_act(const void* x, q8_dtype dtype, int64_t M, int64_t K, int64_t ldx,
                          int8_t* q, uint16_t* d, void* stream) {
  if (dtype != Q8_F32 && dtype != Q8_BF16) return Q8_ERR_DTYPE;
  if (M < 0 || !valid_k(K) || ldx < K) return Q8_ERR_SHAPE;
  if (M == 0) return Q8_OK;
  if (x == nullptr || q == nullptr || d == nullptr) return Q8_ERR_NULL;
  const int64_t esize = dtype == Q8_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(q, 16) || !aligned(d, 2))
    return Q8_ERR_ALIGN;
  if (M * (K / q8::kQK) * 4 / 256 >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_quantize(x, static_cast<int>(dtype), M, K, ldx, q, d, as_stream(stream)) ==
                 hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_gemm(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                  const void* w_packed, float* C, int64_t ldc, void* stream) {
  if (M < 0 || N < 1 || N >= kMaxDim || !valid_k(K) || ldc < N) return Q8_ERR_SHAPE;
  if (M == 0) return Q8_OK;
  if (q_a == nullptr || d_a == nullptr || w_packed == nullptr || C == nullptr) return Q8_ERR_NULL;
  if (!aligned(q_a, 16) || !aligned(d_a, 2) || !aligned(w_packed, 16) || !aligned(C, 4))
    return Q8_ERR_ALIGN;
  // workgroup count of the matrix-core kernel: ceil(M/128) * ceil(N/128)
  if (((M + 127) / 128) * ((N + 127) / 128) >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  const uint8_t* wp = static_cast<const uint8_t*>(w_packed);
  hipError_t e;
  if (M <= q8::kGemvMaxM)
    e = q8::launch_gemv(static_cast<int>(M), N, K, q_a, d_a, wp, C, ldc, as_stream(stream));
  else
    e = q8::launch_gemm(M, N, K, q_a, d_a, wp, C, ldc, as_stream(stream));
  return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH;
}

q8_status q8_pack_weights_gateup(const void* w_gate, const void* w_up, int64_t I, int64_t K,
                                 void* w_packed, size_t* packed_bytes, void* stream) {
  if (packed_bytes == nullptr) return Q8_ERR_NULL;
  if (I < 32 || I % 32 != 0 || 2 * I >= kMaxDim || !valid_k(K)) return Q8_ERR_SHAPE;
  const int64_t NG = q8::num_groups(2 * I);
  const int64_t KB = K / q8::kQK;
  const size_t need = static_cast<size_t>(NG * KB) * (q8::kGroupBlockBytes + 2 * q8::kGroupRows);
  if (w_packed == nullptr) {
    *packed_bytes = need;
    return Q8_OK;
  }
  if (w_gate == nullptr || w_up == nullptr) return Q8_ERR_NULL;
  if (!aligned(w_packed, 16)) return Q8_ERR_ALIGN;
  if (*packed_bytes < need) return Q8_ERR_SIZE;
  if (NG * KB * 2 * q8::kGroupRows / 256 >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_pack_gateup(static_cast<const uint8_t*>(w_gate),
                                static_cast<const uint8_t*>(w_up), I, K,
                                static_cast<uint8_t*>(w_packed), as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_gemm_swiglu(int64_t M, int64_t I, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                         const void* w_packed, int8_t* q_h, uint16_t* d_h, void* stream) {
  if (M < 0 || I < 32 || I % 32 != 0 || 2 * I >= kMaxDim || !valid_k(K)) return Q8_ERR_SHAPE;
  if (M == 0) return Q8_OK;
  if (q_a == nullptr || d_a == nullptr || w_packed == nullptr || q_h == nullptr ||
      d_h == nullptr)
    return Q8_ERR_NULL;
  if (!aligned(q_a, 16) || !aligned(d_a, 2) || !aligned(w_packed, 16) || !aligned(q_h, 16) ||
      !aligned(d_h, 2))
    return Q8_ERR_ALIGN;
  if (((M + 127) / 128) * ((2 * I + 127) / 128) >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  const uint8_t* wp = static_cast<const uint8_t*>(w_packed);
  const hipError_t e =
      M <= q8::kGemvMaxM
          ? q8::launch_gemv_swiglu(static_cast<int>(M), I, K, q_a, d_a, wp, q_h, d_h,
                                   as_stream(stream))
          : q8::launch_gemm_swiglu(M, I, K, q_a, d_a, wp, q_h, d_h, as_stream(stream));
  return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH;
}

q8_status q8_gemm_act(const void* x, q8_dtype dtype, int64_t M, int64_t N, int64_t K,
                      int64_t ldx, const void* w_packed, float* C, int64_t ldc, int8_t* q_a,
                      uint16_t* d_a, void* stream) {
  if (dtype != Q8_F32 && dtype != Q8_BF16) return Q8_ERR_DTYPE;
  if (M < 0 || N < 1 || N >= kMaxDim || !valid_k(K) || ldx < K || ldc < N) return Q8_ERR_SHAPE;
  if (M == 0) return Q8_OK;
  if (x == nullptr || w_packed == nullptr || C == nullptr) return Q8_ERR_NULL;
  // q_a and d_a: both or neither; required above the decode size
  if ((q_a == nullptr) != (d_a == nullptr)) return Q8_ERR_NULL;
  if (M > q8::kGemvMaxM && q_a == nullptr) return Q8_ERR_NULL;
  const int64_t esize = dtype == Q8_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(w_packed, 16) || !aligned(C, 4))
    return Q8_ERR_ALIGN;
  if (q_a != nullptr && (!aligned(q_a, 16) || !aligned(d_a, 2))) return Q8_ERR_ALIGN;
  if (M * (K / q8::kQK) * 4 / 256 >= kMaxDim) return Q8_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= kMaxDim) return Q8_ERR_SHAPE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  const uint8_t* wp = static_cast<const uint8_t*>(w_packed);
  hipError_t e;
  if (M <= q8::kGemvMaxM) {
    e = q8::launch_gemv_act(static_cast<int>(M), x, static_cast<int>(dtype), ldx, N, K, wp, C,
                            ldc, q_a, d_a, as_stream(stream));
  } else if (q8::small_act_applies(M, static_cast<int>(dtype), ldx)) {
    e = q8::launch_small_act(M, x, static_cast<int>(dtype), ldx, N, K, wp, C, ldc, q_a, d_a,
                             as_stream(stream));
  } else {
    e = q8::launch_quantize(x, static_cast<int>(dtype), M, K, ldx, q_a, d_a, as_stream(stream));
    if (e == hipSuccess) e = q8::launch_gemm(M, N, K, q_a, d_a, wp, C, ldc, as_stream(stream));
  }
  return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH;
}

q8_status q8_gemm_act_noalloc(const void* x, q8_dtype dtype, int64_t M, int64_t N, int64_t K,
                              int64_t ldx, const void* w_packed, float* C, int64_t ldc,
                              void* stream) {
  if (dtype != Q8_F32 && dtype != Q8_BF16) return Q8_ERR_DTYPE;
  if (M < 0 || N < 1 || N >= kMaxDim || !valid_k(K) || ldx < K || ldc < N) return Q8_ERR_SHAPE;
  if (M == 0) return Q8_OK;
  if (x == nullptr || w_packed == nullptr || C == nullptr) return Q8_ERR_NULL;
  const int64_t esize = dtype == Q8_F32 ? 4 : 2;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(w_packed, 16) || !aligned(C, 4))
    return Q8_ERR_ALIGN;
  if (M * (K / q8::kQK) * 4 / 256 >= kMaxDim) return Q8_ERR_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) >= kMaxDim) return Q8_ERR_SHAPE;
  // the quantised rows must fit the workspace (decode sizes need none)
  if (M > q8::kGemvMaxM &&
      scratch_scale_offset(M, K) + static_cast<size_t>(M * (K / q8::kQK)) * 2 > kScratchBytes)
    return Q8_ERR_SIZE;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  const uint8_t* wp = static_cast<const uint8_t*>(w_packed);
  hipError_t e;
  if (M <= q8::kGemvMaxM) {
    e = q8::launch_gemv_act(static_cast<int>(M), x, static_cast<int>(dtype), ldx, N, K, wp, C,
                            ldc, nullptr, nullptr, as_stream(stream));
  } else {
    uint8_t* ws = scratch_ptr();
    if (ws == nullptr) return Q8_ERR_DEVICE;
    int8_t* q_a = reinterpret_cast<int8_t*>(ws);
    uint16_t* d_a = reinterpret_cast<uint16_t*>(ws + scratch_scale_offset(M, K));
    e = q8::launch_quantize(x, static_cast<int>(dtype), M, K, ldx, q_a, d_a, as_stream(stream));
    if (e == hipSuccess) e = q8::launch_gemm(M, N, K, q_a, d_a, wp, C, ldc, as_stream(stream));
  }
  return e == hipSuccess ? Q8_OK : Q8_ERR_LAUNCH;
}

q8_status q8_kv3_encode(const void* x, q8_dtype dtype, int64_t R, int64_t D, int64_t ldx,
                        uint8_t* codes, float* scales, void* stream) {
  if (dtype != Q8_F32 && dtype != Q8_BF16) return Q8_ERR_DTYPE;
  const int64_t esize = dtype == Q8_F32 ? 4 : 2;
  if (R < 0 || !valid_head_dim(D) || ldx < D || (R + 3) / 4 >= kMaxDim ||
      ldx * esize * 64 >= (int64_t(1) << 31))
    return Q8_ERR_SHAPE;
  if (R == 0) return Q8_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return Q8_ERR_NULL;
  if (!aligned(x, 16) || (ldx * esize) % 16 != 0 || !aligned(codes, 16) || !aligned(scales, 4))
    return Q8_ERR_ALIGN;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_kv3_encode(x, static_cast<int>(dtype), R, D, ldx, codes, scales,
                               as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_kv3_decode(const uint8_t* codes, const float* scales, int64_t R, int64_t D,
                        q8_dtype out_dtype, void* out, int64_t ldo, void* stream) {
  if (out_dtype != Q8_F32 && out_dtype != Q8_BF16) return Q8_ERR_DTYPE;
  const int64_t esize = out_dtype == Q8_F32 ? 4 : 2;
  if (R < 0 || !valid_head_dim(D) || ldo < D || (R + 3) / 4 >= kMaxDim ||
      ldo * esize * 64 >= (int64_t(1) << 31))
    return Q8_ERR_SHAPE;
  if (R == 0) return Q8_OK;
  if (codes == nullptr || scales == nullptr || out == nullptr) return Q8_ERR_NULL;
  if (!aligned(out, 16) || (ldo * esize) % 16 != 0 || !aligned(codes, 16) || !aligned(scales, 4))
    return Q8_ERR_ALIGN;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_kv3_decode(codes, scales, R, D, static_cast<int>(out_dtype), out, ldo,
                               as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_attn_pool(const void* x, int64_t L, int64_t ldx, int64_t H, int64_t D, float* pooled,
                       void* stream) {
  if (L < 0 || H < 1 || !valid_attn_dim(D) || ldx < H * D || ldx >= kMaxAttnLd) return Q8_ERR_SHAPE;
  if (L == 0) return Q8_OK;
  const int64_t NB = (L + 63) / 64;
  if (NB > kMaxAttnBlocks || H * NB >= kMaxDim) return Q8_ERR_SHAPE;
  if (x == nullptr || pooled == nullptr) return Q8_ERR_NULL;
  if (!aligned(x, 16) || (ldx * 2) % 16 != 0 || !aligned(pooled, 16)) return Q8_ERR_ALIGN;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_attn_pool(static_cast<const uint16_t*>(x), L, ldx, H, D, pooled,
                              as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_attn_select(const float* pooled_q, const float* pooled_k, int64_t Hq, int64_t Hkv,
                         int64_t NB, int64_t D, int k, int kmax, int32_t* idx, int32_t* cnt,
                         void* stream) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || NB < 0 || NB > kMaxAttnBlocks || !valid_attn_dim(D) ||
      k < 2 || kmax < k || Hkv * NB >= kMaxDim)
    return Q8_ERR_SHAPE;
  if (NB == 0) return Q8_OK;
  if (pooled_q == nullptr || pooled_k == nullptr || idx == nullptr || cnt == nullptr)
    return Q8_ERR_NULL;
  if (!aligned(pooled_q, 16) || !aligned(pooled_k, 16) || !aligned(idx, 4) || !aligned(cnt, 4))
    return Q8_ERR_ALIGN;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_attn_select(pooled_q, pooled_k, Hq, Hkv, NB, D, k, kmax, idx, cnt,
                                as_stream(stream)) == hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

q8_status q8_attn_fwd(const void* q, const void* k, const void* v, int64_t L, int64_t ldq,
                      int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t D,
                      const int32_t* idx, const int32_t* cnt, int kmax, q8_dtype out_dtype,
                      void* out, int64_t ldo, void* stream) {
  if (out_dtype != Q8_F32 && out_dtype != Q8_BF16) return Q8_ERR_DTYPE;
  if (L < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !valid_attn_dim(D) || kmax < 1 ||
      ldq < Hq * D || ldk < Hkv * D || ldv < Hkv * D || ldo < Hq * D || ldq >= kMaxAttnLd ||
      ldk >= kMaxAttnLd || ldv >= kMaxAttnLd || ldo >= kMaxAttnLd)
    return Q8_ERR_SHAPE;
  if (L == 0) return Q8_OK;
  const int64_t NB = (L + 63) / 64;
  if (NB > kMaxAttnBlocks || Hq * NB >= kMaxDim) return Q8_ERR_SHAPE;
  if (q == nullptr || k == nullptr || v == nullptr || idx == nullptr || cnt == nullptr ||
      out == nullptr)
    return Q8_ERR_NULL;
  const int64_t oalign = out_dtype == Q8_F32 ? 16 : 8, osize = out_dtype == Q8_F32 ? 4 : 2;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || (ldq * 2) % 16 != 0 ||
      (ldk * 2) % 16 != 0 || (ldv * 2) % 16 != 0 || !aligned(idx, 4) || !aligned(cnt, 4) ||
      !aligned(out, static_cast<uintptr_t>(oalign)) || (ldo * osize) % oalign != 0)
    return Q8_ERR_ALIGN;
  const q8_status dev = check_device();
  if (dev != Q8_OK) return dev;
  return q8::launch_attn_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                             static_cast<const uint16_t*>(v), L, ldq, ldk, ldv, Hq, Hkv, D, idx, cnt,
                             kmax, static_cast<int>(out_dtype), out, ldo, as_stream(stream)) ==
                 hipSuccess
             ? Q8_OK
             : Q8_ERR_LAUNCH;
}

}  // extern "C"
