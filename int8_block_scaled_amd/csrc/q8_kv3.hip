// q8_kv3.hip -- 3-bit KV-cache codec: rows of D values (a key or value
// head vector) <-> 3-bit Lloyd-Max codes of their Walsh-Hadamard transform
// plus one binary32 scale.
//
// The source engine keeps its 256K-token KV cache in 3 bits with a
// Walsh-Hadamard transform and a Lloyd-Max quantiser, 17 GB -> 3.5 GB
// (news.hada.io topic 29953, "CUDA inference engine for running
// Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)", list of
// non-throttled paths, KV-cache item).  The pages give nothing more; the
// format implemented here is specified in include/q8.h (q8_kv3_encode).
//
// Cost model.  The codec moves 5.12 bytes of bfloat16 per byte of codes and
// does ~2 log2(D) binary32 operations per element; with no packed binary32
// arithmetic, a wave64 VALU instruction occupies a SIMD for four cycles, so
// at D = 256 the VALU time per row is of the same order as the HBM time.
// The kernels are therefore built to spend as few VALU instructions per
// element as possible and to move data with LDS instructions instead:
//   - P = D/32 lanes own a row, 32 elements per lane.  The butterfly stages
//     len = 1 .. 16 run on the lane's consecutive elements; the row is then
//     transposed through LDS so that lane p' holds the elements
//     32k + (32/P) p' + b (k < P, b < 32/P) and the stages len = 32 ..
//     D/2 also run inside the lane.  No stage needs a lane exchange.
//   - The sum of squares is pairwise over adjacent elements, so it reduces
//     inside the lane first; only P values per lane cross lanes.
//   - Codes come from a 1024-entry table in LDS (q8_kv3_table.h: key = top
//     ten bits of u, code = base + (thr <= u)), 4 VALU instructions each.
//   - Decoding looks each code up in an 8-entry table of the row's scaled
//     levels s * L_k in LDS, 2 VALU instructions each.
//   - Rows move between HBM and registers through a per-wave LDS tile, so
//     that global accesses are 16 bytes per lane over contiguous rows.
// Workgroups are persistent: a wave walks over row tiles with a grid
// stride, and the encoder issues the global loads of its next tile before
// it computes the current one.  Every stage runs in the order the format
// fixes, so the results are bit-identical to any implementation of it.
#include <float.h>

#include <atomic>

#include "q8_kernels.h"
#include "q8_kv3_table.h"

// Every product and sum below is its own binary32 operation: no fused
// multiply-add.
#pragma clang fp contract(off)

namespace q8 {
namespace {

constexpr int kE = 32;                    // elements per lane
constexpr int kEncWaves = 8;              // waves per workgroup (share one code table)
constexpr int kDecWaves = 4;
constexpr int kBufChunks = 576;           // per-wave LDS tile, 16-byte chunks (9216 bytes)

// Orders the LDS accesses of the lanes of one wave: those before it are
// performed, and seen by every lane, before those after it (LDS executes a
// wave's accesses in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
struct Layout {
  static constexpr int P = D / kE;                 // lanes per row
  static constexpr int kRows = 64 / P;             // rows per wave tile
  static constexpr int B = kE / P;                 // consecutive elements per block after transposing
  // binary32 row image for the transpose: each 32-element segment padded by
  // 4 floats, so the 16-byte accesses of 16 consecutive lanes hit distinct
  // banks (for P = 8)
  static constexpr int kSegFloats = kE + 4;
  static constexpr int kRowFloats = P * kSegFloats;
  static_assert(kRows * kRowFloats * 4 <= kBufChunks * 16, "tile");
};

// 16-byte-chunk tile of kRows rows, each P segments of S chunks plus one
// chunk of padding: the layout rows pass through between HBM and lanes.
template <int D, int S>
struct ChunkTile {
  static constexpr int P = D / kE;
  static constexpr int kRowChunks = P * (S + 1);
  static constexpr int C = P * S;                  // chunks of data per row
  static_assert((64 / P) * kRowChunks <= kBufChunks, "tile");
  static __device__ __forceinline__ int at(int r, int c) {
    return r * kRowChunks + (c / S) * (S + 1) + c % S;
  }
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));
constexpr int kNonTemporal = 2;           // buffer access cache policy: streamed once

// Raw buffer over [base, base + bytes): accesses past the end read zero and
// are not written -- how the rows past the last one of a tile are handled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Butterfly stages len = 1 .. 16 on a lane's 32 consecutive elements.
__device__ __forceinline__ void stages_low(float (&v)[kE]) {
#pragma unroll
  for (int len = 1; len < kE; len <<= 1)
#pragma unroll
    for (int j = 0; j < kE; ++j)
      if ((j & len) == 0) {
        const float a = v[j], b = v[j + len];
        v[j] = a + b;
        v[j + len] = a - b;
      }
}

// Butterfly stages len = 32 .. D/2 after the transpose: register k*B + b
// holds element 32k + B p' + b, so stage len = 32 * 2^t pairs k and k + 2^t.
template <int P>
__device__ __forceinline__ void stages_high(float (&v)[kE]) {
  constexpr int B = kE / P;
#pragma unroll
  for (int kl = 1; kl < P; kl <<= 1)
#pragma unroll
    for (int k = 0; k < P; ++k)
      if ((k & kl) == 0)
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const float a = v[k * B + b], c = v[(k + kl) * B + b];
          v[k * B + b] = a + c;
          v[(k + kl) * B + b] = a - c;
        }
}

// Lane exchange within a group of up to 8 lanes (DPP): lane l reads lane
// l ^ m; xor 4 is a half-row mirror (l ^ 7) then a quad permutation (l ^ 3).
template <int m>
__device__ __forceinline__ float lane_xor(float v) {
  const int b = __float_as_int(v);
  if constexpr (m == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true));
  if constexpr (m == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x4E, 0xF, 0xF, true));
  static_assert(m == 1 || m == 2 || m == 4, "lane exchange within 8 lanes");
  const int t = __builtin_amdgcn_update_dpp(0, b, 0x141, 0xF, 0xF, true);
  return __int_as_float(__builtin_amdgcn_update_dpp(0, t, 0x1B, 0xF, 0xF, true));
}

// Transpose a row's segments through the wave's binary32 row image: lane
// (r, p) holds elements 32p .. 32p+31 on entry and 32k + B p + b on exit.
template <int D>
__device__ __forceinline__ void transpose(float* img, int r, int p, float (&v)[kE]) {
  using Ly = Layout<D>;
  constexpr int B = Ly::B, P = Ly::P;
  float* row = img + r * Ly::kRowFloats;
#pragma unroll
  for (int m = 0; m < kE / 4; ++m)
    *reinterpret_cast<float4*>(row + p * Ly::kSegFloats + 4 * m) =
        make_float4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < P; ++k)
#pragma unroll
    for (int h = 0; h < B / 4; ++h) {
      const float4 t = *reinterpret_cast<const float4*>(row + k * Ly::kSegFloats + B * p + 4 * h);
      v[k * B + 4 * h + 0] = t.x;
      v[k * B + 4 * h + 1] = t.y;
      v[k * B + 4 * h + 2] = t.z;
      v[k * B + 4 * h + 3] = t.w;
    }
  wave_lds_sync();
}

// ---------------------------------------------------------------- encode

template <int D, bool kBf16>
__global__ __launch_bounds__(kEncWaves * 64, 4) void kv3_encode_kernel(
    const void* __restrict__ x, int64_t R, int64_t ldx, uint8_t* __restrict__ codes,
    float* __restrict__ scales, int64_t tiles) {
  using Ly = Layout<D>;
  constexpr int P = Ly::P, NR = Ly::kRows, B = Ly::B;
  constexpr int kEsize = kBf16 ? 2 : 4;
  constexpr int S = kE * kEsize / 16;              // input chunks per lane segment
  using T = ChunkTile<D, S>;
  constexpr int C = T::C;
  constexpr int kRowBytes = 3 * D / 8;             // codes per row

  // one block of LDS with the table first, at offset 0, so that a table
  // address is just the key times 8 (no base to add)
  __shared__ struct {
    uint2 table[1024];
    float4 buf[kEncWaves][kBufChunks];
  } smem;
  uint2* table = smem.table;
  float4 (*buf_all)[kBufChunks] = smem.buf;
  for (int k = threadIdx.x; k < 1024; k += kEncWaves * 64) {
    const kv3::Entry e = kv3::entry(static_cast<uint32_t>(k));
    table[k] = make_uint2(e.base, e.thr);
  }
  __syncthreads();

  // the wave index, as a wave-uniform (scalar) value: tile indices, row
  // bases and buffer descriptors derived from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint4* tile = reinterpret_cast<uint4*>(buf_all[wave]);
  float* img = reinterpret_cast<float*>(buf_all[wave]);
  uint8_t* ctile = reinterpret_cast<uint8_t*>(buf_all[wave]);
  const int r = lane / P, p = lane % P;
  const char* xb = static_cast<const char*>(x);
  const uint32_t pitch = static_cast<uint32_t>(ldx * kEsize);   // < 2^31 / 64 (host check)
  const int64_t step = static_cast<int64_t>(gridDim.x) * kEncWaves;
  // chunk g = i*64 + lane of a tile: row g / C, chunk g % C of the row; as
  // 64 % C == 0 the lane's row offset is the same for every i
  static_assert(64 % C == 0, "chunks per row");
  const uint32_t lane_off = (lane / C) * pitch + (lane % C) * 16;

  // global loads of tile t (rows past R read as zeros)
  uint4 st[S];
  auto load = [&](int64_t t) {
    const int64_t row0 = t * NR;
    const int64_t nrows = R - row0 < NR ? R - row0 : NR;
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(xb + row0 * pitch, static_cast<uint32_t>(nrows * pitch));
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const v4u w = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, i * (64 / C) * pitch, kNonTemporal);
      st[i] = make_uint4(w.x, w.y, w.z, w.w);
    }
  };

  // bfloat16 rows: the next tile's loads are issued before this tile's
  // work (16 registers); binary32 rows would need 32, so they are loaded at
  // the top of each tile instead
  constexpr bool kPrefetch = kBf16;
  int64_t t = static_cast<int64_t>(blockIdx.x) * kEncWaves + wave;
  if (kPrefetch && t < tiles) load(t);
  for (; t < tiles; t += step) {
    const int64_t row0 = t * NR;
    if (!kPrefetch) load(t);
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int g = i * 64 + lane;
      tile[T::at(g / C, g % C)] = st[i];
    }
    if (kPrefetch && t + step < tiles) load(t + step);   // in flight while this tile computes
    wave_lds_sync();

    // the lane's segment: elements 32p .. 32p+31 of row r
    float y[kE];
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const uint4 w = tile[r * T::kRowChunks + p * (S + 1) + k];
      if constexpr (kBf16) {
        y[8 * k + 0] = __uint_as_float(w.x << 16);
        y[8 * k + 1] = __uint_as_float(w.x & 0xffff0000u);
        y[8 * k + 2] = __uint_as_float(w.y << 16);
        y[8 * k + 3] = __uint_as_float(w.y & 0xffff0000u);
        y[8 * k + 4] = __uint_as_float(w.z << 16);
        y[8 * k + 5] = __uint_as_float(w.z & 0xffff0000u);
        y[8 * k + 6] = __uint_as_float(w.w << 16);
        y[8 * k + 7] = __uint_as_float(w.w & 0xffff0000u);
      } else {
        y[4 * k + 0] = __uint_as_float(w.x);
        y[4 * k + 1] = __uint_as_float(w.y);
        y[4 * k + 2] = __uint_as_float(w.z);
        y[4 * k + 3] = __uint_as_float(w.w);
      }
    }
    wave_lds_sync();

    stages_low(y);
    transpose<D>(img, r, p, y);
    stages_high<P>(y);

    // S: squares summed pairwise over adjacent elements.  Element bits:
    // b (in the lane), then p (across the group's lanes), then k (in the
    // lane); the lane exchanges run on one value per k.
    float q[P];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      float v[B];
#pragma unroll
      for (int b = 0; b < B; ++b) v[b] = y[k * B + b] * y[k * B + b];
#pragma unroll
      for (int len = 1; len < B; len <<= 1)
#pragma unroll
        for (int b = 0; b < B; b += 2 * len) v[b] = v[b] + v[b + len];
      q[k] = v[0];
    }
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if constexpr (P >= 2) q[k] = q[k] + lane_xor<1>(q[k]);
      if constexpr (P >= 4) q[k] = q[k] + lane_xor<2>(q[k]);
      if constexpr (P >= 8) q[k] = q[k] + lane_xor<4>(q[k]);
    }
#pragma unroll
    for (int len = 1; len < P; len <<= 1)
#pragma unroll
      for (int k = 0; k < P; k += 2 * len) q[k] = q[k] + q[k + len];
    const float sum = q[0];

    float s = sqrtf(sum / static_cast<float>(D));
    // a zero, binary32-subnormal or NaN scale: s = 0 and every code 4.
    // With inv = 0, u = y * 0 = +-0 (code 4) for finite y.  A NaN sum (y
    // holds a NaN, or infinities of both signs) can leave u NaN, so its
    // rows read table entry 0 ({4, NaN}: code 4 whatever u is) -- the
    // key's byte mask below is 0 for them.
    const bool flat = !(s >= FLT_MIN);
    const float inv = flat ? 0.0f : 1.0f / s;
    if (flat) s = 0.0f;
    const uint32_t key_mask = (sum != sum) ? 0u : 0x1ff8u;
    const char* tab = reinterpret_cast<const char*>(table);

    // codes, and their bits: block k of the lane (B consecutive elements
    // starting at element 32k + B p) is 3B bits at bit 96k + 3Bp of the row
    uint32_t g[P][(3 * B + 31) / 32];
#pragma unroll
    for (int k = 0; k < P; ++k) {
#pragma unroll
      for (int i = 0; i < (3 * B + 31) / 32; ++i) g[k][i] = 0;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float u = y[k * B + b] * inv;
        const uint32_t ub = __float_as_uint(u);   // entry (ub >> 22), 8 bytes each
        const uint2 e = *reinterpret_cast<const uint2*>(tab + ((ub >> 19) & key_mask));
        const uint32_t c = e.x + (__uint_as_float(e.y) <= u ? 1u : 0u);
        const int pos = 3 * b;
        g[k][pos >> 5] |= c << (pos & 31);
        if ((pos & 31) > 29) g[k][(pos >> 5) + 1] |= c >> (32 - (pos & 31));
      }
      // at most 16 table reads in flight (registers)
      if ((k * B) % 16 == 16 - B) asm volatile("" ::: "memory");
    }
    // the tile's codes, row after row as stored: 12 bytes per 32 elements
    uint8_t* crow = ctile + r * kRowBytes;
    if constexpr (P == 8) {
      // 12 bits per block: lanes 2i and 2i+1 form 3 bytes at 12k + 3i
#pragma unroll
      for (int k = 0; k < P; ++k) {
        const uint32_t mate = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(g[k][0]), 0xB1, 0xF, 0xF, true));
        if ((p & 1) == 0) {
          const uint32_t w24 = g[k][0] | (mate << 12);
          uint8_t* o = crow + 12 * k + 3 * (p >> 1);
          o[0] = static_cast<uint8_t>(w24);
          o[1] = static_cast<uint8_t>(w24 >> 8);
          o[2] = static_cast<uint8_t>(w24 >> 16);
        }
      }
    } else if constexpr (P == 4) {
#pragma unroll
      for (int k = 0; k < P; ++k) {                 // 24 bits at 12k + 3p
        uint8_t* o = crow + 12 * k + 3 * p;
        o[0] = static_cast<uint8_t>(g[k][0]);
        o[1] = static_cast<uint8_t>(g[k][0] >> 8);
        o[2] = static_cast<uint8_t>(g[k][0] >> 16);
      }
    } else {
#pragma unroll
      for (int k = 0; k < P; ++k) {                 // 48 bits at 12k + 6p (2-byte aligned)
        uint16_t* o = reinterpret_cast<uint16_t*>(crow + 12 * k + 6 * p);
        o[0] = static_cast<uint16_t>(g[k][0]);
        o[1] = static_cast<uint16_t>(g[k][0] >> 16);
        o[2] = static_cast<uint16_t>(g[k][1]);
      }
    }
    wave_lds_sync();
    // the tile's NR * 3D/8 = 768 bytes of codes, contiguous in HBM
    const int64_t nbytes = (R - row0 < NR ? R - row0 : NR) * kRowBytes;
    const uint32_t* csrc = reinterpret_cast<const uint32_t*>(ctile);
    uint32_t* cdst = reinterpret_cast<uint32_t*>(codes + row0 * kRowBytes);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int d = i * 64 + lane;
      if (4 * d < nbytes) cdst[d] = csrc[d];
    }
    if (p == 0 && row0 + r < R) scales[row0 + r] = s;
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------- decode

template <int D, bool kBf16>
__global__ __launch_bounds__(kDecWaves * 64) void kv3_decode_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales, int64_t R,
    void* __restrict__ out, int64_t ldo, int64_t tiles) {
  using Ly = Layout<D>;
  constexpr int P = Ly::P, NR = Ly::kRows, B = Ly::B;
  constexpr int kEsize = kBf16 ? 2 : 4;
  constexpr int S = kE * kEsize / 16;              // output chunks per segment
  using T = ChunkTile<D, S>;
  constexpr int C = T::C;
  constexpr int kRowBytes = 3 * D / 8;

  __shared__ float4 buf_all[kDecWaves][kBufChunks];
  __shared__ float lvl_all[kDecWaves][NR * 8];
  // the wave index, as a wave-uniform (scalar) value: tile indices, row
  // bases and buffer descriptors derived from it stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  float* img = reinterpret_cast<float*>(buf_all[wave]);
  uint4* tile = reinterpret_cast<uint4*>(buf_all[wave]);
  float* lvl = lvl_all[wave];
  const int r = lane / P, p = lane % P;
  char* ob = static_cast<char*>(out);
  const uint32_t pitch = static_cast<uint32_t>(ldo * kEsize);   // < 2^31 / 64 (host check)
  const int64_t step = static_cast<int64_t>(gridDim.x) * kDecWaves;
  static_assert(64 % C == 0, "chunks per row");
  const uint32_t lane_off = (lane / C) * pitch + (lane % C) * 16;

  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kDecWaves + wave; t < tiles; t += step) {
    const int64_t row0 = t * NR;
    const uint32_t nrows = static_cast<uint32_t>(R - row0 < NR ? R - row0 : NR);
    // rows past R: codes and scale read as zero, nothing is stored
    const v3u w3 = __builtin_amdgcn_raw_buffer_load_b96(
        rows_rsrc(codes + row0 * kRowBytes, nrows * kRowBytes), r * kRowBytes + 12 * p, 0,
        kNonTemporal);
    const uint32_t w[3] = {w3.x, w3.y, w3.z};
    const float s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rows_rsrc(scales + row0, nrows * 4), r * 4, 0, 0));
    // the row's scaled levels s * L_k, 8 / P of them from each of its lanes
#pragma unroll
    for (int i = 0; i < 8 / P; ++i) lvl[r * 8 + (8 / P) * p + i] = s * kv3::kLevels[(8 / P) * p + i];
    wave_lds_sync();
    float z[kE];
    const float* lrow = lvl + r * 8;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      const int pos = 3 * j;
      uint32_t c = w[pos >> 5] >> (pos & 31);
      if ((pos & 31) > 29) c |= w[(pos >> 5) + 1] << (32 - (pos & 31));
      z[j] = lrow[c & 7u];
    }
    wave_lds_sync();

    stages_low(z);
    transpose<D>(img, r, p, z);
    stages_high<P>(z);

    // the lane's blocks -> the output tile: block k (elements 32k + Bp ..
    // 32k + Bp + B-1) is B*esize bytes at byte B*p*esize of segment k
    constexpr float kInvD = 1.0f / static_cast<float>(D);
    char* trow = reinterpret_cast<char*>(tile) + r * T::kRowChunks * 16;
#pragma unroll
    for (int k = 0; k < P; ++k) {
      char* seg = trow + k * (S + 1) * 16 + B * p * kEsize;
      if constexpr (kBf16) {
        uint32_t h[B / 2];
#pragma unroll
        for (int i = 0; i < B / 2; ++i) {           // pairs, rounded to nearest even
          typedef float f2 __attribute__((ext_vector_type(2)));
          typedef __bf16 b2 __attribute__((ext_vector_type(2)));
          const b2 hb = __builtin_convertvector(
              (f2{z[k * B + 2 * i] * kInvD, z[k * B + 2 * i + 1] * kInvD}), b2);
          h[i] = __builtin_bit_cast(uint32_t, hb);
        }
#pragma unroll
        for (int i = 0; i < B / 2; i += 2)
          *reinterpret_cast<uint2*>(seg + 4 * i) = make_uint2(h[i], h[i + 1]);
      } else {
#pragma unroll
        for (int i = 0; i < B; i += 4)
          *reinterpret_cast<float4*>(seg + 4 * i) =
              make_float4(z[k * B + i] * kInvD, z[k * B + i + 1] * kInvD,
                          z[k * B + i + 2] * kInvD, z[k * B + i + 3] * kInvD);
      }
    }
    wave_lds_sync();
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(ob + row0 * pitch, nrows * pitch);
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int g = i * 64 + lane;
      const uint4 o = tile[T::at(g / C, g % C)];
      __builtin_amdgcn_raw_buffer_store_b128(v4u{o.x, o.y, o.z, o.w}, rs, lane_off,
                                             i * (64 / C) * pitch, kNonTemporal);
    }
    wave_lds_sync();
  }
}

// resident workgroups per CU the launches are sized for
constexpr int kEncBlocksPerCU = 2;
constexpr int kDecBlocksPerCU = 4;

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

uint32_t grid_for(int64_t tiles, int waves, int per_cu) {
  const int64_t need = (tiles + waves - 1) / waves;
  const int64_t cap = static_cast<int64_t>(cu_count()) * per_cu;
  return static_cast<uint32_t>(need < cap ? need : cap);
}

template <int D>
hipError_t launch_enc(const void* x, int dtype, int64_t R, int64_t ldx, uint8_t* codes,
                      float* scales, hipStream_t stream) {
  const int64_t tiles = (R + Layout<D>::kRows - 1) / Layout<D>::kRows;
  const uint32_t grid = grid_for(tiles, kEncWaves, kEncBlocksPerCU);
  if (dtype == 1)
    hipLaunchKernelGGL((kv3_encode_kernel<D, true>), dim3(grid), dim3(kEncWaves * 64), 0, stream,
                       x, R, ldx, codes, scales, tiles);
  else
    hipLaunchKernelGGL((kv3_encode_kernel<D, false>), dim3(grid), dim3(kEncWaves * 64), 0, stream,
                       x, R, ldx, codes, scales, tiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dec(const uint8_t* codes, const float* scales, int64_t R, int dtype, void* out,
                      int64_t ldo, hipStream_t stream) {
  const int64_t tiles = (R + Layout<D>::kRows - 1) / Layout<D>::kRows;
  const uint32_t grid = grid_for(tiles, kDecWaves, kDecBlocksPerCU);
  if (dtype == 1)
    hipLaunchKernelGGL((kv3_decode_kernel<D, true>), dim3(grid), dim3(kDecWaves * 64), 0, stream,
                       codes, scales, R, out, ldo, tiles);
  else
    hipLaunchKernelGGL((kv3_decode_kernel<D, false>), dim3(grid), dim3(kDecWaves * 64), 0, stream,
                       codes, scales, R, out, ldo, tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv3_encode(const void* x, int dtype, int64_t R, int64_t D, int64_t ldx,
                             uint8_t* codes, float* scales, hipStream_t stream) {
  switch (D) {
    case 64: return launch_enc<64>(x, dtype, R, ldx, codes, scales, stream);
    case 128: return launch_enc<128>(x, dtype, R, ldx, codes, scales, stream);
    case 256: return launch_enc<256>(x, dtype, R, ldx, codes, scales, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv3_decode(const uint8_t* codes, const float* scales, int64_t R, int64_t D,
                             int dtype, void* out, int64_t ldo, hipStream_t stream) {
  switch (D) {
    case 64: return launch_dec<64>(codes, scales, R, dtype, out, ldo, stream);
    case 128: return launch_dec<128>(codes, scales, R, dtype, out, ldo, stream);
    case 256: return launch_dec<256>(codes, scales, R, dtype, out, ldo, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q8
