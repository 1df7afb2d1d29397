// q8_attn.hip -- block-sparse causal attention for long-context prefill.
//
// The source engine runs attention on its own FlashAttention kernel with
// MInference-style block sparsity (news.hada.io topic 29953, "CUDA
// inference engine for running Qwen3.5/3.6 hybrid models on mining cards
// (CMP 100-210)", list of non-throttled paths, attention item).  The pages
// give no more; the operation is specified in include/q8.h (q8_attn_pool,
// q8_attn_select, q8_attn_fwd): 64-token blocks, each query block attending
// to block 0, its own (diagonal, causally masked) block and the top-scoring
// earlier blocks by the dot product of block-mean-pooled Q and K; one list
// per K/V head, shared by its group of query heads.
//
// The forward kernel is a FlashAttention forward pass over the listed key
// blocks, on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16):
//   - a workgroup owns one query block (64 queries) of up to four query
//     heads of one K/V head's group, two waves of 32 queries per head; the
//     heads share the group's list, so each K/V block passes through LDS once
//     for all of them;
//   - scores are formed transposed, S^T = K Q^T, so that a lane owns one
//     query (lane % 32) and 16 keys per 32-key tile: the running maximum and
//     sum of the online softmax are per lane (two lanes per query), and the
//     exponentials in bf16 are already the B operand of the next product;
//   - the output is formed transposed too, O^T = V^T P^T; the MFMA's 16-wide
//     reduction index runs over keys in the order the score tiles hold them,
//     and the V^T operand comes from row-major V in LDS through transposing
//     reads (ds_read_b64_tr_b16), so K and V are staged alike;
//   - K and V rows, including those past the sequence end, come through
//     range-checked buffer loads (zeros past L) into two LDS buffers (one
//     block attended while the next is stored), with rows padded so that
//     both operand reads are nearly free of bank conflicts.
// The softmax runs in base 2: scores are scaled by log2(e)/sqrt(D) and
// exponentiated with exp2 (v_exp_f32; a result below 2^-126 of the row's
// maximum term flushes to zero, which no output can resolve).  The running
// maximum is raised lazily (by steps of more than 2^8), so the output is
// rescaled only when a block brings a clearly larger score.
#include <float.h>

#include "q8_kernels.h"

namespace q8 {
namespace {

constexpr int kBlk = 64;                       // tokens per block
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------------------------- pool

// pooled[h][b][d] = mean of x[t][h*D + d] over the block's tokens (binary32,
// summed in token order).  A workgroup takes 256 16-byte column chunks of
// one block (8 columns each, all heads side by side), so a wave's loads read
// 1 KB of a token row.
__global__ __launch_bounds__(256) void attn_pool_kernel(const uint16_t* __restrict__ x, int64_t L,
                                                        int64_t ldx, int64_t H, int64_t D,
                                                        int64_t NB, float* __restrict__ pooled) {
  const int64_t chunks = H * D / 8;              // 16-byte chunks per token row
  const int64_t groups = (chunks + 255) / 256;
  const int64_t b = blockIdx.x / groups;
  const int64_t cc = (blockIdx.x % groups) * 256 + threadIdx.x;
  if (cc >= chunks) return;
  const int64_t t0 = b * kBlk, t1 = t0 + kBlk < L ? t0 + kBlk : L;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* src = x + 8 * cc;
#pragma unroll 8
  for (int64_t t = t0; t < t1; ++t) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + t * ldx);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] += bf16_to_f32(ww[q] & 0xffffu);
      acc[2 * q + 1] += bf16_to_f32(ww[q] >> 16);
    }
  }
  const float n = static_cast<float>(t1 - t0);
  const int64_t h = cc / (D / 8), c8 = cc % (D / 8);
  float* out = pooled + (h * NB + b) * D + 8 * c8;
#pragma unroll
  for (int q = 0; q < 8; ++q) out[q] = acc[q] / n;
}

// ----------------------------------------------------------------- select

constexpr int kSelThreads = 256;
constexpr int kMaxBlocks = 4096;               // 256K tokens

// Order-preserving map of a binary32 score to 32 bits (larger score, larger
// key); -0 is first made +0, so equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (K/V head g, query block i): scores of blocks 0 < j < i,
// the sum of the group's pooled query rows against the pooled key rows; the
// (k-2)'th largest score is found by a radix select over the score keys
// (four 8-bit digits, a histogram each), then every block scoring above it
// is taken, and of those scoring equal to it the lowest blocks, as many as
// complete k - 2 -- the first k - 2 of the order (score descending, block
// ascending).  Block 0 and block i are added, and the list is written in
// ascending order.
template <int D>
__global__ __launch_bounds__(kSelThreads) void attn_select_kernel(
    const float* __restrict__ pq, const float* __restrict__ pk, int64_t Hq, int64_t Hkv,
    int64_t NB, int k, int kmax, int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  static_assert(kSelThreads == 256, "one histogram bin per thread");
  __shared__ uint32_t key[kMaxBlocks];
  __shared__ uint8_t take[kMaxBlocks];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[2];
  __shared__ __attribute__((aligned(16))) float qrow[D];
  const int64_t g = blockIdx.x / NB, i = blockIdx.x % NB;
  const int64_t G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  int32_t* out = idx + (g * NB + i) * kmax;
  for (int m = tid; m < kmax; m += kSelThreads) out[m] = -1;
  for (int64_t j = tid; j <= i; j += kSelThreads) take[j] = (k >= i + 1 || j == 0 || j == i) ? 1 : 0;
  if (tid == 0) cnt[g * NB + i] = static_cast<int32_t>(k >= i + 1 ? i + 1 : k);
  if (k < i + 1 && k > 2) {
    for (int d = tid; d < D; d += kSelThreads) {   // the group's query row
      float a = 0.0f;
      for (int64_t hh = 0; hh < G; ++hh) a += pq[((g * G + hh) * NB + i) * D + d];
      qrow[d] = a;
    }
    __syncthreads();
    // candidates e = j - 1 for j = 1 .. i-1: eight lanes per candidate row,
    // each reading 16-byte pieces 16 (p + 8 k) of it, so that a wave's load
    // covers eight whole 128-byte lines; the eight partial sums are added
    // across the lanes
    const int ncand = static_cast<int>(i - 1);
    {
      const int rs = lane >> 3, pp = lane & 7;
      const int w = tid >> 6;
      for (int e0 = 8 * w; e0 < ncand; e0 += 8 * (kSelThreads / 64)) {
        const int e = e0 + rs;
        const float4* kr = reinterpret_cast<const float4*>(pk + (g * NB + (e < ncand ? e + 1 : 1)) * D);
        float a = 0.0f;
#pragma unroll
        for (int k4 = 0; k4 < D / 32; ++k4) {
          const int d4 = pp + 8 * k4;
          const float4 kv = kr[d4];
          const float4 qv = *reinterpret_cast<const float4*>(&qrow[4 * d4]);
          a += qv.x * kv.x;
          a += qv.y * kv.y;
          a += qv.z * kv.z;
          a += qv.w * kv.w;
        }
        a += __shfl_xor(a, 4);
        a += __shfl_xor(a, 2);
        a += __shfl_xor(a, 1);
        if (pp == 0 && e < ncand) key[e] = score_key(a);
      }
    }
    __syncthreads();
    // radix select of the want'th largest key, most significant digit first
    uint32_t prefix = 0, pmask = 0;
    int want = k - 2;                            // 1 <= want < ncand
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int e = tid; e < ncand; e += kSelThreads) {
        const uint32_t u = key[e];
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds bins 4l .. 4l+3; counts above them from a suffix scan
        const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
        const uint32_t t = c0 + c1 + c2 + c3;
        uint32_t x = t;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_down(x, off);
          if (lane + off < 64) x += y;
        }
        uint32_t cum = x - t;                    // keys in bins above 4l+3
        const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (cum < static_cast<uint32_t>(want) && cum + cs[q] >= static_cast<uint32_t>(want)) {
            sel[0] = static_cast<uint32_t>(4 * lane + q);
            sel[1] = static_cast<uint32_t>(want) - cum;
          }
          cum += cs[q];
        }
      }
      __syncthreads();
      prefix |= sel[0] << shift;
      pmask |= 255u << shift;
      want = static_cast<int>(sel[1]);
    }
    // prefix is now the threshold key; want of the keys equal to it are taken
    for (int e = tid; e < ncand; e += kSelThreads)
      if (key[e] > prefix) take[e + 1] = 1;
    if (tid < 64) {                              // the lowest blocks among the equal keys
      int base = 0;
      for (int e0 = 0; e0 < ncand && base < want; e0 += 64) {
        const int e = e0 + lane;
        const bool f = e < ncand && key[e] == prefix;
        const uint64_t mask = __ballot(f);
        const int rank = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0)));
        if (f && rank < want) take[e + 1] = 1;
        base += __popcll(mask);
      }
    }
  }
  __syncthreads();
  // compact ascending with the first wave
  if (tid < 64) {
    int base = 0;
    for (int64_t j0 = 0; j0 <= i; j0 += 64) {
      const int64_t j = j0 + tid;
      const bool f = j <= i && take[j];
      const uint64_t mask = __ballot(f);
      const int pos = base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
      if (f) out[pos] = static_cast<int32_t>(j);
      base += __popcll(mask);
    }
  }
}

// ---------------------------------------------------------------- forward

typedef float f16v __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// LDS rows of a K or V block (D <= 128), padded so that the operand reads
// spread over the banks: K rows of 272 bytes for the 16-byte reads of 32 rows
// x 2 chunks, V rows of 288 bytes for the transposing 8-byte reads of 8 rows
// x 64 bytes.  Every read is a per-lane base plus a constant offset.
constexpr int kKPitch = 272, kVPitch = 288;
constexpr int kKTile = kBlk * kKPitch, kVTile = kBlk * kVPitch;
constexpr int kBlockBytes = kKTile + kVTile;   // one resident block: 35 KB

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), bf2));
}

// A workgroup owns query block i of GH query heads of K/V head g's group,
// two waves of 32 queries per head; all read the same listed K/V blocks.
template <int D, int GH, bool kBf16Out>
__global__ __launch_bounds__(128 * GH, GH == 4 ? 2 : 1) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t L, int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t NB,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int kmax,
    void* __restrict__ out, int64_t ldo, float scale_log2) {
  constexpr int kThreads = 128 * GH;
  constexpr int KS = D / 16;                     // 16-wide d steps of a score product
  constexpr int DT = D / 32;                     // 32-row d tiles of the output
  constexpr int kRowChunks = D / 8;              // 16-byte chunks per K or V row
  constexpr int kPer = kBlk * kRowChunks / kThreads;   // chunks per thread and block
  static_assert(kBlk * kRowChunks % kThreads == 0, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBlockBytes];   // 2 x (K, V)

  // Tiles (K/V head g, query block i, head part), later blocks first within
  // a head.  Workgroups are dealt to the 8 XCDs in turn; the order below
  // gives each XCD a contiguous run of tiles, so that the query blocks of
  // one K/V head, whose lists overlap, share that XCD's L2.
  const int64_t G = Hq / Hkv, parts = G / GH, per_head = NB * parts, tiles = Hkv * per_head;
  const int64_t wg = blockIdx.x;
  const int64_t T = tiles % 8 == 0 ? (wg % 8) * (tiles / 8) + wg / 8 : wg;
  const int64_t g = T / per_head, rem = T % per_head;
  const int64_t i = NB - 1 - rem / parts, part = rem % parts;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 31, hb = lane >> 5;
  const int64_t h = g * G + part * GH + wave / 2;
  const int qh = wave & 1;
  const int64_t q0 = i * kBlk + 32 * qh;         // the wave's first query

  // Q^T operand: lane holds Q[q0 + c][16 ks + 8 hb .. +8] for every step ks
  bf8 qb[KS];
  {
    const int64_t rows = L - q0 <= 0 ? 0 : (L - q0 < 32 ? L - q0 : 32);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(Q + q0 * ldq + h * D, static_cast<uint32_t>(rows * ldq * 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qb[ks] = __builtin_bit_cast(bf8, __builtin_amdgcn_raw_buffer_load_b128(
                                           rq, static_cast<uint32_t>((c * ldq + 16 * ks + 8 * hb) * 2), 0, 0));
  }

  f16v o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f16v{};
  float m = -INFINITY, lsum = 0.0f;

  // the list is device data: clamp its length and skip entries outside the
  // blocks a query block may see, so that no entry can move a load off its
  // buffer
  const int n_raw = cnt[g * NB + i];
  const int n = n_raw < 0 ? 0 : (n_raw > kmax ? kmax : n_raw);
  const int32_t* list = idx + (g * NB + i) * kmax;   // the K/V head's list
  auto next_valid = [&](int b) {                 // uniform
    for (; b < n; ++b) {
      const int32_t j = list[b];
      if (j >= 0 && j <= i) break;
    }
    return b;
  };

  // K and V blocks: 16-byte chunks through registers into LDS, row-major
  // (rows past L read as zeros).
  v4u kreg[kPer], vreg[kPer];
  auto load_block = [&](int64_t j) {
    const int64_t rows = L - j * kBlk < kBlk ? L - j * kBlk : kBlk;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(K + j * kBlk * ldk + g * D, static_cast<uint32_t>(rows * ldk * 2));
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(V + j * kBlk * ldv + g * D, static_cast<uint32_t>(rows * ldv * 2));
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = u * kThreads + tid, r = e / kRowChunks, ch = e % kRowChunks;
      kreg[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<uint32_t>((r * ldk + 8 * ch) * 2), 0, 0);
      vreg[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, static_cast<uint32_t>((r * ldv + 8 * ch) * 2), 0, 0);
    }
  };
  auto store_block = [&](int buf) {
    uint8_t* kt = lds + buf * kBlockBytes;
    uint8_t* vt = kt + kKTile;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = u * kThreads + tid, r = e / kRowChunks, ch = e % kRowChunks;
      *reinterpret_cast<v4u*>(kt + r * kKPitch + 16 * ch) = kreg[u];
      *reinterpret_cast<v4u*>(vt + r * kVPitch + 16 * ch) = vreg[u];
    }
  };

  // this lane's source row and column for the transposed V reads: lane
  // group gl = lane / 16 reads keys 4 (gl / 2) + (lane % 16) / 4 (+8) of a
  // 16-key step, columns 16 (gl % 2) + 4 (lane % 4) of a 32-column tile
  const int gl = lane >> 4, vrow = 4 * (gl >> 1) + ((lane & 15) >> 2), vcol = 16 * (gl & 1) + 4 * (lane & 3);

  const uint32_t k_off = static_cast<uint32_t>(c * kKPitch + 16 * hb);
  const uint32_t v_off = static_cast<uint32_t>(kKTile + vrow * kVPitch + 2 * vcol);
  auto attend = [&](int buf, int64_t j) {
    const uint8_t* kt = lds + buf * kBlockBytes + k_off;
    const uint8_t* vt = lds + buf * kBlockBytes + v_off;
    // scores: s[t][4 jj + r] = S[key 32 t + 8 jj + 4 hb + r][query c]
    f16v s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f16v acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf8 a = *reinterpret_cast<const bf8*>(kt + 32 * t * kKPitch + 32 * ks);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], acc, 0, 0, 0);
      }
      s[t] = acc;
    }
    // causal mask, in the diagonal block only (uniform branch)
    if (j == i) {
      const int qi = 32 * qh + c;                // query's row in the block
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * t + 8 * (v >> 2) + 4 * hb + (v & 3) > qi) s[t][v] = -INFINITY;
    }
    // row maximum over the block's keys (lanes c and c + 32 share a query)
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; v += 2) mx = fmaxf(fmaxf(mx, s[t][v]), s[t][v + 1]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    mx *= scale_log2;
    // Lazy rescaling: the reference maximum m only moves when a block's
    // maximum exceeds it by more than 8, so exponentials stay <= 2^8 (exact
    // ratios; bfloat16 holds them) and the output is rarely rescaled.
    const bool raise = mx > m + 8.0f;
    if (__any(raise)) {
      const float m_new = raise ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m = m_new;
    }
    // p = 2^(s * log2(e)/sqrt(D) - m); this lane's part of the row sum
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][v], scale_log2, -m));
        s[t][v] = p;
        lsum += p;
      }
    // O^T += V^T P^T in 16-key steps (t, p2): slots 8 hb .. 8 hb + 3 are keys
    // 32 t + 16 p2 + 4 hb + r, slots 8 hb + 4 .. + 7 the same + 8, which is
    // where the score tile holds them (s[t][8 p2 .. 8 p2 + 7])
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        const v4u pw = {pack_bf16(s[t][8 * p2], s[t][8 * p2 + 1]), pack_bf16(s[t][8 * p2 + 2], s[t][8 * p2 + 3]),
                        pack_bf16(s[t][8 * p2 + 4], s[t][8 * p2 + 5]), pack_bf16(s[t][8 * p2 + 6], s[t][8 * p2 + 7])};
        const bf8 pb = __builtin_bit_cast(bf8, pw);
        const int r0 = 32 * t + 16 * p2;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + r0 * kVPitch + 64 * dt));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vt + (r0 + 8) * kVPitch + 64 * dt));
          const v4u aw = {__builtin_bit_cast(v2u, lo)[0], __builtin_bit_cast(v2u, lo)[1],
                          __builtin_bit_cast(v2u, hi)[0], __builtin_bit_cast(v2u, hi)[1]};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8, aw), pb, o[dt], 0, 0, 0);
        }
      }
  };

  // Two LDS buffers: while block b is attended from one, block b+1 (loaded
  // into registers during block b-1) is stored into the other and block b+2
  // is loaded; one barrier per block.
  int cur = next_valid(0);
  int nxt = cur < n ? next_valid(cur + 1) : n;
  if (cur < n) {
    load_block(list[cur]);
    store_block(0);
  }
  if (nxt < n) load_block(list[nxt]);
  __syncthreads();
  int buf = 0;
  while (cur < n) {
    attend(buf, list[cur]);
    int nn = n;
    if (nxt < n) {
      store_block(buf ^ 1);
      nn = next_valid(nxt + 1);
      if (nn < n) load_block(list[nn]);
    }
    __syncthreads();
    cur = nxt;
    nxt = nn;
    buf ^= 1;
  }

  // lanes c and c + 32 hold parts of the query's row sum
  lsum += __shfl_xor(lsum, 32);
  // O[q][h*D + 32 dt + 8 jj + 4 hb + r] = o[dt][4 jj + r] / lsum
  const int64_t q = q0 + c;
  if (q < L) {
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int64_t col = h * D + 32 * dt + 8 * jj + 4 * hb;
        const float a0 = o[dt][4 * jj] * inv, a1 = o[dt][4 * jj + 1] * inv;
        const float a2 = o[dt][4 * jj + 2] * inv, a3 = o[dt][4 * jj + 3] * inv;
        if constexpr (kBf16Out)
          *reinterpret_cast<v2u*>(static_cast<uint16_t*>(out) + q * ldo + col) = v2u{pack_bf16(a0, a1), pack_bf16(a2, a3)};
        else
          *reinterpret_cast<f4*>(static_cast<float*>(out) + q * ldo + col) = f4{a0, a1, a2, a3};
      }
  }
}

}  // namespace

hipError_t launch_attn_pool(const uint16_t* x, int64_t L, int64_t ldx, int64_t H, int64_t D,
                            float* pooled, hipStream_t stream) {
  const int64_t NB = (L + kBlk - 1) / kBlk;
  const int64_t groups = (H * D / 8 + 255) / 256;
  const uint32_t grid = static_cast<uint32_t>(NB * groups);
  hipLaunchKernelGGL(attn_pool_kernel, dim3(grid), dim3(256), 0, stream, x, L, ldx, H, D, NB, pooled);
  return hipGetLastError();
}

hipError_t launch_attn_select(const float* pq, const float* pk, int64_t Hq, int64_t Hkv, int64_t NB,
                              int64_t D, int k, int kmax, int32_t* idx, int32_t* cnt,
                              hipStream_t stream) {
  const uint32_t grid = static_cast<uint32_t>(Hkv * NB);
  if (D == 128)
    hipLaunchKernelGGL((attn_select_kernel<128>), dim3(grid), dim3(kSelThreads), 0, stream, pq, pk,
                       Hq, Hkv, NB, k, kmax, idx, cnt);
  else
    hipLaunchKernelGGL((attn_select_kernel<64>), dim3(grid), dim3(kSelThreads), 0, stream, pq, pk,
                       Hq, Hkv, NB, k, kmax, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t L,
                           int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t D,
                           const int32_t* idx, const int32_t* cnt, int kmax, int out_dtype,
                           void* out, int64_t ldo, hipStream_t stream) {
  const int64_t NB = (L + kBlk - 1) / kBlk;
  const int64_t G = Hq / Hkv;
  const int gh = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);   // query heads per workgroup
  const uint32_t grid = static_cast<uint32_t>(Hq / gh * NB);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
#define Q8_ATTN_LAUNCH(DD, GG, BF)                                                                \
  hipLaunchKernelGGL((attn_fwd_kernel<DD, GG, BF>), dim3(grid), dim3(128 * GG), 0, stream, q, k, v, \
                     L, ldq, ldk, ldv, Hq, Hkv, NB, idx, cnt, kmax, out, ldo, scale_log2)
#define Q8_ATTN_GH(DD, BF)                \
  do {                                    \
    if (gh == 4) Q8_ATTN_LAUNCH(DD, 4, BF); \
    else if (gh == 2) Q8_ATTN_LAUNCH(DD, 2, BF); \
    else Q8_ATTN_LAUNCH(DD, 1, BF);       \
  } while (0)
  if (D == 128) {
    if (out_dtype == 1) Q8_ATTN_GH(128, true);
    else Q8_ATTN_GH(128, false);
  } else {
    if (out_dtype == 1) Q8_ATTN_GH(64, true);
    else Q8_ATTN_GH(64, false);
  }
#undef Q8_ATTN_GH
#undef Q8_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace q8
