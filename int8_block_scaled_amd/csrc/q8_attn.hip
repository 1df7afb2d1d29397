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
// blocks, on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
//   - a workgroup owns one query block (64 queries) of one head, a wave 16
//     queries; the key and value blocks pass through LDS, shared by the four
//     waves;
//   - scores are formed transposed, S^T = K Q^T, so that a lane owns one
//     query (lane % 16) and four keys per 16-key tile: the running maximum
//     and sum of the online softmax are per lane, and the exponentials in
//     bf16 are already the B operand of the next product;
//   - the output is formed transposed too, O^T = V^T P^T; the MFMA's 32-wide
//     reduction index runs over keys in the order the score tiles hold them
//     (lane group g supplies keys 4g..4g+3 of two consecutive 16-key tiles),
//     and the V^T operand is read from LDS in the same order;
//   - V is written to LDS transposed ([d][key]); rows, including those past
//     the sequence end, come through range-checked buffer loads (zeros past
//     L); LDS rows are padded so that the 16 lanes of each operand read hit
//     distinct banks.
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
// summed in token order).  16 threads per (h, b), 8 columns each (D = 128;
// 8 threads for D = 64).
template <int D>
__global__ __launch_bounds__(256) void attn_pool_kernel(const uint16_t* __restrict__ x, int64_t L,
                                                        int64_t ldx, int64_t H, int64_t NB,
                                                        float* __restrict__ pooled) {
  constexpr int kThr = D / 8;
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * (256 / kThr) + threadIdx.x / kThr;
  if (pair >= H * NB) return;
  const int c = threadIdx.x % kThr;
  const int64_t h = pair / NB, b = pair % NB;
  const int64_t t0 = b * kBlk, t1 = t0 + kBlk < L ? t0 + kBlk : L;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t t = t0; t < t1; ++t) {
    const uint4 w = *reinterpret_cast<const uint4*>(x + t * ldx + h * D + 8 * c);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(ww[i] & 0xffffu);
      acc[2 * i + 1] += bf16_to_f32(ww[i] >> 16);
    }
  }
  const float n = static_cast<float>(t1 - t0);
  float* out = pooled + pair * D + 8 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = acc[i] / n;
}

// ----------------------------------------------------------------- select

constexpr int kSelThreads = 256;
constexpr int kMaxBlocks = 4096;               // 256K tokens

// One workgroup per (K/V head g, query block i): scores of blocks 0 < j < i,
// the sum of the group's pooled query rows against the pooled key rows, a
// bitonic sort by (score descending, block ascending), then block 0, block
// i and the first (k - 2) of the sort, written in ascending order.
template <int D>
__global__ __launch_bounds__(kSelThreads) void attn_select_kernel(
    const float* __restrict__ pq, const float* __restrict__ pk, int64_t Hq, int64_t Hkv,
    int64_t NB, int k, int kmax, int32_t* __restrict__ idx, int32_t* __restrict__ cnt) {
  __shared__ float sc[kMaxBlocks];
  __shared__ int32_t id[kMaxBlocks];
  __shared__ uint8_t take[kMaxBlocks];
  __shared__ float qrow[D];
  const int64_t g = blockIdx.x / NB, i = blockIdx.x % NB;
  const int64_t G = Hq / Hkv;
  const int tid = threadIdx.x;
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
    // candidates 1 .. i-1, padded to a power of two with -inf
    const int ncand = static_cast<int>(i - 1);
    int n2 = 1;
    while (n2 < ncand) n2 <<= 1;
    for (int e = tid; e < n2; e += kSelThreads) {
      float s = -INFINITY;
      const int j = e + 1;
      if (e < ncand) {
        const float4* kr = reinterpret_cast<const float4*>(pk + (g * NB + j) * D);
        float a = 0.0f;
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const float4 kv = kr[d4];
          a += qrow[4 * d4] * kv.x;
          a += qrow[4 * d4 + 1] * kv.y;
          a += qrow[4 * d4 + 2] * kv.z;
          a += qrow[4 * d4 + 3] * kv.w;
        }
        s = a;
      }
      sc[e] = s;
      id[e] = e < ncand ? j : 0x7fffffff;
    }
    __syncthreads();
    // bitonic sort, "before" = higher score, then lower block
    for (int size = 2; size <= n2; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int e = tid; e < n2 / 2; e += kSelThreads) {
          const int lo = 2 * e - (e & (stride - 1)), hi = lo + stride;
          const bool up = (lo & size) == 0;         // this run sorts "before"-first
          const float s0 = sc[lo], s1 = sc[hi];
          const int32_t i0 = id[lo], i1 = id[hi];
          const bool hi_first = s1 > s0 || (s1 == s0 && i1 < i0);
          if (hi_first == up) {
            sc[lo] = s1;
            sc[hi] = s0;
            id[lo] = i1;
            id[hi] = i0;
          }
        }
        __syncthreads();
      }
    for (int e = tid; e < k - 2; e += kSelThreads) take[id[e]] = 1;
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

template <int D>
struct FwdLds {
  static constexpr int kKPitch = D + 8;          // bf16 per K row (272 bytes at D = 128)
  static constexpr int kVPitch = kBlk + 8;       // bf16 per V^T row (144 bytes)
  uint16_t k[kBlk * kKPitch];
  uint16_t vt[D * kVPitch];
};

template <int D, bool kBf16Out>
__global__ __launch_bounds__(256, 3) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int64_t L, int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t NB,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int kmax,
    void* __restrict__ out, int64_t ldo, float scale_log2) {
  using Lds = FwdLds<D>;
  __shared__ Lds lds;
  constexpr int KC = D / 32;                     // 32-wide d chunks of a score product
  constexpr int DT = D / 16;                     // 16-row d tiles of the output
  // Tiles (query block i, K/V head g), later blocks first (they list the
  // most key blocks); the G = Hq/Hkv query heads of a tile share its list,
  // so their workgroups are given ids 8 apart: workgroups are dealt to the
  // 8 XCDs in turn, so the G of them run together on one XCD and read the
  // listed K/V blocks through its L2.
  const int64_t wg = blockIdx.x, G = Hq / Hkv, tiles = NB * Hkv;
  int64_t t, hh;
  if (tiles % 8 == 0) {
    const int64_t x = wg % 8, y = wg / 8;
    hh = y % G;
    t = (y / G) * 8 + x;
  } else {
    t = wg / G;
    hh = wg % G;
  }
  const int64_t i = NB - 1 - t / Hkv, g = t % Hkv, h = g * G + hh;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, c = lane & 15, gq = lane >> 4;
  const int64_t q0 = i * kBlk + 16 * wave;       // the wave's first query
  const int64_t q = q0 + c;                      // this lane's query

  // Q^T operand: lane holds Q[q][32 kc + 8 gq .. +8] for every chunk kc
  bf8 qb[KC];
  {
    // rows of the wave's queries inside the sequence (none for a wave of the
    // last, partial block that lies wholly past L)
    const int64_t rows = L - q0 <= 0 ? 0 : (L - q0 < 16 ? L - q0 : 16);
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(Q + q0 * ldq + h * D, static_cast<uint32_t>(rows * ldq * 2));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const v4u w = __builtin_amdgcn_raw_buffer_load_b128(
          rq, static_cast<uint32_t>((c * ldq + 32 * kc + 8 * gq) * 2), 0, 0);
      qb[kc] = __builtin_bit_cast(bf8, w);
    }
  }

  f4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f4{0, 0, 0, 0};
  float m = -INFINITY, lsum = 0.0f;

  // the list is device data: clamp its length and skip entries outside the
  // blocks a query block may see, so that no entry can move a load off its
  // buffer
  const int n_raw = cnt[g * NB + i];
  const int n = n_raw < 0 ? 0 : (n_raw > kmax ? kmax : n_raw);
  const int32_t* list = idx + (g * NB + i) * kmax;   // the K/V head's list
  const int tid = threadIdx.x;
  auto next_valid = [&](int b) {                 // uniform
    for (; b < n; ++b) {
      const int32_t j = list[b];
      if (j >= 0 && j <= i) break;
    }
    return b;
  };

  // Global loads of a K/V block into registers, issued one block ahead.
  // K: 16-byte chunks, row e / (D/8), column chunk e % (D/8).  V: a thread
  // takes 4 consecutive keys (quad kq = e % 16) x 8 columns (octet
  // dc = e / 16), so that its transposed 8-byte writes to LDS fall on
  // distinct banks across 32 lanes.
  constexpr int kKPer = kBlk * D / 8 / 256;      // K chunks per thread
  constexpr int kVGroups = (kBlk / 4) * (D / 8); // (key quad, column octet) pairs
  static_assert(kVGroups <= 256, "one V group per thread");
  v4u kreg[kKPer], vreg[4];
  auto load_block = [&](int64_t j) {
    const int64_t rows = L - j * kBlk < kBlk ? L - j * kBlk : kBlk;
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(K + j * kBlk * ldk + g * D, static_cast<uint32_t>(rows * ldk * 2));
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int e = u * 256 + tid, row = e / (D / 8), cc = e % (D / 8);
      kreg[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, static_cast<uint32_t>((row * ldk + 8 * cc) * 2), 0, 0);
    }
    if (tid < kVGroups) {
      const __amdgpu_buffer_rsrc_t rv = rows_rsrc(V + j * kBlk * ldv + g * D, static_cast<uint32_t>(rows * ldv * 2));
      const int kq = tid % 16, dc = tid / 16;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vreg[r] = __builtin_amdgcn_raw_buffer_load_b128(
            rv, static_cast<uint32_t>(((4 * kq + r) * ldv + 8 * dc) * 2), 0, 0);
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int e = u * 256 + tid, row = e / (D / 8), cc = e % (D / 8);
      *reinterpret_cast<v4u*>(&lds.k[row * Lds::kKPitch + 8 * cc]) = kreg[u];
    }
    if (tid < kVGroups) {
      const int kq = tid % 16, dc = tid / 16;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // columns 8dc + 2w (low halves) and 8dc + 2w + 1 (high halves)
        const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        *reinterpret_cast<v2u*>(&lds.vt[(8 * dc + 2 * w) * Lds::kVPitch + 4 * kq]) = v2u{lo01, lo23};
        *reinterpret_cast<v2u*>(&lds.vt[(8 * dc + 2 * w + 1) * Lds::kVPitch + 4 * kq]) = v2u{hi01, hi23};
      }
    }
  };

  int bi = next_valid(0);
  if (bi < n) load_block(list[bi]);
  while (bi < n) {
    const int64_t j = list[bi];
    __syncthreads();                             // the previous block's LDS reads are done
    store_block();
    __syncthreads();
    bi = next_valid(bi + 1);
    if (bi < n) load_block(list[bi]);            // in flight during this block's products

    // scores: s[kt][r] = S[key 16 kt + 4 gq + r][query c], scaled to base 2
    f4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const bf8 a = *reinterpret_cast<const bf8*>(&lds.k[(16 * kt + c) * Lds::kKPitch + 32 * kc + 8 * gq]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kc], acc, 0, 0, 0);
      }
      s[kt] = acc;
    }
    // causal mask, in the diagonal block only (uniform branch)
    if (j == i) {
      const int qi = static_cast<int>(q - i * kBlk);   // query's row in the block
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kt + 4 * gq + r > qi) s[kt][r] = -INFINITY;
    }
    // row maximum over the block's keys (4 lanes share a query), in base 2
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      mx = fmaxf(fmaxf(mx, fmaxf(s[kt][0], s[kt][1])), fmaxf(s[kt][2], s[kt][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
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
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], scale_log2, -m));
        s[kt][r] = p;
        lsum += p;
      }

    // O^T += V^T P^T, two 32-key chunks: slots 8 gq .. 8 gq + 3 are keys
    // 32 pc + 4 gq + r (tile 2 pc), slots 8 gq + 4 .. + 7 keys 32 pc + 16 + 4 gq + r
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
      typedef float f2 __attribute__((ext_vector_type(2)));
      const bf2 p01 = __builtin_convertvector((f2{s[2 * pc][0], s[2 * pc][1]}), bf2);
      const bf2 p23 = __builtin_convertvector((f2{s[2 * pc][2], s[2 * pc][3]}), bf2);
      const bf2 p45 = __builtin_convertvector((f2{s[2 * pc + 1][0], s[2 * pc + 1][1]}), bf2);
      const bf2 p67 = __builtin_convertvector((f2{s[2 * pc + 1][2], s[2 * pc + 1][3]}), bf2);
      const v4u pw = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23),
                      __builtin_bit_cast(uint32_t, p45), __builtin_bit_cast(uint32_t, p67)};
      const bf8 pb = __builtin_bit_cast(bf8, pw);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* vr = &lds.vt[(16 * dt + c) * Lds::kVPitch + 32 * pc + 4 * gq];
        const v2u lo = *reinterpret_cast<const v2u*>(vr);
        const v2u hi = *reinterpret_cast<const v2u*>(vr + 16);
        const v4u aw = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, aw), pb, o[dt], 0, 0, 0);
      }
    }
  }

  // the 4 lanes of a query hold parts of its row sum
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  // O[q][h*D + 16 dt + 4 gq + r] = o[dt][r] / lsum
  if (q < L) {
    const float inv = 1.0f / lsum;
    if constexpr (kBf16Out) {
      uint16_t* orow = static_cast<uint16_t*>(out) + q * ldo + h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        const bf2 a = __builtin_convertvector((f2{o[dt][0] * inv, o[dt][1] * inv}), bf2);
        const bf2 b = __builtin_convertvector((f2{o[dt][2] * inv, o[dt][3] * inv}), bf2);
        *reinterpret_cast<v2u*>(orow + 16 * dt + 4 * gq) =
            v2u{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
      }
    } else {
      float* orow = static_cast<float*>(out) + q * ldo + h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f4*>(orow + 16 * dt + 4 * gq) = o[dt] * inv;
    }
  }
}

}  // namespace

hipError_t launch_attn_pool(const uint16_t* x, int64_t L, int64_t ldx, int64_t H, int64_t D,
                            float* pooled, hipStream_t stream) {
  const int64_t NB = (L + kBlk - 1) / kBlk;
  const int64_t per = 256 / (D / 8);
  const uint32_t grid = static_cast<uint32_t>((H * NB + per - 1) / per);
  if (D == 128)
    hipLaunchKernelGGL((attn_pool_kernel<128>), dim3(grid), dim3(256), 0, stream, x, L, ldx, H, NB, pooled);
  else
    hipLaunchKernelGGL((attn_pool_kernel<64>), dim3(grid), dim3(256), 0, stream, x, L, ldx, H, NB, pooled);
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
  const uint32_t grid = static_cast<uint32_t>(Hq * NB);
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
#define Q8_ATTN_LAUNCH(DD, BF)                                                                   \
  hipLaunchKernelGGL((attn_fwd_kernel<DD, BF>), dim3(grid), dim3(256), 0, stream, q, k, v, L, ldq, \
                     ldk, ldv, Hq, Hkv, NB, idx, cnt, kmax, out, ldo, scale_log2)
  if (D == 128) {
    if (out_dtype == 1) Q8_ATTN_LAUNCH(128, true);
    else Q8_ATTN_LAUNCH(128, false);
  } else {
    if (out_dtype == 1) Q8_ATTN_LAUNCH(64, true);
    else Q8_ATTN_LAUNCH(64, false);
  }
#undef Q8_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace q8
