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
// of one block for a 32x32 output tile.  A variant runs on
// v_mfma_i32_16x16x32_i8 (half the rate, a quarter of the registers per
// partial), which leaves room to pipeline MFMA and epilogue inside a wave.
//
// Scale epilogue (the binding cost).  Each 32x32 int32 partial needs its
// two per-block scales applied and must be accumulated in binary32.  The
// accumulator input of the MFMA is preset to the bits of 1.5*2^23, so the
// int32 result, read as binary32, is exactly 1.5*2^23 + P (|P| < 2^22).
// Then
//     y   = fma(Pbits, d_w, -1.5*2^23*d_w)   = RN(P * d_w)     (one rounding)
//     acc = fma(y, d_a, acc)                                     (one rounding)
// i.e. two VALU operations per output and block, with no int->float
// conversion.  d_w is per lane (lane = output column); the pair
// (d_w, -1.5*2^23*d_w) is prepared once per block when staged (the product
// is exact: d_w has 11 significant bits).  Against 1024 int8 MACs per clock
// per SIMD, 32 unpacked binary32 FMAs per 32-cycle MFMA tile cap the kernel
// well below the matrix-core peak: a single wave issues an FMA every ~4.6
// clocks, two waves of a SIMD together one every ~2.2-2.7 (measured), and
// an MFMA blocks vector issue on its SIMD while it executes, so one MFMA and
// its 32 FMAs take at least ~104 SIMD cycles: about 0.3 of the peak per
// clock.  The kernel is built to keep the VALU issuing epilogue FMAs and
// little else, and to move as little data as it can: it runs at the chip's
// power limit, where saved data movement comes back as clock.
//
// Data movement.  A workgroup of WAVES_M x WAVES_N waves owns a BM x BN
// output tile; K advances in stages of KBS blocks through two LDS buffers.
// Quant tiles go HBM -> LDS with buffer_load ... lds (no registers, no LDS
// stores), through buffer resources that end at the last valid activation
// row and packed weight group, so ragged edges read as zero without
// branches.  Scales come through registers (to be widened to binary32) and
// are stored after the stage's arithmetic.  LDS holds each operand as
// 16-byte slices in [block][half][row] order, so a fragment load (lane l:
// row l%32, half l/32) reads 512 contiguous bytes per half-wave.
//
// Occupancy.  The epilogue issues at rate only with several waves per SIMD
// (one wave alone issues an FMA every ~4.6 clocks).  Large grids get them
// from 128x384 tiles of twelve 32x128 waves (one workgroup per CU, three
// waves per SIMD, whose priorities rotate block by block because a SIMD
// interleaves only two waves at a time; a 32x128 wave tile reads its
// activation scales once for four MFMAs) when the grid suits them (see
// choose_tile in q8_tilemap.h), else from 128x128 tiles, two
// workgroups of eight waves per CU, each wave issuing its MFMAs ahead of
// their epilogues.  Grids with too few tiles split every stage's blocks
// between K groups of waves instead, and add the groups' partial sums
// through LDS at the end (Tile::KSPLIT).
//
// LDS reads are inline asm with immediate offsets: the compiler cannot tell
// a read of one stage buffer from the asynchronous loads into the other and
// would wait for those before every read; the buffer a stage reads is
// complete once the stage's barrier has passed (every wave waits for its own
// loads before it).  The reads' completion is awaited explicitly before
// their values are used, and the asm carries a memory clobber.
//
// Workgroup order (q8_tilemap.h): tiles run M-fastest so consecutive
// workgroups share a weight tile; when the grid is a multiple of 8 the ids
// are remapped so each of the 8 XCDs (which receive workgroups round-robin)
// gets one contiguous range, or one rectangle, of tiles and keeps its
// operand panels in its own L2.
#include <cstdio>
#include <cstdlib>
#include <type_traits>
#include <utility>

#include "q8_kernels.h"
#include "q8_tilemap.h"

namespace q8 {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr float kBias = 12582912.0f;            // 1.5 * 2^23
constexpr int kBiasBits = 0x4B400000;           // its binary32 bits
[[maybe_unused]] constexpr uint32_t kOutOfRange = 0xFFFFFFFFu;   // buffer offset that reads as zero
constexpr int kStoreNT = 2;   // cache-policy operand of a buffer store: non-temporal

// MF: output tile of one MFMA, 32 (v_mfma_i32_32x32x32_i8) or 16
// (v_mfma_i32_16x16x32_i8).
// KSPLIT_ > 1: the workgroup's waves form KSPLIT groups of WAVES_M x
// WAVES_N; group g computes blocks [g*KBS/KSPLIT, (g+1)*KBS/KSPLIT) of every
// stage, and the groups' partial sums are added through LDS at the end, in
// group order.  This gives grids with few output tiles (small M, narrow N)
// several waves per SIMD.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int KBS_, int NBUF_, int MF_ = 32,
          int PIPE_ = 0, int KSPLIT_ = 1>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, KBS = KBS_;
  static constexpr int NBUF = NBUF_;                           // LDS stage buffers
  static constexpr int MF = MF_;
  static constexpr int PIPE = PIPE_;
  static constexpr int KSPLIT = KSPLIT_;
  static constexpr int NB = KBS / KSPLIT;                      // blocks per wave per stage
  static constexpr int kAccN = MF * MF / 64;                   // accumulator values per lane and tile
  static constexpr int kWavesT = WAVES_M * WAVES_N;            // waves of one K group
  static constexpr int kThreads = kWavesT * KSPLIT * 64;
  static constexpr int kWaves = kWavesT * KSPLIT;
  // Priorities that compute_stage rotates block by block (wave w runs on
  // SIMD w % 4): twelve waves, one workgroup per CU, three per SIMD (period
  // 3); eight waves of one K group, two workgroups per CU, so two of each
  // workgroup's on each SIMD (period 2: measured 1-2 % faster on the large
  // grids that take these tiles; with one workgroup per CU, as the K-group
  // tiles run, it measured 4-6 % slower, so those keep fixed priorities).
  static constexpr bool kRotatePrio = kWaves == 12 || (kWaves == 8 && KSPLIT == 1);
  static constexpr int kPrioPeriod = kWaves == 12 ? 3 : 2;
  static_assert(!kRotatePrio || NB % kPrioPeriod == 0, "priorities rotate over whole stages");
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;   // per-wave tile
  static constexpr int TM = WM / MF, TN = WN / MF;             // MFMA tiles per wave
  static constexpr int kSlots = 2 * KBS;                       // 16-byte slots per row per stage
  // LDS per stage (bytes)
  static constexpr int kAq = KBS * 2 * BM * 16;                // activation quants [kb][h][row]
  static constexpr int kBq = KBS * 2 * BN * 16;                // weight quants [kb][h][col]
  static constexpr int kAs = KBS * BM * 4;                     // d_a [kb][row], binary32
  static constexpr int kBs = KBS * BN * 8;                     // (d_w, -1.5*2^23*d_w) [kb][col]
  static constexpr int kStage = kAq + kBq + kAs + kBs;
  // loads per wave per stage, scales per thread per stage
  static constexpr int kAInst = BM * kSlots / 64 / kWaves;
  static constexpr int kBInst = (BN / kGroupRows) * 2 * KBS / kWaves;
  static constexpr int kASc = (BM * KBS + kThreads - 1) / kThreads;
  // Weight scales go in pairs of adjacent columns (one dword load and one
  // 16-byte LDS write per pair) when there are more than one per thread.
  static constexpr bool kBPair = BN * KBS > kThreads;
  static constexpr int kBPer = kBPair ? 2 : 1;                 // columns per load
  static constexpr int kBSc = (BN * KBS / kBPer + kThreads - 1) / kThreads;
  static_assert(MF == 32 || MF == 16, "MFMA shape");
  static_assert(WM % MF == 0 && WN % MF == 0, "wave tile must be a multiple of the MFMA tile");
  static_assert(BN % kGroupRows == 0, "BN must cover whole 64-row groups");
  static_assert(BM % 64 == 0, "activation loads cover 64 rows each");
  static_assert(kAInst * 64 * kWaves == BM * kSlots, "activation loads split over waves");
  static_assert(kBInst * kWaves == (BN / kGroupRows) * 2 * KBS, "weight loads split over waves");
  static_assert(NBUF >= 2 && NBUF * kStage <= 160 * 1024, "LDS");
  // VMEM instructions per stage: quant loads per wave, scale loads per thread
  static constexpr int kDmaOps = kAInst + kBInst;
  static constexpr int kScaleOps = kASc + kBSc;
  // Loads issued after a stage's quant loads by the time that stage is
  // waited for (see the stage loop).
  static constexpr int kInFlight = (NBUF - 1) * kScaleOps + (NBUF - 2) * kDmaOps;
  static_assert(kInFlight < 64, "vmcnt range");
  static_assert(kStage < 65536, "immediate LDS offsets");
  static_assert(KBS % KSPLIT == 0 && (KSPLIT == 1 || MF == 32), "K groups");
  // partial sums of groups 1.. go through the stage buffers
  static_assert((KSPLIT - 1) * kWavesT * TM * TN * kAccN * 64 * 4 <= NBUF * kStage, "LDS");
};

// ---------------------------------------------------------------------------
// compile-time loops and LDS access
// ---------------------------------------------------------------------------

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_ptr)(const_cast<void*>(p))));
}

template <int OFF>
__device__ __forceinline__ v4i lds_read_b128(uint32_t base) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ v2f lds_read_b64(uint32_t base) {
  v2f v;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(base), "i"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ void lds_write_b32(uint32_t base, float v) {
  asm volatile("ds_write_b32 %0, %1 offset:%2" : : "v"(base), "v"(v), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_write_b64(uint32_t base, v2f v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" : : "v"(base), "v"(v), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void lds_write_b128(uint32_t base, v4f v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(base), "v"(v), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Ties a value to the preceding wait so that no use of it moves above it.
template <class V>
__device__ __forceinline__ void after_wait(V& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, range check against num_records (bytes)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// per-workgroup state
// ---------------------------------------------------------------------------

struct Rsrc {
  __amdgpu_buffer_rsrc_t ra;    // q_a rows [m0, m0 + rows_valid)
  __amdgpu_buffer_rsrc_t rb;    // packed quant pieces of the tile's row groups
  __amdgpu_buffer_rsrc_t rsa;   // d_a rows [m0, m0 + rows_valid)
  __amdgpu_buffer_rsrc_t rsb;   // weight scales of the tile's row groups
  __amdgpu_buffer_rsrc_t rnull; // empty range: every load reads zero, touches no memory
  int KB;
};

// Per-lane byte offsets of one stage's loads, relative to the stage's first
// block (the stage adds a wave-uniform offset).  Computed once per
// workgroup: the stage loop then spends no VALU on addressing.
template <class T>
struct LaneOffsets {
  uint32_t a[T::kAInst];      // activation quant loads (into LDS)
  uint32_t b[T::kBInst];      // weight quant loads (into LDS)
  uint32_t sa[T::kASc];       // activation scale loads
  uint32_t sb[T::kBSc];       // weight scale loads (of kBPer adjacent columns)
  int lim_a[T::kASc];         // the scale load is in range while kb0 < lim
  int lim_b[T::kBSc];
};

template <class T>
__device__ __forceinline__ void lane_offsets(LaneOffsets<T>& o, int tid, int wave, int lane,
                                             uint32_t K, uint32_t KB) {
  constexpr uint32_t BM = T::BM, BN = T::BN, KBS = T::KBS;
#pragma unroll
  for (int u0 = 0; u0 < T::kAInst; ++u0) {
    const uint32_t u = wave * T::kAInst + u0;
    const uint32_t s = u / (BM / 64), mb = u % (BM / 64);
    o.a[u0] = (mb * 64 + lane) * K + s * 16;
  }
#pragma unroll
  for (int u0 = 0; u0 < T::kBInst; ++u0) {
    const uint32_t u = wave * T::kBInst + u0;
    const uint32_t gl = u / (2 * KBS), kbl = (u >> 1) % KBS, h = u & 1;
    o.b[u0] = ((gl * KB + kbl) * 2 + h) * kPieceBytes + lane * 16;
  }
#pragma unroll
  for (int i = 0; i < T::kASc; ++i) {
    const uint32_t idx = i * T::kThreads + tid;
    const uint32_t m = idx % BM, kbl = idx / BM;
    o.sa[i] = (m * KB + kbl) * 2;
    o.lim_a[i] = idx < BM * KBS ? static_cast<int>(KB - kbl) : 0;
  }
#pragma unroll
  for (int i = 0; i < T::kBSc; ++i) {
    const uint32_t idx = T::kBPer * (i * T::kThreads + tid);   // first column of the load
    const uint32_t n = idx % BN, kbl = idx / BN;
    o.sb[i] = (((n / kGroupRows) * KB + kbl) * kGroupRows + n % kGroupRows) * 2;
    o.lim_b[i] = idx < BN * KBS ? static_cast<int>(KB - kbl) : 0;
  }
}

// Issue quant loads [P0, P1) of one stage (the wave's activation loads,
// then its weight loads): HBM -> LDS, no registers.  The stage loop spreads
// a stage's loads over the blocks of the previous stage's arithmetic, so a
// wave never queues all of them at once behind the other waves' loads.
template <class T, int P0, int P1>
__device__ __forceinline__ void issue_quants(const Rsrc& r, const LaneOffsets<T>& o, int wave,
                                             int kb0, uint8_t* buf) {
#if __HIP_DEVICE_COMPILE__   // the buffer builtins exist only in the device pass
  constexpr int BM = T::BM, BN = T::BN, KBS = T::KBS;
  if constexpr (P0 < P1) {
    kb0 = __builtin_amdgcn_readfirstlane(kb0);   // wave-uniform: the loads' scalar offsets
    // Stages past the end load nothing (the pipeline issues them anyway so
    // that its wait counts are the same every iteration).
    const bool live = kb0 < r.KB;
    const __amdgpu_buffer_rsrc_t ra = live ? r.ra : r.rnull;
    const __amdgpu_buffer_rsrc_t rb = live ? r.rb : r.rnull;
    static_for<P1 - P0>([&](auto p_) __attribute__((always_inline)) {
      constexpr int pi = P0 + decltype(p_)::value;
      if constexpr (pi < T::kAInst) {
        const int u = wave * T::kAInst + pi;
        const int s = u / (BM / 64), mb = u % (BM / 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)(buf + (s * BM + mb * 64) * 16),
                                                 16, o.a[pi], static_cast<uint32_t>(kb0 * kQK), 0, 0);
      } else {
        constexpr int u0 = pi - T::kAInst;
        const int u = wave * T::kBInst + u0;
        const int gl = u / (2 * KBS), kbl = (u >> 1) % KBS, h = u & 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_ptr)(buf + T::kAq + ((kbl * 2 + h) * BN + gl * kGroupRows) * 16), 16,
            o.b[u0], static_cast<uint32_t>(kb0 * kGroupBlockBytes), 0, 0);
      }
    });
  }
#endif
}

// Load one stage's binary16 scales into registers (blocks past K/32 read as
// zero through an out-of-range offset).
template <class T>
__device__ __forceinline__ void load_scales(const Rsrc& r, const LaneOffsets<T>& o, int kb0,
                                            uint16_t (&as_r)[T::kASc], uint32_t (&bs_r)[T::kBSc]) {
#if __HIP_DEVICE_COMPILE__
  kb0 = __builtin_amdgcn_readfirstlane(kb0);
#pragma unroll
  for (int i = 0; i < T::kASc; ++i)
    as_r[i] = __builtin_amdgcn_raw_buffer_load_b16(r.rsa, kb0 < o.lim_a[i] ? o.sa[i] : kOutOfRange,
                                                   static_cast<uint32_t>(kb0 * 2), 0);
#pragma unroll
  for (int i = 0; i < T::kBSc; ++i)
    if constexpr (T::kBPair)
      bs_r[i] = __builtin_amdgcn_raw_buffer_load_b32(
          r.rsb, kb0 < o.lim_b[i] ? o.sb[i] : kOutOfRange,
          static_cast<uint32_t>(kb0 * kGroupRows * 2), 0);
    else
      bs_r[i] = __builtin_amdgcn_raw_buffer_load_b16(
          r.rsb, kb0 < o.lim_b[i] ? o.sb[i] : kOutOfRange,
          static_cast<uint32_t>(kb0 * kGroupRows * 2), 0);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Widen the stage's scales and store them: d_a as binary32, d_w as the pair
// (d_w, -1.5*2^23*d_w) the epilogue consumes.
//
// d_a is stored in groups of four rows rotated by one slot (row 4g + t at
// slot 4g + (t + 3) % 4).  A lane reads a group with one 16-byte load into
// four consecutive VGPRs, and its accumulators of the same four rows are
// consecutive VGPRs too; both tuples start on an even register, so unrotated
// the scale and the accumulator of row r always share a VGPR bank (register
// index mod 4), and the epilogue's v_fmac_f32, which reads both, then issues
// at about half the rate when two or more waves of a SIMD interleave
// (measured on gfx950: a block of one MFMA and 32 FMAs per tile took 108 ->
// 92 cycles per MFMA at four waves per SIMD, 113 -> 98 at two).  Rotated,
// the two banks always differ.
template <class T>
__device__ __forceinline__ void store_scales(int tid, uint8_t* buf, const uint16_t (&as_r)[T::kASc],
                                             const uint32_t (&bs_r)[T::kBSc]) {
  static_assert(T::kThreads % 4 == 0 && T::BM % 4 == 0, "a thread keeps its row mod 4");
  const uint32_t as = lds_addr(buf + T::kAq + T::kBq) + (tid & ~3) * 4 + ((tid + 3) & 3) * 4;
  const uint32_t bs = lds_addr(buf + T::kAq + T::kBq + T::kAs) + tid * 8 * T::kBPer;
  static_for<T::kASc>([&](auto i_) __attribute__((always_inline)) {
    constexpr int i = decltype(i_)::value;
    if (i * T::kThreads + tid < T::BM * T::KBS)
      lds_write_b32<i * T::kThreads * 4>(as, f16_bits_to_f32(as_r[i]));
  });
  static_for<T::kBSc>([&](auto i_) __attribute__((always_inline)) {
    constexpr int i = decltype(i_)::value;
    if (T::kBPer * (i * T::kThreads + tid) < T::BN * T::KBS) {
      const float w0 = f16_bits_to_f32(static_cast<uint16_t>(bs_r[i]));
      if constexpr (T::kBPair) {
        const float w1 = f16_bits_to_f32(static_cast<uint16_t>(bs_r[i] >> 16));
        lds_write_b128<i * T::kThreads * 16>(bs, v4f{w0, -kBias * w0, w1, -kBias * w1});
      } else {
        lds_write_b64<i * T::kThreads * 8>(bs, v2f{w0, -kBias * w0});
      }
    }
  });
}

// Wave priorities (Tile::kRotatePrio).  A SIMD interleaves the vector
// instructions of two waves at a time; with three resident, the two of
// higher priority (or, at equal priority, the older two) take nearly every
// issue slot and the third runs only when one of them stalls.  Measured on
// gfx950 with one MFMA and 32 FMAs per tile and no memory access, the third
// wave finished at 1.8x the time of the other two.  Behind a per-stage
// barrier the other two then wait for it.  Rotating the priorities block by
// block, so that each wave is the low one for a third of the blocks, keeps
// the three together: 130 -> 118 cycles per MFMA in that probe with LDS
// operand reads and a barrier every three blocks.  The 128x128 tiles, two
// workgroups of eight waves per CU, alternate the two waves of each
// workgroup on a SIMD the same way.
// The branch on p (0, 1 or 2; s_setprio takes only an immediate) stays
// inside one asm statement, so it splits no basic block of the compiled loop.
__device__ __forceinline__ void set_wave_prio(int p) {
  asm volatile(
      "s_cmp_eq_u32 %0, 2\n\t"
      "s_cbranch_scc0 1f\n\t"
      "s_setprio 2\n\t"
      "s_branch 3f\n"
      "1:\n\t"
      "s_cmp_eq_u32 %0, 1\n\t"
      "s_cbranch_scc0 2f\n\t"
      "s_setprio 1\n\t"
      "s_branch 3f\n"
      "2:\n\t"
      "s_setprio 0\n"
      "3:"
      :
      : "s"(p)
      : "scc");
}

// The arithmetic of one stage (KBS blocks) from an LDS buffer.  Lane-
// dependent parts of every LDS address are in the four base registers; the
// block, tile and row-group parts are immediate offsets.  prio0 (0, 1 or
// 2): the wave's priority for the stage's first block (see set_wave_prio),
// used when three waves share a SIMD (twelve-wave workgroups, one per CU).
template <class T, class F>
__device__ __forceinline__ void compute_stage(uint32_t base_a, uint32_t base_as, uint32_t base_b,
                                              uint32_t base_bs, const v16i& bias,
                                              v16f (&acc)[T::TM][T::TN], F&& at_block, int prio0) {
  constexpr int TM = T::TM, TN = T::TN, BM = T::BM, BN = T::BN;
  static_for<T::NB>([&](auto kb_) __attribute__((always_inline)) {
    constexpr int kb = decltype(kb_)::value;
    if constexpr (T::kRotatePrio) {
      if constexpr (T::kPrioPeriod == 3)
        set_wave_prio(prio0 + kb < 3 ? prio0 + kb : prio0 + kb - 3);
      else
        set_wave_prio((prio0 + kb) & 1);
    }
    v4i af[TM], avq[TM][4], bf[TN];
    v2f wp[TN];
    static_for<TM>([&](auto i_) __attribute__((always_inline)) {
      constexpr int i = decltype(i_)::value;
      af[i] = lds_read_b128<(kb * 2 * BM + 32 * i) * 16>(base_a);
      // Rows held by this lane in the MFMA output: 8*(r/4) + 4*half + r%4.
      static_for<4>([&](auto q_) __attribute__((always_inline)) {
        constexpr int q = decltype(q_)::value;
        avq[i][q] = lds_read_b128<(kb * BM + 32 * i + 8 * q) * 4>(base_as);
      });
    });
    static_for<TN>([&](auto j_) __attribute__((always_inline)) {
      constexpr int j = decltype(j_)::value;
      bf[j] = lds_read_b128<(kb * 2 * BN + 32 * j) * 16>(base_b);
      wp[j] = lds_read_b64<(kb * BN + 32 * j) * 8>(base_bs);
    });
    at_block(kb_);
    lds_wait_all();
    static_for<TM>([&](auto i_) __attribute__((always_inline)) {
      constexpr int i = decltype(i_)::value;
      after_wait(af[i]);
      static_for<4>([&](auto q_) __attribute__((always_inline)) { after_wait(avq[i][decltype(q_)::value]); });
    });
    static_for<TN>([&](auto j_) __attribute__((always_inline)) {
      after_wait(bf[decltype(j_)::value]);
      after_wait(wp[decltype(j_)::value]);
    });
    // One MFMA tile at a time keeps a single 16-register partial live; the
    // other waves of the SIMD cover the matrix-core latency.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float av[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // groups are stored rotated by one (store_scales): row 4q + t at slot (t + 3) % 4
        av[4 * q + 0] = __int_as_float(avq[i][q].w);
        av[4 * q + 1] = __int_as_float(avq[i][q].x);
        av[4 * q + 2] = __int_as_float(avq[i][q].y);
        av[4 * q + 3] = __int_as_float(avq[i][q].z);
      }
      if constexpr (T::PIPE) {
        // All of the row tile's MFMAs first: the later ones run on the matrix
        // core while this wave applies the scales to the first.
        v16i p[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          p[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], bias, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = fmaf(__int_as_float(p[j][r]), wp[j].x, wp[j].y);
            acc[i][j][r] = fmaf(y, av[r], acc[i][j][r]);
          }
      } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], bias, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = fmaf(__int_as_float(p[r]), wp[j].x, wp[j].y);
          acc[i][j][r] = fmaf(y, av[r], acc[i][j][r]);
        }
      }
      }
    }
    // Keep blocks apart: the block's accumulator updates complete before the
    // next block's LDS reads are issued (otherwise the compiler hoists MFMAs
    // of later blocks and their partials overflow the register budget).
    static_for<TM>([&](auto i_) __attribute__((always_inline)) {
      static_for<TN>([&](auto j_) __attribute__((always_inline)) {
        after_wait(acc[decltype(i_)::value][decltype(j_)::value]);
      });
    });
  });
}

// Operands of one block for a wave's 16x16 tiles: quant fragments (lane l:
// row or column l%16, block bytes 8*(l/16) .. +8), d_a for the lane's four
// output rows of each row tile, and the (d_w, -1.5*2^23*d_w) pair of the
// lane's column of each column tile.
template <class T>
struct Frag16 {
  v2i a[T::TM], b[T::TN];
  v4f as[T::TM];
  v2f ws[T::TN];
};

template <class T, int KB>
__device__ __forceinline__ void read_frag16(Frag16<T>& f, uint32_t base_a, uint32_t base_as,
                                            uint32_t base_b, uint32_t base_bs) {
  constexpr int BM = T::BM, BN = T::BN;
  static_for<T::TM>([&](auto i_) __attribute__((always_inline)) {
    constexpr int i = decltype(i_)::value;
    const v2f a = lds_read_b64<(KB * 2 * BM + 16 * i) * 16>(base_a);
    f.a[i] = __builtin_bit_cast(v2i, a);
    const v4i s = lds_read_b128<(KB * BM + 16 * i) * 4>(base_as);
    f.as[i] = __builtin_bit_cast(v4f, s);
  });
  static_for<T::TN>([&](auto j_) __attribute__((always_inline)) {
    constexpr int j = decltype(j_)::value;
    const v2f b = lds_read_b64<(KB * 2 * BN + 16 * j) * 16>(base_b);
    f.b[j] = __builtin_bit_cast(v2i, b);
    f.ws[j] = lds_read_b64<(KB * BN + 16 * j) * 8>(base_bs);
  });
}

template <class T>
__device__ __forceinline__ void tie_frag16(Frag16<T>& f) {
  static_for<T::TM>([&](auto i_) __attribute__((always_inline)) {
    after_wait(f.a[decltype(i_)::value]);
    after_wait(f.as[decltype(i_)::value]);
  });
  static_for<T::TN>([&](auto j_) __attribute__((always_inline)) {
    after_wait(f.b[decltype(j_)::value]);
    after_wait(f.ws[decltype(j_)::value]);
  });
}

// One stage with 16x16 MFMAs, software-pipelined inside the wave: the MFMA
// of tile u+1 is issued before the epilogue of tile u (so its latency is
// covered by this wave's own FMAs), and the operands of block kb+1 are read
// from LDS while block kb is computed.  The empty asm statements order the
// schedule: the MFMA of tile u+2 takes the bias register as it stands after
// the epilogue of tile u, so at most two partials are live.
template <class T, class F>
__device__ __forceinline__ void compute_stage16(uint32_t base_a, uint32_t base_as, uint32_t base_b,
                                                uint32_t base_bs, v4i& bias,
                                                v4f (&acc)[T::TM][T::TN], F&& at_block) {
  constexpr int TM = T::TM, TN = T::TN, NT = TM * TN, KBS = T::KBS;
  Frag16<T> f[2];
  read_frag16<T, 0>(f[0], base_a, base_as, base_b, base_bs);
  lds_wait_all();
  tie_frag16<T>(f[0]);
  v4i p[2];
  p[0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
      __builtin_bit_cast(long, f[0].a[0]), __builtin_bit_cast(long, f[0].b[0]), bias, 0, 0, 0);
  static_for<KBS * NT>([&](auto u_) __attribute__((always_inline)) {
    constexpr int u = decltype(u_)::value;
    constexpr int kb = u / NT, t = u % NT, i = t / TN, j = t % TN;
    Frag16<T>& cur = f[kb & 1];
    if constexpr (t == 0 && kb + 1 < KBS)
      read_frag16<T, kb + 1>(f[(kb + 1) & 1], base_a, base_as, base_b, base_bs);
    if constexpr (t == 0) at_block(std::integral_constant<int, kb>{});
    if constexpr (u + 1 < KBS * NT) {
      constexpr int kb1 = (u + 1) / NT, t1 = (u + 1) % NT, i1 = t1 / TN, j1 = t1 % TN;
      if constexpr (t1 == 0) {   // first tile of the next block: its operands must be in
        lds_wait_all();
        tie_frag16<T>(f[kb1 & 1]);
      }
      Frag16<T>& nxt = f[kb1 & 1];
      p[(u + 1) & 1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          __builtin_bit_cast(long, nxt.a[i1]), __builtin_bit_cast(long, nxt.b[j1]), bias, 0, 0, 0);
    }
    const v4i& pu = p[u & 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float y = fmaf(__int_as_float(pu[r]), cur.ws[j].x, cur.ws[j].y);
      acc[i][j][r] = fmaf(y, cur.as[i][(r + 3) & 3], acc[i][j][r]);   // rotated groups
    }
    asm volatile("" : "+v"(acc[i][j]), "+v"(bias));
  });
}

// kSwiglu: the weight is a gate/up-packed weight (64-row group g = gate
// rows 32g.., then up rows 32g..; N = 2I) and, instead of C, the kernel
// writes h = silu(gate) * up quantised to Q8_0: q_h [M][I], d_h [M][I/32].
template <class T, int kWavesPerEU, bool kSwiglu = false>
__global__ __launch_bounds__(T::kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerEU)))
void gemm_q8_mfma_kernel(const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
                         const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws,
                         float* __restrict__ C, int64_t M, int64_t N, int64_t K, int64_t KB,
                         int64_t NG, int64_t ldc, int tiles_m, int remap,
                         int8_t* __restrict__ q_h, uint16_t* __restrict__ d_h) {
  constexpr int TM = T::TM, TN = T::TN, BM = T::BM, BN = T::BN, KBS = T::KBS;
  __shared__ __align__(16) uint8_t smem[T::NBUF * T::kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware workgroup order (q8_tilemap.h); the launcher passes only an
  // order the grid admits.
  const TileCoord tc = tile_of(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), tiles_m,
                               remap);
  const int tm = tc.tm, tn = tc.tn;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t g0 = n0 / kGroupRows;

  const int64_t rows_valid = (M - m0) < BM ? (M - m0) : BM;
  const int64_t groups_valid = (NG - g0) < (BN / kGroupRows) ? (NG - g0) : (BN / kGroupRows);
  Rsrc rs;
  rs.ra = make_rsrc(q_a + m0 * K, static_cast<uint32_t>(rows_valid * K));
  rs.rb = make_rsrc(wq + g0 * KB * kGroupBlockBytes,
                    static_cast<uint32_t>(groups_valid * KB * kGroupBlockBytes));
  rs.rsa = make_rsrc(d_a + m0 * KB, static_cast<uint32_t>(rows_valid * KB * 2));
  rs.rsb = make_rsrc(ws + g0 * KB * kGroupRows,
                     static_cast<uint32_t>(groups_valid * KB * kGroupRows * 2));
  rs.rnull = make_rsrc(q_a, 0);
  rs.KB = static_cast<int>(KB);
  LaneOffsets<T> lo;
  lane_offsets<T>(lo, tid, wave, lane, static_cast<uint32_t>(K), static_cast<uint32_t>(KB));

  const int kg = wave / T::kWavesT;              // K group
  const int wt = wave % T::kWavesT;              // wave within the group's tile
  const int wm0 = (wt % T::WAVES_M) * T::WM;
  const int wn0 = (wt / T::WAVES_M) * T::WN;
  const uint32_t kofs = static_cast<uint32_t>(kg * T::NB);   // group's first block in a stage
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // lane parts of the LDS addresses read by compute_stage
  // (32x32: lane l reads row/column l%32, half l/32; 16x16: row/column
  // l%16, bytes 8*(l/16) .. +8 of the block, i.e. half g/2, offset 8*(g%2))
  const int g = lane >> 4, l16 = lane & 15;
  const uint32_t lane_a = kofs * 2 * BM * 16 +
                          (T::MF == 32 ? (half * BM + wm0 + l32) * 16
                                       : ((g >> 1) * BM + wm0 + l16) * 16 + (g & 1) * 8);
  const uint32_t lane_as =
      T::kAq + T::kBq + kofs * BM * 4 + (wm0 + (T::MF == 32 ? 4 * half : 4 * g)) * 4;
  const uint32_t lane_b = T::kAq + kofs * 2 * BN * 16 +
                          (T::MF == 32 ? (half * BN + wn0 + l32) * 16
                                       : ((g >> 1) * BN + wn0 + l16) * 16 + (g & 1) * 8);
  const uint32_t lane_bs =
      T::kAq + T::kBq + T::kAs + kofs * BN * 8 + (wn0 + (T::MF == 32 ? l32 : l16)) * 8;
  const uint32_t lds_base = lds_addr(smem);
  // the wave's place among its workgroup's waves on its SIMD (wave w runs on
  // SIMD w % 4)
  const int prio_slot = __builtin_amdgcn_readfirstlane(wave >> 2);

  using acc_t = std::conditional_t<T::MF == 32, v16f, v4f>;
  using bias_t = std::conditional_t<T::MF == 32, v16i, v4i>;
  acc_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < T::kAccN; ++r) acc[i][j][r] = 0.0f;
  bias_t bias;
#pragma unroll
  for (int r = 0; r < T::kAccN; ++r) bias[r] = kBiasBits;

  // Pipeline over NBUF stage buffers.  Iteration s: compute stage s while
  // issuing the quant loads of stage s+NBUF-1, store the scales of stage s+1
  // (loaded one iteration earlier), load the scales of stage s+2, wait for
  // stage s+1's quant loads, barrier.  Every iteration issues the same
  // loads (stages past the end read zeros and touch no memory) so that
  // "stage s+1 has landed" is always "at most kInFlight younger loads
  // remain": loads complete in issue order.
  constexpr int NBUF = T::NBUF;
  const int nstages = static_cast<int>((KB + KBS - 1) / KBS);
  uint16_t as_r[T::kASc];
  uint32_t bs_r[T::kBSc];
  if constexpr (NBUF == 2) {
    // Stage 0's quants and scales and stage 1's scales, all in flight
    // together: stage 1's scales go to the loop's registers, so storing
    // stage 0's waits only for its own loads (one memory round trip for the
    // prologue instead of two).
    uint16_t as0[T::kASc];
    uint32_t bs0[T::kBSc];
    load_scales<T>(rs, lo, 0, as0, bs0);
    issue_quants<T, 0, T::kDmaOps>(rs, lo, wave, 0, smem);
    load_scales<T>(rs, lo, KBS, as_r, bs_r);
    store_scales<T>(tid, smem, as0, bs0);
  } else {
    for (int t = -(NBUF - 1); t < 0; ++t) {
      issue_quants<T, 0, T::kDmaOps>(rs, lo, wave, (t + NBUF - 1) * KBS,
                                     smem + ((t + NBUF - 1) % NBUF) * T::kStage);
      if (t == -1) store_scales<T>(tid, smem, as_r, bs_r);                  // stage 0
      if (t + 2 >= 0) load_scales<T>(rs, lo, (t + 2) * KBS, as_r, bs_r);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    // this stage's share of the loads of stage s+NBUF-1, issued block by block
    uint8_t* const next = smem + ((s + NBUF - 1) % NBUF) * T::kStage;
    const int kb_next = (s + NBUF - 1) * KBS;
    auto at_block = [&](auto kb_) __attribute__((always_inline)) {
      constexpr int kb = decltype(kb_)::value;
      issue_quants<T, kb * T::kDmaOps / T::NB, (kb + 1) * T::kDmaOps / T::NB>(rs, lo, wave,
                                                                             kb_next, next);
    };
    const uint32_t b = lds_base + (s % NBUF) * T::kStage;
    if constexpr (T::MF == 32)
      compute_stage<T>(b + lane_a, b + lane_as, b + lane_b, b + lane_bs, bias, acc, at_block,
                       prio_slot);
    else
      compute_stage16<T>(b + lane_a, b + lane_as, b + lane_b, b + lane_bs, bias, acc, at_block);
    store_scales<T>(tid, smem + ((s + 1) % NBUF) * T::kStage, as_r, bs_r);
    load_scales<T>(rs, lo, (s + 2) * KBS, as_r, bs_r);
    wait_vmcnt<T::kInFlight>();
    lds_wait_all();
    // A bare barrier: __syncthreads() would add a release fence, for which
    // the compiler waits on every outstanding load (the direct-to-LDS loads
    // count as LDS writes), draining the loads issued for later stages.
    // The waits above already cover what the next stage reads.
    asm volatile("s_barrier" ::: "memory");
  }
  if constexpr (T::kRotatePrio) set_wave_prio(0);
  wait_vmcnt<0>();   // the loads issued past the end are done before LDS is released
  if constexpr (T::KSPLIT > 1) {
    // Add the K groups' partial sums, in group order, into group 0's
    // registers ([slot][lane] floats: conflict-free LDS accesses).
    constexpr int kSlots = TM * TN * T::kAccN;
    float* const red = reinterpret_cast<float*>(smem);
    __syncthreads();   // every wave's loads into LDS have landed, and its reads are done
    if (kg > 0) {
      float* const dst = red + ((kg - 1) * T::kWavesT + wt) * kSlots * 64 + lane;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < T::kAccN; ++r) dst[((i * TN + j) * T::kAccN + r) * 64] = acc[i][j][r];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int gg = 1; gg < T::KSPLIT; ++gg) {
      const float* const src = red + ((gg - 1) * T::kWavesT + wt) * kSlots * 64 + lane;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < T::kAccN; ++r) acc[i][j][r] += src[((i * TN + j) * T::kAccN + r) * 64];
    }
  }
  {
    // The lane's position again, from the hardware lane count rather than
    // from values kept across the loop, whose registers it needs.
    const int lane_o = static_cast<int>(
        __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    const int half = lane_o >> 5, l32 = lane_o & 31, g = lane_o >> 4, l16 = lane_o & 15;

  if constexpr (kSwiglu) {
    // Each 64 columns of the wave are one row group: column 64p + l32 is the
    // gate of hidden unit 32*grp + l32 and column 64p + 32 + l32 its up, both
    // in this lane (j = 2p and 2p + 1).  The lane forms h = silu(g) * u for
    // its 16 rows of each group, and the wave passes the values through LDS
    // (the stage buffers, free now) so that one lane holds a whole Q8_0
    // block of h (32 hidden units of one row): it takes the block's maximum
    // and scale itself and writes its 32 codes with two 16-byte stores.
    static_assert(T::MF == 32 && T::TN % 2 == 0, "whole 64-column row groups per wave");
    constexpr int kGroups = TN / 2;
    constexpr int kBlocks = TM * 32 * kGroups;   // (row, group) blocks of the wave tile
    constexpr int kPitch = 36;                   // floats per block in LDS (32 + 4: banks)
    static_assert(T::kWavesT * kBlocks * kPitch * 4 <= T::NBUF * T::kStage, "LDS");
    float* const hb = reinterpret_cast<float*>(smem) + wt * kBlocks * kPitch;
    __syncthreads();   // every wave is done with the stage buffers, and its loads into them
#pragma unroll
    for (int pr = 0; pr < kGroups; ++pr)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rt = 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);   // row in the wave tile
          hb[(rt * kGroups + pr) * kPitch + l32] =
              silu_mul(acc[i][2 * pr][r], acc[i][2 * pr + 1][r]);
        }
    // the wave's own values, written by other lanes: its LDS accesses
    // complete in order, so a wave-level fence suffices
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int64_t I = N / 2;
    for (int bk = lane_o; bk < kBlocks; bk += 64) {
      const int rt = bk / kGroups, pr = bk % kGroups;
      const int64_t row = m0 + wm0 + rt;
      const int64_t grp = (n0 + wn0) / kGroupRows + pr;
      if (row >= M || grp * kGroupRows >= N) continue;
      float h[32];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const v4f v = *reinterpret_cast<const v4f*>(hb + bk * kPitch + 4 * c);
        h[4 * c] = v.x;
        h[4 * c + 1] = v.y;
        h[4 * c + 2] = v.z;
        h[4 * c + 3] = v.w;
      }
      float amax = fabsf(h[0]);
#pragma unroll
      for (int e = 1; e < 32; ++e) amax = fmaxf(amax, fabsf(h[e]));
      float id;
      uint16_t dbits;
      const bool nz = block_scale(amax, id, dbits);
      uint32_t w[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        w[c] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[c] |= (nz ? static_cast<uint32_t>(block_code(h[4 * c + e], id)) & 0xffu : 0u)
                  << (8 * e);
      }
      uint4* const qo = reinterpret_cast<uint4*>(q_h + row * I + grp * kQK);
      qo[0] = make_uint4(w[0], w[1], w[2], w[3]);
      qo[1] = make_uint4(w[4], w[5], w[6], w[7]);
      d_h[row * (I / kQK) + grp] = dbits;
    }
    return;
  }
  // Output.  32x32: lane holds column wn0 + 32j + l32 and rows
  // 8*(r/4) + 4*half + r%4; 16x16: column wn0 + 16j + l16, rows 4*g + r.
  // Through a buffer resource over the tile's valid rows when a whole
  // tile's offsets fit 31 bits: rows past M fall outside the range, and a
  // lane whose column is past N takes an offset of 2^31 and above, also
  // outside it, so the stores need no branches and one 32-bit add each.
  // The stores are marked non-temporal (C is not read again here), which
  // leaves more of the caches to the operand panels.
  if (int64_t(BM) * ldc * 4 <= (int64_t(1) << 31)) {
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(C + m0 * ldc, static_cast<uint32_t>(rows_valid * ldc * 4));
    const uint32_t ldc4 = static_cast<uint32_t>(ldc * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + wn0 + T::MF * j + (T::MF == 32 ? l32 : l16);
      const uint32_t row0 = static_cast<uint32_t>(wm0 + (T::MF == 32 ? 4 * half : 4 * g));
      const uint32_t lane_off =
          col < N ? row0 * ldc4 + static_cast<uint32_t>(col) * 4u : 0x80000000u;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < T::kAccN; ++r) {
          const uint32_t roff =
              static_cast<uint32_t>(T::MF * i + (T::MF == 32 ? 8 * (r >> 2) + (r & 3) : r)) * ldc4;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rc, lane_off + roff,
                                                0, kStoreNT);
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn0 + T::MF * j + (T::MF == 32 ? l32 : l16);
    if (col >= N) continue;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < T::kAccN; ++r) {
        const int64_t row = m0 + wm0 + T::MF * i +
                            (T::MF == 32 ? 8 * (r >> 2) + 4 * half + (r & 3) : 4 * g + r);
        if (row < M) C[row * ldc + col] = acc[i][j][r];
      }
  }
  }
}

// ---------------------------------------------------------------------------
// Small-M kernel (9 <= M <= 64): the decode kernel's weight stream, with the
// block dots on the matrix cores.
//
// Up to about 64 token rows the product is bound by the weight stream.  The
// tiled kernel's grid then has few workgroups, each staging operands
// through LDS a stage at a time, and keeps too little of the stream in
// flight.  Here, as in the decode kernel, a workgroup owns one packed
// 64-row group, its 8 waves split K, and each wave loads a chunk of L blocks
// at once, straight into registers:
//   - weights: the MFMA's B operand for rows 32j.. of the group is lane l:
//     row 32j + l%32, half l/32 of the block, i.e. two contiguous 512-byte
//     runs of the packed pieces: one 16-byte load per lane per 32 rows;
//   - activations: the A operand, lane l: row 32i + l%32, bytes 16*(l/32) ..
//     +16 of the block (rows past M read zero through the buffer range);
//   - scales: the lane's column's d_w (one value per 32-row tile), and the
//     chunk's d_a, which the wave stages as binary32 in an LDS slot of its
//     own and reads back with broadcast loads for its accumulator rows.
// One v_mfma_i32_32x32x32_i8 per 32x32 tile and block, the bias-fold
// epilogue of the tiled kernel, and the 8 waves' partial sums added in a
// fixed pairwise tree through LDS.  With quantised activations a wave
// issues the next chunk's weight loads before the current chunk's block
// dots (a second set of weight registers), so the stream stays in flight.
//
// X selects the activation input: 0, quantised rows q_a/d_a; 1 (binary32)
// or 2 (bfloat16), unquantised rows x that every wave quantises for its own
// chunk (quantize8, the code of the quantise kernel, four lanes per block),
// writing codes and binary32 scales into its slot where the quantised form
// would have been staged.  Codes and scales are therefore bit-identical to
// q8_quantize_act's, and C to quantising first; workgroup 0 also stores
// them to q_out/d_out when those are given.
// ---------------------------------------------------------------------------
constexpr int64_t kSmallMaxM = 64;

// Slot of row r in its group of four when d_a is stored rotated by one (see
// store_scales: keeps a row's scale and accumulator in different VGPR banks).
__device__ __forceinline__ int rot4(int r) { return (r & ~3) | ((r + 3) & 3); }

template <int MT, int L, int W, int X>
__global__ __launch_bounds__(W * 64) void gemm_q8_small_kernel(
    const int8_t* __restrict__ q_a, const uint16_t* __restrict__ d_a,
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ ws, float* __restrict__ C,
    int64_t M, int64_t N, int64_t K, int64_t KB, int64_t ldc, int kb_per_wave,
    const void* __restrict__ x, int64_t ldx, int8_t* __restrict__ q_out,
    uint16_t* __restrict__ d_out) {
#if __HIP_DEVICE_COMPILE__
  // Per-wave LDS slot: the chunk's activation rows [MT*32][L*32 bytes + 16
  // pad] (the pad spreads a column read over the banks), then its d_a as
  // binary32 [MT][L][32].  After the loop the space holds the partial sums
  // of the upper half of the waves ([W/2][MT][2][16][64] floats).
  constexpr int kRow = L * kQK + 16;
  constexpr int kAct = MT * 32 * kRow;
  constexpr int kSlot = kAct + MT * L * 32 * 4;
  constexpr int kRed = W / 2 * MT * 2 * 16 * 64 * 4;
  constexpr int kSegs = MT * 32 * 2 * L;          // 16-byte activation pieces per chunk
  constexpr int kScs = MT * 32 * L;               // activation scales per chunk
  static_assert(kSegs % 64 == 0 && kScs % 64 == 0, "whole wave loads");
  __shared__ __align__(16) uint8_t lds[kRed > W * kSlot ? kRed : W * kSlot];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t g = blockIdx.x;
  const int kb0 = wave * kb_per_wave;
  const int kb1 = kb0 + kb_per_wave < KB ? kb0 + kb_per_wave : static_cast<int>(KB);

  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wq + g * KB * kGroupBlockBytes,
                                              static_cast<uint32_t>(KB * kGroupBlockBytes));
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(ws + g * KB * kGroupRows,
                                               static_cast<uint32_t>(KB * kGroupRows * 2));
  // activation rows: quantised (X == 0) or raw (X != 0; rows past M, and
  // blocks past the wave's range, read as zero through the range check)
  constexpr int kEsz = X == 1 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t ra =
      X == 0 ? make_rsrc(q_a, static_cast<uint32_t>(M * K))
             : make_rsrc(x, static_cast<uint32_t>(M * ldx * kEsz));
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(d_a, static_cast<uint32_t>(X == 0 ? M * KB * 2 : 0));
  const bool store_q = X != 0 && q_out != nullptr && blockIdx.x == 0;
  const uint32_t ow = static_cast<uint32_t>(half * kPieceBytes + l32 * 16);   // + 512 * j
  const uint32_t ows = static_cast<uint32_t>(l32 * 2);                        // + 64 * j
  uint8_t* const slot = lds + wave * kSlot;
  float* const sslot = reinterpret_cast<float*>(slot + kAct);

  v16f acc[MT][2];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  v16i bias;
#pragma unroll
  for (int r = 0; r < 16; ++r) bias[r] = kBiasBits;

  // The weights of a chunk: one 16-byte piece and one scale per lane, block
  // and 32-row tile.  Blocks past the wave's range read as zero through the
  // buffer range check (no memory access); their terms are dropped below.
  auto load_weights = [&](int cc, v4i(&wv)[L][2], uint16_t(&wsc)[L][2]) {
#pragma unroll
    for (int b = 0; b < L; ++b) {
      const bool in = cc + b < kb1;
      const uint32_t kb = static_cast<uint32_t>(cc + b);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        wv[b][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rw, in ? ow + j * 512 + kb * kGroupBlockBytes : kOutOfRange, 0, 0);
        wsc[b][j] = __builtin_amdgcn_raw_buffer_load_b16(
            rws, in ? ows + j * 64 + kb * kGroupRows * 2 : kOutOfRange, 0, 0);
      }
    }
  };
  // A chunk's block dots and epilogue, from its weights and the slot.
  auto compute = [&](int c, const v4i(&wv)[L][2], const uint16_t(&wsc)[L][2]) {
#pragma unroll
    for (int b = 0; b < L; ++b) {
      const float live = c + b < kb1 ? 1.0f : 0.0f;
      v2f wp[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float w = f16_bits_to_f32(wsc[b][j]) * live;
        wp[j] = v2f{w, -kBias * w};
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        // A operand: row 32i + l32, bytes 16*half of block b; d_a of the
        // lane's rows 8*(r/4) + 4*half + r%4 of tile i
        const v4i av = *reinterpret_cast<const v4i*>(slot + (32 * i + l32) * kRow + b * kQK +
                                                     16 * half);
        v4f da[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          da[q] = *reinterpret_cast<const v4f*>(sslot + (i * L + b) * 32 + 8 * q + 4 * half);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, wv[b][j], bias, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float y = fmaf(__int_as_float(p[r]), wp[j].x, wp[j].y);
            acc[i][j][r] = fmaf(y, da[r >> 2][(r + 3) & 3], acc[i][j][r]);   // rot4 groups
          }
        }
      }
      // one block at a time: hoisting later blocks' MFMAs needs a result
      // tile of registers each
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (X == 0) {
    // Software pipeline: each chunk issues its activation loads, then the
    // next chunk's weight loads, then waits for the activations only (loads
    // complete in order), so the weight stream stays in flight through the
    // chunk's arithmetic.
    v4i wv[L][2];
    uint16_t wsc[L][2];
    load_weights(kb0, wv, wsc);
#pragma nounroll
    for (int c = kb0; c < kb1; c += L) {
      v4i xv[kSegs / 64];
      uint16_t xs[kScs / 64];
      // Activations: piece u*64 + lane is row s / (2L), 16 bytes s % (2L)
      // of the chunk (16 consecutive lanes read 256 contiguous bytes of a
      // row; rows past M, or bytes past the last block, read zero or are
      // unused).
#pragma unroll
      for (int u = 0; u < kSegs / 64; ++u) {
        const int sg = u * 64 + lane, row = sg / (2 * L), seg = sg % (2 * L);
        xv[u] = __builtin_amdgcn_raw_buffer_load_b128(
            ra, static_cast<uint32_t>(row * K + c * kQK + seg * 16), 0, 0);
      }
      // Activation scales: item u*64 + lane is row s / L, block s % L.
#pragma unroll
      for (int u = 0; u < kScs / 64; ++u) {
        const int sc = u * 64 + lane, row = sc / L, b = sc % L;
        xs[u] = __builtin_amdgcn_raw_buffer_load_b16(
            rsa, c + b < kb1 ? static_cast<uint32_t>((row * KB + c + b) * 2) : kOutOfRange, 0,
            0);
      }
      v4i wn[L][2];
      uint16_t wsn[L][2];
      load_weights(c + L, wn, wsn);
      // into the slot (this wave's alone; no barrier)
#pragma unroll
      for (int u = 0; u < kSegs / 64; ++u) {
        const int sg = u * 64 + lane, row = sg / (2 * L), seg = sg % (2 * L);
        *reinterpret_cast<v4i*>(slot + row * kRow + seg * 16) = xv[u];
      }
#pragma unroll
      for (int u = 0; u < kScs / 64; ++u) {
        const int sc = u * 64 + lane, row = sc / L, b = sc % L;
        sslot[((row >> 5) * L + b) * 32 + rot4(row & 31)] = f16_bits_to_f32(xs[u]);
      }
      compute(c, wv, wsc);
#pragma unroll
      for (int b = 0; b < L; ++b)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          wv[b][j] = wn[b][j];
          wsc[b][j] = wsn[b][j];
        }
    }
  } else {
    for (int c = kb0; c < kb1; c += L) {
      v4i wv[L][2];
      uint16_t wsc[L][2];
      // Raw activations (X != 0): item t = u*64 + lane is row t / (4L), block
      // (t / 4) % L, values 8*(t % 4) .. +8 of it, so four lanes hold a block
      // and 4L consecutive lanes a contiguous run of a row.  The first batch of
      // items is loaded before the weights, the rest after.
      constexpr int kItems = MT * 32 * L * 4;
      constexpr int kPB = X == 1 ? 4 : 8;   // items per lane per batch: 32 registers
      constexpr int kBatches = X == 0 ? 1 : kItems / 64 / kPB;
      static_assert(X == 0 || kItems % (64 * kPB) == 0, "whole batches");
      v4i raw[kPB][kEsz / 2];
      auto load_batch = [&](int bt) {
#pragma unroll
        for (int e = 0; e < kPB; ++e) {
          const int t = (bt * kPB + e) * 64 + lane;
          const int row = t / (4 * L), b = (t / 4) % L, sub = t % 4;
          const uint32_t off =
              c + b < kb1 ? static_cast<uint32_t>((row * ldx + (c + b) * kQK + sub * 8) * kEsz)
                          : kOutOfRange;
#pragma unroll
          for (int h = 0; h < kEsz / 2; ++h)
            raw[e][h] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, off == kOutOfRange ? kOutOfRange : off + 16 * h, 0, 0);
        }
      };
      auto quantize_batch = [&](int bt) {
#pragma unroll
        for (int e = 0; e < kPB; ++e) {
          const int t = (bt * kPB + e) * 64 + lane;
          const int row = t / (4 * L), b = (t / 4) % L, sub = t % 4;
          float v[8];
          if constexpr (X == 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int q = 0; q < 4; ++q) v[4 * h + q] = __int_as_float(raw[e][h][q]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t w = static_cast<uint32_t>(raw[e][0][q]);
              v[2 * q] = __uint_as_float(w << 16);
              v[2 * q + 1] = __uint_as_float(w & 0xffff0000u);
            }
          }
          uint32_t lo, hi;
          uint16_t dbits;
          quantize8(v, lo, hi, dbits);   // all lanes take part (lane exchanges)
          *reinterpret_cast<uint2*>(slot + row * kRow + b * kQK + sub * 8) = make_uint2(lo, hi);
          if (sub == 0) sslot[((row >> 5) * L + b) * 32 + rot4(row & 31)] = f16_bits_to_f32(dbits);
          if (store_q && row < M && c + b < kb1) {
            *reinterpret_cast<uint2*>(q_out + row * K + (c + b) * kQK + sub * 8) =
                make_uint2(lo, hi);
            if (sub == 0) d_out[row * KB + c + b] = dbits;
          }
        }
      };
      load_batch(0);   // row 0 < M: always live
      load_weights(c, wv, wsc);
      // into the slot (this wave's alone; a wave's LDS accesses complete in
      // order, so no barrier).  Batches whose rows are all past M are
      // skipped: those slot rows only feed outputs that are not stored.
      constexpr int kRowsPerBatch = kPB * 64 / (4 * L);
#pragma nounroll
      for (int bt = 0; bt < kBatches && bt * kRowsPerBatch < M; ++bt) {
        if (bt > 0) load_batch(bt);
        quantize_batch(bt);
      }
      compute(c, wv, wsc);
    }
  }

  // waves' sums in a fixed tree: wave w + W/2 into w, then w + W/4, ..., 1
  float* const red = reinterpret_cast<float*>(lds);
  __syncthreads();   // every wave is done with its slot
#pragma unroll
  for (int span = W / 2; span >= 1; span >>= 1) {
    if (wave >= span && wave < 2 * span) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[((((wave - span) * MT + i) * 2 + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (wave < span) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[i][j][r] += red[(((wave * MT + i) * 2 + j) * 16 + r) * 64 + lane];
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = g * kGroupRows + 32 * j + l32;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
          if (m < M) C[m * ldc + n] = acc[i][j][r];
        }
    }
  }
#endif
}

// 8 waves (two per SIMD: up to 256 registers), chunks of 4 blocks.  16 waves
// would cap a wave at 128 registers, below what a chunk needs without
// spilling (149 at one 32-row activation tile, 191 at two).
template <int MT, int X>
hipError_t launch_small(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                        const void* x, int64_t ldx, int8_t* q_out, uint16_t* d_out,
                        const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  constexpr int W = 8;
  constexpr int L = 4;   // (8 at one tile measured 5-6 % slower, 2 at two tiles 2-10 %)
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  const int kb_per_wave = static_cast<int>((KB + W - 1) / W);
  hipLaunchKernelGGL((gemm_q8_small_kernel<MT, L, W, X>), dim3(static_cast<uint32_t>(NG)),
                     dim3(W * 64), 0, stream, q_a, d_a, w_packed, ws, C, M, N, K, KB, ldc,
                     kb_per_wave, x, ldx, q_out, d_out);
  return hipGetLastError();
}

// Workgroup order for a tile grid (q8_tilemap.h).  Q8_GEMM_REMAP=<order>
// overrides the choice only with an order the grid admits; anything else is
// ignored (and reported under Q8_LOG).
int workgroup_order(int64_t tiles_m, int64_t tiles_n, int64_t bm, int64_t K) {
  const int order = choose_order(tiles_m, tiles_n, bm, K);
  const int forced = env_index("Q8_GEMM_REMAP");
  if (forced < 0) return order;
  if (order_admissible(forced, tiles_m, tiles_n)) return forced;
  if (log_enabled())
    fprintf(stderr, "q8: Q8_GEMM_REMAP=%d not admissible for a %lldx%lld tile grid; order %d\n",
            forced, static_cast<long long>(tiles_m), static_cast<long long>(tiles_n), order);
  return order;
}

template <class T, int kOcc, bool kSwiglu>
hipError_t launch_tile_impl(int64_t M, int64_t N, int64_t K, const int8_t* q_a,
                            const uint16_t* d_a, const uint8_t* w_packed, float* C, int64_t ldc,
                            hipStream_t stream, int8_t* q_h, uint16_t* d_h) {
  const int64_t KB = K / kQK;
  const int64_t NG = num_groups(N);
  const uint16_t* ws = reinterpret_cast<const uint16_t*>(w_packed + NG * KB * kGroupBlockBytes);
  const int64_t tiles_m = (M + T::BM - 1) / T::BM;
  const int64_t tiles_n = (N + T::BN - 1) / T::BN;
  const int64_t grid = tiles_m * tiles_n;
  const int remap = workgroup_order(tiles_m, tiles_n, T::BM, K);
  hipLaunchKernelGGL((gemm_q8_mfma_kernel<T, kOcc, kSwiglu>), dim3(static_cast<uint32_t>(grid)),
                     dim3(T::kThreads), 0, stream, q_a, d_a, w_packed, ws, C, M, N, K, KB, NG,
                     ldc, static_cast<int>(tiles_m), remap, q_h, d_h);
  return hipGetLastError();
}

template <class T, int kOcc>
hipError_t launch_tile(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  return launch_tile_impl<T, kOcc, false>(M, N, K, q_a, d_a, w_packed, C, ldc, stream, nullptr,
                                          nullptr);
}

typedef hipError_t (*launcher_t)(int64_t, int64_t, int64_t, const int8_t*, const uint16_t*,
                                 const uint8_t*, float*, int64_t, hipStream_t);

struct TileConfig {
  int bm, bn;
  launcher_t launch;
};

// Compiled tile configurations (index = the one in q8_tilemap.h's
// kTileDims).  Occupancy hint = waves per SIMD the register allocation must
// allow.
using Tile0 = Tile<128, 128, 4, 2, 4, 2>;                    // 8 waves 32x64, KBS 4
using Tile1 = Tile<64, 128, 2, 2, 2, 2>;                     // 4 waves 32x64, KBS 2
using Tile2 = Tile<128, 128, 4, 2, 4, 2, 16>;                // as 0 on 16x16 MFMAs
using Tile3 = Tile<128, 256, 4, 4, 4, 2>;                    // 16 waves 32x64
using Tile4 = Tile<128, 128, 4, 2, 4, 2, 32, 1>;             // as 0, MFMAs first
using Tile5 = Tile<64, 64, 2, 1, 8, 2, 32, 0, 4>;            // 4 K groups of 2 waves
using Tile6 = Tile<64, 128, 2, 2, 8, 2, 32, 1, 2>;           // 2 K groups of 4 waves, MFMAs first (LDS: one per CU)
using Tile7 = Tile<64, 128, 2, 2, 4, 2, 32, 0, 2>;           // 2 K groups of 4 waves, stages of 4
using Tile8 = Tile<64, 192, 2, 3, 6, 2, 32, 1, 2>;           // 2 K groups of 6 waves, MFMAs first
using Tile9 = Tile<128, 384, 4, 3, 3, 2, 32, 0, 1>;          // 12 waves 32x128, KBS 3

template <class T>
constexpr bool dims_match(int i) {
  return T::BM == kTileDims[i].bm && T::BN == kTileDims[i].bn;
}
static_assert(dims_match<Tile0>(0) && dims_match<Tile1>(1) && dims_match<Tile2>(2) &&
                  dims_match<Tile3>(3) && dims_match<Tile4>(4) && dims_match<Tile5>(5) &&
                  dims_match<Tile6>(6) && dims_match<Tile7>(7) && dims_match<Tile8>(8) &&
                  dims_match<Tile9>(9),
              "tile table and q8_tilemap.h agree");

const TileConfig kTiles[] = {
    {128, 128, launch_tile<Tile0, 4>}, {64, 128, launch_tile<Tile1, 4>},
    {128, 128, launch_tile<Tile2, 4>}, {128, 256, launch_tile<Tile3, 4>},
    {128, 128, launch_tile<Tile4, 4>}, {64, 64, launch_tile<Tile5, 4>},
    {64, 128, launch_tile<Tile6, 2>},  {64, 128, launch_tile<Tile7, 4>},
    {64, 192, launch_tile<Tile8, 3>},  {128, 384, launch_tile<Tile9, 3>},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
static_assert(kNumTiles == kNumTileDims, "tile table and q8_tilemap.h agree");

bool tile_fits(int t, int64_t K) { return buffer_ranges_fit(kTiles[t].bm, kTiles[t].bn, K); }

int pick_tile(int64_t M, int64_t N, int64_t K) {
  // Q8_GEMM_TILE=<index> forces a configuration (benchmarking aid), if it
  // exists and its buffer ranges hold K.
  const int forced = env_index("Q8_GEMM_TILE");
  if (forced >= 0 && forced < kNumTiles && tile_fits(forced, K)) return forced;
  if (forced >= 0 && log_enabled())
    fprintf(stderr, "q8: Q8_GEMM_TILE=%d ignored (no such tile, or K=%lld too large for it)\n",
            forced, static_cast<long long>(K));
  // The automatic choice (q8_tilemap.h): by the grid's size and shape, and
  // only among configurations whose buffer ranges hold K.
  return choose_tile(M, N, K);
}

}  // namespace

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const int8_t* q_a, const uint16_t* d_a,
                       const uint8_t* w_packed, float* C, int64_t ldc, hipStream_t stream) {
  // 9 <= M <= 64: the weight-streaming kernel, unless a tile is forced
  if (M <= kSmallMaxM && env_index("Q8_GEMM_TILE") < 0) {
    if (log_enabled())
      fprintf(stderr, "q8: product M=%lld N=%lld K=%lld: small-M matrix-core kernel, %lld row tiles\n",
              static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
              static_cast<long long>((M + 31) / 32));
    return M <= 32 ? launch_small<1, 0>(M, N, K, q_a, d_a, nullptr, 0, nullptr, nullptr,
                                        w_packed, C, ldc, stream)
                   : launch_small<2, 0>(M, N, K, q_a, d_a, nullptr, 0, nullptr, nullptr,
                                        w_packed, C, ldc, stream);
  }
  const int t = pick_tile(M, N, K);
  if (log_enabled())
    fprintf(stderr, "q8: product M=%lld N=%lld K=%lld: matrix-core kernel, tile %d (%dx%d)\n",
            static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K), t,
            kTiles[t].bm, kTiles[t].bn);
  return kTiles[t].launch(M, N, K, q_a, d_a, w_packed, C, ldc, stream);
}

// Opt-in (Q8_GEMM_ACT_FUSED=1): at the decode layer's N12288 K4096 every one
// of the 192 workgroups re-quantises all M rows, and with the quantise loads
// in the weight stream's critical path the fused kernel measured slower than
// quantising first (bf16, graph replay: M9 20.9 vs 19.8 us, M32 31.6 vs
// 21.4, M64 54.0 vs 27.4).
bool small_act_applies(int64_t M, int dtype, int64_t ldx) {
  if (M > kSmallMaxM || env_index("Q8_GEMM_TILE") >= 0 || env_index("Q8_GEMM_ACT_FUSED") != 1)
    return false;
  // the raw rows' 32-bit buffer range covers every 32-row tile's rows
  const int64_t rows = (M + 31) / 32 * 32;
  return rows * ldx * (dtype == 0 ? 4 : 2) < (int64_t(1) << 32);
}

hipError_t launch_small_act(int64_t M, const void* x, int dtype, int64_t ldx, int64_t N,
                            int64_t K, const uint8_t* w_packed, float* C, int64_t ldc,
                            int8_t* q_out, uint16_t* d_out, hipStream_t stream) {
  if (log_enabled())
    fprintf(stderr,
            "q8: product M=%lld N=%lld K=%lld: small-M matrix-core kernel quantising its rows, "
            "%lld row tiles\n",
            static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K),
            static_cast<long long>((M + 31) / 32));
  if (dtype == 0)
    return M <= 32 ? launch_small<1, 1>(M, N, K, nullptr, nullptr, x, ldx, q_out, d_out,
                                        w_packed, C, ldc, stream)
                   : launch_small<2, 1>(M, N, K, nullptr, nullptr, x, ldx, q_out, d_out,
                                        w_packed, C, ldc, stream);
  return M <= 32 ? launch_small<1, 2>(M, N, K, nullptr, nullptr, x, ldx, q_out, d_out, w_packed,
                                      C, ldc, stream)
                 : launch_small<2, 2>(M, N, K, nullptr, nullptr, x, ldx, q_out, d_out, w_packed,
                                      C, ldc, stream);
}

hipError_t launch_gemm_swiglu(int64_t M, int64_t I, int64_t K, const int8_t* q_a,
                              const uint16_t* d_a, const uint8_t* w_packed, int8_t* q_h,
                              uint16_t* d_h, hipStream_t stream) {
  // The 32x32-MFMA tiles (all but 2) carry the epilogue: their wave tiles
  // are whole 64-column row groups; the 16x16 variant (2) is replaced by
  // tile 0.
  const int64_t N = 2 * I;
  const int t = pick_tile(M, N, K);
  if (log_enabled())
    fprintf(stderr, "q8: gated step M=%lld I=%lld K=%lld: matrix-core kernel, tile %d\n",
            static_cast<long long>(M), static_cast<long long>(I), static_cast<long long>(K), t);
  const auto go = [&](auto launch) { return launch(M, N, K, q_a, d_a, w_packed, nullptr, N,
                                                   stream, q_h, d_h); };
  switch (t) {
    case 1: return go(launch_tile_impl<Tile1, 4, true>);
    case 3: return go(launch_tile_impl<Tile3, 4, true>);
    case 5: return go(launch_tile_impl<Tile5, 4, true>);
    case 6: return go(launch_tile_impl<Tile6, 2, true>);
    case 7: return go(launch_tile_impl<Tile7, 4, true>);
    case 8: return go(launch_tile_impl<Tile8, 3, true>);
    case 9: return go(launch_tile_impl<Tile9, 3, true>);
    case 0:
    case 2: return go(launch_tile_impl<Tile0, 4, true>);
    default: return go(launch_tile_impl<Tile4, 4, true>);
  }
}

}  // namespace q8
