/*
 * q8.h -- C ABI of libq8gemm: the Q8_0 weight x activation product on
 * AMD Instinct MI355X (gfx950).
 *
 * Source of the operation.  news.hada.io topic 29953, "CUDA inference engine
 * for running Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)":
 * its list of paths that avoid the throttled units does the model's GEMMs
 * with a self-written int8 DP4A kernel, and its benchmark and limitations
 * lists name Q8_0 GGUF as the one supported weight format.  Q8_0 stores 32
 * consecutive values along K as int8 q[32] plus one IEEE binary16 scale d
 * (value = d*q).  Activations are quantised on the fly into the same block
 * format, so each output is
 *
 *     C[m][n] = sum_kb  d_a[m][kb] * d_w[n][kb] * int32( sum_{j<32} q_a[m][32kb+j] * q_w[n][32kb+j] )
 *
 * i.e. C = A * W^T with A = tokens x K and W = output features x K.
 *
 * Conventions for every call:
 *   - all data pointers are DEVICE pointers of the current HIP device;
 *   - work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream); calls return at once, never synchronise, never
 *     allocate, and keep no state beyond a one-time per-device check (and,
 *     for q8_gemm_act_noalloc, its per-device workspace address);
 *   - arguments are validated on the host before any HIP call; a failed
 *     check returns its status and enqueues nothing;
 *   - the caller owns every buffer; outputs are overwritten, never read;
 *   - faults during execution surface at the caller's next synchronisation,
 *     as for any HIP kernel.
 *   - input/output buffers must not overlap.
 *
 * Environment: Q8_LOG set (and not "0") makes the product calls print their
 * dispatch decision (decode or matrix-core kernel and its configuration) to
 * stderr, one line per call.  Q8_GEMM_TILE=<i> and Q8_GEMV_CFG=<c> force a
 * compiled configuration of the matrix-core or decode kernel (benchmarking
 * and tests); every configuration computes the same product.  A forced
 * matrix-core configuration whose 32-bit buffer ranges cannot hold K
 * (tile rows or columns times K >= 2^32) is ignored.  Q8_GEMM_REMAP=<o>
 * forces the matrix-core kernel's workgroup order: 0 (tile order), 1 (a
 * contiguous range of tiles per XCD; only when the tile count is a
 * multiple of 8), or 2, 4, 8 (the tile grid cut into o x 8/o rectangles,
 * one per XCD; only when the tile rows divide by o and the tile columns by
 * 8/o).  Any other value, or one the grid does not admit, is ignored (the
 * automatic choice is kept).  Q8_GEMM_ACT_FUSED=1 makes q8_gemm_act with
 * 9 <= M <= 64 run a single kernel that quantises the rows as it streams the
 * weights (the same codes, scales and C bit for bit; measured slower than
 * the default two kernels at N12288 K4096, since every workgroup
 * re-quantises all M rows).  Values that are not plain decimal numbers are
 * ignored by all four.
 *
 * Domain: finite inputs whose block maxima stay below 65504*127 (larger
 * scales overflow binary16).  NaN and infinity are outside the domain.
 */
#ifndef Q8_H
#define Q8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Under C++ both enumerations have int as their fixed underlying type, so
 * that any int a C caller passes is a value of the type: an unknown dtype is
 * then rejected by the checks below (Q8_ERR_DTYPE), never undefined.  The
 * layout is an int either way. */
#ifdef __cplusplus
#define Q8_ENUM_BASE : int
#else
#define Q8_ENUM_BASE
#endif

typedef enum q8_status_e Q8_ENUM_BASE {
    Q8_OK = 0,
    Q8_ERR_NULL = 1,    /* a required pointer is NULL                        */
    Q8_ERR_SHAPE = 2,   /* K < 32, K % 32 != 0, K > 2^24, N <= 0, M < 0,
                           ldx < K, ldc < N, or a grid too large to launch  */
    Q8_ERR_ALIGN = 3,   /* a pointer or a row pitch breaks the stated alignment */
    Q8_ERR_DTYPE = 4,   /* unknown q8_dtype                                  */
    Q8_ERR_SIZE = 5,    /* *packed_bytes smaller than the packed layout, or
                           (q8_gemm_act_noalloc) quantised rows larger than
                           its static workspace                              */
    Q8_ERR_DEVICE = 6,  /* the current device is not gfx950, or no device    */
    Q8_ERR_LAUNCH = 7   /* the kernel launch was rejected by the runtime     */
} q8_status;

typedef enum q8_dtype_e Q8_ENUM_BASE {
    Q8_F32 = 0,         /* IEEE binary32                                     */
    Q8_BF16 = 1         /* bfloat16 (upper half of a binary32)               */
} q8_dtype;

/*
 * q8_pack_weights -- repack Q8_0 weight rows into the layout q8_gemm reads.
 *
 * Operation: a byte permutation of the GGUF Q8_0 blocks (the format the
 * source names, see above); no arithmetic.  Done once when weights load.
 *
 * w_blocks  [N][K/32] blocks of 34 bytes: binary16 d (little-endian), then
 *           int8 q[32]; block (n, kb) at byte (n*(K/32) + kb)*34.  Any
 *           alignment.
 * N, K      output features and reduction length; N >= 1, 32 <= K <= 2^24,
 *           K % 32 == 0.
 * w_packed  device buffer, 16-byte aligned, or NULL to query the size.
 * packed_bytes  in: capacity of w_packed; out (when w_packed is NULL): the
 *           required size, NG*KB*2176 with NG = ceil(N/64), KB = K/32
 *           (= 1.0625*N*K bytes when N % 64 == 0).
 *
 * Packed layout (row groups of 64 output features):
 *   quant plane, NG*KB*2048 bytes: byte ((g*KB + kb)*2 + h)*1024 + r*16 + t
 *     holds q[64g + r][32kb + 16h + t]   (h in {0,1}, r < 64, t < 16),
 *   scale plane, right after it, NG*KB*64 binary16 values: element
 *     (g*KB + kb)*64 + r holds d[64g + r][kb].
 *   Rows 64g + r >= N are zero.  Each 1 KB piece (g, kb, h) is what one
 *   64-lane wave loads with one 16-byte load per lane.
 *
 * Errors: Q8_ERR_NULL (packed_bytes NULL, or w_blocks NULL when packing),
 * Q8_ERR_SHAPE, Q8_ERR_ALIGN (w_packed), Q8_ERR_SIZE, Q8_ERR_DEVICE,
 * Q8_ERR_LAUNCH.
 */
q8_status q8_pack_weights(const void *w_blocks, int64_t N, int64_t K,
                          void *w_packed, size_t *packed_bytes, void *stream);

/*
 * q8_quantize_act -- quantise activation rows to Q8_0 blocks.
 *
 * Operation, per block of 32 values x[0..31] (bfloat16 is widened exactly):
 *   amax = max |x_j|;  d32 = amax / 127  (binary32, correctly rounded);
 *   if d32 < FLT_MIN (all-zero and denormal-scale blocks): q = 0, d = +0;
 *   else id = 1 / d32 (correctly rounded), q_j = x_j * id rounded half
 *   away from zero, d = binary16(d32) rounded to nearest even.
 *   (The Q8_0 quantiser; see the source note at the top.)
 *
 * x     [M][ldx] binary32 or bfloat16 (dtype); 16-byte aligned and
 *       ldx*sizeof(elem) % 16 == 0.  Only the first K columns are read.
 * M     rows (M == 0: nothing is enqueued); 32 <= K <= 2^24, K % 32 == 0;
 *       ldx >= K.
 * q     [M][K] int8 out, 16-byte aligned.
 * d     [M][K/32] binary16 bits out, 2-byte aligned.
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DTYPE,
 * Q8_ERR_DEVICE, Q8_ERR_LAUNCH.
 */
q8_status q8_quantize_act(const void *x, q8_dtype dtype, int64_t M, int64_t K,
                          int64_t ldx, int8_t *q, uint16_t *d, void *stream);

/*
 * q8_gemm -- C = A * W^T on Q8_0 operands (the formula at the top).
 *
 * q_a   [M][K] int8 and d_a [M][K/32] binary16 bits, as written by
 *       q8_quantize_act; q_a 16-byte aligned, d_a 2-byte aligned.
 * w_packed  the output of q8_pack_weights for the same N and K.
 * C     [M][ldc] binary32 out, ldc >= N, 4-byte aligned; overwritten.
 * M     M == 0 enqueues nothing.  M <= 8 runs the bandwidth-bound
 *       decode kernel, larger M the int8 matrix-core kernel; both give
 *       the same value within the bound below.
 *
 * Accuracy: every block's int32 dot is exact; each block term is scaled
 * and accumulated in binary32, so |C - C_exact| <= (K/32 + 2) * 2^-24 *
 * sum_kb |d_a d_w| sum_j |q_a q_w|.  Results are bitwise reproducible from
 * run to run for the same inputs and shape.
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DEVICE,
 * Q8_ERR_LAUNCH.
 */
q8_status q8_gemm(int64_t M, int64_t N, int64_t K,
                  const int8_t *q_a, const uint16_t *d_a, const void *w_packed,
                  float *C, int64_t ldc, void *stream);

/*
 * q8_gemm_act -- quantise activation rows and multiply: C = A * W^T with A
 * quantised on the fly (q8_quantize_act followed by q8_gemm, in one call).
 *
 * Operation: exactly that of q8_quantize_act on x, then q8_gemm on its
 * output.  For M <= 8 (decode) one kernel does both: every workgroup
 * quantises the activation blocks it needs as it streams the weights, so
 * the quantised rows never go through memory; C, and q_a/d_a when given,
 * are bit-identical to the two separate calls.  For M > 8 the two kernels
 * run one after the other on the stream, through q_a/d_a (for M <= 64 with
 * Q8_GEMM_ACT_FUSED=1, one kernel that also writes q_a/d_a; see above).  (The source
 * engine quantises activations on the fly for its int8 GEMM; see the note
 * at the top.)
 *
 * x, dtype, ldx  as for q8_quantize_act (16-byte aligned, ldx*elem % 16 == 0).
 * w_packed, N, C, ldc  as for q8_gemm.
 * q_a, d_a  [M][K] int8 and [M][K/32] binary16 outputs: both NULL or both
 *       set (16-byte and 2-byte aligned).  Optional for M <= 8 (not written
 *       when NULL); required for M > 8, where they hold the quantised rows
 *       between the two kernels.
 *
 * Errors: Q8_ERR_NULL (x, w_packed or C NULL; only one of q_a/d_a; q_a NULL
 * with M > 8), Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DTYPE, Q8_ERR_DEVICE,
 * Q8_ERR_LAUNCH.
 */
q8_status q8_gemm_act(const void *x, q8_dtype dtype, int64_t M, int64_t N, int64_t K,
                      int64_t ldx, const void *w_packed, float *C, int64_t ldc,
                      int8_t *q_a, uint16_t *d_a, void *stream);

/*
 * q8_gemm_act_noalloc -- q8_gemm_act for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same operation and the same
 * kernels, with the quantised rows kept in a workspace the library holds
 * instead of caller buffers.
 *
 * x, dtype, M, N, K, ldx, w_packed, C, ldc, stream  as for q8_gemm_act.
 *
 * C is bit-identical to q8_gemm_act's for the same inputs.  For M <= 8 no
 * workspace is used (one fused kernel).  For M > 8 the rows' codes and
 * scales, M*K + 2*M*K/32 bytes (the scales at a 256-byte boundary after the
 * codes), go through a 48 MiB static device array: one per GPU, held by the
 * library until the process ends, looked up once per device on the first
 * call that needs it.  Every call on a GPU shares that array, so calls that
 * may overlap on one GPU (on different streams or from different threads)
 * race and must be ordered by the caller.  Nothing is allocated, nothing
 * is synchronised.
 *
 * Errors: as q8_gemm_act (no Q8_ERR_NULL for q_a/d_a, which it has not),
 * plus Q8_ERR_SIZE when M > 8 and the rows exceed the workspace (e.g. M =
 * 8192 at K = 5120 fits, M = 8192 at K = 17408 does not), and
 * Q8_ERR_DEVICE if the workspace's address cannot be obtained.
 */
q8_status q8_gemm_act_noalloc(const void *x, q8_dtype dtype, int64_t M, int64_t N, int64_t K,
                              int64_t ldx, const void *w_packed, float *C, int64_t ldc,
                              void *stream);

/*
 * q8_pack_weights_gateup -- pack the gate and up weights of a gated
 * feed-forward layer together, for q8_gemm_swiglu.
 *
 * Operation: a byte permutation, as q8_pack_weights, of the 2I rows
 * obtained by interleaving the two weights by 32-row blocks: packed row
 * 64g + r is gate row 32g + r for r < 32 and up row 32g + r - 32 for
 * r >= 32.  The result is the packed layout (see q8_pack_weights) of that
 * 2I x K matrix, so the gate and the up rows of a hidden unit share a row
 * group.  (The step after the product in the source engine's Qwen3.5/3.6
 * layers: their feed-forward blocks are gated; see the note at the top.)
 *
 * w_gate, w_up  [I][K/32] GGUF Q8_0 blocks of 34 bytes each (as w_blocks).
 * I     hidden units; I >= 32, I % 32 == 0.  K as for q8_pack_weights.
 * w_packed, packed_bytes  as for q8_pack_weights with N = 2I.
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_SIZE,
 * Q8_ERR_DEVICE, Q8_ERR_LAUNCH.
 */
q8_status q8_pack_weights_gateup(const void *w_gate, const void *w_up, int64_t I, int64_t K,
                                 void *w_packed, size_t *packed_bytes, void *stream);

/*
 * q8_gemm_swiglu -- gate and up products, the gated activation and its
 * quantisation for the down projection, in one call:
 *
 *     g = A * Wg^T,  u = A * Wu^T       (each as q8_gemm, binary32)
 *     h = silu(g) * u,  silu(x) = x / (1 + e^-x)     (binary32)
 *     (q_h, d_h) = Q8_0 quantisation of the rows of h (as q8_quantize_act)
 *
 * g and u never go through memory: the matrix-core kernel (M > 8) and the
 * decode kernel (M <= 8) apply the step to their accumulators.  Precision:
 * g and u carry the bound of q8_gemm; silu uses the device's binary32 exp
 * and a correctly rounded division, and the product is rounded once; the
 * codes are then decided in binary32 like q8_quantize_act.  A value of h
 * within a few binary32 units of a rounding boundary of the quantiser may
 * therefore land on either side of it.
 *
 * q_a, d_a  the quantised activations [M][K] (as for q8_gemm).
 * w_packed  the output of q8_pack_weights_gateup for the same I and K.
 * q_h   [M][I] int8 out (16-byte aligned); d_h [M][I/32] binary16 out
 *       (2-byte aligned).
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE (I < 32 or I % 32 != 0, bad K or M),
 * Q8_ERR_ALIGN, Q8_ERR_DEVICE, Q8_ERR_LAUNCH.
 */
q8_status q8_gemm_swiglu(int64_t M, int64_t I, int64_t K, const int8_t *q_a,
                         const uint16_t *d_a, const void *w_packed, int8_t *q_h,
                         uint16_t *d_h, void *stream);

/*
 * q8_kv3_encode -- compress key or value vectors to 3 bits per element.
 *
 * Source: the source engine holds a 256K-token context by storing its KV
 * cache in 3 bits, transformed by a Walsh-Hadamard transform (WHT) and
 * quantised with a Lloyd-Max quantiser, which shrinks the cache from 17 GB
 * to 3.5 GB (news.hada.io topic 29953, list of paths that avoid the
 * throttled units, KV-cache item).  The pages give no more than that; the
 * format below is this library's reading of it, defined exactly so that
 * every implementation of it produces the same bits.
 *
 * Operation, per row x of D values (bfloat16 is widened exactly):
 *   y = H x, the unnormalised WHT, computed in binary32 as the radix-2
 *       butterfly: for len = 1, 2, 4, ..., D/2, for every i with
 *       (i & len) == 0: (y_i, y_{i+len}) <- (y_i + y_{i+len}, y_i - y_{i+len});
 *   S = sum of y_i^2 by pairwise summation over adjacent pairs: the
 *       squares v_i = y_i^2, then for len = 1, 2, 4, ..., D/2:
 *       v_i <- v_i + v_{i+len} for every i that is a multiple of 2 len;
 *       S = v_0 (all binary32);
 *   s = sqrtf(S / D)  (correctly rounded; the RMS of y, so y/s has unit
 *       variance, the Gaussian the quantiser is designed for);
 *   if s < FLT_MIN (a zero row, binary32 underflow, or NaN): s = 0 and
 *       every code is 4;
 *   else u_i = y_i * (1/s) (the reciprocal correctly rounded) and code_i =
 *       the number of thresholds t_k <= u_i, where t_k = (L_k + L_{k+1})/2
 *       in binary32 and L = {-2.1520, -1.3440, -0.7560, -0.2451, 0.2451,
 *       0.7560, 1.3440, 2.1520} (binary32 nearest) are the levels of the
 *       8-level Lloyd-Max quantiser of a unit Gaussian.
 * No operation is fused (no fma).
 *
 * Storage: codes [R][3D/8] bytes; code i of a row sits at bits 3*(i % 8)
 * of the little-endian 24-bit word in bytes 3*(i/8) .. 3*(i/8)+2 of the
 * row.  scales [R] binary32 (s).  3.125 bits per element at D = 128.
 *
 * x      [R][ldx] binary32 or bfloat16 (dtype); 16-byte aligned,
 *        ldx >= D, ldx*elem % 16 == 0, ldx*elem < 2^25 (32 MiB).
 * R      rows (tokens x heads), R >= 0; R == 0 is a no-op.
 * D      head dimension: 64, 128 or 256.
 * codes  out, [R][3D/8] bytes, 16-byte aligned.
 * scales out, [R] binary32, 4-byte aligned.
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE (D not 64/128/256, R < 0, ldx < D, R
 * too large to launch), Q8_ERR_ALIGN, Q8_ERR_DTYPE, Q8_ERR_DEVICE,
 * Q8_ERR_LAUNCH.
 */
q8_status q8_kv3_encode(const void *x, q8_dtype dtype, int64_t R, int64_t D, int64_t ldx,
                        uint8_t *codes, float *scales, void *stream);

/*
 * q8_kv3_decode -- expand 3-bit KV rows written by q8_kv3_encode.
 *
 * Operation, per row: z_i = s * L[code_i] (binary32), then the same
 * butterfly as the encoder (H is its own inverse up to a factor D), then
 * out_i = z_i * (1/D).  For out_dtype Q8_BF16 the binary32 result is
 * rounded to bfloat16, nearest-even.
 *
 * codes, scales  as written by q8_kv3_encode for the same D (codes
 *        16-byte aligned, scales 4-byte aligned).
 * R, D   as for q8_kv3_encode.
 * out    [R][ldo] of out_dtype; 16-byte aligned, ldo >= D,
 *        ldo*elem % 16 == 0, ldo*elem < 2^25 (32 MiB).
 *
 * Errors: Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DTYPE,
 * Q8_ERR_DEVICE, Q8_ERR_LAUNCH.
 */
q8_status q8_kv3_decode(const uint8_t *codes, const float *scales, int64_t R, int64_t D,
                        q8_dtype out_dtype, void *out, int64_t ldo, void *stream);

/*
 * Block-sparse causal attention for long-context prefill: q8_attn_pool,
 * q8_attn_select, q8_attn_fwd.
 *
 * Source: the source engine computes attention with its own FlashAttention
 * kernel and MInference-style block sparsity (news.hada.io topic 29953,
 * list of paths that avoid the throttled units, attention item).  The pages
 * say no more; the operation below is this library's reading of it.
 *
 * Tokens form blocks of 64 (block b: tokens 64b .. min(64b+63, L-1)).
 * Q [L][ldq], K [L][ldk], V [L][ldv] are bfloat16, token-major: query head
 * h occupies columns h*D .. h*D+D-1 of Q, and reads key/value head
 * g = h / (Hq/Hkv) at columns g*D .. of K and V (grouped-query heads).
 *
 * q8_attn_pool: pooled[h][b][d] (binary32) = mean over block b's tokens of
 *   x[t][h*D + d].  x is Q (H = Hq) or K (H = Hkv).  pooled has
 *   H * NB * D floats, NB = ceil(L/64), and is 16-byte aligned.
 *   x: 16-byte aligned, ldx >= H*D, ldx*2 % 16 == 0, ldx < 2^24.
 *
 * q8_attn_select: for every K/V head g and query block i, the key blocks
 *   the block's queries attend to, shared by the Hq/Hkv query heads of g's
 *   group (they read the same K and V): block 0, block i, and the k - 2
 *   blocks 0 < j < i with the highest score
 *   (sum over the group's heads h of pooled_q[h][i]) . pooled_k[g][j]
 *   (higher score first, the lower j on equal scores); every block j <= i
 *   when k >= i + 1.  idx [Hkv][NB][kmax] int32 receives them in ascending
 *   order, -1 after the last; cnt [Hkv][NB] int32 receives min(k, i + 1).
 *   2 <= k <= kmax,
 *   NB <= 4096.  Scores are binary32 dot products of the binary32 pooled
 *   rows; blocks whose scores differ from the k-2'th by a few binary32
 *   units may be chosen either way.
 *
 * q8_attn_fwd: out[t][h*D + d] = sum_u p_u V[u][g*D + d] / sum_u p_u over
 *   the keys u <= t of the blocks listed for (g, t's block) (idx/cnt
 *   [Hkv][NB] as written by q8_attn_select, or any lists of blocks
 *   0 <= j <= i in ascending order),
 *   p_u = exp(q_t . k_u / sqrt(D) - max).  Scores and sums in binary32 on
 *   the bf16 matrix cores, p rounded to bfloat16 for the product with V (as
 *   in FlashAttention), so |out - exact| <= ~2^-8 * sum_u p_u |V_u| / sum_u p_u
 *   (plus the output's rounding for bfloat16).  List entries outside
 *   [0, i] are skipped and cnt is clamped to [0, kmax]; an empty list gives
 *   non-finite output.  out: out_dtype Q8_F32 (16-byte aligned,
 *   ldo*4 % 16 == 0) or Q8_BF16 (8-byte aligned, ldo*2 % 8 == 0), ldo >= Hq*D.
 *   Q, K, V: 16-byte aligned, ld*2 % 16 == 0, ld >= heads*D, ld < 2^24.
 *   D = 64 or 128; Hq % Hkv == 0; L <= 262144.
 *
 * Errors (all three): Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_DTYPE
 * (q8_attn_fwd), Q8_ERR_DEVICE, Q8_ERR_LAUNCH.  L == 0 (NB == 0) is a no-op.
 */
q8_status q8_attn_pool(const void *x, int64_t L, int64_t ldx, int64_t H, int64_t D,
                       float *pooled, void *stream);
q8_status q8_attn_select(const float *pooled_q, const float *pooled_k, int64_t Hq, int64_t Hkv,
                         int64_t NB, int64_t D, int k, int kmax, int32_t *idx, int32_t *cnt,
                         void *stream);
q8_status q8_attn_fwd(const void *q, const void *k, const void *v, int64_t L, int64_t ldq,
                      int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int64_t D,
                      const int32_t *idx, const int32_t *cnt, int kmax, q8_dtype out_dtype,
                      void *out, int64_t ldo, void *stream);

/* Static description of a status code (never NULL). */
const char *q8_status_string(q8_status s);

#ifdef __cplusplus
}
#endif
#endif /* Q8_H */
