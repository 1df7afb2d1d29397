/*
 * q8ref.c -- plain, slow CPU oracle for the Q8_0 weight x activation product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library and includes nothing from it.
 *
 * Source.  news.hada.io topic 29953, "CUDA inference engine for running
 * Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)".  Its list of
 * paths that avoid the throttled units has the GEMM done by a self-written
 * int8 DP4A kernel; its benchmark list and its limitations list name Q8_0
 * GGUF as the one supported weight format.  The pages do not spell Q8_0
 * out.  The format used here is the GGUF Q8_0 block: 32 consecutive values
 * along K stored as int8 q[32] with one IEEE binary16 scale d, the value
 * being d*q.  A block is quantised with d = amax/127 and q = x/d rounded
 * half away from zero.  Activations are quantised on the fly into the same
 * block format, so every product term is int8*int8 inside a block and the
 * two scales multiply the block's integer dot.
 *
 * Precision.  The quantiser decides integers, so it runs in binary32 exactly
 * as the kernel does (IEEE division, one multiply, no FMA; build with
 * -ffp-contract=off).  The GEMM is the definition written out: exact int32
 * block dots, each times the exact product of the two binary16 scales,
 * summed over blocks in double (every product is exact in double: the scale
 * product has at most 22 significant bits and |dot| < 2^20).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (oracle/build.py).
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QK 32                 /* values per Q8_0 block along K */
#define BLOCK_BYTES 34        /* GGUF Q8_0 block: binary16 d, then int8 q[32] */

/* ------------------------------------------------------------------------ */
/* binary16 and bfloat16 conversions, from the IEEE 754 encodings.          */
/* ------------------------------------------------------------------------ */

/* Round the non-negative integer v / 2^s to nearest, ties to even. */
static uint32_t shift_rne(uint32_t v, int s)
{
    if (s <= 0) return v << (-s);
    if (s >= 32) return 0;                     /* v < 2^24, so v/2^s < 1/2 */
    uint32_t q = v >> s;
    uint32_t rem = v & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return q;
}

/* binary32 -> binary16 bits, round to nearest even, subnormals kept,
 * overflow to infinity.  NaN maps to a quiet NaN. */
uint16_t q8ref_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a >= 0x7f800000u) return sign | (a > 0x7f800000u ? 0x7e00u : 0x7c00u);
    if (a < 0x00800000u) return sign;          /* binary32 subnormal or zero */
    int e = (int)(a >> 23) - 127;              /* |f| = sig * 2^(e-23) */
    uint32_t sig = (a & 0x7fffffu) | 0x800000u;
    if (e >= -14) {
        /* normal binary16 target: keep 11 significant bits */
        uint32_t m = shift_rne(sig, 13);       /* in [1024, 2048] */
        if (m == 2048u) { m = 1024u; e += 1; }
        if (e > 15) return sign | 0x7c00u;
        return sign | (uint16_t)(((uint32_t)(e + 15) << 10) | (m & 0x3ffu));
    }
    /* subnormal binary16 target: unit 2^-24, |f|/2^-24 = sig * 2^(e+1) */
    uint32_t m = shift_rne(sig, -(e + 1));     /* in [0, 1024]; 1024 = min normal */
    return sign | (uint16_t)m;
}

/* Elementwise form of q8ref_f32_to_f16 over an array. */
void q8ref_f32_to_f16_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = q8ref_f32_to_f16(x[i]);
}

/* binary16 bits -> exact double value. */
double q8ref_f16_to_f64(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m | 0x400), e - 25);
    return s ? -v : v;
}

/* bfloat16 bits -> binary32 (exact: the upper half of a binary32). */
float q8ref_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Quantiser: one 32-value block.                                           */
/* ------------------------------------------------------------------------ */

/* Round half away from zero, written out from its definition rather than
 * taken from the C library: r = sign(v) * floor(|v| + 1/2), evaluated
 * without the binary32 rounding trap of floor(v + 0.5f).  For |v| < 2^23
 * the fractional part of |v| is exact in binary32. */
static float round_half_away(float v)
{
    float a = fabsf(v);
    if (!(a < 8388608.0f)) return v;          /* already an integer (or NaN) */
    float t = truncf(a);                      /* integer part, exact */
    float frac = a - t;                       /* exact: both share an exponent range */
    float r = (frac >= 0.5f) ? t + 1.0f : t;
    return v < 0.0f ? -r : r;
}

/* Quantise x[0..31] (binary32) into q[0..31] and the binary16 scale *d.
 * Steps: amax = max |x_j|; d32 = amax / 127 (binary32, correctly rounded);
 * if d32 is below the smallest normal binary32 (this covers the all-zero
 * block) every q is 0 and d is +0; otherwise id = 1 / d32 (binary32,
 * correctly rounded), q_j = round_half_away(x_j * id) and d = binary16(d32),
 * round to nearest even.  Returns 0, or -1 if some |q_j| would exceed 127
 * (impossible for finite input; kept as a self-check). */
int q8ref_quantize_block(const float *x, int8_t *q, uint16_t *d)
{
    float amax = 0.0f;
    for (int j = 0; j < QK; ++j) {
        float ax = fabsf(x[j]);
        if (ax > amax) amax = ax;
    }
    float d32 = amax / 127.0f;
    if (d32 < FLT_MIN) {
        for (int j = 0; j < QK; ++j) q[j] = 0;
        *d = 0;
        return 0;
    }
    float id = 1.0f / d32;
    int bad = 0;
    for (int j = 0; j < QK; ++j) {
        float v = x[j] * id;
        float r = round_half_away(v);
        if (r > 127.0f || r < -127.0f) { bad = 1; r = r > 0 ? 127.0f : -127.0f; }
        q[j] = (int8_t)r;
    }
    *d = q8ref_f32_to_f16(d32);
    return bad ? -1 : 0;
}

/* Quantise M rows of K values (K % 32 == 0).  x is binary32 (dtype 0) or
 * bfloat16 bits (dtype 1) with row stride ldx elements.  q is [M][K],
 * d is [M][K/32].  Returns the number of blocks that failed the self-check. */
int64_t q8ref_quantize_rows(const void *x, int dtype, int64_t M, int64_t K,
                            int64_t ldx, int8_t *q, uint16_t *d)
{
    int64_t KB = K / QK, bad = 0;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float blk[QK];
        for (int64_t kb = 0; kb < KB; ++kb) {
            for (int j = 0; j < QK; ++j) {
                int64_t k = kb * QK + j;
                if (dtype == 0) blk[j] = ((const float *)x)[m * ldx + k];
                else blk[j] = q8ref_bf16_to_f32(((const uint16_t *)x)[m * ldx + k]);
            }
            if (q8ref_quantize_block(blk, q + m * K + kb * QK, d + m * KB + kb) != 0)
                bad += 1;
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* GGUF Q8_0 block bytes <-> separate q / d arrays.                         */
/* ------------------------------------------------------------------------ */

/* Block (n, kb) of a [N][K] weight is 34 bytes at offset (n*KB + kb)*34:
 * the binary16 scale, little-endian, then q[0..31]. */
void q8ref_blocks_from_qd(const int8_t *q, const uint16_t *d, int64_t N, int64_t K,
                          uint8_t *blocks)
{
    int64_t KB = K / QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            uint8_t *b = blocks + (n * KB + kb) * BLOCK_BYTES;
            uint16_t h = d[n * KB + kb];
            b[0] = (uint8_t)(h & 0xff);
            b[1] = (uint8_t)(h >> 8);
            memcpy(b + 2, q + n * K + kb * QK, QK);
        }
}

void q8ref_qd_from_blocks(const uint8_t *blocks, int64_t N, int64_t K,
                          int8_t *q, uint16_t *d)
{
    int64_t KB = K / QK;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t kb = 0; kb < KB; ++kb) {
            const uint8_t *b = blocks + (n * KB + kb) * BLOCK_BYTES;
            d[n * KB + kb] = (uint16_t)(b[0] | (b[1] << 8));
            memcpy(q + n * K + kb * QK, b + 2, QK);
        }
}

/* ------------------------------------------------------------------------ */
/* GEMM: C[m][n] = sum_kb d_a[m][kb] * d_w[n][kb] * sum_j q_a * q_w.          */
/* ------------------------------------------------------------------------ */

/* Block integer dot of two 32-value int8 blocks (exact in int32). */
static int32_t block_dot(const int8_t *a, const int8_t *w)
{
    int32_t s = 0;
    for (int j = 0; j < QK; ++j) s += (int32_t)a[j] * (int32_t)w[j];
    return s;
}

static int32_t block_absdot(const int8_t *a, const int8_t *w)
{
    int32_t s = 0;
    for (int j = 0; j < QK; ++j) s += abs((int32_t)a[j] * (int32_t)w[j]);
    return s;
}

/* One output element, by the definition.  Also returns the magnitude
 * sum_kb |d_a|*|d_w|*sum_j |q_a*q_w| (the abs-dot used to normalise errors).
 * qa_row / da_row: activation row m; qw_row / dw_row: weight row n. */
static void one_output(const int8_t *qa_row, const uint16_t *da_row,
                       const int8_t *qw_row, const uint16_t *dw_row, int64_t KB,
                       double *c, double *absdot)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t kb = 0; kb < KB; ++kb) {
        double s = q8ref_f16_to_f64(da_row[kb]) * q8ref_f16_to_f64(dw_row[kb]);
        int32_t p = block_dot(qa_row + kb * QK, qw_row + kb * QK);
        acc += s * (double)p;
        mag += fabs(s) * (double)block_absdot(qa_row + kb * QK, qw_row + kb * QK);
    }
    *c = acc;
    *absdot = mag;
}

/* Full product.  q_a [M][K], d_a [M][K/32], q_w [N][K], d_w [N][K/32];
 * C and absdot are [M][N] doubles (absdot may be NULL). */
void q8ref_gemm(int64_t M, int64_t N, int64_t K,
                const int8_t *q_a, const uint16_t *d_a,
                const int8_t *q_w, const uint16_t *d_w,
                double *C, double *absdot)
{
    int64_t KB = K / QK;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double c, a;
            one_output(q_a + m * K, d_a + m * KB, q_w + n * K, d_w + n * KB, KB, &c, &a);
            C[m * N + n] = c;
            if (absdot) absdot[m * N + n] = a;
        }
}

/* Selected outputs only: (rows[i], cols[i]) for i < count. */
void q8ref_gemm_sampled(int64_t K, const int8_t *q_a, const uint16_t *d_a,
                        const int8_t *q_w, const uint16_t *d_w,
                        const int64_t *rows, const int64_t *cols, int64_t count,
                        double *C, double *absdot)
{
    int64_t KB = K / QK;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double c, a;
        one_output(q_a + rows[i] * K, d_a + rows[i] * KB,
                   q_w + cols[i] * K, d_w + cols[i] * KB, KB, &c, &a);
        C[i] = c;
        if (absdot) absdot[i] = a;
    }
}

/* Block integer dots P[m][n][kb] (exact int32), for checking integer work. */
void q8ref_block_dots(int64_t M, int64_t N, int64_t K,
                      const int8_t *q_a, const int8_t *q_w, int32_t *P)
{
    int64_t KB = K / QK;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t kb = 0; kb < KB; ++kb)
                P[(m * N + n) * KB + kb] = block_dot(q_a + m * K + kb * QK, q_w + n * K + kb * QK);
}

/* ------------------------------------------------------------------------ */
/* The packed weight layout of the library's pack call, written from its    */
/* published description (not from the library's code):                    */
/*   NG = ceil(N/64) row groups, KB = K/32 blocks.                           */
/*   Quant plane, NG*KB*2048 bytes: byte ((g*KB + kb)*2 + h)*1024 + r*16 + t */
/*     holds q[64g + r][32kb + 16h + t] (0 when 64g + r >= N),               */
/*     for h in {0,1}, r in [0,64), t in [0,16).                             */
/*   Scale plane, right after it, NG*KB*64 binary16 values: element          */
/*     (g*KB + kb)*64 + r holds d[64g + r][kb] (0 when 64g + r >= N).        */
/* ------------------------------------------------------------------------ */

size_t q8ref_packed_bytes(int64_t N, int64_t K)
{
    int64_t NG = (N + 63) / 64, KB = K / QK;
    return (size_t)(NG * KB) * (2048u + 128u);
}

void q8ref_pack(const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed)
{
    int64_t NG = (N + 63) / 64, KB = K / QK;
    uint8_t *qplane = packed;
    uint16_t *splane = (uint16_t *)(packed + (size_t)(NG * KB) * 2048u);
    for (int64_t g = 0; g < NG; ++g)
        for (int64_t kb = 0; kb < KB; ++kb)
            for (int r = 0; r < 64; ++r) {
                int64_t n = 64 * g + r;
                const uint8_t *b = (n < N) ? blocks + (n * KB + kb) * BLOCK_BYTES : NULL;
                for (int h = 0; h < 2; ++h)
                    for (int t = 0; t < 16; ++t)
                        qplane[((g * KB + kb) * 2 + h) * 1024 + r * 16 + t] =
                            b ? b[2 + 16 * h + t] : 0;
                splane[(g * KB + kb) * 64 + r] = b ? (uint16_t)(b[0] | (b[1] << 8)) : 0;
            }
}

/* ------------------------------------------------------------------------ */
/* Gated feed-forward step after the gate and up products (the step after   */
/* the path; the pages' engine runs Qwen3.5/3.6 models, whose FFNs are      */
/* gated; the pages do not spell the FFN out, so this is the plainest       */
/* reading): h = silu(g) * u with silu(x) = x / (1 + e^-x), then each row   */
/* of h quantised to Q8_0 blocks of 32 along the hidden dimension -- the    */
/* activation format the down projection consumes.                          */
/* ------------------------------------------------------------------------ */

double q8ref_silu(double x)
{
    return x / (1.0 + exp(-x));
}

/* G, U: [M][I] doubles (the gate and up products, e.g. from q8ref_gemm).
 * h: [M][I] doubles out (may be NULL).  q [M][I] int8 and d [M][I/32]
 * binary16 out: h rounded to binary32, then quantised block by block
 * (q8ref_quantize_block).  I % 32 == 0. */
void q8ref_swiglu_quant(int64_t M, int64_t I, const double *G, const double *U,
                        double *h, int8_t *q, uint16_t *d)
{
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t b = 0; b < I / QK; ++b) {
            float x[QK];
            for (int j = 0; j < QK; ++j) {
                int64_t i = m * I + b * QK + j;
                double v = q8ref_silu(G[i]) * U[i];
                if (h) h[i] = v;
                x[j] = (float)v;
            }
            q8ref_quantize_block(x, q + m * I + b * QK, d + m * (I / QK) + b);
        }
}

/* ------------------------------------------------------------------------ */
/* 3-bit KV-cache codec (the pages' "3-bit KV cache (WHT + Lloyd-Max)",     */
/* 17 GB -> 3.5 GB at 256K context; the pages give no more detail, so the   */
/* format below is the plainest reading, written from its description in    */
/* the library header):                                                     */
/*   a row x of D values (D = 64, 128 or 256) is transformed by the         */
/*   unnormalised Sylvester Hadamard matrix, y = H x, with the radix-2      */
/*   butterfly in binary32 (stages len = 1, 2, 4, ..., D/2; a pair (i,      */
/*   i+len) becomes (a+b, a-b));                                            */
/*   s = sqrt(S/D) with S the sum of y_i^2 by the pairwise tree over       */
/*   adjacent pairs (len = 1, 2, 4, ..., D/2: v_i += v_{i+len} for i a      */
/*   multiple of 2 len), binary32, correctly rounded sqrt;                  */
/*   u_i = y_i * (1/s);                                                     */
/*   code_i = the number of decision thresholds t_k <= u_i, the thresholds  */
/*   being the binary32 midpoints (L_k + L_{k+1}) * 0.5 of the codebook L   */
/*   (the 8-level Lloyd-Max quantiser of a unit Gaussian, levels +-0.2451,  */
/*   +-0.7560, +-1.3440, +-2.1520 as binary32);                             */
/*   rows with s < FLT_MIN get every code 4 and s = 0;                      */
/*   8 codes pack into 3 bytes little-endian, code j of a group at bits     */
/*   3j..3j+2; decode: z_i = s * L[code_i], x^ = (H z) * (1/D).             */
/* ------------------------------------------------------------------------ */

static const float kv3_levels[8] = {-2.1520f, -1.3440f, -0.7560f, -0.2451f,
                                    0.2451f,  0.7560f,  1.3440f,  2.1520f};

void q8ref_kv3_levels(float *out)
{
    for (int i = 0; i < 8; ++i) out[i] = kv3_levels[i];
}

/* In-place binary32 fast Walsh-Hadamard transform (unnormalised). */
void q8ref_fwht(float *v, int D)
{
    for (int len = 1; len < D; len <<= 1)
        for (int i = 0; i < D; i += 2 * len)
            for (int j = i; j < i + len; ++j) {
                float a = v[j], b = v[j + len];
                v[j] = a + b;
                v[j + len] = a - b;
            }
}

static int kv3_code(float u)
{
    int c = 0;
    for (int k = 0; k < 7; ++k) {
        float t = (kv3_levels[k] + kv3_levels[k + 1]) * 0.5f;
        if (t <= u) ++c;
    }
    return c;
}

/* x: [R][ldx] binary32 (dtype 0) or bfloat16 bits (dtype 1).
 * codes: [R][3D/8] bytes; scales: [R] binary32. */
void q8ref_kv3_encode(const void *x, int dtype, int64_t R, int D, int64_t ldx,
                      uint8_t *codes, float *scales)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        float y[256], v[256];
        for (int i = 0; i < D; ++i)
            y[i] = dtype == 1 ? q8ref_bf16_to_f32(((const uint16_t *)x)[r * ldx + i])
                              : ((const float *)x)[r * ldx + i];
        q8ref_fwht(y, D);
        for (int i = 0; i < D; ++i) v[i] = y[i] * y[i];
        for (int len = 1; len < D; len <<= 1)
            for (int i = 0; i < D; i += 2 * len) v[i] = v[i] + v[i + len];
        float s = sqrtf(v[0] / (float)D);
        uint8_t *out = codes + r * (3 * D / 8);
        memset(out, 0, (size_t)(3 * D / 8));
        if (!(s >= FLT_MIN)) {
            s = 0.0f;
            for (int i = 0; i < D; ++i) y[i] = 0.0f;   /* code 4 below */
        }
        float inv = s > 0.0f ? 1.0f / s : 0.0f;
        for (int g = 0; g < D / 8; ++g) {
            uint32_t w = 0;
            for (int j = 0; j < 8; ++j) {
                int c = kv3_code(y[8 * g + j] * inv);
                w |= (uint32_t)c << (3 * j);
            }
            out[3 * g + 0] = (uint8_t)(w & 0xff);
            out[3 * g + 1] = (uint8_t)((w >> 8) & 0xff);
            out[3 * g + 2] = (uint8_t)((w >> 16) & 0xff);
        }
        scales[r] = s;
    }
}

/* codes, scales as written by q8ref_kv3_encode -> out [R][D] binary32. */
void q8ref_kv3_decode(const uint8_t *codes, const float *scales, int64_t R, int D, float *out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        float z[256];
        const uint8_t *in = codes + r * (3 * D / 8);
        for (int g = 0; g < D / 8; ++g) {
            uint32_t w = in[3 * g] | ((uint32_t)in[3 * g + 1] << 8) | ((uint32_t)in[3 * g + 2] << 16);
            for (int j = 0; j < 8; ++j) z[8 * g + j] = scales[r] * kv3_levels[(w >> (3 * j)) & 7u];
        }
        q8ref_fwht(z, D);
        for (int i = 0; i < D; ++i) out[r * D + i] = z[i] * (1.0f / (float)D);
    }
}

/* ------------------------------------------------------------------------ */
/* Block-sparse causal attention, prefill (the pages' "own FlashAttention + */
/* MInference-style block-sparse"; nothing more is given, so the reading   */
/* below is the plainest one, written from its description in the library */
/* header):                                                                 */
/*   Q [L][ldq], K [L][ldk], V [L][ldv] bfloat16, token-major; head h of Q  */
/*   at columns h*D .. h*D+D-1, its K/V head g = h / (Hq/Hkv) likewise.     */
/*   Blocks of 64 tokens; block i holds tokens 64i .. min(64i+63, L-1).     */
/*   Pooled rows: the mean over a block's tokens of Q (per query head) and  */
/*   of K (per K/V head).                                                   */
/*   Selection, per K/V head g (shared by its group of Hq/Hkv query heads): */
/*   query block i keeps block 0, block i, and the top (k - 2) blocks      */
/*   0 < j < i by score (sum over the group's heads of their pooled query   */
/*   rows) . (pooled key row of block j) (ties: lower j first); all blocks  */
/*   j <= i when k >= i + 1.  Listed in ascending order, cnt = min(k,i+1). */
/*   Output: token t of query block i attends to the keys u <= t of its     */
/*   listed blocks: o = sum_u p_u v_u / sum_u p_u, p_u = exp(q.k_u / sqrt D */
/*   - max), computed in double.                                            */
/* ------------------------------------------------------------------------ */

#define ATTN_BLK 64

static double bf16d(const uint16_t *p) { return (double)q8ref_bf16_to_f32(*p); }

/* pooled [H][NB][D] (double): mean over each block's tokens of x's head h. */
void q8ref_attn_pool(const uint16_t *x, int64_t L, int64_t ldx, int64_t H, int D,
                     double *pooled)
{
    const int64_t NB = (L + ATTN_BLK - 1) / ATTN_BLK;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t h = 0; h < H; ++h)
        for (int64_t b = 0; b < NB; ++b) {
            const int64_t t0 = b * ATTN_BLK, t1 = t0 + ATTN_BLK < L ? t0 + ATTN_BLK : L;
            double *out = pooled + (h * NB + b) * D;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t t = t0; t < t1; ++t) acc += bf16d(x + t * ldx + h * D + d);
                out[d] = acc / (double)(t1 - t0);
            }
        }
}

/* idx [Hkv][NB][kmax] (ascending, the rest -1), cnt [Hkv][NB]; k <= kmax. */
void q8ref_attn_select(const double *pq, const double *pk, int64_t Hq, int64_t Hkv, int64_t NB,
                       int D, int k, int kmax, int32_t *idx, int32_t *cnt)
{
    const int64_t group = Hq / Hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic, 16)
    for (int64_t h = 0; h < Hkv; ++h)
        for (int64_t i = 0; i < NB; ++i) {
            int32_t *row = idx + (h * NB + i) * kmax;
            for (int m = 0; m < kmax; ++m) row[m] = -1;
            char *take = calloc((size_t)i + 1, 1);
            int n = 0;
            if (k >= i + 1) {
                for (int64_t j = 0; j <= i; ++j) take[j] = 1;
                n = (int)i + 1;
            } else {
                take[0] = 1;
                take[i] = 1;
                n = i > 0 ? 2 : 1;
                double *q = calloc((size_t)D, sizeof(double));   /* the group's query row */
                for (int64_t hq = h * group; hq < (h + 1) * group; ++hq)
                    for (int d = 0; d < D; ++d) q[d] += pq[(hq * NB + i) * D + d];
                while (n < k) {                          /* next best: highest score, lowest j */
                    int64_t best = -1;
                    double bs = 0.0;
                    for (int64_t j = 1; j < i; ++j) {
                        if (take[j]) continue;
                        const double *kk = pk + (h * NB + j) * D;
                        double sc = 0.0;
                        for (int d = 0; d < D; ++d) sc += q[d] * kk[d];
                        if (best < 0 || sc > bs) { best = j; bs = sc; }
                    }
                    take[best] = 1;
                    ++n;
                }
                free(q);
            }
            int m = 0;
            for (int64_t j = 0; j <= i; ++j)
                if (take[j]) row[m++] = (int32_t)j;
            cnt[h * NB + i] = n;
            free(take);
        }
}

/* One output row: token t of query head h -> o[D], m[D] (double). */
static void attn_row(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t L,
                     int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int D,
                     const int32_t *idx, const int32_t *cnt, int kmax, int64_t t, int64_t h,
                     double *o, double *mg)
{
    const int64_t NB = (L + ATTN_BLK - 1) / ATTN_BLK, group = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)D);
    const int64_t i = t / ATTN_BLK, g = h / group;
    const int32_t *row = idx + (g * NB + i) * kmax;       /* the K/V head's list */
    const int n = cnt[g * NB + i];
    double *s = malloc(sizeof(double) * (size_t)n * ATTN_BLK);
    int64_t *u_of = malloc(sizeof(int64_t) * (size_t)n * ATTN_BLK);
    int ns = 0;
    double mx = -INFINITY;
    for (int m = 0; m < n; ++m)
        for (int64_t u = (int64_t)row[m] * ATTN_BLK; u < ((int64_t)row[m] + 1) * ATTN_BLK; ++u) {
            if (u > t || u >= L) continue;
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += bf16d(Q + t * ldq + h * D + d) * bf16d(K + u * ldk + g * D + d);
            s[ns] = dot * scale;
            u_of[ns] = u;
            if (s[ns] > mx) mx = s[ns];
            ++ns;
        }
    double den = 0.0;
    for (int a = 0; a < ns; ++a) { s[a] = exp(s[a] - mx); den += s[a]; }
    for (int d = 0; d < D; ++d) {
        double num = 0.0, am = 0.0;
        for (int a = 0; a < ns; ++a) {
            const double v = bf16d(V + u_of[a] * ldv + g * D + d);
            num += s[a] * v;
            am += s[a] * fabs(v);
        }
        o[d] = num / den;
        mg[d] = am / den;
    }
    free(s);
    free(u_of);
}

/* out [L][Hq*D] and mag [L][Hq*D] (double): the attention output and, per
 * element, sum_u p_u |v_u| / sum_u p_u (the scale of its rounding error). */
void q8ref_attn_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t L,
                    int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int D,
                    const int32_t *idx, const int32_t *cnt, int kmax, double *out, double *mag)
{
    #pragma omp parallel for collapse(2) schedule(dynamic, 8)
    for (int64_t h = 0; h < Hq; ++h)
        for (int64_t t = 0; t < L; ++t)
            attn_row(Q, K, V, L, ldq, ldk, ldv, Hq, Hkv, D, idx, cnt, kmax, t, h,
                     out + t * Hq * D + h * D, mag + t * Hq * D + h * D);
}

/* The same at n chosen (token, head) pairs: out, mag [n][D]. */
void q8ref_attn_fwd_at(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t L,
                       int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int D,
                       const int32_t *idx, const int32_t *cnt, int kmax, const int64_t *tok,
                       const int64_t *head, int64_t n, double *out, double *mag)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t a = 0; a < n; ++a)
        attn_row(Q, K, V, L, ldq, ldk, ldv, Hq, Hkv, D, idx, cnt, kmax, tok[a], head[a],
                 out + a * D, mag + a * D);
}

/* Threads the OpenMP runtime will use (for reporting the CPU baseline). */
int q8ref_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
