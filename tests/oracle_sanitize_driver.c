/* Drives every entry point of the CPU oracle (oracle/q8ref.c) on small and
 * edge-case inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).  Every
 * buffer is allocated at exactly the size the entry point's contract states,
 * so an access past it is reported.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int64_t q8ref_quantize_rows(const void *x, int dtype, int64_t M, int64_t K, int64_t ldx,
                            int8_t *q, uint16_t *d);
void q8ref_blocks_from_qd(const int8_t *q, const uint16_t *d, int64_t N, int64_t K,
                          uint8_t *blocks);
void q8ref_qd_from_blocks(const uint8_t *blocks, int64_t N, int64_t K, int8_t *q, uint16_t *d);
void q8ref_gemm(int64_t M, int64_t N, int64_t K, const int8_t *q_a, const uint16_t *d_a,
                const int8_t *q_w, const uint16_t *d_w, double *C, double *absdot);
void q8ref_gemm_sampled(int64_t K, const int8_t *q_a, const uint16_t *d_a, const int8_t *q_w,
                        const uint16_t *d_w, const int64_t *rows, const int64_t *cols,
                        int64_t count, double *C, double *absdot);
void q8ref_block_dots(int64_t M, int64_t N, int64_t K, const int8_t *q_a, const int8_t *q_w,
                      int32_t *P);
size_t q8ref_packed_bytes(int64_t N, int64_t K);
void q8ref_pack(const uint8_t *blocks, int64_t N, int64_t K, uint8_t *packed);
void q8ref_swiglu_quant(int64_t M, int64_t I, const double *G, const double *U, double *h,
                        int8_t *q, uint16_t *d);
void q8ref_kv3_levels(float *out);
void q8ref_fwht(float *v, int D);
void q8ref_kv3_encode(const void *x, int dtype, int64_t R, int D, int64_t ldx, uint8_t *codes,
                      float *scales);
void q8ref_kv3_decode(const uint8_t *codes, const float *scales, int64_t R, int D, float *out);
void q8ref_attn_pool(const uint16_t *x, int64_t L, int64_t ldx, int64_t H, int D,
                     double *pooled);
void q8ref_attn_select(const double *pq, const double *pk, int64_t Hq, int64_t Hkv, int64_t NB,
                       int D, int k, int kmax, int32_t *idx, int32_t *cnt);
void q8ref_attn_fwd(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t L,
                    int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int D,
                    const int32_t *idx, const int32_t *cnt, int kmax, double *out, double *mag);
void q8ref_attn_fwd_at(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t L,
                       int64_t ldq, int64_t ldk, int64_t ldv, int64_t Hq, int64_t Hkv, int D,
                       const int32_t *idx, const int32_t *cnt, int kmax, const int64_t *tok,
                       const int64_t *head, int64_t n, double *out, double *mag);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {   /* xorshift64*, in [-1, 1) */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static uint16_t bf16_of(float f) {   /* truncation is enough for inputs */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static double checksum = 0.0;
static void add(double v) { if (isfinite(v)) checksum += v; }

static void gemm_path(int64_t M, int64_t N, int64_t K, int with_edges) {
    const int64_t KB = K / 32;
    float *x = xmalloc(sizeof(float) * M * (K + 3));   /* row pitch K + 3 */
    uint16_t *xb = xmalloc(sizeof(uint16_t) * M * K);
    float *w = xmalloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < M * (K + 3); ++i) x[i] = (float)uniform();
    for (int64_t i = 0; i < M * K; ++i) xb[i] = bf16_of((float)uniform() * 4.0f);
    for (int64_t i = 0; i < N * K; ++i) w[i] = (float)(0.02 * uniform());
    if (with_edges) {
        for (int64_t j = 0; j < 32; ++j) x[j] = 0.0f;             /* zero block */
        x[32] = 1e-42f;                                            /* subnormal amax */
        for (int64_t j = 33; j < 64; ++j) x[j] = 0.0f;
        x[K + 3] = 65504.0f * 127.0f;                              /* large amax */
    }
    int8_t *qa = xmalloc((size_t)(M * K)), *qb = xmalloc((size_t)(M * K)), *qw = xmalloc((size_t)(N * K));
    uint16_t *da = xmalloc(sizeof(uint16_t) * M * KB), *db = xmalloc(sizeof(uint16_t) * M * KB);
    uint16_t *dw = xmalloc(sizeof(uint16_t) * N * KB);
    add((double)q8ref_quantize_rows(x, 0, M, K, K + 3, qa, da));
    add((double)q8ref_quantize_rows(xb, 1, M, K, K, qb, db));
    add((double)q8ref_quantize_rows(w, 0, N, K, K, qw, dw));
    uint8_t *blocks = xmalloc((size_t)(N * KB * 34));
    q8ref_blocks_from_qd(qw, dw, N, K, blocks);
    int8_t *qw2 = xmalloc((size_t)(N * K));
    uint16_t *dw2 = xmalloc(sizeof(uint16_t) * N * KB);
    q8ref_qd_from_blocks(blocks, N, K, qw2, dw2);
    if (memcmp(qw, qw2, (size_t)(N * K)) || memcmp(dw, dw2, sizeof(uint16_t) * N * KB)) {
        fprintf(stderr, "block round trip differs\n");
        exit(3);
    }
    double *C = xmalloc(sizeof(double) * M * N), *ad = xmalloc(sizeof(double) * M * N);
    q8ref_gemm(M, N, K, qa, da, qw, dw, C, ad);
    q8ref_gemm(M, N, K, qb, db, qw, dw, C, NULL);
    for (int64_t i = 0; i < M * N; ++i) add(C[i]);
    int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {N - 1, 0, N / 2};
    double Cs[3], as[3];
    q8ref_gemm_sampled(K, qa, da, qw, dw, rows, cols, 3, Cs, as);
    add(Cs[0] + as[2]);
    int32_t *P = xmalloc(sizeof(int32_t) * M * N * KB);
    q8ref_block_dots(M, N, K, qa, qw, P);
    add((double)P[M * N * KB - 1]);
    const size_t pb = q8ref_packed_bytes(N, K);
    uint8_t *packed = xmalloc(pb);
    q8ref_pack(blocks, N, K, packed);
    add((double)packed[pb - 1]);
    free(x); free(xb); free(w); free(qa); free(qb); free(qw); free(da); free(db); free(dw);
    free(blocks); free(qw2); free(dw2); free(C); free(ad); free(P); free(packed);
}

static void swiglu_path(int64_t M, int64_t I) {
    double *G = xmalloc(sizeof(double) * M * I), *U = xmalloc(sizeof(double) * M * I);
    for (int64_t i = 0; i < M * I; ++i) { G[i] = 8.0 * uniform(); U[i] = 3.0 * uniform(); }
    G[0] = -800.0;   /* silu underflow side */
    double *h = xmalloc(sizeof(double) * M * I);
    int8_t *q = xmalloc((size_t)(M * I));
    uint16_t *d = xmalloc(sizeof(uint16_t) * M * (I / 32));
    q8ref_swiglu_quant(M, I, G, U, h, q, d);
    add(h[M * I - 1] + (double)q[0] + (double)d[0]);
    free(G); free(U); free(h); free(q); free(d);
}

static void kv3_path(int64_t R, int D) {
    const int64_t ld = D + 8;
    float *x = xmalloc(sizeof(float) * R * ld);
    uint16_t *xb = xmalloc(sizeof(uint16_t) * R * ld);
    for (int64_t i = 0; i < R * ld; ++i) { x[i] = (float)uniform(); xb[i] = bf16_of(x[i]); }
    for (int j = 0; j < D; ++j) x[j] = 0.0f;                       /* flat row */
    if (R > 1) x[ld] = 1e-40f;                                     /* subnormal row start */
    uint8_t *codes = xmalloc((size_t)(R * D * 3 / 8));
    float *scales = xmalloc(sizeof(float) * R), *out = xmalloc(sizeof(float) * R * D);
    q8ref_kv3_encode(x, 0, R, D, ld, codes, scales);
    q8ref_kv3_decode(codes, scales, R, D, out);
    add(out[R * D - 1]);
    q8ref_kv3_encode(xb, 1, R, D, ld, codes, scales);
    add(scales[R - 1]);
    float lv[8];
    q8ref_kv3_levels(lv);
    float *v = xmalloc(sizeof(float) * D);
    for (int j = 0; j < D; ++j) v[j] = (float)uniform();
    q8ref_fwht(v, D);
    add(v[D - 1] + lv[7]);
    free(x); free(xb); free(codes); free(scales); free(out); free(v);
}

static void attn_path(int64_t L, int64_t Hq, int64_t Hkv, int D, int k) {
    const int64_t NB = (L + 63) / 64, kmax = k + 2;
    const int64_t ldq = Hq * D + 8, ldk = Hkv * D + 8, ldv = Hkv * D;
    uint16_t *Q = xmalloc(sizeof(uint16_t) * L * ldq), *K = xmalloc(sizeof(uint16_t) * L * ldk);
    uint16_t *V = xmalloc(sizeof(uint16_t) * L * ldv);
    for (int64_t i = 0; i < L * ldq; ++i) Q[i] = bf16_of((float)uniform());
    for (int64_t i = 0; i < L * ldk; ++i) K[i] = bf16_of((float)uniform());
    for (int64_t i = 0; i < L * ldv; ++i) V[i] = bf16_of((float)uniform());
    double *pq = xmalloc(sizeof(double) * Hq * NB * D), *pk = xmalloc(sizeof(double) * Hkv * NB * D);
    q8ref_attn_pool(Q, L, ldq, Hq, D, pq);
    q8ref_attn_pool(K, L, ldk, Hkv, D, pk);
    int32_t *idx = xmalloc(sizeof(int32_t) * Hkv * NB * kmax), *cnt = xmalloc(sizeof(int32_t) * Hkv * NB);
    q8ref_attn_select(pq, pk, Hq, Hkv, NB, D, k, (int)kmax, idx, cnt);
    double *out = xmalloc(sizeof(double) * L * Hq * D), *mag = xmalloc(sizeof(double) * L * Hq * D);
    q8ref_attn_fwd(Q, K, V, L, ldq, ldk, ldv, Hq, Hkv, D, idx, cnt, (int)kmax, out, mag);
    add(out[L * Hq * D - 1] + mag[0]);
    int64_t tok[3] = {0, L - 1, L / 2}, head[3] = {Hq - 1, 0, Hq / 2};
    double o3[3 * 128], m3[3 * 128];
    q8ref_attn_fwd_at(Q, K, V, L, ldq, ldk, ldv, Hq, Hkv, D, idx, cnt, (int)kmax, tok, head, 3, o3, m3);
    add(o3[0] + m3[3 * D - 1]);
    free(Q); free(K); free(V); free(pq); free(pk); free(idx); free(cnt); free(out); free(mag);
}

int main(void) {
    gemm_path(3, 5, 64, 1);
    gemm_path(16, 70, 96, 0);
    gemm_path(1, 64, 32, 0);
    swiglu_path(2, 64);
    swiglu_path(3, 96);
    for (int D = 64; D <= 256; D *= 2) kv3_path(5, D);
    kv3_path(1, 128);
    attn_path(130, 4, 2, 64, 3);
    attn_path(64, 2, 1, 128, 2);
    attn_path(300, 3, 3, 64, 8);
    printf("ok %.6g\n", checksum);
    return 0;
}
