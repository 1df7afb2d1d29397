/* Drives the argument checks of every C-ABI entry point (include/q8.h) with
 * invalid arguments -- null pointers, bad shapes, misaligned pointers and
 * pitches, bad dtypes -- for a build of the library whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_abi_sanitizers.py).  Every call must return an error status
 * without touching device memory; the pointers passed are host buffers that
 * a check must reject before any HIP call.  Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "q8.h"

static int failures = 0;
static void expect_error(q8_status s, const char *what) {
    if (s == Q8_OK || (int)s < 0 || (int)s > (int)Q8_ERR_LAUNCH) {
        fprintf(stderr, "%s: status %d\n", what, (int)s);
        ++failures;
    }
}

int main(void) {
    /* 16-byte aligned host buffers, and one misaligned view */
    static _Alignas(16) uint8_t buf[1 << 16];
    void *p = buf, *odd = buf + 1;
    size_t bytes = 0;

    /* pack */
    expect_error(q8_pack_weights(NULL, 64, 64, p, &bytes, NULL), "pack null");
    expect_error(q8_pack_weights(p, 64, 63, p, &bytes, NULL), "pack K%32");
    expect_error(q8_pack_weights(p, 0, 64, p, &bytes, NULL), "pack N=0");
    expect_error(q8_pack_weights(p, 64, 64, p, NULL, NULL), "pack null size");
    bytes = 1;
    expect_error(q8_pack_weights(odd, 64, 64, p, &bytes, NULL), "pack small/misaligned");
    expect_error(q8_pack_weights_gateup(p, NULL, 64, 64, p, &bytes, NULL), "gateup null");
    expect_error(q8_pack_weights_gateup(p, p, 48, 64, p, &bytes, NULL), "gateup I%32");

    /* quantise */
    expect_error(q8_quantize_act(NULL, Q8_BF16, 4, 64, 64, (int8_t *)p, (uint16_t *)p, NULL), "quant null");
    expect_error(q8_quantize_act(p, (q8_dtype)7, 4, 64, 64, (int8_t *)p, (uint16_t *)p, NULL), "quant dtype");
    expect_error(q8_quantize_act(p, Q8_F32, 4, 64, 32, (int8_t *)p, (uint16_t *)p, NULL), "quant ldx<K");
    expect_error(q8_quantize_act(p, Q8_F32, -1, 64, 64, (int8_t *)p, (uint16_t *)p, NULL), "quant M<0");
    expect_error(q8_quantize_act(odd, Q8_F32, 4, 64, 64, (int8_t *)p, (uint16_t *)p, NULL), "quant align");

    /* products */
    expect_error(q8_gemm(4, 64, 64, NULL, (uint16_t *)p, p, (float *)p, 64, NULL), "gemm null");
    expect_error(q8_gemm(4, 64, 65, (int8_t *)p, (uint16_t *)p, p, (float *)p, 64, NULL), "gemm K");
    expect_error(q8_gemm(4, 64, 64, (int8_t *)p, (uint16_t *)p, p, (float *)p, 32, NULL), "gemm ldc");
    expect_error(q8_gemm(4, 64, 64, (int8_t *)odd, (uint16_t *)p, p, (float *)p, 64, NULL), "gemm align");
    expect_error(q8_gemm_act(p, (q8_dtype)5, 4, 64, 64, 64, p, (float *)p, 64, NULL, NULL, NULL), "gemm_act dtype");
    expect_error(q8_gemm_act(p, Q8_BF16, 4, 64, 64, 16, p, (float *)p, 64, NULL, NULL, NULL), "gemm_act ldx");
    expect_error(q8_gemm_swiglu(4, 48, 64, (int8_t *)p, (uint16_t *)p, p, (int8_t *)p, (uint16_t *)p, NULL), "swiglu I");
    expect_error(q8_gemm_swiglu(4, 64, 64, NULL, (uint16_t *)p, p, (int8_t *)p, (uint16_t *)p, NULL), "swiglu null");

    /* KV codec */
    expect_error(q8_kv3_encode(p, Q8_BF16, 4, 96, 96, (uint8_t *)p, (float *)p, NULL), "kv3 D");
    expect_error(q8_kv3_encode(NULL, Q8_BF16, 4, 128, 128, (uint8_t *)p, (float *)p, NULL), "kv3 null");
    expect_error(q8_kv3_encode(p, Q8_F32, 4, 128, 130, (uint8_t *)p, (float *)p, NULL), "kv3 pitch");
    expect_error(q8_kv3_decode((uint8_t *)p, (float *)p, 4, 128, (q8_dtype)9, p, 128, NULL), "kv3 dec dtype");
    expect_error(q8_kv3_decode((uint8_t *)p, NULL, 4, 128, Q8_F32, p, 128, NULL), "kv3 dec null");

    /* attention */
    expect_error(q8_attn_pool(p, 100, 64, 1, 96, (float *)p, NULL), "pool D");
    expect_error(q8_attn_pool(p, 100, 32, 1, 64, (float *)p, NULL), "pool ldx");
    expect_error(q8_attn_pool(NULL, 100, 64, 1, 64, (float *)p, NULL), "pool null");
    expect_error(q8_attn_select((float *)p, (float *)p, 3, 2, 4, 64, 2, 2, (int32_t *)p, (int32_t *)p, NULL), "select Hq%Hkv");
    expect_error(q8_attn_select((float *)p, (float *)p, 2, 1, 4, 64, 4, 2, (int32_t *)p, (int32_t *)p, NULL), "select kmax<k");
    expect_error(q8_attn_select((float *)p, (float *)p, 2, 1, 5000, 64, 4, 4, (int32_t *)p, (int32_t *)p, NULL), "select NB");
    expect_error(q8_attn_fwd(p, p, p, 100, 128, 64, 64, 2, 1, 64, (int32_t *)p, (int32_t *)p, 4, (q8_dtype)3, p, 128, NULL), "fwd dtype");
    expect_error(q8_attn_fwd(p, p, p, 100, 64, 64, 64, 2, 1, 64, (int32_t *)p, (int32_t *)p, 4, Q8_F32, p, 128, NULL), "fwd ldq");
    expect_error(q8_attn_fwd(p, p, NULL, 100, 128, 64, 64, 2, 1, 64, (int32_t *)p, (int32_t *)p, 4, Q8_F32, p, 128, NULL), "fwd null");
    expect_error(q8_attn_fwd(odd, p, p, 100, 128, 64, 64, 2, 1, 64, (int32_t *)p, (int32_t *)p, 4, Q8_F32, p, 128, NULL), "fwd align");

    /* every status has a description, out-of-range ones included */
    for (int s = -1; s <= (int)Q8_ERR_LAUNCH + 1; ++s)
        if (q8_status_string((q8_status)s) == NULL) {
            fprintf(stderr, "no string for %d\n", s);
            ++failures;
        }
    if (failures) return 1;
    printf("ok\n");
    return 0;
}
