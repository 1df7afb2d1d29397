"""The C ABI without a GPU: the library loads, exports every function that
include/q8.h declares, and rejects bad arguments on the host before any HIP
call (so these paths run on a machine with no GPU at all)."""
import ctypes
import os
import re

import pytest

import int8_block_scaled_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8.h")

OK, NULL, SHAPE, ALIGN, DTYPE, SIZE = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return q8.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(q8.EXPORTS)
    for n in names:
        assert hasattr(L, n), "libq8gemm.so does not export %s" % n


def test_status_strings(L):
    for s in range(8):
        assert L.q8_status_string(s)
    assert L.q8_status_string(99) == b"unknown status"


def test_packed_size_query_matches_layout(orc):
    for N, K in [(1, 32), (64, 512), (70, 96), (12288, 4096), (17408, 5120)]:
        assert q8.q8_packed_bytes(N, K) == orc.packed_bytes(N, K)
    assert q8.q8_packed_bytes(12288, 4096) == 12288 * 4096 * 34 // 32


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: checks fail first
ODD = ctypes.c_void_p(0x10001)


def test_pack_validation(L):
    n = ctypes.c_size_t(1 << 40)
    assert L.q8_pack_weights(FAKE, 64, 512, FAKE, None, None) == NULL
    assert L.q8_pack_weights(FAKE, 0, 512, FAKE, ctypes.byref(n), None) == SHAPE
    assert L.q8_pack_weights(FAKE, 64, 48, FAKE, ctypes.byref(n), None) == SHAPE
    assert L.q8_pack_weights(FAKE, 64, 0, FAKE, ctypes.byref(n), None) == SHAPE
    assert L.q8_pack_weights(None, 64, 512, FAKE, ctypes.byref(n), None) == NULL
    assert L.q8_pack_weights(FAKE, 64, 512, ODD, ctypes.byref(n), None) == ALIGN
    small = ctypes.c_size_t(100)
    assert L.q8_pack_weights(FAKE, 64, 512, FAKE, ctypes.byref(small), None) == SIZE


def test_quantize_validation(L):
    assert L.q8_quantize_act(FAKE, 2, 4, 64, 64, FAKE, FAKE, None) == DTYPE
    assert L.q8_quantize_act(FAKE, 0, -1, 64, 64, FAKE, FAKE, None) == SHAPE
    assert L.q8_quantize_act(FAKE, 0, 4, 48, 64, FAKE, FAKE, None) == SHAPE
    assert L.q8_quantize_act(FAKE, 0, 4, 64, 32, FAKE, FAKE, None) == SHAPE   # ldx < K
    assert L.q8_quantize_act(None, 0, 0, 64, 64, None, None, None) == OK      # M == 0: no-op
    assert L.q8_quantize_act(None, 0, 4, 64, 64, FAKE, FAKE, None) == NULL
    assert L.q8_quantize_act(ODD, 0, 4, 64, 64, FAKE, FAKE, None) == ALIGN
    assert L.q8_quantize_act(FAKE, 0, 4, 64, 66, FAKE, FAKE, None) == ALIGN   # pitch 264 B
    assert L.q8_quantize_act(FAKE, 1, 4, 64, 68, FAKE, FAKE, None) == ALIGN   # pitch 136 B
    assert L.q8_quantize_act(FAKE, 0, 4, 64, 64, ODD, FAKE, None) == ALIGN
    assert L.q8_quantize_act(FAKE, 0, 4, 64, 64, FAKE, ODD, None) == ALIGN


def test_gemm_validation(L):
    assert L.q8_gemm(-1, 64, 64, FAKE, FAKE, FAKE, FAKE, 64, None) == SHAPE
    assert L.q8_gemm(4, 0, 64, FAKE, FAKE, FAKE, FAKE, 64, None) == SHAPE
    assert L.q8_gemm(4, 64, 65, FAKE, FAKE, FAKE, FAKE, 64, None) == SHAPE
    assert L.q8_gemm(4, 64, 64, FAKE, FAKE, FAKE, FAKE, 63, None) == SHAPE   # ldc < N
    assert L.q8_gemm(0, 64, 64, None, None, None, None, 64, None) == OK      # M == 0: no-op
    assert L.q8_gemm(4, 64, 64, None, FAKE, FAKE, FAKE, 64, None) == NULL
    assert L.q8_gemm(4, 64, 64, FAKE, None, FAKE, FAKE, 64, None) == NULL
    assert L.q8_gemm(4, 64, 64, FAKE, FAKE, None, FAKE, 64, None) == NULL
    assert L.q8_gemm(4, 64, 64, FAKE, FAKE, FAKE, None, 64, None) == NULL
    assert L.q8_gemm(4, 64, 64, ODD, FAKE, FAKE, FAKE, 64, None) == ALIGN
    assert L.q8_gemm(4, 64, 64, FAKE, ODD, FAKE, FAKE, 64, None) == ALIGN
    assert L.q8_gemm(4, 64, 64, FAKE, FAKE, ODD, FAKE, 64, None) == ALIGN
    assert L.q8_gemm(4, 64, 64, FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), 64, None) == ALIGN


def test_gemm_act_validation(L):
    f = L.q8_gemm_act
    #        x     dt  M   N   K   ldx  w     C     ldc  q     d
    assert f(FAKE, 2, 4, 64, 64, 64, FAKE, FAKE, 64, None, None, None) == DTYPE
    assert f(FAKE, 0, -1, 64, 64, 64, FAKE, FAKE, 64, None, None, None) == SHAPE
    assert f(FAKE, 0, 4, 0, 64, 64, FAKE, FAKE, 64, None, None, None) == SHAPE
    assert f(FAKE, 0, 4, 64, 48, 64, FAKE, FAKE, 64, None, None, None) == SHAPE
    assert f(FAKE, 0, 4, 64, 64, 32, FAKE, FAKE, 64, None, None, None) == SHAPE      # ldx < K
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, FAKE, 63, None, None, None) == SHAPE      # ldc < N
    assert f(None, 0, 0, 64, 64, 64, None, None, 64, None, None, None) == OK         # M == 0
    assert f(None, 0, 4, 64, 64, 64, FAKE, FAKE, 64, None, None, None) == NULL
    assert f(FAKE, 0, 4, 64, 64, 64, None, FAKE, 64, None, None, None) == NULL
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, None, 64, None, None, None) == NULL
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, FAKE, 64, FAKE, None, None) == NULL       # q without d
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, FAKE, 64, None, FAKE, None) == NULL       # d without q
    assert f(FAKE, 0, 9, 64, 64, 64, FAKE, FAKE, 64, None, None, None) == NULL       # M > 8 needs q, d
    assert f(ODD, 0, 4, 64, 64, 64, FAKE, FAKE, 64, None, None, None) == ALIGN
    assert f(FAKE, 0, 4, 64, 64, 66, FAKE, FAKE, 64, None, None, None) == ALIGN      # pitch 264 B
    assert f(FAKE, 0, 4, 64, 64, 64, ODD, FAKE, 64, None, None, None) == ALIGN
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, ctypes.c_void_p(0x10002), 64, None, None, None) == ALIGN
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, FAKE, 64, ODD, FAKE, None) == ALIGN
    assert f(FAKE, 0, 4, 64, 64, 64, FAKE, FAKE, 64, FAKE, ODD, None) == ALIGN


def test_gateup_pack_validation(L, orc):
    n = ctypes.c_size_t(0)
    assert L.q8_pack_weights_gateup(None, None, 64, 512, None, ctypes.byref(n), None) == OK
    assert n.value == orc.packed_bytes(128, 512) == q8.q8_packed_bytes_gateup(64, 512)
    big = ctypes.c_size_t(1 << 40)
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 64, 512, FAKE, None, None) == NULL
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 48, 512, FAKE, ctypes.byref(big), None) == SHAPE
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 0, 512, FAKE, ctypes.byref(big), None) == SHAPE
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 64, 48, FAKE, ctypes.byref(big), None) == SHAPE
    assert L.q8_pack_weights_gateup(None, FAKE, 64, 512, FAKE, ctypes.byref(big), None) == NULL
    assert L.q8_pack_weights_gateup(FAKE, None, 64, 512, FAKE, ctypes.byref(big), None) == NULL
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 64, 512, ODD, ctypes.byref(big), None) == ALIGN
    small = ctypes.c_size_t(100)
    assert L.q8_pack_weights_gateup(FAKE, FAKE, 64, 512, FAKE, ctypes.byref(small), None) == SIZE


def test_gemm_swiglu_validation(L):
    f = L.q8_gemm_swiglu
    #        M   I   K    qa    da    w     qh    dh
    assert f(-1, 64, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(4, 48, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(4, 16, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(4, 64, 65, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(0, 64, 64, None, None, None, None, None, None) == OK      # M == 0: no-op
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        assert f(4, 64, 64, *args, None) == NULL
    assert f(4, 64, 64, ODD, FAKE, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(4, 64, 64, FAKE, ODD, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(4, 64, 64, FAKE, FAKE, ODD, FAKE, FAKE, None) == ALIGN
    assert f(4, 64, 64, FAKE, FAKE, FAKE, ODD, FAKE, None) == ALIGN
    assert f(4, 64, 64, FAKE, FAKE, FAKE, FAKE, ODD, None) == ALIGN


def test_kv3_encode_validation(L):
    f = L.q8_kv3_encode
    #        x   dtype R   D    ldx  codes scales
    assert f(FAKE, 2, 8, 128, 128, FAKE, FAKE, None) == DTYPE
    for D in (0, 32, 96, 192, 512):
        assert f(FAKE, 0, 8, D, 512, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 0, -1, 128, 128, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 0, 8, 128, 120, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 0, 1 << 34, 128, 128, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 0, 8, 128, 1 << 23, FAKE, FAKE, None) == SHAPE    # pitch 32 MiB
    assert f(FAKE, 1, 8, 128, 1 << 24, FAKE, FAKE, None) == SHAPE
    assert f(None, 0, 0, 128, 128, None, None, None) == OK        # R == 0: no-op
    for i in (0, 5, 6):
        args = [FAKE, 0, 8, 128, 128, FAKE, FAKE]
        args[i] = None
        assert f(*args, None) == NULL
    assert f(ODD, 0, 8, 128, 128, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 0, 8, 128, 130, FAKE, FAKE, None) == ALIGN      # 520-byte pitch
    assert f(FAKE, 1, 8, 128, 132, FAKE, FAKE, None) == ALIGN      # 264-byte pitch
    assert f(FAKE, 0, 8, 128, 128, FAKE, ODD, None) == ALIGN
    assert f(FAKE, 0, 8, 128, 128, ctypes.c_void_p(0x10008), FAKE, None) == ALIGN


def test_kv3_decode_validation(L):
    f = L.q8_kv3_decode
    #        codes scales R  D  dtype out  ldo
    assert f(FAKE, FAKE, 8, 128, 7, FAKE, 128, None) == DTYPE
    for D in (0, 16, 100, 512):
        assert f(FAKE, FAKE, 8, D, 0, FAKE, 512, None) == SHAPE
    assert f(FAKE, FAKE, -2, 128, 0, FAKE, 128, None) == SHAPE
    assert f(FAKE, FAKE, 8, 256, 0, FAKE, 128, None) == SHAPE
    assert f(FAKE, FAKE, 8, 128, 0, FAKE, 1 << 23, None) == SHAPE
    assert f(None, None, 0, 64, 0, None, 64, None) == OK
    for i in (0, 1, 5):
        args = [FAKE, FAKE, 8, 128, 0, FAKE, 128]
        args[i] = None
        assert f(*args, None) == NULL
    assert f(FAKE, FAKE, 8, 128, 0, ODD, 128, None) == ALIGN
    assert f(FAKE, FAKE, 8, 128, 1, FAKE, 132, None) == ALIGN
    assert f(FAKE, ODD, 8, 128, 0, FAKE, 128, None) == ALIGN
    assert f(ctypes.c_void_p(0x10004), FAKE, 8, 128, 0, FAKE, 128, None) == ALIGN


def test_attn_pool_validation(L):
    f = L.q8_attn_pool
    #          x   L    ldx  H  D   pooled
    assert f(FAKE, 100, 512, 5, 128, FAKE, None) == SHAPE          # ldx < H*D
    assert f(FAKE, 100, 512, 4, 96, FAKE, None) == SHAPE           # D not 64/128
    assert f(FAKE, -1, 512, 4, 64, FAKE, None) == SHAPE
    assert f(FAKE, 64 * 4097, 512, 4, 64, FAKE, None) == SHAPE     # > 4096 blocks
    assert f(None, 0, 512, 4, 64, None, None) == OK                # L == 0
    assert f(None, 100, 512, 4, 64, FAKE, None) == NULL
    assert f(ODD, 100, 512, 4, 64, FAKE, None) == ALIGN
    assert f(FAKE, 100, 516, 4, 64, FAKE, None) == ALIGN           # 1032-byte pitch
    assert f(FAKE, 100, 512, 4, 64, ctypes.c_void_p(0x10008), None) == ALIGN


def test_attn_select_validation(L):
    f = L.q8_attn_select
    #         pq    pk   Hq Hkv NB   D   k  kmax idx  cnt
    assert f(FAKE, FAKE, 6, 4, 10, 128, 4, 4, FAKE, FAKE, None) == SHAPE   # Hq % Hkv
    assert f(FAKE, FAKE, 4, 2, 10, 128, 1, 4, FAKE, FAKE, None) == SHAPE   # k < 2
    assert f(FAKE, FAKE, 4, 2, 10, 128, 5, 4, FAKE, FAKE, None) == SHAPE   # kmax < k
    assert f(FAKE, FAKE, 4, 2, 4097, 128, 4, 4, FAKE, FAKE, None) == SHAPE
    assert f(None, None, 4, 2, 0, 128, 4, 4, None, None, None) == OK
    for i in range(4):
        args = [FAKE, FAKE, 4, 2, 10, 128, 4, 4, FAKE, FAKE]
        args[[0, 1, 8, 9][i]] = None
        assert f(*args, None) == NULL
    assert f(ODD, FAKE, 4, 2, 10, 128, 4, 4, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, FAKE, 4, 2, 10, 128, 4, 4, FAKE, ODD, None) == ALIGN


def test_attn_fwd_validation(L):
    f = L.q8_attn_fwd
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, L=100, ldq=512, ldk=256, ldv=256, Hq=4, Hkv=2, D=128,
                 idx=FAKE, cnt=FAKE, kmax=4, dt=1, out=FAKE, ldo=512)
        a.update(kw)
        return f(a["q"], a["k"], a["v"], a["L"], a["ldq"], a["ldk"], a["ldv"], a["Hq"], a["Hkv"],
                 a["D"], a["idx"], a["cnt"], a["kmax"], a["dt"], a["out"], a["ldo"], None)
    assert call(dt=3) == DTYPE
    assert call(Hkv=3) == SHAPE
    assert call(D=256, ldq=1024, ldk=512, ldv=512, ldo=1024) == SHAPE
    assert call(ldq=500) == SHAPE and call(ldk=200) == SHAPE and call(ldo=256) == SHAPE
    assert call(kmax=0) == SHAPE
    assert call(L=64 * 4096 + 1) == SHAPE
    assert call(ldq=1 << 24) == SHAPE
    assert call(q=None, L=0) == OK
    for name in ("q", "k", "v", "idx", "cnt", "out"):
        assert call(**{name: None}) == NULL
    assert call(q=ODD) == ALIGN and call(v=ctypes.c_void_p(0x10008)) == ALIGN
    assert call(ldq=516) == ALIGN
    assert call(dt=0, out=ctypes.c_void_p(0x10008)) == ALIGN        # fp32 out needs 16
    # (a bf16 output at an 8-byte-aligned address passes every argument check:
    # covered, with no device to launch on, by test_device_error.py)
    assert call(dt=1, ldo=514) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        q8.q8_quantize_act(torch.zeros(4, 64))
    with pytest.raises(TypeError):
        q8.q8_kv3_encode(torch.zeros(4, 128))
