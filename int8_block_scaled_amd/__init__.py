"""Python binding of libq8gemm: the Q8_0 weight x activation product on MI355X.

Argument marshalling only.  Every step runs in the HIP kernels of
``libq8gemm.so`` behind the C ABI of ``include/q8.h``; torch supplies device
memory and the current HIP stream.  There is no CPU fallback: if the library
is missing or the device is not gfx950 these functions raise.

The calls keep the C names:

* ``q8_pack_weights(w_blocks, N, K)``  GGUF Q8_0 blocks -> packed layout
* ``q8_quantize_act(x, K=None)``       fp32/bf16 rows -> (int8 q, fp16 d)
* ``q8_gemm(q_a, d_a, w_packed, N, K)``  C = A W^T in fp32
* ``q8_gemm_act(x, w_packed, N, K)``  quantise x on the fly, then C = A W^T
* ``q8_gemm_act_noalloc(x, w_packed, N, K)``  the same with a library-held workspace
* ``q8_pack_weights_gateup(w_gate, w_up, I, K)``  gate and up weights packed together
* ``q8_gemm_swiglu(q_a, d_a, w_packed, I, K)``  Q8_0(silu(A Wg^T) * (A Wu^T))
"""
import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8gemm.so")

Q8_F32, Q8_BF16 = 0, 1
STATUS = {0: "Q8_OK", 1: "Q8_ERR_NULL", 2: "Q8_ERR_SHAPE", 3: "Q8_ERR_ALIGN",
          4: "Q8_ERR_DTYPE", 5: "Q8_ERR_SIZE", 6: "Q8_ERR_DEVICE", 7: "Q8_ERR_LAUNCH"}
EXPORTS = ("q8_pack_weights", "q8_quantize_act", "q8_gemm", "q8_gemm_act", "q8_gemm_act_noalloc",
           "q8_pack_weights_gateup", "q8_gemm_swiglu", "q8_kv3_encode", "q8_kv3_decode",
           "q8_attn_pool", "q8_attn_select", "q8_attn_fwd", "q8_status_string")

_lib = None


class Q8Error(RuntimeError):
    def __init__(self, call, status):
        self.status = status
        msg = _load().q8_status_string(status).decode()
        super().__init__("%s failed: %s (%s)" % (call, STATUS.get(status, status), msg))


def _load():
    """Load libq8gemm.so (built by __graft_entry__.build() or
    int8_block_scaled_amd/build.py).  Raises if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libq8gemm.so is not built (%s); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.q8_pack_weights.argtypes = [vp, i64, i64, vp, ctypes.POINTER(sz), vp]
        L.q8_pack_weights.restype = ctypes.c_int
        L.q8_quantize_act.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp]
        L.q8_quantize_act.restype = ctypes.c_int
        L.q8_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, i64, vp]
        L.q8_gemm.restype = ctypes.c_int
        L.q8_gemm_act.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, i64, vp, vp, vp]
        L.q8_gemm_act.restype = ctypes.c_int
        L.q8_gemm_act_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64, vp, vp, i64, vp]
        L.q8_gemm_act_noalloc.restype = ctypes.c_int
        L.q8_pack_weights_gateup.argtypes = [vp, vp, i64, i64, vp, ctypes.POINTER(sz), vp]
        L.q8_pack_weights_gateup.restype = ctypes.c_int
        L.q8_gemm_swiglu.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.q8_gemm_swiglu.restype = ctypes.c_int
        L.q8_kv3_encode.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp]
        L.q8_kv3_encode.restype = ctypes.c_int
        L.q8_kv3_decode.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp, i64, vp]
        L.q8_kv3_decode.restype = ctypes.c_int
        L.q8_attn_pool.argtypes = [vp, i64, i64, i64, i64, vp, vp]
        L.q8_attn_pool.restype = ctypes.c_int
        L.q8_attn_select.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp, vp,
                                     vp]
        L.q8_attn_select.restype = ctypes.c_int
        L.q8_attn_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp, vp,
                                  ctypes.c_int, ctypes.c_int, vp, i64, vp]
        L.q8_attn_fwd.restype = ctypes.c_int
        L.q8_status_string.argtypes = [ctypes.c_int]
        L.q8_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def lib():
    return _load()


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check(call, st):
    if st != 0:
        raise Q8Error(call, st)


def _need_cuda(name, t):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)


@functools.lru_cache(maxsize=256)
def q8_packed_bytes(N: int, K: int) -> int:
    """Size of the packed weight buffer for an N x K weight."""
    n = ctypes.c_size_t(0)
    _check("q8_pack_weights", _load().q8_pack_weights(None, N, K, None, ctypes.byref(n), None))
    return n.value


def q8_pack_weights(w_blocks: torch.Tensor, N: int, K: int, out: torch.Tensor = None) -> torch.Tensor:
    """GGUF Q8_0 blocks (uint8, N*K/32*34 bytes, on the GPU) -> packed uint8."""
    _need_cuda("w_blocks", w_blocks)
    if w_blocks.dtype != torch.uint8 or not w_blocks.is_contiguous():
        raise TypeError("w_blocks must be contiguous uint8")
    if w_blocks.numel() != N * (K // 32) * 34:
        raise ValueError("w_blocks holds %d bytes, expected N*K/32*34 = %d"
                         % (w_blocks.numel(), N * (K // 32) * 34))
    need = q8_packed_bytes(N, K)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=w_blocks.device)
    n = ctypes.c_size_t(out.numel())
    _check("q8_pack_weights", _load().q8_pack_weights(
        _ptr(w_blocks), N, K, _ptr(out), ctypes.byref(n), _stream(w_blocks)))
    return out


def _act_dtype(x):
    if x.dtype == torch.float32:
        return Q8_F32
    if x.dtype == torch.bfloat16:
        return Q8_BF16
    raise TypeError("x must be float32 or bfloat16")


def _qd_out(q, d, M, K, device):
    """The quantised-row outputs: allocated when absent, else checked to be
    int8 [M][K] and float16 [M][K/32], contiguous, on the device."""
    if q is None:
        q = torch.empty((M, K), dtype=torch.int8, device=device)
    if d is None:
        d = torch.empty((M, K // 32), dtype=torch.float16, device=device)
    _need_cuda("q", q)
    _need_cuda("d", d)
    if q.dtype != torch.int8 or not q.is_contiguous() or tuple(q.shape) != (M, K):
        raise TypeError("q must be contiguous int8 [M][K]")
    if d.dtype not in (torch.float16, torch.int16) or not d.is_contiguous() \
            or tuple(d.shape) != (M, K // 32):
        raise TypeError("d must be contiguous float16 [M][K/32]")
    return q, d


def _row_length(x, K):
    """K defaults to the row length; a K beyond it would read past the rows."""
    K = x.shape[1] if K is None else K
    if K > x.shape[1]:
        raise ValueError("K=%d exceeds the row length %d of x" % (K, x.shape[1]))
    return K


def q8_quantize_act(x: torch.Tensor, K: int = None, q: torch.Tensor = None,
                    d: torch.Tensor = None):
    """Rows of x (float32 or bfloat16, [M][ldx], unit column stride) ->
    (q int8 [M][K], d float16 [M][K/32])."""
    _need_cuda("x", x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _act_dtype(x)
    M = x.shape[0]
    K = _row_length(x, K)
    ldx = x.stride(0) if M > 1 else max(x.stride(0), K)
    q, d = _qd_out(q, d, M, K, x.device)
    _check("q8_quantize_act", _load().q8_quantize_act(
        _ptr(x), dt, M, K, ldx, _ptr(q), _ptr(d), _stream(x)))
    return q, d


def q8_gemm(q_a: torch.Tensor, d_a: torch.Tensor, w_packed: torch.Tensor, N: int, K: int,
            out: torch.Tensor = None) -> torch.Tensor:
    """C[M][N] float32 = dequant(q_a, d_a) @ dequant(W)^T for packed W."""
    for name, t in (("q_a", q_a), ("d_a", d_a), ("w_packed", w_packed)):
        _need_cuda(name, t)
    if q_a.dtype != torch.int8 or not q_a.is_contiguous() or q_a.dim() != 2 or q_a.shape[1] != K:
        raise TypeError("q_a must be contiguous int8 [M][K]")
    if d_a.dtype not in (torch.float16, torch.int16) or not d_a.is_contiguous() \
            or tuple(d_a.shape) != (q_a.shape[0], K // 32):
        raise TypeError("d_a must be contiguous float16 [M][K/32]")
    if w_packed.numel() < q8_packed_bytes(N, K):
        raise ValueError("w_packed is smaller than the packed layout for N=%d K=%d" % (N, K))
    M = q_a.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=q_a.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1 or out.shape[1] < N \
            or out.shape[0] != M:
        raise TypeError("out must be float32 [M][>=N] with unit column stride")
    ldc = out.stride(0) if M > 1 else max(out.stride(0), N)
    _check("q8_gemm", _load().q8_gemm(M, N, K, _ptr(q_a), _ptr(d_a), _ptr(w_packed),
                                      _ptr(out), ldc, _stream(q_a)))
    return out


def q8_gemm_act(x: torch.Tensor, w_packed: torch.Tensor, N: int, K: int = None,
                out: torch.Tensor = None, q: torch.Tensor = None, d: torch.Tensor = None):
    """C[M][N] float32 for activation rows x (float32 or bfloat16, [M][ldx]),
    quantised on the fly.  q/d (int8 [M][K], float16 [M][K/32]) receive the
    quantised rows when given; for M > 8 they are allocated here if absent
    (the two kernels exchange the rows through them)."""
    _need_cuda("x", x)
    _need_cuda("w_packed", w_packed)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _act_dtype(x)
    M = x.shape[0]
    K = _row_length(x, K)
    ldx = x.stride(0) if M > 1 else max(x.stride(0), K)
    if w_packed.numel() < q8_packed_bytes(N, K):
        raise ValueError("w_packed is smaller than the packed layout for N=%d K=%d" % (N, K))
    if (q is None) != (d is None):
        raise ValueError("give both q and d, or neither")
    if q is not None or M > 8:
        q, d = _qd_out(q, d, M, K, x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1 or out.shape[1] < N \
            or out.shape[0] != M:
        raise TypeError("out must be float32 [M][>=N] with unit column stride")
    ldc = out.stride(0) if M > 1 else max(out.stride(0), N)
    qp = _ptr(q) if q is not None else None
    dp = _ptr(d) if d is not None else None
    _check("q8_gemm_act", _load().q8_gemm_act(_ptr(x), dt, M, N, K, ldx, _ptr(w_packed),
                                              _ptr(out), ldc, qp, dp, _stream(x)))
    return out


@functools.lru_cache(maxsize=256)
def q8_packed_bytes_gateup(I: int, K: int) -> int:
    """Size of the packed gate/up weight for I hidden units."""
    n = ctypes.c_size_t(0)
    _check("q8_pack_weights_gateup",
           _load().q8_pack_weights_gateup(None, None, I, K, None, ctypes.byref(n), None))
    return n.value


def q8_gemm_act_noalloc(x: torch.Tensor, w_packed: torch.Tensor, N: int, K: int = None,
                        out: torch.Tensor = None) -> torch.Tensor:
    """As q8_gemm_act, with the quantised rows in the library's static
    workspace (no device allocation by the library; `out` may be given so
    that the call allocates nothing at all)."""
    _need_cuda("x", x)
    _need_cuda("w_packed", w_packed)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _act_dtype(x)
    M = x.shape[0]
    K = _row_length(x, K)
    ldx = x.stride(0) if M > 1 else max(x.stride(0), K)
    if w_packed.numel() < q8_packed_bytes(N, K):
        raise ValueError("w_packed is smaller than the packed layout for N=%d K=%d" % (N, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or out.dim() != 2 or out.stride(1) != 1 or out.shape[1] < N \
            or out.shape[0] != M:
        raise TypeError("out must be float32 [M][>=N] with unit column stride")
    ldc = out.stride(0) if M > 1 else max(out.stride(0), N)
    _check("q8_gemm_act_noalloc", _load().q8_gemm_act_noalloc(
        _ptr(x), dt, M, N, K, ldx, _ptr(w_packed), _ptr(out), ldc, _stream(x)))
    return out


def q8_pack_weights_gateup(w_gate: torch.Tensor, w_up: torch.Tensor, I: int, K: int,
                           out: torch.Tensor = None) -> torch.Tensor:
    """GGUF Q8_0 blocks of the gate and up weights (uint8, I*K/32*34 bytes
    each, on the GPU) -> one packed uint8 buffer for q8_gemm_swiglu."""
    for name, t in (("w_gate", w_gate), ("w_up", w_up)):
        _need_cuda(name, t)
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise TypeError("%s must be contiguous uint8" % name)
        if t.numel() != I * (K // 32) * 34:
            raise ValueError("%s holds %d bytes, expected I*K/32*34 = %d"
                             % (name, t.numel(), I * (K // 32) * 34))
    need = q8_packed_bytes_gateup(I, K)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=w_gate.device)
    n = ctypes.c_size_t(out.numel())
    _check("q8_pack_weights_gateup", _load().q8_pack_weights_gateup(
        _ptr(w_gate), _ptr(w_up), I, K, _ptr(out), ctypes.byref(n), _stream(w_gate)))
    return out


def q8_gemm_swiglu(q_a: torch.Tensor, d_a: torch.Tensor, w_packed: torch.Tensor, I: int, K: int,
                   q: torch.Tensor = None, d: torch.Tensor = None):
    """(q_h int8 [M][I], d_h float16 [M][I/32]) = Q8_0 of silu(A Wg^T) * (A Wu^T)."""
    for name, t in (("q_a", q_a), ("d_a", d_a), ("w_packed", w_packed)):
        _need_cuda(name, t)
    if q_a.dtype != torch.int8 or not q_a.is_contiguous() or q_a.dim() != 2 or q_a.shape[1] != K:
        raise TypeError("q_a must be contiguous int8 [M][K]")
    if d_a.dtype not in (torch.float16, torch.int16) or not d_a.is_contiguous() \
            or tuple(d_a.shape) != (q_a.shape[0], K // 32):
        raise TypeError("d_a must be contiguous float16 [M][K/32]")
    if w_packed.numel() < q8_packed_bytes_gateup(I, K):
        raise ValueError("w_packed is smaller than the gate/up packed layout for I=%d K=%d" % (I, K))
    M = q_a.shape[0]
    if q is None:
        q = torch.empty((M, I), dtype=torch.int8, device=q_a.device)
    if d is None:
        d = torch.empty((M, I // 32), dtype=torch.float16, device=q_a.device)
    if q.dtype != torch.int8 or not q.is_contiguous() or tuple(q.shape) != (M, I):
        raise TypeError("q must be contiguous int8 [M][I]")
    if d.dtype not in (torch.float16, torch.int16) or not d.is_contiguous() \
            or tuple(d.shape) != (M, I // 32):
        raise TypeError("d must be contiguous float16 [M][I/32]")
    _check("q8_gemm_swiglu", _load().q8_gemm_swiglu(M, I, K, _ptr(q_a), _ptr(d_a), _ptr(w_packed),
                                                    _ptr(q), _ptr(d), _stream(q_a)))
    return q, d


def q8_kv3_encode(x: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """Rows of x (float32 or bfloat16, [R][ldx] with D = x.shape[1] in
    {64, 128, 256}, unit column stride) -> (codes uint8 [R][3D/8],
    scales float32 [R]): the 3-bit WHT + Lloyd-Max KV-cache format."""
    _need_cuda("x", x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _act_dtype(x)
    R, D = x.shape
    ldx = x.stride(0) if R > 1 else max(x.stride(0), D)
    if codes is None:
        codes = torch.empty((R, 3 * D // 8), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((R,), dtype=torch.float32, device=x.device)
    if codes.dtype != torch.uint8 or not codes.is_contiguous() or tuple(codes.shape) != (R, 3 * D // 8):
        raise TypeError("codes must be contiguous uint8 [R][3D/8]")
    if scales.dtype != torch.float32 or not scales.is_contiguous() or tuple(scales.shape) != (R,):
        raise TypeError("scales must be contiguous float32 [R]")
    _check("q8_kv3_encode", _load().q8_kv3_encode(
        _ptr(x), dt, R, D, ldx, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def q8_kv3_decode(codes: torch.Tensor, scales: torch.Tensor, D: int,
                  dtype: torch.dtype = torch.float32, out: torch.Tensor = None) -> torch.Tensor:
    """(codes [R][3D/8], scales [R]) from q8_kv3_encode -> rows [R][D] of
    dtype (float32 or bfloat16)."""
    for name, t in (("codes", codes), ("scales", scales)):
        _need_cuda(name, t)
    R = scales.shape[0] if scales.dim() == 1 else -1
    if codes.dtype != torch.uint8 or not codes.is_contiguous() or tuple(codes.shape) != (R, 3 * D // 8):
        raise TypeError("codes must be contiguous uint8 [R][3D/8]")
    if scales.dtype != torch.float32 or not scales.is_contiguous():
        raise TypeError("scales must be contiguous float32 [R]")
    if out is None:
        out = torch.empty((R, D), dtype=dtype, device=codes.device)
    odt = _act_dtype(out)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != R or out.shape[1] < D:
        raise TypeError("out must be [R][>=D] with unit column stride")
    ldo = out.stride(0) if R > 1 else max(out.stride(0), D)
    _check("q8_kv3_decode", _load().q8_kv3_decode(
        _ptr(codes), _ptr(scales), R, D, odt, _ptr(out), ldo, _stream(codes)))
    return out


def _bf16_rows(name, t):
    _need_cuda(name, t)
    if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
        raise TypeError("%s must be 2-D bfloat16 with unit column stride" % name)
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def q8_attn_pool(x: torch.Tensor, H: int, D: int, out: torch.Tensor = None) -> torch.Tensor:
    """Token-major bfloat16 rows x [L][>=H*D] -> pooled block means float32
    [H][ceil(L/64)][D]."""
    ldx = _bf16_rows("x", x)
    if x.shape[1] < H * D:
        raise ValueError("x rows hold %d values, fewer than H*D = %d" % (x.shape[1], H * D))
    L = x.shape[0]
    NB = (L + 63) // 64
    if out is None:
        out = torch.empty((H, NB, D), dtype=torch.float32, device=x.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (H, NB, D):
        raise TypeError("out must be contiguous float32 [H][NB][D]")
    _check("q8_attn_pool", _load().q8_attn_pool(_ptr(x), L, ldx, H, D, _ptr(out), _stream(x)))
    return out


def q8_attn_select(pooled_q: torch.Tensor, pooled_k: torch.Tensor, k: int, kmax: int = None,
                   idx: torch.Tensor = None, cnt: torch.Tensor = None):
    """Pooled rows [Hq][NB][D], [Hkv][NB][D] -> (idx int32 [Hkv][NB][kmax],
    cnt int32 [Hkv][NB]): the key blocks of every query block, per K/V head."""
    for name, t in (("pooled_q", pooled_q), ("pooled_k", pooled_k)):
        _need_cuda(name, t)
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 3:
            raise TypeError("%s must be contiguous float32 [H][NB][D]" % name)
    Hq, NB, D = pooled_q.shape
    Hkv = pooled_k.shape[0]
    if tuple(pooled_k.shape[1:]) != (NB, D):
        raise TypeError("pooled_k must be [Hkv][NB][D] with the NB and D of pooled_q")
    kmax = k if kmax is None else kmax
    if idx is None:
        idx = torch.empty((Hkv, NB, kmax), dtype=torch.int32, device=pooled_q.device)
    if cnt is None:
        cnt = torch.empty((Hkv, NB), dtype=torch.int32, device=pooled_q.device)
    for name, t, shape in (("idx", idx, (Hkv, NB, kmax)), ("cnt", cnt, (Hkv, NB))):
        _need_cuda(name, t)
        if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise TypeError("%s must be contiguous int32 %s" % (name, list(shape)))
    _check("q8_attn_select", _load().q8_attn_select(_ptr(pooled_q), _ptr(pooled_k), Hq, Hkv, NB, D,
                                                    k, kmax, _ptr(idx), _ptr(cnt),
                                                    _stream(pooled_q)))
    return idx, cnt


def q8_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, Hq: int, Hkv: int, D: int,
                idx: torch.Tensor, cnt: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                out: torch.Tensor = None) -> torch.Tensor:
    """Block-sparse causal attention over the listed key blocks (idx
    [Hkv][NB][kmax], cnt [Hkv][NB]): q [L][>=Hq*D], k, v [L][>=Hkv*D]
    bfloat16 -> out [L][Hq*D] (bfloat16 or float32)."""
    ldq, ldk, ldv = _bf16_rows("q", q), _bf16_rows("k", k), _bf16_rows("v", v)
    for name, t in (("idx", idx), ("cnt", cnt)):
        _need_cuda(name, t)
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("%s must be contiguous int32" % name)
    L = q.shape[0]
    for name, t, h in (("q", q, Hq), ("k", k, Hkv), ("v", v, Hkv)):
        if t.shape[0] < L or t.shape[1] < h * D:
            raise ValueError("%s must hold [L=%d][>=%d] values" % (name, L, h * D))
    NB = (L + 63) // 64
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (Hkv, NB) or tuple(cnt.shape) != (Hkv, NB):
        raise TypeError("idx must be [Hkv][NB][kmax] and cnt [Hkv][NB], NB = ceil(L/64)")
    if out is None:
        out = torch.empty((L, Hq * D), dtype=out_dtype, device=q.device)
    odt = _act_dtype(out)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != L or out.shape[1] < Hq * D:
        raise TypeError("out must be [L][>=Hq*D] with unit column stride")
    ldo = out.stride(0) if L > 1 else out.shape[1]
    _check("q8_attn_fwd", _load().q8_attn_fwd(_ptr(q), _ptr(k), _ptr(v), L, ldq, ldk, ldv, Hq, Hkv,
                                              D, _ptr(idx), _ptr(cnt), idx.shape[-1], odt,
                                              _ptr(out), ldo, _stream(q)))
    return out
