"""CPU oracle for the Q8_0 weight x activation product (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The library under
``int8_block_scaled_amd/`` never imports it and shares no code with it; the
two meet only through the seeded inputs of ``workloads.py``.

The arithmetic lives in ``q8ref.c`` (plain C loops, see its header for the
definition followed and the source it is read from); this module marshals
numpy arrays.  ``exact.py`` holds a rational-arithmetic brute force used to
pin the C code on tiny shapes.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))


def _bind(L):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.q8ref_f32_to_f16.argtypes = [ctypes.c_float]
    L.q8ref_f32_to_f16.restype = ctypes.c_uint16
    L.q8ref_f32_to_f16_array.argtypes = [vp, i64, vp]
    L.q8ref_f32_to_f16_array.restype = None
    L.q8ref_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.q8ref_f16_to_f64.restype = ctypes.c_double
    L.q8ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.q8ref_bf16_to_f32.restype = ctypes.c_float
    L.q8ref_quantize_block.argtypes = [vp, vp, vp]
    L.q8ref_quantize_block.restype = ctypes.c_int
    L.q8ref_quantize_rows.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp]
    L.q8ref_quantize_rows.restype = i64
    L.q8ref_blocks_from_qd.argtypes = [vp, vp, i64, i64, vp]
    L.q8ref_blocks_from_qd.restype = None
    L.q8ref_qd_from_blocks.argtypes = [vp, i64, i64, vp, vp]
    L.q8ref_qd_from_blocks.restype = None
    L.q8ref_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.q8ref_gemm.restype = None
    L.q8ref_gemm_sampled.argtypes = [i64, vp, vp, vp, vp, vp, vp, i64, vp, vp]
    L.q8ref_gemm_sampled.restype = None
    L.q8ref_block_dots.argtypes = [i64, i64, i64, vp, vp, vp]
    L.q8ref_block_dots.restype = None
    L.q8ref_packed_bytes.argtypes = [i64, i64]
    L.q8ref_packed_bytes.restype = ctypes.c_size_t
    L.q8ref_pack.argtypes = [vp, i64, i64, vp]
    L.q8ref_pack.restype = None
    L.q8ref_silu.argtypes = [ctypes.c_double]
    L.q8ref_silu.restype = ctypes.c_double
    L.q8ref_swiglu_quant.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    L.q8ref_swiglu_quant.restype = None
    L.q8ref_kv3_levels.argtypes = [vp]
    L.q8ref_kv3_levels.restype = None
    L.q8ref_fwht.argtypes = [vp, ctypes.c_int]
    L.q8ref_fwht.restype = None
    L.q8ref_kv3_encode.argtypes = [vp, ctypes.c_int, i64, ctypes.c_int, i64, vp, vp]
    L.q8ref_kv3_encode.restype = None
    L.q8ref_kv3_decode.argtypes = [vp, vp, i64, ctypes.c_int, vp]
    L.q8ref_kv3_decode.restype = None
    L.q8ref_attn_pool.argtypes = [vp, i64, i64, i64, ctypes.c_int, vp]
    L.q8ref_attn_pool.restype = None
    L.q8ref_attn_select.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, vp, vp]
    L.q8ref_attn_select.restype = None
    L.q8ref_attn_fwd.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, vp, vp,
                                 ctypes.c_int, vp, vp]
    L.q8ref_attn_fwd.restype = None
    L.q8ref_attn_fwd_at.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_int, vp,
                                    vp, ctypes.c_int, vp, vp, i64, vp, vp]
    L.q8ref_attn_fwd_at.restype = None
    L.q8ref_num_threads.argtypes = []
    L.q8ref_num_threads.restype = ctypes.c_int
    return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """The oracle's entry points over one loaded build of q8ref.c.  The
    module-level functions use the default build; tests can load another
    build (for instance one with a planted mistake) as ``Oracle(path)``."""

    def __init__(self, path):
        self.path = path
        self.L = _bind(ctypes.CDLL(path))

    def f32_to_f16_bits(self, x) -> np.ndarray:
        """binary32 -> binary16 bits (round to nearest even), elementwise."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.L.q8ref_f32_to_f16_array(_p(x), x.size, _p(out))
        return out

    def f16_bits_to_f64(self, h) -> np.ndarray:
        h = np.asarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float64)
        fi, fo = h.reshape(-1), out.reshape(-1)
        for i in range(fi.size):
            fo[i] = self.L.q8ref_f16_to_f64(int(fi[i]))
        return out

    def quantize_block(self, x):
        """One 32-value block -> (q int8[32], d binary16 bits, status)."""
        x = _c(x, np.float32)
        assert x.shape == (32,)
        q = np.empty(32, dtype=np.int8)
        d = np.empty(1, dtype=np.uint16)
        st = self.L.q8ref_quantize_block(_p(x), _p(q), _p(d))
        return q, int(d[0]), st

    def quantize_rows(self, x, K=None, ldx=None):
        """Quantise rows of ``x`` ([M][>=K] float32, or uint16 holding bfloat16
        bits) -> (q int8 [M][K], d uint16 [M][K/32])."""
        if x.dtype == np.float32:
            dtype = 0
        elif x.dtype == np.uint16:
            dtype = 1
        else:
            raise TypeError("x must be float32 or uint16 (bfloat16 bits)")
        x = np.ascontiguousarray(x)
        M = x.shape[0]
        ldx = x.shape[1] if ldx is None else ldx
        K = ldx if K is None else K
        assert K % 32 == 0 and K <= ldx
        q = np.empty((M, K), dtype=np.int8)
        d = np.empty((M, K // 32), dtype=np.uint16)
        bad = self.L.q8ref_quantize_rows(_p(x), dtype, M, K, ldx, _p(q), _p(d))
        if bad:
            raise ValueError("%d blocks failed the |q| <= 127 self-check" % bad)
        return q, d

    def blocks_from_qd(self, q, d) -> np.ndarray:
        """Separate (q [N][K], d [N][K/32]) -> GGUF Q8_0 bytes [N][K/32*34]."""
        q, d = _c(q, np.int8), _c(d, np.uint16)
        N, K = q.shape
        out = np.empty((N, K // 32 * 34), dtype=np.uint8)
        self.L.q8ref_blocks_from_qd(_p(q), _p(d), N, K, _p(out))
        return out

    def qd_from_blocks(self, blocks, N, K):
        blocks = _c(blocks, np.uint8)
        q = np.empty((N, K), dtype=np.int8)
        d = np.empty((N, K // 32), dtype=np.uint16)
        self.L.q8ref_qd_from_blocks(_p(blocks), N, K, _p(q), _p(d))
        return q, d

    def gemm(self, q_a, d_a, q_w, d_w):
        """Full product in double: returns (C [M][N], absdot [M][N])."""
        q_a, d_a = _c(q_a, np.int8), _c(d_a, np.uint16)
        q_w, d_w = _c(q_w, np.int8), _c(d_w, np.uint16)
        M, K = q_a.shape
        N = q_w.shape[0]
        C = np.empty((M, N), dtype=np.float64)
        A = np.empty((M, N), dtype=np.float64)
        self.L.q8ref_gemm(M, N, K, _p(q_a), _p(d_a), _p(q_w), _p(d_w), _p(C), _p(A))
        return C, A

    def gemm_sampled(self, q_a, d_a, q_w, d_w, rows, cols):
        """Selected outputs C[rows[i], cols[i]] and their abs-dots, in double."""
        q_a, d_a = _c(q_a, np.int8), _c(d_a, np.uint16)
        q_w, d_w = _c(q_w, np.int8), _c(d_w, np.uint16)
        rows, cols = _c(rows, np.int64), _c(cols, np.int64)
        K = q_a.shape[1]
        C = np.empty(rows.size, dtype=np.float64)
        A = np.empty(rows.size, dtype=np.float64)
        self.L.q8ref_gemm_sampled(K, _p(q_a), _p(d_a), _p(q_w), _p(d_w), _p(rows), _p(cols),
                                  rows.size, _p(C), _p(A))
        return C, A

    def block_dots(self, q_a, q_w):
        """Exact int32 block dots P [M][N][K/32]."""
        q_a, q_w = _c(q_a, np.int8), _c(q_w, np.int8)
        M, K = q_a.shape
        N = q_w.shape[0]
        P = np.empty((M, N, K // 32), dtype=np.int32)
        self.L.q8ref_block_dots(M, N, K, _p(q_a), _p(q_w), _p(P))
        return P

    def packed_bytes(self, N, K) -> int:
        return int(self.L.q8ref_packed_bytes(N, K))

    def pack(self, blocks, N, K) -> np.ndarray:
        """GGUF Q8_0 bytes [N][K/32*34] -> the library's packed layout (bytes)."""
        blocks = _c(blocks, np.uint8)
        out = np.empty(self.packed_bytes(N, K), dtype=np.uint8)
        self.L.q8ref_pack(_p(blocks), N, K, _p(out))
        return out

    def silu(self, x: float) -> float:
        return float(self.L.q8ref_silu(float(x)))

    def swiglu_quant(self, G, U):
        """Gate and up products G, U ([M][I] float64) -> (h float64 [M][I],
        q int8 [M][I], d uint16 [M][I/32]): h = silu(G)*U, quantised per 32
        along I."""
        G, U = _c(G, np.float64), _c(U, np.float64)
        M, I = G.shape
        assert U.shape == (M, I) and I % 32 == 0
        h = np.empty((M, I), dtype=np.float64)
        q = np.empty((M, I), dtype=np.int8)
        d = np.empty((M, I // 32), dtype=np.uint16)
        self.L.q8ref_swiglu_quant(M, I, _p(G), _p(U), _p(h), _p(q), _p(d))
        return h, q, d

    @staticmethod
    def interleave_gateup(gate_rows, up_rows):
        """Rows of the gate and up weights ([I][...] each, I % 32 == 0) ->
        [2I][...] in the order of the gate/up packed layout: 64-row group g
        holds gate rows 32g..32g+31, then up rows 32g..32g+31."""
        gate_rows, up_rows = np.asarray(gate_rows), np.asarray(up_rows)
        I = gate_rows.shape[0]
        assert up_rows.shape == gate_rows.shape and I % 32 == 0
        rest = gate_rows.shape[1:]
        g = gate_rows.reshape((I // 32, 32) + rest)
        u = up_rows.reshape((I // 32, 32) + rest)
        return np.ascontiguousarray(np.concatenate([g, u], axis=1).reshape((2 * I,) + rest))

    def pack_gateup(self, gate_blocks, up_blocks, I, K) -> np.ndarray:
        """GGUF Q8_0 bytes of the gate and up weights ([I][K/32*34] each) ->
        the packed layout of their interleaved rows (2I rows)."""
        return self.pack(self.interleave_gateup(gate_blocks, up_blocks), 2 * I, K)

    # ---- 3-bit KV-cache codec -------------------------------------------

    def kv3_levels(self) -> np.ndarray:
        out = np.empty(8, dtype=np.float32)
        self.L.q8ref_kv3_levels(_p(out))
        return out

    def fwht(self, v) -> np.ndarray:
        """Unnormalised Walsh-Hadamard transform of one binary32 vector."""
        v = np.array(v, dtype=np.float32, copy=True)
        self.L.q8ref_fwht(_p(v), v.size)
        return v

    def kv3_encode(self, x, D=None):
        """Rows of x ([R][>=D] float32, or uint16 bfloat16 bits) ->
        (codes uint8 [R][3D/8], scales float32 [R])."""
        dtype = 1 if x.dtype == np.uint16 else 0
        x = _c(x, np.uint16 if dtype else np.float32)
        R, ldx = x.shape
        D = ldx if D is None else D
        assert D in (64, 128, 256) and D <= ldx
        codes = np.empty((R, 3 * D // 8), dtype=np.uint8)
        scales = np.empty(R, dtype=np.float32)
        self.L.q8ref_kv3_encode(_p(x), dtype, R, D, ldx, _p(codes), _p(scales))
        return codes, scales

    def kv3_decode(self, codes, scales, D) -> np.ndarray:
        codes, scales = _c(codes, np.uint8), _c(scales, np.float32)
        R = codes.shape[0]
        out = np.empty((R, D), dtype=np.float32)
        self.L.q8ref_kv3_decode(_p(codes), _p(scales), R, D, _p(out))
        return out

    # -- block-sparse causal attention (64-token blocks) -------------------
    ATTN_BLK = 64

    def attn_pool(self, x, H, D):
        """x: [L][>=H*D] uint16 bfloat16 bits, token-major -> pooled
        [H][NB][D] float64, the mean of each 64-token block (the last block
        may be shorter)."""
        x = _c(x, np.uint16)
        L, ldx = x.shape
        NB = (L + 63) // 64
        out = np.empty((H, NB, D), dtype=np.float64)
        self.L.q8ref_attn_pool(_p(x), L, ldx, H, D, _p(out))
        return out

    def attn_select(self, pq, pk, k, kmax=None):
        """Pooled rows ([Hq][NB][D], [Hkv][NB][D]) -> (idx int32
        [Hkv][NB][kmax], cnt int32 [Hkv][NB]): per K/V head, block 0, the
        diagonal block and the others scoring highest against the sum of the
        group's pooled query rows, ascending, -1 past cnt."""
        pq, pk = _c(pq, np.float64), _c(pk, np.float64)
        Hq, NB, D = pq.shape
        Hkv = pk.shape[0]
        kmax = k if kmax is None else kmax
        idx = np.empty((Hkv, NB, kmax), dtype=np.int32)
        cnt = np.empty((Hkv, NB), dtype=np.int32)
        self.L.q8ref_attn_select(_p(pq), _p(pk), Hq, Hkv, NB, D, k, kmax, _p(idx), _p(cnt))
        return idx, cnt

    def attn_fwd(self, q, k, v, Hq, Hkv, D, idx, cnt):
        """q [L][>=Hq*D], k, v [L][>=Hkv*D] uint16 bfloat16 bits; idx/cnt as
        from attn_select -> (out, mag) float64 [L][Hq*D]."""
        q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
        idx, cnt = _c(idx, np.int32), _c(cnt, np.int32)
        L = q.shape[0]
        out = np.empty((L, Hq * D), dtype=np.float64)
        mag = np.empty((L, Hq * D), dtype=np.float64)
        self.L.q8ref_attn_fwd(_p(q), _p(k), _p(v), L, q.shape[1], k.shape[1], v.shape[1], Hq, Hkv,
                              D, _p(idx), _p(cnt), idx.shape[2], _p(out), _p(mag))
        return out, mag

    def attn_fwd_at(self, q, k, v, Hq, Hkv, D, idx, cnt, tok, head):
        """attn_fwd at chosen (token, head) pairs -> (out, mag) [n][D]."""
        q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
        idx, cnt = _c(idx, np.int32), _c(cnt, np.int32)
        tok, head = _c(tok, np.int64), _c(head, np.int64)
        n = tok.size
        out = np.empty((n, D), dtype=np.float64)
        mag = np.empty((n, D), dtype=np.float64)
        self.L.q8ref_attn_fwd_at(_p(q), _p(k), _p(v), q.shape[0], q.shape[1], k.shape[1],
                                 v.shape[1], Hq, Hkv, D, _p(idx), _p(cnt), idx.shape[2],
                                 _p(tok), _p(head), n, _p(out), _p(mag))
        return out, mag

    def num_threads(self) -> int:
        return int(self.L.q8ref_num_threads())


_default = None


def default() -> Oracle:
    """The oracle built from oracle/q8ref.c (built with gcc if missing)."""
    global _default
    if _default is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _default = Oracle(path)
    return _default


def __getattr__(name):
    # module-level access to the default build's methods: oracle.gemm(...)
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
