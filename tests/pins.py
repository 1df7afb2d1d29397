"""Pins for the CPU oracle: checks against what the definition and the
mathematics fix, independent of the oracle's own code.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them on the oracle as built;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires every mutant to fail at least one pin.

What pins what:
* binary16 encoding   -- numpy's float16 cast (IEEE round to nearest even)
                         and the exhaustive round trip of every binary16;
* block quantiser     -- hand-derived cases (tests/golden), an exact
                         rational re-derivation of each binary32 step
                         (oracle/exact.py), and invariants of the format;
* block integer dots  -- numpy int64 products;
* the product         -- hand-derived cases, an exact rational
                         dequantise-then-multiply brute force, and the
                         unit-scale case where C is an exact integer;
* GGUF block bytes and the packed layout -- hand-picked byte positions.
"""
import os
import struct
from fractions import Fraction

import math

import numpy as np

from oracle import exact

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# golden file parsing
# --------------------------------------------------------------------------

def _num(tok):
    t = tok.lstrip("-")
    v = float.fromhex(t) if t.startswith("0x") else float(t)
    return -v if tok.startswith("-") else v


def _pad32(vals):
    vals = list(vals)
    assert len(vals) <= 32
    return vals + [0] * (32 - len(vals))


def load_block_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "q8_0_block_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            toks = [t for t in rest.split() if t != "..."]
            if key == "case":
                cur = {"name": rest.strip()}
                cases.append(cur)
            elif key == "x":
                xs = _pad32([_num(t) for t in toks])
                x32 = np.array(xs, dtype=np.float32)
                assert np.array_equal(x32.astype(np.float64), np.array(xs)), \
                    "golden x not exact in binary32: %s" % cur["name"]
                cur["x"] = x32
            elif key == "q":
                cur["q"] = np.array(_pad32(int(t) for t in toks), dtype=np.int8)
            elif key == "d":
                cur["d"] = int(rest.strip(), 16)
    return cases


def _rle(toks):
    out = []
    for t in toks:
        v, _, c = t.partition("*")
        out += [int(v)] * (int(c) if c else 1)
    return out


def load_gemm_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "q8_0_gemm_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip(), "C": {}, "absdot": {}}
                cases.append(cur)
            elif key == "shape":
                M, N, K = map(int, rest.split())
                cur.update(M=M, N=N, K=K,
                           qa=np.zeros((M, K), np.int8), qw=np.zeros((N, K), np.int8),
                           da=np.zeros((M, K // 32), np.uint16),
                           dw=np.zeros((N, K // 32), np.uint16))
            elif key in ("qa", "qw"):
                r, _, vals = rest.partition(":")
                cur[key][int(r)] = np.array(_rle(vals.split()), dtype=np.int8)
            elif key in ("da", "dw"):
                r, _, vals = rest.partition(":")
                cur[key][int(r)] = [int(v, 16) for v in vals.split()]
            elif key in ("C", "absdot"):
                m, n, v = rest.split()
                cur[key][(int(m), int(n))] = Fraction(v)
    return cases


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------

def pin_f16_roundtrip_all(orc):
    """Every finite binary16 value converts back to its own bits."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7C00) != 0x7C00
    bits = bits[finite]
    vals = bits.view(np.float16).astype(np.float32)
    got = orc.f32_to_f16_bits(vals)
    # -0 and +0 keep their sign
    assert np.array_equal(got, bits), "binary16 round trip differs"


def pin_f16_vs_numpy(orc):
    """Ties, near-ties, overflow edge and random values against numpy's
    float16 cast (IEEE 754 round to nearest even)."""
    h = np.arange(0, 0x7BFF, dtype=np.uint16)            # positive finite, not max
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)             # exact: <= 12 bits
    xs = [mid,
          np.nextafter(mid, np.float32(np.inf)),
          np.nextafter(mid, np.float32(0)),
          np.array([65504, 65519.996, 65520, 1e5, 2.0 ** -25, 2.0 ** -26,
                    3 * 2.0 ** -26, 2.0 ** -24, 1e-30, 0.0], dtype=np.float32)]
    r = np.random.default_rng(7)
    xs.append((r.standard_normal(200000) * np.exp2(r.uniform(-30, 17, 200000))).astype(np.float32))
    x = np.concatenate(xs).astype(np.float32)
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16_bits(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "binary16 differs from numpy at %r" % (x[bad[:5]],)


# --------------------------------------------------------------------------
# block quantiser
# --------------------------------------------------------------------------

def pin_quant_golden(orc):
    for c in load_block_cases():
        q, d, st = orc.quantize_block(c["x"])
        assert st == 0, c["name"]
        assert np.array_equal(q, c["q"]), "%s: q %s" % (c["name"], q)
        assert d == c["d"], "%s: d %#06x want %#06x" % (c["name"], d, c["d"])


def _random_blocks(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = i % 5
        x = r.standard_normal(32)
        if kind == 1:
            x *= 10.0 ** r.uniform(-6, 6)
        elif kind == 2:                       # integer-ish values -> many ties
            x = np.round(r.uniform(-127, 127, 32) * 2) / 2
        elif kind == 3:                       # fp16-subnormal scales
            x *= 2.0 ** r.uniform(-24, -14)
        elif kind == 4:                       # one outlier
            x[r.integers(32)] *= 50
        out.append(x.astype(np.float32))
    return out


def pin_quant_exact_random(orc, n=300):
    """Each binary32 step re-derived with exact rationals (oracle/exact.py)."""
    for x in _random_blocks(n, 11):
        q, d, st = orc.quantize_block(x)
        qe, de = exact.quantize_block_exact([float(v) for v in x])
        assert st == 0
        assert list(q.astype(int)) == qe, "q differs from exact re-derivation for %r" % (x,)
        assert d == de, "d %#06x != exact %#06x" % (d, de)


def pin_quant_invariants(orc, n=400):
    """|q| <= 127; the amax element maps to +-127; q(-x) = -q(x); scaling by
    2^e leaves q unchanged and scales d32; |x - d32 q| <= d32/2 (+ rounding)."""
    for x in _random_blocks(n, 12):
        q, d, _ = orc.quantize_block(x)
        amax = np.max(np.abs(x))
        d32 = np.float32(amax) / np.float32(127)
        assert np.all(np.abs(q.astype(int)) <= 127)
        if d32 >= np.finfo(np.float32).tiny:
            i = int(np.argmax(np.abs(x)))
            assert abs(int(q[i])) == 127
            err = np.abs(x.astype(np.float64) - float(d32) * q.astype(np.float64))
            assert np.all(err <= float(d32) * (0.5 + 2.0 ** -20)), "reconstruction bound"
        qn, dn, _ = orc.quantize_block(-x)
        assert np.array_equal(qn, -q) and dn == d
        for e in (-3, 5):
            xs = (x * np.float32(2.0 ** e)).astype(np.float32)
            qs, ds, _ = orc.quantize_block(xs)
            if np.float32(amax) * np.float32(2.0 ** min(e, 0)) > 1e-30:
                assert np.array_equal(qs, q), "q changed under power-of-two scaling"


def pin_quant_rows(orc):
    """Rows: bfloat16 input equals its exact binary32 widening; ldx > K
    ignores trailing columns; every block equals the single-block call."""
    r = np.random.default_rng(3)
    M, K, ldx = 5, 96, 128
    x = (r.standard_normal((M, ldx)) * 3).astype(np.float32)
    q, d = orc.quantize_rows(x, K=K, ldx=ldx)
    for m in range(M):
        for kb in range(K // 32):
            qb, db, _ = orc.quantize_block(x[m, 32 * kb:32 * kb + 32])
            assert np.array_equal(q[m, 32 * kb:32 * kb + 32], qb) and d[m, kb] == db
    b = (x.view(np.uint32) >> 16).astype(np.uint16)       # some bfloat16 bits
    wide = (b.astype(np.uint32) << 16).view(np.float32)
    qb16, db16 = orc.quantize_rows(b, K=K, ldx=ldx)
    qf, df = orc.quantize_rows(np.ascontiguousarray(wide), K=K, ldx=ldx)
    assert np.array_equal(qb16, qf) and np.array_equal(db16, df)


# --------------------------------------------------------------------------
# the product
# --------------------------------------------------------------------------

def pin_gemm_golden(orc):
    for c in load_gemm_cases():
        C, A = orc.gemm(c["qa"], c["da"], c["qw"], c["dw"])
        for (m, n), v in c["C"].items():
            assert Fraction(C[m, n]) == v, "%s C[%d][%d] = %r" % (c["name"], m, n, C[m, n])
        for (m, n), v in c["absdot"].items():
            assert Fraction(A[m, n]) == v, "%s absdot[%d][%d]" % (c["name"], m, n)


def _tiny_problem(seed, M, N, K):
    r = np.random.default_rng(seed)
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    da = (np.abs(r.standard_normal((M, K // 32))) * 0.02 + 1e-4).astype(np.float16).view(np.uint16)
    dw = (np.abs(r.standard_normal((N, K // 32))) * 4e-4 + 1e-6).astype(np.float16).view(np.uint16)
    sa = r.choice([-1, 1], size=da.shape)
    da = np.where(sa < 0, da | 0x8000, da).astype(np.uint16)
    return qa, da, qw, dw


def pin_gemm_exact(orc):
    """Against exact rational dequantise-then-multiply, on tiny shapes."""
    for seed, (M, N, K) in enumerate([(3, 4, 64), (2, 5, 96), (1, 3, 160)]):
        qa, da, qw, dw = _tiny_problem(100 + seed, M, N, K)
        C, A = orc.gemm(qa, da, qw, dw)
        E = exact.gemm_exact(qa.tolist(), da.tolist(), qw.tolist(), dw.tolist())
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(C[m, n]) - E[m][n])
                assert err <= Fraction(A[m, n]) * Fraction(1, 2 ** 48), (m, n, float(err))
                assert A[m, n] >= abs(C[m, n])


def pin_gemm_unit_scale(orc):
    """With every scale 1.0 the product is the integer matrix product."""
    r = np.random.default_rng(5)
    M, N, K = 7, 9, 1024
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    ones_a = np.full((M, K // 32), 0x3C00, np.uint16)
    ones_w = np.full((N, K // 32), 0x3C00, np.uint16)
    C, _ = orc.gemm(qa, ones_a, qw, ones_w)
    want = qa.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(C, want.astype(np.float64))


def pin_block_dots(orc):
    r = np.random.default_rng(6)
    M, N, K = 3, 4, 128
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    P = orc.block_dots(qa, qw)
    want = np.einsum("mbj,nbj->mnb", qa.reshape(M, K // 32, 32).astype(np.int64),
                     qw.reshape(N, K // 32, 32).astype(np.int64))
    assert np.array_equal(P, want)


def pin_gemm_sampled(orc):
    qa, da, qw, dw = _tiny_problem(9, 6, 10, 128)
    C, A = orc.gemm(qa, da, qw, dw)
    rows = np.array([0, 5, 3, 2, 5])
    cols = np.array([9, 0, 4, 4, 7])
    Cs, As = orc.gemm_sampled(qa, da, qw, dw, rows, cols)
    assert np.array_equal(Cs, C[rows, cols]) and np.array_equal(As, A[rows, cols])


# --------------------------------------------------------------------------
# byte layouts
# --------------------------------------------------------------------------

def pin_block_bytes(orc):
    """GGUF Q8_0 block = binary16 d (little-endian) then int8 q[32]."""
    q = np.arange(-32, 32, dtype=np.int8).reshape(1, 64)
    d = np.array([[0x3C01, 0xABCD]], dtype=np.uint16)
    b = orc.blocks_from_qd(q, d)
    assert b.shape == (1, 68)
    assert list(b[0, :2]) == [0x01, 0x3C] and list(b[0, 34:36]) == [0xCD, 0xAB]
    assert list(b[0, 2:34].view(np.int8)) == list(range(-32, 0))
    assert list(b[0, 36:68].view(np.int8)) == list(range(0, 32))
    q2, d2 = orc.qd_from_blocks(b, 1, 64)
    assert np.array_equal(q2, q) and np.array_equal(d2, d)


def pin_pack_layout(orc):
    """Hand-picked byte positions of the packed layout (see include/q8.h):
    quant byte ((g*KB + kb)*2 + h)*1024 + r*16 + t = q[64g+r][32kb+16h+t];
    scale (g*KB + kb)*64 + r after the quant plane; rows >= N are zero."""
    N, K = 70, 96                       # 2 row groups (second one ragged), 3 blocks
    KB, NG = 3, 2
    r = np.random.default_rng(8)
    q = r.integers(-127, 128, (N, K)).astype(np.int8)
    d = r.integers(1, 0x7BFF, (N, KB)).astype(np.uint16)
    packed = orc.pack(orc.blocks_from_qd(q, d), N, K)
    assert packed.size == NG * KB * (2048 + 128) == orc.packed_bytes(N, K)
    qp = packed[:NG * KB * 2048].view(np.int8)
    sp = packed[NG * KB * 2048:].view(np.uint16)
    for (g, kb, h, rr, t) in [(0, 0, 0, 0, 0), (0, 1, 1, 2, 3), (1, 2, 0, 5, 15),
                              (0, 2, 1, 63, 15), (1, 0, 1, 0, 7)]:
        assert qp[((g * KB + kb) * 2 + h) * 1024 + rr * 16 + t] == q[64 * g + rr, 32 * kb + 16 * h + t]
    for (g, kb, rr) in [(0, 0, 0), (0, 2, 17), (1, 1, 5)]:
        assert sp[(g * KB + kb) * 64 + rr] == d[64 * g + rr, kb]
    # rows 70..127 of group 1 are padding: zero quants and scales
    for kb in range(KB):
        for h in range(2):
            base = ((1 * KB + kb) * 2 + h) * 1024
            assert not np.any(qp[base + 6 * 16: base + 1024])
        assert not np.any(sp[(1 * KB + kb) * 64 + 6:(1 * KB + kb) * 64 + 64])
    # a permutation: the multiset of real bytes is preserved
    assert sorted(qp[qp != 0].tolist()) == sorted(q[q != 0].tolist())


# --------------------------------------------------------------------------
# gated FFN step: h = silu(g) * u, quantised per 32 along the hidden dimension
# --------------------------------------------------------------------------

def pin_silu(orc):
    """silu(x) = x / (1 + e^-x), checked through properties and other
    formulas: silu(x) - silu(-x) = x exactly in the reals; silu(x) =
    x (1 + tanh(x/2)) / 2 for x >= 0 and x e^x / (1 + e^x) for x < 0 (both
    free of cancellation there); silu(0) = 0; silu(x) = x where e^-x
    vanishes against 1 in double; silu -> -0 where e^-x overflows."""
    assert orc.silu(0.0) == 0.0
    r = np.random.default_rng(31)
    xs = np.concatenate([np.linspace(-30, 30, 601), r.standard_normal(500) * 8])
    for x in xs:
        x = float(x)
        a, b = orc.silu(x), orc.silu(-x)
        assert abs((a - b) - x) <= 4e-16 * max(1.0, abs(x)), x
        if x >= 0:
            ref = x * (1.0 + np.tanh(x / 2.0)) / 2.0
        else:
            ref = x * np.exp(x) / (1.0 + np.exp(x))
        assert abs(a - ref) <= 1e-15 * max(abs(ref), 1e-300) + 1e-300, (x, a, ref)
    assert orc.silu(50.0) == 50.0 and orc.silu(64.0) == 64.0
    assert orc.silu(-800.0) == 0.0


def pin_swiglu_golden(orc):
    """Hand-derived blocks.  Block 0: g = 64 (silu(64) = 64 in double) and
    u = t/64 with integers t in [-127, 127] that reach +-127, so h = t
    exactly, d32 = 1, q = t, d = binary16(1) = 0x3C00.  Block 1: g = -800
    (silu = -0), so h = 0, q = 0, d = 0.  Block 2: h = t + 1/2 for t < 127
    next to an element 127, so d32 = 1 and the halves round away from zero."""
    r = np.random.default_rng(32)
    t = r.integers(-126, 127, 32)
    t[5], t[20] = 127, -127
    t2 = r.integers(-120, 120, 32)
    half = t2 + 0.5
    half[0] = 127.0
    G = np.concatenate([np.full(32, 64.0), np.full(32, -800.0), np.full(32, 64.0)])[None, :]
    U = np.concatenate([t / 64.0, r.standard_normal(32), half / 64.0])[None, :]
    h, q, d = orc.swiglu_quant(G, U)
    assert np.array_equal(h[0, :32], t.astype(np.float64))
    assert np.array_equal(q[0, :32], t.astype(np.int8)) and d[0, 0] == 0x3C00
    assert not np.any(q[0, 32:64]) and d[0, 1] == 0
    want = np.where(half >= 0, np.floor(half) + 1, -(np.floor(-half) + 1))
    want[0] = 127
    assert np.array_equal(q[0, 64:96], want.astype(np.int8)) and d[0, 2] == 0x3C00


def pin_swiglu_rows(orc):
    """Random gate/up products: h equals silu (tanh form) times u, and q, d
    are the pinned quantiser applied to h rounded to binary32."""
    r = np.random.default_rng(33)
    M, I = 3, 160
    G = r.standard_normal((M, I)) * 3.0
    U = r.standard_normal((M, I)) * 2.0
    h, q, d = orc.swiglu_quant(G, U)
    sig = np.where(G >= 0, (1.0 + np.tanh(G / 2.0)) / 2.0, np.exp(G) / (1.0 + np.exp(G)))
    ref = G * sig * U
    assert np.all(np.abs(h - ref) <= 1e-14 * np.maximum(np.abs(ref), 1e-300))
    q2, d2 = orc.quantize_rows(h.astype(np.float32))
    assert np.array_equal(q, q2) and np.array_equal(d, d2)


def pin_gateup_layout(orc):
    """The gate/up interleave, by brute force from its description: 64-row
    group g of the packed weight holds gate rows 32g..32g+31, then up rows
    32g..32g+31; and the packed bytes are the pack of those rows."""
    I, K = 96, 64
    r = np.random.default_rng(34)
    gate = r.integers(0, 256, (I, 5)).astype(np.uint8)
    up = r.integers(0, 256, (I, 5)).astype(np.uint8)
    rows = orc.interleave_gateup(gate, up)
    assert rows.shape == (2 * I, 5)
    for n in range(2 * I):
        g, rr = divmod(n, 64)
        src = gate[32 * g + rr] if rr < 32 else up[32 * g + rr - 32]
        assert np.array_equal(rows[n], src), n
    qg = r.integers(-127, 128, (I, K)).astype(np.int8)
    qu = r.integers(-127, 128, (I, K)).astype(np.int8)
    dg = r.integers(1, 0x7BFF, (I, K // 32)).astype(np.uint16)
    du = r.integers(1, 0x7BFF, (I, K // 32)).astype(np.uint16)
    packed = orc.pack_gateup(orc.blocks_from_qd(qg, dg), orc.blocks_from_qd(qu, du), I, K)
    KB, NG = K // 32, 2 * I // 64
    qp = packed[:NG * KB * 2048].view(np.int8)
    sp = packed[NG * KB * 2048:].view(np.uint16)
    for (g, kb, h_, rr, t_) in [(0, 0, 0, 0, 0), (0, 1, 1, 31, 15), (1, 0, 1, 32, 3), (2, 1, 0, 63, 9)]:
        srcq = qg if rr < 32 else qu
        assert qp[((g * KB + kb) * 2 + h_) * 1024 + rr * 16 + t_] == \
            srcq[32 * g + rr % 32, 32 * kb + 16 * h_ + t_]
    for (g, kb, rr) in [(0, 0, 3), (1, 1, 40), (2, 0, 33)]:
        srcd = dg if rr < 32 else du
        assert sp[(g * KB + kb) * 64 + rr] == srcd[32 * g + rr % 32, kb]


# --------------------------------------------------------------------------
# 3-bit KV-cache codec
# --------------------------------------------------------------------------

def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi) if math.isfinite(x) else 0.0


def _Phi(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) if math.isfinite(x) else (1.0 if x > 0 else 0.0)


def pin_kv3_codebook(orc):
    """The codebook is the 8-level Lloyd-Max quantiser of a unit Gaussian:
    symmetric, and each level is the centroid E[X | cell] of its cell, the
    cells being cut at the midpoints of adjacent levels (closed form:
    (phi(a) - phi(b)) / (Phi(b) - Phi(a))); the levels are given to 4
    decimals, so to 5e-4."""
    L = orc.kv3_levels().astype(np.float64)
    assert np.all(np.diff(L) > 0) and np.allclose(L, -L[::-1], atol=0, rtol=0)
    t = [-math.inf] + [(L[k] + L[k + 1]) / 2 for k in range(7)] + [math.inf]
    for k in range(8):
        a, b = t[k], t[k + 1]
        c = (_phi(a) - _phi(b)) / (_Phi(b) - _Phi(a))
        assert abs(c - L[k]) < 5e-4, (k, L[k], c)


def _sylvester(D):
    H = np.array([[1.0]])
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def pin_fwht(orc):
    """The binary32 butterfly equals the Sylvester Hadamard matrix: exactly
    on unit vectors and small integers (then H H x = D x exactly too), and
    within its rounding bound on random vectors."""
    for D in (64, 128, 256):
        H = _sylvester(D)
        for k in (0, 1, 5, D - 1):
            e = np.zeros(D, np.float32)
            e[k] = 1
            assert np.array_equal(orc.fwht(e), H[:, k].astype(np.float32))
        r = np.random.default_rng(D)
        xi = r.integers(-50, 51, D).astype(np.float32)
        assert np.array_equal(orc.fwht(xi), (H @ xi).astype(np.float32))
        assert np.array_equal(orc.fwht(orc.fwht(xi)), (D * xi).astype(np.float32))
        x = r.standard_normal(D).astype(np.float32)
        ref = H @ x.astype(np.float64)
        assert np.all(np.abs(orc.fwht(x) - ref) <= D * 2.0 ** -24 * np.abs(x).sum() + 1e-30)


def pin_kv3_golden(orc):
    """Hand-derived rows (D = 128).  e_0: y = all ones, s = 1, every u = 1,
    code 5 (level 0.7560), bytes 6D DB B6 repeated, decode 0.756 e_0.  A
    column h_k of H: y = 128 e_k, s = sqrt(128), code 7 at k and code 4
    (u = 0 sits on the middle threshold) elsewhere.  The zero row: every
    code 4 (bytes 24 49 92), s = 0, decode 0."""
    D = 128
    H = _sylvester(D).astype(np.float32)
    x = np.zeros((3, D), np.float32)
    x[0, 0] = 1.0
    x[1] = H[:, 37]
    codes, scales = orc.kv3_encode(x)
    assert list(codes[0]) == [0x6D, 0xDB, 0xB6] * 16 and scales[0] == 1.0
    assert scales[1] == np.float32(math.sqrt(128.0))
    want = [4] * D
    want[37] = 7
    w = [sum(want[8 * g + j] << (3 * j) for j in range(8)) for g in range(16)]
    assert list(codes[1]) == [b for v in w for b in (v & 255, (v >> 8) & 255, v >> 16)]
    assert list(codes[2]) == [0x24, 0x49, 0x92] * 16 and scales[2] == 0.0
    out = orc.kv3_decode(codes, scales, D)
    e0 = np.zeros(D, np.float32)
    e0[0] = np.float32(0.7560)
    assert np.array_equal(out[0], e0) and not np.any(out[2])


def pin_kv3_sum_order(orc):
    """The order of the sum of squares (adjacent pairs, len = 1, 2, 4, ...),
    fixed by a hand-derived row (D = 64) on which other orders round
    differently.  y = H x with y_0 = 2^12 (square 2^24), y_1 = 0, y_2 ..
    y_41 = 1 and the rest 0; x = H y / 64 is exact in binary32 (multiples of
    1/64 below 2^7) and so is the butterfly back to y.  Adjacent pairs: the
    level-1 pair (2^24, 0) is exact, every other pair is 0, 1 + 1 = 2 or a
    sum of such, and each later partial sum with 2^24 in it is 2^24 plus an
    even number, which binary32 holds exactly (ulp 2 there): S = 2^24 + 40
    exactly, S/64 = 2^18 + 0.625 exactly, and sqrt of that is 512 +
    0.000610 = 512 + 10 ulp (ulp 2^-14 at 512; the second-order term is
    1e-5 ulp): s bits 0x4400000A.  A halving order (len = 32, 16, ...)
    first adds 2^24 + 1, a tie that rounds to 2^24, and a left-to-right sum
    loses every one: each gives a different s.  The codes: u_0 = 4096/s
    lies above the top threshold (code 7); u = 1/s and u = 0 sit at or
    above the middle threshold 0 (code 4)."""
    D = 64
    H = _sylvester(D)
    y = np.zeros(D, np.int64)
    y[0] = 4096
    y[2:42] = 1
    x = (H @ y).astype(np.float64) / D
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    codes, scales = orc.kv3_encode(x.astype(np.float32)[None, :])
    assert np.array_equal(orc.fwht(x.astype(np.float32)), y.astype(np.float32))
    assert scales.view(np.uint32)[0] == 0x4400000A, hex(scales.view(np.uint32)[0])
    want = [4] * D
    want[0] = 7
    w = [sum(want[8 * g + j] << (3 * j) for j in range(8)) for g in range(D // 8)]
    assert list(codes[0]) == [b for v in w for b in (v & 255, (v >> 8) & 255, v >> 16)]


def pin_kv3_code_positions(orc):
    """Code j of a 3-byte group sits at bits 3j..3j+2: decoding rows with a
    single non-middle code at a known position gives back, through the
    transform (H x^ = z), the level at exactly that position."""
    D = 64
    L = orc.kv3_levels()
    for pos, c in [(0, 0), (7, 7), (8, 1), (21, 6), (63, 2)]:
        codes4 = [4] * D
        codes4[pos] = c
        w = [sum(codes4[8 * g + j] << (3 * j) for j in range(8)) for g in range(D // 8)]
        row = np.array([b for v in w for b in (v & 255, (v >> 8) & 255, v >> 16)], np.uint8)
        out = orc.kv3_decode(row[None, :], np.array([2.0], np.float32), D)[0]
        z = orc.fwht(out)
        want = np.full(D, 2.0 * L[4], np.float64)
        want[pos] = 2.0 * L[c]
        assert np.all(np.abs(z - want) < 1e-5), (pos, c)


def pin_kv3_roundtrip(orc):
    """Gaussian rows: the relative mean squared error of decode(encode(x))
    is that of the 3-bit Lloyd-Max quantiser of a Gaussian (about 0.0345);
    scaling a row by a power of two scales s and nothing else; a bf16 row
    codes as its exact binary32 widening."""
    r = np.random.default_rng(40)
    for D in (64, 128, 256):
        x = r.standard_normal((1500, D)).astype(np.float32)
        codes, scales = orc.kv3_encode(x)
        xh = orc.kv3_decode(codes, scales, D)
        nmse = float(np.mean((xh - x) ** 2) / np.mean(x ** 2))
        assert 0.030 < nmse < 0.038, (D, nmse)
        c2, s2 = orc.kv3_encode(x * np.float32(8.0))
        assert np.array_equal(c2, codes) and np.array_equal(s2, scales * np.float32(8.0))
    xb = np.frombuffer(r.standard_normal((40, 128)).astype(np.float32).tobytes(), np.uint32)
    bits = (xb >> 16).astype(np.uint16).reshape(40, 128)
    wide = (bits.astype(np.uint32) << 16).view(np.float32)
    ca, sa = orc.kv3_encode(bits)
    cb, sb = orc.kv3_encode(wide)
    assert np.array_equal(ca, cb) and np.array_equal(sa, sb)


# -- block-sparse causal attention --------------------------------------

def _bf16(a):
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _widen(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _attn_inputs(L, Hq, Hkv, D, seed):
    r = np.random.default_rng(seed)
    q = _bf16(r.standard_normal((L, Hq * D)))
    k = _bf16(r.standard_normal((L, Hkv * D)))
    v = _bf16(r.standard_normal((L, Hkv * D)))
    return q, k, v


def _sdpa(q, k, v, Hq, Hkv, D, allowed):
    """torch's float64 scaled_dot_product_attention; allowed [Hq][L][L] bool
    (query t may attend key u)."""
    import torch
    L = q.shape[0]
    Q = torch.from_numpy(_widen(q).reshape(L, Hq, D).transpose(1, 0, 2).copy())
    K = torch.from_numpy(_widen(k).reshape(L, Hkv, D).transpose(1, 0, 2).copy())
    V = torch.from_numpy(_widen(v).reshape(L, Hkv, D).transpose(1, 0, 2).copy())
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None], V[None], attn_mask=torch.from_numpy(allowed)[None])
    return o[0].numpy().transpose(1, 0, 2).reshape(L, Hq * D)


def _allowed_from_lists(idx, cnt, L, Hq):
    """Lists per K/V head [Hkv][NB][kmax] -> mask per query head."""
    Hkv, NB, _ = idx.shape
    allowed = np.zeros((Hq, L, L), dtype=bool)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(NB):
            for j in idx[g, i, :cnt[g, i]]:
                allowed[h, 64 * i:64 * i + 64, 64 * j:64 * j + 64] = True
    return allowed & np.tril(np.ones((L, L), dtype=bool))[None]


def pin_attn_dense(orc):
    """With every block listed, block-sparse attention is dense causal
    attention: torch's scaled_dot_product_attention in float64 (grouped
    query heads expanded by repetition), ragged L."""
    for L, Hq, Hkv, D in ((200, 4, 2, 64), (130, 2, 1, 128)):
        q, k, v = _attn_inputs(L, Hq, Hkv, D, L + D)
        NB = (L + 63) // 64
        idx, cnt = orc.attn_select(orc.attn_pool(q, Hq, D), orc.attn_pool(k, Hkv, D), NB)
        out, mag = orc.attn_fwd(q, k, v, Hq, Hkv, D, idx, cnt)
        ref = _sdpa(q, k, v, Hq, Hkv, D, np.broadcast_to(np.tril(np.ones((L, L), bool)), (Hq, L, L)).copy())
        assert np.max(np.abs(out - ref)) < 1e-12, np.max(np.abs(out - ref))
        assert np.all(mag >= np.abs(out) - 1e-12)


def pin_attn_masked(orc):
    """Arbitrary block lists (block 0 and the diagonal always present):
    the output is torch's attention under the block-and-causal mask."""
    L, Hq, Hkv, D = 330, 4, 2, 64
    q, k, v = _attn_inputs(L, Hq, Hkv, D, 7)
    NB = (L + 63) // 64
    r = np.random.default_rng(8)
    kmax = 4
    idx = np.full((Hkv, NB, kmax), -1, np.int32)
    cnt = np.zeros((Hkv, NB), np.int32)
    for g in range(Hkv):
        for i in range(NB):
            extra = [j for j in range(1, i) if r.random() < 0.4][:kmax - 2]
            blocks = sorted(set([0, i] + extra))
            idx[g, i, :len(blocks)] = blocks
            cnt[g, i] = len(blocks)
    out, _ = orc.attn_fwd(q, k, v, Hq, Hkv, D, idx, cnt)
    ref = _sdpa(q, k, v, Hq, Hkv, D, _allowed_from_lists(idx, cnt, L, Hq))
    assert np.max(np.abs(out - ref)) < 1e-12, np.max(np.abs(out - ref))


def pin_attn_invariants(orc):
    """Constant value rows give that constant; the first token sees only
    itself, so its output is its own value row; outputs are convex
    combinations (within [min v, max v] per column)."""
    L, Hq, Hkv, D = 150, 2, 2, 64
    q, k, v = _attn_inputs(L, Hq, Hkv, D, 11)
    pq, pk = orc.attn_pool(q, Hq, D), orc.attn_pool(k, Hkv, D)
    idx, cnt = orc.attn_select(pq, pk, 2)
    out, _ = orc.attn_fwd(q, k, v, Hq, Hkv, D, idx, cnt)
    assert np.array_equal(out[0], _widen(v[0]))
    vw = _widen(v).reshape(L, Hkv, D)
    o = out.reshape(L, Hq, D)
    assert np.all(o <= vw.max(axis=0)[None] + 1e-12) and np.all(o >= vw.min(axis=0)[None] - 1e-12)
    c = _bf16(np.tile(np.linspace(-3, 3, Hkv * D), (L, 1)))
    out_c, _ = orc.attn_fwd(q, k, c, Hq, Hkv, D, idx, cnt)
    assert np.max(np.abs(out_c - np.tile(_widen(c[0]), (L, 1)).reshape(L, Hkv, D).repeat(Hq // Hkv, axis=1).reshape(L, -1))) < 1e-14


def pin_attn_pool(orc):
    """Pooled rows are numpy's means over each block's tokens (a shorter
    last block included)."""
    L, H, D = 170, 3, 64
    x = _bf16(np.random.default_rng(3).standard_normal((L, H * D)))
    p = orc.attn_pool(x, H, D)
    w = _widen(x).reshape(L, H, D)
    for b in range(3):
        assert np.allclose(p[:, b], w[64 * b:64 * b + 64].mean(axis=0), rtol=0, atol=1e-15)


def pin_attn_select(orc):
    """Selection rules, and a planted ranking: K rows of block j all equal
    c_j e_0 and Q rows equal e_0, so the score of block j is c_j; the kept
    blocks are 0, i and the (k-2) largest c_j among 0 < j < i, the lower j
    first on equal c_j."""
    D, NB = 64, 12
    L = 64 * NB
    c = np.array([0.5, 3, 1, 3, 2, 0.25, 3, 1.5, 0.75, 2, 1, 0.125])   # per key block
    q = np.zeros((L, D), np.float32)
    q[:, 0] = 1.0
    kk = np.zeros((L, D), np.float32)
    for j in range(NB):
        kk[64 * j:64 * j + 64, 0] = c[j]
    pq, pk = orc.attn_pool(_bf16(q), 1, D), orc.attn_pool(_bf16(kk), 1, D)
    for k in (2, 3, 4, 5):
        idx, cnt = orc.attn_select(pq, pk, k)
        for i in range(NB):
            got = list(idx[0, i, :cnt[0, i]])
            assert cnt[0, i] == min(k, i + 1) and got == sorted(set(got)), (k, i, got)
            assert all(j <= i for j in got) and (0 in got) and (i in got)
            if k >= i + 1:
                assert got == list(range(i + 1))
                continue
            others = sorted(range(1, i), key=lambda j: (-c[j], j))[:k - 2]
            assert got == sorted(set([0, i] + others)), (k, i, got, others)
    # hand check of one row: i = 9, k = 4: scores 3 (j=1), 3 (3), 3 (6): keep 1, 3
    idx, cnt = orc.attn_select(pq, pk, 4)
    assert list(idx[0, 9, :4]) == [0, 1, 3, 9]
    # a group of two query heads over one K/V head ranks by the sum of the
    # heads' scores: head 0 rows e_0, head 1 rows e_1, K block j rows
    # a_j e_0 + b_j e_1, so the score of block j is a_j + b_j.  Head 0 alone
    # would keep blocks 1, 4 (a = 3, 2.5), head 1 alone 2, 3 (b = 3, 2); the
    # sums are 3, 3, 4, 4.25, so the group keeps 3 and 4.
    a = np.array([0, 3, 0, 2, 2.5, 0, 0, 0, 0, 0])
    b = np.array([0, 0, 3, 2, 1.75, 0, 0, 0, 0, 0])
    NB2 = a.size
    q2 = np.zeros((64 * NB2, 2 * D), np.float32)
    q2[:, 0] = 1.0
    q2[:, D + 1] = 1.0
    k2 = np.zeros((64 * NB2, D), np.float32)
    for j in range(NB2):
        k2[64 * j:64 * j + 64, 0] = a[j]
        k2[64 * j:64 * j + 64, 1] = b[j]
    idx2, cnt2 = orc.attn_select(orc.attn_pool(_bf16(q2), 2, D), orc.attn_pool(_bf16(k2), 1, D), 4)
    assert idx2.shape == (1, NB2, 4)
    assert list(idx2[0, 9, :4]) == [0, 3, 4, 9] and list(idx2[0, 5, :4]) == [0, 3, 4, 5]


ALL_PINS = [pin_f16_roundtrip_all, pin_f16_vs_numpy, pin_quant_golden, pin_quant_exact_random,
            pin_quant_invariants, pin_quant_rows, pin_gemm_golden, pin_gemm_exact,
            pin_gemm_unit_scale, pin_block_dots, pin_gemm_sampled, pin_block_bytes,
            pin_pack_layout, pin_silu, pin_swiglu_golden, pin_swiglu_rows, pin_gateup_layout,
            pin_kv3_codebook, pin_fwht, pin_kv3_golden, pin_kv3_sum_order, pin_kv3_code_positions, pin_kv3_roundtrip,
            pin_attn_dense, pin_attn_masked, pin_attn_invariants, pin_attn_pool, pin_attn_select]
