"""Property tests of the CPU oracle over random blocks (hypothesis).

Invariants of the Q8_0 block quantiser and of the block-scaled product that
follow from their definition (news.hada.io topic 29953, "CUDA inference
engine for running Qwen3.5/3.6 hybrid models on mining cards (CMP
100-210)": Q8_0 is the weight format of the limitations list, quantised on
the fly for the int8 GEMM of the engine list), checked on inputs hypothesis
draws: sign symmetry, permutation equivariance, exact power-of-two scaling,
the half-step reconstruction bound, the extreme code, and for the product
its symmetry, exact negation and exact power-of-two scaling.  None of them
re-types the oracle's formulas.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")

SETTINGS = dict(max_examples=150, deadline=None,
                suppress_health_check=[HealthCheck.function_scoped_fixture])

# Finite float32 values.  Tests that need every scale normal keep only blocks
# with 2^-13 * 127 <= amax <= 65504 * 127 / 4 (a binade of margin each side
# of the binary16 normal range).
_val = st.floats(min_value=-3.0e6, max_value=3.0e6, allow_nan=False, allow_infinity=False,
                 width=32)
_block = st.lists(_val, min_size=32, max_size=32).map(lambda v: np.array(v, dtype=np.float32))


def _normal_block(x):
    amax = float(np.max(np.abs(x)))
    return 127 * 2.0 ** -13 <= amax <= 65504 * 127 / 4


def _f16(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


@settings(**SETTINGS)
@given(_block)
def test_quantiser_codes_bounded_and_signed(orc, x):
    q, d, st_ = orc.quantize_block(x)
    assert st_ == 0
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # a code never has the opposite sign of its value
    assert np.all(q.astype(np.int64) * np.sign(x).astype(np.int64) >= 0)


@settings(**SETTINGS)
@given(_block)
def test_quantiser_sign_symmetry(orc, x):
    q, d, _ = orc.quantize_block(x)
    qn, dn, _ = orc.quantize_block(-x)
    assert dn == d
    assert np.array_equal(qn, -q)


@settings(**SETTINGS)
@given(_block, st.permutations(list(range(32))))
def test_quantiser_permutation_equivariance(orc, x, perm):
    perm = np.array(perm)
    q, d, _ = orc.quantize_block(x)
    qp, dp, _ = orc.quantize_block(x[perm])
    assert dp == d
    assert np.array_equal(qp, q[perm])


@settings(**SETTINGS)
@given(_block, st.integers(min_value=-6, max_value=6))
def test_quantiser_power_of_two_scaling(orc, x, e):
    """Scaling a block by 2^e scales d by 2^e and keeps every code, while
    every scale involved stays a normal binary16 / binary32 number."""
    xs = (x * np.float32(2.0 ** e)).astype(np.float32)
    if not (_normal_block(x) and _normal_block(xs)):
        return
    q, d, _ = orc.quantize_block(x)
    qs, ds, _ = orc.quantize_block(xs)
    assert np.array_equal(qs, q)
    assert _f16(ds) == _f16(d) * 2.0 ** e


@settings(**SETTINGS)
@given(_block)
def test_quantiser_reconstruction_within_half_step(orc, x):
    """Each value is within half a step of its code: |x - q * amax/127| <=
    amax/254, up to the binary32 roundings of the step and its reciprocal;
    the largest magnitude gets the extreme code."""
    if not _normal_block(x):
        return
    q, d, _ = orc.quantize_block(x)
    amax = float(np.max(np.abs(x)))
    step = amax / 127.0
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * step)
    assert np.all(err <= step * (0.5 + 1e-4))
    assert abs(int(q[int(np.argmax(np.abs(x)))])) == 127
    # d is the binary16 nearest the step (within half an ulp of binary16)
    assert abs(_f16(d) - step) <= step * 2.0 ** -11 * 1.0001


def test_quantiser_zero_block(orc):
    q, d, st_ = orc.quantize_block(np.zeros(32, dtype=np.float32))
    assert st_ == 0 and d == 0 and not np.any(q)


_small = st.integers(min_value=1, max_value=3)


@st.composite
def _problem(draw):
    M, N, KB = draw(_small), draw(_small), draw(st.integers(min_value=1, max_value=4))
    K = 32 * KB
    r = np.random.default_rng(draw(st.integers(min_value=0, max_value=2 ** 31)))
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    # binary16 scales from a few binades (exact products in binary64)
    da = np.float16(2.0) ** r.integers(-8, 8, (M, KB)).astype(np.float16)
    dw = (r.integers(1, 2048, (N, KB)) * 2.0 ** -10).astype(np.float16)
    return qa, da.view(np.uint16), qw, dw.view(np.uint16)


@settings(**SETTINGS)
@given(_problem())
def test_product_symmetry_and_negation(orc, p):
    qa, da, qw, dw = p
    C, A = orc.gemm(qa, da, qw, dw)
    Ct, At = orc.gemm(qw, dw, qa, da)
    assert np.array_equal(C, Ct.T) and np.array_equal(A, At.T)
    Cn, An = orc.gemm(qa, da, -qw, dw)
    assert np.array_equal(Cn, -C) and np.array_equal(An, A)
    assert np.all(np.abs(C) <= A)


@settings(**SETTINGS)
@given(_problem(), st.integers(min_value=-4, max_value=4))
def test_product_power_of_two_scale(orc, p, e):
    qa, da, qw, dw = p
    C, _ = orc.gemm(qa, da, qw, dw)
    da2 = (da.view(np.float16).astype(np.float32) * np.float32(2.0 ** e)).astype(np.float16)
    C2, _ = orc.gemm(qa, da2.view(np.uint16), qw, dw)
    assert np.array_equal(C2, C * 2.0 ** e)
