"""The gated feed-forward step through the C ABI: q8_pack_weights_gateup
(bit-exact against the oracle's interleave + pack) and q8_gemm_swiglu
against the CPU oracle (exact gate and up products, h = silu(g) * u in
double, the Q8_0 quantiser).

The kernel decides the codes from binary32 values of h (g and u within the
q8_gemm bound, silu with the device's binary32 exp), so a value of h close
to a rounding boundary of the quantiser may land on either side.  The
checks are therefore: every dequantised value d*q lies within the
quantisation bound of the exact h (plus the error bound of the binary32 h);
every block scale is within one binary16 step of the oracle's; and nearly
all codes equal the oracle's exactly."""
import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import workloads
from gpu_util import DEV, blocks_to_dev, d_bits, qd_to_dev, say

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24


def _f16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _gateup(orc, I, K, seed, scale_w=0.02):
    g = workloads.weights_f32(I, K, case=95, tensor=2 * seed, std=scale_w)
    u = workloads.weights_f32(I, K, case=95, tensor=2 * seed + 1, std=scale_w)
    qg, dg = orc.quantize_rows(g)
    qu, du = orc.quantize_rows(u)
    bg, bu = orc.blocks_from_qd(qg, dg), orc.blocks_from_qd(qu, du)
    wp = q8.q8_pack_weights_gateup(blocks_to_dev(bg), blocks_to_dev(bu), I, K)
    return qg, dg, qu, du, bg, bu, wp


def check_swiglu(q_gpu, d_gpu, G, absG, U, absU, h_ref, q_ref, d_ref, K, what):
    """q_gpu/d_gpu: [R][32*B] codes and [R][B] scale bits; the rest the
    oracle's exact products (and abs-dots), h and quantisation."""
    eps = (K / 32 + 2) * U24
    dG, dU = eps * absG, eps * absU
    with np.errstate(over="ignore"):
        sil = np.abs(G / (1.0 + np.exp(-G)))                      # |silu(G)|
    tol_h = 1.1 * (np.abs(U) + dU) * dG + (sil + 1.1 * dG) * dU + 2.0 ** -20 * np.abs(h_ref) + 1e-30
    R, I = q_gpu.shape
    B = I // 32
    dg = _f16(d_gpu)
    dr = _f16(d_ref)
    amax = np.abs(h_ref).reshape(R, B, 32).max(axis=2)
    tolb = tol_h.reshape(R, B, 32).max(axis=2)
    # scales: within the binary16 rounding of amax/127 plus the h bound
    assert np.all(np.abs(q_gpu.astype(np.int32)) <= 127), what
    dev = np.abs(dg - amax / 127.0)
    lim = tolb / 127.0 + 2.0 ** -11 * amax / 127.0 + 2.0 ** -25
    bad = np.nonzero(dev > lim)
    assert bad[0].size == 0, "%s: scale off at %s: %r vs amax/127 %r" % (
        what, tuple(b[0] for b in bad), dg[bad][0], (amax / 127.0)[bad][0])
    ulp = np.maximum(np.abs(dr) * 2.0 ** -10, 2.0 ** -24)       # >= one binary16 step
    assert np.all(np.abs(dg - dr) <= ulp * 1.0001), "%s: scale differs from the oracle's by > 1 step" % what
    # reconstruction: |d q - h| <= d (1/2 + 127 * 2^-11) + tol_h
    dq = np.repeat(dg, 32, axis=1) * q_gpu.astype(np.float64)
    lim = np.repeat(dg, 32, axis=1) * (0.5 + 127 * 2.0 ** -11) + tol_h
    bad = np.nonzero(np.abs(dq - h_ref) > lim)
    assert bad[0].size == 0, "%s: %d codes off; first at %s: d*q %r, h %r" % (
        what, bad[0].size, tuple(b[0] for b in bad), dq[bad][0], h_ref[bad][0])
    same = np.mean(q_gpu == q_ref)
    assert same >= 0.99, "%s: only %.4f of codes equal the oracle's" % (what, same)
    return same


@pytest.mark.parametrize("I,K", [(32, 32), (96, 160), (160, 1056), (12288, 4096)])
def test_pack_gateup_bitexact(orc, I, K):
    r = np.random.default_rng(I + K)
    qg = r.integers(-127, 128, (I, K)).astype(np.int8)
    qu = r.integers(-127, 128, (I, K)).astype(np.int8)
    dg = r.integers(0, 0x7BFF, (I, K // 32)).astype(np.uint16)
    du = r.integers(0, 0x7BFF, (I, K // 32)).astype(np.uint16)
    bg, bu = orc.blocks_from_qd(qg, dg), orc.blocks_from_qd(qu, du)
    say("pack gate/up I=%d K=%d" % (I, K))
    got = q8.q8_pack_weights_gateup(blocks_to_dev(bg), blocks_to_dev(bu), I, K).cpu().numpy()
    assert np.array_equal(got, orc.pack_gateup(bg, bu, I, K))


@pytest.mark.parametrize("M,I,K", [(1, 32, 32), (3, 96, 160), (8, 160, 1056), (5, 64, 4096),
                                   (9, 96, 160), (130, 160, 544), (300, 224, 1056), (64, 96, 32)])
def test_swiglu_against_oracle(orc, M, I, K):
    qg, dg, qu, du, bg, bu, wp = _gateup(orc, I, K, M)
    x = workloads.acts_f32(M, K, case=96, tensor=M)
    qa, da = orc.quantize_rows(x)
    say("swiglu M=%d I=%d K=%d" % (M, I, K))
    qt, dt = qd_to_dev(qa, da)
    q_h, d_h = q8.q8_gemm_swiglu(qt, dt, wp, I, K)
    G, absG = orc.gemm(qa, da, qg, dg)
    U, absU = orc.gemm(qa, da, qu, du)
    h_ref, q_ref, d_ref = orc.swiglu_quant(G, U)
    check_swiglu(q_h.cpu().numpy(), d_bits(d_h), G, absG, U, absU, h_ref, q_ref, d_ref, K,
                 "M%d I%d K%d" % (M, I, K))


def test_swiglu_feeds_down_projection(orc):
    """The step's output is a valid activation for the down projection."""
    M, I, K, N = 12, 96, 160, 70
    qg, dg, qu, du, bg, bu, wp = _gateup(orc, I, K, 7)
    qa, da = orc.quantize_rows(workloads.acts_f32(M, K, case=97))
    qt, dt = qd_to_dev(qa, da)
    q_h, d_h = q8.q8_gemm_swiglu(qt, dt, wp, I, K)
    qd_ = workloads.weights_f32(N, I, case=98)
    qw, dw = orc.quantize_rows(qd_)
    wd = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, I)
    C = q8.q8_gemm(q_h, d_h, wd, N, I).cpu().numpy()
    C_ref, absdot = orc.gemm(q_h.cpu().numpy(), d_bits(d_h), qw, dw)
    from gpu_util import check_close
    check_close(C, C_ref, absdot, I, "down after swiglu")


@pytest.mark.parametrize("M", [512, 509, 4])
def test_swiglu_gateup_workload(orc, M):
    """The 9B-like gate+up layer (I = 12288 hidden units, K = 4096) with the
    sweep's outlier activations, at M = 512, 509 (matrix cores) and 4
    (decode): 96 sampled (row, block) pairs, 3072 hidden units each of gate
    and up, against the oracle."""
    I, K = 12288, 4096
    qg, dg, qu, du, bg, bu, wp = _gateup(orc, I, K, 11)
    x = workloads.acts_outliers(M, K, case=99)
    qa, da = orc.quantize_rows(x)
    say("swiglu workload M=%d I=%d K=%d" % (M, I, K))
    qt, dt = qd_to_dev(qa, da)
    q_h, d_h = q8.q8_gemm_swiglu(qt, dt, wp, I, K)
    q_h, d_h = q_h.cpu().numpy(), d_bits(d_h)
    r = np.random.default_rng(12)
    rows = r.integers(0, M, 96)
    blks = r.integers(0, I // 32, 96)
    rr = np.repeat(rows, 32)
    cols = (blks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    G, absG = orc.gemm_sampled(qa, da, qg, dg, rr, cols)
    U, absU = orc.gemm_sampled(qa, da, qu, du, rr, cols)
    G, absG, U, absU = (a.reshape(96, 32) for a in (G, absG, U, absU))
    h_ref, q_ref, d_ref = orc.swiglu_quant(G, U)
    qg_ = q_h[rows[:, None], (blks[:, None] * 32 + np.arange(32)[None, :])]
    dg_ = d_h[rows, blks][:, None]
    check_swiglu(qg_, dg_, G, absG, U, absU, h_ref, q_ref, d_ref, K, "workload M%d" % M)


@pytest.mark.parametrize("tile", [0, 1, 3, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("M,I,K", [(130, 160, 544), (300, 224, 1056)])
def test_swiglu_every_tile(orc, monkeypatch, tile, M, I, K):
    """The gated epilogue on every matrix-core tile configuration (forced
    through its benchmarking switch), including the ones whose waves split
    K into groups and add their partial sums before the epilogue."""
    monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    qg, dg, qu, du, bg, bu, wp = _gateup(orc, I, K, M)
    x = workloads.acts_f32(M, K, case=97, tensor=M + tile)
    qa, da = orc.quantize_rows(x)
    say("swiglu tile %d M=%d I=%d K=%d" % (tile, M, I, K))
    qt, dt = qd_to_dev(qa, da)
    q_h, d_h = q8.q8_gemm_swiglu(qt, dt, wp, I, K)
    G, absG = orc.gemm(qa, da, qg, dg)
    U, absU = orc.gemm(qa, da, qu, du)
    h_ref, q_ref, d_ref = orc.swiglu_quant(G, U)
    check_swiglu(q_h.cpu().numpy(), d_bits(d_h), G, absG, U, absU, h_ref, q_ref, d_ref, K,
                 "tile %d M%d I%d K%d" % (tile, M, I, K))


@pytest.mark.parametrize("M", [3, 40, 300])
def test_swiglu_guard_bands(orc, M):
    """q_h and d_h are written exactly where the rows go (decode kernel,
    small M, matrix-core tiles): sentinel rows before and after stay intact,
    and the rows between match a call into fresh buffers bit for bit."""
    I, K = 160, 544
    qg, dg, qu, du, bg, bu, wp = _gateup(orc, I, K, 90 + M)
    x = workloads.acts_f32(M, K, case=98, tensor=M)
    qa, da = orc.quantize_rows(x)
    qt, dt = qd_to_dev(qa, da)
    say("swiglu guard bands M=%d I=%d K=%d" % (M, I, K))
    qbuf = torch.full((M + 2, I), 77, dtype=torch.int8, device=DEV)
    dbuf = torch.full((M + 2, I // 32), 3.0, dtype=torch.float16, device=DEV)
    q8.q8_gemm_swiglu(qt, dt, wp, I, K, q=qbuf[1:M + 1], d=dbuf[1:M + 1])
    q_ref, d_ref = q8.q8_gemm_swiglu(qt, dt, wp, I, K)
    qh, dh = qbuf.cpu().numpy(), d_bits(dbuf)
    assert np.all(qh[0] == 77) and np.all(qh[M + 1] == 77), "q_h written outside its rows"
    assert np.all(dh[0] == 0x4200) and np.all(dh[M + 1] == 0x4200), "d_h written outside its rows"
    assert np.array_equal(qh[1:M + 1], q_ref.cpu().numpy())
    assert np.array_equal(dh[1:M + 1], d_bits(d_ref))
