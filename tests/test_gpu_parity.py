"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every input is seeded (workloads.py); the oracle quantises the weights into
GGUF Q8_0 blocks, which both sides then consume.  Activations are quantised
by both sides and must agree bit for bit before the products are compared.
"""
import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import pins
import workloads
from gpu_util import DEV, blocks_to_dev, check_close, d_bits, qd_to_dev, say, x_to_dev

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------

def test_quantize_golden_blocks():
    cases = pins.load_block_cases()
    x = np.stack([c["x"] for c in cases])
    say("quantize golden blocks: %d rows x 32 (fp32)" % len(cases))
    q, d = q8.q8_quantize_act(x_to_dev(x))
    q, d = q.cpu().numpy(), d_bits(d)
    for i, c in enumerate(cases):
        assert np.array_equal(q[i], c["q"]), "%s: q %s" % (c["name"], q[i])
        assert d[i, 0] == c["d"], "%s: d %#06x" % (c["name"], d[i, 0])


def _random_scale_rows(M, K, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((M, K))
    mag = 2.0 ** r.uniform(-30, 20, (M, K // 32, 1))          # incl. binary16-subnormal scales
    x = (x.reshape(M, K // 32, 32) * mag).reshape(M, K)
    ties = r.random((M, K // 32)) < 0.2                       # blocks of half-integers, amax 127
    for m, kb in zip(*np.nonzero(ties)):
        blk = np.round(r.uniform(-126, 126, 32) * 2) / 2
        blk[r.integers(32)] = 127 * r.choice([-1, 1])
        x[m, 32 * kb:32 * kb + 32] = blk
    x[:, :32] = 0.0                                            # an all-zero block per row
    return x.astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_random_scales(orc, dtype):
    x = _random_scale_rows(64, 1024, 21)
    if dtype == "bf16":
        x = workloads.f32_to_bf16_bits(x)
    say("quantize random scales %s 64x1024" % dtype)
    q, d = q8.q8_quantize_act(x_to_dev(x))
    qr, dr = orc.quantize_rows(x)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(d_bits(d), dr)


def test_quantize_row_pitch(orc):
    x = _random_scale_rows(9, 256, 22)
    K = 160                                                    # read the first 160 of 256 columns
    say("quantize ldx=256 K=160")
    xt = x_to_dev(x)
    q, d = q8.q8_quantize_act(xt, K=K)
    qr, dr = orc.quantize_rows(x, K=K, ldx=256)
    assert np.array_equal(q.cpu().numpy(), qr) and np.array_equal(d_bits(d), dr)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (9, 1056), (300, 2080)])
def test_quantize_guard_bands(orc, dtype, M, K):
    """q and d are written exactly where the rows go: a row of sentinels
    before and after each output (and the bytes around them) stays intact."""
    x = _random_scale_rows(M, K, 31 + M)
    xs = x if dtype == "f32" else workloads.f32_to_bf16_bits(x)
    say("quantize guard bands %s M=%d K=%d" % (dtype, M, K))
    qbuf = torch.full((M + 2, K), 77, dtype=torch.int8, device=DEV)
    dbuf = torch.full((M + 2, K // 32), 3.0, dtype=torch.float16, device=DEV)
    q8.q8_quantize_act(x_to_dev(xs), q=qbuf[1:M + 1], d=dbuf[1:M + 1])
    qh, dh = qbuf.cpu().numpy(), d_bits(dbuf)
    assert np.all(qh[0] == 77) and np.all(qh[M + 1] == 77), "q written outside its rows"
    assert np.all(dh[0] == 0x4200) and np.all(dh[M + 1] == 0x4200), "d written outside its rows"
    qr, dr = orc.quantize_rows(xs)
    assert np.array_equal(qh[1:M + 1], qr) and np.array_equal(dh[1:M + 1], dr)


@pytest.mark.parametrize("M,K", [(4 * 65535 + 4 * 37 + 3, 64), (65536 + 300, 2048)])
def test_quantize_rows_past_grid_limit(orc, M, K):
    """More rows than a launch grid holds in y (65535): the workgroups loop
    over further rows and stop at M (four lanes per block at K = 64, one lane
    per block at K = 2048)."""
    r = np.random.default_rng(41)
    x = r.standard_normal((M, K), dtype=np.float32)
    x *= (2.0 ** r.uniform(-8, 8, (M, 1))).astype(np.float32)
    xs = workloads.f32_to_bf16_bits(x)
    del x
    say("quantize bf16 M=%d K=%d (rows past the grid's y limit)" % (M, K))
    qbuf = torch.full((M + 1, K), 77, dtype=torch.int8, device=DEV)
    dbuf = torch.full((M + 1, K // 32), 3.0, dtype=torch.float16, device=DEV)
    q8.q8_quantize_act(x_to_dev(xs), q=qbuf[:M], d=dbuf[:M])
    qh, dh = qbuf.cpu().numpy(), d_bits(dbuf)
    assert np.all(qh[M] == 77) and np.all(dh[M] == 0x4200), "written past the last row"
    qr, dr = orc.quantize_rows(xs)
    assert np.array_equal(qh[:M], qr) and np.array_equal(dh[:M], dr)


QUANT_LAYERS = [workloads.TINY, workloads.DECODE_M4, workloads.PREFILL, workloads.LARGE_UP,
                workloads.LARGE_DOWN] + workloads.sweep(509)[::3]


@pytest.mark.parametrize("layer", QUANT_LAYERS, ids=lambda l: l.name)
def test_quantize_workload_bitexact(orc, layer):
    x = workloads.activations(layer)
    say("quantize %s (%s)" % (layer.name, x.dtype))
    q, d = q8.q8_quantize_act(x_to_dev(x))
    qr, dr = orc.quantize_rows(x)
    assert np.array_equal(q.cpu().numpy(), qr), "q differs"
    assert np.array_equal(d_bits(d), dr), "d differs"


@pytest.mark.parametrize("layer", [workloads.TINY, workloads.PREFILL], ids=lambda l: l.name)
def test_quantize_weights_bitexact(orc, layer):
    """The same quantiser applied to weight rows (binary32) matches too."""
    w = workloads.weights(layer)
    say("quantize weights %s" % layer.name)
    q, d = q8.q8_quantize_act(x_to_dev(w))
    qr, dr = orc.quantize_rows(w)
    assert np.array_equal(q.cpu().numpy(), qr) and np.array_equal(d_bits(d), dr)


# --------------------------------------------------------------------------
# pack
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(64, 32), (70, 96), (256, 512), (130, 1056), (12288, 4096)])
def test_pack_bitexact(orc, N, K):
    r = np.random.default_rng(N * 7 + K)
    q = r.integers(-127, 128, (N, K)).astype(np.int8)
    d = r.integers(0, 0x7BFF, (N, K // 32)).astype(np.uint16)
    blocks = orc.blocks_from_qd(q, d)
    say("pack N=%d K=%d" % (N, K))
    got = q8.q8_pack_weights(blocks_to_dev(blocks), N, K).cpu().numpy()
    assert np.array_equal(got, orc.pack(blocks, N, K))


# --------------------------------------------------------------------------
# product: integer exactness, small shapes in full, determinism, guards
# --------------------------------------------------------------------------

def _problem(M, N, K, seed, unit=False):
    r = np.random.default_rng(seed)
    qa = r.integers(-127, 128, (M, K)).astype(np.int8)
    qw = r.integers(-127, 128, (N, K)).astype(np.int8)
    if unit:
        da = np.full((M, K // 32), 0x3C00, np.uint16)
        dw = np.full((N, K // 32), 0x3C00, np.uint16)
    else:
        da = (np.abs(r.standard_normal((M, K // 32))) * 0.02 + 1e-3).astype(np.float16).view(np.uint16)
        dw = (np.abs(r.standard_normal((N, K // 32))) * 5e-4 + 1e-5).astype(np.float16).view(np.uint16)
    return qa, da, qw, dw


def _run(qa, da, blocks, N, K, out=None):
    qt, dt = qd_to_dev(qa, da)
    wp = q8.q8_pack_weights(blocks_to_dev(blocks), N, K)
    C = q8.q8_gemm(qt, dt, wp, N, K, out=out)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("K", [32, 64, 512, 1024])
@pytest.mark.parametrize("M", [1, 4, 8, 9, 16, 130])
def test_gemm_unit_scale_is_exact_integer(orc, M, K):
    """All scales 1.0 and K <= 1024: C is an integer below 2^24, so every
    block's int32 dot must come out exactly."""
    N = 200
    qa, da, qw, dw = _problem(M, N, K, 1000 + M * 31 + K, unit=True)
    say("unit-scale gemm M=%d N=%d K=%d" % (M, N, K))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    want = (qa.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(C.astype(np.float64), want)


NUM_TILES = 10               # compiled matrix-core tile configurations


def _index_problem(M, N, K, which):
    """Index-encoded operands with unit scales: one side one-hot (row m
    selects k = m % K), the other a code of its (row, k) position, so every
    output is one known code and a misplaced operand or result lane (a
    transposed fragment, a swapped half, a wrong row or column of a tile)
    changes it."""
    m = np.arange(M)[:, None]
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    if which == "a_onehot":
        qa = (k == m % K).astype(np.int8)
        qw = ((n * 7 + k * 3) % 251 - 125).astype(np.int8)
    else:
        qa = ((m * 5 + k * 11) % 251 - 125).astype(np.int8)
        qw = (k == n % K).astype(np.int8)
    one = lambda rows: np.full((rows, K // 32), 0x3C00, np.uint16)
    return qa, one(M), qw, one(N)


INDEX_CASES = [(1, 200, 64, None), (5, 200, 96, None), (8, 4100, 64, None), (9, 200, 64, None),
               (40, 4100, 96, None), (64, 200, 64, None), (130, 200, 96, None),
               (300, 1000, 64, None)]


@pytest.mark.parametrize("which", ["a_onehot", "w_onehot"])
@pytest.mark.parametrize("M,N,K,tile", INDEX_CASES + [(300, 1000, 96, t) for t in range(NUM_TILES)])
def test_gemm_lane_layout_index_encoded(orc, monkeypatch, which, M, N, K, tile):
    """Operand and result lane mappings of every kernel (decode, small-M,
    each matrix-core tile), checked exactly with index-encoded inputs."""
    if tile is not None:
        monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    qa, da, qw, dw = _index_problem(M, N, K, which)
    say("index-encoded %s M=%d N=%d K=%d tile %s" % (which, M, N, K, tile))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    want = (qa.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64)
    assert np.array_equal(C.astype(np.float64), want)


SMALL_SHAPES = [(M, 256, 512) for M in range(1, 10)] + [
    (16, 256, 512), (17, 70, 96), (33, 130, 160), (127, 200, 544), (128, 128, 128),
    (129, 64, 32), (255, 257, 1056), (300, 330, 2080), (509, 640, 1024)]


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_gemm_parity_small(orc, M, N, K):
    qa, da, qw, dw = _problem(M, N, K, 7 * M + 13 * N + K)
    say("gemm parity M=%d N=%d K=%d" % (M, N, K))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(C, C_ref, absdot, K, "M%d N%d K%d" % (M, N, K))


# Every compiled tile configuration of the matrix-core kernel (the default
# choice depends on the shape), forced through its benchmarking switch, on
# shapes with ragged M, N and K-stage tails.
TILE_SHAPES = [(9, 64, 32), (130, 200, 544), (300, 330, 2080), (257, 520, 1056)]


@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_gemm_parity_every_tile(orc, monkeypatch, tile, M, N, K):
    monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    qa, da, qw, dw = _problem(M, N, K, 5 * M + 3 * N + K + tile)
    say("gemm tile %d M=%d N=%d K=%d" % (tile, M, N, K))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(C, C_ref, absdot, K, "tile %d M%d N%d K%d" % (tile, M, N, K))


# The weight-streaming kernel for 9 <= M <= 64 (the default there): every
# number of 16-row activation tiles, ragged M and N, one block and many.
@pytest.mark.parametrize("M", [9, 15, 16, 17, 31, 33, 48, 63, 64])
@pytest.mark.parametrize("N,K", [(70, 96), (200, 1056), (1000, 32), (4100, 4096)])
def test_small_m_kernel(orc, M, N, K):
    qa, da, qw, dw = _problem(M, N, K, 3 * M + N + K)
    say("small-M kernel M=%d N=%d K=%d" % (M, N, K))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(C, C_ref, absdot, K, "small M%d N%d K%d" % (M, N, K))


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("M,N,K", [(1, 70, 96), (3, 200, 1056), (8, 130, 2080), (5, 64, 32)])
def test_gemv_parity_every_config(orc, monkeypatch, cfg, M, N, K):
    """Every configuration of the decode kernel (forced through its
    benchmarking switch)."""
    monkeypatch.setenv("Q8_GEMV_CFG", str(cfg))
    qa, da, qw, dw = _problem(M, N, K, 11 * M + N + K + cfg)
    say("gemv cfg %d M=%d N=%d K=%d" % (cfg, M, N, K))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K).cpu().numpy()
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(C, C_ref, absdot, K, "gemv cfg %d M%d N%d K%d" % (cfg, M, N, K))


def test_gemm_tiny_workload_every_m(orc):
    """The tiny workload, through the quantiser, at every M from 1 to 16
    (1..8 take the decode kernel, 9..16 the matrix-core kernel)."""
    layer = workloads.TINY
    N, K = layer.N, layer.K
    x = workloads.activations(layer)
    qw, dw = orc.quantize_rows(workloads.weights(layer))
    say("tiny workload M=1..16")
    wp = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)
    qa_t, da_t = q8.q8_quantize_act(x_to_dev(x))
    qa, da = orc.quantize_rows(x)
    assert np.array_equal(qa_t.cpu().numpy(), qa) and np.array_equal(d_bits(da_t), da)
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    for M in range(1, layer.M + 1):
        C = q8.q8_gemm(qa_t[:M].contiguous(), da_t[:M].contiguous(), wp, N, K).cpu().numpy()
        check_close(C, C_ref[:M], absdot[:M], K, "tiny M=%d" % M)


@pytest.mark.parametrize("M,tile", [(3, None), (40, None), (300, None)] +
                         [(300, t) for t in range(NUM_TILES)])
def test_gemm_guard_bands(orc, monkeypatch, M, tile):
    """Columns past N (ldc > N) and rows past M are never written (the
    default choice, and every matrix-core tile configuration)."""
    if tile is not None:
        monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    N, K, ldc, extra = 70, 160, 96, 5
    qa, da, qw, dw = _problem(M, N, K, 77 + M)
    say("guard bands M=%d N=%d ldc=%d tile %s" % (M, N, ldc, tile))
    out = torch.full((M + extra, ldc), float("nan"), dtype=torch.float32, device=DEV)
    view = out[:M]
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K, out=view)
    assert C.data_ptr() == out.data_ptr()
    host = out.cpu().numpy()
    assert np.all(np.isnan(host[:, N:])), "wrote past column N"
    assert np.all(np.isnan(host[M:])), "wrote past row M"
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(host[:M, :N], C_ref, absdot, K, "guarded")


@pytest.mark.parametrize("tile", [None, 4, 8])
def test_gemm_wide_output_pitch(orc, monkeypatch, tile):
    """An output pitch so wide that a tile's rows span more than 2^31 bytes
    (ldc = 2^23 + 64 floats): the matrix-core kernel then stores with
    per-element checks instead of its buffer range; exactly the M x N
    outputs are written (2.3 GB output allocation)."""
    if tile is not None:
        monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    M, N, K, ldc = 70, 200, 64, (1 << 23) + 64
    qa, da, qw, dw = _problem(M, N, K, 4242)
    say("wide output pitch M=%d N=%d ldc=%d tile %s" % (M, N, ldc, tile))
    flat = torch.full(((M - 1) * ldc + N + 64,), float("nan"), dtype=torch.float32, device=DEV)
    view = flat.as_strided((M, N), (ldc, 1))
    C = _run(qa, da, orc.blocks_from_qd(qw, dw), N, K, out=view)
    assert C.data_ptr() == flat.data_ptr()
    assert int(torch.isfinite(flat).sum()) == M * N, "wrote outside the M x N outputs"
    host = view.cpu().numpy()
    del flat, view, C
    torch.cuda.empty_cache()
    C_ref, absdot = orc.gemm(qa, da, qw, dw)
    check_close(host, C_ref, absdot, K, "wide pitch")


@pytest.mark.parametrize("M,tile", [(4, None), (40, None), (512, None), (512, 4), (512, 5), (512, 7), (512, 9)])
def test_gemm_deterministic(orc, monkeypatch, M, tile):
    """Two calls give the same bits (every sum, including the K groups'
    partial sums, is added in a fixed order)."""
    if tile is not None:
        monkeypatch.setenv("Q8_GEMM_TILE", str(tile))
    N, K = 4096, 4096
    qa, da, qw, dw = _problem(M, N, K, 99 + M)
    say("determinism M=%d N=%d K=%d tile %s" % (M, N, K, tile))
    qt, dt = qd_to_dev(qa, da)
    wp = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)
    C1 = q8.q8_gemm(qt, dt, wp, N, K)
    C2 = q8.q8_gemm(qt, dt, wp, N, K)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_gemm_m_zero():
    say("gemm M=0")
    qt = torch.empty((0, 64), dtype=torch.int8, device=DEV)
    dt = torch.empty((0, 2), dtype=torch.float16, device=DEV)
    wp = torch.zeros(q8.q8_packed_bytes(64, 64), dtype=torch.uint8, device=DEV)
    C = q8.q8_gemm(qt, dt, wp, 64, 64)
    assert C.shape == (0, 64)


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------

FULL_LAYERS = [workloads.DECODE_M1, workloads.DECODE_M4, workloads.PREFILL, workloads.LARGE_UP,
               workloads.LARGE_DOWN] + workloads.sweep(512) + workloads.sweep(509)


# Products up to this size (the prefill workload and every sweep layer) are
# compared in full; the oracle takes a few seconds on the host's cores.
FULL_COMPARE_MACS = 2048 * 12288 * 4096


def _sample_points(M, N, n, seed, tile=128):
    """Outputs the oracle recomputes one by one for the largest products:
    n random outputs; two whole rows and two whole columns; and in every
    tile x tile output tile its four corners, one point on each of its four
    edges and one inside (a tile the kernel left unwritten, or wrote from
    the wrong rows or columns, shows up in all of them)."""
    r = np.random.default_rng(seed)
    rows = [r.integers(0, M, n)]
    cols = [r.integers(0, N, n)]
    for m in sorted({0, M - 1}):
        rows.append(np.full(N, m))
        cols.append(np.arange(N))
    for c in sorted({0, N - 1}):
        rows.append(np.arange(M))
        cols.append(np.full(M, c))
    tm, tn = np.meshgrid(np.arange(0, M, tile), np.arange(0, N, tile), indexing="ij")
    tm, tn = tm.ravel(), tn.ravel()
    last_m = np.minimum(tm + tile, M) - 1
    last_n = np.minimum(tn + tile, N) - 1

    def inside(lo, hi):
        return lo + (r.random(lo.size) * (hi - lo + 1)).astype(np.int64)

    for rr, cc in ((tm, tn), (tm, last_n), (last_m, tn), (last_m, last_n),       # corners
                   (tm, inside(tn, last_n)), (last_m, inside(tn, last_n)),       # top, bottom
                   (inside(tm, last_m), tn), (inside(tm, last_m), last_n),       # left, right
                   (inside(tm, last_m), inside(tn, last_n))):                    # interior
        rows.append(rr)
        cols.append(cc)
    return np.concatenate(rows), np.concatenate(cols)


@pytest.mark.parametrize("layer", FULL_LAYERS, ids=lambda l: l.name)
def test_workload_full_size(orc, layer):
    M, N, K = layer.M, layer.N, layer.K
    say("full size %s: generating" % layer.name)
    x = workloads.activations(layer)
    qw, dw = orc.quantize_rows(workloads.weights(layer))
    qa, da = orc.quantize_rows(x)
    say("full size %s: GPU quantise + pack + gemm" % layer.name)
    wp = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)
    qa_t, da_t = q8.q8_quantize_act(x_to_dev(x))
    # every output written: the buffer starts as NaN
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q8.q8_gemm(qa_t, da_t, wp, N, K, out=C)
    assert bool(torch.isfinite(C).all()), "outputs left unwritten (NaN) or non-finite"
    assert np.array_equal(qa_t.cpu().numpy(), qa), "quantised activations differ"
    assert np.array_equal(d_bits(da_t), da), "activation scales differ"
    if M * N * K <= FULL_COMPARE_MACS:
        say("full size %s: oracle, every output" % layer.name)
        C_ref, absdot = orc.gemm(qa, da, qw, dw)
        check_close(C.cpu().numpy(), C_ref, absdot, K, layer.name)
    else:
        rows, cols = _sample_points(M, N, 4096, M + N + K)
        say("full size %s: oracle, %d sampled outputs (every 128x128 tile)" % (layer.name, rows.size))
        C_ref, absdot = orc.gemm_sampled(qa, da, qw, dw, rows, cols)
        got = C[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].cpu().numpy()
        check_close(got, C_ref, absdot, K, layer.name)


def test_dispatch_log(orc, monkeypatch, capfd):
    """Q8_LOG names the kernel each product call takes (decode for M <= 8,
    the small-M kernel up to 64, a matrix-core tile above), on stderr."""
    monkeypatch.setenv("Q8_LOG", "1")
    for M, want in ((3, "decode kernel"), (40, "small-M matrix-core kernel, 2 row tiles"),
                    (100, "matrix-core kernel, tile")):
        qa, da, qw, dw = _problem(M, 96, 128, 17 * M)
        C = _run(qa, da, orc.blocks_from_qd(qw, dw), 96, 128).cpu().numpy()
        C_ref, absdot = orc.gemm(qa, da, qw, dw)
        check_close(C, C_ref, absdot, 128, "logged M%d" % M)
        err = capfd.readouterr().err
        assert "q8: product M=%d N=96 K=128: %s" % (M, want) in err, err
