"""The fused call q8_gemm_act (quantise on the fly, then multiply) through the
C ABI: bit-identical to q8_quantize_act followed by q8_gemm, and within the
bound of the CPU oracle.  Inputs are seeded (workloads.py)."""
import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import workloads
from gpu_util import DEV, blocks_to_dev, check_close, d_bits, say, x_to_dev

pytestmark = pytest.mark.gpu


def _weights(orc, N, K, seed):
    w = workloads.weights_f32(N, K, case=90, tensor=seed)
    qw, dw = orc.quantize_rows(w)
    return qw, dw, q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)


def _hard_rows(M, K, seed):
    """Blocks over a wide range of scales (binary16-subnormal ones too), blocks
    of half-integer ties with amax 127, and an all-zero block per row."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((M, K))
    x = (x.reshape(M, K // 32, 32) * 2.0 ** r.uniform(-30, 16, (M, K // 32, 1))).reshape(M, K)
    for m, kb in zip(*np.nonzero(r.random((M, K // 32)) < 0.2)):
        blk = np.round(r.uniform(-126, 126, 32) * 2) / 2
        blk[r.integers(32)] = 127 * r.choice([-1, 1])
        x[m, 32 * kb:32 * kb + 32] = blk
    x[:, 32:64] = 0.0
    return x.astype(np.float32)


def _as_dtype(x, dtype):
    return x if dtype == "f32" else workloads.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", [(70, 96), (200, 1056), (130, 2080)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fused_bitidentical_to_two_calls(orc, dtype, N, K, M):
    qw, dw, wp = _weights(orc, N, K, 1)
    xt = x_to_dev(_as_dtype(_hard_rows(M, K, 100 + M + K), dtype))
    say("fused vs two calls %s M=%d N=%d K=%d" % (dtype, M, N, K))
    q_ref, d_ref = q8.q8_quantize_act(xt)
    C_ref = q8.q8_gemm(q_ref, d_ref, wp, N, K)
    q = torch.full_like(q_ref, 77)
    d = torch.full_like(d_ref, 3.0)
    C = q8.q8_gemm_act(xt, wp, N, K, q=q, d=d)
    C_noqd = q8.q8_gemm_act(xt, wp, N, K)
    torch.cuda.synchronize()
    assert torch.equal(q, q_ref), "quantised rows differ"
    assert np.array_equal(d_bits(d), d_bits(d_ref)), "scales differ"
    Cn, Cf, Cr = C.cpu().numpy(), C_noqd.cpu().numpy(), C_ref.cpu().numpy()
    assert np.array_equal(Cn.view(np.uint32), Cr.view(np.uint32)), "C differs from the two calls"
    assert np.array_equal(Cf.view(np.uint32), Cr.view(np.uint32)), "C (no q/d) differs"
    # and against the oracle
    qa, da = orc.quantize_rows(_as_dtype(_hard_rows(M, K, 100 + M + K), dtype))
    C_o, absdot = orc.gemm(qa, da, qw, dw)
    check_close(Cn, C_o, absdot, K, "fused %s M%d" % (dtype, M))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K", [(70, 96), (200, 1056), (130, 2080)])
@pytest.mark.parametrize("M", [9, 16, 31, 32, 33, 47, 64])
def test_fused_small_m_bitidentical_to_two_calls(orc, monkeypatch, dtype, N, K, M):
    """9 <= M <= 64 with Q8_GEMM_ACT_FUSED=1: the small-M kernel quantises
    its own chunks; C, q and d are bit-identical to the two calls (ragged N,
    K not a multiple of a chunk, blocks over the whole binary16 range)."""
    monkeypatch.setenv("Q8_GEMM_ACT_FUSED", "1")
    qw, dw, wp = _weights(orc, N, K, 4)
    x = _as_dtype(_hard_rows(M, K, 300 + M + K), dtype)
    xt = x_to_dev(x)
    say("fused small-M vs two calls %s M=%d N=%d K=%d" % (dtype, M, N, K))
    q_ref, d_ref = q8.q8_quantize_act(xt)
    C_ref = q8.q8_gemm(q_ref, d_ref, wp, N, K)
    q = torch.full_like(q_ref, 77)
    d = torch.full_like(d_ref, 3.0)
    C = q8.q8_gemm_act(xt, wp, N, K, q=q, d=d)
    torch.cuda.synchronize()
    assert torch.equal(q, q_ref), "quantised rows differ"
    assert np.array_equal(d_bits(d), d_bits(d_ref)), "scales differ"
    Cn, Cr = C.cpu().numpy(), C_ref.cpu().numpy()
    assert np.array_equal(Cn.view(np.uint32), Cr.view(np.uint32)), "C differs from the two calls"
    qa, da = orc.quantize_rows(x)
    C_o, absdot = orc.gemm(qa, da, qw, dw)
    check_close(Cn, C_o, absdot, K, "fused small-M %s M%d" % (dtype, M))


@pytest.mark.parametrize("M", [9, 33, 64])
def test_fused_small_m_full_decode_shape(orc, monkeypatch, M):
    """N12288 K4096 (the decode layer) at small batches, bf16 rows, fused
    small-M kernel: every output against the two calls, sampled outputs
    against the oracle."""
    monkeypatch.setenv("Q8_GEMM_ACT_FUSED", "1")
    N, K = 12288, 4096
    qw, dw = orc.quantize_rows(workloads.weights_f32(N, K, case=91, tensor=0))
    wp = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)
    x = workloads.f32_to_bf16_bits(_hard_rows(M, K, 500 + M))
    xt = x_to_dev(x)
    say("fused small-M full decode shape M=%d" % M)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    C = q8.q8_gemm_act(xt, wp, N, K, out=out).cpu().numpy()
    q_ref, d_ref = q8.q8_quantize_act(xt)
    C2 = q8.q8_gemm(q_ref, d_ref, wp, N, K).cpu().numpy()
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32))
    qa, da = orc.quantize_rows(x)
    r = np.random.default_rng(5)
    rows, cols = r.integers(0, M, 512), r.integers(0, N, 512)
    C_o, absdot = orc.gemm_sampled(qa, da, qw, dw, rows, cols)
    check_close(C[rows, cols], C_o, absdot, K, "fused small-M full M%d" % M)


@pytest.mark.parametrize("M", [65, 130])
def test_fused_prefill_sizes_use_two_kernels(orc, M):
    N, K = 200, 544
    qw, dw, wp = _weights(orc, N, K, 2)
    xt = x_to_dev(_hard_rows(M, K, 7 + M))
    say("fused M=%d (two kernels)" % M)
    q_ref, d_ref = q8.q8_quantize_act(xt)
    C_ref = q8.q8_gemm(q_ref, d_ref, wp, N, K)
    C = q8.q8_gemm_act(xt, wp, N, K)          # binding allocates q, d for M > 8
    assert torch.equal(C.view(torch.int32), C_ref.view(torch.int32))


@pytest.mark.parametrize("layer", [workloads.DECODE_M1, workloads.DECODE_M4], ids=lambda l: l.name)
def test_fused_decode_workload(orc, layer):
    """The decode workloads at full size (bf16 activations), sampled outputs
    against the oracle and every output against the two-call path."""
    N, K, M = layer.N, layer.K, layer.M
    qw, dw = orc.quantize_rows(workloads.weights(layer))
    wp = q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)
    x = workloads.activations(layer)
    xt = x_to_dev(x)
    say("fused decode workload %s" % layer.name)
    C = q8.q8_gemm_act(xt, wp, N, K).cpu().numpy()
    q_ref, d_ref = q8.q8_quantize_act(xt)
    C2 = q8.q8_gemm(q_ref, d_ref, wp, N, K).cpu().numpy()
    assert np.array_equal(C.view(np.uint32), C2.view(np.uint32))
    qa, da = orc.quantize_rows(x)
    r = np.random.default_rng(3)
    rows, cols = r.integers(0, M, 256), r.integers(0, N, 256)
    C_o, absdot = orc.gemm_sampled(qa, da, qw, dw, rows, cols)
    check_close(C[rows, cols], C_o, absdot, K, "fused %s" % layer.name)


@pytest.mark.parametrize("M,fused", [(3, "0"), (40, "0"), (40, "1")])
def test_fused_row_pitch_and_output_pitch(orc, monkeypatch, M, fused):
    """x with ldx > K and C with ldc > N: only the first K columns are read,
    only the first N columns written (decode kernel, quantise + small-M
    kernel, and the fused small-M kernel)."""
    monkeypatch.setenv("Q8_GEMM_ACT_FUSED", fused)
    N, K, ldx, ldc = 70, 160, 256, 96
    qw, dw, wp = _weights(orc, N, K, 3)
    x = _hard_rows(M, ldx, 55)
    xt = x_to_dev(x)
    out = torch.full((M, ldc), float("nan"), dtype=torch.float32, device=DEV)
    q8.q8_gemm_act(xt, wp, N, K, out=out[:, :N].as_strided((M, N), (ldc, 1)))
    host = out.cpu().numpy()
    assert np.all(np.isnan(host[:, N:]))
    qa, da = orc.quantize_rows(x[:, :K])
    C_o, absdot = orc.gemm(qa, da, qw, dw)
    check_close(host[:, :N], C_o, absdot, K, "pitched")


def test_fused_dispatch_log(orc, monkeypatch, capfd):
    """Q8_LOG: q8_gemm_act takes the fused decode kernel for M <= 8; up to
    64 the quantiser then the small-M kernel, or with Q8_GEMM_ACT_FUSED=1
    the small-M kernel quantising its rows; two kernels above."""
    monkeypatch.setenv("Q8_LOG", "1")
    N, K = 96, 128
    qw, dw, wp = _weights(orc, N, K, 6)
    for M, fused, want in ((3, "1", "fused decode kernel"),
                           (40, "0", "small-M matrix-core kernel, 2 row tiles"),
                           (40, "1", "small-M matrix-core kernel quantising its rows"),
                           (100, "1", "matrix-core kernel, tile")):
        monkeypatch.setenv("Q8_GEMM_ACT_FUSED", fused)
        xt = x_to_dev(_hard_rows(M, K, 11 + M))
        q8.q8_gemm_act(xt, wp, N, K)
        torch.cuda.synchronize()
        err = capfd.readouterr().err
        assert want in err, (M, err)
