"""The 3-bit KV-cache codec (q8_kv3_encode / q8_kv3_decode) through the C ABI,
against the CPU oracle.  The format fixes the order of every binary32
operation (include/q8.h), so the bar is bit-exact: codes, scales and decoded
values equal the oracle's bit for bit.  Inputs are seeded (workloads.py)."""
import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import workloads
from gpu_util import DEV, say, x_to_dev

pytestmark = pytest.mark.gpu


def _edge_rows(D):
    """Rows that reach the format's special cases."""
    rows = []
    rows.append(np.zeros(D))                                  # s = 0: every code 4
    e = np.zeros(D); e[3] = 1.0; rows.append(e)               # H e = +-1 everywhere
    rows.append(np.full(D, 0.75))                             # all energy in y_0
    rows.append(workloads.kv_rows(1, D, 70)[0] * 2.0 ** -70)   # subnormal squares, s normal
    rows.append(workloads.kv_rows(1, D, 71)[0] * 2.0 ** -120)  # squares underflow
    rows.append(workloads.kv_rows(1, D, 72)[0] * 2.0 ** -140)  # values subnormal, s < FLT_MIN
    rows.append(workloads.kv_rows(1, D, 73)[0] * 2.0 ** 40)    # large, squares still finite
    t = np.zeros(D); t[0] = 1e-30; rows.append(t)              # tiny one-hot
    return np.array(rows, dtype=np.float32)


def _inputs(R, D, dtype, seed, pitch=0):
    x = workloads.kv_rows(R, D, 500 + seed)
    edge = _edge_rows(D)
    x[: min(R, len(edge))] = edge[: min(R, len(edge))]
    if pitch:
        x = np.concatenate([x, np.full((R, pitch), 9.0, dtype=np.float32)], axis=1)
    return x if dtype == "f32" else workloads.f32_to_bf16_bits(x)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _encode_check(orc, x_np, D, what):
    xt = x_to_dev(x_np)
    if x_np.shape[1] != D:
        xt = xt[:, :D]
    say("kv3 encode", what)
    codes, scales = q8.q8_kv3_encode(xt)
    torch.cuda.synchronize()
    c_ref, s_ref = orc.kv3_encode(x_np, D)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.nonzero(np.any(c != c_ref, axis=1))[0]
    assert bad.size == 0, "%s: %d rows with wrong codes; first row %d: %s vs %s" % (
        what, bad.size, bad[0], c[bad[0]][:12], c_ref[bad[0]][:12])
    assert np.array_equal(_bits(s), _bits(s_ref)), "%s: scales differ at rows %s" % (
        what, np.nonzero(_bits(s) != _bits(s_ref))[0][:8])
    return c_ref, s_ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("R", [1, 3, 4, 7, 1001])
def test_kv3_encode_bitexact(orc, D, dtype, R):
    _encode_check(orc, _inputs(R, D, dtype, R + D), D, "%s R=%d D=%d" % (dtype, R, D))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_kv3_encode_pitch(orc, D, dtype):
    _encode_check(orc, _inputs(37, D, dtype, 7, pitch=24), D, "%s pitch D=%d" % (dtype, D))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("R", [1, 7, 1001])
def test_kv3_encode_guard_bands(orc, D, R):
    """Codes and scales are written exactly where the rows go: sentinel rows
    before and after each output stay intact."""
    x_np = _inputs(R, D, "bf16", 11 + R)
    say("kv3 encode guard bands R=%d D=%d" % (R, D))
    row, pad = 3 * D // 8, 64                    # pad keeps the outputs 16-byte aligned
    cbuf = torch.full((pad + R * row + pad,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((16 + R + 16,), -7.0, dtype=torch.float32, device=DEV)
    q8.q8_kv3_encode(x_to_dev(x_np), codes=cbuf[pad:pad + R * row].view(R, row),
                     scales=sbuf[16:16 + R])
    c, s = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(c[:pad] == 0xA5) and np.all(c[pad + R * row:] == 0xA5), \
        "codes written outside their rows"
    assert np.all(s[:16] == -7.0) and np.all(s[16 + R:] == -7.0), "scales written outside their rows"
    c_ref, s_ref = orc.kv3_encode(x_np, D)
    assert np.array_equal(c[pad:pad + R * row].reshape(R, row), c_ref)
    assert np.array_equal(_bits(s[16:16 + R]), _bits(s_ref))


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("R", [1, 5, 1001])
def test_kv3_decode_bitexact(orc, D, R):
    """Decode the oracle's codes (so the input does not come from the kernel
    under test): binary32 output bit-exact, bfloat16 output the binary32
    value rounded to nearest even."""
    x = _inputs(R, D, "f32", 3 * R + D)
    c_ref, s_ref = orc.kv3_encode(x, D)
    out_ref = orc.kv3_decode(c_ref, s_ref, D)
    ct = torch.from_numpy(c_ref).to(DEV)
    st = torch.from_numpy(s_ref).to(DEV)
    say("kv3 decode R=%d D=%d" % (R, D))
    out = q8.q8_kv3_decode(ct, st, D).cpu().numpy()
    assert np.array_equal(_bits(out), _bits(out_ref)), "decode differs at rows %s" % (
        np.nonzero(np.any(_bits(out) != _bits(out_ref), axis=1))[0][:8])
    ob = q8.q8_kv3_decode(ct, st, D, dtype=torch.bfloat16)
    ob = ob.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ob, workloads.f32_to_bf16_bits(out_ref))


def test_kv3_decode_pitch(orc):
    D, R = 128, 33
    x = _inputs(R, D, "f32", 11)
    c_ref, s_ref = orc.kv3_encode(x, D)
    out_ref = orc.kv3_decode(c_ref, s_ref, D)
    ct, st = torch.from_numpy(c_ref).to(DEV), torch.from_numpy(s_ref).to(DEV)
    for dt, pad in ((torch.float32, 4), (torch.bfloat16, 8)):
        buf = torch.full((R, D + pad), 5.0, dtype=dt, device=DEV)
        q8.q8_kv3_decode(ct, st, D, out=buf)
        got = buf.float().cpu().numpy()
        assert np.all(got[:, D:] == 5.0), "decode wrote past D"
        want = out_ref if dt == torch.float32 else workloads.bf16_bits_to_f32(
            workloads.f32_to_bf16_bits(out_ref))
        assert np.array_equal(_bits(got[:, :D]), _bits(want))


def test_kv3_overflowing_row_matches(orc):
    """A row whose sum of squares overflows binary32: s = inf, every code 4,
    on both sides (the decoded row is NaN on both)."""
    D = 128
    x = workloads.kv_rows(4, D, 81)
    x[1] *= np.float32(2.0 ** 100)
    c_ref, s_ref = orc.kv3_encode(x, D)
    assert np.isinf(s_ref[1]) and np.all(c_ref[1] == np.array([0x24, 0x49, 0x92] * (D // 8), np.uint8))
    _encode_check(orc, x, D, "overflow row")


def test_kv3_zero_rows_is_noop():
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    codes, scales = q8.q8_kv3_encode(x)
    assert codes.shape == (0, 48) and scales.shape == (0,)
    assert q8.q8_kv3_decode(codes, scales, 128).shape == (0, 128)


def test_kv3_layer_workload_sampled(orc):
    """One layer's keys and values at 256K context (262144 tokens x 4 KV
    heads x 2, D = 256, bfloat16), encoded and decoded in the launch
    configuration the benchmark times; 4096 sampled rows checked bit-exact
    against the oracle."""
    R, D = 262144 * 8, 256
    x = workloads.kv_rows_device(R, D, 600, DEV)
    say("kv3 layer workload R=%d D=%d" % (R, D))
    codes, scales = q8.q8_kv3_encode(x)
    out = q8.q8_kv3_decode(codes, scales, D, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(5).choice(R, 4096, replace=False))
    idx[0], idx[-1] = 0, R - 1                      # the first and the last row
    it = torch.from_numpy(idx).to(DEV)
    xs = x[it].cpu().view(torch.int16).numpy().view(np.uint16)
    c_ref, s_ref = orc.kv3_encode(xs, D)
    assert np.array_equal(codes[it].cpu().numpy(), c_ref)
    assert np.array_equal(_bits(scales[it].cpu().numpy()), _bits(s_ref))
    o_ref = workloads.f32_to_bf16_bits(orc.kv3_decode(c_ref, s_ref, D))
    assert np.array_equal(out[it].cpu().view(torch.int16).numpy().view(np.uint16), o_ref)
