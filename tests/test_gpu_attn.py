"""Block-sparse causal attention (q8_attn_pool / q8_attn_select / q8_attn_fwd)
through the C ABI, against the CPU oracle.

Bars (include/q8.h):
  - pooled means: binary32 sums of <= 64 bfloat16 values, within
    64 * 2^-24 * mean|x| + tiny of the oracle's double;
  - selection: the same block sets, except that a block whose oracle score
    lies within eps of the cut (the (k-2)'th best score) may be swapped for
    another such block; eps bounds the binary32 error of a score;
  - output, given the same lists: |out - exact| <= 1.25 * 2^-8 * mag
    (+ 2^-8 |exact| for bfloat16 output), mag = sum p |v| / sum p from the
    oracle: p is rounded to bfloat16 for the product with V.
Inputs are seeded (workloads.py)."""
import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import workloads
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def _host_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _check_out(got, ref, mag, bf16_out, what):
    got = np.asarray(got, dtype=np.float64)
    tol = 1.25 * 2.0 ** -8 * mag + 1e-6
    if bf16_out:
        tol = tol + 1.01 * 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    bad = np.nonzero(~(err <= tol))
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError("%s: %d outputs off; first %s: got %r want %r mag %r"
                             % (what, bad[0].size, i, got[i], ref[i], mag[i]))
    return float(np.max(err / np.maximum(mag, 1e-30)))


def _check_lists(idx_g, cnt_g, pq, pk, k, rows):
    """GPU lists for the given (K/V head, block) rows, against the selection
    rule applied to the oracle's pooled rows (double): block 0 and the
    diagonal, then every candidate whose score (the group's summed pooled
    query row against the pooled key row) lies clearly above the cut ((k-2)'th
    best score) and none clearly below it; within eps of the cut either choice
    is right.  eps bounds the binary32 error of a GPU score."""
    Hq, Hkv = pq.shape[0], pk.shape[0]
    G = Hq // Hkv
    assert idx_g.shape[0] == Hkv and cnt_g.shape == (Hkv, pq.shape[1])
    for g, i in rows:
        n = min(k, i + 1)
        assert int(cnt_g[g, i]) == n, (g, i, cnt_g[g, i], n)
        a = [int(j) for j in idx_g[g, i, :n]]
        assert a == sorted(set(a)) and 0 in a and i in a and max(a) <= i, (g, i, a)
        assert np.all(idx_g[g, i, n:] == -1), (g, i)
        if k >= i + 1:
            assert a == list(range(i + 1))
            continue
        q = pq[g * G:(g + 1) * G, i].sum(axis=0)
        qa = np.abs(pq[g * G:(g + 1) * G, i]).sum(axis=0)
        cand = list(range(1, i))
        sc = np.array([q @ pk[g, j] for j in cand])
        eps = 5e-5 * np.array([qa @ np.abs(pk[g, j]) for j in cand]) + 1e-6
        cut = np.sort(sc)[::-1][k - 3] if k > 2 else np.inf
        chosen = set(a) - {0, i}
        for j, s_, e in zip(cand, sc, eps):
            if s_ > cut + e:
                assert j in chosen, (g, i, j, s_, cut)
            elif s_ < cut - e:
                assert j not in chosen, (g, i, j, s_, cut)


def _run(orc, L, Hq, Hkv, D, k, case, out_dtype=torch.bfloat16, pitch=0):
    qb, kb, vb = workloads.attn_qkv(L, Hq, Hkv, D, case)
    if pitch:
        pad = lambda a: np.concatenate([a, np.zeros((L, pitch), np.uint16)], axis=1)
        qb, kb, vb = pad(qb), pad(kb), pad(vb)
    qt, kt, vt = _dev_bf16(qb), _dev_bf16(kb), _dev_bf16(vb)
    if pitch:
        qt, kt, vt = qt[:, :Hq * D], kt[:, :Hkv * D], vt[:, :Hkv * D]
    return qb, kb, vb, qt, kt, vt


@pytest.mark.parametrize("L,H,D", [(64, 2, 64), (100, 3, 128), (1000, 4, 64), (1111, 2, 128)])
def test_attn_pool(orc, L, H, D):
    xb = workloads.attn_qkv(L, H, H, D, 31)[0]
    say("attn pool L=%d H=%d D=%d" % (L, H, D))
    got = q8.q8_attn_pool(_dev_bf16(xb), H, D).cpu().numpy().astype(np.float64)
    ref = orc.attn_pool(xb, H, D)
    w = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(L, H, D)
    scale = np.abs(w).max()
    assert np.max(np.abs(got - ref)) <= 64 * 2.0 ** -24 * scale + 1e-30


@pytest.mark.parametrize("L,Hq,Hkv,D,k", [(640, 4, 2, 64, 4), (1111, 4, 1, 128, 3),
                                          (2048, 2, 2, 128, 8), (3000, 8, 2, 64, 2),
                                          (700, 2, 1, 128, 64)])
def test_attn_select(orc, L, Hq, Hkv, D, k):
    qb, kb, _ = workloads.attn_qkv(L, Hq, Hkv, D, 40 + k)
    pq, pk = orc.attn_pool(qb, Hq, D), orc.attn_pool(kb, Hkv, D)
    idx_o, cnt_o = orc.attn_select(pq, pk, k, kmax=k + 2)
    say("attn select L=%d Hq=%d Hkv=%d D=%d k=%d" % (L, Hq, Hkv, D, k))
    pqt = q8.q8_attn_pool(_dev_bf16(qb), Hq, D)
    pkt = q8.q8_attn_pool(_dev_bf16(kb), Hkv, D)
    idx, cnt = q8.q8_attn_select(pqt, pkt, k, kmax=k + 2)
    NB = (L + 63) // 64
    rows = [(g, i) for g in range(Hkv) for i in range(NB)]
    _check_lists(idx.cpu().numpy(), cnt.cpu().numpy(), pq, pk, k, rows)
    # the oracle's own lists satisfy the same rule (and equal the GPU's
    # wherever no score sits near the cut)
    _check_lists(idx_o, cnt_o, pq, pk, k, rows)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("L,Hq,Hkv,D,k", [(64, 2, 1, 64, 2), (100, 4, 2, 128, 2),
                                          (640, 4, 2, 64, 4), (1111, 2, 2, 128, 5),
                                          (1000, 8, 2, 128, 100), (777, 4, 4, 64, 3),
                                          # groups of 8, 6 and 3 query heads: a group
                                          # spans 2 or 3 workgroups of 4, 2 or 1 heads
                                          (500, 16, 2, 128, 4), (300, 12, 2, 64, 3),
                                          (257, 9, 3, 128, 2)])
def test_attn_fwd(orc, L, Hq, Hkv, D, k, out_dtype):
    """The oracle's lists fed to the kernel; output within the bar."""
    qb, kb, vb, qt, kt, vt = _run(orc, L, Hq, Hkv, D, k, 50 + L % 97)
    idx_o, cnt_o = orc.attn_select(orc.attn_pool(qb, Hq, D), orc.attn_pool(kb, Hkv, D), k)
    ref, mag = orc.attn_fwd(qb, kb, vb, Hq, Hkv, D, idx_o, cnt_o)
    say("attn fwd L=%d Hq=%d Hkv=%d D=%d k=%d %s" % (L, Hq, Hkv, D, k, out_dtype))
    out = q8.q8_attn_fwd(qt, kt, vt, Hq, Hkv, D, torch.from_numpy(idx_o).to(DEV),
                         torch.from_numpy(cnt_o).to(DEV), out_dtype=out_dtype)
    _check_out(out.float().cpu().numpy(), ref, mag, out_dtype == torch.bfloat16,
               "L=%d Hq=%d D=%d k=%d" % (L, Hq, D, k))


def test_attn_fwd_pitch(orc):
    L, Hq, Hkv, D, k = 300, 4, 2, 128, 3
    qb, kb, vb, qt, kt, vt = _run(orc, L, Hq, Hkv, D, k, 77, pitch=64)
    idx_o, cnt_o = orc.attn_select(orc.attn_pool(qb, Hq, D), orc.attn_pool(kb, Hkv, D), k)
    ref, mag = orc.attn_fwd(qb, kb, vb, Hq, Hkv, D, idx_o, cnt_o)
    for dt, extra in ((torch.float32, 4), (torch.bfloat16, 8)):
        buf = torch.full((L, Hq * D + extra), 7.0, dtype=dt, device=DEV)
        q8.q8_attn_fwd(qt, kt, vt, Hq, Hkv, D, torch.from_numpy(idx_o).to(DEV),
                       torch.from_numpy(cnt_o).to(DEV), out=buf)
        got = buf.float().cpu().numpy()
        assert np.all(got[:, Hq * D:] == 7.0), "wrote past Hq*D"
        _check_out(got[:, :Hq * D], ref, mag, dt == torch.bfloat16, "pitch")


def test_attn_end_to_end(orc):
    """Pool, select and attend on the GPU; the oracle attends over the GPU's
    lists (integers, so the same input) and the lists are valid."""
    L, Hq, Hkv, D, k = 2500, 8, 2, 128, 6
    qb, kb, vb, qt, kt, vt = _run(orc, L, Hq, Hkv, D, k, 91)
    say("attn end to end L=%d" % L)
    idx, cnt = q8.q8_attn_select(q8.q8_attn_pool(qt, Hq, D), q8.q8_attn_pool(kt, Hkv, D), k)
    out = q8.q8_attn_fwd(qt, kt, vt, Hq, Hkv, D, idx, cnt, out_dtype=torch.float32)
    idx_g, cnt_g = idx.cpu().numpy(), cnt.cpu().numpy()
    pq, pk = orc.attn_pool(qb, Hq, D), orc.attn_pool(kb, Hkv, D)
    _check_lists(idx_g, cnt_g, pq, pk, k, [(g, i) for g in range(Hkv) for i in range((L + 63) // 64)])
    ref, mag = orc.attn_fwd(qb, kb, vb, Hq, Hkv, D, idx_g, cnt_g)
    _check_out(out.cpu().numpy(), ref, mag, False, "end to end")


def test_attn_list_entries_outside_range_are_skipped(orc):
    """Entries outside [0, i] are skipped and cnt is clamped to kmax: the
    output equals attention over the remaining entries."""
    L, Hq, Hkv, D = 400, 4, 2, 64
    qb, kb, vb, qt, kt, vt = _run(orc, L, Hq, Hkv, D, 4, 93)
    NB = (L + 63) // 64
    kmax = 5
    idx = np.full((Hkv, NB, kmax), -1, np.int32)
    cnt = np.zeros((Hkv, NB), np.int32)
    clean = np.full((Hkv, NB, kmax), -1, np.int32)
    ccnt = np.zeros((Hkv, NB), np.int32)
    for h in range(Hkv):
        for i in range(NB):
            good = sorted(set([0, i] + ([i // 2] if i > 2 else [])))
            raw = [-3] + good + [i + 1 + h, NB + 7][: kmax - 1 - len(good)]
            idx[h, i, :len(raw)] = raw
            cnt[h, i] = 1000 if (h + i) % 2 else len(raw)      # clamped to kmax
            clean[h, i, :len(good)] = good
            ccnt[h, i] = len(good)
    ref, mag = orc.attn_fwd(qb, kb, vb, Hq, Hkv, D, clean, ccnt)
    out = q8.q8_attn_fwd(qt, kt, vt, Hq, Hkv, D, torch.from_numpy(idx).to(DEV),
                         torch.from_numpy(cnt).to(DEV), out_dtype=torch.float32)
    _check_out(out.cpu().numpy(), ref, mag, False, "skipped entries")


def test_attn_bench_workload_sampled(orc):
    """The benchmark's layer (64K tokens, 32 query heads over 8 K/V heads,
    D = 128, 64 blocks per query block), in the launches the benchmark
    times; 48 sampled (token, head) outputs (the first and last tokens
    included) against the oracle over the GPU's lists, and the lists of 16
    sampled (K/V head, block) rows checked against the oracle's scores."""
    L, Hq, Hkv, D, k = 65536, 32, 8, 128, 64
    qt, kt, vt = workloads.attn_qkv_device(L, Hq, Hkv, D, 700, DEV)
    say("attn bench workload L=%d" % L)
    pqt, pkt = q8.q8_attn_pool(qt, Hq, D), q8.q8_attn_pool(kt, Hkv, D)
    idx, cnt = q8.q8_attn_select(pqt, pkt, k)
    out = q8.q8_attn_fwd(qt, kt, vt, Hq, Hkv, D, idx, cnt)
    torch.cuda.synchronize()
    qb, kb, vb = _host_bits(qt), _host_bits(kt), _host_bits(vt)
    idx_g, cnt_g = idx.cpu().numpy(), cnt.cpu().numpy()
    r = np.random.default_rng(9)
    tok = np.concatenate([[0, L - 1, L - 64, 64 * 700 + 5], r.integers(0, L, 44)])
    head = r.integers(0, Hq, tok.size)
    ref, mag = orc.attn_fwd_at(qb, kb, vb, Hq, Hkv, D, idx_g, cnt_g, tok, head)
    got = out.float().cpu().numpy()
    got = np.stack([got[t, h * D:(h + 1) * D] for t, h in zip(tok, head)])
    _check_out(got, ref, mag, True, "bench layer")
    pq, pk = orc.attn_pool(qb, Hq, D), orc.attn_pool(kb, Hkv, D)
    rows = list(zip(r.integers(0, Hkv, 16).tolist(),
                    [1023, 1022, 63, 64] + r.integers(0, 1024, 12).tolist()))
    _check_lists(idx_g, cnt_g, pq, pk, k, rows)
