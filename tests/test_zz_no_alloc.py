"""q8_gemm_act_noalloc (the allocation-free q8_gemm_act) through the C ABI:
bit-identical to q8_gemm_act on two calls in a row (the second smaller, so
the shared workspace holds the first call's rows when it starts), for the
matrix-core path (rows through the library's static workspace) and the
decode path (none); rows beyond the workspace are refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import int8_block_scaled_amd as q8
import workloads
from gpu_util import DEV, blocks_to_dev, say

pytestmark = pytest.mark.gpu


def _weights(orc, N, K, case):
    w = workloads.acts_f32(N, K, case=case, tensor=1) * np.float32(0.02)
    qw, dw = orc.quantize_rows(w)
    return q8.q8_pack_weights(blocks_to_dev(orc.blocks_from_qd(qw, dw)), N, K)


def _acts(M, K, case, bf16=True):
    x = torch.from_numpy(workloads.acts_f32(M, K, case=case, tensor=2)).to(DEV)
    return x.to(torch.bfloat16) if bf16 else x


@pytest.mark.parametrize("bf16", [True, False])
def test_noalloc_matches_gemm_act_twice(orc, bf16):
    N, K = 1024, 2048
    wp = _weights(orc, N, K, 301)
    for M in (700, 300, 5):                      # second and third calls smaller
        x = _acts(M, K, 302 + M, bf16)
        say("noalloc M=%d N=%d K=%d bf16=%s" % (M, N, K, bf16))
        ref = q8.q8_gemm_act(x, wp, N, K)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        q8.q8_gemm_act_noalloc(x, wp, N, K, out=out)      # result lands in out
        assert torch.cuda.memory_allocated() == before
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), "M=%d differs" % M


def test_noalloc_largest_workload_fits(orc):
    """The prefill rows (2048 x 4096, 8.9 MB) go through the workspace."""
    M, N, K = 2048, 512, 4096
    wp = _weights(orc, N, K, 303)
    x = _acts(M, K, 304)
    say("noalloc prefill rows M=%d K=%d" % (M, K))
    ref = q8.q8_gemm_act(x, wp, N, K)
    got = q8.q8_gemm_act_noalloc(x, wp, N, K)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


def test_noalloc_refuses_rows_beyond_workspace():
    """M x K beyond the 48 MiB workspace: Q8_ERR_SIZE from the host check,
    before anything is enqueued (stand-in pointers, never dereferenced)."""
    L = q8.lib()
    P = ctypes.c_void_p(0x100000)
    assert L.q8_gemm_act_noalloc(P, 1, 8192, 256, 17408, 17408, P, P, 256, None) == 5
    assert L.q8_gemm_act_noalloc(P, 1, 48 * 1024, 256, 1024, 1024, P, P, 256, None) == 5
