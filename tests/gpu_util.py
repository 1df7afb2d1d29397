"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library through its Python binding (which calls the C ABI), and compare
with the CPU oracle.  Tolerances follow include/q8.h: quantised ints and
scales bit-exact; C within 1e-4 of the abs-dot magnitude and within the
analytic binary32 bound (K/32 + 2) * 2^-24 * absdot."""
import numpy as np
import torch

import int8_block_scaled_amd as q8

DEV = torch.device("cuda:0")
REL_TOL = 1e-4


def say(*a):
    print(*a, flush=True)


def x_to_dev(x: np.ndarray) -> torch.Tensor:
    """float32 array, or uint16 bfloat16 bits -> device tensor."""
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    assert x.dtype == np.uint16
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)


def d_bits(d: torch.Tensor) -> np.ndarray:
    return d.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def blocks_to_dev(blocks: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(blocks).reshape(-1)).to(DEV)


def qd_to_dev(q: np.ndarray, d: np.ndarray):
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(DEV)
    dt = torch.from_numpy(np.ascontiguousarray(d).view(np.int16)).to(DEV).view(torch.float16)
    return qt, dt


def check_close(C_gpu: np.ndarray, C_ref: np.ndarray, absdot: np.ndarray, K: int, what=""):
    """Element by element: |C - C_ref| <= min(1e-4, (K/32+2) 2^-24) * absdot,
    and C == 0 exactly where absdot == 0."""
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    assert C_gpu.shape == C_ref.shape, (C_gpu.shape, C_ref.shape)
    assert np.all(np.isfinite(C_gpu)), "%s: non-finite output" % what
    err = np.abs(C_gpu - C_ref)
    bound = (K / 32 + 2) * 2.0 ** -24
    tol = min(REL_TOL, bound) * absdot
    bad = np.nonzero(err > tol)
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError("%s: %d outputs off; first at %s: got %r want %r absdot %r (rel %g)"
                             % (what, bad[0].size, i, C_gpu[i], C_ref[i], absdot[i],
                                err[i] / max(absdot[i], 1e-300)))
    rel = float(np.max(err / np.maximum(absdot, 1e-300)))
    return rel
