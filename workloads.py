"""Seeded synthetic inputs for the Q8_0 weight x activation product.

This module is shared by the tests, the smoke check and the benchmark.  It
holds none of the product's arithmetic: it draws real-valued weights and
activations and, where a workload asks for bfloat16 activations, rounds them
to bfloat16 (round to nearest even) -- the input format, not the method.
Quantisation to Q8_0 is done by each side on its own (the CPU oracle in the
tests, the library's quantiser in the benchmark).

The shapes stand in for the dense layers of the 9B and 27B hybrid models the
source pages run (news.hada.io topic 29953, "CUDA inference engine for
running Qwen3.5/3.6 hybrid models on mining cards (CMP 100-210)", list of
supported models and benchmark list); the pages publish no shapes, weights or
prompts, so every tensor here is drawn from a fixed distribution:

* weights      ~ N(0, 0.02^2), float32, row n = output feature, K contiguous;
* activations  ~ N(0, 1), float32 (tiny case) or rounded to bfloat16;
* down-projection inputs: silu(g) * u with g, u ~ N(0, 1) independent,
  computed in float64, rounded to bfloat16;
* "outlier" activations: round(0.01*K) channels (drawn once per layer,
  shared by every row) multiplied by 50 before rounding to bfloat16.

KV-cache rows (the 3-bit KV-cache codec, same pages, KV-cache item of the
engine's list): the pages give only the context length (256K tokens) and the
bfloat16 size (17 GB).  Rows of D = 256 with 64 rows per token (layers x KV
heads, keys and values each) reproduce that size: 262144 * 64 * 2 * 256 * 2
bytes = 17.2 GB.  Each row is

* kv rows      x[r][i] = z * c_i * g_r with z ~ N(0, 1), per-channel gains
  c_i = exp(0.5 N(0, 1)) (2 % of channels, drawn once per case, times 10:
  the outlier channels of attention keys) and per-row gains g_r = 2^U(-2, 2),
  rounded to bfloat16 where the workload is bfloat16.

Attention inputs (block-sparse prefill attention, same pages, attention item
of the engine's list; no shapes given): token-major bfloat16 Q [L][Hq*D] and
K, V [L][Hkv*D] with block structure for the selection to find -- every
(K/V head, 64-token block) has a topic vector c ~ N(0, 1); K rows are
N(0, 1) + c of their block; every (query head, query block) picks 4 earlier
blocks (uniformly, with repetition) and its Q rows are N(0, 1) + 0.75 times
the sum of those blocks' topics; V rows are N(0, 1).

Streams: numpy ``default_rng(SeedSequence([seed, case, tensor]))``; the
device generator for full-size KV caches uses torch's Philox stream seeded
with the same three numbers folded into one.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


def rng(case: int, tensor: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, case, tensor]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest even.  Inputs are
    finite; NaN handling is not needed for generated data."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights_f32(N: int, K: int, case: int, tensor: int = 0, std: float = 0.02,
                seed: int = 0) -> np.ndarray:
    return (rng(case, tensor, seed).standard_normal((N, K), dtype=np.float32)
            * np.float32(std))


def acts_f32(M: int, K: int, case: int, tensor: int = 1, seed: int = 0) -> np.ndarray:
    return rng(case, tensor, seed).standard_normal((M, K), dtype=np.float32)


def acts_silu_mul(M: int, K: int, case: int, tensor: int = 1, seed: int = 0) -> np.ndarray:
    r = rng(case, tensor, seed)
    out = np.empty((M, K), dtype=np.float32)
    step = max(1, (1 << 22) // max(K, 1))          # bounded float64 temporaries
    for m0 in range(0, M, step):
        m1 = min(M, m0 + step)
        g = r.standard_normal((m1 - m0, K))
        u = r.standard_normal((m1 - m0, K))
        out[m0:m1] = (g / (1.0 + np.exp(-g))) * u
    return out


def acts_outliers(M: int, K: int, case: int, tensor: int = 1, seed: int = 0,
                  frac: float = 0.01, gain: float = 50.0) -> np.ndarray:
    x = rng(case, tensor, seed).standard_normal((M, K), dtype=np.float32)
    x[:, outlier_channels(K, case, seed, frac)] *= np.float32(gain)
    return x


def outlier_channels(K: int, case: int, seed: int = 0, frac: float = 0.01) -> np.ndarray:
    """The round(frac*K) outlier channels of a layer, from their own stream so
    that every M of the same layer shares them."""
    return rng(case, 99, seed).choice(K, size=int(round(frac * K)), replace=False)


def kv_channel_gains(D: int, case: int, seed: int = 0) -> np.ndarray:
    r = rng(case, 98, seed)
    c = np.exp(0.5 * r.standard_normal(D)).astype(np.float32)
    c[r.choice(D, size=max(1, int(round(0.02 * D))), replace=False)] *= np.float32(10.0)
    return c


def kv_rows(R: int, D: int, case: int, tensor: int = 3, seed: int = 0) -> np.ndarray:
    """[R][D] float32 KV-cache rows (see the module docstring)."""
    r = rng(case, tensor, seed)
    z = r.standard_normal((R, D), dtype=np.float32)
    g = np.exp2(r.uniform(-2.0, 2.0, (R, 1))).astype(np.float32)
    return z * kv_channel_gains(D, case, seed)[None, :] * g


def kv_rows_device(R: int, D: int, case: int, device, tensor: int = 3, seed: int = 0):
    """The same distribution as kv_rows, drawn on the device as bfloat16 (for
    caches too large to draw on the host); a different stream from kv_rows."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1000003 + case) * 1000003 + tensor)
    c = torch.from_numpy(kv_channel_gains(D, case, seed)).to(device)
    out = torch.empty((R, D), dtype=torch.bfloat16, device=device)
    step = 1 << 20
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        z = torch.randn((r1 - r0, D), generator=gen, device=device, dtype=torch.float32)
        g = torch.exp2(torch.rand((r1 - r0, 1), generator=gen, device=device) * 4.0 - 2.0)
        out[r0:r1] = (z * c * g).to(torch.bfloat16)
    return out


def attn_qkv(L: int, Hq: int, Hkv: int, D: int, case: int, seed: int = 0):
    """(q, k, v) uint16 bfloat16 bits, token-major (see the module docstring)."""
    r = rng(case, 5, seed)
    NB = (L + 63) // 64
    topic = r.standard_normal((Hkv, NB, D)).astype(np.float32)
    blk = np.arange(L) // 64
    k = r.standard_normal((L, Hkv, D)).astype(np.float32) + topic[:, blk, :].transpose(1, 0, 2)
    picks = (r.random((Hq, NB, 4)) * np.maximum(np.arange(NB), 1)[None, :, None]).astype(np.int64)
    g = np.arange(Hq) // (Hq // Hkv)
    qt = 0.75 * topic[g[:, None, None], picks, :].sum(axis=2)          # [Hq][NB][D]
    q = r.standard_normal((L, Hq, D)).astype(np.float32) + qt[:, blk, :].transpose(1, 0, 2)
    v = r.standard_normal((L, Hkv, D)).astype(np.float32)
    return (f32_to_bf16_bits(q.reshape(L, Hq * D)), f32_to_bf16_bits(k.reshape(L, Hkv * D)),
            f32_to_bf16_bits(v.reshape(L, Hkv * D)))


def attn_qkv_device(L: int, Hq: int, Hkv: int, D: int, case: int, device, seed: int = 0):
    """The distribution of attn_qkv drawn on the device as bfloat16 tensors
    (for sequences too long to draw on the host); a different stream."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1000003 + case) * 1000003 + 5)
    NB = (L + 63) // 64
    topic = torch.randn((Hkv, NB, D), generator=gen, device=device)
    blk = torch.arange(L, device=device) // 64
    k = torch.empty((L, Hkv * D), dtype=torch.bfloat16, device=device)
    v = torch.empty((L, Hkv * D), dtype=torch.bfloat16, device=device)
    q = torch.empty((L, Hq * D), dtype=torch.bfloat16, device=device)
    picks = (torch.rand((Hq, NB, 4), generator=gen, device=device)
             * torch.clamp(torch.arange(NB, device=device), min=1)[None, :, None]).long()
    g = torch.arange(Hq, device=device) // (Hq // Hkv)
    qt = 0.75 * topic[g[:, None, None], picks, :].sum(dim=2)          # [Hq][NB][D]
    step = 8192
    for t0 in range(0, L, step):
        t1 = min(L, t0 + step)
        b = blk[t0:t1]
        kk = torch.randn((t1 - t0, Hkv, D), generator=gen, device=device) + topic[:, b, :].transpose(0, 1)
        k[t0:t1] = kk.reshape(t1 - t0, -1).to(torch.bfloat16)
        v[t0:t1] = torch.randn((t1 - t0, Hkv * D), generator=gen, device=device).to(torch.bfloat16)
        qq = torch.randn((t1 - t0, Hq, D), generator=gen, device=device) + qt[:, b, :].transpose(0, 1)
        q[t0:t1] = qq.reshape(t1 - t0, -1).to(torch.bfloat16)
    return q, k, v


@dataclass(frozen=True)
class Layer:
    """One product C[M][N] = A[M][K] * W[N][K]^T."""
    name: str
    M: int
    N: int
    K: int
    act: str            # "f32", "bf16", "silu_bf16", "outlier_bf16"
    case: int           # seed stream id


def activations(layer: Layer, seed: int = 0, M: Optional[int] = None) -> np.ndarray:
    """Activation rows for a layer: float32 array, or uint16 bfloat16 bits."""
    M = layer.M if M is None else M
    if layer.act == "f32":
        return acts_f32(M, layer.K, layer.case, seed=seed)
    if layer.act == "bf16":
        return f32_to_bf16_bits(acts_f32(M, layer.K, layer.case, seed=seed))
    if layer.act == "silu_bf16":
        return f32_to_bf16_bits(acts_silu_mul(M, layer.K, layer.case, seed=seed))
    if layer.act == "outlier_bf16":
        return f32_to_bf16_bits(acts_outliers(M, layer.K, layer.case, seed=seed))
    raise ValueError(layer.act)


def weights(layer: Layer, seed: int = 0) -> np.ndarray:
    return weights_f32(layer.N, layer.K, layer.case, seed=seed)


# The five workloads.  Case ids keep every tensor on its own stream.
TINY = Layer("tiny M16 N256 K512", 16, 256, 512, "f32", 1)
DECODE_M1 = Layer("decode M1 N12288 K4096", 1, 12288, 4096, "bf16", 2)
DECODE_M4 = Layer("decode M4 N12288 K4096", 4, 12288, 4096, "bf16", 2)
PREFILL = Layer("prefill M2048 N12288 K4096", 2048, 12288, 4096, "bf16", 3)
LARGE_UP = Layer("large up M8192 N17408 K5120", 8192, 17408, 5120, "bf16", 4)
LARGE_DOWN = Layer("large down M8192 N5120 K17408", 8192, 5120, 17408, "silu_bf16", 5)


def sweep(M: int):
    """Chunked-prefill layer sweep, 9B-like shapes, 1% outlier channels x50."""
    return [
        Layer("sweep qkv M%d N6144 K4096" % M, M, 6144, 4096, "outlier_bf16", 6),
        Layer("sweep o M%d N4096 K4096" % M, M, 4096, 4096, "outlier_bf16", 7),
        Layer("sweep gate_up M%d N24576 K4096" % M, M, 24576, 4096, "outlier_bf16", 8),
        Layer("sweep down M%d N4096 K12288" % M, M, 4096, 12288, "outlier_bf16", 9),
    ]


ALL_LAYERS = [TINY, DECODE_M1, DECODE_M4, PREFILL, LARGE_UP, LARGE_DOWN] + sweep(512) + sweep(509)
