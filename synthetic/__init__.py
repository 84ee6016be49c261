"""Seeded synthetic inputs shaped like the OPT layers the RPTQ write-up evaluates.

This module only draws random inputs.  It holds none of the method's
arithmetic (no LayerNorm, clustering, quantization or packing), so both the
oracle and the HIP library can be fed from it without sharing code.

Activation model (per channel c of K):
    mu_c ~ N(0, 2)  (2 is the standard deviation),  sigma_c ~ LogNormal(0, 1),
    a fraction of channels (1% by default) are outliers with mu_c and sigma_c
    both multiplied by 100 -- the write-up's Fig. 1 shows channels whose max or
    min is hundreds of times larger than the others, and channels whose ranges
    differ widely;
    x[t, c] = fp16(mu_c + sigma_c * eps),  eps ~ N(0, 1), saturated to +-65504.
The "range-ratio" variant draws sigma_c = ratio ** U(0, 1) with no outliers,
so channel ranges span a factor of up to `ratio`.
Weights: W ~ N(0, 0.02), fp32 [K][N] (y = x W).
LayerNorm parameters: gamma = 1, beta = 0 (default init), or random
gamma ~ U(0.5, 1.5), beta ~ N(0, 0.5) so the reordered-parameter path is
exercised.

Every host draw comes from numpy's PCG64 seeded with (seed, stream); the
stream ids below separate channel parameters, calibration tokens, evaluation
tokens, weights, LayerNorm parameters and the KMeans seeding uniforms.  The
K/V cache workload is too large for host generation and is drawn on the GPU
with torch's Philox generator (``tokens_device``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAM_CHANNELS = 0
STREAM_CALIB = 1
STREAM_EVAL = 2
STREAM_WEIGHTS = 3
STREAM_LN = 4
STREAM_KMEANS = 5
STREAM_CALIB_V = 6
STREAM_EVAL_V = 7
STREAM_CHANNELS_V = 8

FP16_MAX = 65504.0


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


@dataclass(frozen=True)
class Workload:
    """One OPT-shaped layer: M tokens x K channels -> N outputs, g clusters."""
    name: str
    M: int
    K: int
    N: int
    g: int
    a_bits: int
    w_bits: int
    seed: int
    outlier_frac: float = 0.01
    range_ratio: float | None = None
    calib_tokens: int = 512
    extra_a_bits: tuple = field(default_factory=tuple)


# The five workloads: an OPT-125m-shaped layer, an OPT-1.3B fc1, an OPT-13B
# QKV projection, an OPT-66B fc1 and an OPT-66B K/V cache (T = batch 64 x
# seq 8192 rows of 72 heads x 128 channels).
WORKLOADS = {
    "opt125m_w8a8": Workload("opt125m_w8a8", 128, 768, 3072, 4, 8, 8, 1001),
    "opt1.3b_fc1_w4a4": Workload("opt1.3b_fc1_w4a4", 2048, 2048, 8192, 8, 4, 4, 1002,
                                 outlier_frac=0.005),
    "opt13b_qkv_w4a4": Workload("opt13b_qkv_w4a4", 4096, 5120, 15360, 16, 4, 4, 1003,
                                outlier_frac=0.0, range_ratio=300.0, extra_a_bits=(8,)),
    "opt66b_fc1_w4a4": Workload("opt66b_fc1_w4a4", 16384, 9216, 36864, 32, 4, 4, 1004,
                                extra_a_bits=(3,)),
}


@dataclass(frozen=True)
class KVWorkload:
    name: str
    batch: int
    seq: int
    heads: int
    head_dim: int
    g: int
    bits: int
    seed: int
    outlier_frac: float = 0.01
    calib_tokens: int = 512

    @property
    def T(self) -> int:
        return self.batch * self.seq

    @property
    def C(self) -> int:
        return self.heads * self.head_dim


KV_WORKLOADS = {
    "opt66b_kv_a3": KVWorkload("opt66b_kv_a3", 64, 8192, 72, 128, 32, 3, 1005),
}


def channel_params(K: int, seed: int, outlier_frac: float = 0.01, outlier_scale: float = 100.0,
                   range_ratio: float | None = None, stream: int = STREAM_CHANNELS):
    """Per-channel (mu, sigma), float64 [K] each."""
    r = rng(seed, stream)
    mu = r.normal(0.0, 2.0, K)
    if range_ratio is not None:
        sigma = float(range_ratio) ** r.random(K)
        return mu, sigma
    sigma = r.lognormal(0.0, 1.0, K)
    n_out = int(round(outlier_frac * K))
    if n_out:
        idx = r.choice(K, n_out, replace=False)
        mu[idx] *= outlier_scale
        sigma[idx] *= outlier_scale
    return mu, sigma


def tokens(M: int, mu, sigma, seed: int, stream: int, chunk: int = 4096) -> np.ndarray:
    """fp16 [M][K] activations, generated in row chunks (bounded temporaries)."""
    mu32 = np.asarray(mu, np.float32)
    sg32 = np.asarray(sigma, np.float32)
    K = mu32.size
    out = np.empty((M, K), np.float16)
    r = rng(seed, stream)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        e = r.standard_normal((r1 - r0, K), dtype=np.float32)
        v = mu32 + sg32 * e
        np.clip(v, -FP16_MAX, FP16_MAX, out=v)
        out[r0:r1] = v.astype(np.float16)
    return out


def tokens_device(T: int, mu, sigma, seed: int, stream: int, out=None, chunk: int = 8192):
    """Large fp16 [T][K] activations drawn directly in GPU memory with torch's
    counter-based (Philox) generator, one generator per row chunk so any chunk
    can be regenerated on its own.  Returns a torch tensor on cuda."""
    import torch
    mu_t = torch.as_tensor(np.asarray(mu, np.float32), device="cuda")
    sg_t = torch.as_tensor(np.asarray(sigma, np.float32), device="cuda")
    K = mu_t.numel()
    if out is None:
        out = torch.empty((T, K), dtype=torch.float16, device="cuda")
    for ci, r0 in enumerate(range(0, T, chunk)):
        r1 = min(T, r0 + chunk)
        gen = torch.Generator(device="cuda")
        gen.manual_seed((int(seed) * 1000003 + int(stream)) * 1000003 + ci)
        e = torch.randn((r1 - r0, K), generator=gen, device="cuda", dtype=torch.float32)
        e.mul_(sg_t).add_(mu_t).clamp_(-FP16_MAX, FP16_MAX)
        out[r0:r1].copy_(e)
        del e
    return out


def weights(K: int, N: int, seed: int, std: float = 0.02) -> np.ndarray:
    r = rng(seed, STREAM_WEIGHTS)
    return r.normal(0.0, std, (K, N)).astype(np.float32)


def ln_params(K: int, seed: int, random: bool = True):
    if not random:
        return np.ones(K, np.float32), np.zeros(K, np.float32)
    r = rng(seed, STREAM_LN)
    gamma = r.uniform(0.5, 1.5, K).astype(np.float32)
    beta = r.normal(0.0, 0.5, K).astype(np.float32)
    return gamma, beta


def kmeans_uniforms(seed: int, n_init: int, g: int) -> np.ndarray:
    """The uniforms the KMeans seeding consumes, drawn once and handed to
    every implementation so all of them make the same draws."""
    return rng(seed, STREAM_KMEANS).random(n_init * g)


def codes(M: int, K: int, bits: int, seed: int, stream: int = 9) -> np.ndarray:
    """Uniform random codes in [0, 2^bits), uint8 [M][K]."""
    return rng(seed, stream).integers(0, 1 << bits, (M, K), dtype=np.uint8)


def small(w: Workload, M: int | None = None, K: int | None = None, N: int | None = None,
          g: int | None = None) -> Workload:
    """A reduced copy of a workload (same distributions and bit widths)."""
    from dataclasses import replace
    return replace(w, name=w.name + "_small", M=M or w.M, K=K or w.K, N=N or w.N, g=g or w.g)
