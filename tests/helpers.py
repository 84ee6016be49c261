"""Test infrastructure: builds seeded cases with the oracle (CPU) and moves
inputs to the GPU.  Every expected value comes from the oracle."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle as orc
import synthetic


@dataclass
class LayerCase:
    M: int
    K: int
    N: int
    g: int
    a_bits: int
    w_bits: int
    x: np.ndarray          # fp16 [M][K]
    gamma: np.ndarray      # natural order
    beta: np.ndarray
    R: np.ndarray
    bounds: np.ndarray
    s: np.ndarray
    z: np.ndarray
    Wq: np.ndarray | None = None     # int8 [K][N] natural rows
    s_w: np.ndarray | None = None


def layer_case(M, K, N, g, a_bits, w_bits=4, seed=1, outlier_frac=0.01, range_ratio=None,
               random_ln=True, calib_tokens=256, n_init=3, with_weights=True) -> LayerCase:
    mu, sg = synthetic.channel_params(K, seed, outlier_frac, range_ratio=range_ratio)
    gamma, beta = synthetic.ln_params(K, seed, random=random_ln)
    xc = synthetic.tokens(calib_tokens, mu, sg, seed, synthetic.STREAM_CALIB)
    mx, mn = orc.channel_minmax(orc.layernorm(xc, gamma, beta))
    R, bounds, s, z = orc.calibrate(mx, mn, g, a_bits, synthetic.kmeans_uniforms(seed, n_init, g), n_init=n_init)
    x = synthetic.tokens(M, mu, sg, seed, synthetic.STREAM_EVAL)
    case = LayerCase(M, K, N, g, a_bits, w_bits, x, gamma, beta, R, bounds, s, z)
    if with_weights:
        case.Wq, case.s_w = orc.quantize_weights(synthetic.weights(K, N, seed), w_bits)
    return case


def explicit_case(M, K, N, bounds, a_bits, w_bits=4, seed=1):
    """Hand-chosen cluster bounds (edge cases: size-1 clusters, g = 1, g = 64)."""
    r = np.random.default_rng(seed)
    bounds = np.asarray(bounds, np.int32)
    g = bounds.size - 1
    mu, sg = synthetic.channel_params(K, seed, 0.02)
    gamma, beta = synthetic.ln_params(K, seed)
    xc = synthetic.tokens(64, mu, sg, seed, synthetic.STREAM_CALIB)
    R = r.permutation(K).astype(np.int32)
    y = orc.layernorm(xc, gamma, beta)
    mx, mn = orc.channel_minmax(y)
    s, z = orc.cluster_params(mx, mn, R, bounds, a_bits)
    x = synthetic.tokens(M, mu, sg, seed, synthetic.STREAM_EVAL)
    case = LayerCase(M, K, N, g, a_bits, w_bits, x, gamma, beta, R, bounds, s, z)
    case.Wq, case.s_w = orc.quantize_weights(synthetic.weights(K, N, seed), w_bits)
    return case


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def seg32_pitch(bounds, bits) -> int:
    """The library's row pitch of SEG32 codes: the oracle's row bytes
    (K_pad * bits / 8) rounded up to a multiple of 64."""
    return (orc.seg32_row_bytes(bounds, bits) + 63) // 64 * 64


def code_bytes(codes, bounds, bits) -> np.ndarray:
    """Host copy of the code bytes of pitched SEG32 rows (a GPU tensor or an
    array), without the pitch's tail: comparable with the oracle's rows."""
    a = codes.cpu().numpy() if hasattr(codes, "cpu") else np.asarray(codes)
    return np.ascontiguousarray(a[:, :orc.seg32_row_bytes(bounds, bits)])


def pitched(codes_o, bounds, bits) -> np.ndarray:
    """The oracle's SEG32 rows laid out at the library's row pitch (zero tail),
    as the GEMM reads them."""
    out = np.zeros((codes_o.shape[0], seg32_pitch(bounds, bits)), np.uint8)
    out[:, :codes_o.shape[1]] = codes_o
    return out
