"""RPTQ oracle -- TEST INFRASTRUCTURE ONLY.

A plain CPU implementation (C++ in ``rptq_oracle.cpp``, loaded through ctypes)
of what the reorder-based post-training quantization hot path computes.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
``post_quantization_layernorm_amd`` and never imports it.

Every function takes and returns numpy arrays.  Citations of the pages are in
the C++ source next to each routine.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rptq_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

CXXFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp", "-shared", "-fPIC", "-std=c++17"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with g++ (auto-vectorisation only, no intrinsics)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", *CXXFLAGS, _SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float


def _declare(L):
    sig = {
        "orc_num_threads": (ctypes.c_int, []),
        "orc_half_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_float_to_half": (ctypes.c_uint16, [_F]),
        "orc_double_to_half": (ctypes.c_uint16, [ctypes.c_double]),
        "orc_half_to_double_array": (None, [_P, _I64, _P]),
        "orc_float_to_half_array": (None, [_P, _I64, _P]),
        "orc_layernorm": (None, [_P, _I64, _I32, _P, _P, _F, _P, _P]),
        "orc_channel_minmax_f32": (None, [_P, _I64, _I32, _P, _P]),
        "orc_channel_minmax_f16": (None, [_P, _I64, _I32, _P, _P]),
        "orc_kmeans": (ctypes.c_int, [_P, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _P]),
        "orc_order_clusters": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
        "orc_cluster_params": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _P, _P]),
        "orc_quantize": (None, [_P, _I64, _I32, _P, _I32, _P, _P, _I32, _P]),
        "orc_dequantize": (None, [_P, _I64, _I32, _P, _I32, _P, _P, _P]),
        "orc_dense_row_bytes": (_I64, [_I32, _I32]),
        "orc_seg32_kpad": (_I32, [_P, _I32]),
        "orc_seg32_row_bytes": (_I64, [_P, _I32, _I32]),
        "orc_pack_dense": (ctypes.c_int, [_P, _I64, _I32, _I32, _P]),
        "orc_unpack_dense": (ctypes.c_int, [_P, _I64, _I32, _I32, _P]),
        "orc_pack_seg32": (ctypes.c_int, [_P, _I64, _I32, _P, _I32, _I32, _P]),
        "orc_unpack_seg32": (ctypes.c_int, [_P, _I64, _I32, _P, _I32, _I32, _P, _P]),
        "orc_ln_reorder_quant": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _F, _P, _P, _I32,
                                                _P, _P, _I32, _P, _P]),
        "orc_quantize_weights": (None, [_P, _I32, _I32, _I32, _P, _P]),
        "orc_qgemm": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, _P, _I32, _P, _P, _P, _P, _P]),
        "orc_kv_quant_pack": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, _P, _P, _I32, _P]),
        "orc_kv_dequant": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _I32, _P, _P, _I32, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _c(a, dtype):
    """Contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ----------------------------------------------------------------------------- helpers
def num_threads() -> int:
    return lib().orc_num_threads()


def half_to_double(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_half_to_double_array(_p(h), h.size, _p(out))
    return out


def float_to_half_bits(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_float_to_half_array(_p(x), x.size, _p(out))
    return out


# ----------------------------------------------------------------------------- LN / calibration
def layernorm(x_f16_bits, gamma, beta, eps=1e-5, R=None) -> np.ndarray:
    """x: [M][K] fp16 bit patterns (uint16) or float16; returns fp32 [M][K] in R order."""
    x = _c(np.asarray(x_f16_bits).view(np.uint16), np.uint16)
    M, K = x.shape
    g = _c(gamma, np.float32); b = _c(beta, np.float32)
    Rr = None if R is None else _c(R, np.int32)
    y = np.empty((M, K), np.float32)
    lib().orc_layernorm(_p(x), M, K, _p(g), _p(b), eps, _p(Rr), _p(y))
    return y


def channel_minmax(v):
    v = np.asarray(v)
    rows, K = v.shape
    mx = np.empty(K, np.float32); mn = np.empty(K, np.float32)
    if v.dtype == np.float16 or v.dtype == np.uint16:
        vv = _c(v.view(np.uint16), np.uint16)
        lib().orc_channel_minmax_f16(_p(vv), rows, K, _p(mx), _p(mn))
    else:
        vv = _c(v, np.float32)
        lib().orc_channel_minmax_f32(_p(vv), rows, K, _p(mx), _p(mn))
    return mx, mn


def kmeans(points, g, u, n_init, max_iter=300):
    pts = _c(points, np.float64)
    C = pts.shape[0]
    uu = _c(u, np.float64)
    assert uu.size >= n_init * g
    labels = np.empty(C, np.int32); cen = np.empty((g, 2), np.float64)
    inertia = ctypes.c_double(); iters = ctypes.c_int32()
    rc = lib().orc_kmeans(_p(pts), C, g, _p(uu), n_init, max_iter, _p(labels), _p(cen),
                          ctypes.byref(inertia), ctypes.byref(iters))
    _check(rc, "kmeans")
    return labels, cen, inertia.value, iters.value


def order_clusters(labels, centroids):
    lab = _c(labels, np.int32); cen = _c(centroids, np.float64)
    C = lab.size; g = cen.shape[0]
    R = np.empty(C, np.int32); bounds = np.empty(g + 1, np.int32)
    _check(lib().orc_order_clusters(_p(lab), _p(cen), C, g, _p(R), _p(bounds)), "order_clusters")
    return R, bounds


def cluster_params(mx, mn, R, bounds, bits):
    mx = _c(mx, np.float32); mn = _c(mn, np.float32)
    Rr = None if R is None else _c(R, np.int32)
    b = _c(bounds, np.int32); g = b.size - 1
    s = np.empty(g, np.float32); z = np.empty(g, np.int32)
    _check(lib().orc_cluster_params(_p(mx), _p(mn), _p(Rr), _p(b), g, bits, _p(s), _p(z)),
           "cluster_params")
    return s, z


def calibrate(mx, mn, g, bits, u, n_init=10, max_iter=300):
    """(max, min) per channel -> KMeans -> R, bounds -> per-cluster s, z."""
    pts = np.stack([np.asarray(mx, np.float64), np.asarray(mn, np.float64)], axis=1)
    labels, cen, _, _ = kmeans(pts, g, u, n_init, max_iter)
    R, bounds = order_clusters(labels, cen)
    s, z = cluster_params(mx, mn, R, bounds, bits)
    return R, bounds, s, z


# ----------------------------------------------------------------------------- quantization
def quantize(y, bounds, s, z, bits) -> np.ndarray:
    y = _c(y, np.float32); M, K = y.shape
    b = _c(bounds, np.int32)
    q = np.empty((M, K), np.uint8)
    lib().orc_quantize(_p(y), M, K, _p(b), b.size - 1, _p(_c(s, np.float32)),
                       _p(_c(z, np.int32)), bits, _p(q))
    return q


def dequantize(q, bounds, s, z) -> np.ndarray:
    q = _c(q, np.uint8); M, K = q.shape
    b = _c(bounds, np.int32)
    out = np.empty((M, K), np.float32)
    lib().orc_dequantize(_p(q), M, K, _p(b), b.size - 1, _p(_c(s, np.float32)),
                         _p(_c(z, np.int32)), _p(out))
    return out


def dense_row_bytes(K, bits) -> int:
    return int(lib().orc_dense_row_bytes(K, bits))


def seg32_kpad(bounds) -> int:
    b = _c(bounds, np.int32)
    return int(lib().orc_seg32_kpad(_p(b), b.size - 1))


def seg32_row_bytes(bounds, bits) -> int:
    b = _c(bounds, np.int32)
    return int(lib().orc_seg32_row_bytes(_p(b), b.size - 1, bits))


def pack_dense(q, bits) -> np.ndarray:
    q = _c(q, np.uint8); M, K = q.shape
    out = np.empty((M, K * bits // 8), np.uint8)
    _check(lib().orc_pack_dense(_p(q), M, K, bits, _p(out)), "pack_dense")
    return out


def unpack_dense(packed, K, bits) -> np.ndarray:
    p = _c(packed, np.uint8); M = p.shape[0]
    q = np.empty((M, K), np.uint8)
    _check(lib().orc_unpack_dense(_p(p), M, K, bits, _p(q)), "unpack_dense")
    return q


def pack_seg32(q, bounds, bits) -> np.ndarray:
    q = _c(q, np.uint8); M, K = q.shape
    b = _c(bounds, np.int32)
    out = np.empty((M, seg32_row_bytes(b, bits)), np.uint8)
    _check(lib().orc_pack_seg32(_p(q), M, K, _p(b), b.size - 1, bits, _p(out)), "pack_seg32")
    return out


def unpack_seg32(packed, K, bounds, bits, return_pad=False):
    p = _c(packed, np.uint8); M = p.shape[0]
    b = _c(bounds, np.int32)
    q = np.empty((M, K), np.uint8)
    pad = np.empty((M, seg32_kpad(b) - K), np.uint8)
    _check(lib().orc_unpack_seg32(_p(p), M, K, _p(b), b.size - 1, bits, _p(q), _p(pad)),
           "unpack_seg32")
    return (q, pad) if return_pad else q


def ln_reorder_quant(x_f16, gamma, beta, eps, R, bounds, s, z, bits, return_y=False):
    """Reordered LayerNorm -> per-cluster quant -> SEG32 packed codes."""
    x = _c(np.asarray(x_f16).view(np.uint16), np.uint16); M, K = x.shape
    b = _c(bounds, np.int32)
    codes = np.empty((M, seg32_row_bytes(b, bits)), np.uint8)
    y = np.empty((M, K), np.float32) if return_y else None
    Rr = None if R is None else _c(R, np.int32)
    rc = lib().orc_ln_reorder_quant(_p(x), M, K, _p(_c(gamma, np.float32)), _p(_c(beta, np.float32)),
                                    eps, _p(Rr), _p(b), b.size - 1, _p(_c(s, np.float32)),
                                    _p(_c(z, np.int32)), bits, _p(codes), _p(y))
    _check(rc, "ln_reorder_quant")
    return (codes, y) if return_y else codes


# ----------------------------------------------------------------------------- dynamic ranges
def dynamic_cluster_params(y, bounds, bits):
    """Dynamic ranges (quantization lecture 1.1: the scale is decided at run
    time from the current activations).  The calibration rule applied to THIS
    batch: per reordered position the (max, min) over the rows of y (fp32
    [M][K], R order), then each cluster's (s, z) from them.  Returns (s, z)."""
    mx, mn = channel_minmax(np.asarray(y, np.float32))
    return cluster_params(mx, mn, None, bounds, bits)


def quantize_dynamic(y, bounds, bits):
    """Quantize-only mode with dynamic ranges: y fp32 [M][K] in R order.
    Returns (SEG32 codes, s, z)."""
    s, z = dynamic_cluster_params(y, bounds, bits)
    return pack_seg32(quantize(y, bounds, s, z, bits), bounds, bits), s, z


def ln_reorder_quant_dynamic(x_f16, gamma, beta, eps, R, bounds, bits, return_y=False):
    """Reordered LayerNorm, then dynamic (s, z) from this batch's y, then the
    per-cluster quantization and SEG32 pack.  Returns (codes, s, z[, y])."""
    y = layernorm(x_f16, gamma, beta, eps, R)
    codes, s, z = quantize_dynamic(y, bounds, bits)
    return (codes, s, z, y) if return_y else (codes, s, z)


# ----------------------------------------------------------------------------- weights / GEMM
def quantize_weights(W, wbits):
    W = _c(W, np.float32); K, N = W.shape
    Wq = np.empty((K, N), np.int8); sw = np.empty(N, np.float32)
    lib().orc_quantize_weights(_p(W), K, N, wbits, _p(Wq), _p(sw))
    return Wq, sw


def qgemm(q, Wq, R, bounds, s, z, s_w, return_acc=False):
    """q: [M][K] codes (reordered order); Wq: [K][N] int8 natural rows."""
    q = _c(q, np.uint8); M, K = q.shape
    Wq = _c(Wq, np.int8); N = Wq.shape[1]
    b = _c(bounds, np.int32); g = b.size - 1
    Rr = None if R is None else _c(R, np.int32)
    Y = np.empty((M, N), np.float32)
    acc = np.empty((g, M, N), np.int32) if return_acc else None
    rc = lib().orc_qgemm(_p(q), M, K, _p(Wq), _p(Rr), N, _p(b), g, _p(_c(s, np.float32)),
                         _p(_c(z, np.int32)), _p(_c(s_w, np.float32)), _p(Y), _p(acc))
    _check(rc, "qgemm")
    return (Y, acc) if return_acc else Y


def qgemm_quant(q, Wq, R, bounds, s, z, s_w, act, R_out, out_bounds, out_s, out_z, out_bits, return_y=False):
    """A linear layer whose weights are reordered so that it produces its
    output directly in the next layer's sorted order (RPTQ write-up, method
    and Fig. 3), quantized per next-layer cluster and packed (SEG32):
      Y      = qgemm(...)                        fp32 [M][N], natural order
      y[:,j] = act(Y[:, R_out[j]])               act 0: identity, 1: max(., 0)
      codes  = pack_seg32(quantize(y, out_bounds, out_s, out_z, out_bits))
    The steps are the oracle's own GEMM, quantizer and packer, in this order."""
    Y = qgemm(q, Wq, R, bounds, s, z, s_w)
    if act:
        Y = np.maximum(Y, np.float32(0.0))
    y = Y if R_out is None else Y[:, np.asarray(R_out)]
    y = np.ascontiguousarray(y, np.float32)
    codes = pack_seg32(quantize(y, out_bounds, out_s, out_z, out_bits), out_bounds, out_bits)
    return (codes, y) if return_y else codes


# ----------------------------------------------------------------------------- KV cache
def kv_quant_pack(kv_f16, R, bounds, s, z, bits) -> np.ndarray:
    kv = _c(np.asarray(kv_f16).view(np.uint16), np.uint16); T, C = kv.shape
    b = _c(bounds, np.int32)
    out = np.empty((T, C * bits // 8), np.uint8)
    Rr = None if R is None else _c(R, np.int32)
    rc = lib().orc_kv_quant_pack(_p(kv), T, C, _p(Rr), _p(b), b.size - 1, _p(_c(s, np.float32)),
                                 _p(_c(z, np.int32)), bits, _p(out))
    _check(rc, "kv_quant_pack")
    return out


def kv_attention(q_f16, k_packed, v_packed, B, T, C, head_dim, scale, k_params, v_params, bits):
    """Decode attention over a packed K/V cache (RPTQ write-up, evaluation:
    the KV-cache settings keep the keys and values quantized because they
    hold most of the memory; attention reads them back).  The cache is what
    kv_dequant produces from the packed rows (fp16, natural order); per
    sequence b, head h (channels h*head_dim .. +head_dim) and token t:
      score[h][t] = scale * sum_d q[b][h, d] * K[b*T + t][h, d]
      p[h][t]     = exp(score[h][t] - max_t score[h]) / sum_t exp(...)
      out[b][h, d] = sum_t p[h][t] * V[b*T + t][h, d]
    in fp64.  q_f16: fp16 bit patterns [B][C]; k_params / v_params:
    (R, bounds, s, z).  Returns fp64 [B][C]."""
    H = C // head_dim
    Kc = half_to_double(kv_dequant(k_packed, C, *k_params, bits)).reshape(B, T, H, head_dim)
    Vc = half_to_double(kv_dequant(v_packed, C, *v_params, bits)).reshape(B, T, H, head_dim)
    q = half_to_double(np.asarray(q_f16).view(np.uint16)).reshape(B, H, head_dim)
    out = np.empty((B, H, head_dim), np.float64)
    for b in range(B):
        sc = np.einsum("hd,thd->ht", q[b], Kc[b]) * float(scale)
        sc = np.exp(sc - sc.max(axis=1, keepdims=True))
        p = sc / sc.sum(axis=1, keepdims=True)
        out[b] = np.einsum("ht,thd->hd", p, Vc[b])
    return out.reshape(B, C)


def kv_dequant(packed, C, R, bounds, s, z, bits) -> np.ndarray:
    """Returns fp16 bit patterns (uint16) [T][C] in natural order."""
    p = _c(packed, np.uint8); T = p.shape[0]
    b = _c(bounds, np.int32)
    out = np.empty((T, C), np.uint16)
    Rr = None if R is None else _c(R, np.int32)
    rc = lib().orc_kv_dequant(_p(p), T, C, _p(Rr), _p(b), b.size - 1, _p(_c(s, np.float32)),
                              _p(_c(z, np.int32)), bits, _p(out))
    _check(rc, "kv_dequant")
    return out
