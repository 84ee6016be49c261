"""MI355X (gfx950) RPTQ hot path: thin Python binding of the C ABI in
``include/rptq.h`` (library ``librptq.so`` built in-tree by ``build.py``).

Each ``rptq_*`` function here has the name of the C entry point it wraps and
only marshals arguments: torch tensors supply device memory and the current
HIP stream, small host arrays (bounds, s, z) are passed as numpy arrays, and
caller-supplied tensors are checked to be large enough for the rows the call
touches (codes and packed weights at their 64-byte row pitch).
Every step of the hot path runs in the library's HIP kernels; there is no
fallback -- if the library is missing or fails, the call raises.

``import torch`` happens before the library is loaded so that the library's
HIP runtime dependency binds to the runtime torch has already loaded.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # noqa: F401  (must precede loading librptq.so)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librptq.so")

RPTQ_OK = 0
RPTQ_ERR_INVALID_ARG = -1
RPTQ_ERR_UNSUPPORTED = -2
RPTQ_ERR_ALIGNMENT = -3
RPTQ_ERR_HIP = -4
RPTQ_IN_FP16_RAW = 0
RPTQ_IN_FP32_NORMALIZED = 1
RPTQ_CALIB_RAW = 2
RPTQ_ACT_NONE = 0
RPTQ_ACT_RELU = 1
RPTQ_MAX_CLUSTERS = 64
RPTQ_MAX_K = 16384

EXPORTED = [
    "rptq_ln_reorder_quant", "rptq_ln_reorder_quant_dynamic", "rptq_ln_dynamic_workspace_bytes",
    "rptq_ln_reorder_quant_dynamic_noalloc",
    "rptq_qgemm", "rptq_qgemm_dynamic",
    "rptq_qgemm_quant", "rptq_kv_quant_pack", "rptq_kv_dequant",
    "rptq_kv_attention", "rptq_kv_attention_workspace_bytes",
    "rptq_calib_minmax", "rptq_kmeans_reorder", "rptq_cluster_params", "rptq_quantize_weights",
    "rptq_pack_weights", "rptq_pack_weights_out", "rptq_codes_kpad", "rptq_codes_row_bytes", "rptq_weights_row_bytes",
    "rptq_kv_row_bytes", "rptq_status_string", "rptq_last_error", "rptq_version",
]


class RptqError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where} failed: status {status} ({_status_name(status)}): {detail}")
        self.status = status


def _status_name(st: int) -> str:
    return {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "misaligned pointer",
            -4: "HIP error"}.get(st, "unknown")


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def lib() -> ctypes.CDLL:
    """Load librptq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python post_quantization_layernorm_amd/build.py` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "rptq_ln_reorder_quant": (_I32, [_P, _I32, _I64, _I32, _P, _P, ctypes.c_float, _P, _P, _I32,
                                             _P, _P, _I32, _P, _P]),
            "rptq_ln_reorder_quant_dynamic": (_I32, [_P, _I32, _I64, _I32, _P, _P, ctypes.c_float, _P, _P,
                                                     _I32, _I32, _P, _P, _P, _P, _I64, _P]),
            "rptq_ln_dynamic_workspace_bytes": (_I64, [_I32]),
            "rptq_ln_reorder_quant_dynamic_noalloc": (_I32, [_P, _I32, _I64, _I32, _P, _P, ctypes.c_float, _P, _P,
                                                             _I32, _I32, _P, _P, _P, _P]),
            "rptq_qgemm": (_I32, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _P, _P, _P]),
            "rptq_qgemm_dynamic": (_I32, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _P,
                                          _P]),
            "rptq_qgemm_quant": (_I32, [_P, _I64, _I32, _I32, _P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _I32,
                                        _P, _I32, _P, _P, _I32, _P, _P, _P]),
            "rptq_kv_quant_pack": (_I32, [_P, _I64, _I32, _P, _P, _I32, _P, _P, _I32, _P, _P]),
            "rptq_kv_dequant": (_I32, [_P, _I64, _I32, _P, _P, _I32, _P, _P, _I32, _P, _P]),
            "rptq_kv_attention": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, _I32, _P, _P,
                                         _P, _P, _I32, _P, _P, _I32, _P, _P, _I64, _P]),
            "rptq_kv_attention_workspace_bytes": (_I64, [_I32, _I32, _I32, _I32]),
            "rptq_calib_minmax": (_I32, [_P, _I32, _I64, _I32, _P, _P, ctypes.c_float, _P, _P, _P]),
            "rptq_kmeans_reorder": (_I32, [_P, _P, _I32, _I32, _P, _I32, _I32, _P, _P]),
            "rptq_cluster_params": (_I32, [_P, _P, _P, _P, _I32, _I32, _P, _P]),
            "rptq_quantize_weights": (_I32, [_P, _I32, _I32, _I32, _P, _P]),
            "rptq_pack_weights": (_I32, [_P, _I32, _I32, _I32, _P, _P, _I32, _P, _P]),
            "rptq_pack_weights_out": (_I32, [_P, _I32, _I32, _I32, _P, _P, _I32, _P, _P, _I32, _P, _P, _P, _P]),
            "rptq_codes_kpad": (_I32, [_P, _I32]),
            "rptq_codes_row_bytes": (_I64, [_P, _I32, _I32]),
            "rptq_weights_row_bytes": (_I64, [_P, _I32, _I32]),
            "rptq_kv_row_bytes": (_I64, [_I32, _I32]),
            "rptq_status_string": (ctypes.c_char_p, [_I32]),
            "rptq_last_error": (ctypes.c_char_p, []),
            "rptq_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(st: int, where: str):
    if st != RPTQ_OK:
        raise RptqError(st, where, lib().rptq_last_error().decode())


def _need(t, nbytes: int, where: str, what: str):
    """A caller's tensor must hold the bytes the call reads or writes through
    its pointer (the C entry points take bare pointers and cannot check)."""
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise RptqError(RPTQ_ERR_INVALID_ARG, where, f"{what} holds {have} bytes, {nbytes} needed")


def _codes_bytes(M: int, bounds, bits: int, where: str) -> int:
    rb = rptq_codes_row_bytes(bounds, bits)
    if rb < 0:
        _check(RPTQ_ERR_INVALID_ARG, where)
    return M * rb


def _h(a, dtype):
    """Host numpy array of the given dtype, contiguous."""
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=dtype)


def _hp(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dp(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("expected a torch tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A device tensor allocated on the stream the library call will run on
    (the caching allocator then never hands its memory to other work while
    that stream may still use it)."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


# ---------------------------------------------------------------------------- sizes
def rptq_codes_kpad(bounds) -> int:
    b = _h(bounds, np.int32)
    return int(lib().rptq_codes_kpad(_hp(b), b.size - 1))


def rptq_codes_row_bytes(bounds, bits: int) -> int:
    b = _h(bounds, np.int32)
    return int(lib().rptq_codes_row_bytes(_hp(b), b.size - 1, bits))


def rptq_weights_row_bytes(bounds, w_bits: int) -> int:
    b = _h(bounds, np.int32)
    return int(lib().rptq_weights_row_bytes(_hp(b), b.size - 1, w_bits))


def rptq_kv_row_bytes(C: int, bits: int) -> int:
    return int(lib().rptq_kv_row_bytes(C, bits))


def rptq_version() -> str:
    return lib().rptq_version().decode()


# ---------------------------------------------------------------------------- hot path
def rptq_ln_reorder_quant(x, R, gamma_r, beta_r, bounds, s, z, bits, eps=1e-5,
                          in_mode=RPTQ_IN_FP16_RAW, out=None, stream=None):
    """x: cuda fp16 [M][K] (mode 0) or fp32 [M][K] R-ordered (mode 1).
    Returns cuda uint8 [M][row_bytes] SEG32 codes."""
    M, K = x.shape
    b = _h(bounds, np.int32); sh = _h(s, np.float32); zh = _h(z, np.int32)
    rb = rptq_codes_row_bytes(b, bits)
    if rb < 0:
        _check(RPTQ_ERR_INVALID_ARG, "rptq_codes_row_bytes")
    if out is None:
        out = _empty((M, rb), torch.uint8, x.device, stream)
    _need(out, M * rb, "rptq_ln_reorder_quant", "out")
    st = lib().rptq_ln_reorder_quant(_dp(x), in_mode, M, K, _dp(gamma_r), _dp(beta_r), eps, _dp(R),
                                     _hp(b), b.size - 1, _hp(sh), _hp(zh), bits, _dp(out), _stream(stream))
    _check(st, "rptq_ln_reorder_quant")
    return out


def rptq_ln_dynamic_workspace_bytes(g: int) -> int:
    return int(lib().rptq_ln_dynamic_workspace_bytes(g))


def rptq_ln_reorder_quant_dynamic(x, R, gamma_r, beta_r, bounds, bits, eps=1e-5,
                                  in_mode=RPTQ_IN_FP16_RAW, out=None, s_out=None, z_out=None, workspace=None,
                                  stream=None):
    """Dynamic ranges: the clusters' (s, z) come from this batch.  Returns
    (codes cuda uint8 [M][row_bytes], s cuda fp32 [g], z cuda int32 [g]).
    workspace: cuda uint8 of at least rptq_ln_dynamic_workspace_bytes(g)
    bytes (allocated here when None)."""
    M, K = x.shape
    b = _h(bounds, np.int32); g = b.size - 1
    rb = rptq_codes_row_bytes(b, bits)
    if rb < 0:
        _check(RPTQ_ERR_INVALID_ARG, "rptq_codes_row_bytes")
    if out is None:
        out = _empty((M, rb), torch.uint8, x.device, stream)
    if s_out is None:
        s_out = _empty(max(g, 1), torch.float32, x.device, stream)
    if z_out is None:
        z_out = _empty(max(g, 1), torch.int32, x.device, stream)
    if workspace is None:
        workspace = _empty(max(rptq_ln_dynamic_workspace_bytes(g), 16), torch.uint8, x.device, stream)
    _need(out, M * rb, "rptq_ln_reorder_quant_dynamic", "out")
    st = lib().rptq_ln_reorder_quant_dynamic(_dp(x), in_mode, M, K, _dp(gamma_r), _dp(beta_r), eps, _dp(R),
                                             _hp(b), g, bits, _dp(out), _dp(s_out), _dp(z_out), _dp(workspace),
                                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "rptq_ln_reorder_quant_dynamic")
    return out, s_out, z_out


def rptq_ln_reorder_quant_dynamic_noalloc(x, R, gamma_r, beta_r, bounds, bits, out, s_out, z_out, eps=1e-5,
                                          in_mode=RPTQ_IN_FP16_RAW, stream=None):
    """rptq_ln_reorder_quant_dynamic with the library's own partials array
    instead of a workspace: the caller passes every output (codes cuda uint8
    [M][row_bytes], s_out cuda fp32 [g], z_out cuda int32 [g]) and nothing is
    allocated on the device.  Calls that may overlap on one GPU race."""
    M, K = x.shape
    b = _h(bounds, np.int32); g = b.size - 1
    if M > 0:
        _need(out, _codes_bytes(M, b, bits, "rptq_ln_reorder_quant_dynamic_noalloc"),
              "rptq_ln_reorder_quant_dynamic_noalloc", "out")
    st = lib().rptq_ln_reorder_quant_dynamic_noalloc(_dp(x), in_mode, M, K, _dp(gamma_r), _dp(beta_r), eps,
                                                     _dp(R), _hp(b), g, bits, _dp(out), _dp(s_out), _dp(z_out),
                                                     _stream(stream))
    _check(st, "rptq_ln_reorder_quant_dynamic_noalloc")
    return out, s_out, z_out


def rptq_qgemm_dynamic(codes, M, K, N, bounds, s_dev, z_dev, a_bits, w_packed, w_bits, s_w, colsum, out=None,
                       stream=None):
    """rptq_qgemm with (s, z) as cuda tensors (fp32 [g], int32 [g])."""
    b = _h(bounds, np.int32)
    _need(codes, _codes_bytes(M, b, a_bits, "rptq_qgemm_dynamic"), "rptq_qgemm_dynamic", "codes")
    _need(w_packed, N * max(rptq_weights_row_bytes(b, w_bits), 0), "rptq_qgemm_dynamic", "w_packed")
    if out is None:
        out = _empty((M, N), torch.float32, codes.device, stream)
    st = lib().rptq_qgemm_dynamic(_dp(codes), M, K, N, _hp(b), b.size - 1, _dp(s_dev), _dp(z_dev), a_bits,
                                  _dp(w_packed), w_bits, _dp(s_w), _dp(colsum), _dp(out), _stream(stream))
    _check(st, "rptq_qgemm_dynamic")
    return out


def rptq_qgemm(codes, M, K, N, bounds, s, z, a_bits, w_packed, w_bits, s_w, colsum, out=None,
               acc_debug=None, stream=None):
    """codes: cuda uint8 SEG32 [M][row_bytes]; w_packed: cuda uint8 [N][rptq_weights_row_bytes];
    s_w: cuda fp32 [N]; colsum: cuda int32 [g][N].  Returns Y cuda fp32 [M][N]."""
    b = _h(bounds, np.int32); sh = _h(s, np.float32); zh = _h(z, np.int32)
    _need(codes, _codes_bytes(M, b, a_bits, "rptq_qgemm"), "rptq_qgemm", "codes")
    _need(w_packed, N * max(rptq_weights_row_bytes(b, w_bits), 0), "rptq_qgemm", "w_packed")
    if out is None:
        out = _empty((M, N), torch.float32, codes.device, stream)
    st = lib().rptq_qgemm(_dp(codes), M, K, N, _hp(b), b.size - 1, _hp(sh), _hp(zh), a_bits, _dp(w_packed),
                          w_bits, _dp(s_w), _dp(colsum), _dp(out), _dp(acc_debug), _stream(stream))
    _check(st, "rptq_qgemm")
    return out


def rptq_qgemm_quant(codes, M, K, N_pad, bounds, s, z, a_bits, w_packed, w_bits, s_w, colsum, act,
                     out_bounds, out_s, out_z, out_bits, out=None, y_out=None, stream=None):
    """The GEMM with its output quantized for the next layer.  w_packed, s_w,
    colsum: cuda, from rptq_pack_weights_out.  Returns cuda uint8 SEG32 codes
    [M][rptq_codes_row_bytes(out_bounds, out_bits)]; y_out (optional cuda fp32
    [M][N_pad]) receives the activated output before quantization."""
    b = _h(bounds, np.int32); sh = _h(s, np.float32); zh = _h(z, np.int32)
    ob = _h(out_bounds, np.int32); osh = _h(out_s, np.float32); ozh = _h(out_z, np.int32)
    _need(codes, _codes_bytes(M, b, a_bits, "rptq_qgemm_quant"), "rptq_qgemm_quant", "codes")
    _need(w_packed, N_pad * max(rptq_weights_row_bytes(b, w_bits), 0), "rptq_qgemm_quant", "w_packed")
    orb = rptq_codes_row_bytes(ob, out_bits)
    if orb < 0:
        _check(RPTQ_ERR_INVALID_ARG, "rptq_codes_row_bytes")
    if out is None:
        out = _empty((M, orb), torch.uint8, codes.device, stream)
    _need(out, M * orb, "rptq_qgemm_quant", "out")
    st = lib().rptq_qgemm_quant(_dp(codes), M, K, N_pad, _hp(b), b.size - 1, _hp(sh), _hp(zh), a_bits,
                                _dp(w_packed), w_bits, _dp(s_w), _dp(colsum), act, _hp(ob), ob.size - 1,
                                _hp(osh), _hp(ozh), out_bits, _dp(out), _dp(y_out), _stream(stream))
    _check(st, "rptq_qgemm_quant")
    return out


def rptq_kv_quant_pack(kv, R, bounds, s, z, bits, out=None, stream=None):
    """kv: cuda fp16 [T][C] natural order.  Returns cuda uint8 [T][C*bits/8]."""
    T, C = kv.shape
    b = _h(bounds, np.int32); sh = _h(s, np.float32); zh = _h(z, np.int32)
    if out is None:
        rb = rptq_kv_row_bytes(C, bits)
        if rb < 0:
            _check(RPTQ_ERR_UNSUPPORTED, "rptq_kv_row_bytes")
        out = _empty((T, rb), torch.uint8, kv.device, stream)
    st = lib().rptq_kv_quant_pack(_dp(kv), T, C, _dp(R), _hp(b), b.size - 1, _hp(sh), _hp(zh), bits,
                                  _dp(out), _stream(stream))
    _check(st, "rptq_kv_quant_pack")
    return out


def rptq_kv_attention_workspace_bytes(B, T, C, head_dim) -> int:
    return int(lib().rptq_kv_attention_workspace_bytes(B, T, C, head_dim))


def rptq_kv_attention(q, k_packed, v_packed, B, T, C, head_dim, scale, k_params, v_params, bits, out=None,
                      workspace=None, stream=None):
    """Decode attention over packed K/V.  q: cuda fp16 [B][C]; k_params /
    v_params: (R cuda int32 [C] or None, bounds, s, z).  Returns cuda fp32
    [B][C]."""
    Rk, bk, sk, zk = k_params
    Rv, bv, sv, zv = v_params
    bk = _h(bk, np.int32); sk = _h(sk, np.float32); zk = _h(zk, np.int32)
    bv = _h(bv, np.int32); sv = _h(sv, np.float32); zv = _h(zv, np.int32)
    if out is None:
        out = _empty((B, C), torch.float32, q.device, stream)
    need = rptq_kv_attention_workspace_bytes(B, T, C, head_dim)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    wsz = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().rptq_kv_attention(_dp(q), _dp(k_packed), _dp(v_packed), B, T, C, head_dim, scale, _dp(Rk),
                                 _hp(bk), bk.size - 1, _hp(sk), _hp(zk), _dp(Rv), _hp(bv), bv.size - 1,
                                 _hp(sv), _hp(zv), bits, _dp(out), _dp(workspace), wsz, _stream(stream))
    _check(st, "rptq_kv_attention")
    return out


def rptq_kv_dequant(packed, C, R, bounds, s, z, bits, out=None, stream=None):
    """packed: cuda uint8 [T][C*bits/8].  Returns cuda fp16 [T][C] natural order."""
    T = packed.shape[0]
    b = _h(bounds, np.int32); sh = _h(s, np.float32); zh = _h(z, np.int32)
    if out is None:
        out = _empty((T, C), torch.float16, packed.device, stream)
    st = lib().rptq_kv_dequant(_dp(packed), T, C, _dp(R), _hp(b), b.size - 1, _hp(sh), _hp(zh), bits,
                               _dp(out), _stream(stream))
    _check(st, "rptq_kv_dequant")
    return out


# ---------------------------------------------------------------------------- calibration
def rptq_calib_minmax(x, mode=RPTQ_IN_FP16_RAW, gamma=None, beta=None, eps=1e-5, stream=None):
    """x: cuda fp16 [M][K].  Returns (mx, mn) cuda fp32 [K], natural order."""
    M, K = x.shape
    mx = _empty(K, torch.float32, x.device, stream)
    mn = _empty(K, torch.float32, x.device, stream)
    st = lib().rptq_calib_minmax(_dp(x), mode, M, K, _dp(gamma), _dp(beta), eps, _dp(mx), _dp(mn),
                                 _stream(stream))
    _check(st, "rptq_calib_minmax")
    return mx, mn


def rptq_kmeans_reorder(mx, mn, g, init_u, n_init=10, max_iter=300):
    """Host.  Returns (R int32 [K], bounds int32 [g+1])."""
    mxh = _h(mx, np.float32); mnh = _h(mn, np.float32); u = _h(init_u, np.float64)
    K = mxh.size
    if u.size < n_init * g:
        raise ValueError("init_u needs n_init * g uniforms")
    R = np.empty(K, np.int32); bounds = np.empty(g + 1, np.int32)
    _check(lib().rptq_kmeans_reorder(_hp(mxh), _hp(mnh), K, g, _hp(u), n_init, max_iter, _hp(R), _hp(bounds)),
           "rptq_kmeans_reorder")
    return R, bounds


def rptq_cluster_params(mx, mn, R, bounds, bits):
    """Host.  Returns (s fp32 [g], z int32 [g])."""
    mxh = _h(mx, np.float32); mnh = _h(mn, np.float32)
    Rh = None if R is None else _h(R, np.int32)
    b = _h(bounds, np.int32); g = b.size - 1
    s = np.empty(g, np.float32); z = np.empty(g, np.int32)
    _check(lib().rptq_cluster_params(_hp(mxh), _hp(mnh), _hp(Rh), _hp(b), g, bits, _hp(s), _hp(z)),
           "rptq_cluster_params")
    return s, z


def rptq_quantize_weights(W, w_bits):
    """Host.  W fp32 [K][N] -> (wq int8 [K][N], s_w fp32 [N])."""
    Wh = _h(W, np.float32)
    K, N = Wh.shape
    wq = np.empty((K, N), np.int8); sw = np.empty(N, np.float32)
    _check(lib().rptq_quantize_weights(_hp(Wh), K, N, w_bits, _hp(wq), _hp(sw)), "rptq_quantize_weights")
    return wq, sw


def rptq_pack_weights(wq, R, bounds, w_bits):
    """Host.  Returns (w_packed uint8 [N][rptq_weights_row_bytes], colsum int32 [g][N])."""
    wqh = _h(wq, np.int8)
    K, N = wqh.shape
    Rh = None if R is None else _h(R, np.int32)
    b = _h(bounds, np.int32); g = b.size - 1
    rb = rptq_weights_row_bytes(b, w_bits)
    if rb < 0:
        _check(RPTQ_ERR_INVALID_ARG, "rptq_weights_row_bytes")
    wp = np.empty((N, rb), np.uint8); cs = np.empty((g, N), np.int32)
    _check(lib().rptq_pack_weights(_hp(wqh), K, N, w_bits, _hp(Rh), _hp(b), g, _hp(wp), _hp(cs)),
           "rptq_pack_weights")
    return wp, cs


def rptq_pack_weights_out(wq, R, bounds, w_bits, R_out, out_bounds, s_w):
    """Host.  Returns (w_packed uint8 [N_pad][rptq_weights_row_bytes], colsum int32
    [g][N_pad], s_w_out fp32 [N_pad]) with the output features in the next
    layer's padded order."""
    wqh = _h(wq, np.int8)
    K, N = wqh.shape
    Rh = None if R is None else _h(R, np.int32)
    Roh = None if R_out is None else _h(R_out, np.int32)
    b = _h(bounds, np.int32); g = b.size - 1
    ob = _h(out_bounds, np.int32)
    swh = _h(s_w, np.float32)
    rb = rptq_weights_row_bytes(b, w_bits)
    npad = rptq_codes_kpad(ob)
    if rb < 0 or npad < 0:
        _check(RPTQ_ERR_INVALID_ARG, "rptq_pack_weights_out sizes")
    wp = np.empty((npad, rb), np.uint8); cs = np.empty((g, npad), np.int32); swo = np.empty(npad, np.float32)
    _check(lib().rptq_pack_weights_out(_hp(wqh), K, N, w_bits, _hp(Rh), _hp(b), g, _hp(Roh), _hp(ob),
                                       ob.size - 1, _hp(swh), _hp(wp), _hp(cs), _hp(swo)),
           "rptq_pack_weights_out")
    return wp, cs, swo
