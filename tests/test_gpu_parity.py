"""GPU parity: every entry point of the C ABI against the oracle, element by
element, on seeded inputs.  Bars: codes and int32 accumulators bit-exact;
KV dequant fp16 bit-exact; fused LayerNorm codes within 0.1% of positions
differing by at most 1; Y within 1e-3 relative L2."""
import numpy as np
import pytest

import oracle as orc
import synthetic
from helpers import code_bytes, dev, explicit_case, layer_case, pitched, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_quantization_layernorm_amd as P
    P.lib()
    print(f"[gpu] {torch.cuda.get_device_name(0)} | {P.rptq_version()}", flush=True)
    return P


def _say(*a):
    print("[case]", *a, flush=True)


# ----------------------------------------------------------------------------- K/V cache
def _kv_params(kv, g, bits, seed, identity=False):
    mx, mn = orc.channel_minmax(kv)
    R, bounds, s, z = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(seed, 3, g), n_init=3)
    if identity:
        # the cache is already in reordered order: R = NULL on the device
        kv = np.ascontiguousarray(kv[:, R])
        R = None
    return kv, R, bounds, s, z


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("T,C,g,identity", [(333, 512, 8, False), (37, 9216, 32, False),
                                             (5, 1024, 16, True), (1, 128, 4, False)])
def test_kv_quant_pack_and_dequant_bit_exact(P, bits, T, C, g, identity):
    _say("kv", bits, T, C, g, identity)
    mu, sg = synthetic.channel_params(C, 40 + bits, 0.01)
    kv = synthetic.tokens(T, mu, sg, 40 + bits, synthetic.STREAM_EVAL)
    kvd, R, bounds, s, z = _kv_params(kv, g, bits, 40 + bits, identity)
    want = orc.kv_quant_pack(kvd, R, bounds, s, z, bits)
    Rd = None if R is None else dev(R)
    got = P.rptq_kv_quant_pack(dev(kvd.view(np.int16)).view(torch.float16), Rd, bounds, s, z, bits)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)
    want_deq = orc.kv_dequant(want, C, R, bounds, s, z, bits)
    got_deq = P.rptq_kv_dequant(dev(want), C, Rd, bounds, s, z, bits)
    torch.cuda.synchronize()
    assert np.array_equal(got_deq.cpu().numpy().view(np.uint16), want_deq)


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_kv_extremes_and_size_one_clusters(P, bits):
    """inf / max-half inputs, clusters of one channel, zero points near +-2^21."""
    C, T = 64, 9
    r = np.random.default_rng(bits)
    kv = (r.standard_normal((T, C)) * 50).astype(np.float16)
    kv[0, :8] = [np.inf, -np.inf, 65504, -65504, 0.0, -0.0, 6e-8, -6e-8]
    bounds = np.arange(C + 1, dtype=np.int32)                  # g = 64, one channel each
    R = r.permutation(C).astype(np.int32)
    s = r.uniform(1e-3, 10, C).astype(np.float32)
    z = r.integers(-(2 ** 21), 2 ** 21 + 1, C).astype(np.int32)
    z[:4] = [2 ** 21, -(2 ** 21), 0, (1 << bits) - 1]
    want = orc.kv_quant_pack(kv, R, bounds, s, z, bits)
    got = P.rptq_kv_quant_pack(dev(kv.view(np.int16)).view(torch.float16), dev(R), bounds, s, z, bits)
    assert np.array_equal(got.cpu().numpy(), want)
    want_deq = orc.kv_dequant(want, C, R, bounds, s, z, bits)
    got_deq = P.rptq_kv_dequant(dev(want), C, dev(R), bounds, s, z, bits)
    assert np.array_equal(got_deq.cpu().numpy().view(np.uint16), want_deq)


# ----------------------------------------------------------------------------- LayerNorm + quant
LN_SHAPES = [  # (M, K, g, outlier_frac, range_ratio)
    (128, 768, 4, 0.01, None),          # OPT-125m-shaped
    (70, 2048, 8, 0.005, None),         # OPT-1.3B-shaped
    (33, 5120, 16, 0.0, 300.0),         # OPT-13B-shaped, 10x-300x channel ranges
    (41, 9216, 32, 0.01, None),         # OPT-66B-shaped
    (6, 16384, 64, 0.01, None),         # largest K, 512-thread path
]


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("shape", LN_SHAPES, ids=lambda s: f"K{s[1]}g{s[2]}")
def test_ln_quant_only_mode_bit_exact(P, bits, shape):
    M, K, g, frac, rr = shape
    _say("ln quant-only", bits, shape)
    c = layer_case(M, K, 8, g, bits, seed=K + bits, outlier_frac=frac, range_ratio=rr, with_weights=False)
    y = orc.layernorm(c.x, c.gamma, c.beta, 1e-5, c.R)
    y[0, : min(K, 16)] = [1e30, -1e30, np.inf, -np.inf, 0.0, -0.0, 3e-39, 1e-3] * (min(K, 16) // 8)
    want = orc.pack_seg32(orc.quantize(y, c.bounds, c.s, c.z, bits), c.bounds, bits)
    got = P.rptq_ln_reorder_quant(dev(y), None, None, None, c.bounds, c.s, c.z, bits,
                                  in_mode=P.RPTQ_IN_FP32_NORMALIZED)
    torch.cuda.synchronize()
    assert np.array_equal(code_bytes(got, c.bounds, bits), want)


def _fused(P, c, bits, eps=1e-5):
    gr, br = c.gamma[c.R], c.beta[c.R]
    return P.rptq_ln_reorder_quant(dev(c.x.view(np.int16)).view(torch.float16), dev(c.R), dev(gr), dev(br),
                                   c.bounds, c.s, c.z, bits, eps=eps)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("shape", LN_SHAPES, ids=lambda s: f"K{s[1]}g{s[2]}")
def test_ln_fused_codes_within_tolerance(P, bits, shape):
    M, K, g, frac, rr = shape
    _say("ln fused", bits, shape)
    c = layer_case(M, K, 8, g, bits, seed=K + bits, outlier_frac=frac, range_ratio=rr, with_weights=False)
    want = orc.ln_reorder_quant(c.x, c.gamma, c.beta, 1e-5, c.R, c.bounds, c.s, c.z, bits)
    got = code_bytes(_fused(P, c, bits), c.bounds, bits)
    qg, pad_g = orc.unpack_seg32(got, K, c.bounds, bits, return_pad=True)
    qw = orc.unpack_seg32(want, K, c.bounds, bits)
    assert not pad_g.any()
    d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
    assert d.max() <= 1
    assert (d > 0).mean() <= 1e-3, (d > 0).mean()


def test_ln_fused_edge_rows(P):
    """M = 1, a constant row (zero variance), rows whose mean dwarfs their
    spread (the kernel's exact second pass), identity R, single cluster."""
    K = 256
    x = np.full((5, K), 7.0, np.float16)
    x[1] = np.linspace(-100, 100, K).astype(np.float16)
    x[2, ::2] = -3.0
    x[3] = (300.0 + np.random.default_rng(3).normal(0, 0.5, K)).astype(np.float16)
    x[4] = (-1000.0 + np.where(np.arange(K) % 2, 0.5, -0.5)).astype(np.float16)
    gamma, beta = synthetic.ln_params(K, 3)
    bounds = np.array([0, K], np.int32)
    y = orc.layernorm(x, gamma, beta)
    mx, mn = orc.channel_minmax(y)
    s, z = orc.cluster_params(mx, mn, None, bounds, 4)
    want = orc.ln_reorder_quant(x, gamma, beta, 1e-5, None, bounds, s, z, 4)
    for M in (1, 5):
        got = code_bytes(P.rptq_ln_reorder_quant(dev(x[:M].view(np.int16)).view(torch.float16), None, dev(gamma),
                                                 dev(beta), bounds, s, z, 4), bounds, 4)
        qg = orc.unpack_seg32(got, K, bounds, 4).astype(np.int32)
        qw = orc.unpack_seg32(want[:M], K, bounds, 4).astype(np.int32)
        assert np.abs(qg - qw).max() <= 1 and (qg != qw).mean() <= 1e-3


def test_ln_m0_noop(P):
    x = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    out = P.rptq_ln_reorder_quant(x, None, dev(np.ones(64, np.float32)), dev(np.zeros(64, np.float32)),
                                  np.array([0, 64], np.int32), np.ones(1, np.float32), np.zeros(1, np.int32), 4)
    assert out.shape[0] == 0


# ----------------------------------------------------------------------------- dynamic ranges
DYN_SHAPES = [  # (M, K, g, outlier_frac, range_ratio)
    (128, 768, 4, 0.01, None),
    (41, 9216, 32, 0.01, None),
    (6, 16384, 64, 0.01, None),
    (1, 2048, 8, 0.0, None),            # one row
    (3001, 1024, 8, 0.01, None),        # many rows per workgroup, odd row count
]


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("shape", DYN_SHAPES, ids=lambda s: f"M{s[0]}K{s[1]}g{s[2]}")
def test_ln_dynamic_quant_only_bit_exact(P, bits, shape):
    """Dynamic ranges in quant-only mode: (s, z) and the codes equal the
    oracle's bit for bit; a second call on other rows with the same (s, z)
    buffers starts its ranges afresh."""
    M, K, g, frac, rr = shape
    _say("ln dynamic quant-only", bits, shape)
    c = layer_case(M, K, 8, g, bits, seed=3 * K + bits, outlier_frac=frac, range_ratio=rr, with_weights=False)
    y = orc.layernorm(c.x, c.gamma, c.beta, 1e-5, c.R)
    y[0, :4] = [0.0, -0.0, 1e-3, -1e-3]
    sd = torch.empty(g, dtype=torch.float32, device="cuda")
    zd = torch.empty(g, dtype=torch.int32, device="cuda")
    for yy in (y * np.float32(3.0), y):
        want, s_o, z_o = orc.quantize_dynamic(yy, c.bounds, bits)
        got, sd, zd = P.rptq_ln_reorder_quant_dynamic(dev(yy), None, None, None, c.bounds, bits,
                                                      in_mode=P.RPTQ_IN_FP32_NORMALIZED, s_out=sd, z_out=zd)
        torch.cuda.synchronize()
        assert np.array_equal(sd.cpu().numpy(), s_o)
        assert np.array_equal(zd.cpu().numpy(), z_o)
        assert np.array_equal(code_bytes(got, c.bounds, bits), want)


@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("shape", DYN_SHAPES, ids=lambda s: f"M{s[0]}K{s[1]}g{s[2]}")
def test_ln_dynamic_fused_within_tolerance(P, bits, shape):
    """Fused LayerNorm with dynamic ranges: s within 1e-5 relative of the
    oracle's (the kernel's fp32 LayerNorm moves the extremes by a few ulps),
    z within 1, codes as for the calibrated path (at most 0.1% differ, by 1)."""
    M, K, g, frac, rr = shape
    _say("ln dynamic fused", bits, shape)
    c = layer_case(M, K, 8, g, bits, seed=3 * K + bits, outlier_frac=frac, range_ratio=rr, with_weights=False)
    want, s_o, z_o = orc.ln_reorder_quant_dynamic(c.x, c.gamma, c.beta, 1e-5, c.R, c.bounds, bits)
    gr, br = c.gamma[c.R], c.beta[c.R]
    got, sd, zd = P.rptq_ln_reorder_quant_dynamic(dev(c.x.view(np.int16)).view(torch.float16), dev(c.R),
                                                  dev(gr), dev(br), c.bounds, bits)
    sg, zg = sd.cpu().numpy(), zd.cpu().numpy()
    assert np.abs(sg.astype(np.float64) / s_o - 1.0).max() <= 1e-5
    assert np.abs(zg.astype(np.int64) - z_o).max() <= 1
    qg, pad = orc.unpack_seg32(code_bytes(got, c.bounds, bits), K, c.bounds, bits, return_pad=True)
    qw = orc.unpack_seg32(want, K, c.bounds, bits)
    assert not pad.any()
    d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (d.max(), (d > 0).mean())


@pytest.mark.parametrize("ab,wb,g", [(4, 4, 8), (3, 3, 8), (8, 8, 8), (8, 4, 8), (3, 4, 8), (4, 4, 20)])
def test_qgemm_dynamic(P, ab, wb, g):
    """The GEMM reading (s, z) from device memory: Y equals rptq_qgemm's with
    the same (s, z) passed from the host, bit for bit, and the oracle's GEMM
    of the kernel's codes within 1e-3."""
    M, K, N = 150, 2048, 520
    _say("gemm dynamic", ab, wb)
    c = layer_case(M, K, N, g, ab, wb, seed=900 + ab + wb + g)
    gr, br = c.gamma[c.R], c.beta[c.R]
    codes, sd, zd = P.rptq_ln_reorder_quant_dynamic(dev(c.x.view(np.int16)).view(torch.float16), dev(c.R),
                                                    dev(gr), dev(br), c.bounds, ab)
    wp, cs, sw = _gemm_inputs(P, c)
    Y = P.rptq_qgemm_dynamic(codes, M, K, N, c.bounds, sd, zd, ab, wp, wb, sw, cs)
    sh, zh = sd.cpu().numpy(), zd.cpu().numpy()
    Y_s = P.rptq_qgemm(codes, M, K, N, c.bounds, sh, zh, ab, wp, wb, sw, cs)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_s)
    q = orc.unpack_seg32(code_bytes(codes, c.bounds, ab), K, c.bounds, ab)
    Y_o = orc.qgemm(q, c.Wq, c.R, c.bounds, sh, zh, c.s_w)
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3


# ----------------------------------------------------------------------------- GEMM
def _gemm_inputs(P, c):
    wp, cs = P.rptq_pack_weights(c.Wq, c.R, c.bounds, c.w_bits)
    return dev(wp), dev(cs), dev(c.s_w)


def _oracle_codes(c):
    y = orc.layernorm(c.x, c.gamma, c.beta, 1e-5, c.R)
    q = orc.quantize(y, c.bounds, c.s, c.z, c.a_bits)
    return q, orc.pack_seg32(q, c.bounds, c.a_bits)


GEMM_CASES = [  # (M, K, N, g, a_bits, w_bits)
    (128, 768, 3072, 4, 8, 8),          # OPT-125m-shaped W8A8
    (200, 2048, 392, 8, 4, 4),          # OPT-1.3B-shaped W4A4, ragged M and N
    (96, 5120, 256, 16, 8, 4),          # OPT-13B-shaped W4A8
    (130, 5120, 264, 16, 4, 4),
    (64, 9216, 136, 32, 3, 4),          # OPT-66B-shaped W4A3
    (33, 9216, 128, 32, 4, 4),
    (1, 512, 72, 4, 4, 8),              # M = 1
    (64, 9216, 136, 32, 3, 3),          # OPT-66B-shaped W3A3 (the write-up's W3A3KV setting)
    (70, 2048, 392, 8, 4, 3),           # W3A4, ragged M and N
    (40, 768, 200, 4, 8, 3),            # W3A8
    (77, 512, 101, 4, 4, 4),            # odd N: a ragged last column tile
    (3, 768, 1, 2, 8, 8),               # N = 1
    (130, 40, 33, 2, 3, 3),             # K = 40 (two clusters padded to 64 codes), odd N
    (1300, 512, 520, 4, 4, 4),          # 11 x 5 tiles: a partial last group of the grouped tile walk
    (150, 2560, 264, 20, 4, 4),         # g = 20 and g = 37: the epilogue's colsum loads in batches of
    (70, 4096, 136, 37, 3, 4),          # 16 clusters end with a partial batch
    (100, 2560, 200, 20, 8, 8),         # (the 8-bit operand tile configuration too)
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "M{}K{}N{}g{}A{}W{}".format(*c))
def test_qgemm_accumulators_bit_exact_and_y(P, case):
    M, K, N, g, ab, wb = case
    _say("gemm", case)
    c = layer_case(M, K, N, g, ab, wb, seed=M + K + N)
    q, codes = _oracle_codes(c)
    Y_o, acc_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, return_acc=True)
    wp, cs, sw = _gemm_inputs(P, c)
    acc = torch.full((g, M, N), -7, dtype=torch.int32, device="cuda")
    Y = P.rptq_qgemm(dev(pitched(codes, c.bounds, ab)), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs, acc_debug=acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3
    # the debug buffer does not change Y
    Y2 = P.rptq_qgemm(dev(pitched(codes, c.bounds, ab)), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs)
    assert torch.equal(Y, Y2)


# More than 256 tiles (several workgroups per compute unit, both grouped
# tile walks of every XCD complete): every accumulator and Y against the
# oracle, for 4-, 8- and 3-bit codes.
@pytest.mark.parametrize("case", [(2048, 1024, 2176, 8, 4, 4), (1024, 768, 4224, 4, 8, 8),
                                  (1536, 1280, 2816, 16, 3, 3)],
                         ids=lambda c: "M{}K{}N{}g{}A{}W{}".format(*c))
def test_qgemm_many_tiles_bit_exact(P, case):
    M, K, N, g, ab, wb = case
    _say("gemm many tiles", case)
    c = layer_case(M, K, N, g, ab, wb, seed=M + N)
    q, codes = _oracle_codes(c)
    Y_o, acc_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, return_acc=True)
    wp, cs, sw = _gemm_inputs(P, c)
    acc = torch.full((g, M, N), -7, dtype=torch.int32, device="cuda")
    Y = P.rptq_qgemm(dev(pitched(codes, c.bounds, ab)), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs, acc_debug=acc)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    del acc
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3
    Y2 = P.rptq_qgemm(dev(pitched(codes, c.bounds, ab)), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs)
    assert torch.equal(Y, Y2)


# With 4-bit weights the GEMM reads the codes of its last, partial 128-code
# stage past K (the row's pitch tail, and for 8-bit codes here also the
# first bytes of the next row) against the zero tail of the weight rows: any
# values there leave every accumulator and Y unchanged.
@pytest.mark.parametrize("case", [(200, 2048, 392, 8, 4, 4), (64, 9216, 136, 32, 3, 4), (33, 9216, 128, 32, 8, 4)],
                         ids=lambda c: "M{}K{}N{}g{}A{}W{}".format(*c))
def test_qgemm_ignores_code_bytes_past_k(P, case):
    M, K, N, g, ab, wb = case
    _say("gemm code bytes past K", case)
    c = layer_case(M, K, N, g, ab, wb, seed=M + 7)
    kp = orc.seg32_kpad(c.bounds)
    assert (kp // 32) % 4 != 0              # a partial last stage
    q, codes = _oracle_codes(c)
    Y_o, acc_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, return_acc=True)
    wp, cs, sw = _gemm_inputs(P, c)
    clean = pitched(codes, c.bounds, ab)
    dirty = clean.copy()
    dirty[:, codes.shape[1]:] = 0xA5        # the pitch tail the producers leave unwritten
    out = []
    for a in (clean, dirty):
        acc = torch.full((g, M, N), -7, dtype=torch.int32, device="cuda")
        Y = P.rptq_qgemm(dev(a), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs, acc_debug=acc)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        out.append(P.rptq_qgemm(dev(a), M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs))
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])
    assert rel_l2(out[1].cpu().numpy(), Y_o) <= 1e-3


@pytest.mark.parametrize("bounds", [[0, 1, 2, 3, 64, 96, 97, 160, 256], [0, 256],
                                    list(range(0, 65)) + [256]],
                         ids=["size1", "g1", "g65"])
@pytest.mark.parametrize("ab,wb", [(3, 4), (4, 4), (8, 8), (8, 4), (3, 3), (8, 3)])
def test_qgemm_ragged_clusters(P, bounds, ab, wb):
    if len(bounds) - 1 > 64:
        bounds = bounds[:64] + [256]                  # g = 64: 63 singletons + one big cluster
    c = explicit_case(67, 256, 96, bounds, ab, wb, seed=len(bounds) + ab)
    q, codes = _oracle_codes(c)
    Y_o, acc_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, return_acc=True)
    wp, cs, sw = _gemm_inputs(P, c)
    acc = torch.zeros((c.g, c.M, c.N), dtype=torch.int32, device="cuda")
    Y = P.rptq_qgemm(dev(pitched(codes, c.bounds, ab)), c.M, c.K, c.N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs, acc_debug=acc)
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3


@pytest.mark.parametrize("ab,wb", [(3, 4), (4, 4), (8, 4), (3, 3)])
def test_end_to_end_ln_then_gemm(P, ab, wb):
    M, K, N, g = 150, 2048, 520, 8
    c = layer_case(M, K, N, g, ab, wb, seed=77 + ab)
    _, codes_o = _oracle_codes(c)
    q = orc.unpack_seg32(codes_o, K, c.bounds, ab)
    Y_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w)
    codes = _fused(P, c, ab)
    wp, cs, sw = _gemm_inputs(P, c)
    Y = P.rptq_qgemm(codes, M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs)
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3


# ----------------------------------------------------------------------------- GEMM with quantized output
@pytest.mark.parametrize("ab,wb,ob,act,N,g", [(4, 4, 4, 1, 330, 8), (3, 3, 3, 1, 200, 8), (8, 4, 8, 0, 130, 8),
                                               (4, 4, 3, 1, 1024, 8), (4, 4, 4, 1, 330, 20)])
def test_qgemm_quant_output(P, ab, wb, ob, act, N, g):
    """The epilogue quantizes the (activated) output for the next layer: the
    codes equal the oracle's quantization of the kernel's own y bit for bit,
    y matches the oracle's GEMM, and against the oracle end to end at most
    0.1% of the codes differ, by 1."""
    M, K, g2 = 150, 2048, 6
    _say("gemm quant-out", ab, wb, ob, act, N, g)
    c = layer_case(M, K, N, g, ab, wb, seed=500 + N + ab + g)
    q, codes = _oracle_codes(c)
    Y_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w)
    a_o = np.maximum(Y_o, np.float32(0)) if act else Y_o
    omx, omn = orc.channel_minmax(a_o)
    R2, b2, s2, z2 = orc.calibrate(omx, omn, g2, ob, synthetic.kmeans_uniforms(N, 2, g2), n_init=2)
    want, y_want = orc.qgemm_quant(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, act, R2, b2, s2, z2, ob,
                                   return_y=True)
    wp, cs, swo = P.rptq_pack_weights_out(c.Wq, c.R, c.bounds, wb, R2, b2, c.s_w)
    npad = orc.seg32_kpad(b2)
    yd = torch.full((M, npad), 7.0, dtype=torch.float32, device="cuda")
    got = P.rptq_qgemm_quant(dev(pitched(codes, c.bounds, ab)), M, K, npad, c.bounds, c.s, c.z, ab, dev(wp), wb,
                             dev(swo), dev(cs), act, b2, s2, z2, ob, y_out=yd)
    got = code_bytes(got, b2, ob); yg = yd.cpu().numpy()
    # padded position of each real output channel (in R2 order)
    pos = np.concatenate([orc.seg32_kpad(b2[:c2 + 1]) + np.arange(b2[c2 + 1] - b2[c2]) for c2 in range(g2)])
    real = np.zeros(npad, bool); real[pos] = True
    assert not yg[:, ~real].any()
    y_real = np.ascontiguousarray(yg[:, pos])
    assert rel_l2(y_real, y_want) <= 1e-3
    if act:
        assert (y_real >= 0).all()
    # bit-exact on the kernel's own y
    assert np.array_equal(got, orc.pack_seg32(orc.quantize(y_real, b2, s2, z2, ob), b2, ob))
    # end to end
    qg, pad = orc.unpack_seg32(got, N, b2, ob, return_pad=True)
    qw = orc.unpack_seg32(want, N, b2, ob)
    d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
    assert not pad.any()
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (d.max(), (d > 0).mean())


# ----------------------------------------------------------------------------- attention over packed KV
def _attn_inputs(B, T, C, g, bits, seed):
    out = []
    for k, (sch, scal, sev) in enumerate(((synthetic.STREAM_CHANNELS, synthetic.STREAM_CALIB, synthetic.STREAM_EVAL),
                                          (synthetic.STREAM_CHANNELS_V, synthetic.STREAM_CALIB_V,
                                           synthetic.STREAM_EVAL_V))):
        mu, sg = synthetic.channel_params(C, seed, 0.01, stream=sch)
        xc = synthetic.tokens(256, mu, sg, seed, scal)
        mx, mn = orc.channel_minmax(xc)
        R, bounds, s, z = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(seed + k, 2, g), n_init=2)
        x = synthetic.tokens(B * T, mu, sg, seed, sev)
        out.append((orc.kv_quant_pack(x, R, bounds, s, z, bits), (R, bounds, s, z)))
    return out


@pytest.mark.parametrize("B,T,C,D,g,bits", [(2, 300, 1024, 128, 8, 3), (3, 129, 512, 64, 4, 4),
                                           (1, 1, 256, 128, 2, 8), (2, 1000, 9216, 128, 32, 3),
                                           (5, 77, 640, 64, 5, 3)])
def test_kv_attention_matches_oracle(P, B, T, C, D, g, bits):
    """Decode attention reading the packed caches: per sequence within 1e-3
    (relative L2, the fp32 tolerance used for Y) of the oracle's fp64
    attention over the dequantized caches (ragged last chunk, T = 1, both
    head sizes, 3/4/8 bits)."""
    _say("kv attention", B, T, C, D, g, bits)
    (kp, kpar), (vp, vpar) = _attn_inputs(B, T, C, g, bits, seed=T + C + bits)
    q = (np.random.default_rng(T + C).standard_normal((B, C)) * 0.25).astype(np.float16)
    scale = 1.0 / np.sqrt(D)
    want = orc.kv_attention(q, kp, vp, B, T, C, D, scale, kpar, vpar, bits)
    qd = dev(q.view(np.int16)).view(torch.float16)
    dp = lambda par: (dev(par[0]), par[1], par[2], par[3])
    got = P.rptq_kv_attention(qd, dev(kp), dev(vp), B, T, C, D, float(scale), dp(kpar), dp(vpar), bits)
    got = got.cpu().numpy().astype(np.float64)
    for b in range(B):
        assert rel_l2(got[b], want[b]) <= 1e-3, (b, rel_l2(got[b], want[b]))


# ----------------------------------------------------------------------------- calibration
def test_calib_minmax_matches_oracle(P):
    K = 1024
    mu, sg = synthetic.channel_params(K, 5, 0.01)
    x = synthetic.tokens(200, mu, sg, 5, synthetic.STREAM_CALIB)
    x[3, :4] = [-0.0, 0.0, 65504, -65504]
    gamma, beta = synthetic.ln_params(K, 5)
    mx, mn = P.rptq_calib_minmax(dev(x.view(np.int16)).view(torch.float16), P.RPTQ_CALIB_RAW)
    mx_o, mn_o = orc.channel_minmax(x)
    assert np.array_equal(mx.cpu().numpy(), mx_o) and np.array_equal(mn.cpu().numpy(), mn_o)
    mx, mn = P.rptq_calib_minmax(dev(x.view(np.int16)).view(torch.float16), P.RPTQ_IN_FP16_RAW,
                                 dev(gamma), dev(beta))
    mx_o, mn_o = orc.channel_minmax(orc.layernorm(x, gamma, beta))
    np.testing.assert_allclose(mx.cpu().numpy(), mx_o, rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(mn.cpu().numpy(), mn_o, rtol=2e-5, atol=2e-5)


# ----------------------------------------------------------------------------- HIP graphs
def test_hot_path_replays_from_a_hip_graph(P):
    """The layer (fused LayerNorm-quant -> GEMM, and the dynamic-range
    pipeline -> device-scale GEMM) captured once in a HIP graph and replayed
    several times, with eager work and synchronizations between replays:
    every replay reproduces the eager results bit for bit (the library
    records no memset and allocates nothing, so its launches capture as
    plain kernel nodes)."""
    M, K, N, g, ab, wb = 96, 2048, 264, 8, 4, 4
    c = layer_case(M, K, N, g, ab, wb, seed=4242)
    xd = dev(c.x.view(np.int16)).view(torch.float16)
    Rd, gr, br = dev(c.R), dev(c.gamma[c.R]), dev(c.beta[c.R])
    wp, cs, sw = _gemm_inputs(P, c)
    rb = P.rptq_codes_row_bytes(c.bounds, ab)
    # zero-filled: the rows' pitch tails are never written, by eager runs or replays
    codes = torch.zeros((M, rb), dtype=torch.uint8, device="cuda")
    codes_d = torch.zeros_like(codes)
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Yd = torch.empty_like(Y)
    sd = torch.empty(g, dtype=torch.float32, device="cuda")
    zd = torch.empty(g, dtype=torch.int32, device="cuda")
    ws = torch.empty(P.rptq_ln_dynamic_workspace_bytes(g), dtype=torch.uint8, device="cuda")

    def layer():
        P.rptq_ln_reorder_quant(xd, Rd, gr, br, c.bounds, c.s, c.z, ab, out=codes)
        P.rptq_qgemm(codes, M, K, N, c.bounds, c.s, c.z, ab, wp, wb, sw, cs, out=Y)
        P.rptq_ln_reorder_quant_dynamic(xd, Rd, gr, br, c.bounds, ab, out=codes_d, s_out=sd, z_out=zd,
                                        workspace=ws)
        P.rptq_qgemm_dynamic(codes_d, M, K, N, c.bounds, sd, zd, ab, wp, wb, sw, cs, out=Yd)

    layer()
    torch.cuda.synchronize()
    want = [t.clone() for t in (codes, Y, codes_d, sd, zd, Yd)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()                                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    for rep in range(4):
        for t in (codes, Y, codes_d, sd, zd, Yd):
            t.zero_()                               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((codes, Y, codes_d, sd, zd, Yd), want):
            assert torch.equal(got, exp), rep


def test_kv_path_replays_from_a_hip_graph(P):
    """K/V pack, dequantize and decode attention (tables, chunk and merge
    kernels) captured once in a HIP graph and replayed with eager work
    between replays: every replay equals the eager results bit for bit."""
    B, T, C, D, g, bits = 2, 300, 1024, 128, 8, 3
    (kp, kpar), (vp, vpar) = _attn_inputs(B, T, C, g, bits, seed=77)
    R, bounds, s, z = kpar
    kv = orc.half_to_double(orc.kv_dequant(kp, C, R, bounds, s, z, bits)).astype(np.float16)
    kvd = dev(kv.view(np.int16)).view(torch.float16)
    q = (np.random.default_rng(5).standard_normal((B, C)) * 0.25).astype(np.float16)
    qd = dev(q.view(np.int16)).view(torch.float16)
    dp = lambda par: (dev(par[0]), par[1], par[2], par[3])
    kpar_d, vpar_d = dp(kpar), dp(vpar)
    kpd, vpd = dev(kp), dev(vp)
    packed = torch.empty((B * T, P.rptq_kv_row_bytes(C, bits)), dtype=torch.uint8, device="cuda")
    deq = torch.empty((B * T, C), dtype=torch.float16, device="cuda")
    att = torch.empty((B, C), dtype=torch.float32, device="cuda")
    ws = torch.empty(P.rptq_kv_attention_workspace_bytes(B, T, C, D), dtype=torch.uint8, device="cuda")

    def path():
        P.rptq_kv_quant_pack(kvd, kpar_d[0], bounds, s, z, bits, out=packed)
        P.rptq_kv_dequant(packed, C, kpar_d[0], bounds, s, z, bits, out=deq)
        P.rptq_kv_attention(qd, kpd, vpd, B, T, C, D, 0.125, kpar_d, vpar_d, bits, out=att, workspace=ws)

    path()
    torch.cuda.synchronize()
    want = [t.clone() for t in (packed, deq, att)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(4):
        for t in (packed, deq, att):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, exp in zip((packed, deq, att), want):
            assert torch.equal(got, exp), rep


# ----------------------------------------------------------------------------- smallest shapes
@pytest.mark.parametrize("bits", [3, 4, 8])
@pytest.mark.parametrize("bounds", [[0, 8], [0, 1, 2, 3, 4, 5, 6, 7, 8], [0, 3, 8]], ids=["g1", "g8", "g2"])
def test_smallest_layer(P, bits, bounds):
    """K = 8 (one 8-code unit of real channels), every cluster padded to 32:
    LayerNorm-quant (fused within tolerance, quant-only and dynamic bit
    exact), the GEMM (accumulators exact) and the dynamic-range GEMM."""
    M, K, N = 5, 8, 24
    _say("smallest", bits, bounds)
    c = explicit_case(M, K, N, bounds, bits, 4, seed=len(bounds) + bits)
    y = orc.layernorm(c.x, c.gamma, c.beta, 1e-5, c.R)
    want = orc.pack_seg32(orc.quantize(y, c.bounds, c.s, c.z, bits), c.bounds, bits)
    got = P.rptq_ln_reorder_quant(dev(y), None, None, None, c.bounds, c.s, c.z, bits,
                                  in_mode=P.RPTQ_IN_FP32_NORMALIZED)
    assert np.array_equal(code_bytes(got, c.bounds, bits), want)
    wd, sd_o, zd_o = orc.quantize_dynamic(y, c.bounds, bits)
    gd, sd, zd = P.rptq_ln_reorder_quant_dynamic(dev(y), None, None, None, c.bounds, bits,
                                                 in_mode=P.RPTQ_IN_FP32_NORMALIZED)
    assert np.array_equal(code_bytes(gd, c.bounds, bits), wd)
    assert np.array_equal(sd.cpu().numpy(), sd_o) and np.array_equal(zd.cpu().numpy(), zd_o)
    fused = code_bytes(_fused(P, c, bits), c.bounds, bits)
    qf = orc.unpack_seg32(fused, K, c.bounds, bits).astype(np.int32)
    qo = orc.unpack_seg32(orc.ln_reorder_quant(c.x, c.gamma, c.beta, 1e-5, c.R, c.bounds, c.s, c.z, bits),
                          K, c.bounds, bits).astype(np.int32)
    assert np.abs(qf - qo).max() <= 1
    q = orc.unpack_seg32(want, K, c.bounds, bits)
    Y_o, acc_o = orc.qgemm(q, c.Wq, c.R, c.bounds, c.s, c.z, c.s_w, return_acc=True)
    wp, cs, sw = _gemm_inputs(P, c)
    acc = torch.zeros((c.g, M, N), dtype=torch.int32, device="cuda")
    Y = P.rptq_qgemm(dev(pitched(want, c.bounds, bits)), M, K, N, c.bounds, c.s, c.z, bits, wp, 4, sw, cs,
                     acc_debug=acc)
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    assert rel_l2(Y.cpu().numpy(), Y_o) <= 1e-3
    Yd = P.rptq_qgemm_dynamic(gd, M, K, N, c.bounds, sd, zd, bits, wp, 4, sw, cs)
    Ys = P.rptq_qgemm(gd, M, K, N, c.bounds, sd.cpu().numpy(), zd.cpu().numpy(), bits, wp, 4, sw, cs)
    assert torch.equal(Yd, Ys)


@pytest.mark.parametrize("bits,C", [(4, 8), (8, 8), (3, 32), (4, 32)])
def test_smallest_kv_rows(P, bits, C):
    """The narrowest K/V rows (C = 8, 3-bit C = 32), single-channel clusters
    included: pack and dequant bit-exact."""
    T = 7
    r = np.random.default_rng(C + bits)
    kv = (r.standard_normal((T, C)) * 3).astype(np.float16)
    bounds = np.array(sorted({0, C} | {int(v) for v in r.integers(1, C, 3)}), np.int32)
    R = r.permutation(C).astype(np.int32)
    mx, mn = orc.channel_minmax(kv)
    s, z = orc.cluster_params(mx, mn, R, bounds, bits)
    want = orc.kv_quant_pack(kv, R, bounds, s, z, bits)
    got = P.rptq_kv_quant_pack(dev(kv.view(np.int16)).view(torch.float16), dev(R), bounds, s, z, bits)
    assert np.array_equal(got.cpu().numpy(), want)
    deq = P.rptq_kv_dequant(dev(want), C, dev(R), bounds, s, z, bits)
    assert np.array_equal(deq.cpu().numpy().view(np.uint16), orc.kv_dequant(want, C, R, bounds, s, z, bits))
