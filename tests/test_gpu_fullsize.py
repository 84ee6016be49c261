"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times: the OPT-66B fc1 layer (16384 tokens x 9216 -> 36864, g = 32,
W4A4, W4A3 and W3A3), the OPT-66B K/V cache (524288 tokens x 9216 channels,
3 bit), and the three smaller layers (OPT-125m W8A8, OPT-1.3B fc1 W4A4,
OPT-13B QKV W4A4 / W4A8).  The device runs every row.  The oracle checks
every row of the fused LayerNorm codes, and samples the outputs whose oracle
cost grows with the product (GEMM rows over the full N, int32 accumulators
on 64-row slices, one K/V row per 8192-row chunk).  All parameters (R,
bounds, s, z, Wq) come from the oracle's calibration."""
import numpy as np
import pytest

import oracle as orc
import synthetic
from helpers import code_bytes, dev, pitched, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_quantization_layernorm_amd as P
    P.lib()
    return P


def _say(*a):
    print("[fullsize]", *a, flush=True)


@pytest.fixture(scope="module")
def fc1():
    """OPT-66B fc1 layer: inputs from the synthetic generator, parameters from
    the oracle's calibration (3 KMeans restarts to keep the CPU time short)."""
    w = synthetic.WORKLOADS["opt66b_fc1_w4a4"]
    M, K, N, g = w.M, w.K, w.N, w.g
    _say("generating", M, K, N)
    mu, sg = synthetic.channel_params(K, w.seed, w.outlier_frac)
    gamma, beta = synthetic.ln_params(K, w.seed, random=True)
    xc = synthetic.tokens(w.calib_tokens, mu, sg, w.seed, synthetic.STREAM_CALIB)
    mx, mn = orc.channel_minmax(orc.layernorm(xc, gamma, beta))
    x = synthetic.tokens(M, mu, sg, w.seed, synthetic.STREAM_EVAL)
    W = synthetic.weights(K, N, w.seed)
    wq = {wb: orc.quantize_weights(W, wb) for wb in (w.w_bits, 3)}
    del W
    u = synthetic.kmeans_uniforms(w.seed, 3, g)
    params = {}
    for ab in (4, 3):
        params[ab] = orc.calibrate(mx, mn, g, ab, u, n_init=3)
    _say("calibrated")
    return dict(M=M, K=K, N=N, g=g, x=x, gamma=gamma, beta=beta, wq=wq, params=params)


ROWS = np.array([0, 1, 255, 256, 4097, 9000, 16382, 16383])


def _spread_rows(M, n):
    """n rows evenly spaced over [0, M), first and last included."""
    return np.unique(np.round(np.linspace(0, M - 1, n)).astype(np.int64))


@pytest.mark.parametrize("ab", [4, 3])
def test_fc1_fullsize_ln_quant_every_row(P, fc1, ab):
    """The fused kernel's codes for all 16384 rows against the oracle's: at
    most 0.1% differ, each by at most 1; pad codes are 0."""
    M, K = fc1["M"], fc1["K"]
    R, bounds, s, z = fc1["params"][ab]
    _say("ln", ab)
    xd = dev(fc1["x"].view(np.int16)).view(torch.float16)
    codes = P.rptq_ln_reorder_quant(xd, dev(R), dev(fc1["gamma"][R]), dev(fc1["beta"][R]), bounds, s, z, ab)
    got = code_bytes(codes, bounds, ab)
    del codes, xd
    want = orc.ln_reorder_quant(fc1["x"], fc1["gamma"], fc1["beta"], 1e-5, R, bounds, s, z, ab)
    for r0 in range(0, M, 4096):                 # unpacked in slices to bound host memory
        qg, pad = orc.unpack_seg32(got[r0:r0 + 4096], K, bounds, ab, return_pad=True)
        qw = orc.unpack_seg32(want[r0:r0 + 4096], K, bounds, ab)
        d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
        assert not pad.any()
        assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (r0, d.max(), (d > 0).mean())


@pytest.mark.parametrize("ab,wb", [(4, 4), (3, 4), (3, 3)])
def test_fc1_fullsize_gemm_sampled(P, fc1, ab, wb):
    M, K, N, g = fc1["M"], fc1["K"], fc1["N"], fc1["g"]
    R, bounds, s, z = fc1["params"][ab]
    Wq, s_w = fc1["wq"][wb]
    _say("gemm", ab, wb)
    # every row's codes from the oracle, so Y isolates the GEMM
    codes_o = orc.ln_reorder_quant(fc1["x"], fc1["gamma"], fc1["beta"], 1e-5, R, bounds, s, z, ab)
    wp, cs = P.rptq_pack_weights(Wq, R, bounds, wb)
    wp, cs, sw = dev(wp), dev(cs), dev(s_w)
    cd = dev(pitched(codes_o, bounds, ab))
    Y = P.rptq_qgemm(cd, M, K, N, bounds, s, z, ab, wp, wb, sw, cs)
    # 256 evenly spaced rows (two in every 128-row tile-row) over the full N
    rows = _spread_rows(M, 256)
    Ys = Y[torch.from_numpy(rows).cuda()].cpu().numpy()
    del Y
    q = orc.unpack_seg32(codes_o[rows], K, bounds, ab)
    Y_o = orc.qgemm(q, Wq, R, bounds, s, z, s_w)
    assert rel_l2(Ys, Y_o) <= 1e-3
    for i in range(len(rows)):
        assert rel_l2(Ys[i], Y_o[i]) <= 1e-3, rows[i]
    # int32 accumulators bit-exact over full K and N on two 64-row slices
    # (a full-size debug buffer would be g x M x N x 4 bytes), in two places
    # of the batch (the middle and the last tile-row)
    for r0 in (4096, M - 64):
        acc = torch.zeros((g, 64, N), dtype=torch.int32, device="cuda")
        P.rptq_qgemm(cd[r0:r0 + 64], 64, K, N, bounds, s, z, ab, wp, wb, sw, cs, acc_debug=acc)
        q64 = orc.unpack_seg32(codes_o[r0:r0 + 64], K, bounds, ab)
        _, acc64 = orc.qgemm(q64, Wq, R, bounds, s, z, s_w, return_acc=True)
        assert np.array_equal(acc.cpu().numpy(), acc64), r0
        del acc


def test_fc1_fullsize_dynamic_sampled(P, fc1):
    """Dynamic ranges over the whole 16384-token batch: (s, z) against the
    oracle's (its ranges see every row), sampled rows' codes against the
    oracle's, and the device-scale GEMM equal to the host-scale one."""
    M, K, N, g = fc1["M"], fc1["K"], fc1["N"], fc1["g"]
    R, bounds, _, _ = fc1["params"][4]
    Wq, s_w = fc1["wq"][4]
    _say("dynamic ln + gemm")
    y = orc.layernorm(fc1["x"], fc1["gamma"], fc1["beta"], 1e-5, R)
    s_o, z_o = orc.dynamic_cluster_params(y, bounds, 4)
    want = orc.pack_seg32(orc.quantize(y[ROWS], bounds, s_o, z_o, 4), bounds, 4)
    del y
    xd = dev(fc1["x"].view(np.int16)).view(torch.float16)
    codes, sd, zd = P.rptq_ln_reorder_quant_dynamic(xd, dev(R), dev(fc1["gamma"][R]), dev(fc1["beta"][R]),
                                                    bounds, 4)
    sh, zh = sd.cpu().numpy(), zd.cpu().numpy()
    assert np.abs(sh.astype(np.float64) / s_o - 1.0).max() <= 1e-5
    assert np.abs(zh.astype(np.int64) - z_o).max() <= 1
    qg, pad = orc.unpack_seg32(code_bytes(codes[torch.from_numpy(ROWS).cuda()], bounds, 4), K, bounds, 4,
                               return_pad=True)
    qw = orc.unpack_seg32(want, K, bounds, 4)
    d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
    assert not pad.any()
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (d.max(), (d > 0).mean())
    del xd
    wp, cs = P.rptq_pack_weights(Wq, R, bounds, 4)
    wp, cs, sw = dev(wp), dev(cs), dev(s_w)
    Y = P.rptq_qgemm_dynamic(codes, M, K, N, bounds, sd, zd, 4, wp, 4, sw, cs)
    Ys = P.rptq_qgemm(codes, M, K, N, bounds, sh, zh, 4, wp, 4, sw, cs)
    assert torch.equal(Y, Ys)
    del Ys
    q = orc.unpack_seg32(code_bytes(codes[torch.from_numpy(ROWS).cuda()], bounds, 4), K, bounds, 4)
    Y_o = orc.qgemm(q, Wq, R, bounds, sh, zh, s_w)
    assert rel_l2(Y[torch.from_numpy(ROWS).cuda()].cpu().numpy(), Y_o) <= 1e-3


def test_kv_fullsize_sampled(P):
    kw = synthetic.KV_WORKLOADS["opt66b_kv_a3"]
    T, C, g, bits = kw.T, kw.C, kw.g, kw.bits
    _say("kv", T, C)
    mu, sg = synthetic.channel_params(C, kw.seed, kw.outlier_frac, stream=synthetic.STREAM_CHANNELS)
    kc = synthetic.tokens(kw.calib_tokens, mu, sg, kw.seed, synthetic.STREAM_CALIB)
    mx, mn = orc.channel_minmax(kc)
    R, bounds, s, z = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(kw.seed, 3, g), n_init=3)
    kv = synthetic.tokens_device(T, mu, sg, kw.seed, synthetic.STREAM_EVAL)
    packed = P.rptq_kv_quant_pack(kv, dev(R), bounds, s, z, bits)
    out = P.rptq_kv_dequant(packed, C, dev(R), bounds, s, z, bits)
    # one row in every 8192-row chunk (at a different offset in each), plus
    # the first and last rows
    rows = np.unique(np.concatenate([np.arange(64) * 8192 + (np.arange(64) * 1031) % 8192, [0, T - 1]]))
    ri = torch.from_numpy(rows).cuda()
    x_rows = kv[ri].cpu().numpy().view(np.uint16)
    want_p = orc.kv_quant_pack(x_rows, R, bounds, s, z, bits)
    assert np.array_equal(packed[ri].cpu().numpy(), want_p)
    want_d = orc.kv_dequant(want_p, C, R, bounds, s, z, bits)
    assert np.array_equal(out[ri].cpu().numpy().view(np.uint16), want_d)


def test_kv_attention_fullsize_sampled(P):
    """Decode attention over the whole OPT-66B cache (64 sequences x 8192
    tokens, 9216 channels = 72 heads x 128, 3 bit), in the launch the
    benchmark times; the oracle checks two sequences, packing their rows
    itself from the same fp16 cache rows."""
    kw = synthetic.KV_WORKLOADS["opt66b_kv_a3"]
    T, C, g, bits = kw.T, kw.C, kw.g, kw.bits
    B, Ts, D = 64, T // 64, 128
    _say("kv attention", B, Ts, C)
    params, packed, raw = [], [], []
    for k, (sch, scal, sev) in enumerate(((synthetic.STREAM_CHANNELS, synthetic.STREAM_CALIB, synthetic.STREAM_EVAL),
                                          (synthetic.STREAM_CHANNELS_V, synthetic.STREAM_CALIB_V,
                                           synthetic.STREAM_EVAL_V))):
        mu, sg = synthetic.channel_params(C, kw.seed, kw.outlier_frac, stream=sch)
        mx, mn = orc.channel_minmax(synthetic.tokens(kw.calib_tokens, mu, sg, kw.seed, scal))
        par = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(kw.seed + k, 3, g), n_init=3)
        x = synthetic.tokens_device(T, mu, sg, kw.seed, sev)
        packed.append(P.rptq_kv_quant_pack(x, dev(par[0]), par[1], par[2], par[3], bits))
        raw.append(x)
        params.append(par)
    q = (np.random.default_rng(5).standard_normal((B, C)) * 0.25).astype(np.float16)
    dp = lambda par: (dev(par[0]), par[1], par[2], par[3])
    got = P.rptq_kv_attention(dev(q.view(np.int16)).view(torch.float16), packed[0], packed[1], B, Ts, C, D,
                              float(1.0 / np.sqrt(D)), dp(params[0]), dp(params[1]), bits).cpu().numpy()
    del packed
    for b in (0, 41):
        rows = slice(b * Ts, (b + 1) * Ts)
        kp, vp = (orc.kv_quant_pack(r[rows].cpu().numpy().view(np.uint16), *par, bits)
                  for r, par in zip(raw, params))
        want = orc.kv_attention(q[b:b + 1], kp, vp, 1, Ts, C, D, 1.0 / np.sqrt(D), params[0], params[1], bits)
        assert rel_l2(got[b], want[0]) <= 1e-3, (b, rel_l2(got[b], want[0]))


# ----------------------------------------------------------------------------- the three smaller layers
SMALLER = [("opt125m_w8a8", 8), ("opt1.3b_fc1_w4a4", 4), ("opt13b_qkv_w4a4", 4), ("opt13b_qkv_w4a4", 8)]


@pytest.mark.parametrize("name,ab", SMALLER, ids=[f"{n}-A{a}" for n, a in SMALLER])
def test_layer_fullsize_sampled(P, name, ab):
    """The OPT-125m layer (W8A8), the OPT-1.3B fc1 (W4A4) and the OPT-13B
    QKV projection (W4A4 and W4A8, 10x-300x channel ranges) at their full
    sizes: the fused LayerNorm kernel over every row (every row's codes
    within the code tolerance), the GEMM over every row on the oracle's codes
    (at least 64 evenly spaced rows of Y within 1e-3, and the int32
    accumulators of a 64-row slice bit exact over full K and N)."""
    w = synthetic.WORKLOADS[name]
    M, K, N, g, wb = w.M, w.K, w.N, w.g, w.w_bits
    _say("layer", name, ab, M, K, N)
    mu, sg = synthetic.channel_params(K, w.seed, w.outlier_frac, range_ratio=w.range_ratio)
    gamma, beta = synthetic.ln_params(K, w.seed, random=True)
    xc = synthetic.tokens(w.calib_tokens, mu, sg, w.seed, synthetic.STREAM_CALIB)
    mx, mn = orc.channel_minmax(orc.layernorm(xc, gamma, beta))
    R, bounds, s, z = orc.calibrate(mx, mn, g, ab, synthetic.kmeans_uniforms(w.seed, 3, g), n_init=3)
    x = synthetic.tokens(M, mu, sg, w.seed, synthetic.STREAM_EVAL)
    Wq, s_w = orc.quantize_weights(synthetic.weights(K, N, w.seed), wb)
    rows = np.unique(np.concatenate([_spread_rows(M, 64), [1, M // 2 - 1, M // 2, M - 2]]))

    # fused LayerNorm + reorder + quantize + pack over every row, every row
    # compared with the oracle's codes
    xd = dev(x.view(np.int16)).view(torch.float16)
    codes = P.rptq_ln_reorder_quant(xd, dev(R), dev(gamma[R]), dev(beta[R]), bounds, s, z, ab)
    got = code_bytes(codes, bounds, ab)
    codes_o = orc.ln_reorder_quant(x, gamma, beta, 1e-5, R, bounds, s, z, ab)
    qg, pad = orc.unpack_seg32(got, K, bounds, ab, return_pad=True)
    qw = orc.unpack_seg32(codes_o, K, bounds, ab)
    d = np.abs(qg.astype(np.int32) - qw.astype(np.int32))
    assert not pad.any()
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (d.max(), (d > 0).mean())
    del codes

    # the GEMM over every row, on the oracle's codes
    wp, cs = P.rptq_pack_weights(Wq, R, bounds, wb)
    wp, cs, sw = dev(wp), dev(cs), dev(s_w)
    cd = dev(pitched(codes_o, bounds, ab))
    Y = P.rptq_qgemm(cd, M, K, N, bounds, s, z, ab, wp, wb, sw, cs)
    Ys = Y[torch.from_numpy(rows).cuda()].cpu().numpy()
    del Y
    Y_o = orc.qgemm(orc.unpack_seg32(codes_o[rows], K, bounds, ab), Wq, R, bounds, s, z, s_w)
    for i in range(len(rows)):
        assert rel_l2(Ys[i], Y_o[i]) <= 1e-3, rows[i]
    r0 = max(0, M // 2 - 32)
    n64 = min(64, M - r0)
    acc = torch.zeros((g, n64, N), dtype=torch.int32, device="cuda")
    P.rptq_qgemm(cd[r0:r0 + n64], n64, K, N, bounds, s, z, ab, wp, wb, sw, cs, acc_debug=acc)
    _, acc_o = orc.qgemm(orc.unpack_seg32(codes_o[r0:r0 + n64], K, bounds, ab), Wq, R, bounds, s, z, s_w,
                         return_acc=True)
    assert np.array_equal(acc.cpu().numpy(), acc_o)
