"""Pins of the oracle against facts the pages and the mathematics fix.

None of these re-types an oracle formula: each checks a closed form, an
invariant, a worked example from the pages, a library routine on a special
case, or brute force on tiny inputs, chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one.
"""
import itertools
import math
import json
import os

import numpy as np
import pytest

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- fp16
def test_half_decode_all_bit_patterns_match_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_half_encode_matches_numpy_round_to_nearest_even(orc):
    r = np.random.default_rng(7)
    x = np.concatenate([
        r.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (r.standard_normal(50000) * 1e-5).astype(np.float32),          # subnormal halves
        (r.standard_normal(50000) * 3e4).astype(np.float32),           # near the top
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e9, -np.inf, np.inf,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11], np.float32),
    ])
    # exact ties between neighbouring halves: k + 0.5 ulp for random halves
    h = r.integers(0x0400, 0x7bff, 5000).astype(np.uint16).view(np.float16).astype(np.float64)
    ulp = np.spacing(h.astype(np.float16)).astype(np.float64)
    ties = (h + ulp / 2).astype(np.float32)
    x = np.concatenate([x, ties])
    ours = orc.float_to_half_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------- quantization
def test_round_half_even_ties_and_clipping(orc):
    # s = 1 -> inv_s = 1: the code is round-half-even(y) + z, clipped to [0, qmax]
    bounds = np.array([0, 1], np.int32)
    s = np.array([1.0], np.float32)
    y = np.array([[2.5], [3.5], [-2.5], [0.5], [1.5], [-0.5], [7.49], [7.5], [8.5], [-9.0], [1e30],
                  [-1e30], [np.inf], [-np.inf], [np.nan]], np.float32)
    q = orc.quantize(y, bounds, s, np.array([8], np.int32), 4)[:, 0]
    # 2.5->2, 3.5->4, -2.5->-2, 0.5->0, 1.5->2, -0.5->-0, 7.49->7, 7.5->8, 8.5->8 (ties to even), +8
    assert q.tolist() == [10, 12, 6, 8, 10, 8, 15, 15, 15, 0, 15, 0, 15, 0, 0]
    q0 = orc.quantize(y, bounds, s, np.array([0], np.int32), 3)[:, 0]
    assert q0.tolist() == [2, 4, 0, 0, 2, 0, 7, 7, 7, 0, 7, 0, 7, 0, 0]


def test_product_is_rounded_once(orc):
    # y * inv_s lands within one fp32 ulp of a half-integer; a quantizer that
    # first rounds the product to fp32 would hit the tie and round to even.
    s = np.array([1.0 / 3.0], np.float32)                       # inv_s = fp32(1/s)
    inv_s = np.float32(1.0) / s[0]
    # choose y with exact product y*inv_s slightly above 2.5
    y = np.float32(2.5) / inv_s
    for _ in range(64):
        p = np.float64(y) * np.float64(inv_s)
        if p > 2.5 and np.float32(p) == np.float32(2.5):
            break
        y = np.nextafter(y, np.float32(np.inf))
    p = np.float64(y) * np.float64(inv_s)
    assert p > 2.5 and np.float32(p) == np.float32(2.5)
    q = orc.quantize(np.array([[y]], np.float32), np.array([0, 1], np.int32), s,
                     np.array([0], np.int32), 8)
    assert q[0, 0] == 3


def _in_range_error_bound(s, lo, hi):
    return s / 2 * (1 + 2.0 ** -20) + 2.0 ** -22 * max(abs(lo), abs(hi))


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_dequant_error_at_most_half_step_inside_cluster_range(orc, bits):
    # |y - s_c (q - z_c)| <= s_c / 2 for y inside the cluster's calibrated range
    r = np.random.default_rng(bits)
    K, g = 96, 6
    lo = np.sort(r.normal(0, 30, K)).astype(np.float32)
    width = r.lognormal(0, 1.5, K).astype(np.float32)
    mn, mx = lo, (lo + width).astype(np.float32)
    mx[5] = mn[5] = 3.0                                    # a constant channel
    bounds = np.array(np.linspace(0, K, g + 1), np.int32)
    s, z = orc.cluster_params(mx, mn, None, bounds, bits)
    for c in range(g):
        a, b = bounds[c], bounds[c + 1]
        clo, chi = float(mn[a:b].min()), float(mx[a:b].max())
        y = r.uniform(clo, chi, (4000, 1)).astype(np.float32)
        y = np.concatenate([y, [[clo], [chi]]]).astype(np.float32)
        yy = np.repeat(y, b - a, axis=1)
        q = orc.quantize(np.pad(yy, ((0, 0), (a, K - b))), bounds, s, z, bits)[:, a:b]
        deq = float(s[c]) * (q.astype(np.float64) - z[c])
        err = np.abs(yy.astype(np.float64) - deq).max()
        assert err <= _in_range_error_bound(float(s[c]), clo, chi), (c, err, s[c])


def test_two_channel_example_per_cluster_beats_per_tensor(orc):
    """The write-up's example: ranges [-100,-50] and [80,100]."""
    gold = json.load(open(os.path.join(GOLDEN, "two_channel_example.json")))
    (a_lo, a_hi), (b_lo, b_hi) = gold["ranges"]
    r = np.random.default_rng(11)
    n = 200
    chA = np.concatenate([[a_lo, a_hi], r.uniform(a_lo, a_hi, n - 2)]).astype(np.float32)
    chB = np.concatenate([[b_lo, b_hi], r.uniform(b_lo, b_hi, n - 2)]).astype(np.float32)
    acts = np.stack([chA, chB], axis=1)                     # [tokens][2 channels]
    mx, mn = orc.channel_minmax(acts)
    assert mx.tolist() == [a_hi, b_hi] and mn.tolist() == [a_lo, b_lo]
    u = synthetic.kmeans_uniforms(5, 10, 2)
    R, bounds, s, z = orc.calibrate(mx, mn, 2, 8, u)
    # KMeans separates the two channels; lower minimum first
    assert bounds.tolist() == [0, 1, 2] and R.tolist() == [0, 1]
    for bits in (8, 4, 3):
        R, bounds, s, z = orc.calibrate(mx, mn, 2, bits, u)
        s_t, z_t = orc.cluster_params(mx, mn, None, np.array([0, 2], np.int32), bits)
        hs = gold["half_step"][str(bits)]
        np.testing.assert_allclose(s / 2, hs["per_cluster"], rtol=1e-6)
        np.testing.assert_allclose(s_t / 2, hs["per_tensor"], rtol=1e-6)
        # measured errors: per cluster vs per tensor
        q = orc.quantize(acts[:, R], bounds, s, z, bits)
        deq = orc.dequantize(q, bounds, s, z)
        err_c = np.abs(deq - acts[:, R]).astype(np.float64)
        qt = orc.quantize(acts, np.array([0, 2], np.int32), s_t, z_t, bits)
        deqt = orc.dequantize(qt, np.array([0, 2], np.int32), s_t, z_t)
        err_t = np.abs(deqt - acts).astype(np.float64)
        for j in range(2):
            assert err_c[:, j].max() <= hs["per_cluster"][j] * (1 + 1e-5)
            assert err_t[:, j].max() <= hs["per_tensor"] * (1 + 1e-5)
            assert (err_c[:, j] ** 2).mean() < (err_t[:, j] ** 2).mean()
        if bits == 8:
            th = gold["mse_uniform_theory_s2_over_12"]["8"]
            for j in range(2):
                assert (err_c[:, j] ** 2).mean() == pytest.approx(th["per_cluster"][j], rel=0.35)
                assert (err_t[:, j] ** 2).mean() == pytest.approx(th["per_tensor"], rel=0.35)


def test_cluster_scale_never_exceeds_tensor_scale(orc):
    """A cluster's range lies inside the tensor's range, so s_c <= s_tensor."""
    for name, w in synthetic.WORKLOADS.items():
        K = min(w.K, 2048)
        mu, sg = synthetic.channel_params(K, w.seed, w.outlier_frac, range_ratio=w.range_ratio)
        x = synthetic.tokens(128, mu, sg, w.seed, synthetic.STREAM_CALIB)
        mx, mn = orc.channel_minmax(x)
        for bits in (3, 4, 8):
            R, bounds, s, z = orc.calibrate(mx, mn, w.g, bits, synthetic.kmeans_uniforms(w.seed, 3, w.g),
                                            n_init=3)
            s_t, _ = orc.cluster_params(mx, mn, None, np.array([0, K], np.int32), bits)
            assert (s <= s_t[0] * (1 + 2.0 ** -23)).all(), name
            assert np.abs(z).max() <= 2 ** 21


def test_zero_point_floor_keeps_far_from_zero_clusters_exact(orc):
    # a constant cluster far from zero: the scale floor keeps |z| <= 2^21 and
    # the value is reproduced by dequantization
    mx = np.array([5000.0, 5000.0, -1.0], np.float32)
    mn = np.array([5000.0, 5000.0, -2.0], np.float32)
    bounds = np.array([0, 2, 3], np.int32)
    s, z = orc.cluster_params(mx, mn, None, bounds, 4)
    assert abs(int(z[0])) <= 2 ** 21 and s[0] > 0
    q = orc.quantize(np.array([[5000.0, 5000.0, -1.5]], np.float32), bounds, s, z, 4)
    deq = orc.dequantize(q, bounds, s, z)
    assert abs(float(deq[0, 0]) - 5000.0) <= float(s[0]) / 2 + 1e-3
    # identically zero cluster
    s0, z0 = orc.cluster_params(np.zeros(1, np.float32), np.zeros(1, np.float32), None,
                                np.array([0, 1], np.int32), 3)
    assert s0[0] == 1.0 and z0[0] == 0


# ----------------------------------------------------------------------------- LayerNorm
def _x_small(M, K, seed=3, frac=0.02):
    mu, sg = synthetic.channel_params(K, seed, frac)
    return synthetic.tokens(M, mu, sg, seed, synthetic.STREAM_EVAL)


def test_layernorm_identity_params_match_textbook_numpy(orc):
    x = _x_small(64, 256)
    y = orc.layernorm(x, np.ones(256, np.float32), np.zeros(256, np.float32), 1e-5)
    xd = x.astype(np.float64)
    ref = (xd - xd.mean(1, keepdims=True)) / np.sqrt(xd.var(1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(y, ref, rtol=2e-7, atol=1e-6)
    # closed form: mean 0 and variance var/(var+eps) per row
    assert np.abs(y.astype(np.float64).mean(1)).max() < 1e-5


def test_layernorm_random_affine_matches_textbook_numpy(orc):
    """gamma and beta away from (1, 0): y = gamma * (x - mean) / sqrt(var + eps)
    + beta against a plain fp64 numpy LayerNorm, in natural and in reordered
    order (RPTQ write-up, method section and Fig. 3: the LayerNorm emits
    reordered activations with reordered gamma and beta).  Dropping beta,
    dividing by gamma or indexing gamma without R each fail here."""
    K = 320
    x = _x_small(40, K, seed=5)
    gamma, beta = synthetic.ln_params(K, 17)
    assert np.abs(beta).max() > 0.1 and np.abs(gamma - 1).max() > 0.1
    xd = x.astype(np.float64)
    mu = xd.mean(1, keepdims=True)
    var = ((xd - mu) ** 2).mean(1, keepdims=True)
    ref = gamma.astype(np.float64) * (xd - mu) / np.sqrt(var + 1e-5) + beta.astype(np.float64)
    y = orc.layernorm(x, gamma, beta, 1e-5)
    np.testing.assert_allclose(y, ref, rtol=2e-7, atol=2e-7)
    R = np.random.default_rng(8).permutation(K).astype(np.int32)
    np.testing.assert_allclose(orc.layernorm(x, gamma, beta, 1e-5, R), ref[:, R], rtol=2e-7, atol=2e-7)


def test_layernorm_hand_worked_example(orc):
    """Four channels worked by hand (tests/golden/layernorm_hand_example.json):
    mean 2, variance 1, eps 3, so the normalizer is exactly 1/2 and every
    output is exact in fp32."""
    ex = json.load(open(os.path.join(GOLDEN, "layernorm_hand_example.json")))
    x = np.array([ex["x"]], np.float16)
    gamma = np.array(ex["gamma"], np.float32)
    beta = np.array(ex["beta"], np.float32)
    R = np.array(ex["R"], np.int32)
    y = orc.layernorm(x, gamma, beta, ex["eps"])
    assert y[0].tolist() == ex["y_natural"]
    yr = orc.layernorm(x, gamma, beta, ex["eps"], R)
    assert yr[0].tolist() == ex["y_reordered"]


def test_layernorm_reordered_params_equal_permuted_output(orc):
    """LN(x; gamma, beta)[R] == LN(x[R]; gamma[R], beta[R])."""
    K = 384
    x = _x_small(48, K)
    gamma, beta = synthetic.ln_params(K, 9)
    R = np.random.default_rng(2).permutation(K).astype(np.int32)
    fused = orc.layernorm(x, gamma, beta, 1e-5, R)
    natural = orc.layernorm(x, gamma, beta, 1e-5)
    assert np.array_equal(fused, natural[:, R])
    explicit = orc.layernorm(x[:, R], gamma[R], beta[R], 1e-5)
    # the statistics are summed in another order: within one fp32 ulp
    np.testing.assert_array_max_ulp(fused, explicit, maxulp=1)
    assert (fused == explicit).mean() > 0.999
    # a gamma indexed without R would break it
    wrong = orc.layernorm(x, gamma[R], beta[R], 1e-5, R)
    assert not np.allclose(wrong, fused)


def test_explicit_reorder_equals_fused_codes(orc):
    """Gather by R, LN with reordered params, quantize, pack == the fused oracle."""
    K, g, bits = 320, 5, 4
    x = _x_small(40, K, seed=4)
    gamma, beta = synthetic.ln_params(K, 4)
    mx, mn = orc.channel_minmax(orc.layernorm(x, gamma, beta))
    R, bounds, s, z = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(4, 4, g), n_init=4)
    fused = orc.ln_reorder_quant(x, gamma, beta, 1e-5, R, bounds, s, z, bits)
    y = orc.layernorm(np.ascontiguousarray(x[:, R]), gamma[R], beta[R], 1e-5)
    explicit = orc.pack_seg32(orc.quantize(y, bounds, s, z, bits), bounds, bits)
    assert np.array_equal(fused, explicit)


# ----------------------------------------------------------------------------- packing
def test_pack_hand_examples(orc):
    gold = json.load(open(os.path.join(GOLDEN, "pack_examples.json")))
    for case in gold["cases"]:
        c = np.array([case["codes"]], np.uint8)
        got = orc.pack_dense(c, case["bits"])[0].tolist()
        assert got == case["bytes"], case
        assert orc.unpack_dense(np.array([case["bytes"]], np.uint8), c.shape[1], case["bits"]).tolist() == c.tolist()


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_pack_round_trips(orc, bits):
    r = np.random.default_rng(bits)
    q = r.integers(0, 1 << bits, (7, 192), dtype=np.uint8)
    p = orc.pack_dense(q, bits)
    assert p.shape == (7, 192 * bits // 8)
    assert np.array_equal(orc.unpack_dense(p, 192, bits), q)
    # SEG32 with ragged clusters (sizes 1, 31, 32, 33, 95)
    bounds = np.array([0, 1, 32, 64, 97, 192], np.int32)
    assert orc.seg32_kpad(bounds) == 32 + 32 + 32 + 64 + 96
    ps = orc.pack_seg32(q, bounds, bits)
    assert ps.shape[1] == orc.seg32_kpad(bounds) * bits // 8
    back, pad = orc.unpack_seg32(ps, 192, bounds, bits, return_pad=True)
    assert np.array_equal(back, q)
    assert pad.shape[1] == orc.seg32_kpad(bounds) - 192 and not pad.any()


def test_pack_every_code_moves_only_its_bits(orc):
    # setting one code to its maximum changes exactly b bits of the packed row
    for bits, gs in ((3, 32), (4, 8), (8, 1)):
        base = orc.pack_dense(np.zeros((1, 32), np.uint8), bits)
        seen = np.zeros(base.shape[1] * 8, bool)
        for j in range(32):
            q = np.zeros((1, 32), np.uint8)
            q[0, j] = (1 << bits) - 1
            diff = np.unpackbits(orc.pack_dense(q, bits) ^ base)
            assert diff.sum() == bits
            assert not (seen & diff.astype(bool)).any()
            seen |= diff.astype(bool)
        assert seen.all()


# ----------------------------------------------------------------------------- KMeans
def _brute_force_kmeans(pts, g):
    best = np.inf
    C = len(pts)
    for lab in itertools.product(range(g), repeat=C):
        lab = np.array(lab)
        if len(set(lab.tolist())) < g:
            continue
        tot = 0.0
        for c in range(g):
            p = pts[lab == c]
            tot += ((p - p.mean(0)) ** 2).sum()
        best = min(best, tot)
    return best


def test_kmeans_matches_brute_force_on_separated_points(orc):
    r = np.random.default_rng(5)
    for trial in range(6):
        g = 2 + trial % 2
        C = 7 if g == 3 else 8
        centres = r.normal(0, 50, (g, 2))
        lab_true = np.arange(C) % g
        pts = centres[lab_true] + r.normal(0, 1, (C, 2))
        labels, cen, inertia, _ = orc.kmeans(pts, g, r.random(10 * g), 10)
        opt = _brute_force_kmeans(pts, g)
        assert inertia >= opt - 1e-9
        assert inertia == pytest.approx(opt, rel=1e-9, abs=1e-9)


def test_kmeans_never_beats_optimum_and_is_lloyd_fixed_point(orc):
    r = np.random.default_rng(6)
    for trial in range(6):
        g = 2 + trial % 2
        C = 7
        pts = r.normal(0, 10, (C, 2))
        labels, cen, inertia, iters = orc.kmeans(pts, g, r.random(4 * g), 4)
        assert inertia >= _brute_force_kmeans(pts, g) - 1e-9
        # fixed point: every point is nearest to its own centre, centres are means
        d = ((pts[:, None, :] - cen[None, :, :]) ** 2).sum(-1)
        assert (d[np.arange(C), labels] <= d.min(1) + 1e-12).all()
        for c in range(g):
            assert (labels == c).any()
            np.testing.assert_allclose(cen[c], pts[labels == c].mean(0), rtol=1e-12, atol=1e-12)


def test_kmeans_extreme_cluster_counts(orc):
    r = np.random.default_rng(8)
    pts = r.normal(0, 5, (9, 2))
    lab1, cen1, in1, _ = orc.kmeans(pts, 1, r.random(3), 3)
    assert (lab1 == 0).all()
    np.testing.assert_allclose(cen1[0], pts.mean(0), rtol=1e-12)
    labC, _, inC, _ = orc.kmeans(pts, 9, r.random(27), 3)
    assert sorted(labC.tolist()) == list(range(9)) and inC == 0.0
    # g = 1 reduces to per-tensor quantization
    mx, mn = pts[:, 0].astype(np.float32), np.minimum(pts[:, 0], pts[:, 1]).astype(np.float32)
    mx = np.maximum(mx, mn)
    R, bounds, s, z = orc.calibrate(mx, mn, 1, 4, r.random(3), n_init=3)
    s_t, z_t = orc.cluster_params(mx, mn, None, np.array([0, 9], np.int32), 4)
    assert bounds.tolist() == [0, 9] and s[0] == s_t[0] and z[0] == z_t[0]


def test_order_clusters_contiguous_and_sorted(orc):
    labels = np.array([2, 0, 1, 2, 0, 1, 1], np.int32)
    cen = np.array([[5.0, 1.0], [9.0, -3.0], [0.0, 1.0]])   # (max, min)
    R, bounds = orc.order_clusters(labels, cen)
    # min ascending: cluster 1 (-3), then clusters 2 and 0 tie on min 1 -> max 0 < 5
    assert bounds.tolist() == [0, 3, 5, 7]
    assert R.tolist() == [2, 5, 6, 0, 3, 1, 4]


# ----------------------------------------------------------------------------- GEMM
def test_qgemm_single_cluster_reduces_to_integer_matmul(orc):
    r = np.random.default_rng(10)
    M, K, N = 13, 70, 33
    q = r.integers(0, 256, (M, K), dtype=np.uint8)
    Wq = r.integers(-127, 128, (K, N)).astype(np.int8)
    R = r.permutation(K).astype(np.int32)
    one = np.ones(1, np.float32)
    Y, acc = orc.qgemm(q, Wq, R, np.array([0, K], np.int32), one, np.zeros(1, np.int32),
                       np.ones(N, np.float32), return_acc=True)
    ref = q.astype(np.int64) @ Wq[R].astype(np.int64)
    assert np.array_equal(acc[0], ref)
    assert np.array_equal(Y, ref.astype(np.float32))


def _dequant_reference(q, R, bounds, s, z, Wq, s_w):
    """fp64 sum over NATURAL channels of dequantized activation x dequantized
    weight, with a per-channel cluster lookup: no reordering at all."""
    M, K = q.shape
    cl = np.empty(K, np.int64)
    for c in range(len(bounds) - 1):
        cl[R[bounds[c]:bounds[c + 1]]] = c
    qn = np.empty_like(q)
    qn[:, R] = q
    xh = s.astype(np.float64)[cl] * (qn.astype(np.float64) - z.astype(np.float64)[cl])
    wh = Wq.astype(np.float64) * s_w.astype(np.float64)[None, :]
    return xh @ wh


def test_qgemm_brute_force_over_reorderings(orc):
    """Every R inducing the same partition gives the same per-cluster int32
    accumulators, and Y equals the natural-order dequantize-then-matmul."""
    r = np.random.default_rng(12)
    K, M, N = 6, 3, 5
    for g in (1, 2, 3):
        part = np.sort(np.arange(K) % g)                       # channel -> cluster
        part = r.permutation(part)
        members = [np.flatnonzero(part == c) for c in range(g)]
        sizes = [len(m) for m in members]
        bounds = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        a = r.normal(0, 3, (M, K)).astype(np.float32)          # natural-order activations
        s = r.uniform(0.05, 0.5, g).astype(np.float32)
        z = r.integers(-3, 12, g).astype(np.int32)
        Wq = r.integers(-7, 8, (K, N)).astype(np.int8)
        s_w = r.uniform(0.01, 0.1, N).astype(np.float32)
        ref_acc = None
        n_checked = 0
        for perm in itertools.permutations(range(K)):
            R = np.array(perm, np.int32)
            if any(set(R[bounds[c]:bounds[c + 1]].tolist()) != set(members[c].tolist()) for c in range(g)):
                continue
            q = orc.quantize(np.ascontiguousarray(a[:, R]), bounds, s, z, 4)
            Y, acc = orc.qgemm(q, Wq, R, bounds, s, z, s_w, return_acc=True)
            if ref_acc is None:
                ref_acc, ref_Y = acc, Y
            assert np.array_equal(acc, ref_acc)
            np.testing.assert_allclose(Y, ref_Y, rtol=1e-6, atol=0)
            deq = _dequant_reference(q, R, bounds, s, z, Wq, s_w)
            np.testing.assert_allclose(Y.astype(np.float64), deq, rtol=1e-6, atol=1e-9)
            n_checked += 1
        assert n_checked == int(np.prod([math.factorial(n) for n in sizes]))


def test_qgemm_matches_dequantized_matmul_realistic(orc):
    w = synthetic.small(synthetic.WORKLOADS["opt1.3b_fc1_w4a4"], M=24, K=256, N=48, g=6)
    mu, sg = synthetic.channel_params(w.K, w.seed, 0.02)
    x = synthetic.tokens(w.M, mu, sg, w.seed, synthetic.STREAM_EVAL)
    gamma, beta = synthetic.ln_params(w.K, w.seed)
    xc = synthetic.tokens(256, mu, sg, w.seed, synthetic.STREAM_CALIB)
    mx, mn = orc.channel_minmax(orc.layernorm(xc, gamma, beta))
    R, bounds, s, z = orc.calibrate(mx, mn, w.g, 4, synthetic.kmeans_uniforms(w.seed, 4, w.g), n_init=4)
    q = orc.quantize(orc.layernorm(x, gamma, beta, 1e-5, R), bounds, s, z, 4)
    Wq, s_w = orc.quantize_weights(synthetic.weights(w.K, w.N, w.seed), 4)
    Y = orc.qgemm(q, Wq, R, bounds, s, z, s_w)
    ref = _dequant_reference(q, R, bounds, s, z, Wq, s_w)
    np.testing.assert_allclose(Y.astype(np.float64), ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("out_bits", [3, 4, 8])
def test_qgemm_quant_error_bound_and_order_invariance(orc, out_bits):
    """The epilogue-quantized output of a reordered linear layer: every code
    dequantizes to within s_c / 2 of the activated output (values inside the
    calibrated cluster range), pads are 0, and the code of an output channel
    does not depend on where inside its cluster the channel is placed."""
    K, N, M, g, g2 = 128, 96, 24, 4, 5
    mu, sg = synthetic.channel_params(K, 31, 0.02)
    x = synthetic.tokens(M, mu, sg, 31, synthetic.STREAM_EVAL)
    gamma, beta = synthetic.ln_params(K, 31)
    y_in = orc.layernorm(x, gamma, beta)
    mx, mn = orc.channel_minmax(y_in)
    R, bounds, s, z = orc.calibrate(mx, mn, g, 4, synthetic.kmeans_uniforms(31, 2, g), n_init=2)
    q = orc.quantize(orc.layernorm(x, gamma, beta, 1e-5, R), bounds, s, z, 4)
    Wq, s_w = orc.quantize_weights(synthetic.weights(K, N, 31), 4)
    act = np.maximum(orc.qgemm(q, Wq, R, bounds, s, z, s_w), np.float32(0))
    omx, omn = orc.channel_minmax(act)
    R2, b2, s2, z2 = orc.calibrate(omx, omn, g2, out_bits, synthetic.kmeans_uniforms(32, 2, g2), n_init=2)
    codes, y = orc.qgemm_quant(q, Wq, R, bounds, s, z, s_w, 1, R2, b2, s2, z2, out_bits, return_y=True)
    assert np.array_equal(y, act[:, R2])
    qo, pad = orc.unpack_seg32(codes, N, b2, out_bits, return_pad=True)
    assert not pad.any()
    dq = orc.dequantize(qo, b2, s2, z2).astype(np.float64)
    for c in range(g2):
        sl = slice(b2[c], b2[c + 1])
        assert np.all(np.abs(dq[:, sl] - y[:, sl]) <= s2[c] / 2 * (1 + 1e-6) + 1e-12), c
    # the same partition, members in reverse order inside each cluster
    R3 = R2.copy()
    for c in range(g2):
        R3[b2[c]:b2[c + 1]] = R2[b2[c]:b2[c + 1]][::-1]
    q3 = orc.unpack_seg32(orc.qgemm_quant(q, Wq, R, bounds, s, z, s_w, 1, R3, b2, s2, z2, out_bits), N, b2,
                          out_bits)
    nat2 = np.empty_like(qo); nat2[:, R2] = qo
    nat3 = np.empty_like(q3); nat3[:, R3] = q3
    assert np.array_equal(nat2, nat3)


@pytest.mark.parametrize("wbits", [3, 4, 8])
def test_weight_quantization_bounds(orc, wbits):
    W = synthetic.weights(64, 40, 3)
    W[:, 7] = 0.0
    Wq, s_w = orc.quantize_weights(W, wbits)
    qm = 2 ** (wbits - 1) - 1
    mxq = np.abs(Wq.astype(np.int32)).max(0)
    assert (mxq[np.arange(40) != 7] == qm).all() and mxq[7] == 0 and s_w[7] == 1.0
    err = np.abs(W.astype(np.float64) - s_w.astype(np.float64) * Wq)
    assert (err <= s_w.astype(np.float64) / 2 * (1 + 1e-6)).all()


# ----------------------------------------------------------------------------- KV attention
def _attn_case(orc, B, T, C, bits, seed):
    mu, sg = synthetic.channel_params(C, seed, 0.02)
    kv = [synthetic.tokens(B * T, mu, sg, seed, st) for st in (synthetic.STREAM_EVAL, synthetic.STREAM_CALIB)]
    params = []
    for x in kv:
        mx, mn = orc.channel_minmax(x)
        R, bounds, s, z = orc.calibrate(mx, mn, 4, bits, synthetic.kmeans_uniforms(seed, 2, 4), n_init=2)
        params.append((R, bounds, s, z))
    packed = [orc.kv_quant_pack(x, *p, bits) for x, p in zip(kv, params)]
    return packed, params


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_attention_special_cases(orc, bits):
    """Closed forms of softmax attention: a zero query weighs every token
    equally (out = mean of the dequantized values); one cached token gives
    its value row; a query aligned with one key and scaled up selects that
    token's value row."""
    B, T, C, D = 2, 6, 64, 16
    (kp, vp), (kpar, vpar) = _attn_case(orc, B, T, C, bits, 41)
    V = orc.half_to_double(orc.kv_dequant(vp, C, *vpar, bits)).reshape(B, T, C)
    K = orc.half_to_double(orc.kv_dequant(kp, C, *kpar, bits)).reshape(B, T, C)
    q0 = np.zeros((B, C), np.float16)
    out = orc.kv_attention(q0, kp, vp, B, T, C, D, 0.25, kpar, vpar, bits)
    np.testing.assert_allclose(out, V.mean(axis=1), rtol=1e-12, atol=1e-12)
    out1 = orc.kv_attention(q0[:, :], kp.reshape(B, T, -1)[:, :1].reshape(B, -1),
                            vp.reshape(B, T, -1)[:, :1].reshape(B, -1), B, 1, C, D, 0.25, kpar, vpar, bits)
    np.testing.assert_allclose(out1, V[:, 0], rtol=0, atol=0)
    # query = the key of token 3 (per head), with a large scale: softmax -> one-hot
    qk = K[:, 3].astype(np.float16)
    outk = orc.kv_attention(qk, kp, vp, B, T, C, D, 1e3, kpar, vpar, bits)
    for b in range(B):
        for h in range(C // D):
            sl = slice(h * D, (h + 1) * D)
            sc = K[b, :, sl] @ qk[b, sl].astype(np.float64)
            if np.sort(sc)[-1] - np.sort(sc)[-2] > 0.05:        # a clear winner
                np.testing.assert_allclose(outk[b, sl], V[b, int(np.argmax(sc)), sl], rtol=1e-6, atol=1e-6)


# ----------------------------------------------------------------------------- KV cache
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_kv_round_trip_error_and_natural_order(orc, bits):
    T, C, g = 20, 256, 8
    mu, sg = synthetic.channel_params(C, 21, 0.02)
    kv = synthetic.tokens(T, mu, sg, 21, synthetic.STREAM_EVAL)
    mx, mn = orc.channel_minmax(kv)
    R, bounds, s, z = orc.calibrate(mx, mn, g, bits, synthetic.kmeans_uniforms(21, 3, g), n_init=3)
    packed = orc.kv_quant_pack(kv, R, bounds, s, z, bits)
    assert packed.shape == (T, C * bits // 8)
    out = orc.kv_dequant(packed, C, R, bounds, s, z, bits).view(np.float16).astype(np.float64)
    cl = np.empty(C, np.int64)
    for c in range(g):
        cl[R[bounds[c]:bounds[c + 1]]] = c
    xs = kv.astype(np.float64)
    lo, hi = mn.astype(np.float64), mx.astype(np.float64)
    bound = s.astype(np.float64)[cl] / 2 * (1 + 2.0 ** -20) + 2.0 ** -22 * np.maximum(np.abs(lo), np.abs(hi))
    # plus one fp16 rounding of the dequantized value
    bound = bound + np.abs(out) * 2.0 ** -11
    assert (np.abs(out - xs) <= bound[None, :]).all()
    # codes in reordered order: unpacked code j belongs to channel R[j]
    q = orc.unpack_dense(packed, C, bits)
    q2 = orc.quantize(np.ascontiguousarray(kv[:, R].astype(np.float32)), bounds, s, z, bits)
    assert np.array_equal(q, q2)


def _double_rounding_cases(count):
    """(s, n) pairs, s fp32 and n = q - z a small integer, whose exact product
    s * n lies just off a midpoint of two fp16 neighbours while its fp32
    rounding lands exactly on that midpoint: rounding the exact value once to
    fp16 and rounding it to fp32 first give different fp16 results."""
    cases = []
    for n in (3, 5, 7, -3, -6, 11):
        for base in (0.75, 1.0, 3.0, 100.0, -2.0 ** -16):
            h = np.float16(abs(base))
            ulp = float(np.spacing(h))
            for k in range(4):
                s0 = np.float32((float(h) + (k + 0.5) * ulp) / abs(n))
                for d in (-2, -1, 1, 2):
                    s_ = s0
                    for _ in range(abs(d)):
                        s_ = np.nextafter(s_, np.float32(np.inf) if d > 0 else np.float32(0))
                    v = float(s_) * n
                    if np.float16(v) != np.float16(np.float32(v)):
                        cases.append((s_, n))
    assert len(cases) >= count
    return cases[::max(1, len(cases) // count)][:count]


def test_kv_dequant_rounds_the_exact_product_once(orc):
    """Dequantization W = S (Wq - Z) (quantization lecture, 1.3) with the
    product formed exactly and rounded once to fp16, the plainest reading of a
    formula that names no intermediate precision: the oracle's fp16 outputs
    equal numpy's direct float64 -> float16 conversion (a library routine,
    round to nearest even) of s * (q - z) on cases built so that rounding to
    fp32 first would give the other fp16 neighbour."""
    cases = _double_rounding_cases(8)
    C = len(cases)                       # one channel per cluster, 4-bit codes
    bounds = np.arange(C + 1, dtype=np.int32)
    s = np.array([c[0] for c in cases], np.float32)
    q = np.array([[5, 9, 1, 15, 0, 7, 12, 3]], np.uint8)[:, :C]
    z = (q[0].astype(np.int32) - np.array([c[1] for c in cases], np.int32)).astype(np.int32)
    packed = orc.pack_dense(q, 4)
    out = orc.kv_dequant(packed, C, None, bounds, s, z, 4).view(np.float16)[0]
    exact = s.astype(np.float64) * (q[0].astype(np.int64) - z)
    once = exact.astype(np.float16)
    twice = exact.astype(np.float32).astype(np.float16)
    assert (once != twice).all()         # every case separates the two readings
    assert np.array_equal(out.view(np.uint16), once.view(np.uint16))


def test_kv_attention_two_token_closed_form(orc):
    """Two cached tokens: softmax over two scores is a logistic function, so
    out = V0 + (V1 - V0) * sigmoid(scale * q . (K1 - K0)) per head, over the
    dequantized cache.  A moderate, non-power-of-two scale keeps both weights
    well inside (0, 1), so a squared or doubly applied scale fails; doubling
    the scale moves the output exactly as the closed form predicts."""
    B, T, C, D, bits = 3, 2, 64, 32, 4
    (kp, vp), (kpar, vpar) = _attn_case(orc, B, T, C, bits, 43)
    K = orc.half_to_double(orc.kv_dequant(kp, C, *kpar, bits)).reshape(B, T, C)
    V = orc.half_to_double(orc.kv_dequant(vp, C, *vpar, bits)).reshape(B, T, C)
    rng = np.random.default_rng(4)
    q = np.empty((B, C), np.float16)
    for b in range(B):
        for h in range(C // D):
            sl = slice(h * D, (h + 1) * D)
            dk = K[b, 1, sl] - K[b, 0, sl]
            # a query whose margin q . (K1 - K0) is 5 (1.5 at scale 0.3), plus
            # a component orthogonal to K1 - K0 that changes no score gap
            nrm = np.sqrt(np.dot(dk, dk))
            noise = rng.standard_normal(D)
            noise -= np.dot(noise, dk) / nrm ** 2 * dk
            v = dk / nrm ** 2 * 5.0 + noise / np.sqrt(D) * (2.0 / nrm)
            q[b, sl] = v.astype(np.float16)
    qd = q.astype(np.float64)

    def closed(scale):
        out = np.empty((B, C))
        for b in range(B):
            for h in range(C // D):
                sl = slice(h * D, (h + 1) * D)
                a = scale * np.dot(qd[b, sl], K[b, 1, sl] - K[b, 0, sl])
                w1 = 1.0 / (1.0 + np.exp(-a))
                assert 0.05 < w1 < 0.95 or scale != 0.3
                out[b, sl] = V[b, 0, sl] + (V[b, 1, sl] - V[b, 0, sl]) * w1
        return out

    for scale in (0.3, 0.6):
        got = orc.kv_attention(q, kp, vp, B, T, C, D, scale, kpar, vpar, bits)
        np.testing.assert_allclose(got, closed(scale), rtol=1e-12, atol=1e-12)
    assert np.abs(closed(0.3) - closed(0.09)).max() > 1e-2       # scale^2 would be caught


# ----------------------------------------------------------------------------- dynamic ranges
def test_dynamic_ranges_hand_worked_example(orc):
    # quantization lecture 1.1 (dynamic: the scale comes from the current
    # activations) with 1.3's asymmetric s, z.  Two clusters of two channels,
    # two rows, 4 bits (qmax 15), worked by hand:
    #   cluster 0: values -1, 0.5, 2, 0 -> lo -1, hi 2, s = fp32(3/15) = fp32(0.2),
    #              z = rne(1/s) = 5 (1/s = 4.99999993), 1/s in fp32 = 5.0:
    #              -1 -> -5+5 = 0, 0.5 -> rne(2.5) = 2 -> 7, 2 -> 15, 0 -> 5
    #   cluster 1: values 3, 4, 5, 3.5 (range excludes 0) -> lo 3, hi 5,
    #              s = fp32(2/15), z = rne(-3/s) = rne(-22.4999994) = -22,
    #              1/s in fp32 = 7.4999995: 3 -> 22 -> 0, 4 -> 30 -> 8,
    #              5 -> 37 -> 15, 3.5 -> 26 -> 4
    y = np.array([[-1.0, 0.5, 3.0, 4.0], [2.0, 0.0, 5.0, 3.5]], np.float32)
    b = np.array([0, 2, 4], np.int32)
    s, z = orc.dynamic_cluster_params(y, b, 4)
    assert s[0] == np.float32(0.2) and s[1] == np.float32(2.0 / 15.0)
    assert z.tolist() == [5, -22]
    codes, s2, z2 = orc.quantize_dynamic(y, b, 4)
    q = orc.unpack_seg32(codes, 4, b, 4)
    assert q.tolist() == [[0, 7, 0, 8], [15, 5, 15, 4]]
    assert np.array_equal(s, s2) and np.array_equal(z, z2)


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_dynamic_ranges_cover_the_batch(orc, bits):
    # every value lies inside its cluster's own range, so (up to rounding at
    # the two ends) nothing is clipped: the smallest code of each cluster is 0
    # or 1, the largest qmax - 1 or qmax, and every value dequantizes within
    # one step; the extremes sit in rows other than the first (a range taken
    # from one row, or one range per channel, fails these)
    r = np.random.default_rng(31 + bits)
    M, K, g = 48, 160, 5
    b = np.array([0, 8, 40, 72, 130, 160], np.int32)
    y = (r.standard_normal((M, K)) * r.uniform(0.1, 6.0, K)).astype(np.float32)
    y[:, 40:72] += np.float32(9.0)               # a cluster whose range excludes 0
    y[M - 1, 3] = np.float32(50.0)               # extremes in the last rows
    y[M - 2, 100] = np.float32(-70.0)
    qmax = (1 << bits) - 1
    codes, s, z = orc.quantize_dynamic(y, b, bits)
    q = orc.unpack_seg32(codes, K, b, bits).astype(np.int64)
    for c in range(g):
        qc = q[:, b[c]:b[c + 1]]
        yc = y[:, b[c]:b[c + 1]].astype(np.float64)
        assert qc.min() in (0, 1) and qc.max() in (qmax - 1, qmax), (c, qc.min(), qc.max())
        deq = float(s[c]) * (qc - int(z[c]))
        assert np.abs(deq - yc).max() <= float(s[c]) * 1.0001
        # the step follows the batch's own range
        assert abs(float(s[c]) * qmax - (yc.max() - yc.min())) <= 1e-6 * (yc.max() - yc.min())
    assert q[M - 1, 3] == qmax and q[M - 2, 100] == 0


def test_dynamic_ranges_power_of_two_equivariance(orc):
    # scaling the batch by 2^k scales every s by 2^k exactly and keeps z and
    # the codes (all fp32 steps are exact under a power-of-two scaling)
    r = np.random.default_rng(5)
    y = (r.standard_normal((20, 96)) * 2.0 + 0.7).astype(np.float32)
    b = np.array([0, 30, 64, 96], np.int32)
    c1, s1, z1 = orc.quantize_dynamic(y, b, 4)
    c2, s2, z2 = orc.quantize_dynamic(y * np.float32(8.0), b, 4)
    assert np.array_equal(s2, s1 * np.float32(8.0))
    assert np.array_equal(z1, z2) and np.array_equal(c1, c2)


def test_dynamic_ln_matches_static_with_its_own_ranges(orc):
    # the dynamic LayerNorm path is the static one with (s, z) calibrated on
    # the same batch, and its ranges are those of the normalized rows
    r = np.random.default_rng(9)
    M, K = 24, 128
    x = orc.float_to_half_bits((r.standard_normal((M, K)) * 2.0 + 0.3).astype(np.float32))
    gamma = r.uniform(0.5, 1.5, K).astype(np.float32)
    beta = (r.standard_normal(K) * 0.1).astype(np.float32)
    R = r.permutation(K).astype(np.int32)
    b = np.array([0, 17, 64, 100, 128], np.int32)
    codes, s, z, y = orc.ln_reorder_quant_dynamic(x, gamma, beta, 1e-5, R, b, 4, return_y=True)
    codes_static = orc.ln_reorder_quant(x, gamma, beta, 1e-5, R, b, s, z, 4)
    assert np.array_equal(codes, codes_static)
    # with gamma = 1, beta = 0 every row of the normalized output has mean 0
    # and (biased) variance var / (var + eps), about 1 here
    y1 = orc.layernorm(x, np.ones(K, np.float32), np.zeros(K, np.float32), 1e-5, R)
    assert np.abs(y1.astype(np.float64).mean(axis=1)).max() < 1e-5
    assert np.abs(y1.astype(np.float64).var(axis=1) - 1.0).max() < 1e-4
    lo = [y[:, b[c]:b[c + 1]].min() for c in range(4)]
    q = orc.unpack_seg32(codes, K, b, 4)
    for c in range(4):
        j = np.argwhere(y[:, b[c]:b[c + 1]] == lo[c])[0]
        assert q[j[0], b[c] + j[1]] in (0, 1)
