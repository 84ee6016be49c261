"""Benchmark of the RPTQ hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  1. fused LayerNorm + reorder + per-cluster quantize (4-bit), OPT-66B fc1
     input: 16384 tokens (batch 8 x seq 2048) x 9216 channels, g = 32;
  2. cluster-segmented int8-MFMA GEMM 9216 -> 36864 on those codes (W4A4);
  3. + 4. the same pair with 3-bit activations (W4A3);
  5. K/V cache quantize + pack, 3-bit, g = 32, of K and of V, each
     [64 x 8192 tokens][72 heads x 128] fp16 (OPT-66B KV cache);
  6. K/V dequantize of both back to fp16.
Inputs are generated (seeded, synthetic) and resident in HBM before the timed
region.  `value` is the tokens/s of the W4A4 LayerNorm-quant -> GEMM pair,
tokens / (t_LN + t_GEMM), with kernel times from HIP events recorded on the
stream the kernels are launched on; the other kernels' rates are extra keys.
`--gpus N` with N > 1 is refused: the library drives one GPU per process and
has no multi-GPU path.

Each timed step is preceded by a 1 GiB device write that flushes L2 and the
MALL (outside the kernel events); per-kernel times are medians over the
timed steps, with p10 / p90 and the mean beside them.  After the timed steps,
the three smaller layers (OPT-125m W8A8, OPT-1.3B fc1 W4A4, OPT-13B QKV W4A4
and W4A8) are timed cold and cache-resident (their inputs fit the MALL), and
the CPU baseline (the oracle) runs a row sample of the W4A4 layer and one
8192-token batch of the K/V pack.

Profiling helpers (not part of the timed step):
  --copy-probe       after the timed region, one plain device copy of
                     COPY_PROBE_BYTES, whose counter readings calibrate the HBM
                     byte counters;
  --ingest-pmc F W   read two rocprofv3 --pmc counter CSVs (FETCH_SIZE, then
                     WRITE_SIZE), scale them by the copy probe and write the
                     per-launch HBM traffic of each kernel to
                     profiles/hbm_traffic.json;
  --summarize-pmc CSV...  per-dispatch counters with derived rates (MFMA busy,
                     clock, LDS activity).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA (5.0 POPS)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "qgemm": ["post_quantization_layernorm_amd/csrc/qgemm.hip",
              "post_quantization_layernorm_amd/csrc/rptq_device.hpp"],
    "qgemm_quant_out": ["post_quantization_layernorm_amd/csrc/qgemm.hip",
                        "post_quantization_layernorm_amd/csrc/rptq_device.hpp"],
    "ln_reorder_quant": ["post_quantization_layernorm_amd/csrc/ln_quant.hip",
                         "post_quantization_layernorm_amd/csrc/rptq_device.hpp"],
    "kv_quant_pack": ["post_quantization_layernorm_amd/csrc/kv.hip",
                      "post_quantization_layernorm_amd/csrc/rptq_device.hpp"],
}


def measured_traffic(kernel: str, launches_bytes: float, path=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path)).get(kernel)
    if not d or d.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return d.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline leg (0: leave it out)")
    ap.add_argument("--no-flush", action="store_true",
                    help="leave out the cache flush (a 1 GiB device write) before each timed step")
    ap.add_argument("--no-small-configs", action="store_true",
                    help="leave out the OPT-125m / OPT-1.3B / OPT-13B layer timings after the timed steps")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed region, run one plain device copy of COPY_PROBE_BYTES")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print per-dispatch counters and derived rates (MFMA busy, clock, LDS activity) "
                         "from rocprofv3 --pmc counter CSVs and exit")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows shard across GPUs without any exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import post_quantization_layernorm_amd as P
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t_setup = time.time()

    # ------------------------------------------------------------------ OPT-66B fc1 layer
    w = synthetic.WORKLOADS["opt66b_fc1_w4a4"]
    M, K, N, g = w.M, w.K, w.N, w.g
    mu, sg = synthetic.channel_params(K, w.seed, w.outlier_frac)
    gamma, beta = synthetic.ln_params(K, w.seed, random=False)         # LayerNorm default init
    g_d = torch.from_numpy(gamma).to(dev); b_d = torch.from_numpy(beta).to(dev)
    xc = torch.from_numpy(synthetic.tokens(w.calib_tokens, mu, sg, w.seed, synthetic.STREAM_CALIB)).to(dev)
    mx, mn = P.rptq_calib_minmax(xc, P.RPTQ_IN_FP16_RAW, g_d, b_d)
    mx, mn = mx.cpu().numpy(), mn.cpu().numpy()
    R, bounds = P.rptq_kmeans_reorder(mx, mn, g, synthetic.kmeans_uniforms(w.seed, 10, g), n_init=10)
    R_d = torch.from_numpy(R).to(dev)
    gr_d = g_d[R_d].contiguous(); br_d = b_d[R_d].contiguous()
    x = torch.from_numpy(synthetic.tokens(M, mu, sg, w.seed, synthetic.STREAM_EVAL)).to(dev)
    log(f"[bench] layer inputs ready ({time.time() - t_setup:.1f}s)")
    W = synthetic.weights(K, N, w.seed)
    wts = {}                       # weight bits -> (packed W', colsum, s_w) on the device
    for wb in (w.w_bits, 3):
        wq, s_w = P.rptq_quantize_weights(W, wb)
        wp, cs = P.rptq_pack_weights(wq, R, bounds, wb)
        wts[wb] = (torch.from_numpy(wp).to(dev), torch.from_numpy(cs).to(dev), torch.from_numpy(s_w).to(dev))
        del wq, wp
    variants = {}
    for ab in (4, 3):
        s, z = P.rptq_cluster_params(mx, mn, R, bounds, ab)
        rb = P.rptq_codes_row_bytes(bounds, ab)
        variants[ab] = dict(s=s, z=z, codes=torch.empty((M, rb), dtype=torch.uint8, device=dev))
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    kpad = P.rptq_codes_kpad(bounds)
    # dynamic ranges: (s, z) of the 4-bit clusters from each batch, on the device
    dyn = dict(s=torch.empty(g, dtype=torch.float32, device=dev), z=torch.empty(g, dtype=torch.int32, device=dev),
               codes=torch.empty((M, P.rptq_codes_row_bytes(bounds, 4)), dtype=torch.uint8, device=dev),
               ws=torch.empty(P.rptq_ln_dynamic_workspace_bytes(g), dtype=torch.uint8, device=dev))
    log(f"[bench] weights ready, K_pad={kpad} ({time.time() - t_setup:.1f}s)")

    # fc1 with its output quantized for fc2 (ReLU, then fc2's 4-bit clusters):
    # fc2's input clusters come from fc1's own output on the calibration tokens
    v4 = variants[4]
    cc = P.rptq_ln_reorder_quant(xc, R_d, gr_d, br_d, bounds, v4["s"], v4["z"], 4)
    wp_d, cs_d, sw_d = wts[w.w_bits]
    yc = torch.relu(P.rptq_qgemm(cc, xc.shape[0], K, N, bounds, v4["s"], v4["z"], 4, wp_d, w.w_bits, sw_d, cs_d))
    omx, omn = yc.amax(0).cpu().numpy(), yc.amin(0).cpu().numpy()
    del cc, yc
    R2, b2 = P.rptq_kmeans_reorder(omx, omn, g, synthetic.kmeans_uniforms(w.seed + 1, 10, g), n_init=10)
    s2, z2 = P.rptq_cluster_params(omx, omn, R2, b2, 4)
    wq, s_w = P.rptq_quantize_weights(W, w.w_bits)
    wpo, cso, swo = P.rptq_pack_weights_out(wq, R, bounds, w.w_bits, R2, b2, s_w)
    del wq, W
    n_pad = P.rptq_codes_kpad(b2)
    qout = dict(w=torch.from_numpy(wpo).to(dev), cs=torch.from_numpy(cso).to(dev), sw=torch.from_numpy(swo).to(dev),
                bounds=b2, s=s2, z=z2, n_pad=n_pad,
                codes=torch.empty((M, P.rptq_codes_row_bytes(b2, 4)), dtype=torch.uint8, device=dev))
    del wpo
    log(f"[bench] fc2 input clusters ready, N_pad={n_pad} ({time.time() - t_setup:.1f}s)")

    # ------------------------------------------------------------------ OPT-66B KV cache
    kvw = synthetic.KV_WORKLOADS["opt66b_kv_a3"]
    T, C, kvb = kvw.T, kvw.C, kvw.bits
    kv = {}
    for name, (s_ch, s_cal, s_ev) in {"K": (synthetic.STREAM_CHANNELS, synthetic.STREAM_CALIB,
                                            synthetic.STREAM_EVAL),
                                      "V": (synthetic.STREAM_CHANNELS_V, synthetic.STREAM_CALIB_V,
                                            synthetic.STREAM_EVAL_V)}.items():
        kmu, ksg = synthetic.channel_params(C, kvw.seed, kvw.outlier_frac, stream=s_ch)
        kc = torch.from_numpy(synthetic.tokens(kvw.calib_tokens, kmu, ksg, kvw.seed, s_cal)).to(dev)
        kmx, kmn = P.rptq_calib_minmax(kc, P.RPTQ_CALIB_RAW)
        kmx, kmn = kmx.cpu().numpy(), kmn.cpu().numpy()
        kR, kbnd = P.rptq_kmeans_reorder(kmx, kmn, kvw.g, synthetic.kmeans_uniforms(kvw.seed + len(name), 10,
                                                                                  kvw.g), n_init=10)
        ks, kz = P.rptq_cluster_params(kmx, kmn, kR, kbnd, kvb)
        data = synthetic.tokens_device(T, kmu, ksg, kvw.seed, s_ev)
        kv[name] = dict(x=data, R=torch.from_numpy(kR).to(dev), bounds=kbnd, s=ks, z=kz,
                        packed=torch.empty((T, P.rptq_kv_row_bytes(C, kvb)), dtype=torch.uint8, device=dev),
                        out=torch.empty((T, C), dtype=torch.float16, device=dev))
    # decode attention over the packed caches: 64 sequences x 8192 tokens, 72 heads x 128
    AB, AD = 64, 128
    AT = T // AB
    q_att = torch.from_numpy((np.random.default_rng(5).standard_normal((AB, C)) * 0.25).astype(np.float16)).to(dev)
    att_ws = torch.empty(P.rptq_kv_attention_workspace_bytes(AB, AT, C, AD), dtype=torch.uint8, device=dev)
    att_out = torch.empty((AB, C), dtype=torch.float32, device=dev)
    log(f"[bench] KV caches ready ({time.time() - t_setup:.1f}s)")
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ one step
    names = ["ln4", "gemm4", "ln3", "gemm3", "gemm3w3", "gemm4q", "ln4d", "gemm4d", "kvq_K", "kvq_V", "kvd_K",
             "kvd_V", "kv_attn"]

    def step(ev=None):
        def rec(i):
            if ev is not None:
                ev[i].record(stream)
        k = 0
        for ab in (4, 3):
            v = variants[ab]
            rec(k)
            P.rptq_ln_reorder_quant(x, R_d, gr_d, br_d, bounds, v["s"], v["z"], ab, out=v["codes"], stream=stream)
            rec(k + 1)
            wp_d, cs_d, sw_d = wts[w.w_bits]
            P.rptq_qgemm(v["codes"], M, K, N, bounds, v["s"], v["z"], ab, wp_d, w.w_bits, sw_d, cs_d, out=Y,
                         stream=stream)
            k += 2
            if ab == 3:                    # the same 3-bit codes against 3-bit weights (W3A3)
                rec(k)
                wp_d, cs_d, sw_d = wts[3]
                P.rptq_qgemm(v["codes"], M, K, N, bounds, v["s"], v["z"], ab, wp_d, 3, sw_d, cs_d, out=Y,
                             stream=stream)
                k += 1
        rec(k)
        # fc1 on the 4-bit codes, output quantized for fc2
        v = variants[4]
        P.rptq_qgemm_quant(v["codes"], M, K, qout["n_pad"], bounds, v["s"], v["z"], 4, qout["w"], w.w_bits,
                           qout["sw"], qout["cs"], P.RPTQ_ACT_RELU, qout["bounds"], qout["s"], qout["z"], 4,
                           out=qout["codes"], stream=stream)
        k += 1
        rec(k)
        # the same layer with dynamic ranges (ranges pass + quantizing pass,
        # then the GEMM reading (s, z) from device memory)
        P.rptq_ln_reorder_quant_dynamic(x, R_d, gr_d, br_d, bounds, 4, out=dyn["codes"], s_out=dyn["s"],
                                        z_out=dyn["z"], workspace=dyn["ws"], stream=stream)
        k += 1
        rec(k)
        wp_d, cs_d, sw_d = wts[w.w_bits]
        P.rptq_qgemm_dynamic(dyn["codes"], M, K, N, bounds, dyn["s"], dyn["z"], 4, wp_d, w.w_bits, sw_d, cs_d,
                             out=Y, stream=stream)
        k += 1
        rec(k)
        for name in ("K", "V"):
            d = kv[name]
            P.rptq_kv_quant_pack(d["x"], d["R"], d["bounds"], d["s"], d["z"], kvb, out=d["packed"], stream=stream)
            k += 1
            rec(k)
        for name in ("K", "V"):
            d = kv[name]
            P.rptq_kv_dequant(d["packed"], C, d["R"], d["bounds"], d["s"], d["z"], kvb, out=d["out"],
                              stream=stream)
            k += 1
            rec(k)
        dk, dv = kv["K"], kv["V"]
        P.rptq_kv_attention(q_att, dk["packed"], dv["packed"], AB, AT, C, AD, float(1.0 / np.sqrt(AD)),
                            (dk["R"], dk["bounds"], dk["s"], dk["z"]), (dv["R"], dv["bounds"], dv["s"], dv["z"]),
                            kvb, out=att_out, workspace=att_ws, stream=stream)
        k += 1
        rec(k)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({time.time() - t_setup:.1f}s)")

    nev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    # L2 + MALL flush before every step (outside the kernel events; inside
    # the wall-clock of the steps, ~0.2 ms of a ~50 ms step)
    flush_buf = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xFF)
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)      # seconds
    # per-kernel medians (robust to one slow launch); mean and p10 / p90 are
    # reported beside them
    avg = {n: float(np.median(v)) for n, v in per.items()}
    stats = {n: {"median": float(np.median(v)) * 1e3, "mean": float(np.mean(v)) * 1e3,
                 "p10": float(np.percentile(v, 10)) * 1e3, "p90": float(np.percentile(v, 90)) * 1e3}
             for n, v in per.items()}
    log("[bench] per-kernel median ms: " + ", ".join(f"{n}={avg[n] * 1e3:.3f}" for n in names))

    ops = 2.0 * M * N * K
    res_layer = {}
    for ab in (4, 3):
        t_ln, t_gm = avg[f"ln{ab}"], avg[f"gemm{ab}"]
        ln_bytes = M * K * (2 + ab / 8)
        res_layer[ab] = dict(tokens_per_s=M / (t_ln + t_gm), ln_ms=t_ln * 1e3, gemm_ms=t_gm * 1e3,
                             gemm_tops=ops / t_gm / 1e12, gemm_frac_int8_peak=ops / t_gm / 1e12 / INT8_PEAK_TOPS,
                             ln_GBps=ln_bytes / t_ln / 1e9, ln_frac_hbm_peak=ln_bytes / t_ln / 1e9 / HBM_PEAK_GBPS)
    out = {}
    kv_bytes = T * C * (2 + kvb / 8)
    tq = (avg["kvq_K"] + avg["kvq_V"]) / 2
    td = (avg["kvd_K"] + avg["kvd_V"]) / 2
    out["kv_pack_GBps"] = kv_bytes / tq / 1e9
    out["kv_pack_frac_hbm_peak"] = kv_bytes / tq / 1e9 / HBM_PEAK_GBPS
    out["kv_dequant_GBps"] = kv_bytes / td / 1e9
    out["kv_pack_ms"] = tq * 1e3
    out["kv_dequant_ms"] = td * 1e3
    att_bytes = 2 * T * C * kvb / 8
    out["kv_attention"] = {"ms": avg["kv_attn"] * 1e3, "GBps": att_bytes / avg["kv_attn"] / 1e9,
                           "frac_hbm_peak": att_bytes / avg["kv_attn"] / 1e9 / HBM_PEAK_GBPS,
                           "shape": f"{AB} sequences x {AT} tokens, {C // AD} heads x {AD}, {kvb}-bit K and V",
                           "bytes": "packed K + V read once (the dequantize path writes and rereads "
                                    f"{2 * T * C * 2 / 1e9:.1f} GB of fp16)"}

    gemm_ops_launch = ops
    t_gemm = avg["gemm4"]
    traffic = measured_traffic("qgemm", gemm_ops_launch)
    roofline = {"bound": "mfma", "achieved": ops / t_gemm / 1e12, "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": ops / t_gemm / 1e12 / INT8_PEAK_TOPS, "traffic": traffic,
                "kernel": "qgemm_kernel<4,4>", "work_per_launch": f"2*M*N*K = {ops:.4g} int8 ops (unpadded K)"}
    ln_bytes = M * K * (2 + 4 / 8)
    rooflines = [roofline,
                 {"bound": "hbm", "kernel": "ln_reorder_quant_kernel<4,0,5,0>", "achieved": ln_bytes / avg["ln4"] / 1e9,
                  "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": ln_bytes / avg["ln4"] / 1e9 / HBM_PEAK_GBPS,
                  "traffic": measured_traffic("ln_reorder_quant", ln_bytes)}]
    rooflines.append({"bound": "hbm", "kernel": "kv_quant_pack_kernel<3>", "achieved": out["kv_pack_GBps"],
                      "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": out["kv_pack_frac_hbm_peak"],
                      "traffic": measured_traffic("kv_quant_pack", T * C * (2 + kvb / 8))})

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, x, gamma, beta, R, bounds, variants[4]["s"], variants[4]["z"], N, args.cpu_seconds)
        cpu["kv"] = cpu_baseline_kv({n: (kv[n]["x"], kv[n]["R"].cpu().numpy(), kv[n]["bounds"], kv[n]["s"],
                                         kv[n]["z"]) for n in ("K", "V")}, C, kvb)
    small = None
    if not args.no_small_configs:
        del Y, wts, variants, qout, dyn, kv
        torch.cuda.empty_cache()
        small = small_configs(P, torch, dev, stream, flush_buf)

    line = {
        "metric": "tokens/s + TOPS of fused LN-quant->qGEMM (% int8 MFMA peak); KV-pack GB/s",
        "value": res_layer[4]["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        # value is the W4A4 LayerNorm-quant -> GEMM pair alone; a step also
        # runs the other layer variants and the K/V kernels, so M per step
        # over the whole step is a different (smaller) figure
        "value_basis": "M / (t_LN + t_GEMM) of the W4A4 pair; ms_per_step covers every kernel of the step",
        "step_tokens_per_s": M / (elapsed / args.steps),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded per-channel N(mu_c, sigma_c) activations with 1% x100 outlier channels; "
                "W ~ N(0, 0.02))",
        "config": {"workload": "OPT-66B fc1 layer W4A4 (+W4A3, W3A3): LayerNorm(9216)+per-cluster quant -> "
                               "9216x36864 GEMM, 16384 tokens, g=32; plus OPT-66B KV cache 3-bit, "
                               "2 x [524288 x 9216] fp16",
                   "M": M, "K": K, "N": N, "g": g, "K_pad": kpad, "tokens_per_step": M},
        "tops": res_layer[4]["gemm_tops"],
        "gemm_frac_int8_peak": res_layer[4]["gemm_frac_int8_peak"],
        "ln_quant_GBps": res_layer[4]["ln_GBps"],
        "ln_quant_frac_hbm_peak": res_layer[4]["ln_frac_hbm_peak"],
        "w4a3": res_layer[3],
        "w4a4": res_layer[4],
        "w4a4_quant_out": {"gemm_ms": avg["gemm4q"] * 1e3, "gemm_tops": ops / avg["gemm4q"] / 1e12,
                           "gemm_frac_int8_peak": ops / avg["gemm4q"] / 1e12 / INT8_PEAK_TOPS,
                           "n_pad": n_pad, "out": "ReLU, fc2's 4-bit per-cluster codes (SEG32)"},
        "w4a4_dynamic": {"ln_ms": avg["ln4d"] * 1e3, "gemm_ms": avg["gemm4d"] * 1e3,
                         "tokens_per_s": M / (avg["ln4d"] + avg["gemm4d"]),
                         "ln_GBps_two_reads": M * K * (4 + 4 / 8) / avg["ln4d"] / 1e9,
                         "ln_frac_hbm_peak_two_reads": M * K * (4 + 4 / 8) / avg["ln4d"] / 1e9 / HBM_PEAK_GBPS,
                         "gemm_tops": ops / avg["gemm4d"] / 1e12,
                         "ln": "3 launches: ranges pass over x, (s, z), quantizing pass"},
        "w3a3": {"gemm_ms": avg["gemm3w3"] * 1e3, "gemm_tops": ops / avg["gemm3w3"] / 1e12,
                 "gemm_frac_int8_peak": ops / avg["gemm3w3"] / 1e12 / INT8_PEAK_TOPS,
                 "tokens_per_s": M / (avg["ln3"] + avg["gemm3w3"])},
        **out,
        "per_kernel_ms": {n: avg[n] * 1e3 for n in names},
        "per_kernel_ms_stats": stats,
        "timing": ("HIP events on the launch stream around each kernel, median over the timed steps "
                   "(p10 / p90 and mean in per_kernel_ms_stats); " +
                   ("a 1 GiB device write flushes L2 and the MALL before every step"
                    if flush_buf is not None else "no cache flush")),
        "roofline": roofline,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "smaller_layers": small,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {COPY_PROBE_BYTES} bytes read and written")


# Kernels whose HBM traffic bench.py reports, matched on rocprofv3's kernel
# names (pattern, which matching dispatch of the one-step counter run: an
# index in dispatch order, or None for the mean of all): the W4A4 GEMM (the
# step's 4-4 GEMMs are, in order, the plain one, fc1 with its output quantized
# for fc2, and the dynamic-range one), the 4-bit fused LayerNorm-quant with
# calibrated ranges (5 units per lane at K = 9216; the step's, after the
# calibration one), the 3-bit KV pack (K and V).
PMC_KERNELS = {
    "qgemm": ("qgemm_kernel<4, 4, false", -3),
    "qgemm_quant_out": ("qgemm_kernel<4, 4, false", -2),
    "ln_reorder_quant": ("ln_reorder_quant_kernel<4, 0, 5, 0>", -1),
    "kv_quant_pack": ("kv_quant_pack_kernel<3,", None),
}
COPY_PROBE_BYTES = 1 << 30


def _pmc_per_dispatch(path, counter):
    """{dispatch id: (kernel name, counter value summed over its rows)} from a
    rocprofv3 counter-collection CSV."""
    import csv
    out = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, v = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, v + float(r["Counter_Value"]))
    return out


def ingest_pmc(fetch_csv, write_csv, out_path=None):
    """HBM bytes per launch = FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each
    scaled so that the copy probe (the last copy dispatch of the run) reads
    and writes exactly COPY_PROBE_BYTES."""
    res = {}
    scale = {}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = _pmc_per_dispatch(path, counter)
        copies = [k for k, (n, _) in d.items() if "copy" in n.lower()]
        if not copies:
            raise SystemExit(f"{path}: no copy dispatch (run bench.py with --copy-probe)")
        probe = d[max(copies)][1] * 1024.0
        scale[counter] = COPY_PROBE_BYTES / probe
        per[counter] = d
    for key, (pat, pick) in PMC_KERNELS.items():
        vals = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            v = [x for _, (n, x) in sorted(per[counter].items()) if pat in n]
            if not v:
                break
            x = float(np.mean(v)) if pick is None else v[pick]
            vals[counter] = x * 1024.0 * scale[counter]
        if len(vals) == 2:
            res[key] = {"source_hash": source_hash(KERNEL_SOURCES[key]),
                        "bytes_per_launch": vals["FETCH_SIZE"] + vals["WRITE_SIZE"],
                        "fetch_bytes": vals["FETCH_SIZE"], "write_bytes": vals["WRITE_SIZE"],
                        "scale_fetch": scale["FETCH_SIZE"], "scale_write": scale["WRITE_SIZE"],
                        "kernel_match": pat}
    path = out_path or os.path.join(ROOT, "profiles", "hbm_traffic.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1, sort_keys=True)
    print(json.dumps(res, indent=1))
    return res


FLUSH_BYTES = 1 << 30                   # > 8 x 4 MB L2 + 256 MB MALL
N_XCD, N_CU, N_SIMD = 8, 256, 1024      # MI355X


_SLEEP_CYCLES_PER_MS = []


def _gpu_sleep_ms(torch, stream, ms):
    """Keep `stream` busy for about `ms` milliseconds with a spin kernel that
    touches no memory (calibrated once against HIP events)."""
    if not _SLEEP_CYCLES_PER_MS:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(1 << 22)
        e1.record(stream)
        e1.synchronize()
        _SLEEP_CYCLES_PER_MS.append((1 << 22) / max(e0.elapsed_time(e1), 1e-3))
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS[0]))


def _time_launches(torch, stream, fn, iters, flush_buf=None):
    """HIP-event times (seconds) of `iters` launches of fn on `stream`; with
    flush_buf, a cache flush before each launch (outside the events).
    Without it the launches run back to back on warm caches: a spin kernel
    holds the stream while they are queued, so no launch waits for the host
    (short kernels would otherwise be timed together with the host's
    enqueue latency)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * iters)]
    if flush_buf is None:
        fn()
        _gpu_sleep_ms(torch, stream, 2.0 + 0.2 * iters)
    for i in range(iters):
        if flush_buf is not None:
            flush_buf.fill_(i & 0xFF)
        ev[2 * i].record(stream)
        fn()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e-3 for i in range(iters)])


def small_configs(P, torch, dev, stream, flush_buf, iters=20):
    """The OPT-125m (W8A8), OPT-1.3B fc1 (W4A4) and OPT-13B QKV (W4A4, W4A8)
    layers: fused LayerNorm-quant and segmented GEMM, each timed cold (cache
    flushed before every launch) and warm (launches back to back, inputs
    resident in the 256 MB MALL / L2).  Their LayerNorm inputs (0.2-42 MB)
    fit the MALL, so their HBM fractions are cache-assisted, not HBM rates."""
    import synthetic
    res = {}
    for name, ab in (("opt125m_w8a8", 8), ("opt1.3b_fc1_w4a4", 4), ("opt13b_qkv_w4a4", 4), ("opt13b_qkv_w4a4", 8)):
        w = synthetic.WORKLOADS[name]
        M, K, N, g, wb = w.M, w.K, w.N, w.g, w.w_bits
        mu, sg = synthetic.channel_params(K, w.seed, w.outlier_frac, range_ratio=w.range_ratio)
        gamma, beta = synthetic.ln_params(K, w.seed, random=False)
        g_d = torch.from_numpy(gamma).to(dev); b_d = torch.from_numpy(beta).to(dev)
        xc = torch.from_numpy(synthetic.tokens(w.calib_tokens, mu, sg, w.seed, synthetic.STREAM_CALIB)).to(dev)
        mx, mn = P.rptq_calib_minmax(xc, P.RPTQ_IN_FP16_RAW, g_d, b_d)
        mx, mn = mx.cpu().numpy(), mn.cpu().numpy()
        R, bounds = P.rptq_kmeans_reorder(mx, mn, g, synthetic.kmeans_uniforms(w.seed, 10, g), n_init=10)
        s, z = P.rptq_cluster_params(mx, mn, R, bounds, ab)
        R_d = torch.from_numpy(R).to(dev)
        gr, br = g_d[R_d].contiguous(), b_d[R_d].contiguous()
        x = torch.from_numpy(synthetic.tokens(M, mu, sg, w.seed, synthetic.STREAM_EVAL)).to(dev)
        wq, s_w = P.rptq_quantize_weights(synthetic.weights(K, N, w.seed), wb)
        wp, cs = P.rptq_pack_weights(wq, R, bounds, wb)
        wp, cs, sw = (torch.from_numpy(a).to(dev) for a in (wp, cs, s_w))
        codes = torch.empty((M, P.rptq_codes_row_bytes(bounds, ab)), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ln = lambda: P.rptq_ln_reorder_quant(x, R_d, gr, br, bounds, s, z, ab, out=codes, stream=stream)
        gm = lambda: P.rptq_qgemm(codes, M, K, N, bounds, s, z, ab, wp, wb, sw, cs, out=Y, stream=stream)
        for _ in range(3):
            ln(); gm()
        torch.cuda.synchronize()
        ops, ln_bytes = 2.0 * M * N * K, M * K * (2 + ab / 8)
        entry = {"M": M, "K": K, "N": N, "g": g, "a_bits": ab, "w_bits": wb, "K_pad": P.rptq_codes_kpad(bounds)}
        for mode, fb in (("cold", flush_buf), ("warm_cache_resident", None)):
            t_ln = _time_launches(torch, stream, ln, iters, fb)
            t_gm = _time_launches(torch, stream, gm, iters, fb)
            mln, mgm = float(np.median(t_ln)), float(np.median(t_gm))
            entry[mode] = {
                "ln_ms": {"median": mln * 1e3, "p10": float(np.percentile(t_ln, 10)) * 1e3,
                          "p90": float(np.percentile(t_ln, 90)) * 1e3},
                "gemm_ms": {"median": mgm * 1e3, "p10": float(np.percentile(t_gm, 10)) * 1e3,
                            "p90": float(np.percentile(t_gm, 90)) * 1e3},
                "tokens_per_s": M / (mln + mgm),
                "gemm_tops": ops / mgm / 1e12, "gemm_frac_int8_peak": ops / mgm / 1e12 / INT8_PEAK_TOPS,
                "ln_GBps": ln_bytes / mln / 1e9, "ln_frac_hbm_peak": ln_bytes / mln / 1e9 / HBM_PEAK_GBPS}
        res[f"{name}_a{ab}"] = entry
        log(f"[bench] {name} A{ab}: cold LN {entry['cold']['ln_ms']['median']:.4f} ms, GEMM "
            f"{entry['cold']['gemm_ms']['median']:.4f} ms ({entry['cold']['gemm_tops']:.0f} TOPS); warm LN "
            f"{entry['warm_cache_resident']['ln_ms']['median']:.4f} ms, GEMM "
            f"{entry['warm_cache_resident']['gemm_ms']['median']:.4f} ms")
        del x, codes, Y, wp, cs, sw
    return res


def summarize_pmc(paths):
    """Per dispatch (kernel, grid): duration, every counter summed over its
    instances, and the derived rates.  GRBM_GUI_ACTIVE is reported summed
    over the 8 XCDs, so one XCD's active cycles are a 1/8 share; MFMA busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x active cycles); the clock is active
    cycles over the dispatch's duration; LDS active = SQ_LDS_IDX_ACTIVE /
    (CUs x active cycles); MFMA ops = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512."""
    import csv
    from collections import OrderedDict, defaultdict
    rows = []
    for path in paths:
        per = OrderedDict()
        for r in csv.DictReader(open(path, newline="")):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]))
            d = per.setdefault(key, {"dur_ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                                     "vgpr": r.get("VGPR_Count"), "agpr": r.get("Accum_VGPR_Count"),
                                     "lds": r.get("LDS_Block_Size"), "c": defaultdict(float)})
            d["c"][r["Counter_Name"]] += float(r["Counter_Value"])
        for (disp, name, grid), d in per.items():
            c = d["c"]
            short = name.replace("(anonymous namespace)::", "")
            short = short[5:] if short.startswith("void ") else short
            out = {"file": os.path.basename(path), "dispatch": disp, "kernel": short.split("(")[0],
                   "grid_threads": grid, "dur_us": d["dur_ns"] / 1e3, "counters": dict(c)}
            if "GRBM_GUI_ACTIVE" in c:
                cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
                out["active_cycles_per_xcd"] = cyc
                out["clock_GHz"] = cyc / d["dur_ns"]
                if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                    out["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc)
                if "SQ_LDS_IDX_ACTIVE" in c:
                    out["lds_active_frac"] = c["SQ_LDS_IDX_ACTIVE"] / (N_CU * cyc)
            if "SQ_LDS_IDX_ACTIVE" in c and "SQ_LDS_BANK_CONFLICT" in c and c["SQ_LDS_IDX_ACTIVE"]:
                out["lds_conflict_frac_of_active"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
            if "SQ_INSTS_VALU_MFMA_MOPS_I8" in c:
                out["mfma_int8_ops"] = c["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512
            if "SQ_ACTIVE_INST_VALU" in c and "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"]:
                out["valu_active_frac_of_wave_cycles"] = c["SQ_ACTIVE_INST_VALU"] / c["SQ_WAVE_CYCLES"]
            if "GRBM_GUI_ACTIVE" in c:
                simd_cyc = N_SIMD * c["GRBM_GUI_ACTIVE"] / N_XCD
                # SQ_ACTIVE_INST_VALU counts 4-cycle issue slots of a wave64 VALU instruction
                if "SQ_ACTIVE_INST_VALU" in c:
                    out["valu_busy_frac"] = 4 * c["SQ_ACTIVE_INST_VALU"] / simd_cyc
                if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                    out["valu_mfma_coexec_frac"] = c["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cyc
                if "TA_TA_BUSY" in c:
                    out["ta_busy_frac"] = c["TA_TA_BUSY"] / (N_CU * c["GRBM_GUI_ACTIVE"] / N_XCD)
            if c.get("SQ_WAVE_CYCLES"):
                for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY"):
                    if k in c:
                        out[k.lower()[3:] + "_frac_of_wave_cycles"] = c[k] / c["SQ_WAVE_CYCLES"]
            waves = grid / 64
            for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU"):
                if k in c:
                    out[k.lower()[3:] + "_per_wave"] = c[k] / waves
            if c.get("SQ_INSTS_VMEM_RD") and "SQ_INST_LEVEL_VMEM" in c:
                # in-flight level accumulated per cycle over instructions issued: mean residence
                out["vmem_level_per_vmem_rd"] = c["SQ_INST_LEVEL_VMEM"] / c["SQ_INSTS_VMEM_RD"]
            rows.append(out)
            print(json.dumps(out))
    return rows


def cpu_baseline(w, x_dev, gamma, beta, R, bounds, s, z, N, budget_s):
    """The oracle (plain C++/OpenMP, never tuned) on a bounded row sample of
    the same layer: LayerNorm + reorder + quantize + pack, then the
    segmented integer GEMM with its epilogue.  Rows are added until about
    `budget_s` seconds of CPU work."""
    import oracle as orc
    import synthetic
    rows_x = x_dev[:4096].cpu().numpy()
    W = synthetic.weights(w.K, N, w.seed)
    Wq, s_w = orc.quantize_weights(W, w.w_bits)
    del W
    done, t_tot = 0, 0.0
    chunk = 32
    while t_tot < budget_s and done + chunk <= rows_x.shape[0]:
        xs = rows_x[done:done + chunk]
        t0 = time.perf_counter()
        codes = orc.ln_reorder_quant(xs, gamma, beta, 1e-5, R, bounds, s, z, 4)
        q = orc.unpack_seg32(codes, w.K, bounds, 4)
        orc.qgemm(q, Wq, R, bounds, s, z, s_w)
        t_tot += time.perf_counter() - t0
        done += chunk
    return {"value": done / t_tot, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"{done} of {w.M} tokens of the W4A4 layer (LN+quant+pack+segmented GEMM, N={N})",
            "seconds": t_tot}


def cpu_baseline_kv(tensors, C, bits, rows=8192):
    """The oracle's K/V quantize + pack on one 8192-token batch of K and of V
    (the first batch of each cache), in GB/s of the same algorithmic bytes
    as the GPU kernel (fp16 in + packed codes out)."""
    import oracle as orc
    t_tot, nbytes = 0.0, 0
    for name, (x_dev, R, bounds, s, z) in tensors.items():
        xs = x_dev[:rows].cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        orc.kv_quant_pack(xs, R, bounds, s, z, bits)
        t_tot += time.perf_counter() - t0
        nbytes += rows * C * (2 + bits / 8)
    return {"value": nbytes / t_tot / 1e9, "unit": "GB/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"K/V quantize + pack, one {rows}-token batch of K and of V ({C} channels, {bits} bit)",
            "seconds": t_tot}


if __name__ == "__main__":
    main()
