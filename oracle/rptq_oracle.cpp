// RPTQ oracle: a plain, slow, obviously-correct CPU implementation of what the
// reorder-based post-training quantization hot path computes.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
// CPU-baseline leg of the benchmark may load this library.  The product path
// (the HIP library and its Python binding) never calls it, and the two share no
// code, header, table or constant.
//
// Sources (cited by page title and passage, never by line):
//   [W]  RPTQ write-up "基于重排序的新量化方法RPTQ：实现大型语言模型的 3 比特量化"
//        - motivation: per-channel (max, min) points (Fig. 1 caption), the
//          two-channel example [-100,-50] vs [80,100];
//        - method: calibration max/min per channel, KMeans into g clusters on
//          the (max, min) points, reorder so a cluster is contiguous, one
//          (scale s, zero point z) per cluster; Fig. 3: reorder indices R1..R5;
//          LayerNorm emits reordered activations, linear weights are reordered;
//        - evaluation: W4A8/W4A4 and KV-cache-only settings W4A3KV etc.
//   [H]  Houmo article on RPTQ / PB-LLM, RPTQ section: 3-bit activations,
//        fusion makes the reorder nearly free.
//   [L]  quantization lecture (gitcode.csdn.net): section 1 uniform quantization
//        (scale = range / integer range, quant/dequant = multiply/divide by the
//        scale); 1.1 static calibration with clipping to the profiled range;
//        1.3 asymmetric W = S (Wq - Z) and symmetric (no Z); 1.4 granularity
//        (per tensor, per channel).
//   The GEMM identity Y = s_w * sum_c s_c (Q_c W_c - z_c colsum(W_c)) follows
//   from [L] 1.3 applied to both operands and from the fact that permuting a
//   summation index is exact ([W] method: reordered weights and LayerNorm).
//
// Numerics: fp64 for every floating-point step the pages leave open.  The only
// fp32 values are the ones the method hands on as fp32 (the normalized
// activations y, the scales s and their reciprocals).  A quantized code is
// decided as round-half-even of the EXACT product y * (1/s) (computed in fp64,
// where it is exact), then the integer zero point is added and the result
// clipped to [0, 2^b - 1].
//
// Build: g++ -O3 -march=x86-64-v3 -ffp-contract=off -fopenmp -shared -fPIC

#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include <numeric>
#include <omp.h>

extern "C" {

int orc_num_threads(void) { return omp_get_max_threads(); }

// ---------------------------------------------------------------------------
// IEEE 754 binary16 <-> binary64/binary32, written from the format definition
// (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).
// ---------------------------------------------------------------------------
double orc_half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0)       v = std::ldexp((double)f, -24);                 // zero / subnormal
    else if (e == 31) v = f ? NAN : INFINITY;
    else              v = std::ldexp((double)(1024 + f), e - 25);     // 1.f * 2^(e-15)
    return sign ? -v : v;
}

// Round-to-nearest-even conversion to binary16 of a value held exactly in a
// double (one rounding).
uint16_t orc_double_to_half(double x) {
    const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
    if (std::isnan(x)) return sign | 0x7e00;
    const double a = std::fabs(x);
    // 65504 is the largest finite half; the midpoint to the next binade step
    // (65536) is 65520, which ties to the even neighbour: infinity.
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < std::ldexp(1.0, -14)) {
        // subnormal range: integer multiples of 2^-24; 1024 * 2^-24 = 2^-14 is
        // the smallest normal and encodes to 0x0400 naturally
        const double r = std::nearbyint(a * std::ldexp(1.0, 24));
        return sign | (uint16_t)r;
    }
    int e2;
    std::frexp(a, &e2);            // a in [2^(e2-1), 2^e2)
    int E = e2 - 1;                // a in [2^E, 2^(E+1)), E in [-14, 15]
    double r = std::nearbyint(std::ldexp(a, 10 - E));   // in [1024, 2048]
    if (r == 2048.0) { r = 1024.0; E += 1; }
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024);
}

// Round-to-nearest-even conversion of a binary32 value to binary16.
uint16_t orc_float_to_half(float x) { return orc_double_to_half((double)x); }

void orc_half_to_double_array(const uint16_t* h, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_double(h[i]);
}
void orc_float_to_half_array(const float* x, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_half(x[i]);
}

// ---------------------------------------------------------------------------
// LayerNorm emitting reordered activations ([W] method, Fig. 3: LayerNorm is
// modified to produce the reordered activations directly).
//   mu   = mean_k x[k]                    (natural channel order, fp64)
//   var  = mean_k (x[k] - mu)^2           (biased)
//   y[j] = gamma[R[j]] * (x[R[j]] - mu) / sqrt(var + eps) + beta[R[j]]
// computed in fp64 and rounded once to fp32.  gamma/beta are in NATURAL order;
// R == NULL means the identity.  Output y is [M][K] in reordered order.
// ---------------------------------------------------------------------------
void orc_layernorm(const uint16_t* x, int64_t M, int32_t K,
                   const float* gamma, const float* beta, float eps,
                   const int32_t* R, float* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * (int64_t)K;
        std::vector<double> v(K);
        for (int32_t k = 0; k < K; ++k) v[k] = orc_half_to_double(row[k]);
        double sum = 0.0;
        for (int32_t k = 0; k < K; ++k) sum += v[k];
        const double mu = sum / K;
        double ss = 0.0;
        for (int32_t k = 0; k < K; ++k) ss += (v[k] - mu) * (v[k] - mu);
        const double var = ss / K;
        const double rstd = 1.0 / std::sqrt(var + (double)eps);
        float* out = y + m * (int64_t)K;
        for (int32_t j = 0; j < K; ++j) {
            const int32_t k = R ? R[j] : j;
            const double t = (double)gamma[k] * ((v[k] - mu) * rstd) + (double)beta[k];
            out[j] = (float)t;
        }
    }
}

// Per-channel (max, min) over the rows of a calibration batch ([W] motivation,
// Fig. 1: every activation channel is a (max, min) point; [W] method: the
// calibration set is run and each channel's max and min are recorded).
void orc_channel_minmax_f32(const float* v, int64_t rows, int32_t K, float* mx, float* mn) {
    for (int32_t k = 0; k < K; ++k) { mx[k] = -INFINITY; mn[k] = INFINITY; }
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < K; ++k) {
            const float t = v[r * (int64_t)K + k];
            if (t > mx[k]) mx[k] = t;
            if (t < mn[k]) mn[k] = t;
        }
}
void orc_channel_minmax_f16(const uint16_t* v, int64_t rows, int32_t K, float* mx, float* mn) {
    for (int32_t k = 0; k < K; ++k) { mx[k] = -INFINITY; mn[k] = INFINITY; }
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t k = 0; k < K; ++k) {
            const float t = (float)orc_half_to_double(v[r * (int64_t)K + k]);
            if (t > mx[k]) mx[k] = t;
            if (t < mn[k]) mn[k] = t;
        }
}

// ---------------------------------------------------------------------------
// KMeans on 2-D points ([W] method: the channels are split into g clusters by
// KMeans on the points formed by each channel's max and min).
// Seeding is k-means++ (Arthur & Vassilvitskii 2007): the first centre is the
// point at index floor(u * C); each further centre is drawn with probability
// proportional to the squared distance to the nearest chosen centre, by
// inverting the cumulative sum with a uniform u.  The uniforms are INPUTS
// (u has n_init * g entries, in [0, 1)), so the draw is reproducible.
// Lloyd iterations: assign every point to its nearest centre (squared
// Euclidean distance, ties to the lowest centre index), then move each centre
// to the mean of its points; an empty cluster is re-seeded at the point that
// is farthest from its own centre.  Stop when no label changes or after
// max_iter iterations.  The run with the lowest inertia (sum of squared
// distances) wins; ties go to the earliest run.
// Returns 0 on success.
// ---------------------------------------------------------------------------
static double sqd(const double* p, const double* q) {
    const double a = p[0] - q[0], b = p[1] - q[1];
    return a * a + b * b;
}

static void assign_all(const double* pts, int32_t C, int32_t g, const double* cen,
                       int32_t* lab) {
    for (int32_t i = 0; i < C; ++i) {
        int32_t best = 0;
        double bd = sqd(pts + 2 * i, cen);
        for (int32_t c = 1; c < g; ++c) {
            const double d = sqd(pts + 2 * i, cen + 2 * c);
            if (d < bd) { bd = d; best = c; }
        }
        lab[i] = best;
    }
}

static double inertia_of(const double* pts, int32_t C, const double* cen, const int32_t* lab) {
    double s = 0.0;
    for (int32_t i = 0; i < C; ++i) s += sqd(pts + 2 * i, cen + 2 * lab[i]);
    return s;
}

int orc_kmeans(const double* pts, int32_t C, int32_t g, const double* u,
               int32_t n_init, int32_t max_iter,
               int32_t* labels, double* centroids, double* inertia_out, int32_t* iters_out) {
    if (C < 1 || g < 1 || g > C || n_init < 1 || max_iter < 1) return -1;
    std::vector<double> cen(2 * g), best_cen(2 * g);
    std::vector<int32_t> lab(C), prev(C), best_lab(C);
    std::vector<double> d2(C);
    double best_inertia = INFINITY;
    int32_t best_iters = 0;
    for (int32_t run = 0; run < n_init; ++run) {
        const double* ur = u + (int64_t)run * g;
        // k-means++ seeding
        int32_t first = (int32_t)std::floor(ur[0] * C);
        if (first >= C) first = C - 1;
        cen[0] = pts[2 * first]; cen[1] = pts[2 * first + 1];
        for (int32_t i = 0; i < C; ++i) d2[i] = sqd(pts + 2 * i, cen.data());
        for (int32_t c = 1; c < g; ++c) {
            double total = 0.0;
            for (int32_t i = 0; i < C; ++i) total += d2[i];
            int32_t pick = C - 1;
            if (total > 0.0) {
                const double target = ur[c] * total;
                double acc = 0.0;
                for (int32_t i = 0; i < C; ++i) {
                    acc += d2[i];
                    if (acc > target) { pick = i; break; }
                }
            } else {
                // every point coincides with a chosen centre: take the first
                // point not yet used as a centre
                pick = c < C ? c : C - 1;
            }
            cen[2 * c] = pts[2 * pick]; cen[2 * c + 1] = pts[2 * pick + 1];
            for (int32_t i = 0; i < C; ++i) {
                const double d = sqd(pts + 2 * i, cen.data() + 2 * c);
                if (d < d2[i]) d2[i] = d;
            }
        }
        // Lloyd iterations
        std::fill(prev.begin(), prev.end(), -1);
        int32_t it = 0;
        for (it = 1; it <= max_iter; ++it) {
            assign_all(pts, C, g, cen.data(), lab.data());
            // new centres = means; empty clusters re-seeded at the farthest point
            std::vector<double> sx(g, 0.0), sy(g, 0.0);
            std::vector<int32_t> cnt(g, 0);
            for (int32_t i = 0; i < C; ++i) {
                sx[lab[i]] += pts[2 * i]; sy[lab[i]] += pts[2 * i + 1]; cnt[lab[i]]++;
            }
            for (int32_t c = 0; c < g; ++c) {
                if (cnt[c] > 0) { cen[2 * c] = sx[c] / cnt[c]; cen[2 * c + 1] = sy[c] / cnt[c]; }
            }
            for (int32_t c = 0; c < g; ++c) {
                if (cnt[c] > 0) continue;
                int32_t far = 0; double fd = -1.0;
                for (int32_t i = 0; i < C; ++i) {
                    const double d = sqd(pts + 2 * i, cen.data() + 2 * lab[i]);
                    if (d > fd) { fd = d; far = i; }
                }
                cnt[lab[far]]--;
                lab[far] = c; cnt[c] = 1;
                cen[2 * c] = pts[2 * far]; cen[2 * c + 1] = pts[2 * far + 1];
            }
            if (lab == prev) break;
            prev = lab;
        }
        if (it > max_iter) it = max_iter;
        // final consistent labelling for the inertia
        assign_all(pts, C, g, cen.data(), lab.data());
        const double in = inertia_of(pts, C, cen.data(), lab.data());
        if (in < best_inertia) {
            best_inertia = in; best_lab = lab; best_cen = cen; best_iters = it;
        }
    }
    std::copy(best_lab.begin(), best_lab.end(), labels);
    if (centroids) std::copy(best_cen.begin(), best_cen.end(), centroids);
    if (inertia_out) *inertia_out = best_inertia;
    if (iters_out) *iters_out = best_iters;
    return 0;
}

// ---------------------------------------------------------------------------
// Reorder index from cluster labels ([W] method: channels of one cluster are
// placed next to each other; Fig. 3: reorder indices).  Clusters are ordered
// by centroid min ascending, then centroid max ascending, then smallest member
// channel; members of a cluster keep ascending channel order.  R[j] is the
// natural channel at reordered position j; cluster c occupies positions
// [bounds[c], bounds[c+1]).  Labels must use every cluster id in [0, g).
// Returns 0 on success, -1 if a cluster is empty.
// ---------------------------------------------------------------------------
int orc_order_clusters(const int32_t* labels, const double* centroids, int32_t C, int32_t g,
                       int32_t* R, int32_t* bounds) {
    std::vector<int32_t> first(g, C), cnt(g, 0);
    for (int32_t i = 0; i < C; ++i) {
        cnt[labels[i]]++;
        if (i < first[labels[i]]) first[labels[i]] = i;
    }
    for (int32_t c = 0; c < g; ++c) if (cnt[c] == 0) return -1;
    std::vector<int32_t> order(g);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        if (centroids[2 * a + 1] != centroids[2 * b + 1]) return centroids[2 * a + 1] < centroids[2 * b + 1];
        if (centroids[2 * a] != centroids[2 * b]) return centroids[2 * a] < centroids[2 * b];
        return first[a] < first[b];
    });
    int32_t pos = 0;
    bounds[0] = 0;
    for (int32_t oc = 0; oc < g; ++oc) {
        const int32_t c = order[oc];
        for (int32_t i = 0; i < C; ++i) if (labels[i] == c) R[pos++] = i;
        bounds[oc + 1] = pos;
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Per-cluster asymmetric uniform parameters ([W] method: one scale s and zero
// point z per cluster, computed for that cluster's channels; [L] section 1:
// scale = (max - min) / (qmax - qmin); [L] 1.3: W = S (Wq - Z), Z is where the
// real 0 lands).  For cluster c with reordered channels [bounds[c], bounds[c+1]):
//   lo = min of the channel minima, hi = max of the channel maxima
//   s  = fp32((hi - lo) / qmax), floored at max(|lo|, |hi|) * 2^-21 so that the
//        zero point stays within +-2^21 (a constant cluster keeps a tiny step);
//        s = 1 if the cluster is identically zero
//   z  = round-half-even(-lo / s), NOT clipped to [0, qmax]: a cluster whose
//        range excludes 0 keeps its own range (the two-channel example).
// mx/mn are in NATURAL channel order, R maps reordered position -> channel.
// ---------------------------------------------------------------------------
int orc_cluster_params(const float* mx, const float* mn, const int32_t* R,
                       const int32_t* bounds, int32_t g, int32_t bits,
                       float* s, int32_t* z) {
    const double qmax = (double)((1 << bits) - 1);
    for (int32_t c = 0; c < g; ++c) {
        if (bounds[c + 1] <= bounds[c]) return -1;
        double lo = INFINITY, hi = -INFINITY;
        for (int32_t j = bounds[c]; j < bounds[c + 1]; ++j) {
            const int32_t k = R ? R[j] : j;
            lo = std::min(lo, (double)mn[k]);
            hi = std::max(hi, (double)mx[k]);
        }
        float sc = (float)((hi - lo) / qmax);
        const float floor_s = (float)(std::max(std::fabs(lo), std::fabs(hi)) * std::ldexp(1.0, -21));
        if (sc < floor_s) sc = floor_s;
        if (sc == 0.0f) sc = 1.0f;
        s[c] = sc;
        z[c] = (int32_t)std::nearbyint(-lo / (double)sc);
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Quantization of one value with a cluster's (s, z) ([L] section 1 and 1.3,
// [L] 1.1: static ranges, out-of-range values clipped).  inv_s = 1/s rounded
// to fp32; the product v * inv_s is formed exactly (fp64), rounded half-to-
// even to an integer, z is added, and the result clipped to [0, qmax].
// NaN maps to 0, +-inf to qmax / 0.
// ---------------------------------------------------------------------------
static inline uint8_t quant_one(double v, float inv_s, int32_t z, int32_t qmax) {
    const double p = v * (double)inv_s;        // exact: <= 24 + 24 significant bits
    if (std::isnan(p)) return 0;
    const double r = std::nearbyint(p) + (double)z;
    if (r <= 0.0) return 0;
    if (r >= (double)qmax) return (uint8_t)qmax;
    return (uint8_t)r;
}

static inline int32_t cluster_of(const int32_t* bounds, int32_t g, int32_t j) {
    int32_t c = 0;
    while (c + 1 < g && j >= bounds[c + 1]) ++c;
    return c;
}

// y: [M][K] fp32 in reordered order -> q: [M][K] one code per byte.
void orc_quantize(const float* y, int64_t M, int32_t K, const int32_t* bounds, int32_t g,
                  const float* s, const int32_t* z, int32_t bits, uint8_t* q) {
    const int32_t qmax = (1 << bits) - 1;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < K; ++j) {
            const int32_t c = cluster_of(bounds, g, j);
            const float inv_s = 1.0f / s[c];
            q[m * (int64_t)K + j] = quant_one((double)y[m * (int64_t)K + j], inv_s, z[c], qmax);
        }
}

// Dequantization of one code ([L] 1.3: W = S (Wq - Z)); q - z is an exact
// integer, the product with s is rounded to fp32.
void orc_dequantize(const uint8_t* q, int64_t M, int32_t K, const int32_t* bounds, int32_t g,
                    const float* s, const int32_t* z, float* out) {
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < K; ++j) {
            const int32_t c = cluster_of(bounds, g, j);
            out[m * (int64_t)K + j] = s[c] * (float)((int32_t)q[m * (int64_t)K + j] - z[c]);
        }
}

// ---------------------------------------------------------------------------
// Code packing.  The pages fix no bit layout; this is the library's layout.
// A row of codes is cut into groups, each group packed on its own:
//   8-bit: a group is 1 code, stored as one byte.
//   4-bit: a group is 8 codes c0..c7 in 4 bytes; byte i (i = 0..3) holds
//          c_i in its low nibble and c_(4+i) in its high nibble.
//   3-bit: a group is 32 codes c0..c31 in 12 bytes = three little-endian
//          32-bit words d0, d1, d2.  In byte i (i = 0..3) of each word:
//            d0: bits 0-2 c_i,      bits 3-5 c_(4+i),  bits 6-7 low two bits of c_(24+i)
//            d1: bits 0-2 c_(8+i),  bits 3-5 c_(12+i), bits 6-7 low two bits of c_(28+i)
//            d2: bits 0-2 c_(16+i), bits 3-5 c_(20+i), bit 6 top bit of c_(24+i),
//                                                      bit 7 top bit of c_(28+i)
// DENSE rows (K/V cache): the codes of a row in reordered order, groups back
// to back (the row length must be a multiple of the group size).
// SEG32 rows (LayerNorm output / GEMM input): cluster c is placed at padded
// position off_c = sum over earlier clusters of ceil(size/32)*32 and padded
// with code 0 up to the next multiple of 32; K_pad = off_g.
// ---------------------------------------------------------------------------
static int group_size(int32_t bits) { return bits == 8 ? 1 : bits == 4 ? 8 : 32; }

static void pack_group(const uint8_t* c, int32_t bits, uint8_t* out) {
    if (bits == 8) { out[0] = c[0]; return; }
    if (bits == 4) {
        for (int i = 0; i < 4; ++i) out[i] = (uint8_t)((c[i] & 15) | ((c[4 + i] & 15) << 4));
        return;
    }
    for (int i = 0; i < 4; ++i) {
        out[i]     = (uint8_t)((c[i] & 7)      | ((c[4 + i] & 7) << 3)  | ((c[24 + i] & 3) << 6));
        out[4 + i] = (uint8_t)((c[8 + i] & 7)  | ((c[12 + i] & 7) << 3) | ((c[28 + i] & 3) << 6));
        out[8 + i] = (uint8_t)((c[16 + i] & 7) | ((c[20 + i] & 7) << 3) |
                               (((c[24 + i] >> 2) & 1) << 6) | (((c[28 + i] >> 2) & 1) << 7));
    }
}

static void unpack_group(const uint8_t* in, int32_t bits, uint8_t* c) {
    if (bits == 8) { c[0] = in[0]; return; }
    if (bits == 4) {
        for (int i = 0; i < 4; ++i) { c[i] = in[i] & 15; c[4 + i] = in[i] >> 4; }
        return;
    }
    for (int i = 0; i < 4; ++i) {
        const uint8_t b0 = in[i], b1 = in[4 + i], b2 = in[8 + i];
        c[i] = b0 & 7;       c[4 + i] = (b0 >> 3) & 7;
        c[8 + i] = b1 & 7;   c[12 + i] = (b1 >> 3) & 7;
        c[16 + i] = b2 & 7;  c[20 + i] = (b2 >> 3) & 7;
        c[24 + i] = (uint8_t)((b0 >> 6) | (((b2 >> 6) & 1) << 2));
        c[28 + i] = (uint8_t)((b1 >> 6) | (((b2 >> 7) & 1) << 2));
    }
}

int64_t orc_dense_row_bytes(int32_t K, int32_t bits) {
    if (K % group_size(bits)) return -1;
    return (int64_t)K * bits / 8;
}

int32_t orc_seg32_kpad(const int32_t* bounds, int32_t g) {
    int32_t kp = 0;
    for (int32_t c = 0; c < g; ++c) kp += (bounds[c + 1] - bounds[c] + 31) / 32 * 32;
    return kp;
}

int64_t orc_seg32_row_bytes(const int32_t* bounds, int32_t g, int32_t bits) {
    return (int64_t)orc_seg32_kpad(bounds, g) * bits / 8;
}

// q: [M][K] codes (reordered order) -> out: [M][row_bytes]
int orc_pack_dense(const uint8_t* q, int64_t M, int32_t K, int32_t bits, uint8_t* out) {
    const int gs = group_size(bits);
    if (K % gs) return -1;
    const int64_t rb = (int64_t)K * bits / 8, gb = (int64_t)gs * bits / 8;
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < K; j += gs)
            pack_group(q + m * (int64_t)K + j, bits, out + m * rb + (j / gs) * gb);
    return 0;
}

int orc_unpack_dense(const uint8_t* in, int64_t M, int32_t K, int32_t bits, uint8_t* q) {
    const int gs = group_size(bits);
    if (K % gs) return -1;
    const int64_t rb = (int64_t)K * bits / 8, gb = (int64_t)gs * bits / 8;
    for (int64_t m = 0; m < M; ++m)
        for (int32_t j = 0; j < K; j += gs)
            unpack_group(in + m * rb + (j / gs) * gb, bits, q + m * (int64_t)K + j);
    return 0;
}

// Expands reordered codes [M][K] into the padded SEG32 code sequence
// [M][K_pad] (pad codes 0), then packs.
int orc_pack_seg32(const uint8_t* q, int64_t M, int32_t K, const int32_t* bounds, int32_t g,
                   int32_t bits, uint8_t* out) {
    const int32_t kp = orc_seg32_kpad(bounds, g);
    const int64_t rb = (int64_t)kp * bits / 8;
    std::vector<uint8_t> padded(kp);
    for (int64_t m = 0; m < M; ++m) {
        std::fill(padded.begin(), padded.end(), 0);
        int32_t off = 0;
        for (int32_t c = 0; c < g; ++c) {
            const int32_t n = bounds[c + 1] - bounds[c];
            for (int32_t i = 0; i < n; ++i) padded[off + i] = q[m * (int64_t)K + bounds[c] + i];
            off += (n + 31) / 32 * 32;
        }
        if (orc_pack_dense(padded.data(), 1, kp, bits, out + m * rb)) return -1;
    }
    return 0;
}

// Inverse of orc_pack_seg32; also returns the pad codes so tests can check
// they are 0 (pad_codes may be NULL; otherwise [M][K_pad - K]).
int orc_unpack_seg32(const uint8_t* in, int64_t M, int32_t K, const int32_t* bounds, int32_t g,
                     int32_t bits, uint8_t* q, uint8_t* pad_codes) {
    const int32_t kp = orc_seg32_kpad(bounds, g);
    const int64_t rb = (int64_t)kp * bits / 8;
    std::vector<uint8_t> padded(kp);
    for (int64_t m = 0; m < M; ++m) {
        if (orc_unpack_dense(in + m * rb, 1, kp, bits, padded.data())) return -1;
        int32_t off = 0, p = 0;
        for (int32_t c = 0; c < g; ++c) {
            const int32_t n = bounds[c + 1] - bounds[c];
            const int32_t np = (n + 31) / 32 * 32;
            for (int32_t i = 0; i < n; ++i) q[m * (int64_t)K + bounds[c] + i] = padded[off + i];
            for (int32_t i = n; i < np; ++i)
                if (pad_codes) pad_codes[m * (int64_t)(kp - K) + p++] = padded[off + i];
            off += np;
        }
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Fused oracle of the LayerNorm step of the hot path: reordered LayerNorm,
// per-cluster quantization, SEG32 packing.  Also returns the fp32 normalized
// activations (reordered) when y_out is not NULL.
// ---------------------------------------------------------------------------
int orc_ln_reorder_quant(const uint16_t* x, int64_t M, int32_t K,
                         const float* gamma, const float* beta, float eps, const int32_t* R,
                         const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                         int32_t bits, uint8_t* codes, float* y_out) {
    std::vector<float> y((size_t)M * K);
    std::vector<uint8_t> q((size_t)M * K);
    orc_layernorm(x, M, K, gamma, beta, eps, R, y.data());
    orc_quantize(y.data(), M, K, bounds, g, s, z, bits, q.data());
    if (y_out) std::copy(y.begin(), y.end(), y_out);
    return orc_pack_seg32(q.data(), M, K, bounds, g, bits, codes);
}

// ---------------------------------------------------------------------------
// Weight quantization: symmetric, one scale per output channel, round to
// nearest ([L] 1.3 symmetric: no zero point; [L] 1.4 per-channel granularity).
//   s_w[n] = max_k |W[k][n]| / (2^(wb-1) - 1)
//   Wq[k][n] = clip(round-half-even(W[k][n] / s_w[n]), -(2^(wb-1)-1), 2^(wb-1)-1)
// W is [K][N] fp32 (y = x W); a zero column gets s_w = 1.
// ---------------------------------------------------------------------------
void orc_quantize_weights(const float* W, int32_t K, int32_t N, int32_t wbits,
                          int8_t* Wq, float* s_w) {
    const int32_t qm = (1 << (wbits - 1)) - 1;
    #pragma omp parallel for schedule(static)
    for (int32_t n = 0; n < N; ++n) {
        double amax = 0.0;
        for (int32_t k = 0; k < K; ++k) amax = std::max(amax, std::fabs((double)W[(int64_t)k * N + n]));
        float sw = (float)(amax / qm);
        if (sw == 0.0f) sw = 1.0f;
        s_w[n] = sw;
        for (int32_t k = 0; k < K; ++k) {
            double r = std::nearbyint((double)W[(int64_t)k * N + n] / (double)sw);
            r = std::min(std::max(r, (double)-qm), (double)qm);
            Wq[(int64_t)k * N + n] = (int8_t)r;
        }
    }
}

// ---------------------------------------------------------------------------
// Cluster-segmented integer GEMM and its epilogue.
//   q : [M][K] activation codes in reordered order (one code per byte)
//   Wq: [K][N] quantized weights in NATURAL row order; the oracle reorders the
//       rows itself, W'[j][n] = Wq[R[j]][n] ([W] method: reordered weights).
//   acc_c[m][n] = sum over j in cluster c of q[m][j] * W'[j][n]   (int64, must fit int32)
//   colsum_c[n] = sum over j in cluster c of W'[j][n]
//   Y[m][n]     = s_w[n] * sum_c s_c * (acc_c[m][n] - z_c * colsum_c[n])   (fp64, stored fp32)
// acc (nullable) receives [g][M][N] int32.  Returns 0, or -2 when an
// accumulator does not fit int32.
// ---------------------------------------------------------------------------
int orc_qgemm(const uint8_t* q, int64_t M, int32_t K, const int8_t* Wq, const int32_t* R,
              int32_t N, const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
              const float* s_w, float* Y, int32_t* acc) {
    std::vector<int64_t> colsum((size_t)g * N, 0);
    for (int32_t c = 0; c < g; ++c)
        for (int32_t j = bounds[c]; j < bounds[c + 1]; ++j) {
            const int32_t k = R ? R[j] : j;
            for (int32_t n = 0; n < N; ++n) colsum[(size_t)c * N + n] += Wq[(int64_t)k * N + n];
        }
    int bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(|:bad)
    for (int64_t m = 0; m < M; ++m) {
        std::vector<int64_t> a(N);
        std::vector<double> yrow(N, 0.0);
        for (int32_t c = 0; c < g; ++c) {
            std::fill(a.begin(), a.end(), 0);
            for (int32_t j = bounds[c]; j < bounds[c + 1]; ++j) {
                const int64_t qv = q[m * (int64_t)K + j];
                const int32_t k = R ? R[j] : j;
                const int8_t* wr = Wq + (int64_t)k * N;
                for (int32_t n = 0; n < N; ++n) a[n] += qv * wr[n];
            }
            for (int32_t n = 0; n < N; ++n) {
                if (a[n] > INT32_MAX || a[n] < INT32_MIN) bad = 1;
                if (acc) acc[((int64_t)c * M + m) * N + n] = (int32_t)a[n];
                yrow[n] += (double)s[c] * ((double)a[n] - (double)z[c] * (double)colsum[(size_t)c * N + n]);
            }
        }
        for (int32_t n = 0; n < N; ++n) Y[m * (int64_t)N + n] = (float)((double)s_w[n] * yrow[n]);
    }
    return bad ? -2 : 0;
}

// ---------------------------------------------------------------------------
// K/V cache path ([W] evaluation: the KV-cache-only settings quantize the key
// and value caches, which dominate memory at large batch x sequence).
// kv: [T][C] fp16, natural channel order.  Codes are produced in reordered
// order (position j reads channel R[j]) and DENSE-packed.
// Dequantization writes fp16 back in natural order:
//   out[t][R[j]] = fp16_rne( s_c * (q - z_c) )
// with the product formed exactly (fp64) and rounded once, half to even.
// ---------------------------------------------------------------------------
int orc_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R,
                      const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                      int32_t bits, uint8_t* packed) {
    if (C % group_size(bits)) return -1;
    const int32_t qmax = (1 << bits) - 1;
    const int64_t rb = (int64_t)C * bits / 8;
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t t = 0; t < T; ++t) {
        std::vector<uint8_t> q(C);
        for (int32_t j = 0; j < C; ++j) {
            const int32_t c = cluster_of(bounds, g, j);
            const int32_t k = R ? R[j] : j;
            q[j] = quant_one(orc_half_to_double(kv[t * (int64_t)C + k]), 1.0f / s[c], z[c], qmax);
        }
        if (orc_pack_dense(q.data(), 1, C, bits, packed + t * rb)) bad = 1;
    }
    return bad ? -1 : 0;
}

int orc_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R,
                   const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                   int32_t bits, uint16_t* out) {
    if (C % group_size(bits)) return -1;
    const int64_t rb = (int64_t)C * bits / 8;
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t t = 0; t < T; ++t) {
        std::vector<uint8_t> q(C);
        if (orc_unpack_dense(packed + t * rb, 1, C, bits, q.data())) bad = 1;
        for (int32_t j = 0; j < C; ++j) {
            const int32_t c = cluster_of(bounds, g, j);
            const int32_t k = R ? R[j] : j;
            const double v = (double)s[c] * (double)((int32_t)q[j] - z[c]);   // exact
            out[t * (int64_t)C + k] = orc_double_to_half(v);
        }
    }
    return bad ? -1 : 0;
}

}  // extern "C"
