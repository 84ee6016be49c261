/*
 * rptq.h -- C ABI of the MI355X (gfx950) library for the runtime hot path of
 * RPTQ, reorder-based post-training quantization of LLM activations.
 *
 * Method (RPTQ write-up "基于重排序的新量化方法RPTQ：实现大型语言模型的 3 比特量化",
 * method section): activation channels are grouped by KMeans on their
 * calibration (max, min) points into g clusters; a reorder index R places the
 * channels of a cluster next to each other; every cluster has its own scale s
 * and zero point z.  Explicit runtime reordering is avoided: LayerNorm emits
 * the reordered activations directly (gamma/beta taken in R order) and the
 * rows of the next linear layer's weights are permuted by R offline (Fig. 3).
 * Quantization follows the uniform asymmetric rule of the quantization
 * lecture (gitcode.csdn.net, sections 1 and 1.3): W = S (Wq - Z), one (S, Z)
 * per cluster for activations, symmetric per-output-channel scales for weights.
 *
 * Notation.  M tokens (rows), K channels, N output features, g clusters
 * (1 <= g <= 64), b = activation bits in {3, 4, 8}, qmax = 2^b - 1.
 *   R[j]       natural channel at reordered position j (int32 [K]).
 *   bounds     int32 [g+1]; cluster c holds reordered positions
 *              [bounds[c], bounds[c+1]); bounds[0] = 0, bounds[g] = K,
 *              strictly increasing.
 *   s, z       per-cluster scale (fp32 > 0, finite) and zero point (int32,
 *              |z| <= 2^21).  Not clipped to [0, qmax]: a cluster whose range
 *              excludes 0 keeps its own range.
 *
 * Quantization of a value v in cluster c (every entry point, bit-exact):
 *   inv_s = 1.0f / s_c                (fp32, correctly rounded, host side)
 *   q     = clip( rne(v * inv_s) + z_c, 0, qmax )
 * where v * inv_s is the exact product (fused multiply-add on the device),
 * rne rounds half to even, and the clip is exact integer arithmetic.  NaN
 * inputs give an unspecified code; +-inf clip to qmax / 0.
 *
 * Code layouts (the pages fix none; these are the library's).  A row of codes
 * is cut into groups packed independently:
 *   b = 8: one byte per code.
 *   b = 4: 8 codes c0..c7 in 4 bytes; byte i (0..3) = c_i | c_(4+i) << 4.
 *   b = 3: 32 codes c0..c31 in 12 bytes = little-endian words d0, d1, d2; in
 *          byte i (0..3) of each word:
 *            d0: bits 0-2 c_i,      bits 3-5 c_(4+i),  bits 6-7 = c_(24+i) & 3
 *            d1: bits 0-2 c_(8+i),  bits 3-5 c_(12+i), bits 6-7 = c_(28+i) & 3
 *            d2: bits 0-2 c_(16+i), bits 3-5 c_(20+i), bit 6 = c_(24+i) >> 2,
 *                                                      bit 7 = c_(28+i) >> 2
 *   DENSE rows (K/V cache): the row's codes in reordered order, groups back
 *     to back; row bytes = C * b / 8.
 *   SEG32 rows (LayerNorm output, GEMM input): cluster c starts at padded
 *     position off_c = sum_{c'<c} ceil(n_c'/32)*32 (n_c = cluster size) and is
 *     padded with code 0 up to a multiple of 32; K_pad = off_g.  A row holds
 *     K_pad * b / 8 bytes of codes, and rows are laid out with a pitch of
 *     that size rounded up to a multiple of 64 bytes (rptq_codes_row_bytes),
 *     so that the GEMM's 64-byte stage segments of a row never straddle two
 *     64-byte memory sectors.  The bytes between the codes and the pitch are
 *     not written by the producers; the GEMM may read them (and the first
 *     bytes of the next row) when K ends inside one of its 128-code stages,
 *     and takes their products with zero weights, so any values there are
 *     harmless.  Packed weights use the same pitch (rptq_weights_row_bytes),
 *     and the bytes between a row's weights and its pitch must be zero (the
 *     weight packers write them so).
 *
 * Conventions for every entry point.
 *   - Pointers marked "device" are GPU memory owned by the caller (for
 *     instance torch tensors); they must stay valid until the work queued on
 *     `stream` has run.  Pointers marked "host" are read before the call
 *     returns and may be freed afterwards.  The library allocates nothing and
 *     keeps no state between calls; it is reentrant.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device entry
 *     points only enqueue work and return; they do not synchronize.
 *   - Every argument is validated on the host before any HIP call; on error
 *     nothing is launched.  M = 0 (or T = 0) is a valid no-op.
 *   - Device pointers must be 16-byte aligned (RPTQ_ERR_ALIGNMENT).
 *   - Return value: RPTQ_OK or a negative rptq_status; rptq_last_error()
 *     returns a message for the calling thread's last failure.
 */
#ifndef RPTQ_H
#define RPTQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RPTQ_OK = 0,
    RPTQ_ERR_INVALID_ARG = -1,   /* bad value, null pointer, inconsistent sizes   */
    RPTQ_ERR_UNSUPPORTED = -2,   /* valid but outside what the kernels implement  */
    RPTQ_ERR_ALIGNMENT = -3,     /* device pointer not 16-byte aligned            */
    RPTQ_ERR_HIP = -4            /* a HIP call or kernel launch failed            */
} rptq_status;

#define RPTQ_MAX_CLUSTERS 64
#define RPTQ_MAX_K 16384
#define RPTQ_MAX_GEMM_N 4194303  /* a 128-row tile of fp32 Y spans N * 512 bytes < 2^31 */
#define RPTQ_MAX_ABS_ZERO_POINT (1 << 21)

enum {
    RPTQ_IN_FP16_RAW = 0,         /* x: fp16 [M][K], natural channel order: LayerNorm, then quantize */
    RPTQ_IN_FP32_NORMALIZED = 1   /* x: fp32 [M][K], already normalized, already in R order: quantize only */
};

/* ---------------------------------------------------------------- hot path */

/*
 * Fused LayerNorm + reorder + per-cluster quantize + SEG32 pack, one pass
 * over each row (RPTQ write-up, method section and Fig. 3: LayerNorm emits
 * the reordered activations, so no explicit reorder pass exists; Houmo
 * article, RPTQ section: fused, the reorder costs almost nothing).
 *   in_mode RPTQ_IN_FP16_RAW: per row, mu = mean(x), var = mean((x-mu)^2)
 *     (biased), y[j] = gamma_r[j] * (x[R[j]] - mu) / sqrt(var + eps) + beta_r[j]
 *     computed in fp32, then quantized with cluster(j)'s (s, z).
 *   in_mode RPTQ_IN_FP32_NORMALIZED: y = x (already reordered); quantize only.
 * x        device, fp16 [M][K] (mode 0) or fp32 [M][K] (mode 1), row-major.
 * gamma_r, beta_r  device fp32 [K] in R order (gamma[R[j]]); mode 0 only.
 * eps      > 0, mode 0 only.
 * R        device int32 [K], a permutation of 0..K-1 (not checked); NULL = identity.
 *          Mode 0 only.
 * bounds, s, z   host, as above.  bits in {3, 4, 8}.
 * codes    device uint8 [M][rptq_codes_row_bytes(bounds, g, bits)], SEG32.
 * Limits: K % 8 == 0 and K <= RPTQ_MAX_K (RPTQ_ERR_UNSUPPORTED otherwise).
 */
int rptq_ln_reorder_quant(const void* x, int32_t in_mode, int64_t M, int32_t K,
                          const float* gamma_r, const float* beta_r, float eps,
                          const int32_t* R,
                          const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                          int32_t bits, uint8_t* codes, void* stream);

/*
 * Cluster-segmented integer GEMM with the zero-point correction folded into
 * the epilogue (RPTQ write-up, motivation: quantization speeds up matrix
 * multiplication and linear layers; method / Fig. 3: weights reordered so the
 * layer consumes the reordered activations).  With W' the reordered,
 * quantized weights and colsum_c[n] = sum_{j in c} W'[j][n]:
 *   acc_c[m][n] = sum_{j in c} q[m][j] * W'[j][n]          (int32, exact)
 *   Y[m][n]     = s_w[n] * sum_c s_c * (acc_c[m][n] - z_c * colsum_c[n])
 * which is the product of the dequantized activations s_c (q - z_c) and the
 * dequantized weights s_w[n] W' (quantization lecture 1.3), summed in
 * reordered order -- exact, because a permutation of the summation index
 * does not change the sum.
 * codes    device, SEG32 [M][rptq_codes_row_bytes(bounds, g, a_bits)] (the
 *          output of rptq_ln_reorder_quant); pad codes must be 0.
 * K        number of real channels (bounds[g] == K).
 * bounds, s, z   host; a_bits in {3, 4, 8}.
 * w_packed device, output of rptq_pack_weights: [N][K_pad] w_bits-bit two's
 *          complement codes, K contiguous per output feature, grouped like
 *          the activation codes (w_bits in {3, 4, 8}; 3-bit weights are
 *          the W3 settings of the write-up's evaluation, W3A3KV); pad rows
 *          are 0.
 * s_w      device fp32 [N];  colsum device int32 [g][N].
 * Y        device fp32 [M][N], row-major.
 * acc_debug device int32 [g][M][N] or NULL: receives every acc_c (validation).
 * Limits: K <= RPTQ_MAX_K (RPTQ_ERR_UNSUPPORTED), which also keeps every
 * |acc_c| within int32; 1 <= N <= RPTQ_MAX_GEMM_N (RPTQ_ERR_UNSUPPORTED
 * above); any M >= 0.
 */
int rptq_qgemm(const uint8_t* codes, int64_t M, int32_t K, int32_t N,
               const int32_t* bounds, int32_t g, const float* s, const int32_t* z, int32_t a_bits,
               const uint8_t* w_packed, int32_t w_bits, const float* s_w, const int32_t* colsum,
               float* Y, int32_t* acc_debug, void* stream);

/* Activation applied to Y before the quantized output of rptq_qgemm_quant. */
enum {
    RPTQ_ACT_NONE = 0,
    RPTQ_ACT_RELU = 1             /* max(y, 0): OPT's fc1 -> fc2 */
};

/*
 * The same GEMM, with its output quantized for the next layer in the
 * epilogue (RPTQ write-up, method and Fig. 3: the weights of a linear layer
 * are reordered so that the layer produces its activations directly in the
 * sorted (reordered) order of the layer that consumes them; this is how the
 * inputs that no LayerNorm produces -- e.g. fc2's, after fc1 and the
 * activation -- reach the next GEMM as per-cluster codes without an explicit
 * reorder).
 *   y[m][p]        = act(Y[m][p])   for the output features in the next
 *                    layer's reordered SEG32 positions p
 *   out_codes[m]   = SEG32 pack of q = clip(rne(y * (1/s_c)) + z_c, 0, qmax)
 *                    with c the next layer's cluster of p; pad codes 0
 * which is exactly rptq_ln_reorder_quant's quantization (mode 1) applied to
 * the fp32 y.
 * N_pad    the next layer's K_pad (rptq_codes_kpad(out_bounds, out_g)): the
 *          GEMM's output features are the padded positions, so w_packed,
 *          s_w and colsum come from rptq_pack_weights_out (pad features have
 *          zero weights).
 * act      RPTQ_ACT_NONE or RPTQ_ACT_RELU.
 * out_bounds, out_s, out_z, out_bits   host: the next layer's clusters (its
 *          R is folded into the weight layout); out_bits in {3, 4, 8}.
 * out_codes device [M][rptq_codes_row_bytes(out_bounds, out_g, out_bits)].
 * Y        device fp32 [M][N_pad] or NULL: also receives y (after the
 *          activation; pad columns 0), for validation.
 * Other arguments, limits and errors as rptq_qgemm.
 */
int rptq_qgemm_quant(const uint8_t* codes, int64_t M, int32_t K, int32_t N_pad,
                     const int32_t* bounds, int32_t g, const float* s, const int32_t* z, int32_t a_bits,
                     const uint8_t* w_packed, int32_t w_bits, const float* s_w, const int32_t* colsum,
                     int32_t act, const int32_t* out_bounds, int32_t out_g, const float* out_s,
                     const int32_t* out_z, int32_t out_bits, uint8_t* out_codes, float* Y, void* stream);

/*
 * Dynamic-range variant of rptq_ln_reorder_quant (quantization lecture 1.1:
 * a dynamic scheme decides the scale at run time from the current
 * activations instead of from offline profiling).  The calibrated R and
 * cluster bounds are kept; each cluster's (s, z) is computed from THIS
 * batch's values with the calibration rule of rptq_cluster_params:
 *   lo_c = min over rows m and positions j of cluster c of y[m][j]
 *   hi_c = max of the same values
 *   s_c  = fp32((hi_c - lo_c) / qmax), at least max(|lo_c|, |hi_c|) * 2^-21,
 *          1 if zero;  z_c = rne(-lo_c / s_c)
 * with y as rptq_ln_reorder_quant defines it for in_mode, and then the codes
 * are that function's codes with these (s, z) (no value is clipped beyond
 * rounding, since every value lies inside its cluster's range).
 * Three launches in stream order: a ranges pass over x (each workgroup
 * writes its own per-cluster (lo, hi) to the workspace), the (s, z) step
 * (one workgroup per cluster), the quantizing pass; x is read twice.
 * s_out    device fp32 [g]: receives s.
 * z_out    device int32 [g]: receives z.
 * workspace device, caller-owned, 16-byte aligned, at least
 *          rptq_ln_dynamic_workspace_bytes(g) bytes; its contents on entry
 *          do not matter and are undefined on return.  Calls that share a
 *          workspace must be ordered on one stream.
 * M >= 1 (ranges of no rows are undefined: RPTQ_ERR_INVALID_ARG).  Other
 * arguments, limits and errors as rptq_ln_reorder_quant, without s and z.
 * Magnitudes below about 2^-100 are outside the supported range (1/s must
 * be a finite fp32).
 */
int rptq_ln_reorder_quant_dynamic(const void* x, int32_t in_mode, int64_t M, int32_t K,
                                  const float* gamma_r, const float* beta_r, float eps,
                                  const int32_t* R, const int32_t* bounds, int32_t g, int32_t bits,
                                  uint8_t* codes, float* s_out, int32_t* z_out, void* workspace,
                                  int64_t workspace_bytes, void* stream);

/* Workspace of rptq_ln_reorder_quant_dynamic for g clusters (1024 * 2 * g
 * floats); -1 if g is outside [1, RPTQ_MAX_CLUSTERS]. */
int64_t rptq_ln_dynamic_workspace_bytes(int32_t g);

/*
 * rptq_ln_reorder_quant_dynamic without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the ranges pass's
 * per-workgroup (lo, hi) partials go to a library-owned device array of
 * RPTQ_LN_DYNAMIC_SCRATCH_BYTES (512 KB, room for RPTQ_MAX_CLUSTERS
 * clusters), of which each GPU the library runs on holds its own copy until
 * the process ends; its device address is looked up once per device, on the
 * first call with that device current.  Every slot the quantizing launches
 * read is written earlier in the same call, so nothing needs clearing, and a
 * call leaves its partials behind.  All calls on one GPU share that GPU's
 * array: calls that may overlap on one GPU (several streams, several host
 * threads) race and must be serialized by the caller.
 * Arguments, results, limits and errors are those of
 * rptq_ln_reorder_quant_dynamic without workspace / workspace_bytes; a g
 * whose partials would not fit the array is RPTQ_ERR_UNSUPPORTED (no legal
 * g does), a failed address lookup RPTQ_ERR_HIP.
 */
#define RPTQ_LN_DYNAMIC_SCRATCH_BYTES (1024 * 2 * RPTQ_MAX_CLUSTERS * 4)
int rptq_ln_reorder_quant_dynamic_noalloc(const void* x, int32_t in_mode, int64_t M, int32_t K,
                                          const float* gamma_r, const float* beta_r, float eps,
                                          const int32_t* R, const int32_t* bounds, int32_t g, int32_t bits,
                                          uint8_t* codes, float* s_out, int32_t* z_out, void* stream);

/*
 * rptq_qgemm with the activation clusters' (s, z) in DEVICE memory (s_dev
 * fp32 [g], z_dev int32 [g], e.g. the outputs of
 * rptq_ln_reorder_quant_dynamic), so no host round trip sits between the
 * dynamic ranges and the GEMM.  The result is rptq_qgemm's for the same
 * values of (s, z), bit for bit.  No acc_debug output.  Other arguments,
 * limits and errors as rptq_qgemm.
 */
int rptq_qgemm_dynamic(const uint8_t* codes, int64_t M, int32_t K, int32_t N,
                       const int32_t* bounds, int32_t g, const float* s_dev, const int32_t* z_dev,
                       int32_t a_bits, const uint8_t* w_packed, int32_t w_bits, const float* s_w,
                       const int32_t* colsum, float* Y, void* stream);

/*
 * K/V-cache quantize + pack (RPTQ write-up, evaluation: the KV-cache settings
 * W4A4KV / W4A3KV / W3A3KV quantize the key and value caches, which hold most
 * of the memory at large batch x sequence length).  Streaming, one pass.
 *   packed row t = DENSE pack of q[t][j] = quant(kv[t][R[j]], cluster(j))
 * kv       device fp16 [T][C], natural channel order (channel = head*head_dim + d).
 * R        device int32 [C] or NULL (identity: the cache is already in R order).
 * bounds, s, z host; bits in {3, 4, 8}.
 * packed   device uint8 [T][C*bits/8].
 * Limits: C % 8 == 0, C <= RPTQ_MAX_K, and C % 32 == 0 when bits == 3.
 */
int rptq_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R,
                       const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                       int32_t bits, uint8_t* packed, void* stream);

/*
 * K/V-cache dequantize, back to natural channel order (quantization lecture
 * 1.3: W = S (Wq - Z)):
 *   out[t][R[j]] = fp16_rne( s_c * (q[t][j] - z_c) )
 * the product taken exactly and rounded once to fp16, half to even.
 * packed   device uint8 [T][C*bits/8] (DENSE, from rptq_kv_quant_pack).
 * out      device fp16 [T][C].  Other arguments and limits as rptq_kv_quant_pack.
 */
int rptq_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R,
                    const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                    int32_t bits, uint16_t* out, void* stream);

/*
 * Decode attention that reads the packed caches directly (RPTQ write-up,
 * evaluation: the KV-cache settings keep keys and values quantized; this is
 * where they are read back).  One query token per sequence b:
 *   K, V        = the caches rptq_kv_dequant would produce from k_packed,
 *                 v_packed (fp16 values fp16_rne(s_c (q - z_c)), natural
 *                 channel order), rows b*T .. b*T + T - 1 of sequence b
 *   score[h][t] = scale * sum_d q[b][h*head_dim + d] * K[b*T + t][h*head_dim + d]
 *   out[b][h*head_dim + d] = sum_t softmax_t(score[h])[t] * V[b*T + t][h*head_dim + d]
 * without materializing K or V: every packed row is dequantized into on-chip
 * memory and consumed there.
 * q        device fp16 [B][C], natural order;  out device fp32 [B][C].
 * k_packed, v_packed  device [B*T][rptq_kv_row_bytes(C, bits)] (outputs of
 *          rptq_kv_quant_pack), each with its own R (device [C] or NULL),
 *          bounds, s, z (host), as given to rptq_kv_quant_pack.
 * head_dim 64 or 128 (RPTQ_ERR_UNSUPPORTED otherwise); C a multiple of 128,
 *          at most 10240 (OPT-66B: 9216); T >= 1; bits in {3, 4, 8}; scale > 0 (usually
 *          1/sqrt(head_dim)).
 * workspace device, >= rptq_kv_attention_workspace_bytes(B, T, C, head_dim)
 *          bytes, 16-byte aligned, owned by the caller (per-chunk partial
 *          outputs and softmax statistics; contents need not be initialized).
 * B = 0 is a no-op.  Errors as rptq_kv_quant_pack.
 */
int rptq_kv_attention(const uint16_t* q, const uint8_t* k_packed, const uint8_t* v_packed,
                      int32_t B, int32_t T, int32_t C, int32_t head_dim, float scale,
                      const int32_t* R_k, const int32_t* bounds_k, int32_t g_k, const float* s_k, const int32_t* z_k,
                      const int32_t* R_v, const int32_t* bounds_v, int32_t g_v, const float* s_v, const int32_t* z_v,
                      int32_t bits, float* out, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes rptq_kv_attention needs; -1 on invalid sizes. */
int64_t rptq_kv_attention_workspace_bytes(int32_t B, int32_t T, int32_t C, int32_t head_dim);

/* ---------------------------------------------------------- calibration
 * Offline steps that produce R, bounds, s, z (RPTQ write-up, method section:
 * run calibration data, record each channel's max and min, KMeans on the
 * (max, min) points into g clusters, reorder, per-cluster parameters).
 */

/*
 * Per-channel max and min over M calibration rows, in NATURAL channel order.
 *   mode RPTQ_IN_FP16_RAW (0): statistics of LayerNorm(x; gamma, beta, eps)
 *        (gamma, beta device fp32 [K], natural order), computed like the
 *        fused kernel computes it;
 *   mode 2 (raw): statistics of x itself (K/V cache); gamma, beta ignored.
 * x device fp16 [M][K]; mx, mn device fp32 [K] (overwritten).
 * Limits: K % 8 == 0, K <= RPTQ_MAX_K, M >= 1.
 */
#define RPTQ_CALIB_RAW 2
int rptq_calib_minmax(const uint16_t* x, int32_t mode, int64_t M, int32_t K,
                      const float* gamma, const float* beta, float eps,
                      float* mx, float* mn, void* stream);

/*
 * KMeans over the points (mx[k], mn[k]) and the reorder index (host only).
 * Seeding is k-means++ driven by the caller's uniforms init_u (host double
 * [n_init * g], each in [0, 1)): the first centre is point floor(u * K), the
 * next ones are drawn with probability proportional to the squared distance
 * to the nearest chosen centre.  Lloyd iterations (nearest centre, ties to the
 * lowest index; centre = mean; an empty cluster is re-seeded at the point
 * farthest from its centre) stop when no label changes or after max_iter.
 * The run with the lowest inertia wins (ties: earliest).  Clusters are then
 * ordered by centroid min, then centroid max, then lowest channel; channels
 * inside a cluster keep ascending order.
 * mx, mn host fp32 [K]; R host int32 [K]; bounds host int32 [g+1].
 */
int rptq_kmeans_reorder(const float* mx, const float* mn, int32_t K, int32_t g,
                        const double* init_u, int32_t n_init, int32_t max_iter,
                        int32_t* R, int32_t* bounds);

/*
 * Per-cluster (s, z) from the channel ranges (host only).  lo = min of the
 * cluster's channel minima, hi = max of its maxima (fp32 inputs, fp64 math):
 *   s = fp32((hi - lo) / qmax), at least max(|lo|, |hi|) * 2^-21, 1 if zero
 *   z = rne(-lo / s)
 * mx, mn host fp32 [K] natural order; R host int32 [K] or NULL; bounds host.
 */
int rptq_cluster_params(const float* mx, const float* mn, const int32_t* R,
                        const int32_t* bounds, int32_t g, int32_t bits,
                        float* s, int32_t* z);

/*
 * Symmetric per-output-channel round-to-nearest weight quantization (host):
 *   s_w[n] = max_k |W[k][n]| / (2^(wb-1) - 1)   (1 for an all-zero column)
 *   wq[k][n] = clip(rne(W[k][n] / s_w[n]), -(2^(wb-1)-1), 2^(wb-1)-1)
 * W host fp32 [K][N]; wq host int8 [K][N]; s_w host fp32 [N]; w_bits in
 * {3, 4, 8} (3 bit: codes in [-3, 3]).
 */
int rptq_quantize_weights(const float* W, int32_t K, int32_t N, int32_t w_bits,
                          int8_t* wq, float* s_w);

/*
 * Reorder, pad and pack quantized weights for rptq_qgemm (host):
 *   W'[j][n] = wq[R[j]][n];  w_packed row n = the SEG32-padded sequence
 *   W'[.][n] (pad entries 0) in w_bits-bit two's complement, grouped like the
 *   activation codes; colsum[c][n] = sum_{j in c} W'[j][n].
 * wq host int8 [K][N] natural rows, values in [-(2^(wb-1)-1), 2^(wb-1)-1];
 * R host int32 [K] or NULL; bounds host;
 * w_packed host uint8 [N][rptq_weights_row_bytes(bounds, g, w_bits)];
 * colsum host int32 [g][N].
 */
int rptq_pack_weights(const int8_t* wq, int32_t K, int32_t N, int32_t w_bits,
                      const int32_t* R, const int32_t* bounds, int32_t g,
                      uint8_t* w_packed, int32_t* colsum);

/*
 * rptq_pack_weights for a layer whose output feeds rptq_qgemm_quant (host):
 * the output features are put in the next layer's reordered order R_out and
 * SEG32-padded by out_bounds (pad features: zero weights, colsum 0, s_w 1),
 * so that output feature p of the packed layer is the next layer's padded
 * position p.
 * s_w host fp32 [N] natural order (from rptq_quantize_weights);
 * w_packed host uint8 [N_pad][rptq_weights_row_bytes(bounds, g, w_bits)];
 * colsum host int32 [g][N_pad]; s_w_out host fp32 [N_pad];
 * N_pad = rptq_codes_kpad(out_bounds, out_g); R_out host int32 [N] or NULL.
 */
int rptq_pack_weights_out(const int8_t* wq, int32_t K, int32_t N, int32_t w_bits,
                          const int32_t* R, const int32_t* bounds, int32_t g,
                          const int32_t* R_out, const int32_t* out_bounds, int32_t out_g,
                          const float* s_w, uint8_t* w_packed, int32_t* colsum, float* s_w_out);

/* ---------------------------------------------------------- sizes, errors */

/* K_pad of the SEG32 layout; -1 on invalid bounds. */
int32_t rptq_codes_kpad(const int32_t* bounds, int32_t g);
/* SEG32 row pitch in bytes for activation codes (K_pad * bits / 8 rounded up
   to a multiple of 64); -1 on invalid input. */
int64_t rptq_codes_row_bytes(const int32_t* bounds, int32_t g, int32_t bits);
/* Row pitch of w_packed in bytes (K_pad * w_bits / 8 rounded up to a multiple
   of 64); -1 on invalid input. */
int64_t rptq_weights_row_bytes(const int32_t* bounds, int32_t g, int32_t w_bits);
/* DENSE K/V row stride in bytes (C * bits / 8); -1 on invalid input. */
int64_t rptq_kv_row_bytes(int32_t C, int32_t bits);

const char* rptq_status_string(int status);
/* Message describing the calling thread's most recent failure ("" if none). */
const char* rptq_last_error(void);
/* Library version string. */
const char* rptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RPTQ_H */
