// Host side of the C ABI declared in include/rptq.h: argument validation
// (before any HIP call), the per-call cluster tables handed to the kernels by
// value, and the offline host helpers (KMeans reorder, cluster parameters,
// weight quantization and packing).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "../../include/rptq.h"
#include "rptq_internal.h"

using namespace rptq;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return RPTQ_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool valid_bits(int32_t b) { return b == 3 || b == 4 || b == 8; }

// weight bits: 3 and 4 (packed) or 8
bool valid_wbits(int32_t b) { return b == 3 || b == 4 || b == 8; }

// bounds: host int32[g+1], 1 <= g <= min(K, 64), 0 = b0 < b1 < ... < bg = K.
int check_bounds(const int32_t* bounds, int32_t g, int32_t K) {
    if (!bounds) return fail(RPTQ_ERR_INVALID_ARG, "bounds is NULL");
    if (g < 1 || g > kMaxClusters) return fail(RPTQ_ERR_INVALID_ARG, "g = %d outside [1, %d]", g, kMaxClusters);
    if (K >= 0 && g > K) return fail(RPTQ_ERR_INVALID_ARG, "g = %d exceeds K = %d", g, K);
    if (bounds[0] != 0) return fail(RPTQ_ERR_INVALID_ARG, "bounds[0] = %d, must be 0", bounds[0]);
    for (int c = 0; c < g; ++c)
        if (bounds[c + 1] <= bounds[c])
            return fail(RPTQ_ERR_INVALID_ARG, "bounds not strictly increasing at cluster %d", c);
    if (K >= 0 && bounds[g] != K) return fail(RPTQ_ERR_INVALID_ARG, "bounds[g] = %d, must equal K = %d", bounds[g], K);
    return RPTQ_OK;
}

int check_params(const float* s, const int32_t* z, int32_t g) {
    if (!s || !z) return fail(RPTQ_ERR_INVALID_ARG, "s or z is NULL");
    for (int c = 0; c < g; ++c) {
        if (!std::isfinite(s[c]) || !(s[c] > 0.0f))
            return fail(RPTQ_ERR_INVALID_ARG, "s[%d] = %g must be finite and > 0", c, (double)s[c]);
        if (z[c] > RPTQ_MAX_ABS_ZERO_POINT || z[c] < -RPTQ_MAX_ABS_ZERO_POINT)
            return fail(RPTQ_ERR_INVALID_ARG, "|z[%d]| = %d exceeds 2^21", c, z[c]);
        const float inv = 1.0f / s[c];
        if (!std::isfinite(inv) || inv == 0.0f)
            return fail(RPTQ_ERR_INVALID_ARG, "1/s[%d] is not a finite non-zero fp32", c);
    }
    return RPTQ_OK;
}

int32_t kpad_of(const int32_t* bounds, int32_t g) {
    int32_t kp = 0;
    for (int c = 0; c < g; ++c) kp += (bounds[c + 1] - bounds[c] + 31) / 32 * 32;
    return kp;
}

ClusterArgs make_cluster_args(const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                              int32_t bits, bool seg32) {
    ClusterArgs ca;
    std::memset(&ca, 0, sizeof ca);
    ca.g = g;
    ca.K = bounds[g];
    ca.bits = bits;
    int32_t off = 0;
    for (int c = 0; c <= g; ++c) {
        ca.bounds[c] = bounds[c];
        ca.off[c] = off;
        if (c < g) off += (bounds[c + 1] - bounds[c] + 31) / 32 * 32;
    }
    ca.K_pad = seg32 ? off : 0;
    for (int c = 0; c < g; ++c) {
        ca.s[c] = s[c];
        ca.inv_s[c] = 1.0f / s[c];
        ca.z[c] = z[c];
    }
    return ca;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RPTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    e = hipGetLastError();
    if (e != hipSuccess) return fail(RPTQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace rptq {

int persistent_grid(const void* kernel, int block, size_t lds_bytes, int64_t rows) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, lds_bytes) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    int64_t grid = (int64_t)cus * per_cu;
    if (grid > rows) grid = rows;
    return (int)std::max<int64_t>(grid, 1);
}

}  // namespace rptq

extern "C" {

const char* rptq_version(void) { return "rptq-mi355x 0.1 (gfx950)"; }

const char* rptq_status_string(int status) {
    switch (status) {
        case RPTQ_OK: return "ok";
        case RPTQ_ERR_INVALID_ARG: return "invalid argument";
        case RPTQ_ERR_UNSUPPORTED: return "unsupported";
        case RPTQ_ERR_ALIGNMENT: return "misaligned pointer";
        case RPTQ_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* rptq_last_error(void) { return g_last_error.c_str(); }

int32_t rptq_codes_kpad(const int32_t* bounds, int32_t g) {
    if (check_bounds(bounds, g, -1) != RPTQ_OK) return -1;
    return kpad_of(bounds, g);
}

// Row pitch of SEG32 codes and packed weights: the K_pad * bits / 8 bytes of
// a row, padded to a multiple of 64 bytes so that the GEMM's 64-byte stage
// segments of a row never straddle two 64-byte sectors.
static int64_t seg32_pitch(int32_t kpad, int32_t bits) { return ((int64_t)kpad * bits / 8 + 63) / 64 * 64; }

int64_t rptq_codes_row_bytes(const int32_t* bounds, int32_t g, int32_t bits) {
    if (!valid_bits(bits) || check_bounds(bounds, g, -1) != RPTQ_OK) return -1;
    return seg32_pitch(kpad_of(bounds, g), bits);
}

int64_t rptq_weights_row_bytes(const int32_t* bounds, int32_t g, int32_t w_bits) {
    if (!valid_wbits(w_bits) || check_bounds(bounds, g, -1) != RPTQ_OK) return -1;
    return seg32_pitch(kpad_of(bounds, g), w_bits);
}

int64_t rptq_kv_row_bytes(int32_t C, int32_t bits) {
    if (!valid_bits(bits) || C < 1 || C % 8 || (bits == 3 && C % 32)) return -1;
    return (int64_t)C * bits / 8;
}

// ------------------------------------------------------------------ hot path
int rptq_ln_reorder_quant(const void* x, int32_t in_mode, int64_t M, int32_t K,
                          const float* gamma_r, const float* beta_r, float eps,
                          const int32_t* R, const int32_t* bounds, int32_t g, const float* s,
                          const int32_t* z, int32_t bits, uint8_t* codes, void* stream) {
    if (in_mode != RPTQ_IN_FP16_RAW && in_mode != RPTQ_IN_FP32_NORMALIZED)
        return fail(RPTQ_ERR_INVALID_ARG, "in_mode = %d", in_mode);
    if (M < 0) return fail(RPTQ_ERR_INVALID_ARG, "M = %lld < 0", (long long)M);
    if (K < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d < 1", K);
    if (!valid_bits(bits)) return fail(RPTQ_ERR_INVALID_ARG, "bits = %d not in {3, 4, 8}", bits);
    int st = check_bounds(bounds, g, K);
    if (st) return st;
    if ((st = check_params(s, z, g))) return st;
    if (in_mode == RPTQ_IN_FP16_RAW) {
        if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(RPTQ_ERR_INVALID_ARG, "eps must be finite and > 0");
        if (!gamma_r || !beta_r) return fail(RPTQ_ERR_INVALID_ARG, "gamma_r / beta_r is NULL");
    }
    if (K % 8) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d is not a multiple of 8", K);
    if (K > kMaxK) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d exceeds %d", K, kMaxK);
    if (M == 0) return ok();
    if (!x || !codes) return fail(RPTQ_ERR_INVALID_ARG, "x or codes is NULL");
    if (!aligned16(x) || !aligned16(codes) ||
        (in_mode == RPTQ_IN_FP16_RAW && (!aligned16(gamma_r) || !aligned16(beta_r) || (R && !aligned16(R)))))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const ClusterArgs ca = make_cluster_args(bounds, g, s, z, bits, true);
    const int64_t row_bytes = seg32_pitch(ca.K_pad, bits);
    return hip_status(launch_ln_reorder_quant(x, in_mode, M, K, gamma_r, beta_r, eps,
                                              in_mode == RPTQ_IN_FP16_RAW ? R : nullptr, ca, row_bytes,
                                              codes, (hipStream_t)stream),
                      "rptq_ln_reorder_quant launch");
}

}  // extern "C"

// Shared by the two dynamic-range entry points: validation, the cluster
// table, the three launches with the partials in `partials`.
static int ln_dynamic_common(const void* x, int32_t in_mode, int64_t M, int32_t K, const float* gamma_r,
                             const float* beta_r, float eps, const int32_t* R, const int32_t* bounds, int32_t g,
                             int32_t bits, uint8_t* codes, float* s_out, int32_t* z_out, void* workspace,
                             int64_t workspace_bytes, bool own_scratch, void* stream, const char* what) {
    if (in_mode != RPTQ_IN_FP16_RAW && in_mode != RPTQ_IN_FP32_NORMALIZED)
        return fail(RPTQ_ERR_INVALID_ARG, "in_mode = %d", in_mode);
    if (M < 1) return fail(RPTQ_ERR_INVALID_ARG, "M = %lld < 1: dynamic ranges need rows", (long long)M);
    if (K < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d < 1", K);
    if (!valid_bits(bits)) return fail(RPTQ_ERR_INVALID_ARG, "bits = %d not in {3, 4, 8}", bits);
    int st = check_bounds(bounds, g, K);
    if (st) return st;
    if (in_mode == RPTQ_IN_FP16_RAW) {
        if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(RPTQ_ERR_INVALID_ARG, "eps must be finite and > 0");
        if (!gamma_r || !beta_r) return fail(RPTQ_ERR_INVALID_ARG, "gamma_r / beta_r is NULL");
    }
    if (K % 8) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d is not a multiple of 8", K);
    if (K > kMaxK) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d exceeds %d", K, kMaxK);
    if (!x || !codes || !s_out || !z_out || (!own_scratch && !workspace))
        return fail(RPTQ_ERR_INVALID_ARG, "x, codes, s_out, z_out or workspace is NULL");
    const int64_t need = rptq_ln_dynamic_workspace_bytes(g);
    if (own_scratch) {
        if (need > ln_dynamic_scratch_bytes())
            return fail(RPTQ_ERR_UNSUPPORTED, "g = %d needs %lld bytes of partials, more than the library's "
                        "%lld-byte array", g, (long long)need, (long long)ln_dynamic_scratch_bytes());
    } else if (workspace_bytes < need) {
        return fail(RPTQ_ERR_INVALID_ARG, "workspace_bytes = %lld < %lld", (long long)workspace_bytes,
                    (long long)need);
    }
    if (!aligned16(x) || !aligned16(codes) || !aligned16(s_out) || !aligned16(z_out) ||
        (!own_scratch && !aligned16(workspace)) ||
        (in_mode == RPTQ_IN_FP16_RAW && (!aligned16(gamma_r) || !aligned16(beta_r) || (R && !aligned16(R)))))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    if (own_scratch) {
        const hipError_t e = ln_dynamic_scratch(&workspace);
        if (e != hipSuccess) return hip_status(e, "device address of the library's partials array");
    }
    // the cluster table's own (s, z) are unused: placeholders
    float s1[kMaxClusters];
    int32_t z0[kMaxClusters];
    for (int c = 0; c < g; ++c) { s1[c] = 1.0f; z0[c] = 0; }
    const ClusterArgs ca = make_cluster_args(bounds, g, s1, z0, bits, true);
    const int64_t row_bytes = seg32_pitch(ca.K_pad, bits);
    return hip_status(launch_ln_reorder_quant_dynamic(x, in_mode, M, K, gamma_r, beta_r, eps,
                                                      in_mode == RPTQ_IN_FP16_RAW ? R : nullptr, ca, row_bytes,
                                                      codes, s_out, z_out, static_cast<float*>(workspace),
                                                      (hipStream_t)stream),
                      what);
}

extern "C" {

int rptq_ln_reorder_quant_dynamic(const void* x, int32_t in_mode, int64_t M, int32_t K,
                                  const float* gamma_r, const float* beta_r, float eps,
                                  const int32_t* R, const int32_t* bounds, int32_t g, int32_t bits,
                                  uint8_t* codes, float* s_out, int32_t* z_out, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    return ln_dynamic_common(x, in_mode, M, K, gamma_r, beta_r, eps, R, bounds, g, bits, codes, s_out, z_out,
                             workspace, workspace_bytes, false, stream, "rptq_ln_reorder_quant_dynamic launch");
}

int rptq_ln_reorder_quant_dynamic_noalloc(const void* x, int32_t in_mode, int64_t M, int32_t K,
                                          const float* gamma_r, const float* beta_r, float eps,
                                          const int32_t* R, const int32_t* bounds, int32_t g, int32_t bits,
                                          uint8_t* codes, float* s_out, int32_t* z_out, void* stream) {
    return ln_dynamic_common(x, in_mode, M, K, gamma_r, beta_r, eps, R, bounds, g, bits, codes, s_out, z_out,
                             nullptr, 0, true, stream, "rptq_ln_reorder_quant_dynamic_noalloc launch");
}

int64_t rptq_ln_dynamic_workspace_bytes(int32_t g) {
    if (g < 1 || g > kMaxClusters) return -1;
    return (int64_t)kLnRangesMaxGrid * 2 * g * (int64_t)sizeof(float);
}

// Shared by rptq_qgemm, rptq_qgemm_dynamic and rptq_qgemm_quant: validation of the GEMM proper,
// the per-cluster tables, the launch.
static int qgemm_common(const uint8_t* codes, int64_t M, int32_t K, int32_t N, const int32_t* bounds,
                        int32_t g, const float* s, const int32_t* z, int32_t a_bits, const uint8_t* w_packed,
                        int32_t w_bits, const float* s_w, const int32_t* colsum, float* Y, int32_t* acc_debug,
                        const QuantOutArgs& qo, const ClusterArgs& qc, void* stream, const char* what,
                        bool dev_params = false) {
    if (M < 0) return fail(RPTQ_ERR_INVALID_ARG, "M = %lld < 0", (long long)M);
    if (K < 1 || N < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d, N = %d must be >= 1", K, N);
    if (!valid_bits(a_bits)) return fail(RPTQ_ERR_INVALID_ARG, "a_bits = %d not in {3, 4, 8}", a_bits);
    if (!valid_wbits(w_bits)) return fail(RPTQ_ERR_INVALID_ARG, "w_bits = %d not in {3, 4, 8}", w_bits);
    int st = check_bounds(bounds, g, K);
    if (st) return st;
    if (dev_params) {
        if (!s || !z) return fail(RPTQ_ERR_INVALID_ARG, "s or z is NULL");
        if (!aligned16(s) || !aligned16(z)) return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    } else if ((st = check_params(s, z, g))) {
        return st;
    }
    if (K > kMaxK) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d exceeds %d", K, kMaxK);
    static_assert(kMaxGemmN == RPTQ_MAX_GEMM_N, "header limit");
    if (N > kMaxGemmN) return fail(RPTQ_ERR_UNSUPPORTED, "N = %d exceeds %d", N, kMaxGemmN);
    if (M == 0) return ok();
    if (!codes || !w_packed || !s_w || !colsum || (!Y && !qo.q_codes))
        return fail(RPTQ_ERR_INVALID_ARG, "codes, w_packed, s_w, colsum and the output must be non-NULL");
    if (!aligned16(codes) || !aligned16(w_packed) || !aligned16(s_w) || !aligned16(colsum) ||
        (Y && !aligned16(Y)) || (acc_debug && !aligned16(acc_debug)) || (qo.q_codes && !aligned16(qo.q_codes)))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    GemmArgs ga;
    std::memset(&ga, 0, sizeof ga);
    ga.g = g;
    ga.code_offset = a_bits == 8 ? 128 : 0;
    int32_t steps = 0;
    for (int c = 0; c < g; ++c) {
        steps += (bounds[c + 1] - bounds[c] + 31) / 32;
        ga.step_end[c] = steps;
    }
    if (dev_params) {
        // the kernel forms the tables below from the device (s, z)
        ga.dev_s = s;
        ga.dev_z = z;
    } else {
        for (int c = 0; c < g; ++c) ga.sz[c] = (double)s[c] * ((double)z[c] - (double)ga.code_offset);
        // flush weights of the running accumulator: d_c = s_c - s_(c+1), s_(g+1) = 0
        // (4-bit weights are staged as 16 * w and 3-bit weights as 32 * w, hence
        // the 1/16 and 1/32)
        for (int c = 0; c < g; ++c) {
            const double d = (double)s[c] - (c + 1 < g ? (double)s[c + 1] : 0.0);
            ga.scale[c] = (float)(w_bits == 4 ? d * 0.0625 : w_bits == 3 ? d * 0.03125 : d);
        }
    }
    ga.nsteps = steps;
    const int64_t a_row_bytes = seg32_pitch(steps * 32, a_bits);
    const int64_t w_row_bytes = seg32_pitch(steps * 32, w_bits);
    return hip_status(launch_qgemm(codes, M, N, a_row_bytes, a_bits, w_packed, w_row_bytes, w_bits, ga, s_w,
                                   colsum, Y, acc_debug, qo, qc, (hipStream_t)stream),
                      what);
}

int rptq_qgemm(const uint8_t* codes, int64_t M, int32_t K, int32_t N, const int32_t* bounds, int32_t g,
               const float* s, const int32_t* z, int32_t a_bits, const uint8_t* w_packed, int32_t w_bits,
               const float* s_w, const int32_t* colsum, float* Y, int32_t* acc_debug, void* stream) {
    if (M > 0 && !Y) return fail(RPTQ_ERR_INVALID_ARG, "Y must be non-NULL");
    QuantOutArgs qo{nullptr, 0, 0};
    ClusterArgs qc;
    std::memset(&qc, 0, sizeof qc);
    return qgemm_common(codes, M, K, N, bounds, g, s, z, a_bits, w_packed, w_bits, s_w, colsum, Y, acc_debug,
                        qo, qc, stream, "rptq_qgemm launch");
}

int rptq_qgemm_dynamic(const uint8_t* codes, int64_t M, int32_t K, int32_t N, const int32_t* bounds,
                       int32_t g, const float* s_dev, const int32_t* z_dev, int32_t a_bits,
                       const uint8_t* w_packed, int32_t w_bits, const float* s_w, const int32_t* colsum,
                       float* Y, void* stream) {
    if (M > 0 && !Y) return fail(RPTQ_ERR_INVALID_ARG, "Y must be non-NULL");
    QuantOutArgs qo{nullptr, 0, 0};
    ClusterArgs qc;
    std::memset(&qc, 0, sizeof qc);
    return qgemm_common(codes, M, K, N, bounds, g, s_dev, z_dev, a_bits, w_packed, w_bits, s_w, colsum, Y,
                        nullptr, qo, qc, stream, "rptq_qgemm_dynamic launch", true);
}

int rptq_qgemm_quant(const uint8_t* codes, int64_t M, int32_t K, int32_t N_pad, const int32_t* bounds,
                     int32_t g, const float* s, const int32_t* z, int32_t a_bits, const uint8_t* w_packed,
                     int32_t w_bits, const float* s_w, const int32_t* colsum, int32_t act,
                     const int32_t* out_bounds, int32_t out_g, const float* out_s, const int32_t* out_z,
                     int32_t out_bits, uint8_t* out_codes, float* Y, void* stream) {
    if (act != RPTQ_ACT_NONE && act != RPTQ_ACT_RELU) return fail(RPTQ_ERR_INVALID_ARG, "act = %d", act);
    if (!valid_bits(out_bits)) return fail(RPTQ_ERR_INVALID_ARG, "out_bits = %d not in {3, 4, 8}", out_bits);
    int st = check_bounds(out_bounds, out_g, -1);
    if (st) return st;
    if ((st = check_params(out_s, out_z, out_g))) return st;
    if (N_pad != kpad_of(out_bounds, out_g))
        return fail(RPTQ_ERR_INVALID_ARG, "N_pad = %d is not the output layout's K_pad %d", N_pad,
                    kpad_of(out_bounds, out_g));
    if (M > 0 && !out_codes) return fail(RPTQ_ERR_INVALID_ARG, "out_codes must be non-NULL");
    QuantOutArgs qo{out_codes, seg32_pitch(N_pad, out_bits), act};
    const ClusterArgs qc = make_cluster_args(out_bounds, out_g, out_s, out_z, out_bits, true);
    return qgemm_common(codes, M, K, N_pad, bounds, g, s, z, a_bits, w_packed, w_bits, s_w, colsum, Y, nullptr,
                        qo, qc, stream, "rptq_qgemm_quant launch");
}

static int kv_checks(int64_t T, int32_t C, const int32_t* bounds, int32_t g, const float* s, const int32_t* z,
                     int32_t bits) {
    if (T < 0) return fail(RPTQ_ERR_INVALID_ARG, "T = %lld < 0", (long long)T);
    if (C < 1) return fail(RPTQ_ERR_INVALID_ARG, "C = %d < 1", C);
    if (!valid_bits(bits)) return fail(RPTQ_ERR_INVALID_ARG, "bits = %d not in {3, 4, 8}", bits);
    int st = check_bounds(bounds, g, C);
    if (st) return st;
    if ((st = check_params(s, z, g))) return st;
    if (C % 8) return fail(RPTQ_ERR_UNSUPPORTED, "C = %d is not a multiple of 8", C);
    if (bits == 3 && C % 32) return fail(RPTQ_ERR_UNSUPPORTED, "3-bit rows need C %% 32 == 0 (C = %d)", C);
    if (C > kMaxK) return fail(RPTQ_ERR_UNSUPPORTED, "C = %d exceeds %d", C, kMaxK);
    return RPTQ_OK;
}

int rptq_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R, const int32_t* bounds,
                       int32_t g, const float* s, const int32_t* z, int32_t bits, uint8_t* packed,
                       void* stream) {
    int st = kv_checks(T, C, bounds, g, s, z, bits);
    if (st) return st;
    if (T == 0) return ok();
    if (!kv || !packed) return fail(RPTQ_ERR_INVALID_ARG, "kv or packed is NULL");
    if (!aligned16(kv) || !aligned16(packed) || (R && !aligned16(R)))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const ClusterArgs ca = make_cluster_args(bounds, g, s, z, bits, false);
    return hip_status(launch_kv_quant_pack(kv, T, C, R, ca, packed, (hipStream_t)stream),
                      "rptq_kv_quant_pack launch");
}

int64_t rptq_kv_attention_workspace_bytes(int32_t B, int32_t T, int32_t C, int32_t head_dim) {
    if (B < 0 || T < 1 || (head_dim != 64 && head_dim != 128) || C < 128 || C % 128 || C > kAttnMaxC) return -1;
    return kv_attention_workspace(B, T, C, head_dim);
}

int rptq_kv_attention(const uint16_t* q, const uint8_t* k_packed, const uint8_t* v_packed, int32_t B, int32_t T,
                      int32_t C, int32_t head_dim, float scale, const int32_t* R_k, const int32_t* bounds_k,
                      int32_t g_k, const float* s_k, const int32_t* z_k, const int32_t* R_v,
                      const int32_t* bounds_v, int32_t g_v, const float* s_v, const int32_t* z_v, int32_t bits,
                      float* out, void* workspace, int64_t workspace_bytes, void* stream) {
    if (B < 0) return fail(RPTQ_ERR_INVALID_ARG, "B = %d < 0", B);
    if (T < 1) return fail(RPTQ_ERR_INVALID_ARG, "T = %d < 1", T);
    if (head_dim != 64 && head_dim != 128) return fail(RPTQ_ERR_UNSUPPORTED, "head_dim = %d not 64 or 128", head_dim);
    if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(RPTQ_ERR_INVALID_ARG, "scale must be finite and > 0");
    int st = kv_checks(T, C, bounds_k, g_k, s_k, z_k, bits);
    if (st) return st;
    if ((st = kv_checks(T, C, bounds_v, g_v, s_v, z_v, bits))) return st;
    if (C % 128) return fail(RPTQ_ERR_UNSUPPORTED, "C = %d is not a multiple of 128", C);
    if (C > kAttnMaxC) return fail(RPTQ_ERR_UNSUPPORTED, "C = %d exceeds %d", C, kAttnMaxC);
    if ((int64_t)B * T > ((int64_t)1 << 31) / 2) return fail(RPTQ_ERR_UNSUPPORTED, "B * T too large");
    if (B == 0) return ok();
    if (!q || !k_packed || !v_packed || !out || !workspace)
        return fail(RPTQ_ERR_INVALID_ARG, "q, k_packed, v_packed, out and workspace must be non-NULL");
    if (!aligned16(q) || !aligned16(k_packed) || !aligned16(v_packed) || !aligned16(out) || !aligned16(workspace) ||
        (R_k && !aligned16(R_k)) || (R_v && !aligned16(R_v)))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const int64_t need = kv_attention_workspace(B, T, C, head_dim);
    if (workspace_bytes < need)
        return fail(RPTQ_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need);
    const ClusterArgs ck = make_cluster_args(bounds_k, g_k, s_k, z_k, bits, false);
    const ClusterArgs cv = make_cluster_args(bounds_v, g_v, s_v, z_v, bits, false);
    return hip_status(launch_kv_attention(q, k_packed, v_packed, B, T, C, head_dim, scale, R_k, ck, R_v, cv, out,
                                          workspace, (hipStream_t)stream),
                      "rptq_kv_attention launch");
}

int rptq_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R, const int32_t* bounds,
                    int32_t g, const float* s, const int32_t* z, int32_t bits, uint16_t* out, void* stream) {
    int st = kv_checks(T, C, bounds, g, s, z, bits);
    if (st) return st;
    if (T == 0) return ok();
    if (!packed || !out) return fail(RPTQ_ERR_INVALID_ARG, "packed or out is NULL");
    if (!aligned16(packed) || !aligned16(out) || (R && !aligned16(R)))
        return fail(RPTQ_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
    const ClusterArgs ca = make_cluster_args(bounds, g, s, z, bits, false);
    return hip_status(launch_kv_dequant(packed, T, C, R, ca, out, (hipStream_t)stream), "rptq_kv_dequant launch");
}

// ------------------------------------------------------------------ calibration
int rptq_calib_minmax(const uint16_t* x, int32_t mode, int64_t M, int32_t K, const float* gamma,
                      const float* beta, float eps, float* mx, float* mn, void* stream) {
    if (mode != RPTQ_IN_FP16_RAW && mode != RPTQ_CALIB_RAW) return fail(RPTQ_ERR_INVALID_ARG, "mode = %d", mode);
    if (M < 1) return fail(RPTQ_ERR_INVALID_ARG, "M = %lld < 1", (long long)M);
    if (M > 0x7fffffff) return fail(RPTQ_ERR_UNSUPPORTED, "M too large");
    if (K < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d < 1", K);
    if (K % 8) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d is not a multiple of 8", K);
    if (K > kMaxK) return fail(RPTQ_ERR_UNSUPPORTED, "K = %d exceeds %d", K, kMaxK);
    if (!x || !mx || !mn) return fail(RPTQ_ERR_INVALID_ARG, "x, mx or mn is NULL");
    if (mode == RPTQ_IN_FP16_RAW) {
        if (!gamma || !beta) return fail(RPTQ_ERR_INVALID_ARG, "gamma / beta is NULL");
        if (!(eps > 0.0f) || !std::isfinite(eps)) return fail(RPTQ_ERR_INVALID_ARG, "eps must be finite and > 0");
    }
    if (!aligned16(x) || !aligned16(mx) || !aligned16(mn)) return fail(RPTQ_ERR_ALIGNMENT, "misaligned pointer");
    return hip_status(launch_calib_minmax(x, mode, M, K, gamma, beta, eps, mx, mn, (hipStream_t)stream),
                      "rptq_calib_minmax launch");
}

static double sq2(double ax, double ay, double bx, double by) {
    const double dx = ax - bx, dy = ay - by;
    return dx * dx + dy * dy;
}

int rptq_kmeans_reorder(const float* mx, const float* mn, int32_t K, int32_t g, const double* init_u,
                        int32_t n_init, int32_t max_iter, int32_t* R, int32_t* bounds) {
    if (!mx || !mn || !init_u || !R || !bounds) return fail(RPTQ_ERR_INVALID_ARG, "NULL argument");
    if (K < 1 || g < 1 || g > K || g > kMaxClusters || n_init < 1 || max_iter < 1)
        return fail(RPTQ_ERR_INVALID_ARG, "K = %d, g = %d, n_init = %d, max_iter = %d", K, g, n_init, max_iter);
    std::vector<double> px(K), py(K);
    for (int k = 0; k < K; ++k) {
        px[k] = mx[k];
        py[k] = mn[k];
        if (!std::isfinite(px[k]) || !std::isfinite(py[k]))
            return fail(RPTQ_ERR_INVALID_ARG, "channel %d has a non-finite max/min", k);
    }
    std::vector<int32_t> best_lab(K), lab(K), prev(K);
    std::vector<double> best_cx(g), best_cy(g), cx(g), cy(g), d2(K);
    double best_in = INFINITY;
    for (int run = 0; run < n_init; ++run) {
        const double* u = init_u + (int64_t)run * g;
        // k-means++: first centre uniform, then D^2-weighted draws
        int first = (int)std::floor(u[0] * K);
        first = std::min(std::max(first, 0), K - 1);
        cx[0] = px[first]; cy[0] = py[first];
        for (int k = 0; k < K; ++k) d2[k] = sq2(px[k], py[k], cx[0], cy[0]);
        for (int c = 1; c < g; ++c) {
            double tot = 0.0;
            for (int k = 0; k < K; ++k) tot += d2[k];
            int pick = K - 1;
            if (tot > 0.0) {
                const double target = u[c] * tot;
                double run_sum = 0.0;
                for (int k = 0; k < K; ++k) {
                    run_sum += d2[k];
                    if (run_sum > target) { pick = k; break; }
                }
            } else {
                pick = std::min(c, K - 1);
            }
            cx[c] = px[pick]; cy[c] = py[pick];
            for (int k = 0; k < K; ++k) d2[k] = std::min(d2[k], sq2(px[k], py[k], cx[c], cy[c]));
        }
        // Lloyd
        std::fill(prev.begin(), prev.end(), -1);
        auto assign = [&]() {
            for (int k = 0; k < K; ++k) {
                int b = 0;
                double bd = sq2(px[k], py[k], cx[0], cy[0]);
                for (int c = 1; c < g; ++c) {
                    const double d = sq2(px[k], py[k], cx[c], cy[c]);
                    if (d < bd) { bd = d; b = c; }
                }
                lab[k] = b;
            }
        };
        for (int it = 1; it <= max_iter; ++it) {
            assign();
            std::vector<double> sx(g, 0.0), sy(g, 0.0);
            std::vector<int> cnt(g, 0);
            for (int k = 0; k < K; ++k) { sx[lab[k]] += px[k]; sy[lab[k]] += py[k]; ++cnt[lab[k]]; }
            for (int c = 0; c < g; ++c)
                if (cnt[c]) { cx[c] = sx[c] / cnt[c]; cy[c] = sy[c] / cnt[c]; }
            for (int c = 0; c < g; ++c) {
                if (cnt[c]) continue;
                int far = 0;
                double fd = -1.0;
                for (int k = 0; k < K; ++k) {
                    const double d = sq2(px[k], py[k], cx[lab[k]], cy[lab[k]]);
                    if (d > fd) { fd = d; far = k; }
                }
                --cnt[lab[far]];
                lab[far] = c;
                cnt[c] = 1;
                cx[c] = px[far]; cy[c] = py[far];
            }
            if (lab == prev) break;
            prev = lab;
        }
        assign();
        double in = 0.0;
        for (int k = 0; k < K; ++k) in += sq2(px[k], py[k], cx[lab[k]], cy[lab[k]]);
        if (in < best_in) { best_in = in; best_lab = lab; best_cx = cx; best_cy = cy; }
    }
    // order clusters: centroid min, then centroid max, then lowest member channel
    std::vector<int> first(g, K), cnt(g, 0);
    for (int k = 0; k < K; ++k) {
        ++cnt[best_lab[k]];
        first[best_lab[k]] = std::min(first[best_lab[k]], k);
    }
    for (int c = 0; c < g; ++c)
        if (!cnt[c]) return fail(RPTQ_ERR_INVALID_ARG, "KMeans left cluster %d empty", c);
    std::vector<int> order(g);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [&](int a, int b) {
        if (best_cy[a] != best_cy[b]) return best_cy[a] < best_cy[b];
        if (best_cx[a] != best_cx[b]) return best_cx[a] < best_cx[b];
        return first[a] < first[b];
    });
    int pos = 0;
    bounds[0] = 0;
    for (int oc = 0; oc < g; ++oc) {
        for (int k = 0; k < K; ++k)
            if (best_lab[k] == order[oc]) R[pos++] = k;
        bounds[oc + 1] = pos;
    }
    return ok();
}

int rptq_cluster_params(const float* mx, const float* mn, const int32_t* R, const int32_t* bounds, int32_t g,
                        int32_t bits, float* s, int32_t* z) {
    if (!mx || !mn || !s || !z) return fail(RPTQ_ERR_INVALID_ARG, "NULL argument");
    if (!valid_bits(bits)) return fail(RPTQ_ERR_INVALID_ARG, "bits = %d", bits);
    int st = check_bounds(bounds, g, -1);
    if (st) return st;
    const double qmax = (double)((1 << bits) - 1);
    for (int c = 0; c < g; ++c) {
        double lo = INFINITY, hi = -INFINITY;
        for (int j = bounds[c]; j < bounds[c + 1]; ++j) {
            const int k = R ? R[j] : j;
            lo = std::min(lo, (double)mn[k]);
            hi = std::max(hi, (double)mx[k]);
        }
        if (!std::isfinite(lo) || !std::isfinite(hi) || hi < lo)
            return fail(RPTQ_ERR_INVALID_ARG, "cluster %d has an invalid range", c);
        float sc = (float)((hi - lo) / qmax);
        const float fl = (float)(std::max(std::fabs(lo), std::fabs(hi)) * std::ldexp(1.0, -21));
        if (sc < fl) sc = fl;
        if (sc == 0.0f) sc = 1.0f;
        s[c] = sc;
        z[c] = (int32_t)std::nearbyint(-lo / (double)sc);
    }
    return ok();
}

int rptq_quantize_weights(const float* W, int32_t K, int32_t N, int32_t w_bits, int8_t* wq, float* s_w) {
    if (!W || !wq || !s_w) return fail(RPTQ_ERR_INVALID_ARG, "NULL argument");
    if (K < 1 || N < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d, N = %d", K, N);
    if (!valid_wbits(w_bits)) return fail(RPTQ_ERR_INVALID_ARG, "w_bits = %d", w_bits);
    const int qm = (1 << (w_bits - 1)) - 1;
    std::vector<double> amax(N, 0.0);
    for (int64_t k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) amax[n] = std::max(amax[n], std::fabs((double)W[k * N + n]));
    for (int n = 0; n < N; ++n) {
        float sw = (float)(amax[n] / qm);
        s_w[n] = sw == 0.0f ? 1.0f : sw;
    }
    const int nt = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&, t]() {
            for (int64_t k = t; k < K; k += nt)
                for (int n = 0; n < N; ++n) {
                    double r = std::nearbyint((double)W[k * N + n] / (double)s_w[n]);
                    r = std::min(std::max(r, (double)-qm), (double)qm);
                    wq[k * N + n] = (int8_t)r;
                }
        });
    for (auto& th : pool) th.join();
    return ok();
}

int rptq_pack_weights(const int8_t* wq, int32_t K, int32_t N, int32_t w_bits, const int32_t* R,
                      const int32_t* bounds, int32_t g, uint8_t* w_packed, int32_t* colsum) {
    if (!wq || !w_packed || !colsum) return fail(RPTQ_ERR_INVALID_ARG, "NULL argument");
    if (K < 1 || N < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d, N = %d", K, N);
    if (!valid_wbits(w_bits)) return fail(RPTQ_ERR_INVALID_ARG, "w_bits = %d", w_bits);
    int st = check_bounds(bounds, g, K);
    if (st) return st;
    const int qm = (1 << (w_bits - 1)) - 1;
    const int32_t kp = kpad_of(bounds, g);
    const int64_t rb = seg32_pitch(kp, w_bits), data_bytes = (int64_t)kp * w_bits / 8;
    // padded position -> natural row (-1 for pad)
    std::vector<int32_t> src(kp, -1);
    std::vector<int32_t> clus(kp, 0);
    int32_t off = 0;
    for (int c = 0; c < g; ++c) {
        const int32_t n_c = bounds[c + 1] - bounds[c];
        for (int32_t i = 0; i < n_c; ++i) {
            const int32_t j = bounds[c] + i;
            const int32_t k = R ? R[j] : j;
            if (k < 0 || k >= K) return fail(RPTQ_ERR_INVALID_ARG, "R[%d] = %d out of range", j, k);
            src[off + i] = k;
        }
        for (int32_t i = 0; i < (n_c + 31) / 32 * 32; ++i) clus[off + i] = c;
        off += (n_c + 31) / 32 * 32;
    }
    for (int64_t k = 0; k < (int64_t)K * N; ++k)
        if (wq[k] < -qm || wq[k] > qm)
            return fail(RPTQ_ERR_INVALID_ARG, "weight code %d outside [-%d, %d]", (int)wq[k], qm, qm);
    std::memset(colsum, 0, sizeof(int32_t) * (size_t)g * N);
    const int nt = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&, t]() {
            std::vector<int8_t> col(kp);
            for (int n = t; n < N; n += nt) {
                for (int32_t p = 0; p < kp; ++p) {
                    col[p] = src[p] < 0 ? 0 : wq[(int64_t)src[p] * N + n];
                    colsum[(int64_t)clus[p] * N + n] += col[p];
                }
                uint8_t* dst = w_packed + (int64_t)n * rb;
                std::memset(dst + data_bytes, 0, (size_t)(rb - data_bytes));
                if (w_bits == 8) {
                    for (int32_t p = 0; p < kp; ++p) dst[p] = (uint8_t)col[p];
                } else if (w_bits == 3) {
                    // 32 weights -> 12 bytes, the activation codes' 3-bit group
                    // layout on the 3-bit two's complement fields
                    for (int32_t p = 0; p < kp; p += 32) {
                        uint8_t* gb = dst + p / 32 * 12;
                        for (int j = 0; j < 4; ++j) {
                            int f[8];
                            for (int e = 0; e < 8; ++e) f[e] = col[p + j + 4 * e] & 7;
                            gb[j] = (uint8_t)(f[0] | f[1] << 3 | (f[6] & 3) << 6);
                            gb[4 + j] = (uint8_t)(f[2] | f[3] << 3 | (f[7] & 3) << 6);
                            gb[8 + j] = (uint8_t)(f[4] | f[5] << 3 | (f[6] >> 2) << 6 | (f[7] >> 2) << 7);
                        }
                    }
                } else {
                    for (int32_t p = 0; p < kp; p += 8)
                        for (int i = 0; i < 4; ++i)
                            dst[p / 2 + i] = (uint8_t)((col[p + i] & 15) | ((col[p + 4 + i] & 15) << 4));
                }
            }
        });
    for (auto& th : pool) th.join();
    return ok();
}

int rptq_pack_weights_out(const int8_t* wq, int32_t K, int32_t N, int32_t w_bits, const int32_t* R,
                          const int32_t* bounds, int32_t g, const int32_t* R_out, const int32_t* out_bounds,
                          int32_t out_g, const float* s_w, uint8_t* w_packed, int32_t* colsum, float* s_w_out) {
    if (!wq || !s_w || !w_packed || !colsum || !s_w_out) return fail(RPTQ_ERR_INVALID_ARG, "NULL argument");
    if (K < 1 || N < 1) return fail(RPTQ_ERR_INVALID_ARG, "K = %d, N = %d", K, N);
    int st = check_bounds(out_bounds, out_g, N);
    if (st) return st;
    const int32_t np = kpad_of(out_bounds, out_g);
    // padded output position -> natural output feature (-1 for pad)
    std::vector<int32_t> src(np, -1);
    std::vector<char> seen(N, 0);
    int32_t off = 0;
    for (int c = 0; c < out_g; ++c) {
        for (int32_t j = out_bounds[c]; j < out_bounds[c + 1]; ++j) {
            const int32_t n = R_out ? R_out[j] : j;
            if (n < 0 || n >= N || seen[n]) return fail(RPTQ_ERR_INVALID_ARG, "R_out is not a permutation");
            seen[n] = 1;
            src[off + j - out_bounds[c]] = n;
        }
        off += (out_bounds[c + 1] - out_bounds[c] + 31) / 32 * 32;
    }
    std::vector<int8_t> wq2((size_t)K * np, 0);
    for (int64_t k = 0; k < K; ++k)
        for (int32_t p = 0; p < np; ++p)
            if (src[p] >= 0) wq2[k * np + p] = wq[k * N + src[p]];
    for (int32_t p = 0; p < np; ++p) s_w_out[p] = src[p] >= 0 ? s_w[src[p]] : 1.0f;
    return rptq_pack_weights(wq2.data(), K, np, w_bits, R, bounds, g, w_packed, colsum);
}

}  // extern "C"
