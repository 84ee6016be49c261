// Calibration statistics: per-channel max and min over a calibration batch
// (RPTQ write-up, method section: the calibration set is run through the
// model and every activation channel's max and min are recorded; Fig. 1
// plots these (max, min) points).  Offline, off the hot path.
//
// One workgroup per calibration row: the row's LayerNorm (same fp32 math as
// the fused kernel) or the raw value, then float max/min merged into the
// per-channel outputs with integer atomics (for IEEE floats, signed-integer
// order matches float order on non-negative values and reversed
// unsigned-integer order matches it on negative values).
#include "rptq_device.hpp"
#include "../../include/rptq.h"

namespace rptq {
namespace {

__global__ void fill_kernel(float* __restrict__ mx, float* __restrict__ mn, int32_t K) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < K) { mx[k] = -__builtin_inff(); mn[k] = __builtin_inff(); }
}

__device__ __forceinline__ void atomic_fmax(float* addr, float v) {
    if (v >= 0.0f) atomicMax(reinterpret_cast<int*>(addr), __builtin_bit_cast(int, v));
    else atomicMin(reinterpret_cast<unsigned int*>(addr), __builtin_bit_cast(unsigned int, v));
}
__device__ __forceinline__ void atomic_fmin(float* addr, float v) {
    if (v >= 0.0f) atomicMin(reinterpret_cast<int*>(addr), __builtin_bit_cast(int, v));
    else atomicMax(reinterpret_cast<unsigned int*>(addr), __builtin_bit_cast(unsigned int, v));
}

template <bool LN>
__global__ __launch_bounds__(kCalibBlock) void calib_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                       int32_t K, const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float eps,
                                                       float* __restrict__ mx, float* __restrict__ mn) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    if (row >= M) return;
    const _Float16* xr = reinterpret_cast<const _Float16*>(x + row * K);
    float mean = 0.0f, rstd = 1.0f;
    if constexpr (LN) {
        float s = 0.0f;
        for (int k = threadIdx.x; k < K; k += kCalibBlock) s += (float)xr[k];
        s = block_sum_256(s, red);
        mean = s / (float)K;
        float ss = 0.0f;
        for (int k = threadIdx.x; k < K; k += kCalibBlock) {
            const float d = (float)xr[k] - mean;
            ss = __builtin_fmaf(d, d, ss);
        }
        ss = block_sum_256(ss, red);
        rstd = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
    }
    const float nmr = -mean * rstd;
    for (int k = threadIdx.x; k < K; k += kCalibBlock) {
        float v = (float)xr[k];
        if constexpr (LN) v = __builtin_fmaf(gamma[k], __builtin_fmaf(v, rstd, nmr), beta[k]);
        v += 0.0f;                      // -0 -> +0 so the integer orders agree
        atomic_fmax(mx + k, v);
        atomic_fmin(mn + k, v);
    }
}

}  // namespace

hipError_t launch_calib_minmax(const uint16_t* x, int mode, int64_t M, int32_t K,
                               const float* gamma, const float* beta, float eps,
                               float* mx, float* mn, hipStream_t stream) {
    fill_kernel<<<dim3((K + 255) / 256), dim3(256), 0, stream>>>(mx, mn, K);
    if (mode == RPTQ_IN_FP16_RAW)
        calib_kernel<true><<<dim3((unsigned)M), dim3(kCalibBlock), 0, stream>>>(x, M, K, gamma, beta, eps, mx, mn);
    else
        calib_kernel<false><<<dim3((unsigned)M), dim3(kCalibBlock), 0, stream>>>(x, M, K, gamma, beta, eps, mx, mn);
    return hipGetLastError();
}

}  // namespace rptq
