// Fused LayerNorm + reorder + per-cluster quantize + SEG32 pack (gfx950).
//
// RPTQ write-up, method section and Fig. 3: LayerNorm is changed to emit the
// reordered activations directly, so the reorder costs no extra pass or
// buffer; each cluster of reordered channels has its own (s, z).  The kernel
// is HBM-bound: it reads fp16 [M][K] once and writes b-bit codes once.
//
// Design (one persistent workgroup of 256 or 512 threads per row at a time):
//   - every lane owns a fixed set of "units" (8 output codes each) for all
//     rows; the source channel R[j], gamma'[j], beta'[j] and the cluster's
//     (1/s, z) of its units stay in registers across rows;
//   - a row is read with 16-byte coalesced loads (the next row's loads are in
//     flight while the current row is quantized), the mean and the biased
//     variance are two wave-shuffle reductions over the register copy
//     (two-pass, fp32), and the row is parked in LDS in natural order;
//   - each unit gathers its 8 inputs from LDS by R, normalizes, quantizes and
//     packs them into an LDS copy of the output row, which is then written
//     with 16-byte coalesced stores.
#include "rptq_device.hpp"
#include "../../include/rptq.h"

namespace rptq {
namespace {

__host__ __device__ constexpr int align16(int64_t b) { return (int)((b + 15) & ~int64_t(15)); }

template <int BLOCK>
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) scratch[w] = v;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < BLOCK / 64; ++i) t += scratch[i];
    __syncthreads();
    return t;
}

template <int BITS, int MODE, int UPL, int BLOCK>
__global__ __launch_bounds__(BLOCK) void ln_reorder_quant_kernel(
    const void* __restrict__ xin, int64_t M, int32_t K, int64_t row_bytes,
    const float* __restrict__ gamma_r, const float* __restrict__ beta_r, float eps,
    const int32_t* __restrict__ R, const ClusterArgs ca, uint8_t* __restrict__ codes) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr bool LN = MODE == RPTQ_IN_FP16_RAW;
    constexpr int ESZ = LN ? 2 : 4;                       // bytes per input element
    constexpr int CH = (kMaxK * ESZ / 16 + BLOCK - 1) / BLOCK;   // 16-B chunks per thread
    const int row_in_bytes = K * ESZ;
    unsigned char* xrow = smem;
    unsigned char* orow = smem + align16(row_in_bytes);
    float* red = reinterpret_cast<float*>(orow + align16(row_bytes));
    const int tid = threadIdx.x;
    const int n_units = ca.K_pad / 8;
    const int nchunks = row_in_bytes / 16;

    // ---- per-lane unit tables (fixed for every row)
    int src[UPL][8];
    float gam[UPL][8], bet[UPL][8];
    float uinv[UPL];
    int uzb[UPL], unv[UPL];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * BLOCK;
        unv[u] = -1;
        uinv[u] = 0.0f;
        uzb[u] = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) { src[u][e] = 0; gam[u][e] = 0.0f; bet[u][e] = 0.0f; }
        if (unit < n_units) {
            const int p0 = UnitGeom<BITS>::first(unit);
            const int c = cluster_of_padded(ca, p0);
            const int n_c = ca.bounds[c + 1] - ca.bounds[c];
            uinv[u] = ca.inv_s[c];
            uzb[u] = ca.z[c] - kRoundMagicBits;
            int nv = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = p0 + e * UnitGeom<BITS>::stride - ca.off[c];
                if (i < n_c) {
                    const int j = ca.bounds[c] + i;
                    nv = e + 1;
                    if constexpr (LN) {
                        src[u][e] = (R ? R[j] : j) * 2;
                        gam[u][e] = gamma_r[j];
                        bet[u][e] = beta_r[j];
                    } else {
                        src[u][e] = j * 4;
                    }
                }
            }
            unv[u] = nv;
        }
    }

    u32x4 buf[CH];
    auto load_row = [&](int64_t row) {
        const u32x4* g = reinterpret_cast<const u32x4*>(static_cast<const char*>(xin) + row * row_in_bytes);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * BLOCK;
            if (c < nchunks) buf[i] = __builtin_nontemporal_load(g + c);
        }
    };

    int64_t row = blockIdx.x;
    if (row < M) load_row(row);
    for (; row < M; row += gridDim.x) {
        float mean = 0.0f, rstd = 0.0f;
        if constexpr (LN) {
            // pass 1: sum (packed fp16 dot products against 1.0, fp32 accumulate)
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (tid + i * BLOCK < nchunks) {
                    const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[k]), one2, s, false);
                }
            }
            s = block_sum<BLOCK>(s, red);
            mean = s / (float)K;
            // pass 2: biased variance around the mean
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (tid + i * BLOCK < nchunks) {
                    const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const half2_t h = __builtin_bit_cast(half2_t, w[k]);
                        const float d0 = (float)h.x - mean, d1 = (float)h.y - mean;
                        ss = __builtin_fmaf(d0, d0, ss);
                        ss = __builtin_fmaf(d1, d1, ss);
                    }
                }
            }
            ss = block_sum<BLOCK>(ss, red);
            rstd = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * BLOCK;
            if (c < nchunks) reinterpret_cast<u32x4*>(xrow)[c] = buf[i];
        }
        __syncthreads();
        if (row + gridDim.x < M) load_row(row + gridDim.x);      // next row in flight

        const float nmr = -mean * rstd;
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            if (unv[u] < 0) continue;
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float y;
                if constexpr (LN) {
                    const float xv = (float)*reinterpret_cast<const _Float16*>(xrow + src[u][e]);
                    const float n = __builtin_fmaf(xv, rstd, nmr);
                    y = __builtin_fmaf(gam[u][e], n, bet[u][e]);
                } else {
                    y = *reinterpret_cast<const float*>(xrow + src[u][e]);
                }
                const int qq = quant_code(y, uinv[u], uzb[u], QMAX);
                q[e] = e < unv[u] ? qq : 0;
            }
            store_unit<BITS>(orow, tid + u * BLOCK, q);
        }
        __syncthreads();
        store_row(codes + row * row_bytes, orow, row_bytes);
    }
}

template <int BITS, int MODE, int BLOCK>
const void* pick_kernel(int upl) {
    switch (upl) {
        case 1: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 1, BLOCK>;
        case 2: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 2, BLOCK>;
        case 3: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 3, BLOCK>;
        case 4: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 4, BLOCK>;
        case 5: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 5, BLOCK>;
        default: return nullptr;
    }
}

template <int BITS, int MODE>
const void* pick(int upl, int block) {
    return block == 256 ? pick_kernel<BITS, MODE, 256>(upl) : pick_kernel<BITS, MODE, 512>(upl);
}

}  // namespace

hipError_t launch_ln_reorder_quant(const void* x, int in_mode, int64_t M, int32_t K,
                                   const float* gamma_r, const float* beta_r, float eps,
                                   const int32_t* R, const ClusterArgs& ca, int64_t row_bytes,
                                   uint8_t* codes, hipStream_t stream) {
    const int n_units = ca.K_pad / 8;
    const int block = n_units <= 5 * 256 ? 256 : 512;
    const int upl = (n_units + block - 1) / block;
    const void* k = nullptr;
    if (in_mode == RPTQ_IN_FP16_RAW) {
        k = ca.bits == 3 ? pick<3, 0>(upl, block) : ca.bits == 4 ? pick<4, 0>(upl, block) : pick<8, 0>(upl, block);
    } else {
        k = ca.bits == 3 ? pick<3, 1>(upl, block) : ca.bits == 4 ? pick<4, 1>(upl, block) : pick<8, 1>(upl, block);
    }
    if (!k) return hipErrorInvalidValue;
    const int esz = in_mode == RPTQ_IN_FP16_RAW ? 2 : 4;
    const size_t lds = (size_t)align16((int64_t)K * esz) + align16(row_bytes) + 64;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int grid = persistent_grid(k, block, lds, M);
    void* args[] = {(void*)&x, (void*)&M, (void*)&K, (void*)&row_bytes, (void*)&gamma_r,
                    (void*)&beta_r, (void*)&eps, (void*)&R, (void*)&ca, (void*)&codes};
    return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, stream);
}

}  // namespace rptq
