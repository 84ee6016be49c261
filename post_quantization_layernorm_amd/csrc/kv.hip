// K/V-cache per-cluster quantize + pack, and dequantize (gfx950).
//
// RPTQ write-up, evaluation section: the W4A4KV / W4A3KV / W3A3KV settings
// quantize only the key and value caches, the memory that dominates at large
// batch x sequence length.  Both kernels are pure streaming (HBM-bound):
//   quant-pack: fp16 [T][C] natural order -> DENSE b-bit codes in R order;
//   dequant:    DENSE codes -> fp16 [T][C] natural order,
//               out[R[j]] = fp16_rne(s_c * (q_j - z_c)).
// A persistent workgroup walks the rows; every lane owns fixed units of 8
// codes (their source/destination channel and cluster constants live in
// registers), rows are staged in LDS so the R permutation is an LDS gather
// (quant-pack) or scatter (dequant), and HBM sees only 16-byte coalesced
// loads and stores.  The next row's loads are issued before the current row
// is processed.
#include "rptq_device.hpp"

namespace rptq {
namespace {

__host__ __device__ constexpr int align16(int64_t b) { return (int)((b + 15) & ~int64_t(15)); }

template <int BITS, int UPL>
__global__ __launch_bounds__(kBlock) void kv_quant_pack_kernel(
    const uint16_t* __restrict__ kv, int64_t T, int32_t C, const int32_t* __restrict__ R,
    const ClusterArgs ca, uint8_t* __restrict__ packed) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int CH = (kMaxK * 2 / 16 + kBlock - 1) / kBlock;
    const int64_t row_bytes = (int64_t)C * BITS / 8;
    unsigned char* xrow = smem;
    unsigned char* orow = smem + align16((int64_t)C * 2);
    const int tid = threadIdx.x;
    const int n_units = C / 8;
    const int nchunks = C / 8;          // 16-byte chunks of an fp16 row

    int src[UPL][8];
    float inv[UPL][8];
    int zb[UPL][8];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * kBlock;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            src[u][e] = 0; inv[u][e] = 0.0f; zb[u][e] = 0;
            if (unit < n_units) {
                const int j = UnitGeom<BITS>::first(unit) + e * UnitGeom<BITS>::stride;
                const int c = cluster_of_pos(ca, j);
                src[u][e] = (R ? R[j] : j) * 2;
                inv[u][e] = ca.inv_s[c];
                zb[u][e] = ca.z[c] - kRoundMagicBits;
            }
        }
    }

    u32x4 buf[CH];
    auto load_row = [&](int64_t t) {
        const u32x4* g = reinterpret_cast<const u32x4*>(kv + t * C);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * kBlock;
            if (c < nchunks) buf[i] = __builtin_nontemporal_load(g + c);
        }
    };

    int64_t t = blockIdx.x;
    if (t < T) load_row(t);
    for (; t < T; t += gridDim.x) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * kBlock;
            if (c < nchunks) reinterpret_cast<u32x4*>(xrow)[c] = buf[i];
        }
        __syncthreads();
        if (t + gridDim.x < T) load_row(t + gridDim.x);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int unit = tid + u * kBlock;
            if (unit >= n_units) continue;
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (float)*reinterpret_cast<const _Float16*>(xrow + src[u][e]);
                q[e] = quant_code(v, inv[u][e], zb[u][e], QMAX);
            }
            store_unit<BITS>(orow, unit, q);
        }
        __syncthreads();
        store_row(packed + t * row_bytes, orow, row_bytes);
    }
}

template <int BITS, int UPL>
__global__ __launch_bounds__(kBlock) void kv_dequant_kernel(
    const uint8_t* __restrict__ packed, int64_t T, int32_t C, const int32_t* __restrict__ R,
    const ClusterArgs ca, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CH = (kMaxK * BITS / 8 / 4 + kBlock - 1) / kBlock;   // 4-byte chunks per thread
    const int64_t row_bytes = (int64_t)C * BITS / 8;
    unsigned char* prow = smem;                                    // packed row
    unsigned char* orow = smem + align16(row_bytes);               // fp16 row, natural order
    const int tid = threadIdx.x;
    const int n_units = C / 8;
    const int nwords = (int)(row_bytes / 4);

    int dst[UPL][8];
    float sc[UPL][8];
    float zf[UPL][8];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * kBlock;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dst[u][e] = 0; sc[u][e] = 0.0f; zf[u][e] = 0.0f;
            if (unit < n_units) {
                const int j = UnitGeom<BITS>::first(unit) + e * UnitGeom<BITS>::stride;
                const int c = cluster_of_pos(ca, j);
                dst[u][e] = (R ? R[j] : j) * 2;
                sc[u][e] = ca.s[c];
                zf[u][e] = (float)ca.z[c];       // |z| <= 2^21: exact
            }
        }
    }

    uint32_t buf[CH];
    auto load_row = [&](int64_t t) {
        const uint32_t* g = reinterpret_cast<const uint32_t*>(packed + t * row_bytes);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * kBlock;
            if (c < nwords) buf[i] = __builtin_nontemporal_load(g + c);
        }
    };

    int64_t t = blockIdx.x;
    if (t < T) load_row(t);
    for (; t < T; t += gridDim.x) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = tid + i * kBlock;
            if (c < nwords) reinterpret_cast<uint32_t*>(prow)[c] = buf[i];
        }
        __syncthreads();
        if (t + gridDim.x < T) load_row(t + gridDim.x);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int unit = tid + u * kBlock;
            if (unit >= n_units) continue;
            int q[8];
            load_unit<BITS>(prow, unit, q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // (q - z) is an exact integer in fp32; the product is rounded
                // once, straight to fp16 (v_fma_mixlo_f16: fused, half to even)
                const float d = (float)q[e] - zf[u][e];
                *reinterpret_cast<_Float16*>(orow + dst[u][e]) = (_Float16)(sc[u][e] * d);
            }
        }
        __syncthreads();
        store_row(reinterpret_cast<uint8_t*>(out + t * C), orow, (int64_t)C * 2);
    }
}

template <int BITS>
const void* pick_quant(int upl) {
    switch (upl) {
        case 1: return (const void*)kv_quant_pack_kernel<BITS, 1>;
        case 2: return (const void*)kv_quant_pack_kernel<BITS, 2>;
        case 3: return (const void*)kv_quant_pack_kernel<BITS, 3>;
        case 4: return (const void*)kv_quant_pack_kernel<BITS, 4>;
        case 5: return (const void*)kv_quant_pack_kernel<BITS, 5>;
        case 6: return (const void*)kv_quant_pack_kernel<BITS, 6>;
        case 7: return (const void*)kv_quant_pack_kernel<BITS, 7>;
        case 8: return (const void*)kv_quant_pack_kernel<BITS, 8>;
        default: return nullptr;
    }
}

template <int BITS>
const void* pick_dequant(int upl) {
    switch (upl) {
        case 1: return (const void*)kv_dequant_kernel<BITS, 1>;
        case 2: return (const void*)kv_dequant_kernel<BITS, 2>;
        case 3: return (const void*)kv_dequant_kernel<BITS, 3>;
        case 4: return (const void*)kv_dequant_kernel<BITS, 4>;
        case 5: return (const void*)kv_dequant_kernel<BITS, 5>;
        case 6: return (const void*)kv_dequant_kernel<BITS, 6>;
        case 7: return (const void*)kv_dequant_kernel<BITS, 7>;
        case 8: return (const void*)kv_dequant_kernel<BITS, 8>;
        default: return nullptr;
    }
}

}  // namespace

hipError_t launch_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R,
                                const ClusterArgs& ca, uint8_t* packed, hipStream_t stream) {
    const int upl = (C / 8 + kBlock - 1) / kBlock;
    const void* k = ca.bits == 3 ? pick_quant<3>(upl) : ca.bits == 4 ? pick_quant<4>(upl) : pick_quant<8>(upl);
    if (!k) return hipErrorInvalidValue;
    const size_t lds = (size_t)align16((int64_t)C * 2) + align16((int64_t)C * ca.bits / 8);
    const int grid = persistent_grid(k, kBlock, lds, T);
    void* args[] = {(void*)&kv, (void*)&T, (void*)&C, (void*)&R, (void*)&ca, (void*)&packed};
    return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, lds, stream);
}

hipError_t launch_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R,
                             const ClusterArgs& ca, uint16_t* out, hipStream_t stream) {
    const int upl = (C / 8 + kBlock - 1) / kBlock;
    const void* k = ca.bits == 3 ? pick_dequant<3>(upl) : ca.bits == 4 ? pick_dequant<4>(upl) : pick_dequant<8>(upl);
    if (!k) return hipErrorInvalidValue;
    const size_t lds = (size_t)align16((int64_t)C * ca.bits / 8) + align16((int64_t)C * 2);
    const int grid = persistent_grid(k, kBlock, lds, T);
    void* args[] = {(void*)&packed, (void*)&T, (void*)&C, (void*)&R, (void*)&ca, (void*)&out};
    return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, lds, stream);
}

}  // namespace rptq
