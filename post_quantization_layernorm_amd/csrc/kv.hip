// K/V-cache per-cluster quantize + pack, and dequantize (gfx950).
//
// RPTQ write-up, evaluation section: the W4A4KV / W4A3KV / W3A3KV settings
// quantize only the key and value caches, the memory that dominates at large
// batch x sequence length.  Both kernels are pure streaming (HBM-bound):
//   quant-pack: fp16 [T][C] natural order -> DENSE b-bit codes in R order;
//   dequant:    DENSE codes -> fp16 [T][C] natural order,
//               out[R[j]] = fp16_rne(s_c * (q_j - z_c)).
// One persistent workgroup per compute unit walks the rows (with this read :
// write mix a plain stream runs faster with fewer rows in flight); every lane
// owns fixed units of 8
// codes (their source/destination channel and cluster constants live in
// registers), rows are staged in LDS so the R permutation is an LDS gather
// (quant-pack) or scatter (dequant), and HBM sees only coalesced buffer loads
// and stores.  Two register buffers keep two rows per workgroup in flight
// while one is processed.  Every memory instruction runs unconditionally
// with a compile-time count (the buffer range check zero-fills / drops what
// lies past a row; idle units write a dummy LDS slot), so the compiler's
// memory-counter waits never cover the next row's loads.
#include <algorithm>

#include "rptq_device.hpp"

namespace rptq {
namespace {

// Per-lane unit tables of a DENSE row (fixed for every row): for code e of
// unit u, its natural channel (R[j], j the reordered position) and its
// cluster's scale entry (1/s or s) and z.  Set-up without dependent-load
// chains: clusters by counting the cluster starts at or below each position
// (starts read with v_readlane from a lane-resident table), the cluster
// entries over the lane crossbar, the R loads all issued together (16-byte
// loads when a unit's positions are consecutive).  Idle units (unit >=
// n_units) read position 0; the caller sends them to a dummy slot.
template <int BITS, int UPL>
__device__ __forceinline__ void kv_unit_tables(const ClusterArgs& ca, const int32_t* R, int32_t C, int n_units,
                                               bool want_inv, int (&chan)[UPL][8], float (&sv)[UPL][8],
                                               int (&zv)[UPL][8]) {
    const int tid = threadIdx.x, BLOCK = blockDim.x;
    const LaneClusters lc = lane_clusters(ca, false);
    const float sl = want_inv ? lc.inv_s : lc.s;
    int pos[UPL * 8], cl[UPL * 8];
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * BLOCK;
        const int p0 = unit < n_units ? UnitGeom<BITS>::first(unit) : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) pos[u * 8 + e] = p0 + e * UnitGeom<BITS>::stride;
    }
    clusters_of<UPL * 8>(lc, ca.g, pos, cl);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(R, R ? (int64_t)C * 4 : 0);
    const bool has_r = R != nullptr;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        int rv[8];
        if constexpr (UnitGeom<BITS>::stride == 1) {
            const uint32_t off = (uint32_t)pos[u * 8] * 4u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 r4 = __builtin_amdgcn_raw_buffer_load_b128(rr, off + 16 * h, 0, 0);
                rv[4 * h] = (int)r4.x; rv[4 * h + 1] = (int)r4.y; rv[4 * h + 2] = (int)r4.z; rv[4 * h + 3] = (int)r4.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                rv[e] = (int)__builtin_amdgcn_raw_buffer_load_b32(rr, (uint32_t)pos[u * 8 + e] * 4u, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = pos[u * 8 + e];
            chan[u][e] = j + (has_r ? rv[e] - j : 0);
            sv[u][e] = from_lane(sl, cl[u * 8 + e]);
            zv[u][e] = from_lane(lc.z, cl[u * 8 + e]);
        }
    }
}

template <int BITS, int UPL, bool OVEC16>
__global__ __launch_bounds__(kKvPackMaxBlock) void kv_quant_pack_kernel(
    const uint16_t* __restrict__ kv, int64_t T, int32_t C, const int32_t* __restrict__ R,
    const ClusterArgs ca, uint8_t* __restrict__ packed) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr int CH = UPL;                                   // fp16 row: C/8 chunks = C/8 units
    constexpr int OCH = chunks_for<OVEC16>(UPL * BITS);       // packed row: C*BITS/8 bytes
    constexpr int OCB = OVEC16 ? 16 : 4;
    const int BLOCK = blockDim.x;
    const int64_t in_bytes = (int64_t)C * 2;
    const int64_t row_bytes = (int64_t)C * BITS / 8;
    unsigned char* xrow = smem;                               // CH * 16 * BLOCK bytes
    unsigned char* orow = xrow + (size_t)CH * 16 * BLOCK;     // OCH * OCB * BLOCK bytes
    unsigned char* dummy = orow + (size_t)OCH * OCB * BLOCK;  // 16 bytes
    const int tid = threadIdx.x;
    const int n_units = C / 8;

    int src[UPL][8], zb[UPL][8], uob[UPL];
    float inv[UPL][8];
    kv_unit_tables<BITS, UPL>(ca, R, C, n_units, true, src, inv, zb);
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * BLOCK;
        uob[u] = unit < n_units ? UnitGeom<BITS>::out_byte(unit) : (int)(dummy - orow);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            src[u][e] *= 2;                          // byte offset of the fp16 input
            zb[u][e] -= kRoundMagicBits;
        }
    }

    u32x4 bufA[CH], bufB[CH];
    auto process = [&](u32x4 (&buf)[CH], int64_t t) {
        put_row_chunks<true, CH>(xrow, buf);
        __syncthreads();
        const int64_t tn = t + 2 * (int64_t)gridDim.x;
        load_row_chunks<true, CH>(buf, kv + tn * C, tn < T ? in_bytes : 0);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (float)*reinterpret_cast<const _Float16*>(xrow + src[u][e]);
                q[e] = quant_code(v, inv[u][e], zb[u][e], QMAX);
            }
            store_unit_at<BITS>(orow + uob[u], q);
        }
        __syncthreads();
        store_row_chunks<OVEC16, OCH>(packed + t * row_bytes, t < T ? row_bytes : 0, orow);
    };

    // Whole pairs of rows: a row at or past T reads zeros and drops its
    // stores, so no load or store is conditional and the compiler's
    // memory-counter waits stay exact.
    const int64_t G = gridDim.x;
    int64_t t = blockIdx.x;
    load_row_chunks<true, CH>(bufA, kv + t * C, t < T ? in_bytes : 0);
    __builtin_amdgcn_sched_barrier(0);      // keep the two rows' loads in this order
    load_row_chunks<true, CH>(bufB, kv + (t + G) * C, t + G < T ? in_bytes : 0);
    for (; t < T; t += 2 * G) {
        process(bufA, t);
        process(bufB, t + G);
    }
}

template <int BITS, int UPL, bool VEC16>
__global__ __launch_bounds__(kMaxBlock) void kv_dequant_kernel(
    const uint8_t* __restrict__ packed, int64_t T, int32_t C, const int32_t* __restrict__ R,
    const ClusterArgs ca, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CB = VEC16 ? 16 : 4;
    constexpr int CH = chunks_for<VEC16>(UPL * BITS);         // packed row: C*BITS/8 bytes
    constexpr int OCH = UPL;                                  // fp16 row: C/8 chunks
    const int BLOCK = blockDim.x;
    const int64_t row_bytes = (int64_t)C * BITS / 8;
    const int64_t out_bytes = (int64_t)C * 2;
    unsigned char* prow = smem;                               // CH * CB * BLOCK bytes
    unsigned char* orow = prow + (size_t)CH * CB * BLOCK;     // OCH * 16 * BLOCK bytes
    unsigned char* dummy = orow + (size_t)OCH * 16 * BLOCK;   // 16 bytes
    const int tid = threadIdx.x;
    const int n_units = C / 8;

    int dst[UPL][8], uib[UPL];
    float sc[UPL][8], zf[UPL][8];
    {
        int zi[UPL][8];
        kv_unit_tables<BITS, UPL>(ca, R, C, n_units, false, dst, sc, zi);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int unit = tid + u * BLOCK;
            const bool live = unit < n_units;
            uib[u] = live ? UnitGeom<BITS>::out_byte(unit) : 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dst[u][e] = live ? dst[u][e] * 2 : (int)(dummy - orow);
                zf[u][e] = (float)zi[u][e];      // |z| <= 2^21: exact
            }
        }
    }

    chunk_t<VEC16> bufA[CH], bufB[CH];
    auto process = [&](chunk_t<VEC16> (&buf)[CH], int64_t t) {
        put_row_chunks<VEC16, CH>(prow, buf);
        __syncthreads();
        const int64_t tn = t + 2 * (int64_t)gridDim.x;
        load_row_chunks<VEC16, CH>(buf, packed + tn * row_bytes, tn < T ? row_bytes : 0);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            int q[8];
            load_unit_at<BITS>(prow + uib[u], q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // (q - z) is an exact integer in fp32; the product is rounded
                // once, straight to fp16 (v_fma_mixlo_f16: fused, half to even)
                const float d = (float)q[e] - zf[u][e];
                *reinterpret_cast<_Float16*>(orow + dst[u][e]) = (_Float16)(sc[u][e] * d);
            }
        }
        __syncthreads();
        store_row_chunks<true, OCH>(out + t * C, t < T ? out_bytes : 0, orow);
    };

    const int64_t G = gridDim.x;
    int64_t t = blockIdx.x;
    load_row_chunks<VEC16, CH>(bufA, packed + t * row_bytes, t < T ? row_bytes : 0);
    __builtin_amdgcn_sched_barrier(0);      // keep the two rows' loads in this order
    load_row_chunks<VEC16, CH>(bufB, packed + (t + G) * row_bytes, t + G < T ? row_bytes : 0);
    for (; t < T; t += 2 * G) {
        process(bufA, t);
        process(bufB, t + G);
    }
}

template <int BITS, bool V>
const void* pick_quant_v(int upl) {
    // workgroups of up to kKvPackMaxBlock lanes: at most two units per lane
    // for any row of up to kMaxK channels
    switch (upl) {
        case 1: return (const void*)kv_quant_pack_kernel<BITS, 1, V>;
        case 2: return (const void*)kv_quant_pack_kernel<BITS, 2, V>;
        default: return nullptr;
    }
}

template <int BITS, bool V>
const void* pick_dequant_v(int upl) {
    switch (upl) {
        case 1: return (const void*)kv_dequant_kernel<BITS, 1, V>;
        case 2: return (const void*)kv_dequant_kernel<BITS, 2, V>;
        case 3: return (const void*)kv_dequant_kernel<BITS, 3, V>;
        case 4: return (const void*)kv_dequant_kernel<BITS, 4, V>;
        case 5: return (const void*)kv_dequant_kernel<BITS, 5, V>;
        default: return nullptr;
    }
}

template <bool QUANT>
const void* pick(int bits, int upl, bool v16) {
    if (QUANT) {
        if (bits == 3) return v16 ? pick_quant_v<3, true>(upl) : pick_quant_v<3, false>(upl);
        if (bits == 4) return v16 ? pick_quant_v<4, true>(upl) : pick_quant_v<4, false>(upl);
        return v16 ? pick_quant_v<8, true>(upl) : pick_quant_v<8, false>(upl);
    }
    if (bits == 3) return v16 ? pick_dequant_v<3, true>(upl) : pick_dequant_v<3, false>(upl);
    if (bits == 4) return v16 ? pick_dequant_v<4, true>(upl) : pick_dequant_v<4, false>(upl);
    return v16 ? pick_dequant_v<8, true>(upl) : pick_dequant_v<8, false>(upl);
}

// LDS bytes: the fp16 row and the packed row, each rounded up to whole lanes
// x chunks, plus the 16-byte dummy slot.
size_t kv_lds(int bits, int upl, int block, bool v16) {
    const int cb = v16 ? 16 : 4;
    const int pch = v16 ? (upl * bits + 15) / 16 : (upl * bits + 3) / 4;
    return (size_t)upl * 16 * block + (size_t)pch * cb * block + 16;
}

}  // namespace

// One workgroup per compute unit: a plain stream with this 5.3 : 1 read :
// write mix runs faster with fewer rows in flight (fewer concurrent streams
// for the memory controllers), and the pack's per-row work is light enough
// for one wide workgroup (2 units per lane) to keep its rows moving.
int stream_grid(int64_t rows) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return (int)std::max<int64_t>(1, std::min<int64_t>(cus, rows));
}

hipError_t launch_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R,
                                const ClusterArgs& ca, uint8_t* packed, hipStream_t stream) {
    int upl = 0, block = 0;
    unit_split(C / 8, upl, block, kKvPackMaxBlock);
    const bool v16 = ((int64_t)C * ca.bits / 8) % 16 == 0;
    const void* k = pick<true>(ca.bits, upl, v16);
    if (!k) return hipErrorInvalidValue;
    const size_t lds = kv_lds(ca.bits, upl, block, v16);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int grid = stream_grid(T);
    void* args[] = {(void*)&kv, (void*)&T, (void*)&C, (void*)&R, (void*)&ca, (void*)&packed};
    return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, stream);
}

hipError_t launch_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R,
                             const ClusterArgs& ca, uint16_t* out, hipStream_t stream) {
    int upl = 0, block = 0;
    unit_split(C / 8, upl, block);
    const bool v16 = ((int64_t)C * ca.bits / 8) % 16 == 0;
    const void* k = pick<false>(ca.bits, upl, v16);
    if (!k) return hipErrorInvalidValue;
    const size_t lds = kv_lds(ca.bits, upl, block, v16);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    // one workgroup per compute unit as well (three units per lane)
    const int grid = stream_grid(T);
    void* args[] = {(void*)&packed, (void*)&T, (void*)&C, (void*)&R, (void*)&ca, (void*)&out};
    return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, stream);
}

}  // namespace rptq
