// Device-side helpers shared by the library's HIP kernels (gfx950, wave64).
#pragma once

#include <cstdint>
#include <type_traits>
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "rptq_internal.h"

namespace rptq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache policy of the streaming kernels' row loads and stores: non-temporal
// (each byte is touched once, so it should not displace reusable lines or
// leave dirty lines behind for the next kernel to write back).
constexpr int kStreamPolicy = 2;

// Raw buffer resource over [base, base + bytes): loads past the end read as
// zero and stores past the end are dropped (range check in hardware).
constexpr uint32_t kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

// Code of one value v with a cluster's fp32 reciprocal scale inv_s and
// zb = z - kRoundMagicBits:
//   u = fl(v * inv_s + 1.5*2^23)    one rounding of the exact product: for
//                                   |v*inv_s| <= 2^22 this is 1.5*2^23 +
//                                   rne(v*inv_s), held in the low mantissa bits
//   clamp u to [2^23, 2^24]         |v*inv_s| >= 2^22 saturates (|z| <= 2^21
//                                   makes the final clip decide those anyway)
//   q = clip(bits(u) - bits(1.5*2^23) + z, 0, qmax)
__device__ __forceinline__ int quant_code(float v, float inv_s, int zb, int qmax) {
    float u = __builtin_fmaf(v, inv_s, kRoundMagic);
    u = __builtin_amdgcn_fmed3f(u, 8388608.0f, 16777216.0f);
    const int k = __builtin_bit_cast(int, u) + zb;
    return __builtin_elementwise_max(__builtin_elementwise_min(k, qmax), 0);
}

// The same code, left in the low bits of a float's bit pattern: with
// zf = (float)z and hi = 1.5*2^23 + qmax,
//   u = fl(v * inv_s + 1.5*2^23)    the exact product rounded once to an
//                                   integer (ties to even: 1.5*2^23 is even)
//   u + zf                          exact (integers below 2^24)
//   clamp to [1.5*2^23, hi]         saturates both ways, q = bits - bits(1.5*2^23)
// The low 22 bits of the result are q (the constant's are zero), so packing
// can take the code's byte without masking.
__device__ __forceinline__ uint32_t quant_bits(float v, float inv_s, float zf, float hi) {
    const float u = __builtin_fmaf(v, inv_s, kRoundMagic) + zf;
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(u, kRoundMagic, hi));
}

// Wave64 sum.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait until this wave has at most n vector-memory operations pending
// (loads, including loads that write LDS, and stores complete in issue order).
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, its memory loads may still be in flight (a full __syncthreads
// would also wait for every prefetch).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over a 256-thread workgroup; `scratch` holds 4 floats.  Ends with a
// barrier, so `scratch` may be reused right after.
__device__ __forceinline__ float block_sum_256(float v, float* scratch) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) scratch[w] = v;
    __syncthreads();
    const float t = scratch[0] + scratch[1] + scratch[2] + scratch[3];
    __syncthreads();
    return t;
}

constexpr int kCalibBlock = 256;

// Positions of the 8 codes a "unit" covers, in a row laid out in groups (see
// rptq.h).  For 4- and 8-bit rows a unit is 8 consecutive codes; for 3-bit
// rows a unit is byte lane `bl` of a 32-code group: codes bl, bl+4, ..., bl+28.
template <int BITS>
struct UnitGeom {
    __device__ __forceinline__ static int first(int unit) {
        return BITS == 3 ? 32 * (unit >> 2) + (unit & 3) : 8 * unit;
    }
    static constexpr int stride = BITS == 3 ? 4 : 1;
    // byte offset of the unit's first output byte in the packed row
    __device__ __forceinline__ static int out_byte(int unit) {
        return BITS == 3 ? 12 * (unit >> 2) + (unit & 3) : unit * BITS;
    }
};

// Pack the 8 codes of a unit (q[e] is the code at position first + e*stride)
// and store them at p, the unit's first output byte in a packed row (LDS).
template <int BITS>
__device__ __forceinline__ void store_unit_at(unsigned char* p, const int (&q)[8]) {
    if constexpr (BITS == 8) {
        uint2 v;
        v.x = (uint32_t)q[0] | (uint32_t)q[1] << 8 | (uint32_t)q[2] << 16 | (uint32_t)q[3] << 24;
        v.y = (uint32_t)q[4] | (uint32_t)q[5] << 8 | (uint32_t)q[6] << 16 | (uint32_t)q[7] << 24;
        *reinterpret_cast<uint2*>(p) = v;
    } else if constexpr (BITS == 4) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) v |= ((uint32_t)q[i] | (uint32_t)q[4 + i] << 4) << (8 * i);
        *reinterpret_cast<uint32_t*>(p) = v;
    } else {
        // byte lane of words d0, d1, d2 of the 32-code group
        p[0] = (unsigned char)(q[0] | q[1] << 3 | (q[6] & 3) << 6);
        p[4] = (unsigned char)(q[2] | q[3] << 3 | (q[7] & 3) << 6);
        p[8] = (unsigned char)(q[4] | q[5] << 3 | (q[6] >> 2) << 6 | (q[7] >> 2) << 7);
    }
}

template <int BITS>
__device__ __forceinline__ void store_unit(unsigned char* out, int unit, const int (&q)[8]) {
    store_unit_at<BITS>(out + UnitGeom<BITS>::out_byte(unit), q);
}

// Pack the 8 codes of a unit given as quant_bits results (low bits = code)
// and store them at p (LDS), in the layout of store_unit_at.
template <int BITS>
__device__ __forceinline__ void store_unit_bits(unsigned char* p, const uint32_t (&b)[8]) {
    // byte 0 of each of four words -> one word (v_perm_b32 picks bytes of
    // its two sources; selector 0x0c yields a zero byte)
    auto gather4 = [](uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
        return __builtin_amdgcn_perm(w1, w0, 0x0C0C0400u) | __builtin_amdgcn_perm(w3, w2, 0x04000C0Cu);
    };
    if constexpr (BITS == 8) {
        *reinterpret_cast<uint2*>(p) = uint2{gather4(b[0], b[1], b[2], b[3]), gather4(b[4], b[5], b[6], b[7])};
    } else if constexpr (BITS == 4) {
        const uint32_t lo = gather4(b[0], b[1], b[2], b[3]), hi = gather4(b[4], b[5], b[6], b[7]);
        *reinterpret_cast<uint32_t*>(p) = lo | hi << 4;
    } else {
        int q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (int)(b[e] & 7u);
        store_unit_at<3>(p, q);
    }
}

// Row transfers with buffer instructions that every lane executes (accesses
// past `bytes` read zeros / are dropped by the buffer range check), so the
// compiler's memory-counter waits stay exact.  Chunk i of lane t is chunk
// t + i * blockDim.x of the row; chunks are 16 bytes (VEC16) or 4 bytes, and
// `bytes` must be a multiple of the chunk size.
template <bool VEC16>
using chunk_t = typename std::conditional<VEC16, u32x4, uint32_t>::type;

template <bool VEC16, int N>
__device__ __forceinline__ void load_row_chunks(chunk_t<VEC16> (&buf)[N], const void* base, int64_t bytes) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
    const int tid = threadIdx.x, nt = blockDim.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (VEC16)
            buf[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(tid + i * nt) * 16u, 0, kStreamPolicy);
        else
            buf[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)(tid + i * nt) * 4u, 0, kStreamPolicy);
    }
}

template <bool VEC16, int N>
__device__ __forceinline__ void put_row_chunks(unsigned char* lds, const chunk_t<VEC16> (&buf)[N]) {
    const int tid = threadIdx.x, nt = blockDim.x;
#pragma unroll
    for (int i = 0; i < N; ++i) reinterpret_cast<chunk_t<VEC16>*>(lds)[tid + i * nt] = buf[i];
}

template <bool VEC16, int N>
__device__ __forceinline__ void store_row_chunks(void* base, int64_t bytes, const unsigned char* lds) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
    const int tid = threadIdx.x, nt = blockDim.x;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int c = tid + i * nt;
        if constexpr (VEC16)
            __builtin_amdgcn_raw_buffer_store_b128(reinterpret_cast<const u32x4*>(lds)[c], r, (uint32_t)c * 16u, 0, kStreamPolicy);
        else
            __builtin_amdgcn_raw_buffer_store_b32(reinterpret_cast<const uint32_t*>(lds)[c], r, (uint32_t)c * 4u, 0, kStreamPolicy);
    }
}

// Chunks per lane that cover `bytes_per_lane` bytes.
template <bool VEC16>
__host__ __device__ constexpr int chunks_for(int bytes_per_lane) {
    return VEC16 ? (bytes_per_lane + 15) / 16 : (bytes_per_lane + 3) / 4;
}

// Inverse of store_unit_at: the 8 codes of a unit whose first byte is at p.
template <int BITS>
__device__ __forceinline__ void load_unit_at(const unsigned char* p, int (&q)[8]) {
    const unsigned char* in = p;
    constexpr int ob = 0;
    if constexpr (BITS == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(in + ob);
#pragma unroll
        for (int i = 0; i < 4; ++i) { q[i] = (v.x >> (8 * i)) & 255; q[4 + i] = (v.y >> (8 * i)) & 255; }
    } else if constexpr (BITS == 4) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(in + ob);
#pragma unroll
        for (int i = 0; i < 4; ++i) { q[i] = (v >> (8 * i)) & 15; q[4 + i] = (v >> (8 * i + 4)) & 15; }
    } else {
        const int b0 = in[ob], b1 = in[ob + 4], b2 = in[ob + 8];
        q[0] = b0 & 7; q[1] = (b0 >> 3) & 7;
        q[2] = b1 & 7; q[3] = (b1 >> 3) & 7;
        q[4] = b2 & 7; q[5] = (b2 >> 3) & 7;
        q[6] = (b0 >> 6) | ((b2 >> 6) & 1) << 2;
        q[7] = (b1 >> 6) | ((b2 >> 7) & 1) << 2;
    }
}

// Cluster holding reordered (unpadded) position j.
// Cluster lookups for a kernel's set-up, without chains of dependent loads:
// lane c (< g) of every wave holds cluster c's table entries (one load per
// lane, all independent), a position's cluster is the number of later
// cluster starts at or below it (starts read with v_readlane at a uniform
// index), and its entries come from lane c over the lane crossbar.
struct LaneClusters {
    int start;       // bounds[c] (DENSE positions) or off[c] (SEG32 positions)
    int bound;       // bounds[c]
    int off;         // off[c]
    float inv_s;
    float s;
    int z;
};
__device__ __forceinline__ LaneClusters lane_clusters(const ClusterArgs& ca, bool seg32) {
    const int l = threadIdx.x & 63;
    const int c = l < ca.g ? l : ca.g - 1;
    LaneClusters t;
    t.bound = ca.bounds[c];
    t.off = ca.off[c];
    t.start = seg32 ? t.off : t.bound;
    if (l >= ca.g) t.start = 0x7fffffff;
    t.inv_s = ca.inv_s[c];
    t.s = ca.s[c];
    t.z = ca.z[c];
    return t;
}
// clusters of N positions q[] (same for every lane pattern: any lane values)
template <int N>
__device__ __forceinline__ void clusters_of(const LaneClusters& t, int g, const int (&q)[N], int (&c)[N]) {
#pragma unroll
    for (int n = 0; n < N; ++n) c[n] = 0;
    for (int k = 1; k < g; ++k) {
        const int st = __builtin_amdgcn_readlane(t.start, k);
#pragma unroll
        for (int n = 0; n < N; ++n) c[n] += q[n] >= st ? 1 : 0;
    }
}
// (every lane of the wave must execute it: a lane that does not run the
// crossbar read supplies no value to the lanes that read from it)
template <class T>
__device__ __forceinline__ T from_lane(T v, int c) {
    return __builtin_bit_cast(T, __shfl(__builtin_bit_cast(int, v), c, 64));
}

__device__ __forceinline__ int cluster_of_pos(const ClusterArgs& ca, int j) {
    int c = 0;
    while (c + 1 < ca.g && j >= ca.bounds[c + 1]) ++c;
    return c;
}

// Cluster holding SEG32 padded position p.
__device__ __forceinline__ int cluster_of_padded(const ClusterArgs& ca, int p) {
    int c = 0;
    while (c + 1 < ca.g && p >= ca.off[c + 1]) ++c;
    return c;
}

// Copy `bytes` (a multiple of 4) from LDS to global memory with the whole
// workgroup; 16-byte stores when both ends allow it.
__device__ __forceinline__ void store_row(uint8_t* __restrict__ dst, const unsigned char* src,
                                          int64_t bytes) {
    if ((bytes & 15) == 0 && ((uintptr_t)dst & 15) == 0) {
        const int n = (int)(bytes >> 4);
        for (int i = threadIdx.x; i < n; i += blockDim.x)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        const int n = (int)(bytes >> 2);
        for (int i = threadIdx.x; i < n; i += blockDim.x)
            reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
    }
}

}  // namespace rptq
