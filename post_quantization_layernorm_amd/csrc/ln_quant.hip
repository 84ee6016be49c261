// Fused LayerNorm + reorder + per-cluster quantize + SEG32 pack (gfx950).
//
// RPTQ write-up, method section and Fig. 3: LayerNorm is changed to emit the
// reordered activations directly, so the reorder costs no extra pass or
// buffer; each cluster of reordered channels has its own (s, z).  The kernel
// is HBM-bound: it reads fp16 [M][K] once and writes b-bit codes once.
//
// Design (persistent workgroups, one row at a time per workgroup):
//   - the workgroup size (a multiple of 64) is chosen so that each lane owns
//     few "units" (8 output codes each); a lane keeps, for all rows, the
//     source channel R[j], gamma'[j], beta'[j] of its units and the cluster's
//     (1/s, z) in registers;
//   - rows are read with 16-byte buffer loads into two register buffers, so
//     two rows per workgroup are in flight while one is quantized.  Every
//     memory instruction runs unconditionally (lanes past the row end read
//     zeros / have their stores dropped by the buffer range check), which
//     keeps the compiler's memory-counter waits exact: a row's wait never
//     covers the next row's loads;
//   - mean and biased variance come from packed-fp16 dot products
//     (sum x and sum x^2 in fp32, one VALU op per element) and one
//     wave-shuffle + LDS reduction; if more than 6 bits would cancel in
//     E[x^2] - E[x]^2, an exact second pass around the mean is taken;
//   - the row is parked in LDS in natural order; each unit gathers its 8
//     inputs by R, normalizes, quantizes and packs them into an LDS copy of
//     the output row, which is written with 16-byte stores.
#include <mutex>

#include "rptq_device.hpp"
#include "../../include/rptq.h"

// Partials of the dynamic-range ranges pass for callers that cannot allocate
// (allocation-free entry point): one (lo, hi) pair per cluster for each of at
// most kLnRangesMaxGrid workgroups, 512 KB.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never uses this name
// as an address: ln_dynamic_scratch() looks the device address up once per
// device (hipGetSymbolAddress) and hands that out.
static __device__ __align__(256) float scratch[rptq::kLnRangesMaxGrid * 2 * rptq::kMaxClusters];

namespace rptq {
namespace {

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 0) red[w] = v;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < nw; ++i) t += red[i];
    __syncthreads();
    return t;
}

// Dynamic ranges (quantization lecture 1.1: the scale is decided at run time
// from the current activations): cluster c's (s, z) from lo = min, hi = max
// of the batch's values over the cluster's channels, by the same rules as the
// calibrated parameters (s = (hi - lo)/qmax in fp32, floored at
// max(|lo|, |hi|) 2^-21, 1 for an all-zero cluster; z = rne(-lo/s)).
__device__ __forceinline__ void dynamic_params(float lo, float hi, int qmax, float& s, int32_t& z) {
    const double dlo = lo, dhi = hi;
    float sc = (float)((dhi - dlo) / (double)qmax);
    const float fl = (float)(__builtin_fmax(__builtin_fabs(dlo), __builtin_fabs(dhi)) * 0x1p-21);
    if (sc < fl) sc = fl;
    if (sc == 0.0f) sc = 1.0f;
    s = sc;
    z = (int32_t)__builtin_rint(-dlo / (double)sc);
}

// DM (dynamic mode): kStatic quantizes with the (s, z) of the cluster table;
// kRanges writes no codes, only this workgroup's min and max of every
// cluster over its rows (dyn_a[blockIdx][0..g) = lo, [g..2g) = hi);
// kDevParams quantizes with the (s, z) in dyn_a / dyn_b (device memory).
enum { kStatic = 0, kRanges = 1, kDevParams = 2 };

template <int BITS, int MODE, int UPL, int DM>
__global__ __launch_bounds__(kMaxBlock) void ln_reorder_quant_kernel(
    const void* __restrict__ xin, int64_t M, int32_t K, int64_t row_bytes,
    const float* __restrict__ gamma_r, const float* __restrict__ beta_r, float eps,
    const int32_t* __restrict__ R, const ClusterArgs ca, uint8_t* __restrict__ codes,
    float* __restrict__ dyn_a, int32_t* __restrict__ dyn_b) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int QMAX = (1 << BITS) - 1;
    constexpr bool LN = MODE == RPTQ_IN_FP16_RAW;
    constexpr int ESZ = LN ? 2 : 4;                       // bytes per input element
    // 16-byte input chunks per lane: a row has K*ESZ/16 chunks and at least
    // K/8 units, so ESZ/2 * UPL chunks per lane always suffice
    constexpr int CH = UPL * ESZ / 2;
    // 16-byte output chunks per lane: a packed row has at most units*BITS bytes
    constexpr int OCH = (UPL * BITS + 15) / 16;
    const int BLOCK = blockDim.x;
    const int row_in_bytes = K * ESZ;
    // LDS: input row (rounded up to whole lanes x chunks), output row, a
    // dummy slot for idle units, reduction scratch
    unsigned char* xrow = smem;
    unsigned char* orow = smem + (size_t)CH * 16 * BLOCK;
    unsigned char* dummy = orow + (size_t)OCH * 16 * BLOCK;
    float* red = reinterpret_cast<float*>(dummy + 16);
    // ranges: per 32-code group (lo, hi)
    float* glo = red + 64;
    float* ghi = glo + ca.K_pad / 32;
    const int tid = threadIdx.x;
    const int n_units = ca.K_pad / 8;
    const int nchunks = row_in_bytes / 16;

    // ---- per-lane unit tables (fixed for every row); idle units gather
    // element 0 and write to the dummy slot.  A padding position (past its
    // cluster's end) gets gamma 0 and beta -FLT_MAX, so its code saturates to
    // 0 without a select (in quant-only mode its value is replaced the same way).
    constexpr float kPad = -3.0e38f;
    int src[UPL][8];
    float gam[UPL][8], bet[UPL][8];
    float uinv[UPL], uzf[UPL];
    int uob[UPL];
    // every unit's cluster first (no dependent memory access), then the table
    // loads all at once, then the padding / idle selections as arithmetic on
    // the loaded values (a select of a loaded value would be turned into a
    // branch around its load, one load and wait at a time): 1 * x + 0 = x,
    // 0 * x + kPad = kPad.  A padding or idle position reads a valid index;
    // gamma 0 and beta kPad decide its code.
    const LaneClusters lc = lane_clusters(ca, true);
    int ucl[UPL], up0[UPL];
#pragma unroll
    for (int u = 0; u < UPL; ++u) up0[u] = UnitGeom<BITS>::first(tid + u * BLOCK);
    clusters_of<UPL>(lc, ca.g, up0, ucl);
    int jb[UPL];                                 // reordered index of element 0
    float um[UPL][8];                            // 1: real position, 0: padding / idle
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int unit = tid + u * BLOCK;
        const bool live = unit < n_units;
        const int c = ucl[u];
        // cluster c's entries, fetched by every lane: a crossbar read takes
        // its value from the source lane only if that lane runs it too, so
        // none of these sits under a condition
        const int cb = from_lane(lc.bound, c), co = from_lane(lc.off, c);
        const int nb = from_lane(lc.bound, c + 1 < ca.g ? c + 1 : c);
        const int cn = c + 1 < ca.g ? nb : ca.K;
        const float cinv = from_lane(lc.inv_s, c);
        const int cz = from_lane(lc.z, c);
        if constexpr (DM == kDevParams) {
            // (loaded for every lane: c is a valid cluster for idle units too)
            const float ds = dyn_a[c];
            const int dz = dyn_b[c];
            uinv[u] = live ? 1.0f / ds : 0.0f;       // correctly rounded, as on the host
            uzf[u] = live ? (float)dz : 0.0f;
        } else {
            uinv[u] = live ? cinv : 0.0f;
            uzf[u] = live ? (float)cz : 0.0f;        // |z| <= 2^21: exact
        }
        uob[u] = live ? UnitGeom<BITS>::out_byte(unit) : (int)(dummy - orow);
        const int i0 = up0[u] - co;                  // >= 0 for a live unit
        jb[u] = live ? cb + i0 : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            um[u][e] = live && i0 + e * UnitGeom<BITS>::stride < cn - cb ? 1.0f : 0.0f;
    }
    if constexpr (LN) {
        // indices past K read zeros (range check); a NULL R reads zeros
        // through a zero-byte descriptor and is replaced by the index itself
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(R, R ? (int64_t)K * 4 : 0);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma_r, (int64_t)K * 4);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(beta_r, (int64_t)K * 4);
        const bool has_r = R != nullptr;
        if constexpr (UnitGeom<BITS>::stride != 1) {
#pragma unroll
            for (int u = 0; u < UPL; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t off = (uint32_t)(jb[u] + e * UnitGeom<BITS>::stride) * 4u;
                    src[u][e] = (int)__builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, 0);
                    gam[u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, off, 0, 0));
                    bet[u][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0));
                }
        }
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            int rv[8];
            float gv[8], bv[8];
            if constexpr (UnitGeom<BITS>::stride == 1) {
                // 8 consecutive indices: two 16-byte loads per table
                const uint32_t off = (uint32_t)jb[u] * 4u;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 r4 = __builtin_amdgcn_raw_buffer_load_b128(rr, off + 16 * h, 0, 0);
                    const u32x4 g4 = __builtin_amdgcn_raw_buffer_load_b128(rg, off + 16 * h, 0, 0);
                    const u32x4 b4 = __builtin_amdgcn_raw_buffer_load_b128(rb, off + 16 * h, 0, 0);
                    const uint32_t rs[4] = {r4.x, r4.y, r4.z, r4.w}, gs[4] = {g4.x, g4.y, g4.z, g4.w},
                                   bs[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        rv[4 * h + k] = (int)rs[k];
                        gv[4 * h + k] = __builtin_bit_cast(float, gs[k]);
                        bv[4 * h + k] = __builtin_bit_cast(float, bs[k]);
                    }
                }
            } else {
                // strided positions: one load per position and table, issued
                // for every unit before the first is used (below)
#pragma unroll
                for (int e = 0; e < 8; ++e) { rv[e] = src[u][e]; gv[e] = gam[u][e]; bv[e] = bet[u][e]; }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = jb[u] + e * UnitGeom<BITS>::stride;
                const int k = j + (has_r ? rv[e] - j : 0);
                src[u][e] = (k < K ? k : 0) * 2;
                if constexpr (DM == kRanges) {
                    // ranges pass: a padding position repeats element 0 of its
                    // unit (real whenever the unit has a real position), which
                    // leaves the unit's min and max unchanged
                    const float m = um[u][e];
                    src[u][e] = m != 0.0f ? src[u][e] : src[u][0];
                    gam[u][e] = __builtin_fmaf(gv[e], m, gv[0] * (1.0f - m));
                    bet[u][e] = __builtin_fmaf(bv[e], m, bv[0] * (1.0f - m));
                } else {
                    gam[u][e] = gv[e] * um[u][e];
                    bet[u][e] = __builtin_fmaf(bv[e], um[u][e], um[u][e] != 0.0f ? 0.0f : kPad);
                }
            }
        }
    } else {
#pragma unroll
        for (int u = 0; u < UPL; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = jb[u] + e * UnitGeom<BITS>::stride;
                src[u][e] = (j < K ? j : 0) * 4;
                if constexpr (DM == kRanges) {
                    // padding repeats element 0 of the unit (see above)
                    src[u][e] = um[u][e] != 0.0f ? src[u][e] : src[u][0];
                    gam[u][e] = 1.0f;
                    bet[u][e] = 0.0f;
                } else {
                    gam[u][e] = um[u][e];
                    bet[u][e] = um[u][e] != 0.0f ? 0.0f : kPad;
                }
            }
    }
    // LayerNorm mode, quantizing passes: gamma' and beta' carry the unit's
    // 1/s, so fma(gamma'/s, n, beta'/s) is y/s (one more rounding than
    // forming y first, well inside the code tolerance of the fused path) and
    // the code is its sum with 1.5 * 2^23 + z (rounded to an integer, ties to
    // even) clamped: one op less per element.  (Quant-only mode keeps the
    // single rounding of y * (1/s).)
    [[maybe_unused]] float umz[UPL];
    if constexpr (LN && DM != kRanges) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            umz[u] = kRoundMagic + uzf[u];            // exact: |z| <= 2^21
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gam[u][e] *= uinv[u];
                bet[u][e] *= uinv[u];
            }
        }
    }
    // units holding at least one real position (bit u)
    uint32_t ureal = 0;
#pragma unroll
    for (int u = 0; u < UPL; ++u) ureal |= um[u][0] != 0.0f ? 1u << u : 0u;
    const float qhi = kRoundMagic + (float)QMAX;
    [[maybe_unused]] float ulo[UPL], uhi[UPL];
#pragma unroll
    for (int u = 0; u < UPL; ++u) { ulo[u] = __builtin_inff(); uhi[u] = -__builtin_inff(); }

    // Two register buffers: while row r (in one) is processed, rows r + G and
    // r + 2G are in flight (G = gridDim.x).  Rows at or past M are read as
    // zeros and their stores dropped (descriptor of zero bytes), so every
    // workgroup runs whole pairs of rows and no load or store is conditional.
    u32x4 bufA[CH], bufB[CH];
    auto load_row = [&](u32x4 (&buf)[CH], int64_t row) {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(static_cast<const uint8_t*>(xin) + row * row_in_bytes, row < M ? row_in_bytes : 0);
#pragma unroll
        for (int i = 0; i < CH; ++i)
            buf[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(tid + i * BLOCK) * 16u, 0, kStreamPolicy);
    };

    // Two barriers per row: (1) the row and the per-wave partial sums are in
    // LDS; (2) the packed output row is in LDS (and every lane is done
    // reading the input row and the partial sums).
    const int lane = tid & 63, wv = tid >> 6, nw = BLOCK >> 6;
    auto process = [&](u32x4 (&buf)[CH], int64_t row) {
        float s1 = 0.0f, s2 = 0.0f;
        if constexpr (LN) {
            // sum x and sum x^2 from packed fp16 dot products (exact
            // products, fp32 accumulation); chunks past the row are zeros
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const uint32_t w[4] = {buf[i].x, buf[i].y, buf[i].z, buf[i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const half2_t h = __builtin_bit_cast(half2_t, w[k]);
                    s1 = __builtin_amdgcn_fdot2(h, one2, s1, false);
                    s2 = __builtin_amdgcn_fdot2(h, h, s2, false);
                }
            }
            s1 = wave_sum(s1);
            s2 = wave_sum(s2);
            if (lane == 0) { red[2 * wv] = s1; red[2 * wv + 1] = s2; }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) reinterpret_cast<u32x4*>(xrow)[tid + i * BLOCK] = buf[i];
        __syncthreads();

        float mean = 0.0f, rstd = 0.0f;
        if constexpr (LN) {
            s1 = 0.0f; s2 = 0.0f;
            for (int i = 0; i < nw; ++i) { s1 += red[2 * i]; s2 += red[2 * i + 1]; }
            const float m1 = s1 / (float)K, m2 = s2 / (float)K;
            float var = m2 - m1 * m1;
            mean = m1;
            if (!(var > m2 * 0.015625f)) {
                // more than 6 bits would cancel (|mean| >> spread, or a
                // constant row): exact second pass around the mean
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
                ss = block_sum(ss, red + 32);
                var = ss / (float)K;
            }
            rstd = 1.0f / __builtin_sqrtf(var + eps);
        }
        load_row(buf, row + 2 * (int64_t)gridDim.x);

        const float nmr = -mean * rstd;
        auto y_of = [&](int u, int e) {
            if constexpr (LN) {
                const float xv = (float)*reinterpret_cast<const _Float16*>(xrow + src[u][e]);
                const float n = __builtin_fmaf(xv, rstd, nmr);
                return __builtin_fmaf(gam[u][e], n, bet[u][e]);
            } else {
                return __builtin_fmaf(gam[u][e], *reinterpret_cast<const float*>(xrow + src[u][e]), bet[u][e]);
            }
        };
        if constexpr (DM == kRanges) {
            // running (lo, hi) of every unit over the rows (padding
            // positions repeat a real one; units without any are reset after
            // the last row); rows past M add nothing
            if (row < M) {
#pragma unroll
                for (int u = 0; u < UPL; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float y = y_of(u, e);
                        ulo[u] = __builtin_fminf(ulo[u], y);
                        uhi[u] = __builtin_fmaxf(uhi[u], y);
                    }
            }
            __syncthreads();          // every lane is done with the row and the sums
            return;
        } else {
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                uint32_t qb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (LN) {
                        const float t = y_of(u, e) + umz[u];      // y_of gives y / s here
                        qb[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(t, kRoundMagic, qhi));
                    } else {
                        qb[e] = quant_bits(y_of(u, e), uinv[u], uzf[u], qhi);
                    }
                }
                store_unit_bits<BITS>(orow + uob[u], qb);
            }
        }
        if constexpr (DM != kRanges) {
            __syncthreads();
            // row_bytes is the row pitch; the row's K_pad * BITS / 8 bytes are
            // stored (3-bit rows are a multiple of 12 bytes: 4-byte stores)
            store_row_chunks<BITS != 3, chunks_for<BITS != 3>(UPL * BITS)>(
                codes + row * row_bytes, row < M ? (int64_t)ca.K_pad * BITS / 8 : 0, orow);
        }
    };

    const int64_t G = gridDim.x;
    int64_t row = blockIdx.x;
    // (the second buffer is loaded first, matching the order in which the
    // loop body issues its prefetches, so the compiler's memory-counter
    // waits stay exact)
    load_row(bufB, row + G);
    load_row(bufA, row);
    for (; row < M; row += 2 * G) {
        process(bufA, row);
        process(bufB, row + G);
    }

    if constexpr (DM == kRanges) {
        // units -> 32-code groups (4 consecutive units in 4 consecutive
        // lanes) -> clusters (one wave per cluster at a time) -> this
        // workgroup's (lo, hi) per cluster; a unit without a real position
        // (idle, or all padding) takes no part
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const bool none = !(ureal >> u & 1u);
            float lo = none ? __builtin_inff() : ulo[u], hi = none ? -__builtin_inff() : uhi[u];
            lo = __builtin_fminf(lo, __shfl_xor(lo, 1, 64));
            hi = __builtin_fmaxf(hi, __shfl_xor(hi, 1, 64));
            lo = __builtin_fminf(lo, __shfl_xor(lo, 2, 64));
            hi = __builtin_fmaxf(hi, __shfl_xor(hi, 2, 64));
            const int unit = tid + u * BLOCK;
            if ((tid & 3) == 0 && unit < n_units) {
                glo[unit >> 2] = lo;
                ghi[unit >> 2] = hi;
            }
        }
        __syncthreads();
        for (int c = wv; c < ca.g; c += nw) {
            float lo = __builtin_inff(), hi = -__builtin_inff();
            for (int q = ca.off[c] / 32 + lane; q < ca.off[c + 1] / 32; q += 64) {
                lo = __builtin_fminf(lo, glo[q]);
                hi = __builtin_fmaxf(hi, ghi[q]);
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                lo = __builtin_fminf(lo, __shfl_xor(lo, o, 64));
                hi = __builtin_fmaxf(hi, __shfl_xor(hi, o, 64));
            }
            // (a workgroup without rows leaves (+inf, -inf))
            if (lane == 0) {
                dyn_a[(int64_t)blockIdx.x * 2 * ca.g + c] = lo;
                dyn_a[(int64_t)blockIdx.x * 2 * ca.g + ca.g + c] = hi;
            }
        }
    }
}

// Cluster c = blockIdx.x: (lo, hi) over the ranges pass's nparts workgroup
// partials, then (s, z).
template <int BITS>
__global__ __launch_bounds__(256) void dynamic_params_kernel(const float* __restrict__ part, int32_t nparts,
                                                             int32_t g, float* __restrict__ s_out,
                                                             int32_t* __restrict__ z_out) {
    __shared__ float red[8];
    const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int w = tid; w < nparts; w += 256) {
        lo = __builtin_fminf(lo, part[(int64_t)w * 2 * g + c]);
        hi = __builtin_fmaxf(hi, part[(int64_t)w * 2 * g + g + c]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = __builtin_fminf(lo, __shfl_xor(lo, o, 64));
        hi = __builtin_fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    if (lane == 0) { red[wv] = lo; red[4 + wv] = hi; }
    __syncthreads();
    if (tid == 0) {
        lo = __builtin_fminf(__builtin_fminf(red[0], red[1]), __builtin_fminf(red[2], red[3]));
        hi = __builtin_fmaxf(__builtin_fmaxf(red[4], red[5]), __builtin_fmaxf(red[6], red[7]));
        float sc;
        int32_t zc;
        dynamic_params(lo + 0.0f, hi + 0.0f, (1 << BITS) - 1, sc, zc);
        s_out[c] = sc;
        z_out[c] = zc;
    }
}

template <int BITS, int MODE, int DM>
const void* pick(int upl) {
    switch (upl) {
        case 1: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 1, DM>;
        case 2: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 2, DM>;
        case 3: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 3, DM>;
        case 4: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 4, DM>;
        case 5: return (const void*)ln_reorder_quant_kernel<BITS, MODE, 5, DM>;
        default: return nullptr;
    }
}

template <int DM>
const void* pick_mode(int in_mode, int bits, int upl) {
    if (in_mode == RPTQ_IN_FP16_RAW)
        return bits == 3 ? pick<3, 0, DM>(upl) : bits == 4 ? pick<4, 0, DM>(upl) : pick<8, 0, DM>(upl);
    return bits == 3 ? pick<3, 1, DM>(upl) : bits == 4 ? pick<4, 1, DM>(upl) : pick<8, 1, DM>(upl);
}

}  // namespace

namespace {

int launch_shape(int dm, int in_mode, const ClusterArgs& ca, int& upl, int& block, const void*& k,
                 size_t& lds) {
    unit_split(ca.K_pad / 8, upl, block, RPTQ_LN_MAX_BLOCK);
    k = dm == kRanges ? pick_mode<kRanges>(in_mode, ca.bits, upl)
        : dm == kDevParams ? pick_mode<kDevParams>(in_mode, ca.bits, upl)
                           : pick_mode<kStatic>(in_mode, ca.bits, upl);
    if (!k) return -1;
    const int esz = in_mode == RPTQ_IN_FP16_RAW ? 2 : 4;
    const int ch = upl * esz / 2, och = (upl * ca.bits + 15) / 16;
    // reduction scratch (64 floats), then (ranges pass) the (lo, hi) of every
    // 32-code group
    const size_t extra = 256 + (dm == kRanges ? (size_t)(2 * (ca.K_pad / 32)) * 4 : 0);
    lds = (size_t)ch * 16 * block + (size_t)och * 16 * block + 16 + extra;
    return 0;
}

hipError_t launch_mode(int dm, const void* x, int in_mode, int64_t M, int32_t K, const float* gamma_r,
                       const float* beta_r, float eps, const int32_t* R, const ClusterArgs& ca,
                       int64_t row_bytes, uint8_t* codes, float* dyn_a, int32_t* dyn_b, int max_grid,
                       hipStream_t stream, int* grid_out = nullptr) {
    int upl = 0, block = 0;
    const void* k = nullptr;
    size_t lds = 0;
    if (launch_shape(dm, in_mode, ca, upl, block, k, lds)) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    int grid = persistent_grid(k, block, lds, M);
    if (max_grid > 0 && grid > max_grid) grid = max_grid;
    if (grid_out) *grid_out = grid;
    void* args[] = {(void*)&x, (void*)&M, (void*)&K, (void*)&row_bytes, (void*)&gamma_r,
                    (void*)&beta_r, (void*)&eps, (void*)&R, (void*)&ca, (void*)&codes, (void*)&dyn_a,
                    (void*)&dyn_b};
    return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, stream);
}

}  // namespace

hipError_t launch_ln_reorder_quant(const void* x, int in_mode, int64_t M, int32_t K,
                                   const float* gamma_r, const float* beta_r, float eps,
                                   const int32_t* R, const ClusterArgs& ca, int64_t row_bytes,
                                   uint8_t* codes, hipStream_t stream) {
    return launch_mode(kStatic, x, in_mode, M, K, gamma_r, beta_r, eps, R, ca, row_bytes, codes, nullptr,
                       nullptr, 0, stream);
}

hipError_t launch_ln_reorder_quant_dynamic(const void* x, int in_mode, int64_t M, int32_t K,
                                           const float* gamma_r, const float* beta_r, float eps,
                                           const int32_t* R, const ClusterArgs& ca, int64_t row_bytes,
                                           uint8_t* codes, float* s_out, int32_t* z_out, float* partials,
                                           hipStream_t stream) {
    // three launches in stream order: per-workgroup (lo, hi) partials, the
    // clusters' (s, z), the quantizing pass
    int nparts = 0;
    hipError_t e = launch_mode(kRanges, x, in_mode, M, K, gamma_r, beta_r, eps, R, ca, row_bytes, codes, partials,
                               nullptr, kLnRangesMaxGrid, stream, &nparts);
    if (e != hipSuccess) return e;
    const int32_t g = ca.g;
    if (ca.bits == 3)
        dynamic_params_kernel<3><<<dim3(g), dim3(256), 0, stream>>>(partials, nparts, g, s_out, z_out);
    else if (ca.bits == 4)
        dynamic_params_kernel<4><<<dim3(g), dim3(256), 0, stream>>>(partials, nparts, g, s_out, z_out);
    else
        dynamic_params_kernel<8><<<dim3(g), dim3(256), 0, stream>>>(partials, nparts, g, s_out, z_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_mode(kDevParams, x, in_mode, M, K, gamma_r, beta_r, eps, R, ca, row_bytes, codes, s_out,
                       z_out, 0, stream);
}

int64_t ln_dynamic_scratch_bytes() { return (int64_t)sizeof(scratch); }

hipError_t ln_dynamic_scratch(void** ptr) {
    // device address of this GPU's copy of the array, looked up on the first
    // call with that device current and kept for the life of the process
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    *ptr = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace rptq
