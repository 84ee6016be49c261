// Decode attention that reads the packed K/V cache directly (gfx950).
//
// RPTQ write-up, evaluation section: the KV-cache settings (W4A4KV, W4A3KV,
// W3A3KV) keep the key and value caches quantized because at large batch x
// sequence length they hold most of the memory.  Attention then has to read
// them back; instead of a separate dequantize pass that writes the fp16
// cache to HBM and an attention pass that reads it again, every packed row
// is dequantized on its way into LDS (exactly as the standalone dequantize
// computes it: fp16_rne(s_c * (q - z_c)), scattered back to natural channel
// order) and consumed there.
//
// One query token per sequence (decode).  Work is split flash-decoding
// style: workgroup (b, k) handles tokens [k*TC, k*TC + TC) of sequence b in
// three phases, all on one LDS row buffer:
//   1. scores: for each key row, LPH = D/16 lanes per head each take 16
//      channels (packed-fp16 dot products), reduced with lane shuffles:
//      S[t][h] = scale * q_h . k_h;
//   2. softmax inside the chunk: m_h = max_t S, p = exp(S - m_h), l_h = sum p;
//   3. values: every lane owns 8-channel slices of the output and adds
//      p[t][h] * v over the chunk's value rows.
// A second kernel merges the chunks of a sequence: with M = max_k m_k,
//   out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k.
#include "rptq_device.hpp"

namespace rptq {
namespace {

constexpr int kAttnBlock = 256;
constexpr int kAttnMaxRounds = 4;          // score tasks per lane: H * D/16 <= 4 * 256

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <int BITS, int UPL, int D>
__global__ __launch_bounds__(kAttnBlock) void kv_attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
    int32_t T, int32_t C, int32_t TC, int32_t nch, float scale,
    const int32_t* __restrict__ Rk, const ClusterArgs ck, const int32_t* __restrict__ Rv, const ClusterArgs cv,
    float* __restrict__ o_part, float* __restrict__ ml) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CH = chunks_for<true>(UPL * BITS);          // packed row: C*BITS/8 bytes
    constexpr int LPH = D / 16;                               // lanes per head for the scores
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int H = C / D;
    const int b = blockIdx.x / nch, kc = blockIdx.x % nch;
    const int t0 = kc * TC;
    const int nv = min(TC, T - t0);                           // tokens of this chunk (>= 1)
    const int64_t row_bytes = (int64_t)C * BITS / 8;
    unsigned char* prow = smem;                               // CH * 16 * block bytes
    unsigned char* xrow = prow + (size_t)CH * 16 * kAttnBlock;   // UPL * 16 * block >= 2 C bytes
    unsigned char* dummy = xrow + (size_t)UPL * 16 * kAttnBlock; // 16 bytes
    float* S = reinterpret_cast<float*>(dummy + 16);          // [TC][H]
    const int n_units = C / 8;

    // per-lane units of 8 codes: destination channel, s and z of each code
    int dst[UPL][8], uib[UPL];
    float sc[UPL][8], zf[UPL][8];
    auto tables = [&](const int32_t* R, const ClusterArgs& ca) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int unit = tid + u * kAttnBlock;
            const bool live = unit < n_units;
            uib[u] = live ? UnitGeom<BITS>::out_byte(unit) : 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dst[u][e] = (int)(dummy - xrow); sc[u][e] = 0.0f; zf[u][e] = 0.0f;
                if (live) {
                    const int j = UnitGeom<BITS>::first(unit) + e * UnitGeom<BITS>::stride;
                    const int c = cluster_of_pos(ca, j);
                    dst[u][e] = (R ? R[j] : j) * 2;
                    sc[u][e] = ca.s[c];
                    zf[u][e] = (float)ca.z[c];
                }
            }
        }
    };

    // Rows b*T + t0 .. + nv - 1 of one tensor: each is staged in LDS,
    // dequantized into xrow (fp16, natural order) and handed to consume(t).
    // The next row's load is in flight meanwhile; a load past the chunk uses
    // a descriptor of size 0 (reads nothing), so no load is conditional.
    u32x4 buf[CH];
    auto run_rows = [&](const uint8_t* base, auto&& consume) {
        const uint8_t* rows = base + ((int64_t)b * T + t0) * row_bytes;
        load_row_chunks<true, CH>(buf, rows, row_bytes);
        for (int t = 0; t < nv; ++t) {
            put_row_chunks<true, CH>(prow, buf);
            __syncthreads();                                  // prow ready; xrow free
            load_row_chunks<true, CH>(buf, rows + (int64_t)(t + 1) * row_bytes, t + 1 < nv ? row_bytes : 0);
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                int qv[8];
                load_unit_at<BITS>(prow + uib[u], qv);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<_Float16*>(xrow + dst[u][e]) = (_Float16)(sc[u][e] * ((float)qv[e] - zf[u][e]));
            }
            __syncthreads();                                  // xrow holds row t
            consume(t);
        }
        __syncthreads();
    };

    // ---- 1. scores.  Task i = tid + 256 r: head i / LPH, channels
    // (i % LPH) * 16 .. +16 of the head; the LPH lanes of a head are
    // consecutive, so the reduction is a few lane swaps.
    const int ntask = H * LPH;
    const int rounds = (ntask + kAttnBlock - 1) / kAttnBlock;
    u32x4 qa[kAttnMaxRounds][2];
#pragma unroll
    for (int r = 0; r < kAttnMaxRounds; ++r) {
        const int i = tid + r * kAttnBlock;
        const int ch = (i / LPH) * D + (i % LPH) * 16;
        const bool on = r < rounds && i < ntask;
        qa[r][0] = on ? *reinterpret_cast<const u32x4*>(q + (int64_t)b * C + ch) : u32x4{0u, 0u, 0u, 0u};
        qa[r][1] = on ? *reinterpret_cast<const u32x4*>(q + (int64_t)b * C + ch + 8) : u32x4{0u, 0u, 0u, 0u};
    }
    tables(Rk, ck);
    run_rows(kp, [&](int t) {
#pragma unroll
        for (int r = 0; r < kAttnMaxRounds; ++r) {
            if (r >= rounds) break;                           // uniform
            const int i = tid + r * kAttnBlock;
            const bool on = i < ntask;
            const int ch = on ? (i / LPH) * D + (i % LPH) * 16 : 0;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(xrow + ch * 2);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(xrow + ch * 2 + 16);
            const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const uint32_t qs[8] = {qa[r][0].x, qa[r][0].y, qa[r][0].z, qa[r][0].w,
                                    qa[r][1].x, qa[r][1].y, qa[r][1].z, qa[r][1].w};
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w)
                s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qs[w]), __builtin_bit_cast(half2_t, xs[w]), s,
                                           false);
#pragma unroll
            for (int o = 1; o < LPH; o <<= 1) s += __shfl_xor(s, o, 64);
            if (on && (i % LPH) == 0) S[t * H + i / LPH] = s * scale;
        }
    });

    // ---- 2. softmax inside the chunk (one wave per head at a time)
    for (int h = wv; h < H; h += kAttnBlock / 64) {
        float m = -__builtin_inff();
        for (int t = lane; t < nv; t += 64) m = __builtin_fmaxf(m, S[t * H + h]);
        m = wave_max(m);
        float l = 0.0f;
        for (int t = lane; t < nv; t += 64) {
            const float p = __expf(S[t * H + h] - m);
            S[t * H + h] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) {
            ml[(((int64_t)b * nch + kc) * H + h) * 2] = m;
            ml[(((int64_t)b * nch + kc) * H + h) * 2 + 1] = l;
        }
    }
    __syncthreads();

    // ---- 3. values: lane owns output slices oc = tid + 256 u (8 channels)
    float acc[UPL][8];
#pragma unroll
    for (int u = 0; u < UPL; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] = 0.0f;
    tables(Rv, cv);
    run_rows(vp, [&](int t) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int oc = tid + u * kAttnBlock;
            if (oc < n_units) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(xrow + oc * 16);
                const float p = S[t * H + oc * 8 / D];
                const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const half2_t hv = __builtin_bit_cast(half2_t, xs[w]);
                    acc[u][2 * w] = __builtin_fmaf(p, (float)hv.x, acc[u][2 * w]);
                    acc[u][2 * w + 1] = __builtin_fmaf(p, (float)hv.y, acc[u][2 * w + 1]);
                }
            }
        }
    });
    float* op = o_part + ((int64_t)b * nch + kc) * C;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const int oc = tid + u * kAttnBlock;
        if (oc < n_units) {
            reinterpret_cast<float4*>(op + oc * 8)[0] = float4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
            reinterpret_cast<float4*>(op + oc * 8)[1] = float4{acc[u][4], acc[u][5], acc[u][6], acc[u][7]};
        }
    }
}

// Merge the chunks of each sequence: one thread per output channel.
__global__ __launch_bounds__(256) void kv_attn_combine_kernel(const float* __restrict__ o_part,
                                                              const float* __restrict__ ml, int32_t C, int32_t D,
                                                              int32_t nch, float* __restrict__ out) {
    const int b = blockIdx.y;
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    const int H = C / D, h = c / D;
    const float* mlb = ml + (int64_t)b * nch * H * 2;
    float M = -__builtin_inff();
    for (int k = 0; k < nch; ++k) M = __builtin_fmaxf(M, mlb[((int64_t)k * H + h) * 2]);
    float o = 0.0f, L = 0.0f;
    for (int k = 0; k < nch; ++k) {
        const float w = __expf(mlb[((int64_t)k * H + h) * 2] - M);
        o = __builtin_fmaf(w, o_part[((int64_t)b * nch + k) * C + c], o);
        L = __builtin_fmaf(w, mlb[((int64_t)k * H + h) * 2 + 1], L);
    }
    out[(int64_t)b * C + c] = o / L;
}

template <int BITS, int D>
const void* pick_upl(int upl) {
    switch (upl) {
        case 1: return (const void*)kv_attn_chunk_kernel<BITS, 1, D>;
        case 2: return (const void*)kv_attn_chunk_kernel<BITS, 2, D>;
        case 3: return (const void*)kv_attn_chunk_kernel<BITS, 3, D>;
        case 4: return (const void*)kv_attn_chunk_kernel<BITS, 4, D>;
        case 5: return (const void*)kv_attn_chunk_kernel<BITS, 5, D>;
        default: return nullptr;
    }
}

const void* pick_attn(int bits, int upl, int D) {
    if (D == 64) return bits == 3 ? pick_upl<3, 64>(upl) : bits == 4 ? pick_upl<4, 64>(upl) : pick_upl<8, 64>(upl);
    return bits == 3 ? pick_upl<3, 128>(upl) : bits == 4 ? pick_upl<4, 128>(upl) : pick_upl<8, 128>(upl);
}

}  // namespace

void kv_attention_geometry(int32_t T, int32_t C, int32_t D, int32_t& TC, int32_t& nch) {
    // tokens per chunk: the score tile TC x H fp32 stays within 48 KB of LDS
    const int H = C / D;
    TC = 128;
    while (TC > 1 && (int64_t)TC * H * 4 > 48 * 1024) TC >>= 1;
    nch = (T + TC - 1) / TC;
}

int64_t kv_attention_workspace(int32_t B, int32_t T, int32_t C, int32_t D) {
    int32_t TC = 0, nch = 0;
    kv_attention_geometry(T, C, D, TC, nch);
    const int64_t o_bytes = (int64_t)B * nch * C * 4;
    const int64_t ml_bytes = (int64_t)B * nch * (C / D) * 2 * 4;
    return (o_bytes + 255) / 256 * 256 + ml_bytes;
}

hipError_t launch_kv_attention(const uint16_t* q, const uint8_t* kp, const uint8_t* vp, int32_t B, int32_t T,
                               int32_t C, int32_t D, float scale, const int32_t* Rk, const ClusterArgs& ck,
                               const int32_t* Rv, const ClusterArgs& cv, float* out, void* workspace,
                               hipStream_t stream) {
    int upl = 0, block = 0;
    unit_split(C / 8, upl, block, kAttnBlock);
    if (upl == 0 || block > kAttnBlock) return hipErrorInvalidValue;
    block = kAttnBlock;
    int32_t TC = 0, nch = 0;
    kv_attention_geometry(T, C, D, TC, nch);
    const void* k = pick_attn(ck.bits, upl, D);
    if (!k) return hipErrorInvalidValue;
    const int ch = chunks_for<true>(upl * ck.bits);
    const size_t lds = (size_t)ch * 16 * block + (size_t)upl * 16 * block + 16 + (size_t)TC * (C / D) * 4;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    float* o_part = static_cast<float*>(workspace);
    float* ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         ((int64_t)B * nch * C * 4 + 255) / 256 * 256);
    void* args[] = {(void*)&q, (void*)&kp, (void*)&vp, (void*)&T, (void*)&C, (void*)&TC, (void*)&nch,
                    (void*)&scale, (void*)&Rk, (void*)&ck, (void*)&Rv, (void*)&cv, (void*)&o_part, (void*)&ml};
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)(B * nch)), dim3(block), args, lds, stream);
    if (e != hipSuccess) return e;
    void* args2[] = {(void*)&o_part, (void*)&ml, (void*)&C, (void*)&D, (void*)&nch, (void*)&out};
    return hipLaunchKernel((const void*)kv_attn_combine_kernel, dim3((unsigned)((C + 255) / 256), (unsigned)B),
                           dim3(256), args2, 0, stream);
}

}  // namespace rptq
