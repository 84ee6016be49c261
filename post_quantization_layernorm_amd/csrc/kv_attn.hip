// Decode attention that reads the packed K/V cache directly (gfx950).
//
// RPTQ write-up, evaluation section: the KV-cache settings (W4A4KV, W4A3KV,
// W3A3KV) keep the key and value caches quantized because at large batch x
// sequence length they hold most of the memory.  Attention then has to read
// them back; instead of a separate dequantize pass that writes the fp16
// cache to HBM and an attention pass that reads it again, every packed row
// is decoded on its way through LDS and consumed there.  The decode forms
// each code's exact (q - z_c) as an fp16 integer (1024 + q is formed from
// the code bits, and one packed fp16 add of -(1024 + z_c) per pair of codes
// leaves q - z_c exactly); for the keys it is scattered back to natural
// channel order, the values are summed in code order.  The cluster scale
// s_c is applied in fp32 outside the per-row work: folded into the query
// for the scores (q_c * s_c), and into each output channel of the value
// sums at the end.  So the cache values enter the arithmetic as
// s_c (q - z_c) without the fp16 rounding of the standalone dequantize (a
// difference of at most half an fp16 ulp per value).
//
// One query token per sequence (decode).  Work is split flash-decoding
// style: workgroup (b, k) handles tokens [k*TC, k*TC + TC) of sequence b in
// three phases, the packed rows streaming through a ring of LDS slots
// several rows ahead:
//   1. scores: for each key row, LPH = D/16 lanes per head each take 16
//      channels (fp32 q_c * s_c against the fp16 (q - z_c)), reduced with
//      lane shuffles: S[t][h] = scale * q_h . k_h;
//   2. softmax inside the chunk: m_h = max_t S, p = exp(S - m_h), l_h = sum p;
//   3. values: every lane keeps, for the codes of its units, the sum of
//      p[t][head] * (q - z) over the chunk's value rows in registers (no
//      scatter, one barrier per row) and stores it to the codes' natural
//      channels at the end.
// A second kernel merges the chunks of a sequence: with M = max_k m_k,
//   out = sum_k e^(m_k - M) o_k / sum_k e^(m_k - M) l_k.
#include "rptq_device.hpp"

namespace rptq {
namespace {

constexpr int kAttnBlock = 256;
constexpr int kAttnMaxRounds = 4;          // score tasks per lane: H * D/16 <= 4 * 256
constexpr int kAttnRing = 4;               // packed rows in flight per workgroup

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Per code of the packed row (unit-major: code e of unit u at u * 8 + e):
// its natural channel and its cluster's z; and per natural channel, its
// cluster's s.
struct AttnTable {
    uint16_t* dst;
    float* s;          // natural channel order
    float* z;          // code order
};

template <int BITS>
__global__ __launch_bounds__(256) void kv_attn_tables_kernel(int32_t C, const int32_t* __restrict__ R,
                                                             const ClusterArgs ca, AttnTable tb) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;       // unit * 8 + e
    if (i >= C) return;
    const int unit = i >> 3, e = i & 7;
    const int j = UnitGeom<BITS>::first(unit) + e * UnitGeom<BITS>::stride;
    const int c = cluster_of_pos(ca, j);
    const int nat = R ? R[j] : j;
    tb.dst[i] = (uint16_t)nat;
    tb.s[nat] = ca.s[c];
    tb.z[i] = (float)ca.z[c];
}

template <int BITS, int UPL, int D>
__global__ __launch_bounds__(kAttnBlock) void kv_attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
    int32_t T, int32_t C, int32_t TC, int32_t nch, float scale, const AttnTable tk, const AttnTable tv,
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
    constexpr int SLOT = CH * 16 * kAttnBlock;                // one packed row
    unsigned char* ring = smem;                               // kAttnRing slots
    unsigned char* xrow = ring + (size_t)kAttnRing * SLOT;    // UPL * 16 * block >= 2 C bytes
    unsigned char* dummy = xrow + (size_t)UPL * 16 * kAttnBlock; // 16 bytes
    float* S = reinterpret_cast<float*>(dummy + 16);          // [TC][H]
    const int n_units = C / 8;

    // per-lane units of 8 codes: destination byte in xrow of each code, and
    // per pair of codes the fp16 pair -(1024 + z) that turns 1024 + q into
    // q - z, from the tables kv_attn_tables_kernel built once per call
    int dst[UPL][8], uib[UPL];
    half2_t nz[UPL][4];
    auto tables = [&](const AttnTable& tb) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int unit = tid + u * kAttnBlock;
            const bool live = unit < n_units;
            uib[u] = live ? UnitGeom<BITS>::out_byte(unit) : 0;
            const int uu = live ? unit : 0;
            const u32x4 d4 = *reinterpret_cast<const u32x4*>(tb.dst + uu * 8);
            const uint32_t dw[4] = {d4.x, d4.y, d4.z, d4.w};
            const float4 z0 = reinterpret_cast<const float4*>(tb.z + uu * 8)[0];
            const float4 z1 = reinterpret_cast<const float4*>(tb.z + uu * 8)[1];
            const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dst[u][e] = live ? (int)((dw[e / 2] >> (16 * (e & 1))) & 0xFFFFu) * 2 : (int)(dummy - xrow);
#pragma unroll
            for (int i = 0; i < 4; ++i)       // integers up to 1279: exact in fp16
                nz[u][i] = half2_t{(_Float16)(-1024.0f - zv[2 * i]), (_Float16)(-1024.0f - zv[2 * i + 1])};
        }
    };

    // Rows b*T + t0 .. + nv - 1 of one tensor.  Packed rows travel straight
    // from HBM into a ring of kAttnRing LDS slots (buffer loads that write
    // LDS: lane l of a wave lands at the wave's base + 16 l, so a row keeps
    // its byte order), kAttnRing rows ahead; each is dequantized into xrow
    // (fp16, natural order) and handed to consume(t).  Every wave issues CH
    // such loads per row, loads past the chunk use a descriptor of size 0,
    // so the memory-counter waits are fixed counts.
    auto issue_row = [&](const uint8_t* rows, int t) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(rows + (int64_t)t * row_bytes, t < nv ? row_bytes : 0);
        unsigned char* slot = ring + (size_t)(t % kAttnRing) * SLOT;
#pragma unroll
        for (int i = 0; i < CH; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(slot + (size_t)(wv * 64 + i * kAttnBlock) * 16),
                                                     16, (uint32_t)(tid + i * kAttnBlock) * 16u, 0, 0, 0);
    };
    auto run_rows = [&](const uint8_t* base, auto&& consume) {
        const uint8_t* rows = base + ((int64_t)b * T + t0) * row_bytes;
        wait_vm<0>();                                         // nothing older in the count
        __syncthreads();                                      // the ring is free
#pragma unroll
        for (int p = 0; p < kAttnRing; ++p) issue_row(rows, p);
        for (int t = 0; t < nv; ++t) {
            wait_vm<(kAttnRing - 1) * CH>();                  // this wave's part of row t is in LDS
            lds_barrier();                                    // every part; xrow free
            const unsigned char* prow = ring + (size_t)(t % kAttnRing) * SLOT;
            // every unit's packed bytes first (their LDS reads overlap), then
            // decode, dequantize and scatter
            uint32_t raw[UPL][BITS == 8 ? 2 : BITS == 4 ? 1 : 3];
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                const unsigned char* pu = prow + uib[u];
                if constexpr (BITS == 8) {
                    const uint2 v = *reinterpret_cast<const uint2*>(pu);
                    raw[u][0] = v.x; raw[u][1] = v.y;
                } else if constexpr (BITS == 4) {
                    raw[u][0] = *reinterpret_cast<const uint32_t*>(pu);
                } else {
                    raw[u][0] = pu[0]; raw[u][1] = pu[4]; raw[u][2] = pu[8];
                }
            }
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                int qv[8];
                if constexpr (BITS == 8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qv[i] = (raw[u][0] >> (8 * i)) & 255;
                        qv[4 + i] = (raw[u][1] >> (8 * i)) & 255;
                    }
                } else if constexpr (BITS == 4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qv[i] = (raw[u][0] >> (8 * i)) & 15;
                        qv[4 + i] = (raw[u][0] >> (8 * i + 4)) & 15;
                    }
                } else {
                    // one byte of each of the group's three words (3-bit layout)
                    const int b0 = raw[u][0], b1 = raw[u][1], b2 = raw[u][2];
                    qv[0] = b0 & 7; qv[1] = (b0 >> 3) & 7;
                    qv[2] = b1 & 7; qv[3] = (b1 >> 3) & 7;
                    qv[4] = b2 & 7; qv[5] = (b2 >> 3) & 7;
                    qv[6] = (b0 >> 6) | ((b2 >> 6) & 1) << 2;
                    qv[7] = (b1 >> 6) | ((b2 >> 7) & 1) << 2;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // (1024 + q) pair from the code bits, + (-(1024 + z)) pair: q - z exactly
                    const uint32_t w = (uint32_t)qv[2 * i] | (uint32_t)qv[2 * i + 1] << 16 | 0x64006400u;
                    const uint32_t x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, w) + nz[u][i]);
                    *reinterpret_cast<uint16_t*>(xrow + dst[u][2 * i]) = (uint16_t)x;
                    *reinterpret_cast<uint16_t*>(xrow + dst[u][2 * i + 1]) = (uint16_t)(x >> 16);
                }
            }
            lds_barrier();                                    // xrow holds row t; slot t free
            issue_row(rows, t + kAttnRing);
            consume(t);
        }
        wait_vm<0>();
        __syncthreads();
    };

    // ---- 1. scores.  Task i = tid + 256 r: head i / LPH, channels
    // (i % LPH) * 16 .. +16 of the head; the LPH lanes of a head are
    // consecutive, so the reduction is a few lane swaps.
    const int ntask = H * LPH;
    const int rounds = (ntask + kAttnBlock - 1) / kAttnBlock;
    // the task's 16 query channels times their key clusters' s, in fp32
    float qs[kAttnMaxRounds][16];
#pragma unroll
    for (int r = 0; r < kAttnMaxRounds; ++r) {
        const int i = tid + r * kAttnBlock;
        const int ch = (i / LPH) * D + (i % LPH) * 16;
        const bool on = r < rounds && i < ntask;
        const int cc = on ? ch : 0;
        const u32x4 q0 = *reinterpret_cast<const u32x4*>(q + (int64_t)b * C + cc);
        const u32x4 q1 = *reinterpret_cast<const u32x4*>(q + (int64_t)b * C + cc + 8);
        const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 s4 = reinterpret_cast<const float4*>(tk.s + cc)[k];
            const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const half2_t h = __builtin_bit_cast(half2_t, qw[(4 * k + e) / 2]);
                const float qf = (float)((4 * k + e) & 1 ? h.y : h.x);
                qs[r][4 * k + e] = on ? qf * sv[e] : 0.0f;
            }
        }
    }
    tables(tk);
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
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const half2_t hx = __builtin_bit_cast(half2_t, xs[w]);
                s = __builtin_fmaf(qs[r][2 * w], (float)hx.x, s);
                s = __builtin_fmaf(qs[r][2 * w + 1], (float)hx.y, s);
            }
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

    // ---- 3. values, in code order: each lane keeps, for the codes of its
    // units, the sum over the chunk's rows of p[t][head] * (q - z) in
    // registers (a channel's sum runs over the rows in the same order as a
    // natural-order pass would), and stores it to the channel's natural place
    // once at the end: no per-row scatter, one barrier per row.
    float acc[UPL][8];
    int hd[UPL][8];                                           // head of each code
    tables(tv);
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        const bool live = tid + u * kAttnBlock < n_units;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[u][e] = 0.0f;
            hd[u][e] = live ? (dst[u][e] >> 1) / D : 0;
        }
    }
    {
        const uint8_t* rows = vp + ((int64_t)b * T + t0) * row_bytes;
        wait_vm<0>();                                         // nothing older in the count
        __syncthreads();                                      // the ring is free
#pragma unroll
        for (int p = 0; p < kAttnRing - 1; ++p) issue_row(rows, p);
        for (int t = 0; t < nv; ++t) {
            wait_vm<(kAttnRing - 2) * CH>();                  // this wave's part of row t is in LDS
            lds_barrier();                                    // every part; every wave done with row t - 1
            issue_row(rows, t + kAttnRing - 1);               // into the slot of row t - 1
            const unsigned char* prow = ring + (size_t)(t % kAttnRing) * SLOT;
            const float* St = S + t * H;
            uint32_t raw[UPL][BITS == 8 ? 2 : BITS == 4 ? 1 : 3];
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                const unsigned char* pu = prow + uib[u];
                if constexpr (BITS == 8) {
                    const uint2 v = *reinterpret_cast<const uint2*>(pu);
                    raw[u][0] = v.x; raw[u][1] = v.y;
                } else if constexpr (BITS == 4) {
                    raw[u][0] = *reinterpret_cast<const uint32_t*>(pu);
                } else {
                    raw[u][0] = pu[0]; raw[u][1] = pu[4]; raw[u][2] = pu[8];
                }
            }
#pragma unroll
            for (int u = 0; u < UPL; ++u) {
                int qv[8];
                if constexpr (BITS == 8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qv[i] = (raw[u][0] >> (8 * i)) & 255;
                        qv[4 + i] = (raw[u][1] >> (8 * i)) & 255;
                    }
                } else if constexpr (BITS == 4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qv[i] = (raw[u][0] >> (8 * i)) & 15;
                        qv[4 + i] = (raw[u][0] >> (8 * i + 4)) & 15;
                    }
                } else {
                    const int b0 = raw[u][0], b1 = raw[u][1], b2 = raw[u][2];
                    qv[0] = b0 & 7; qv[1] = (b0 >> 3) & 7;
                    qv[2] = b1 & 7; qv[3] = (b1 >> 3) & 7;
                    qv[4] = b2 & 7; qv[5] = (b2 >> 3) & 7;
                    qv[6] = (b0 >> 6) | ((b2 >> 6) & 1) << 2;
                    qv[7] = (b1 >> 6) | ((b2 >> 7) & 1) << 2;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w = (uint32_t)qv[2 * i] | (uint32_t)qv[2 * i + 1] << 16 | 0x64006400u;
                    const half2_t hv = __builtin_bit_cast(half2_t, w) + nz[u][i];      // q - z, exact
                    acc[u][2 * i] = __builtin_fmaf(St[hd[u][2 * i]], (float)hv.x, acc[u][2 * i]);
                    acc[u][2 * i + 1] = __builtin_fmaf(St[hd[u][2 * i + 1]], (float)hv.y, acc[u][2 * i + 1]);
                }
            }
        }
        wait_vm<0>();
    }
    // each channel's sum of p (q - z) times its value cluster's s, to its
    // natural place
    float* op = o_part + ((int64_t)b * nch + kc) * C;
#pragma unroll
    for (int u = 0; u < UPL; ++u) {
        if (tid + u * kAttnBlock < n_units) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int chn = dst[u][e] >> 1;
                op[chn] = acc[u][e] * tv.s[chn];
            }
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
    // (both loops unrolled so that their loads are in flight together; the
    // sums keep chunk order)
    float M = -__builtin_inff();
#pragma unroll 16
    for (int k = 0; k < nch; ++k) M = __builtin_fmaxf(M, mlb[((int64_t)k * H + h) * 2]);
    float o = 0.0f, L = 0.0f;
#pragma unroll 16
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
    // tokens per chunk: the score tile TC x H fp32 stays within 40 KB of LDS
    // (two workgroups per CU with the row ring and the dequantized row)
    const int H = C / D;
    TC = 128;
    while (TC > 1 && (int64_t)TC * H * 4 > 40 * 1024) TC >>= 1;
    nch = (T + TC - 1) / TC;
}

// Workspace: per-chunk outputs [B][nch][C] fp32, softmax statistics
// [B][nch][H][2] fp32, then the K and V tables (C x (2 + 4 + 4) bytes each:
// natural channel and z per code, s per natural channel); every part starts
// on a 256-byte boundary.
static int64_t up256(int64_t n) { return (n + 255) / 256 * 256; }

int64_t kv_attention_workspace(int32_t B, int32_t T, int32_t C, int32_t D) {
    int32_t TC = 0, nch = 0;
    kv_attention_geometry(T, C, D, TC, nch);
    const int64_t o_bytes = (int64_t)B * nch * C * 4;
    const int64_t ml_bytes = (int64_t)B * nch * (C / D) * 2 * 4;
    const int64_t tab = up256((int64_t)C * 2) + 2 * up256((int64_t)C * 4);
    return up256(o_bytes) + up256(ml_bytes) + 2 * tab;
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
    const size_t lds = (size_t)kAttnRing * ch * 16 * block + (size_t)upl * 16 * block + 16 + (size_t)TC * (C / D) * 4;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    char* w = static_cast<char*>(workspace);
    float* o_part = reinterpret_cast<float*>(w);
    w += up256((int64_t)B * nch * C * 4);
    float* ml = reinterpret_cast<float*>(w);
    w += up256((int64_t)B * nch * (C / D) * 2 * 4);
    AttnTable tab[2];
    for (int i = 0; i < 2; ++i) {
        tab[i].dst = reinterpret_cast<uint16_t*>(w);
        w += up256((int64_t)C * 2);
        tab[i].s = reinterpret_cast<float*>(w);
        w += up256((int64_t)C * 4);
        tab[i].z = reinterpret_cast<float*>(w);
        w += up256((int64_t)C * 4);
    }
    const void* tk = ck.bits == 3 ? (const void*)kv_attn_tables_kernel<3>
                   : ck.bits == 4 ? (const void*)kv_attn_tables_kernel<4> : (const void*)kv_attn_tables_kernel<8>;
    for (int i = 0; i < 2; ++i) {
        const int32_t* R = i ? Rv : Rk;
        const ClusterArgs& ca = i ? cv : ck;
        void* targs[] = {(void*)&C, (void*)&R, (void*)&ca, (void*)&tab[i]};
        hipError_t e = hipLaunchKernel(tk, dim3((unsigned)((C + 255) / 256)), dim3(256), targs, 0, stream);
        if (e != hipSuccess) return e;
    }
    void* args[] = {(void*)&q, (void*)&kp, (void*)&vp, (void*)&T, (void*)&C, (void*)&TC, (void*)&nch,
                    (void*)&scale, (void*)&tab[0], (void*)&tab[1], (void*)&o_part, (void*)&ml};
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)(B * nch)), dim3(block), args, lds, stream);
    if (e != hipSuccess) return e;
    void* args2[] = {(void*)&o_part, (void*)&ml, (void*)&C, (void*)&D, (void*)&nch, (void*)&out};
    return hipLaunchKernel((const void*)kv_attn_combine_kernel, dim3((unsigned)((C + 255) / 256), (unsigned)B),
                           dim3(256), args2, 0, stream);
}

}  // namespace rptq
