// Cluster-segmented integer GEMM on int8 MFMA (gfx950), zero-point correction
// folded into the epilogue.
//
// RPTQ write-up, method section and Fig. 3: the linear layer's weights are
// reordered offline by R so they consume the reordered, per-cluster-quantized
// activations; motivation section: quantization speeds up matrix
// multiplication.  With s_c, z_c per activation cluster and s_w[n] per output
// feature (quantization lecture 1.3: W = S (Wq - Z) for activations,
// symmetric for weights):
//   Y[m][n] = s_w[n] * sum_c s_c * (acc_c[m][n] - z_c * colsum_c[n]),
//   acc_c   = sum over the cluster's K-segment of q * W'   (int32, exact).
//
// Design:
//   - 128 x 128 output tile per 256-thread workgroup, 2 x 2 waves of 64 x 64,
//     each wave 2 x 2 v_mfma_i32_32x32x32_i8 tiles;
//   - K advances in stages of 64 codes (two MFMA steps of 32); every cluster
//     is padded to a multiple of 32 codes, so a step never straddles clusters;
//   - A (3/4/8-bit activation codes) and W' (4/8-bit weights) are read from
//     global memory packed, unpacked to int8 in registers, and staged in a
//     double-buffered LDS tile (row stride 80 B: conflict-free 16-B fragment
//     reads); the next stage's global loads are in flight during the MFMAs;
//   - the int32 accumulators hold one cluster at a time: at the cluster's
//     last step they are converted and scaled into fp32 accumulators
//     (out += s_c * acc) and restart at zero;
//   - 8-bit codes q are staged as q - 128 (signed int8 MFMA) and 4-bit
//     weights as 16 * w (nibble placed in the high half of the byte, so the
//     sign comes for free); both are undone exactly in the scale / epilogue:
//     corr[n] = sum_c s_c (z_c - offset) colsum_c[n] in fp64.
#include "rptq_device.hpp"

namespace rptq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BKS = 64, LDSS = 80;

// 32 codes of ABITS bits = ABITS 32-bit words, starting 4-byte aligned.
template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, bool ok, uint32_t (&d)[BITS]) {
    if constexpr (BITS == 4) {
        uint4 v = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else if constexpr (BITS == 8) {
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
        if (ok) { v0 = reinterpret_cast<const uint4*>(p)[0]; v1 = reinterpret_cast<const uint4*>(p)[1]; }
        d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w;
        d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
    } else {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        d[0] = ok ? q[0] : 0u; d[1] = ok ? q[1] : 0u; d[2] = ok ? q[2] : 0u;
    }
}

// Activation codes -> 32 int8 in natural code order.
template <int BITS>
__device__ __forceinline__ void unpack_act(const uint32_t (&d)[BITS], uint32_t (&o)[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = d[i] ^ 0x80808080u;        // q - 128
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = d[i] & 0x0F0F0F0Fu;
            o[2 * i + 1] = (d[i] >> 4) & 0x0F0F0F0Fu;
        }
    } else {
        const uint32_t m7 = 0x07070707u, m3 = 0x03030303u, m4 = 0x04040404u;
        o[0] = d[0] & m7;         o[1] = (d[0] >> 3) & m7;
        o[2] = d[1] & m7;         o[3] = (d[1] >> 3) & m7;
        o[4] = d[2] & m7;         o[5] = (d[2] >> 3) & m7;
        o[6] = ((d[0] >> 6) & m3) | ((d[2] >> 4) & m4);
        o[7] = ((d[1] >> 6) & m3) | ((d[2] >> 5) & m4);
    }
}

// Weight codes (two's complement) -> 32 int8; 4-bit weights come out as 16*w.
template <int BITS>
__device__ __forceinline__ void unpack_wgt(const uint32_t (&d)[BITS], uint32_t (&o)[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = d[i];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = (d[i] << 4) & 0xF0F0F0F0u;
            o[2 * i + 1] = d[i] & 0xF0F0F0F0u;
        }
    }
}

__device__ __forceinline__ void store32(int8_t* lds, const uint32_t (&o)[8]) {
    reinterpret_cast<uint4*>(lds)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4*>(lds)[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int ABITS, int WBITS>
__global__ __launch_bounds__(256, 2) void qgemm_kernel(
    const uint8_t* __restrict__ A, int64_t M, int64_t a_row_bytes,
    const uint8_t* __restrict__ B, int32_t N, int64_t b_row_bytes,
    const GemmArgs ga, const float* __restrict__ s_w, const int32_t* __restrict__ colsum,
    float* __restrict__ Y, int32_t* __restrict__ acc_dbg) {
    __shared__ __align__(16) int8_t As[2][BM * LDSS];
    __shared__ __align__(16) int8_t Bs[2][BN * LDSS];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int tiles_n = (N + BN - 1) / BN;
    const int64_t bm = blockIdx.x / tiles_n;
    const int bn = blockIdx.x % tiles_n;
    const int64_t m0 = bm * BM;
    const int n0 = bn * BN;

    // global -> LDS staging: thread owns row `lr`, codes [32*part, 32*part+32) of a stage
    const int lr = tid >> 1, part = tid & 1;
    const bool a_row_ok = m0 + lr < M;
    const bool b_row_ok = n0 + lr < N;
    const uint8_t* a_ptr = A + (a_row_ok ? (m0 + lr) * a_row_bytes : 0) + part * (32 * ABITS / 8);
    const uint8_t* b_ptr = B + (b_row_ok ? (int64_t)(n0 + lr) * b_row_bytes : 0) + part * (32 * WBITS / 8);
    constexpr int ASTAGE = BKS * ABITS / 8, BSTAGE = BKS * WBITS / 8;
    const int nsteps = ga.nsteps;
    const int nstages = (nsteps + 1) / 2;

    uint32_t ra[ABITS], rb[WBITS];
    auto gload = [&](int st) {
        const bool in_k = 2 * st + part < nsteps;
        load_codes<ABITS>(a_ptr + (int64_t)st * ASTAGE, a_row_ok && in_k, ra);
        load_codes<WBITS>(b_ptr + (int64_t)st * BSTAGE, b_row_ok && in_k, rb);
    };
    auto lstore = [&](int buf) {
        uint32_t o[8];
        unpack_act<ABITS>(ra, o);
        store32(&As[buf][lr * LDSS + part * 32], o);
        unpack_wgt<WBITS>(rb, o);
        store32(&Bs[buf][lr * LDSS + part * 32], o);
    };

    v16i acc[2][2];
    float out[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = (v16i)0;
#pragma unroll
            for (int r = 0; r < 16; ++r) out[i][j][r] = 0.0f;
        }

    // output coordinates of this lane's accumulator registers
    const int row_in_tile = (lane >> 5) * 4;      // + (r / 4) * 8 + (r % 4)
    const int col_in_tile = lane & 31;

    int c = 0;
    int c_end = ga.step_end[0];

    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nstages; ++st) {
        const int cur = st & 1;
        if (st + 1 < nstages) gload(st + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int step = 2 * st + ks;
            if (step >= nsteps) break;
            v4i af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const v4i*>(
                    &As[cur][(wm * 64 + i * 32 + (lane & 31)) * LDSS + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const v4i*>(
                    &Bs[cur][(wn * 64 + j * 32 + (lane & 31)) * LDSS + ks * 32 + (lane >> 5) * 16]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
            if (step + 1 == c_end) {
                const float sc = ga.scale[c];
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            out[i][j][r] = __builtin_fmaf(sc, (float)acc[i][j][r], out[i][j][r]);
                        if (acc_dbg) {
                            const int n = n0 + wn * 64 + j * 32 + col_in_tile;
                            const int add = (n < N && ga.code_offset) ? ga.code_offset * colsum[(int64_t)c * N + n] : 0;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + row_in_tile + (r & 3);
                                if (m < M && n < N) {
                                    const int v = WBITS == 4 ? (acc[i][j][r] >> 4) : acc[i][j][r];
                                    acc_dbg[((int64_t)c * M + m) * N + n] = v + add;
                                }
                            }
                        }
                        acc[i][j] = (v16i)0;
                    }
                ++c;
                c_end = c < ga.g ? ga.step_end[c] : 0x7fffffff;
            }
        }
        if (st + 1 < nstages) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: Y = s_w * (out - corr), corr[n] = sum_c s_c (z_c - offset) colsum_c[n]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + col_in_tile;
        if (n >= N) continue;
        double corr = 0.0;
        for (int cc = 0; cc < ga.g; ++cc) corr += ga.sz[cc] * (double)colsum[(int64_t)cc * N + n];
        const double sw = (double)s_w[n];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + row_in_tile + (r & 3);
                if (m < M) Y[m * N + n] = (float)(sw * ((double)out[i][j][r] - corr));
            }
    }
}

template <int ABITS>
const void* pick(int wbits) {
    return wbits == 4 ? (const void*)qgemm_kernel<ABITS, 4> : (const void*)qgemm_kernel<ABITS, 8>;
}

}  // namespace

hipError_t launch_qgemm(const uint8_t* codes, int64_t M, int32_t N, int64_t a_row_bytes,
                        int a_bits, const uint8_t* w_packed, int64_t w_row_bytes, int w_bits,
                        const GemmArgs& ga, const float* s_w, const int32_t* colsum,
                        float* Y, int32_t* acc_debug, hipStream_t stream) {
    const void* k = a_bits == 3 ? pick<3>(w_bits) : a_bits == 4 ? pick<4>(w_bits) : pick<8>(w_bits);
    const int64_t tiles = ((M + BM - 1) / BM) * (int64_t)((N + BN - 1) / BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    void* args[] = {(void*)&codes, (void*)&M, (void*)&a_row_bytes, (void*)&w_packed, (void*)&N,
                    (void*)&w_row_bytes, (void*)&ga, (void*)&s_w, (void*)&colsum, (void*)&Y,
                    (void*)&acc_debug};
    return hipLaunchKernel(k, dim3((unsigned)tiles), dim3(256), args, 0, stream);
}

}  // namespace rptq
