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
// Design (two workgroups per CU, so one workgroup's barrier waits are covered
// by the other's MFMAs, and the waves of a SIMD overlap one another's VALU
// work and MFMAs):
//   - 128 x 128 output tile.  With 3- and 4-bit operands, 8 waves in a 2 x 4
//     grid of 64 x 32 wave tiles (two v_mfma_i32_32x32x32_i8 tiles each):
//     32 int32 and 32 fp32 accumulator registers per lane leave room for
//     four waves per SIMD (at most 128 VGPRs).  With an 8-bit operand the staging
//     registers do not fit that, and 4 waves in a 2 x 2 grid of 64 x 64 (2 x 2
//     MFMA tiles each) run two waves per SIMD;
//   - K advances in stages of 128 codes (4 MFMA steps of 32).  Clusters are
//     padded to multiples of 32 codes, so a step never straddles clusters;
//   - A (3/4/8-bit activation codes) and W' (3/4/8-bit weights) are fetched
//     packed with buffer loads (scalar stage offsets; rows past M or N read
//     as zero) about two stages ahead, one staging piece per lane and MFMA
//     step, and staged in a double-buffered LDS tile, both unpacked to int8
//     on the way in (row stride 144 B: the 16-byte fragment reads of 8
//     consecutive lanes hit disjoint banks).  The next stage's staging is
//     interleaved with the current stage's MFMAs, and each stage's last MFMA
//     step is deferred past the barrier to cover the next stage's first
//     fragment reads;
//   - one running int32 accumulator per MFMA tile for the whole K loop: at
//     the last step of cluster c it is converted and added to fp32 out with
//     weight d_c = s_c - s_(c+1) (summation by parts of sum_c s_c acc_c), so
//     the accumulators are never reset and every step is the same code;
//   - 8-bit codes q are staged as q - 128 (signed MFMA operands), 4-bit
//     weights as 16 * w (nibble moved to the high half of the byte, sign for
//     free) and 3-bit weights as 32 * w; all are undone exactly: s_c / 16 or
//     s_c / 32 in the scale, and
//     corr[n] = sum_c s_c (z_c - offset) colsum_c[n] (fp64, per column) in the
//     epilogue, which writes Y = fma(s_w, out, -s_w corr) in fp32;
//   - workgroups are numbered so that consecutive tiles of a group land on
//     the same XCD (the dispatcher deals workgroups round-robin over the 8
//     XCDs), sharing its L2.
#include "rptq_device.hpp"

namespace rptq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

constexpr int GROUP_M = 8;

// One 32-code piece of BITS-bit codes = BITS 32-bit words.
template <int BITS>
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t (&d)[BITS]) {
    if constexpr (BITS == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, 0, 0);
        d[0] = v.x; d[1] = v.y; d[2] = v.z;
    } else if constexpr (BITS == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else {
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, 0, 0);
        d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w;
        d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
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

// Weight codes (two's complement) -> 32 int8 in natural code order; 4-bit
// weights come out as 16*w and 3-bit weights as 32*w (the field moved to
// the top of its byte, so the byte's sign is the weight's).
template <int BITS>
__device__ __forceinline__ void unpack_wgt(const uint32_t (&d)[BITS], uint32_t (&o)[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = d[i];
    } else if constexpr (BITS == 3) {
        // byte j of words d0, d1, d2 holds codes j, j+4 | j+8, j+12 | j+16,
        // j+20 in bits 0-2 / 3-5; codes j+24 and j+28 keep their low two bits
        // in bits 6-7 of d0 and d1 and their top bit in bits 6 and 7 of d2
        const uint32_t m = 0xE0E0E0E0u;
        o[0] = (d[0] << 5) & m;  o[1] = (d[0] << 2) & m;
        o[2] = (d[1] << 5) & m;  o[3] = (d[1] << 2) & m;
        o[4] = (d[2] << 5) & m;  o[5] = (d[2] << 2) & m;
        o[6] = ((d[0] >> 1) & 0x60606060u) | ((d[2] << 1) & 0x80808080u);
        o[7] = ((d[1] >> 1) & 0x60606060u) | (d[2] & 0x80808080u);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = (d[i] << 4) & 0xF0F0F0F0u;
            o[2 * i + 1] = d[i] & 0xF0F0F0F0u;
        }
    }
}

__device__ __forceinline__ void store32(int8_t* lds, const uint32_t (&o)[8]) {
    reinterpret_cast<u32x4*>(lds)[0] = u32x4{o[0], o[1], o[2], o[3]};
    reinterpret_cast<u32x4*>(lds)[1] = u32x4{o[4], o[5], o[6], o[7]};
}

// Tile configuration: BM x BN output tile, WAVES waves in a (BM/64) x WN grid
// of 64 x (32 TJ) wave tiles, SK 32-code steps per pipeline stage, MINBLK
// resident workgroups per CU.
template <int BM_, int BN_, int WAVES_, int SK_, int MINBLK_, int TJ_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WAVES = WAVES_, SK = SK_, MINBLK = MINBLK_;
    static constexpr int TJ = TJ_;                      // 32-column MFMA tiles per wave
    static constexpr int NT = WAVES * 64, WN = BN / (32 * TJ);
    static constexpr int LDSS = SK * 32 + 16;          // LDS row stride (bytes)
    static constexpr int PA = BM * SK / NT, PB = BN * SK / NT;   // pieces per thread
    static_assert((BM / 64) * WN == WAVES, "one 64 x 32*TJ tile per wave");
    static_assert(PA * NT == BM * SK && PB * NT == BN * SK && PA >= 1 && PB >= 1, "staging split");
};

template <int ABITS, int WBITS, int PA, int PB>
struct StageRegs {
    uint32_t a[PA][ABITS], b[PB][WBITS];
};

template <int ABITS, int WBITS, bool DEBUG, class CFG>
__global__ __launch_bounds__(CFG::NT, CFG::MINBLK) void qgemm_kernel(
    const uint8_t* __restrict__ A, int64_t M, int32_t a_row_bytes,
    const uint8_t* __restrict__ B, int32_t N, int32_t b_row_bytes,
    const GemmArgs ga, const float* __restrict__ s_w, const int32_t* __restrict__ colsum,
    float* __restrict__ Y, int32_t* __restrict__ acc_dbg, int32_t tiles_m, int32_t tiles_n,
    const QuantOutArgs qo, const ClusterArgs qc) {
    constexpr int BM = CFG::BM, BN = CFG::BN, SK = CFG::SK, LDSS = CFG::LDSS, NT = CFG::NT;
    constexpr int PA = CFG::PA, PB = CFG::PB, WN = CFG::WN, TJ = CFG::TJ, WW = 32 * TJ;
    constexpr int NPIECE = PA + PB;
    static_assert(NPIECE <= SK, "one staged piece per step");
    // both operands are unpacked to int8 on their way into LDS (once per
    // workgroup, where unpacking after the fragment reads would repeat it in
    // each of the two waves that read a fragment)
    __shared__ __align__(16) int8_t As[2][BM * LDSS];
    __shared__ __align__(16) int8_t Bs[2][BN * LDSS];
    constexpr int APIECE = 4 * ABITS, BPIECE = 4 * WBITS;           // bytes per 32 codes

    // ---- tile of this workgroup: undo the round-robin XCD dealing, then a
    // grouped (GROUP_M tile-rows at a time) column-major walk
    const int total = tiles_m * tiles_n;
    const int wg = blockIdx.x, xcd = wg & 7, q8 = total >> 3, r8 = total & 7;
    const int logical = (xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8) + (wg >> 3);
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (logical / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int bm = first_m + (logical % per_group) % gsize;
    const int bn = (logical % per_group) / gsize;
    const int64_t m0 = (int64_t)bm * BM;
    const int n0 = bn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;

    // cluster tables held one entry per lane (g <= 64) and read with readlane:
    // no scalar memory loads (and their waits) inside the K loop.  The two
    // vector loads complete here, before any prefetch is issued, so the
    // memory-counter waits inside the loop never have to cover them.
    // (lanes past g hold an end that is never reached, so the loop needs no
    // cluster count: a scalar load of it would be pending in the loop and
    // turn the waits there into waits for every LDS read)
    const int end_l = lane < ga.g ? ga.step_end[lane] : 0x7fffffff;
    float d_l;
    if (ga.dev_s) {
        // dynamic ranges: d_c = s_c - s_(c+1) from the device table, formed
        // like the host forms it for calibrated (s, z)
        const double sc = lane < ga.g ? (double)ga.dev_s[lane] : 0.0;
        const double sn = lane + 1 < ga.g ? (double)ga.dev_s[lane + 1] : 0.0;
        const double d = sc - sn;
        d_l = (float)(WBITS == 4 ? d * 0.0625 : WBITS == 3 ? d * 0.03125 : d);
    } else {
        d_l = lane < ga.g ? ga.scale[lane] : 0.0f;
    }
    asm volatile("" ::"v"(end_l), "v"(d_l) : "memory");

    // ---- staging: piece p = tid + i * NT covers row p / SK, step p % SK of a stage
    uint32_t a_voff[PA], b_voff[PB];
    int a_lds[PA], b_lds[PB], a_step[PA], b_step[PB];
#pragma unroll
    for (int i = 0; i < PA; ++i) {
        const int p = tid + i * NT, row = p / SK, part = p % SK;
        a_voff[i] = (uint32_t)(row * a_row_bytes + part * APIECE);
        a_lds[i] = row * LDSS + part * 32;
        a_step[i] = part;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
        const int p = tid + i * NT, row = p / SK, part = p % SK;
        b_voff[i] = (uint32_t)(row * b_row_bytes + part * BPIECE);
        b_lds[i] = row * LDSS + part * 32;
        b_step[i] = part;
    }
    const uint8_t* a_tile = A + m0 * a_row_bytes;
    const uint8_t* b_tile = B + (int64_t)n0 * b_row_bytes;
    const int64_t a_left = (M - m0) * a_row_bytes;
    const int64_t b_left = (int64_t)(N - n0) * b_row_bytes;
    const int nsteps = ga.nsteps;
    // stages, rounded up to an even count so the loop below always runs
    // whole pairs (a padding stage reads zero pieces and adds nothing); a
    // loop exit between the two halves would make the compiler's
    // memory-counter waits at the loop head conservative
    const int nst = ((nsteps + SK - 1) / SK + 1) & ~1;

    using Stage = StageRegs<ABITS, WBITS, PA, PB>;
    // Bytes from the tile's first row to the end of each operand, clamped to
    // 31 bits once, so that each stage's buffer size is scalar 32-bit
    // arithmetic (a 64-bit clamp per load would take vector compares).
    const int32_t a_left32 = __builtin_amdgcn_readfirstlane((int32_t)(a_left < 0 ? 0 : a_left > 0x7fffffff ? 0x7fffffff : a_left));
    const int32_t b_left32 = __builtin_amdgcn_readfirstlane((int32_t)(b_left < 0 ? 0 : b_left > 0x7fffffff ? 0x7fffffff : b_left));
    // piece k (A pieces first, then W' pieces) of stage st into register set S.
    // Stages past the end of K get an empty buffer (every load reads zero).
    // In the last stage, the steps past K: with 4-bit weights the W' row pitch
    // (64 bytes = 128 codes) covers whole stages and its tail is zero (the
    // weight packer writes it), so those steps read zero weights against
    // whatever codes follow the row and need no per-lane test; other widths
    // send those lanes' loads out of range.
    constexpr bool kStepTest = WBITS != 4;
    auto gload_piece = [&](Stage& S, int st, int k) {
        const int room = nsteps - st * SK;
        if (k < PA) {
            const int32_t ao = st * (SK * APIECE);
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(a_tile) + ao, (short)0, room > 0 ? max(a_left32 - ao, 0) : 0, kRsrcWord3);
            load_piece<ABITS>(r, !kStepTest || a_step[k] < room ? a_voff[k] : 0x80000000u, S.a[k]);
        } else {
            const int32_t bo = st * (SK * BPIECE);
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(b_tile) + bo, (short)0, room > 0 ? max(b_left32 - bo, 0) : 0, kRsrcWord3);
            load_piece<WBITS>(r, !kStepTest || b_step[k - PA] < room ? b_voff[k - PA] : 0x80000000u, S.b[k - PA]);
        }
    };
    auto gload = [&](Stage& S, int st) {
#pragma unroll
        for (int k = 0; k < NPIECE; ++k) gload_piece(S, st, k);
    };
    // stage piece k of register set S into LDS buffer buf
    auto put = [&](const Stage& S, int buf, int k) {
        uint32_t o[8];
        if (k < PA) {
            unpack_act<ABITS>(S.a[k], o);
            store32(&As[buf][a_lds[k]], o);
        } else {
            unpack_wgt<WBITS>(S.b[k - PA], o);
            store32(&Bs[buf][b_lds[k - PA]], o);
        }
    };

    // One running int32 accumulator per MFMA tile over the whole K loop, and
    // fp32 out.  With A_c the running sum at the end of cluster c,
    //   sum_c s_c (A_c - A_(c-1)) = sum_c (s_c - s_(c+1)) A_c,  s_(g+1) = 0,
    // so at each cluster end out += d_c * A_c and nothing is reset.
    v16i acc[2][TJ];
    float out[2][TJ][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            acc[i][j] = (v16i)0;
#pragma unroll
            for (int r = 0; r < 16; ++r) out[i][j][r] = 0.0f;
        }
    [[maybe_unused]] v16i prev[2][TJ];
    if constexpr (DEBUG) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) prev[i][j] = (v16i)0;
    }

    // accumulator register r of this lane holds row (r/4)*8 + (lane/32)*4 + r%4, column lane%32
    const int row_l = (lane >> 5) * 4, col_l = lane & 31;
    const int a_frag = (wm * 64 + (lane & 31)) * LDSS + (lane >> 5) * 16;
    const int b_frag = (wn * WW + (lane & 31)) * LDSS + (lane >> 5) * 16;

    int c = 0, c_end = __builtin_amdgcn_readfirstlane(end_l);

    auto flush = [&](int cl) {
        const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, d_l), cl));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    out[i][j][r] = __builtin_fmaf(d, (float)acc[i][j][r], out[i][j][r]);
                if constexpr (DEBUG) {
                    const int n = n0 + wn * WW + j * 32 + col_l;
                    const int add = (n < N && ga.code_offset) ? ga.code_offset * colsum[(int64_t)cl * N + n] : 0;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + row_l + (r & 3);
                        const int v = acc[i][j][r] - prev[i][j][r];
                        if (m < M && n < N)
                            acc_dbg[((int64_t)cl * M + m) * N + n] = (WBITS == 4 ? (v >> 4) : WBITS == 3 ? (v >> 5) : v) + add;
                    }
                    prev[i][j] = acc[i][j];
                }
            }
    };

    // Fragments: slot 0 holds the even steps, slot 1 the odd ones.  The
    // MFMAs of a stage's last step are deferred past the barrier: they need
    // only registers and cover the latency of the next stage's first
    // fragment reads, which cannot be issued before it.  (Slot 1 starts at
    // zero, so the deferred MFMAs before stage 0 add nothing.)
    v4i af[2][2], bf[2][TJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) af[1][i] = (v4i)0;
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[slot][i], bf[slot][j], acc[i][j], 0, 0, 0);
    };
    auto flush_if_end = [&](int steps_done) {
        if (steps_done == c_end) {
            flush(c);
            ++c;
            c_end = __builtin_amdgcn_readlane(end_l, c & 63);
        }
    };

    // One stage: SK MFMA steps from LDS buffer `buf`; the fragments of step
    // ks + 1 are read before the MFMAs of step ks, and piece ks of the next
    // stage's staging registers `nxt` is unpacked into the other buffer in
    // the same instruction stream and reloaded (on the last stage that buffer
    // is never read again, so the stores are harmless, and the reloads read
    // zero pieces past the end of K).
    auto compute = [&](int buf, int st, Stage& nxt) {
        auto rd = [&](int slot, int ks) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[slot][i] = *reinterpret_cast<const v4i*>(&As[buf][a_frag + i * 32 * LDSS + ks * 32]);
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                bf[slot][j] = *reinterpret_cast<const v4i*>(&Bs[buf][b_frag + j * 32 * LDSS + ks * 32]);
        };
        rd(0, 0);
        mfmas(1);                                  // last step of stage st - 1
        flush_if_end(st * SK);
        const bool last = st + 1 == nst;
#pragma unroll
        for (int ks = 0; ks < SK; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < SK) rd(cur ^ 1, ks + 1);
            if (ks + 1 < SK || last) mfmas(cur);
            if (ks < NPIECE) {
                put(nxt, buf ^ 1, ks);                  // unused on the last stage
                gload_piece(nxt, st + 3, ks);           // that piece is free again: reload it two stages ahead
            }
            // issue order inside the step (64 x 64 wave tiles; with 64 x 32
            // tiles the compiler's own order is as fast): each MFMA is
            // followed by part of the next step's fragment reads, the unpack
            // VALU work, and last the staging stores (so the reads never wait
            // behind them)
            if constexpr (TJ == 2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
            if (ks + 1 < SK || last) flush_if_end(st * SK + ks + 1);
        }
    };

    // ---- pipeline: during stage st, register set R[(st + 1) & 1] holds
    // stage st + 1, which is unpacked into the other LDS buffer piece by
    // piece, each piece reloaded with stage st + 3 right after its unpack (one
    // load per MFMA step rather than a burst); R[st & 1] has stage st + 2 in
    // flight.  Every load thus has about two stages to arrive.  One barrier
    // per stage.
    Stage R0, R1;
    gload(R0, 0);
    gload(R1, 1);
#pragma unroll
    for (int k = 0; k < NPIECE; ++k) put(R0, 0, k);
    gload(R0, 2);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        compute(0, st, R1);
        __syncthreads();
        compute(1, st + 1, R0);
        __syncthreads();
    }

    // ---- epilogue: Y = s_w * (out - corr), corr[n] = sum_c s_c (z_c - offset) colsum_c[n]
    // With a quantized output (the next layer's input, RPTQ write-up, method
    // and Fig. 3: the layer's weights are reordered so that it produces its
    // activations already in the next layer's sorted order), column n is the
    // next layer's SEG32 position n: Y (after ReLU when asked) is quantized
    // with that position's cluster (s, z) like every other activation, pad
    // positions get code 0, and the 128 x 128 code tile is packed through LDS.
    const bool quant = qo.q_codes != nullptr;
    uint8_t* ctile = reinterpret_cast<uint8_t*>(&As[0][0]);     // 128 x 128 codes
    if (quant) __syncthreads();                                 // every wave is done with the staging tiles
    const float qhi = kRoundMagic + (float)((1 << qc.bits) - 1);
    // Y of this tile through one buffer resource: rows past M lie outside it
    // (those stores are dropped), so an element needs only its 32-bit byte
    // offset (a tile spans at most BM * N * 4 < 2^31 bytes, checked at launch)
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(Y ? Y + m0 * N : nullptr, Y ? min(M - m0, (int64_t)BM) * N * 4 : 0);
    // colsum [g][N]: at most 64 x 4194303 int32, under 2^31 bytes
    const __amdgpu_buffer_rsrc_t rcs = make_rsrc(colsum, (int64_t)ga.g * N * 4);
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        const int n = n0 + wn * WW + j * 32 + col_l;
        if (n >= N) continue;
        // colsum[c][n] of every cluster, 16 loads in flight at a time (one
        // wait per 16 clusters, not one per cluster), then summed in cluster
        // order; clusters past g read as zero through the buffer's range
        double corr = 0.0;
        for (int c0 = 0; c0 < ga.g; c0 += 16) {
            int32_t cs[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                cs[k] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(
                    rcs, c0 + k < ga.g ? (uint32_t)(((c0 + k) * N + n) * 4) : 0x80000000u, 0, 0);
            if (ga.dev_s) {
                for (int k = 0; k < 16 && c0 + k < ga.g; ++k)
                    corr += (double)ga.dev_s[c0 + k] * ((double)ga.dev_z[c0 + k] - (double)ga.code_offset) *
                            (double)cs[k];
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (c0 + k < ga.g) corr += ga.sz[c0 + k] * (double)cs[k];
            }
        }
        // y = s_w (out - corr) as one fma: s_w * out exactly, plus the fp32
        // rounding of -s_w * corr (formed in fp64)
        const float swf = s_w[n], nswc = (float)(-(double)swf * corr);
        // the next layer's cluster of position n (pad positions: no cluster)
        float inv = 0.0f, zf = 0.0f;
        bool real = false;
        if (quant)
            for (int cc = 0; cc < qc.g; ++cc)
                if (n >= qc.off[cc]) {
                    real = n - qc.off[cc] < qc.bounds[cc + 1] - qc.bounds[cc];
                    inv = qc.inv_s[cc];
                    zf = (float)qc.z[cc];
                }
        uint32_t ybase = ((uint32_t)(wm * 64 + row_l) * (uint32_t)N + (uint32_t)n) * 4u;
        asm volatile("" : "+v"(ybase));         // keep one base + a scalar row offset per element
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = i * 32 + (r >> 2) * 8 + (r & 3);      // row within the wave tile
                const int rl = wm * 64 + dr + row_l;
                float y = __builtin_fmaf(swf, out[i][j][r], nswc);
                if (quant) {
                    if (qo.act) y = __builtin_fmaxf(y, 0.0f);
                    const uint32_t qb = quant_bits(y, inv, zf, qhi);
                    ctile[rl * 128 + wn * WW + j * 32 + col_l] = real ? (uint8_t)qb : 0;
                }
                if (Y)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __builtin_bit_cast(uint32_t, y), ry,
                        ybase + (uint32_t)__builtin_amdgcn_readfirstlane(dr * N * 4), 0, kStreamPolicy);
            }
    }
    if (quant) {
        __syncthreads();
        // 128 rows x 4 groups of 32 positions: two groups per thread
        constexpr int GPT = BM * (BN / 32) / NT;            // 32-position groups per thread
        static_assert(GPT * NT == BM * (BN / 32) && BN == 128, "code tile split");
#pragma unroll
        for (int k = 0; k < GPT; ++k) {
            const int gi = tid * GPT + k, rl = gi >> 2, grp = gi & 3;
            const int64_t m = m0 + rl;
            if (m >= M || n0 + grp * 32 >= N) continue;
            const u32x4 lo = *reinterpret_cast<const u32x4*>(ctile + rl * 128 + grp * 32);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(ctile + rl * 128 + grp * 32 + 16);
            const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};   // byte = code
            uint8_t* dst = qo.q_codes + m * qo.q_row_bytes + (int64_t)((n0 >> 5) + grp) * 4 * qc.bits;
            if (qc.bits == 8) {
                reinterpret_cast<u32x4*>(dst)[0] = lo;
                reinterpret_cast<u32x4*>(dst)[1] = hi;
            } else if (qc.bits == 4) {
                // unit u = codes 8u .. 8u+7: byte i holds code 8u+i and, in
                // its high nibble, code 8u+4+i
                *reinterpret_cast<u32x4*>(dst) =
                    u32x4{w[0] | w[1] << 4, w[2] | w[3] << 4, w[4] | w[5] << 4, w[6] | w[7] << 4};
            } else {
                // byte j of words d0, d1, d2: codes j, j+4 | j+8, j+12 | j+16,
                // j+20 in bits 0-2 / 3-5; codes j+24, j+28: low two bits in bits
                // 6-7 of d0 / d1, top bit in bit 6 / 7 of d2
                const uint32_t d0 = w[0] | w[1] << 3 | (w[6] & 0x03030303u) << 6;
                const uint32_t d1 = w[2] | w[3] << 3 | (w[7] & 0x03030303u) << 6;
                const uint32_t d2 = w[4] | w[5] << 3 | ((w[6] >> 2) & 0x01010101u) << 6 |
                                    ((w[7] >> 2) & 0x01010101u) << 7;
                reinterpret_cast<uint32_t*>(dst)[0] = d0;
                reinterpret_cast<uint32_t*>(dst)[1] = d1;
                reinterpret_cast<uint32_t*>(dst)[2] = d2;
            }
        }
    }
}

using CfgNarrow = TileCfg<128, 128, 8, 4, 2, 1>;      // 3/4-bit operands: 64 x 32 wave tiles
using CfgWide = TileCfg<128, 128, 4, 4, 2, 2>;        // an 8-bit operand: 64 x 64 wave tiles
static_assert(CfgNarrow::BM == CfgWide::BM && CfgNarrow::BN == CfgWide::BN, "one tile grid");
using Cfg = CfgWide;

template <int ABITS, int WBITS>
using CfgFor = std::conditional_t<(ABITS <= 4 && WBITS <= 4), CfgNarrow, CfgWide>;

template <int ABITS, int WBITS>
const void* pick2(bool debug) {
    using C = CfgFor<ABITS, WBITS>;
    return debug ? (const void*)qgemm_kernel<ABITS, WBITS, true, C> : (const void*)qgemm_kernel<ABITS, WBITS, false, C>;
}

int threads_for(int a_bits, int w_bits) { return a_bits <= 4 && w_bits <= 4 ? CfgNarrow::NT : CfgWide::NT; }

template <int ABITS>
const void* pick(int wbits, bool debug) {
    return wbits == 3 ? pick2<ABITS, 3>(debug) : wbits == 4 ? pick2<ABITS, 4>(debug) : pick2<ABITS, 8>(debug);
}

}  // namespace

hipError_t launch_qgemm(const uint8_t* codes, int64_t M, int32_t N, int64_t a_row_bytes,
                        int a_bits, const uint8_t* w_packed, int64_t w_row_bytes, int w_bits,
                        const GemmArgs& ga, const float* s_w, const int32_t* colsum,
                        float* Y, int32_t* acc_debug, const QuantOutArgs& qo, const ClusterArgs& qc,
                        hipStream_t stream) {
    const bool dbg = acc_debug != nullptr;
    const void* k = a_bits == 3 ? pick<3>(w_bits, dbg) : a_bits == 4 ? pick<4>(w_bits, dbg) : pick<8>(w_bits, dbg);
    const int64_t tm = (M + Cfg::BM - 1) / Cfg::BM, tn = (N + Cfg::BN - 1) / Cfg::BN;
    static_assert((int64_t)kMaxGemmN * 4 * std::max(CfgNarrow::BM, CfgWide::BM) <= 0x7fffffff, "Y tile window");
    if (tm * tn > 0x7fffffff || a_row_bytes > (1 << 20) || w_row_bytes > (1 << 20) || N > kMaxGemmN)
        return hipErrorInvalidValue;
    int32_t tiles_m = (int32_t)tm, tiles_n = (int32_t)tn;
    int32_t arb = (int32_t)a_row_bytes, wrb = (int32_t)w_row_bytes;
    void* args[] = {(void*)&codes, (void*)&M, (void*)&arb, (void*)&w_packed, (void*)&N, (void*)&wrb,
                    (void*)&ga, (void*)&s_w, (void*)&colsum, (void*)&Y, (void*)&acc_debug,
                    (void*)&tiles_m, (void*)&tiles_n, (void*)&qo, (void*)&qc};
    return hipLaunchKernel(k, dim3((unsigned)(tm * tn)), dim3(threads_for(a_bits, w_bits)), args, 0, stream);
}

}  // namespace rptq
