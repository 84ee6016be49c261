// Internal declarations shared by the host-side C ABI (rptq_api.cpp) and the
// HIP kernel sources of the library.  Not installed; not part of the ABI.
#pragma once

#include <cstdint>
#include <hip/hip_runtime.h>

namespace rptq {

constexpr int kMaxClusters = 64;
constexpr int kMaxK = 16384;
constexpr int kMaxGemmN = 4194303;     // GEMM N: 128 rows x N fp32 of a Y tile < 2^31 bytes
constexpr int kMaxBlock = 512;         // largest workgroup of the streaming kernels
constexpr int kKvPackMaxBlock = 1024;  // K/V pack: one wide workgroup per compute unit
constexpr int kMaxUpl = 5;             // most units (8 codes each) one lane handles
#ifndef RPTQ_LN_MAX_BLOCK
#define RPTQ_LN_MAX_BLOCK 256          // LayerNorm kernel: fewer, fatter lanes (two workgroups per CU)
#endif

// Workgroup size and units per lane for a row of n_units units: the smallest
// units-per-lane whose workgroup (rounded up to whole waves) fits pref_block,
// else fits kMaxBlock; upl = 0 if the row is too long for either.
inline void unit_split(int n_units, int& upl, int& block, int pref_block = kMaxBlock) {
    for (int cap : {pref_block, kMaxBlock}) {
        for (upl = 1; upl <= kMaxUpl; ++upl) {
            block = ((n_units + upl - 1) / upl + 63) / 64 * 64;
            if (block <= cap) return;
        }
    }
    upl = 0;
    block = 0;
}

// Cluster table, passed by value as a kernel argument (about 1.6 KB, well
// under the kernel-argument limit).  Built and validated on the host.
struct ClusterArgs {
    int32_t g;
    int32_t K;                          // real channels (bounds[g])
    int32_t K_pad;                      // SEG32 padded length (0 when unused)
    int32_t bits;
    int32_t bounds[kMaxClusters + 1];   // reordered-position boundaries
    int32_t off[kMaxClusters + 1];      // SEG32 padded offsets
    float inv_s[kMaxClusters];          // fp32(1 / s_c)
    float s[kMaxClusters];
    int32_t z[kMaxClusters];
};

// Magic constant 1.5 * 2^23: adding it to |v| < 2^22 rounds v half-to-even to
// an integer held in the low mantissa bits.
constexpr float kRoundMagic = 12582912.0f;
constexpr int32_t kRoundMagicBits = 0x4B400000;

// Per-cluster tables of the GEMM, passed by value.
struct GemmArgs {
    int32_t g;
    int32_t nsteps;                        // K_pad / 32
    int32_t step_end[kMaxClusters];        // exclusive end (in 32-code steps) of cluster c
    float scale[kMaxClusters];             // (s_c - s_(c+1)) divided by the weight pre-scale
    double sz[kMaxClusters];               // s_c * (z_c - code offset), for the epilogue
    int32_t code_offset;                   // 128 for 8-bit activations (stored q - 128), else 0
    // device-resident (s, z) [g] (dynamic ranges): when set, the kernel forms
    // scale[] and sz[] from them itself and the two tables above are unused
    const float* dev_s;
    const int32_t* dev_z;
};

// Launchers (one per kernel family); each returns the launch status.
hipError_t launch_ln_reorder_quant(const void* x, int in_mode, int64_t M, int32_t K,
                                   const float* gamma_r, const float* beta_r, float eps,
                                   const int32_t* R, const ClusterArgs& ca, int64_t row_bytes,
                                   uint8_t* codes, hipStream_t stream);

// Dynamic ranges: per-workgroup (lo, hi) partials of every cluster (at most
// kLnRangesMaxGrid workgroups, 2 g floats each, in `partials`), then (s, z)
// into s_out / z_out (device [g]), then the quantization with them.
constexpr int kLnRangesMaxGrid = 1024;
hipError_t launch_ln_reorder_quant_dynamic(const void* x, int in_mode, int64_t M, int32_t K,
                                           const float* gamma_r, const float* beta_r, float eps,
                                           const int32_t* R, const ClusterArgs& ca, int64_t row_bytes,
                                           uint8_t* codes, float* s_out, int32_t* z_out, float* partials,
                                           hipStream_t stream);

// Allocation-free dynamic ranges: the partials live in a library-owned
// device array (one per GPU) instead of a caller workspace.  Its size, and
// its device address on the current device (looked up on first use).
int64_t ln_dynamic_scratch_bytes();
hipError_t ln_dynamic_scratch(void** ptr);

hipError_t launch_kv_quant_pack(const uint16_t* kv, int64_t T, int32_t C, const int32_t* R,
                                const ClusterArgs& ca, uint8_t* packed, hipStream_t stream);

hipError_t launch_kv_dequant(const uint8_t* packed, int64_t T, int32_t C, const int32_t* R,
                             const ClusterArgs& ca, uint16_t* out, hipStream_t stream);

// Decode attention over packed K/V (chunked, then merged); workspace holds
// the per-chunk partial outputs and softmax statistics.
constexpr int kAttnMaxC = 5 * 256 * 8;   // 256 lanes x 5 units of 8 channels
void kv_attention_geometry(int32_t T, int32_t C, int32_t D, int32_t& TC, int32_t& nch);
int64_t kv_attention_workspace(int32_t B, int32_t T, int32_t C, int32_t D);
hipError_t launch_kv_attention(const uint16_t* q, const uint8_t* kp, const uint8_t* vp, int32_t B, int32_t T,
                               int32_t C, int32_t D, float scale, const int32_t* Rk, const ClusterArgs& ck,
                               const int32_t* Rv, const ClusterArgs& cv, float* out, void* workspace,
                               hipStream_t stream);

hipError_t launch_calib_minmax(const uint16_t* x, int mode, int64_t M, int32_t K,
                               const float* gamma, const float* beta, float eps,
                               float* mx, float* mn, hipStream_t stream);

// Quantized output of the GEMM (the epilogue quantizes Y for the next layer):
// q_codes null = none.  N is then the next layer's SEG32 K_pad and column n
// the padded position n; act 1 applies ReLU to Y first.
struct QuantOutArgs {
    uint8_t* q_codes;                      // device [M][q_row_bytes] SEG32, or null
    int64_t q_row_bytes;
    int32_t act;
};

hipError_t launch_qgemm(const uint8_t* codes, int64_t M, int32_t N, int64_t a_row_bytes,
                        int a_bits, const uint8_t* w_packed, int64_t w_row_bytes, int w_bits,
                        const GemmArgs& ga, const float* s_w, const int32_t* colsum,
                        float* Y, int32_t* acc_debug, const QuantOutArgs& qo, const ClusterArgs& qc,
                        hipStream_t stream);

// Number of workgroups a persistent streaming kernel should launch: the
// device's compute units times the resident workgroups per unit.
int persistent_grid(const void* kernel, int block, size_t lds_bytes, int64_t rows);

}  // namespace rptq
