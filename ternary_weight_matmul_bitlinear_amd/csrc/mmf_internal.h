// mmf_internal.h -- declarations shared by the host dispatch code and the HIP kernels of
// libmmf (gfx950).  Not part of the public ABI (include/mmf.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "mmf.h"

namespace mmf {

// ------------------------------------------------------------------ device helpers
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in bits 0-15), round to nearest even, one instruction
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

__device__ __forceinline__ float round_to_bf16(float f) {
    return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

template <bool BF16>
__device__ __forceinline__ float load_act(const void *p, int64_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    else return static_cast<const float *>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_act(void *p, int64_t i, float v) {
    if constexpr (BF16) static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(v);
    else static_cast<float *>(p)[i] = v;
}

// Logistic sigmoid and SiLU on the hardware transcendental units: 2^x (v_exp_f32) and
// 1/x (v_rcp_f32), each accurate to about 1 ulp.  sigmoid(z) = 1 / (1 + 2^(-z*log2 e));
// large positive z gives exactly 1, large negative z gives exactly 0.
__device__ __forceinline__ float sigmoidf_(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}
__device__ __forceinline__ float siluf_(float z) { return z * sigmoidf_(z); }

// Wave-wide (64 lanes) reductions through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum (or max) of N values per lane over groups of G lanes (G in {16, 32, 64}), N a power
// of two <= G: halving exchanges (each lane keeps the half of the vector picked by its lane
// bit) while more than one value is left, then a plain butterfly.  On return lane l holds
// the group total of value index (l % G) >> (log2 G - log2 N).
template <int N, bool MAX, typename T, int G = 64>
__device__ __forceinline__ T wave_reduce_multi(T (&v)[N]) {
    static_assert((N & (N - 1)) == 0 && N <= G, "N must be a power of two <= G");
    const int lane = threadIdx.x & 63;
    T w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = v[i];
    int n = N;
#pragma unroll
    for (int bit = G / 2; bit > 0; bit >>= 1) {
        if (n > 1) {
            // keep/send picked with an xor blend (a select of w[i] vs w[i + h] on the lane bit
            // is otherwise turned into a dynamically indexed register read)
            const uint32_t m = (lane & bit) ? 0xFFFFFFFFu : 0u;
            const int h = n / 2;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                if (i < h) {
                    const uint32_t lo_b = __builtin_bit_cast(uint32_t, w[i]);
                    const uint32_t hi_b = __builtin_bit_cast(uint32_t, w[i + h]);
                    const uint32_t x = (lo_b ^ hi_b) & m;
                    const T send = __builtin_bit_cast(T, hi_b ^ x);   // lane bit set: w[i]
                    const T keep = __builtin_bit_cast(T, lo_b ^ x);   // lane bit set: w[i + h]
                    const T recv = __shfl_xor(send, bit, 64);
                    w[i] = MAX ? (keep > recv ? keep : recv) : keep + recv;
                }
            }
            n = h;
        } else {
            const T o = __shfl_xor(w[0], bit, 64);
            w[0] = MAX ? (w[0] > o ? w[0] : o) : w[0] + o;
        }
    }
    return w[0];
}

// Ternary unpack: word j of a packed row holds k = 16j + 4a + b at bits 8b + 2a; the
// dword (w >> 2a) & 0x03030303 therefore holds the codes of k = 16j + 4a + 0..3 as four
// int8 lanes.  The returned 128-bit vector holds the 16 codes of word j in k order.
__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
    v4i r;
    r.x = static_cast<int>(w & 0x03030303u);
    r.y = static_cast<int>((w >> 2) & 0x03030303u);
    r.z = static_cast<int>((w >> 4) & 0x03030303u);
    r.w = static_cast<int>((w >> 6) & 0x03030303u);
    return r;
}

// ------------------------------------------------------------ launch descriptors

// Kernel families for per-launch timing (host side, mmf_api.cpp).
enum Family : int {
    FAM_QUANT = 0,
    FAM_GEMM_IFG,
    FAM_GEMM_O,
    FAM_GEMM_GATEUP,
    FAM_GEMM_DOWN,
    FAM_GEMM_OTHER,
    FAM_GEMV,
    FAM_SCAN,
    FAM_EMBED,
    FAM_COUNT
};

void timing_begin(int family, hipStream_t s);
void timing_end(int family, hipStream_t s);


// Optional stage capture, in device pointers (see mmf_stage_capture).
struct CapDev {
    int64_t row0 = 0, row1 = 0;
    float *x_in = nullptr;
    int8_t *q = nullptr;
    float *a = nullptr;
    int32_t *acc = nullptr;
    float *y_out = nullptr;  // stored output of the stage, widened to fp32 (row stride ldo)
    int32_t acc_ld = 0;   // row stride of acc (group width)
    int32_t acc_col0 = 0; // column offset of this launch inside the group
};

// Row quantizer: x [M][K] -> q [M][K] int8, a [M], rowsum [M].
struct QuantArgs {
    const void *x;
    int x_bf16;
    const float *gamma;
    float eps;
    int64_t M;
    int32_t K;
    int8_t *q;
    float *a;
    int32_t *rowsum;
    CapDev cap;
};

// One weight matrix inside a (possibly concatenated) BitLinear launch.
struct Seg {
    const uint32_t *packed = nullptr;
    const float *bias = nullptr;
    float scale = 0.f;
    int32_t n = 0;        // rows of this matrix
    int32_t out_col0 = 0; // first output column of this matrix
    int32_t cap_col0 = 0; // first capture column of this matrix
};

enum Epi : int {
    EPI_STORE = 0,  // y = acc*s*a (+bias)
    EPI_RESID = 1,  // y = resid + acc*s*a (+bias)
    EPI_GLU = 2     // segments 0,1 = gate,up: y = SiLU(gate) * up
};

// Prefill int8-MFMA GEMM with ternary weights.
struct GemmArgs {
    const int8_t *A;       // [M][K] int8 activations
    const int32_t *rowsum; // [M]
    const float *a;        // [M]
    int64_t M;
    int32_t K;
    Seg seg[3];
    int32_t nseg;
    int32_t tiles_n[3];    // N tiles per segment (EPI_GLU: tiles of 64 gate/up pairs)
    int32_t tiles_n_total;
    int32_t tiles_total;   // M tiles x tiles_n_total (set by the launcher)
    int32_t epi;
    void *out;
    int32_t ldo;
    int32_t out_bf16;
    const void *resid;     // [M][ldr] (EPI_RESID), same dtype as out
    int32_t ldr;
    CapDev cap;            // acc capture only
    int32_t family = FAM_GEMM_OTHER;
};

// Decode GEMV (weight streaming).  Input either raw activations (quantized in the
// prologue) or pre-quantized rows.
struct GemvArgs {
    const void *x;         // [M][K] raw activations, or NULL when q is given
    int32_t x_bf16;
    const float *gamma;
    float eps;
    const int8_t *q;       // [M][K] pre-quantized (when x == NULL)
    const float *a;
    const int32_t *rowsum;
    int64_t M;
    int32_t K;
    Seg seg[3];
    int32_t nseg;
    int32_t rows_total;    // sum of segment rows (EPI_GLU: F, the pair count)
    int32_t epi;
    void *out;
    int32_t ldo;
    int32_t out_bf16;
    const void *resid;     // same dtype as out
    int32_t ldr;
    int32_t tokens_per_group;  // rows of q staged in LDS per workgroup (<= kGemvTokens)
    CapDev cap;            // x_in/q/a written by column-block 0, acc by every block
    // one MLGRU step as the input (mlgru != 0, one token, K = D <= 4096): x is the token's
    // i|f|g pre-activations [3D] in the output dtype; gamma/eps are o_proj's
    int32_t mlgru;
    const float *h_prev;   // [D] carried state (NULL: zeros)
    float *h_new;          // [D] new state, written by column-block 0 (NULL: not kept)
    const float *f_bias;   // [D] or NULL
    const float *gnorm_w;  // [D] or NULL (ones)
    float g_eps;
    int32_t gate_mode;
    // optional side copy of copy_n floats (a multiple of 4), done by the first workgroups
    const float *copy_src;
    float *copy_dst;
    int32_t copy_n;
};

// MLGRU scan.
struct ScanArgs {
    const void *ifg;       // [B][T][3D]
    int32_t ifg_bf16;
    const float *f_bias;
    const float *h0;
    float *h_out;
    const float *gnorm_w;
    float eps;
    int32_t gate_mode;
    int64_t B, T;
    int32_t D;
    int32_t chunk;         // tokens per chunk
    int32_t n_chunks;
    float *hloc;           // [B][n_chunks][D] local end state (phase 1)
    float *pf;             // [B][n_chunks][D] product of f over the chunk (phase 1)
    float *hin;            // [B][n_chunks][D] state entering each chunk (phase 2)
    // output: either the gated activation or its int8 quantization for o_proj
    void *out;             // [B*T][D] (out_bf16) when q == NULL
    int32_t out_bf16;
    int8_t *q;             // [B*T][D]
    float *a;
    int32_t *rowsum;
    const float *q_gamma;  // o_proj input gain
    float q_eps;           // o_proj input eps
    CapDev cap;            // x_in/q/a of the o_proj stage
};

// ---------------------------------------------------------------- launchers
hipError_t launch_quant(const QuantArgs &a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemv(const GemvArgs &a, hipStream_t s);
hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
hipError_t launch_embedding(const uint32_t *packed, float scale, int64_t vocab, int32_t D,
                            const int32_t *ids, int64_t m, void *x, int bf16,
                            hipStream_t s);
hipError_t launch_copy_state(const float *h0, float *h_out, int64_t n, hipStream_t s);

// Token rows up to which the MFMA regime uses the mid-size kernel (gemm_mid.hip): weights
// read once per launch, k split over the waves of a workgroup.
constexpr int64_t kMidMaxM = 64;
bool mid_gemm_supported(const GemmArgs &a);
hipError_t launch_gemm_mid(const GemmArgs &a, hipStream_t s);

// Tokens per decode-kernel token group (rows of q staged in LDS).
constexpr int kGemvTokens = 8;
// Chunk length of the prefill scan (tokens per workgroup of the output pass).
constexpr int kScanChunk = 16;

}  // namespace mmf
