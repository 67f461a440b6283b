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

// Round two fp32 values to bf16 (nearest even) in place, widened back to fp32: one
// v_cvt_pk_bf16_f32 and two bit operations.
__device__ __forceinline__ void round_bf16_pair(float &lo, float &hi) {
    const uint32_t w = pack_bf16x2(lo, hi);
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
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

// s_waitcnt with only the vector-memory counter constrained (expcnt, lgkmcnt at maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One 16-byte-per-lane direct load from global memory into LDS: lane l reads 16 bytes at
// base + off_l (base wave-uniform, in SGPRs; off_l a 32-bit lane offset) and they land at
// LDS byte address lds + 16*l (lds wave-uniform, passed in M0).  Issued from inline
// assembly so that the compiler does not order every later LDS read after it (the caller
// orders them: vmcnt waits and barriers); the instruction has no register result.
// M0 is saved and restored around it.
__device__ __forceinline__ void dma16(const void *base_p, uint32_t off, uint32_t lds) {
    const uint64_t b = reinterpret_cast<uintptr_t>(base_p);
    // readfirstlane yields a signed int: take each half back to uint32_t before widening,
    // or a low half with bit 31 set would be sign-extended into the high half
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
    const uint64_t base = (static_cast<uint64_t>(hi) << 32) | lo;
    lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds)
        : "memory");
}

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
    FAM_BWD_G,      // backward: g = s_w dy T
    FAM_BWD_DW,     // backward: dW = (dy a)^T q
    FAM_BWD_SCAN,   // backward: MLGRU + output gate
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
    EPI_GLU = 2,    // segments 0,1 = gate,up: y = SiLU(gate) * up
    EPI_GLU_KEEP = 3  // as EPI_GLU, and gate | up also stored in bf16 to keep [M][2F]
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
    uint16_t *keep = nullptr;  // [M][2F] bf16 gate | up pre-activations (EPI_GLU_KEEP)
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
    // one MLGRU step as the input (mlgru != 0, M <= 4 sequences of one token each, one per
    // grid row, K = D <= 4096): x is [M][3D] i|f|g pre-activations in the output dtype;
    // gamma/eps are o_proj's
    int32_t mlgru;
    const float *h_prev;   // [M][D] carried state (NULL: zeros)
    float *h_new;          // [M][D] new state, row m written by workgroup (0, m) (NULL: not kept)
    const float *f_bias;   // [D] or NULL
    const float *f_lower;  // [D] forget-gate lower bound or NULL (zeros)
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
    const float *f_lower;  // [D] forget-gate lower bound or NULL (zeros)
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

// Decode BitLinear over base-3 packed weights (five per byte, rows of row_bytes bytes).
struct TritArgs {
    const void *x;         // [M][K] activations (quantized in the prologue)
    int32_t x_bf16;
    const float *gamma;
    float eps;
    int64_t M;
    int32_t K;
    int32_t row_bytes;     // 16 * ceil(K / 80)
    const uint8_t *packed; // [N][row_bytes]
    float scale;
    const float *bias;
    int32_t N;
    void *out;             // [M][N]
    int32_t out_bf16;
    CapDev cap;            // x_in/q/a by column-block 0, acc/y_out by every block (stride N)
};

// One decode step of a whole stack for one sequence in one cooperative launch
// (decode_persistent.hip).  The layer table lives in device memory (the caller's workspace).
struct PLayer {
    const uint32_t *w[7];        // packed i, f, g, o, gate, up, down
    float s[7];                  // their absmean scales
    const float *b[7];           // their biases (nullable)
    const float *g_x, *g_o, *g_gu, *g_down;   // input RMSNorm gains (nullable)
    float e_x, e_o, e_gu, e_down;
    const float *f_bias, *f_lower, *gnorm_w;
    float g_eps;
    int32_t gate_mode;
};
struct PersistArgs {
    const PLayer *layers;
    int32_t L, D, F, V;
    const uint32_t *emb;
    float emb_scale;
    int64_t vocab;
    const uint32_t *head;
    float head_scale;
    const float *head_bias, *head_gamma;
    float head_eps;
    const int32_t *ids;          // [1]
    float *h_state;              // [L][D]
    float *logits;               // [V] or NULL
    void *y;                     // [D] bf16 or NULL
    uint64_t *xch;               // exchange words
    uint32_t *ctl;               // [0] epoch, [1] finished workgroups, [2] timeout flag
    int64_t spin_ticks;          // bound of every wait, in 100 MHz ticks
    uint64_t *trace;             // NULL, or [2 * (4 * L + 2)] 100 MHz stamps of workgroup 0:
                                 // the kernel's start, the (start, end) of each layer's waits
                                 // for x (l > 0), i|f|g, y1 and the GLU hidden, the head's
                                 // wait, the end of the work
};
int persist_limits(int *max_units, int *max_words, int *max_k, int *max_d, int *max_rows);
int persist_max_units(int rows, int K);
void persist_stage_units(int (&u)[5]);   // per-stage unit bounds: i|f|g, o, gate|up, down, head
int persist_occupancy(int D, int F, int *blocks_per_cu);
hipError_t launch_decode_persistent(const PersistArgs &a, int grid, hipStream_t s);

// Straight-through BitLinear backward (backward.hip).
struct BitlinearBwdArgs {
    const void *x;         // [M][K] forward input
    int32_t x_bf16;
    const float *gamma;    // [K] or NULL
    float eps;
    int64_t M;
    int32_t K, N;
    const uint32_t *packed;  // [N][K/16]
    float scale;
    const void *dy;        // [M][N]
    int32_t dy_bf16;
    const int8_t *q;       // [M][K] codes of the forward quantizer (workspace)
    const float *a;        // [M] its dequantization scales (workspace)
    float *g;              // [M][K] fp32 gradient at the normalised input (workspace)
    uint16_t *wt;          // [K][N] bf16 copy of the ternary matrix, transposed (workspace)
    int64_t ldm;           // M rounded up to 64: row length of the two copies below
    uint16_t *dyaT;        // [N][ldm] bf16 (dy * a) transposed (workspace)
    uint16_t *qT;          // [K][ldm] bf16 q transposed (workspace)
    float *dg_part;        // bwd_rows_part_bytes(M, K) (workspace)
    float *dx;             // [M][K] or NULL
    float *dgamma;         // [K] or NULL
    float *dw;             // [N][K] or NULL
    float *db;             // [N] or NULL
};

// MLGRU + output gate backward (backward.hip).
struct MlgruBwdArgs {
    const void *ifg;       // [B][T][3D]
    int32_t ifg_bf16;
    const float *f_bias, *f_lower, *h0, *gnorm_w;
    float eps;
    int32_t gate_mode;
    int64_t B, T;
    int32_t D;
    int32_t n_chunks;      // chunks of 16 tokens
    const float *hin;      // [B][n_chunks][D] state entering each chunk (chunk 0: h0)
    const void *dout;      // [B][T][D]
    int32_t dout_bf16;
    const float *dh_last;  // [B][D] or NULL
    void *d_ifg;           // [B][T][3D], fp32 (or bf16 when d_ifg_bf16)
    int32_t d_ifg_bf16;
    float *dh0;            // [B][D] or NULL
    float *dgnorm_w;       // [D] or NULL
    float *df_bias;        // [D] or NULL
    // workspace
    float *stats;          // [B][T][2] per token rho and rho^3/D * sum(dn*h) (gate mode 0)
    float *cb, *cp, *cf0, *cg;  // [B][n_chunks][D] per-chunk scan values
    float *gw_part, *fb_part;   // [B][n_chunks][D] per-chunk partial sums
};

// ---------------------------------------------------------------- launchers
hipError_t launch_quant(const QuantArgs &a, hipStream_t s);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemv(const GemvArgs &a, hipStream_t s);
hipError_t launch_scan(const ScanArgs &a, hipStream_t s);
// phases 1 and 2 of the scan only: the state entering every chunk into a.hin (n_chunks > 1)
hipError_t launch_scan_carries(const ScanArgs &a, hipStream_t s);
hipError_t launch_bitlinear_bwd(const BitlinearBwdArgs &a, hipStream_t s);
hipError_t launch_mlgru_bwd(const MlgruBwdArgs &a, hipStream_t s);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s);
// backward pieces (backward.hip).  Up to three linears that share an input are handled
// together: their output gradients sit side by side in dy [M][ldy] (N columns each).
// Ternary matrices expanded to bf16 W^T: out[k][n] (row stride ldo) = T[n][k], up to seven
// per launch.
struct ExpandJobs {
    const uint32_t *packed[7];
    int32_t N[7], K[7];
    uint16_t *out[7];
    int64_t ldo[7];
    int32_t count;
};
hipError_t launch_expand_wt(const ExpandJobs &j, hipStream_t s);
// g = sum_j scale_j * dy_j T_j  [M][K] fp32 (one launch when N % 64 == 0); wt: [K][nseg*N]
// bf16, filled here unless `expanded` (then it already holds the stacked W^T).
hipError_t bwd_launch_g(const void *dy, int dy_bf16, int64_t ldy, const uint32_t *const *packed,
                        const float *scales, int nseg, int32_t N, int32_t K, int64_t M, uint16_t *wt,
                        int expanded, float *g, hipStream_t s);
// dx / dgamma from g (and the residual gradient, and the GLU product's backward)
struct BwdRowsArgs {
    const void *x;          // [M][K] forward input of the normalisation
    int32_t x_bf16;
    const float *g;         // [M][K]
    const float *gamma;     // [K] or NULL
    float eps;
    int64_t M;
    int32_t K;              // K % 4 == 0, K <= 8192
    float *dx;              // [M][K] fp32 or NULL
    uint16_t *dx_bf16;      // [M][K] bf16 copy or NULL
    const void *res;        // [M][K] residual gradient added to dx, or NULL
    int32_t res_bf16;
    const uint16_t *gu;     // GLU mode: gate | up pre-activations [M][2K] bf16 ...
    uint16_t *dgu;          // ... and dgate | dup [M][2K] bf16 out (dx, dx_bf16 unused)
    float *dgamma;          // [K] or NULL
    int32_t dgamma_zeroed;  // the caller has zeroed dgamma
    float *dg_part;         // workspace: bwd_rows_part_bytes(M, K)
};
size_t bwd_rows_part_bytes(int64_t M, int32_t K);
hipError_t bwd_launch_rows(const BwdRowsArgs &a, hipStream_t s);
hipError_t bwd_launch_qT(const int8_t *q, int64_t M, int32_t K, int64_t ldm, uint16_t *qT, hipStream_t s);
// dW_j = (dy_j a)^T q  [N][K] each, into dw[j] (NULL: not wanted); db_j = sum_M dy_j into db[j]
// (NULL: not wanted).  dyaT: [nseg*N][ldm] bf16 scratch; qT from bwd_launch_qT.  zeroed: the
// caller has zeroed dw and db (they are then only added to).
hipError_t bwd_launch_dw(const void *dy, int dy_bf16, int64_t ldy, const float *a, int64_t M, int nseg,
                         int32_t N, int32_t K, int64_t ldm, const uint16_t *qT, uint16_t *dyaT,
                         float *const *dw, float *const *db, int zeroed, hipStream_t s);
// up to kMax arrays zeroed by one launch (NULL entries skipped)
struct ZeroJobs {
    static constexpr int kMax = 24;
    float *p[kMax];
    int64_t n[kMax];
    int32_t count;
};
hipError_t launch_fill_zero_many(const ZeroJobs &j, hipStream_t s);
hipError_t launch_embedding(const uint32_t *packed, float scale, int64_t vocab, int32_t D,
                            const int32_t *ids, int64_t m, void *x, int bf16,
                            hipStream_t s);
hipError_t launch_copy_state(const float *h0, float *h_out, int64_t n, hipStream_t s);
hipError_t launch_gemv_trits(const TritArgs &a, hipStream_t s);

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
