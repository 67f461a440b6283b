// backward.hip -- gradients of the BitLinear and of the MLGRU with its output gate, for
// training the latent weights (gfx950).
//
// DataCamp "MatMul-free language models": section "Replacing MatMul with ternary
// operations" -- the weights are trained in full precision and ternarized during training;
// section "From optimised GPU to custom FPGA" -- fused training kernels.  The gradient
// crosses the two quantizers straight through: the activation quantizer's dequantized output
// x_hat = q*a passes its gradient to u = x*gamma*r (the RMS-normalised input it
// approximates), the ternarizer's W_hat = s_w*T to the latent weights.
//
// BitLinear (y = x_hat W_hat^T + b), given dy [M][N]:
//   g  = s_w * dy T          [M][K]   bf16 matrix cores over n; T is expanded once to a
//                                     bf16 [K][N] copy (values -1/0/1, exact)
//   dW = (dy*a)^T q_x        [N][K]   bf16 matrix cores over tokens; (dy*a) and q_x are
//                                     first transposed to bf16 [.][m] copies, and the
//                                     token range is split over workgroups (fp32 atomics)
//   dx = r*gamma*g - x*r^3/K * sum_K(g*gamma*x),  dgamma = sum_M g*x*r,  db = sum_M dy
// Both contractions are one kernel with the contraction index contiguous in both operands,
// so its k loop moves only 16-byte vectors.  q_x and a are recomputed by the forward
// quantizer; dy enters the matrix cores rounded to bf16 (exact when dy is bf16), (dy*a)
// rounded to bf16 for dW; accumulation is fp32.
//
// MLGRU + output gate, given dout [B][T][D] (and dh_T): the forward's chunk carries give
// the state entering every 16-token chunk, then
//   phase 1 (gate mode 0; workgroup per chunk, whole rows of D): rerun the recurrence and
//     reduce per token sum h^2 and sum dn*h (dn = dout*w*silu(g)), all 32 sums of a chunk
//     in one LDS reduction; store rho and rho^3/D * sum dn*h per token;
//   phase 2 (thread per chunk and channel): rerun the chunk forward, form the gradient at
//     h from the output gate (dh = rho*dn - h*k3, or dout*sigmoid(g)) and dg, then the
//     chunk's reverse scan of G_t = dh_t + f_{t+1} G_{t+1} from zero, keeping its value at
//     the first token, the product of f over the chunk after the first token, and f at the
//     first token;
//   phase 3 (thread per channel): carry G backwards across chunks; dh0 = f_0 G_0;
//   phase 4 (as phase 2): walk the chunk backwards with the carried G:
//     di = (1-f) G silu'(i), df_pre = (h_{t-1} - c) G (1-lb) sigma'(z).
// Per-chunk partial sums of dgnorm_w and df_bias are reduced by a column-sum kernel.
#include "mmf_internal.h"

namespace mmf {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GT = 256;          // threads of a GEMM workgroup (2 x 2 waves)
constexpr int BR = 128, BS = 128;  // output tile rows x columns

__device__ __forceinline__ uint16_t bf16_bits(float v) { return f32_to_bf16_bits(v); }

// 16 consecutive activations (bf16 or fp32) from element idx on, times mul, as bf16 bits;
// elements at or past `valid` read as zero.  Full chunks are read with 16-byte loads.
template <bool BF16>
__device__ __forceinline__ void load16(const void *base, int64_t idx, int valid, float mul,
                                       uint16_t (&o)[16]) {
    if constexpr (BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(base) + idx;
        if (valid >= 16) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(p), v1 = *reinterpret_cast<const uint4 *>(p + 8);
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[2 * e] = static_cast<uint16_t>(w[e] & 0xFFFFu);
                o[2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
            }
            if (mul != 1.0f) {
#pragma unroll
                for (int e = 0; e < 16; ++e) o[e] = bf16_bits(bf16_bits_to_f32(o[e]) * mul);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                o[e] = e < valid ? bf16_bits(bf16_bits_to_f32(p[e]) * mul) : static_cast<uint16_t>(0);
        }
    } else {
        const float *p = static_cast<const float *>(base) + idx;
        if (valid >= 16) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float4 v = *reinterpret_cast<const float4 *>(p + 4 * e4);
                o[4 * e4] = bf16_bits(v.x * mul);
                o[4 * e4 + 1] = bf16_bits(v.y * mul);
                o[4 * e4 + 2] = bf16_bits(v.z * mul);
                o[4 * e4 + 3] = bf16_bits(v.w * mul);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) o[e] = e < valid ? bf16_bits(p[e] * mul) : static_cast<uint16_t>(0);
        }
    }
}

// C[r][s] = scale * sum_t A[r][t] B[s][t] on v_mfma_f32_32x32x16_bf16, both operands with
// the contraction index t contiguous: A [R][lda] bf16 (or fp32, rounded to bf16 as it is
// loaded), B [S][ldb] bf16, rows 16-byte aligned.  When the t range is split over blockIdx.z
// the partial tiles are added with fp32 atomics into a zeroed C.
// Tiles of 128 x 128 per workgroup (4 waves, 2 x 2, each 64 x 64 = 2 x 2 MFMA blocks), one
// workgroup per tile along blockIdx.x (grouped, XCD-aware order below), contraction steps
// of 64 double-buffered in LDS: the next step's global loads (16-byte
// vectors, 32 elements of A and of B per thread) are issued before the current step's 8
// MFMAs per wave and written to the other buffer after them; one barrier per step.  Rows
// are padded to 72 elements (144 bytes), so every MFMA operand is one 16-byte LDS read.
struct NtGemmArgs {
    const void *A;
    int32_t a_bf16;
    const uint16_t *B;
    int64_t R;
    int32_t S;
    int64_t T;              // contraction length
    int64_t lda, ldb;       // row strides in elements
    float scale;
    float *C;               // [R][S]
    int64_t t_per_split;    // multiple of BT (T when not split)
    int32_t atomic;         // 0: C = v; 1: C += v with fp32 atomics (split); 2: C += v
};

constexpr int BT = 64;           // contraction step (four 16-deep MFMA steps)
constexpr int LP = BT + 8;       // LDS pitch of a tile row in bf16 (144 bytes)

// 16 bf16 values of B's row from t on (valid of them; the rest zero)
__device__ __forceinline__ void load16_bf16(const uint16_t *p, int valid, uint16_t (&o)[16]) {
    if (valid >= 16) {
        const uint4 v0 = *reinterpret_cast<const uint4 *>(p), v1 = *reinterpret_cast<const uint4 *>(p + 8);
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[2 * e] = static_cast<uint16_t>(w[e] & 0xFFFFu);
            o[2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = e < valid ? p[e] : static_cast<uint16_t>(0);
    }
}

__device__ __forceinline__ void store16(uint16_t *d, const uint16_t (&v)[16]) {
    uint4 *q = reinterpret_cast<uint4 *>(d);
    q[0] = make_uint4(v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
                      v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16));
    q[1] = make_uint4(v[8] | (uint32_t(v[9]) << 16), v[10] | (uint32_t(v[11]) << 16),
                      v[12] | (uint32_t(v[13]) << 16), v[14] | (uint32_t(v[15]) << 16));
}

template <bool ABF16>
__global__ __launch_bounds__(GT, 2) void nt_gemm_kernel(NtGemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][BR * LP];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][BS * LP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int r32 = lane & 31, g = lane >> 5;
    // Tile order: workgroups are dispatched round-robin over the 8 XCDs, so tile ids are
    // remapped to give each XCD a contiguous run, walked in groups of GM row tiles (column
    // tile by column tile, the group's row tiles side by side): a column tile's B rows are
    // read once per group and a row tile's A rows once per column sweep of its group,
    // instead of B once per row tile.
    int rt, st;
    {
        const int n_rt = static_cast<int>((p.R + BR - 1) / BR), n_st = (p.S + BS - 1) / BS;
        const int nwg = gridDim.x, bid = blockIdx.x;
        const int qx = nwg >> 3, rx = nwg & 7, xcd = bid & 7, idx = bid >> 3;
        const int tile = (xcd < rx ? xcd * (qx + 1) : rx * (qx + 1) + (xcd - rx) * qx) + idx;
        constexpr int GM = 8;
        const int grp = tile / (GM * n_st), in_g = tile % (GM * n_st);
        const int gm = n_rt - grp * GM < GM ? n_rt - grp * GM : GM;
        rt = grp * GM + in_g % gm;
        st = in_g / gm;
    }
    const int64_t r0 = static_cast<int64_t>(rt) * BR;
    const int s0 = st * BS;
    const int64_t t_begin = static_cast<int64_t>(blockIdx.z) * p.t_per_split;
    const int64_t t_end = t_begin + p.t_per_split < p.T ? t_begin + p.t_per_split : p.T;
    // this thread's rows of the A and B tiles and its 32 t-values of a step, staged as four
    // 16-byte words (8 bf16 each) per operand
    const int lr = tid >> 1, lt = 32 * (tid & 1);
    const int64_t ar = r0 + lr;
    const int bs = s0 + lr;
    const bool rows_in = r0 + BR <= p.R && s0 + BS <= p.S;   // uniform over the workgroup
    uint4 ra0[4], rb0[4], ra1[4], rb1[4];   // two staging sets (even / odd steps)
    auto pack8 = [](const uint16_t (&v)[16], int h, uint4 &o) {
        o = make_uint4(v[8 * h] | (uint32_t(v[8 * h + 1]) << 16), v[8 * h + 2] | (uint32_t(v[8 * h + 3]) << 16),
                       v[8 * h + 4] | (uint32_t(v[8 * h + 5]) << 16), v[8 * h + 6] | (uint32_t(v[8 * h + 7]) << 16));
    };
    auto load_step = [&](int64_t t0, uint4 (&ra)[4], uint4 (&rb)[4]) {
        if (rows_in && t0 + BT <= t_end) {
            // every row and every t of the step in range: unconditional 16-byte loads
            const uint16_t *pb = p.B + static_cast<int64_t>(bs) * p.ldb + t0 + lt;
#pragma unroll
            for (int q = 0; q < 4; ++q) rb[q] = *reinterpret_cast<const uint4 *>(pb + 8 * q);
            if constexpr (ABF16) {
                const uint16_t *pa = static_cast<const uint16_t *>(p.A) + ar * p.lda + t0 + lt;
#pragma unroll
                for (int q = 0; q < 4; ++q) ra[q] = *reinterpret_cast<const uint4 *>(pa + 8 * q);
            } else {
                const float *pa = static_cast<const float *>(p.A) + ar * p.lda + t0 + lt;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 u = *reinterpret_cast<const float4 *>(pa + 8 * q);
                    const float4 v = *reinterpret_cast<const float4 *>(pa + 8 * q + 4);
                    ra[q] = make_uint4(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w), pack_bf16x2(v.x, v.y),
                                       pack_bf16x2(v.z, v.w));
                }
            }
            return;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t t = t0 + lt + 16 * h;
            const int64_t rem = t_end - t;
            const int valid = rem <= 0 ? 0 : (rem < 16 ? static_cast<int>(rem) : 16);
            uint16_t va[16], vb[16];
            load16<ABF16>(p.A, (ar < p.R && valid ? ar * p.lda + t : 0), ar < p.R ? valid : 0, 1.0f, va);
            load16_bf16(p.B + (bs < p.S && valid ? static_cast<int64_t>(bs) * p.ldb + t : 0),
                        bs < p.S ? valid : 0, vb);
            pack8(va, 0, ra[2 * h]);
            pack8(va, 1, ra[2 * h + 1]);
            pack8(vb, 0, rb[2 * h]);
            pack8(vb, 1, rb[2 * h + 1]);
        }
    };
    auto store_step = [&](int buf, const uint4 (&ra)[4], const uint4 (&rb)[4]) {
        uint4 *da = reinterpret_cast<uint4 *>(&sa[buf][lr * LP + lt]);
        uint4 *db = reinterpret_cast<uint4 *>(&sb[buf][lr * LP + lt]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            da[q] = ra[q];
            db[q] = rb[q];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Barrier without the memory fence of __syncthreads (which would also wait for the loads
    // issued two steps ahead): each wave waits for its own LDS stores, then s_barrier.
    auto lds_barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BT / 16; ++ks) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                av[i] = *reinterpret_cast<const bf16x8 *>(&sa[buf][(wr * 64 + i * 32 + r32) * LP + 16 * ks + 8 * g]);
                bv[i] = *reinterpret_cast<const bf16x8 *>(&sb[buf][(wc * 64 + i * 32 + r32) * LP + 16 * ks + 8 * g]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };
    // steps in pairs: LDS buffer 0 and staging set 0 for even steps, 1 for odd ones; a
    // step's loads are issued two steps before its MFMAs
    const int nsteps = t_end > t_begin ? static_cast<int>((t_end - t_begin + BT - 1) / BT) : 0;
    auto tstep = [&](int st) { return t_begin + static_cast<int64_t>(st) * BT; };
    if (nsteps > 0) {
        load_step(tstep(0), ra0, rb0);
        if (nsteps > 1) load_step(tstep(1), ra1, rb1);
        store_step(0, ra0, rb0);
    }
    lds_barrier();
    for (int st = 0; st < nsteps; st += 2) {
        if (st + 2 < nsteps) load_step(tstep(st + 2), ra0, rb0);
        compute(0);
        if (st + 1 < nsteps) store_step(1, ra1, rb1);
        lds_barrier();
        if (st + 1 < nsteps) {
            if (st + 3 < nsteps) load_step(tstep(st + 3), ra1, rb1);
            compute(1);
            if (st + 2 < nsteps) store_step(0, ra0, rb0);
            lds_barrier();
        }
    }
    // C block (i, j): lane holds rows 8*(e/4) + 4*g + e%4, column r32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = s0 + wc * 64 + j * 32 + r32;
            if (col >= p.S) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = r0 + wr * 64 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < p.R) {
                    float *o = p.C + row * p.S + col;
                    if (p.atomic == 1) atomicAdd(o, acc[i][j][e] * p.scale);
                    else if (p.atomic == 2) *o += acc[i][j][e] * p.scale;
                    else *o = acc[i][j][e] * p.scale;
                }
            }
        }
}

// W^T as bf16 values -1/0/1: out[k][n] for the packed [N][K/16] matrix; thread per (k, 8
// consecutive n), one 16-byte store (N % 8 == 0).
__global__ __launch_bounds__(256) void expand_wt_kernel(const uint32_t *packed, int32_t N, int32_t K,
                                                        uint16_t *out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int ng = N / 8;
    if (i >= static_cast<int64_t>(K) * ng) return;
    const int k = static_cast<int>(i / ng), n0 = static_cast<int>(i % ng) * 8;
    const int KW = K / 16, sh = 8 * (k % 4) + 2 * ((k % 16) / 4);
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int code = static_cast<int>((packed[static_cast<int64_t>(n0 + e) * KW + k / 16] >> sh) & 3u);
        v[e] = code == 2 ? 0x3F80u : (code == 0 ? 0xBF80u : 0u);
    }
    *reinterpret_cast<uint4 *>(out + static_cast<int64_t>(k) * N + n0) =
        make_uint4(v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
                   v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16));
}

// dst[c][m] = bf16(src[m][c] * (scale ? scale[m] : 1)) for m < M, 0 for M <= m < ldm (the
// padding of every destination row); src [M][lds] bf16, fp32 (SRC 0/1) or int8 codes (SRC 2).
// 64 x 64 tiles through LDS: rows read and columns written as contiguous runs.
template <int SRC>
__global__ __launch_bounds__(256) void transpose_kernel(const void *src, int64_t lds, const float *scale,
                                                        int64_t M, int32_t C, int64_t ldm, uint16_t *dst) {
    __shared__ float tile[64][65];
    const int tid = threadIdx.x;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 64;
    const int c0 = blockIdx.x * 64;
    {
        const int r = tid >> 2, cc = 16 * (tid & 3);
        const int64_t m = m0 + r;
        const float sc = m < M ? (scale ? scale[m] : 1.0f) : 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int c = c0 + cc + e;
            float v = 0.0f;
            if (m < M && c < C) {
                const int64_t idx = m * lds + c;
                if constexpr (SRC == 0) v = bf16_bits_to_f32(static_cast<const uint16_t *>(src)[idx]);
                else if constexpr (SRC == 1) v = static_cast<const float *>(src)[idx];
                else v = static_cast<float>(static_cast<const int8_t *>(src)[idx]);
            }
            tile[r][cc + e] = v * sc;
        }
    }
    __syncthreads();
    {
        const int c = c0 + (tid >> 2), mm = 16 * (tid & 3);
        if (c < C && m0 + mm < ldm) {
            uint16_t v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) v[e] = bf16_bits(tile[mm + e][tid >> 2]);
            store16(dst + static_cast<int64_t>(c) * ldm + m0 + mm, v);
        }
    }
}

// dx and dgamma from g: workgroup per RPW rows, thread per columns c = tid + 256 j.
//   r = (mean x^2 + eps)^(-1/2), dot = sum_c g*gamma*x, dx = r*gamma*g - x*r^3/K*dot
//   (+ a residual gradient res [M][K], bf16 for RES 1, fp32 for RES 2);
//   dgamma[c] += sum over the workgroup's rows of g*x*r (fp32 atomics into a zeroed array).
constexpr int RPW = 16;
template <bool XBF16, int RES>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const void *x, const float *gsrc, const float *gamma,
                                                       float eps, int64_t M, int32_t K, float *dx,
                                                       float *dgamma, const void *res) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * RPW;
    const int nj = (K + 255) / 256;
    float dg_acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) dg_acc[j] = 0.0f;
    for (int rr = 0; rr < RPW; ++rr) {
        const int64_t m = m0 + rr;
        if (m >= M) break;
        float ss = 0.0f, dot = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int c = tid + 256 * j;
            if (j < nj && c < K) {
                const float xv = load_act<XBF16>(x, m * K + c);
                const float gv = gsrc[m * K + c];
                ss = fmaf(xv, xv, ss);
                dot = fmaf(gv * (gamma ? gamma[c] : 1.0f), xv, dot);
            }
        }
        ss = wave_sum(ss);
        dot = wave_sum(dot);
        if (lane == 0) {
            red[0][wave] = ss;
            red[1][wave] = dot;
        }
        __syncthreads();
        ss = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        dot = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
        __syncthreads();
        const float r = 1.0f / sqrtf(ss / static_cast<float>(K) + eps);
        const float c3 = r * r * r / static_cast<float>(K) * dot;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int c = tid + 256 * j;
            if (j < nj && c < K) {
                const float xv = load_act<XBF16>(x, m * K + c);
                const float gv = gsrc[m * K + c];
                const float gm = gamma ? gamma[c] : 1.0f;
                float d = r * gm * gv - xv * c3;
                if constexpr (RES == 1) d += bf16_bits_to_f32(static_cast<const uint16_t *>(res)[m * K + c]);
                if constexpr (RES == 2) d += static_cast<const float *>(res)[m * K + c];
                if (dx) dx[m * K + c] = d;
                dg_acc[j] = fmaf(gv * xv, r, dg_acc[j]);
            }
        }
    }
    if (dgamma) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int c = tid + 256 * j;
            if (j < nj && c < K) atomicAdd(&dgamma[c], dg_acc[j]);
        }
    }
}

// out[c] += sum over rows [r0, r1) of src[r][c] (src [R][lds], bf16 or fp32), thread per
// column, rows split over blockIdx.y (fp32 atomics into a zeroed array).
template <bool BF16>
__global__ __launch_bounds__(256) void col_sum_kernel(const void *src, int64_t lds, int64_t R, int32_t C,
                                                      int32_t rows_per, float *out) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows_per;
    const int64_t r1 = r0 + rows_per < R ? r0 + rows_per : R;
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) s += load_act<BF16>(src, r * lds + c);
    atomicAdd(&out[c], s);
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

__device__ __forceinline__ float silu_grad(float z) {
    const float s = sigmoidf_(z);
    return s * (1.0f + z * (1.0f - s));
}

// The GLU's gated product from the gate | up pre-activations gu [M][2F] fp32 (gate at column
// f, up at F + f): m = SiLU(gate)*up in the activation dtype (the down projection's input).
template <bool MBF16>
__global__ __launch_bounds__(256) void glu_product_kernel(const float *gu, int64_t M, int32_t F, void *m) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= M * F) return;
    const int64_t row = i / F, f = i % F;
    const float g = gu[row * 2 * F + f], u = gu[row * 2 * F + F + f];
    store_act<MBF16>(m, i, siluf_(g) * u);
}

// Its backward: dgate = dm*up*silu'(gate), dup = dm*SiLU(gate), into dgu [M][2F] (gate | up).
__global__ __launch_bounds__(256) void glu_product_bwd_kernel(const float *gu, const float *dm, int64_t M,
                                                              int32_t F, float *dgu) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= M * F) return;
    const int64_t row = i / F, f = i % F;
    const float g = gu[row * 2 * F + f], u = gu[row * 2 * F + F + f], d = dm[i];
    dgu[row * 2 * F + f] = d * u * silu_grad(g);
    dgu[row * 2 * F + F + f] = d * siluf_(g);
}

// ------------------------------------------------------------------ MLGRU backward
constexpr int kBC = 16;           // tokens per chunk (the forward's chunk)


// Phase 1 (gate mode 0 only): workgroup per (chunk, b); thread per channel quads
// q = tid + 256 j (channels 4q..4q+3).  Reruns the recurrence over the chunk, keeps per token
// the thread's partial sums of h^2 and dn*h (dn = dout*w*silu(g)), reduces all 2x16 of them
// at once through LDS and stores per token rho = (mean h^2 + eps)^(-1/2) and
// k3 = rho^3/D * sum(dn*h).
template <bool IFGBF16, bool DOBF16, int JQ>
__global__ __launch_bounds__(256) void mlgru_bwd_stats_kernel(MlgruBwdArgs p) {
    __shared__ float red[2 * kBC][257];
    __shared__ float tot[2 * kBC];
    const int tid = threadIdx.x;
    const int c = blockIdx.x, b = blockIdx.y;
    const int D = p.D;
    const int64_t t0 = static_cast<int64_t>(c) * kBC;
    const int n = static_cast<int>(t0 + kBC < p.T ? kBC : p.T - t0);
    const int64_t crow = static_cast<int64_t>(b) * p.n_chunks + c;
    float h[JQ][4], fbv[JQ][4], lbv[JQ][4], gwv[JQ][4];
    float hs[kBC], sd[kBC];
#pragma unroll
    for (int k = 0; k < kBC; ++k) hs[k] = sd[k] = 0.0f;
#pragma unroll
    for (int j = 0; j < JQ; ++j) {
        const int d0 = 4 * (tid + 256 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[j][e] = fbv[j][e] = lbv[j][e] = 0.0f;
            gwv[j][e] = 1.0f;
        }
        if (d0 < D) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = d0 + e;
                h[j][e] = c == 0 ? (p.h0 ? p.h0[static_cast<int64_t>(b) * D + d] : 0.0f) : p.hin[crow * D + d];
                fbv[j][e] = p.f_bias ? p.f_bias[d] : 0.0f;
                lbv[j][e] = p.f_lower ? p.f_lower[d] : 0.0f;
                gwv[j][e] = p.gnorm_w ? p.gnorm_w[d] : 1.0f;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        if (k < n) {
            const int64_t row = static_cast<int64_t>(b) * p.T + t0 + k;
#pragma unroll
            for (int j = 0; j < JQ; ++j) {
                const int d0 = 4 * (tid + 256 * j);
                if (d0 < D) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int d = d0 + e;
                        const float iv = load_act<IFGBF16>(p.ifg, row * 3 * D + d);
                        const float fv = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d);
                        const float gv = load_act<IFGBF16>(p.ifg, row * 3 * D + 2 * D + d);
                        const float dov = load_act<DOBF16>(p.dout, row * D + d);
                        const float f = fmaf(1.0f - lbv[j][e], sigmoidf_(fv + fbv[j][e]), lbv[j][e]);
                        h[j][e] = f * h[j][e] + (1.0f - f) * siluf_(iv);
                        const float dn = dov * gwv[j][e] * siluf_(gv);
                        hs[k] = fmaf(h[j][e], h[j][e], hs[k]);
                        sd[k] = fmaf(dn, h[j][e], sd[k]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        red[k][tid] = hs[k];
        red[kBC + k][tid] = sd[k];
    }
    __syncthreads();
    {   // value v = tid / 8 summed by 8 lanes over 32 partials each, then across the 8 lanes
        const int v = tid >> 3, part = tid & 7;
        float acc = 0.0f;
#pragma unroll 8
        for (int i = 0; i < 32; ++i) acc += red[v][part * 32 + i];
        acc += __shfl_xor(acc, 4, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 1, 64);
        if (part == 0) tot[v] = acc;
    }
    __syncthreads();
    if (tid < n) {
        const float rho = 1.0f / sqrtf(tot[tid] / static_cast<float>(D) + p.eps);
        const int64_t row = static_cast<int64_t>(b) * p.T + t0 + tid;
        p.stats[2 * row] = rho;
        p.stats[2 * row + 1] = rho * rho * rho / static_cast<float>(D) * tot[kBC + tid];
    }
}

// Phase 3: thread per (b, d): G entering chunk c from the right (true G at chunk c+1's first
// token) into cg[c]; dh0 = f_0 * G_0.
__global__ __launch_bounds__(256) void mlgru_bwd_carry_kernel(MlgruBwdArgs p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int D = p.D;
    if (i >= p.B * D) return;
    const int64_t b = i / D, d = i % D;
    float Gn = 0.0f;   // true G at the first token of chunk c+1
    for (int c = p.n_chunks - 1; c >= 0; --c) {
        const int64_t crow = b * p.n_chunks + c;
        p.cg[crow * D + d] = Gn;
        const float fnext = c + 1 < p.n_chunks ? p.cf0[(crow + 1) * D + d] : 0.0f;
        Gn = p.cb[crow * D + d] + p.cp[crow * D + d] * fnext * Gn;
    }
    if (p.dh0) p.dh0[i] = p.cf0[b * p.n_chunks * D + d] * Gn;
}

// Phases 2 and 4: thread per (b, chunk, d).  Rerun the chunk forward (state before each
// token, f, c, i in registers), form the gradient at h from the output gate (gate mode 0
// with the per-token rho and k3 of phase 1), then walk the chunk backwards:
//   PASS 0: from zero (G_t = dh_t + f_{t+1} G_{t+1}) -> the chunk's first-token G, the
//           product of f after the first token, f at the first token; dg and the chunk's
//           partial sum of the g_norm weight gradient;
//   PASS 1: from the carried G (phase 3) -> di, df_pre and the chunk's partial sum of df.
template <bool IFGBF16, bool DOBF16, int PASS>
__global__ __launch_bounds__(256) void mlgru_bwd_chan_kernel(MlgruBwdArgs p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int D = p.D;
    if (i >= p.B * p.n_chunks * D) return;
    const int64_t crow = i / D, d = i % D;
    const int64_t b = crow / p.n_chunks, c = crow % p.n_chunks;
    const int64_t t0 = c * kBC;
    const int n = static_cast<int>(t0 + kBC < p.T ? kBC : p.T - t0);
    const float lb = p.f_lower ? p.f_lower[d] : 0.0f;
    const float fb = p.f_bias ? p.f_bias[d] : 0.0f;
    const float gw = p.gnorm_w ? p.gnorm_w[d] : 1.0f;
    float hprev[kBC], fz[kBC], iv[kBC], dh[kBC];
    float h = c == 0 ? (p.h0 ? p.h0[b * D + d] : 0.0f) : p.hin[crow * D + d];
    float gwp = 0.0f;
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        hprev[k] = fz[k] = iv[k] = dh[k] = 0.0f;
        if (k < n) {
            const int64_t row = b * p.T + t0 + k;
            iv[k] = load_act<IFGBF16>(p.ifg, row * 3 * D + d);
            fz[k] = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d) + fb;
            const float gv = load_act<IFGBF16>(p.ifg, row * 3 * D + 2 * D + d);
            const float dov = load_act<DOBF16>(p.dout, row * D + d);
            const float f = fmaf(1.0f - lb, sigmoidf_(fz[k]), lb);
            hprev[k] = h;
            h = f * h + (1.0f - f) * siluf_(iv[k]);
            float dho, dg;
            if (p.gate_mode == 0) {
                const float rho = p.stats[2 * row], k3 = p.stats[2 * row + 1];
                const float nrm = h * rho, sg = siluf_(gv);
                dho = rho * (dov * gw * sg) - h * k3;
                dg = dov * nrm * gw * silu_grad(gv);
                gwp = fmaf(dov * nrm, sg, gwp);
            } else {
                const float s = sigmoidf_(gv);
                dg = dov * h * s * (1.0f - s);
                dho = dov * s;
            }
            if (t0 + k == p.T - 1 && p.dh_last) dho += p.dh_last[b * D + d];
            dh[k] = dho;
            if constexpr (PASS == 0) p.d_ifg[row * 3 * D + 2 * D + d] = dg;
        }
    }
    if constexpr (PASS == 0) {
        float G = 0.0f, fnext = 0.0f, prod = 1.0f, f = 0.0f;
#pragma unroll
        for (int k = kBC - 1; k >= 0; --k) {
            if (k < n) {
                G = dh[k] + fnext * G;
                f = fmaf(1.0f - lb, sigmoidf_(fz[k]), lb);
                if (k > 0) prod *= f;
                fnext = f;
            }
        }
        p.cb[crow * D + d] = G;
        p.cp[crow * D + d] = prod;
        p.cf0[crow * D + d] = f;
        p.gw_part[crow * D + d] = gwp;
    } else {
        float fnext = c + 1 < p.n_chunks ? p.cf0[(crow + 1) * D + d] : 0.0f;
        float G = p.cg[crow * D + d];
        float dfb = 0.0f;
#pragma unroll
        for (int k = kBC - 1; k >= 0; --k) {
            if (k < n) {
                const int64_t row = b * p.T + t0 + k;
                const float sz = sigmoidf_(fz[k]);
                const float f = fmaf(1.0f - lb, sz, lb);
                const float cv = siluf_(iv[k]);
                G = dh[k] + fnext * G;
                p.d_ifg[row * 3 * D + d] = (1.0f - f) * G * silu_grad(iv[k]);
                const float dz = (hprev[k] - cv) * G * (1.0f - lb) * sz * (1.0f - sz);
                p.d_ifg[row * 3 * D + D + d] = dz;
                dfb += dz;
                fnext = f;
            }
        }
        p.fb_part[crow * D + d] = dfb;
    }
}

}  // namespace

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    if (n <= 0 || !p) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_col_sum(const void *src, int bf16, int64_t lds, int64_t R, int32_t C, float *out,
                          hipStream_t s) {
    if (R <= 0 || C <= 0) return hipSuccess;
    // about 64 rows per workgroup, at most 4096 row splits
    int64_t splits = (R + 63) / 64;
    if (splits > 4096) splits = 4096;
    const int32_t rows_per = static_cast<int32_t>((R + splits - 1) / splits);
    splits = (R + rows_per - 1) / rows_per;
    const dim3 grid(static_cast<unsigned>((C + 255) / 256), static_cast<unsigned>(splits));
    if (bf16) hipLaunchKernelGGL((col_sum_kernel<true>), grid, dim3(256), 0, s, src, lds, R, C, rows_per, out);
    else hipLaunchKernelGGL((col_sum_kernel<false>), grid, dim3(256), 0, s, src, lds, R, C, rows_per, out);
    return hipGetLastError();
}

hipError_t bwd_launch_g(const void *dy, int dy_bf16, int64_t ldy, const uint32_t *packed, int32_t N,
                        int32_t K, float scale, int64_t M, uint16_t *wt, float *g, int accumulate,
                        hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const int64_t n = static_cast<int64_t>(K) * (N / 8);
    hipLaunchKernelGGL(expand_wt_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s,
                       packed, N, K, wt);
    NtGemmArgs ga{};
    ga.A = dy;
    ga.a_bf16 = dy_bf16;
    ga.B = wt;
    ga.R = M;
    ga.S = K;
    ga.T = N;
    ga.lda = ldy;
    ga.ldb = N;
    ga.scale = scale;
    ga.C = g;
    ga.t_per_split = N;
    ga.atomic = accumulate ? 2 : 0;
    const dim3 grid(static_cast<unsigned>(((K + BS - 1) / BS) * ((M + BR - 1) / BR)), 1, 1);
    timing_begin(FAM_BWD_G, s);
    if (dy_bf16) hipLaunchKernelGGL((nt_gemm_kernel<true>), grid, dim3(GT), 0, s, ga);
    else hipLaunchKernelGGL((nt_gemm_kernel<false>), grid, dim3(GT), 0, s, ga);
    timing_end(FAM_BWD_G, s);
    return hipGetLastError();
}

hipError_t bwd_launch_rows(const void *x, int x_bf16, const float *g, const float *gamma, float eps,
                           int64_t M, int32_t K, float *dx, float *dgamma, const void *res, int res_kind,
                           hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipError_t e;
    if (dgamma && (e = launch_fill_zero(dgamma, K, s)) != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>((M + RPW - 1) / RPW));
#define MMF_ROWS(XB, RK) hipLaunchKernelGGL((bwd_rows_kernel<XB, RK>), grid, dim3(256), 0, s, x, g, gamma, eps, M, K, dx, dgamma, res)
    if (x_bf16) {
        if (res_kind == 1) MMF_ROWS(true, 1);
        else if (res_kind == 2) MMF_ROWS(true, 2);
        else MMF_ROWS(true, 0);
    } else {
        if (res_kind == 1) MMF_ROWS(false, 1);
        else if (res_kind == 2) MMF_ROWS(false, 2);
        else MMF_ROWS(false, 0);
    }
#undef MMF_ROWS
    return hipGetLastError();
}

hipError_t bwd_launch_qT(const int8_t *q, int64_t M, int32_t K, int64_t ldm, uint16_t *qT, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const dim3 gt(static_cast<unsigned>((K + 63) / 64), static_cast<unsigned>(ldm / 64));
    hipLaunchKernelGGL((transpose_kernel<2>), gt, dim3(256), 0, s, q, static_cast<int64_t>(K), nullptr, M, K, ldm, qT);
    return hipGetLastError();
}

hipError_t bwd_launch_dw(const void *dy, int dy_bf16, int64_t ldy, const float *a, int64_t M, int32_t N,
                         int32_t K, int64_t ldm, const uint16_t *qT, uint16_t *dyaT, float *dw, hipStream_t s) {
    if (M <= 0) return launch_fill_zero(dw, static_cast<int64_t>(N) * K, s);
    const dim3 gt(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>(ldm / 64));
    if (dy_bf16) hipLaunchKernelGGL((transpose_kernel<0>), gt, dim3(256), 0, s, dy, ldy, a, M, N, ldm, dyaT);
    else hipLaunchKernelGGL((transpose_kernel<1>), gt, dim3(256), 0, s, dy, ldy, a, M, N, ldm, dyaT);
    hipError_t e;
    if ((e = launch_fill_zero(dw, static_cast<int64_t>(N) * K, s)) != hipSuccess) return e;
    NtGemmArgs ga{};
    ga.A = dyaT;
    ga.a_bf16 = 1;
    ga.B = qT;
    ga.R = N;
    ga.S = K;
    ga.T = ldm;
    ga.lda = ldm;
    ga.ldb = ldm;
    ga.scale = 1.0f;
    ga.C = dw;
    ga.atomic = 1;
    const int64_t tiles = static_cast<int64_t>((K + BS - 1) / BS) * ((N + BR - 1) / BR);
    // split the tokens so that about 1024 workgroups run, each over >= 8 steps
    int64_t splits = (1024 + tiles - 1) / tiles;
    const int64_t max_splits = (ldm + 8 * BT - 1) / (8 * BT);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    int64_t per = (ldm + splits - 1) / splits;
    per = (per + BT - 1) / BT * BT;
    splits = (ldm + per - 1) / per;
    ga.t_per_split = per;
    const dim3 grid(static_cast<unsigned>(tiles), 1, static_cast<unsigned>(splits));
    timing_begin(FAM_BWD_DW, s);
    hipLaunchKernelGGL((nt_gemm_kernel<true>), grid, dim3(GT), 0, s, ga);
    timing_end(FAM_BWD_DW, s);
    return hipGetLastError();
}

hipError_t bwd_launch_db(const void *dy, int dy_bf16, int64_t ldy, int64_t M, int32_t N, float *db, hipStream_t s) {
    hipError_t e;
    if ((e = launch_fill_zero(db, N, s)) != hipSuccess) return e;
    return launch_col_sum(dy, dy_bf16, ldy, M, N, db, s);
}

hipError_t launch_glu_product(const float *gu, int64_t M, int32_t F, void *m, int m_bf16, hipStream_t s) {
    const int64_t n = M * F;
    if (n <= 0) return hipSuccess;
    if (m_bf16) hipLaunchKernelGGL((glu_product_kernel<true>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, gu, M, F, m);
    else hipLaunchKernelGGL((glu_product_kernel<false>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, gu, M, F, m);
    return hipGetLastError();
}

hipError_t launch_glu_product_bwd(const float *gu, const float *dm, int64_t M, int32_t F, float *dgu, hipStream_t s) {
    const int64_t n = M * F;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(glu_product_bwd_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, gu, dm, M, F, dgu);
    return hipGetLastError();
}

hipError_t launch_bitlinear_bwd(const BitlinearBwdArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    hipError_t e;
    if ((e = bwd_launch_g(a.dy, a.dy_bf16, a.N, a.packed, a.N, a.K, a.scale, a.M, a.wt, a.g, 0, s)) != hipSuccess) return e;
    if ((e = bwd_launch_rows(a.x, a.x_bf16, a.g, a.gamma, a.eps, a.M, a.K, a.dx, a.dgamma, nullptr, 0, s)) != hipSuccess) return e;
    if (a.dw) {
        if ((e = bwd_launch_qT(a.q, a.M, a.K, a.ldm, a.qT, s)) != hipSuccess) return e;
        if ((e = bwd_launch_dw(a.dy, a.dy_bf16, a.N, a.a, a.M, a.N, a.K, a.ldm, a.qT, a.dyaT, a.dw, s)) != hipSuccess) return e;
    }
    if (a.db && (e = bwd_launch_db(a.dy, a.dy_bf16, a.N, a.M, a.N, a.db, s)) != hipSuccess) return e;
    return hipGetLastError();
}

hipError_t launch_mlgru_bwd(const MlgruBwdArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    hipError_t e;
    timing_begin(FAM_BWD_SCAN, s);
    if (a.gate_mode == 0) {
        const dim3 g1(static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(a.B));
        const int jq = (a.D + 1023) / 1024;
#define MMF_STATS(JQ)                                                                                    \
        if (a.ifg_bf16 && a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_stats_kernel<true, true, JQ>), g1, dim3(256), 0, s, a); \
        else if (a.ifg_bf16) hipLaunchKernelGGL((mlgru_bwd_stats_kernel<true, false, JQ>), g1, dim3(256), 0, s, a);         \
        else if (a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_stats_kernel<false, true, JQ>), g1, dim3(256), 0, s, a);        \
        else hipLaunchKernelGGL((mlgru_bwd_stats_kernel<false, false, JQ>), g1, dim3(256), 0, s, a);
        if (jq <= 1) { MMF_STATS(1) }
        else if (jq == 2) { MMF_STATS(2) }
        else if (jq == 3) { MMF_STATS(3) }
        else { MMF_STATS(4) }
#undef MMF_STATS
    }
    const int64_t n3 = a.B * a.n_chunks * a.D;
    const dim3 g3(static_cast<unsigned>((n3 + 255) / 256));
#define MMF_CHAN(PASS)                                                                                   \
    if (a.ifg_bf16 && a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_chan_kernel<true, true, PASS>), g3, dim3(256), 0, s, a); \
    else if (a.ifg_bf16) hipLaunchKernelGGL((mlgru_bwd_chan_kernel<true, false, PASS>), g3, dim3(256), 0, s, a);         \
    else if (a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_chan_kernel<false, true, PASS>), g3, dim3(256), 0, s, a);        \
    else hipLaunchKernelGGL((mlgru_bwd_chan_kernel<false, false, PASS>), g3, dim3(256), 0, s, a);
    MMF_CHAN(0)
    const int64_t nc = a.B * a.D;
    hipLaunchKernelGGL(mlgru_bwd_carry_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, s, a);
    MMF_CHAN(1)
#undef MMF_CHAN
    const int64_t R = a.B * a.n_chunks;
    if (a.dgnorm_w) {
        if ((e = launch_fill_zero(a.dgnorm_w, a.D, s)) != hipSuccess) return e;
        if ((e = launch_col_sum(a.gw_part, 0, a.D, R, a.D, a.dgnorm_w, s)) != hipSuccess) return e;
    }
    if (a.df_bias) {
        if ((e = launch_fill_zero(a.df_bias, a.D, s)) != hipSuccess) return e;
        if ((e = launch_col_sum(a.fb_part, 0, a.D, R, a.D, a.df_bias, s)) != hipSuccess) return e;
    }
    timing_end(FAM_BWD_SCAN, s);
    return hipGetLastError();
}

}  // namespace mmf
