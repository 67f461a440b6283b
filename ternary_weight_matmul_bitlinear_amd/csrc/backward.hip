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
//   g  = s_w * dy T          [M][K]   bf16 matrix cores, T's codes unpacked exactly to bf16
//   dW = (dy*a)^T q_x        [N][K]   bf16 matrix cores, contraction over tokens split
//                                     over workgroups (fp32 atomics)
//   dx = r*gamma*g - x*r^3/K * sum_K(g*gamma*x),  dgamma = sum_M g*x*r,  db = sum_M dy
// q_x and a are recomputed by the forward quantizer; dy enters the matrix cores rounded to
// bf16 (exact when dy is bf16), (dy*a) rounded to bf16 for dW; accumulation is fp32.
//
// MLGRU + output gate, given dout [B][T][D] (and dh_T): the forward's chunk carries give
// the state entering every 16-token chunk, then
//   phase 1 (workgroup per chunk, whole rows of D): rerun the recurrence, the output gate's
//     backward per token (two row reductions: sum h^2, sum dn*h), dh_out and dg; then the
//     chunk's reverse scan of G_t = dh_out_t + f_{t+1} G_{t+1} from zero, keeping its value
//     at the first token, the product of f over the chunk after the first token, and f at
//     the first token;
//   phase 2 (thread per channel): carry G backwards across chunks; dh0 = f_0 G_0;
//   phase 3 (thread per chunk and channel): rerun the chunk forward, then walk it backwards
//     with the carried G: di = (1-f) G silu'(i), df_pre = (h_{t-1} - c) G (1-lb) sigma'(z).
// Per-chunk partial sums of dgnorm_w and df_bias are reduced by a column-sum kernel.
#include "mmf_internal.h"

namespace mmf {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GT = 256;          // threads of a GEMM workgroup (2 x 2 waves)
constexpr int BR = 128, BS = 128;  // output tile rows x columns
constexpr int BT = 32;           // contraction step (two 16-deep MFMA steps)
constexpr int LP = 40;           // LDS pitch of a tile row in bf16 (32 + 8: 80 bytes)

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

// C[r][s] = scale * sum_t A(r, t) B(t, s) on v_mfma_f32_32x32x16_bf16.
//   MODE 0: g = s_w * dy T: r = token m, s = input column k, t = output row n;
//           A(m, n) = dy[m][n], B(n, k) = code of T[n][k] - 1 (exact in bf16).
//   MODE 1: dW = (dy*a)^T q: r = output row n, s = input column k, t = token m;
//           A(n, m) = bf16(dy[m][n] * a[m]), B(m, k) = q[m][k] (exact in bf16); the token
//           range is split over blockIdx.z and the partial tiles are added with fp32 atomics
//           into a zeroed output.
// Tiles of 128 x 128 per workgroup (4 waves, 2 x 2, each 64 x 64 = 2 x 2 MFMA blocks),
// contraction steps of 32 double-buffered in LDS: the next step's global loads are issued
// before the current step's MFMAs and written to the other buffer after them.  Operands are
// stored [row][t] with t contiguous (A) and [column][t] (B), so every MFMA operand is one
// 16-byte LDS read; transposed loads write 2-byte values along a column of the buffer.
struct BwdGemmArgs {
    const void *dy;
    int32_t dy_bf16;
    const uint32_t *packed;  // MODE 0: [N][K/16]
    const int8_t *q;         // MODE 1: [M][K]
    const float *a;          // MODE 1: [M]
    int64_t M;
    int32_t N, K;
    float scale;
    float *out;              // MODE 0: [M][K]; MODE 1: [N][K]
    int32_t t_per_split;     // MODE 1: tokens per blockIdx.z (multiple of BT)
};

template <int MODE, bool DYBF16>
__global__ __launch_bounds__(GT) void bwd_gemm_kernel(BwdGemmArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][BR * LP];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][BS * LP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int r32 = lane & 31, g = lane >> 5;
    const int64_t R = MODE == 0 ? p.M : p.N;
    const int S = p.K;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * BR;
    const int s0 = blockIdx.x * BS;
    int64_t t_begin = 0, t_end = MODE == 0 ? p.N : p.M;
    if constexpr (MODE == 1) {
        t_begin = static_cast<int64_t>(blockIdx.z) * p.t_per_split;
        t_end = t_begin + p.t_per_split < p.M ? t_begin + p.t_per_split : p.M;
    }
    const int KW = p.K / 16;

    // staged operands of one contraction step (bf16 bits)
    uint16_t va[16];
    uint32_t wb = 0;       // MODE 0: one packed word
    uint16_t vb[16];       // MODE 1: 16 codes of q
    auto load_step = [&](int64_t t0) {
        if constexpr (MODE == 0) {
            // A: row m = r0 + tid/2, n = t0 + 16*(tid&1) .. +15
            const int64_t m = r0 + (tid >> 1);
            const int64_t n = t0 + 16 * (tid & 1);
            const int valid = m < p.M ? static_cast<int>(t_end - n < 16 ? (t_end - n > 0 ? t_end - n : 0) : 16) : 0;
            load16<DYBF16>(p.dy, (m < p.M ? m : 0) * p.N + (valid > 0 ? n : 0), valid, 1.0f, va);
            // B: row n = t0 + tid/8, word (s0/16 + tid%8): 16 codes along k
            const int64_t nb = t0 + (tid >> 3);
            const int kw = s0 / 16 + (tid & 7);
            wb = nb < t_end && kw < KW ? p.packed[nb * KW + kw] : 0x55555555u;
        } else {
            // A: token m = t0 + tid/8, outputs n = r0 + 16*(tid%8) .. +15, times a[m]
            const int64_t m = t0 + (tid >> 3);
            const int64_t n = r0 + 16 * (tid & 7);
            const bool mv = m < t_end;
            const int valid = mv ? static_cast<int>(p.N - n < 16 ? (p.N - n > 0 ? p.N - n : 0) : 16) : 0;
            const float am = mv ? p.a[m] : 0.0f;
            load16<DYBF16>(p.dy, (mv ? m : 0) * p.N + (valid > 0 ? n : 0), valid, am, va);
            // B: token m, columns k = s0 + 16*(tid%8) .. +15 of q
            const int k = s0 + 16 * (tid & 7);
            if (mv && k + 16 <= p.K) {
                const uint4 v = *reinterpret_cast<const uint4 *>(p.q + m * p.K + k);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    vb[e] = bf16_bits(static_cast<float>(static_cast<int8_t>((w[e / 4] >> (8 * (e % 4))) & 0xFFu)));
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) vb[e] = 0;
            }
        }
    };
    auto store_step = [&](int buf) {
        if constexpr (MODE == 0) {
            // A row-major: row tid/2, t = 16*(tid&1)
            uint4 *d = reinterpret_cast<uint4 *>(&sa[buf][(tid >> 1) * LP + 16 * (tid & 1)]);
            d[0] = make_uint4(va[0] | (uint32_t(va[1]) << 16), va[2] | (uint32_t(va[3]) << 16),
                              va[4] | (uint32_t(va[5]) << 16), va[6] | (uint32_t(va[7]) << 16));
            d[1] = make_uint4(va[8] | (uint32_t(va[9]) << 16), va[10] | (uint32_t(va[11]) << 16),
                              va[12] | (uint32_t(va[13]) << 16), va[14] | (uint32_t(va[15]) << 16));
            // B transposed: column k = 16*(tid%8) + e, t = tid/8
            const int t = tid >> 3, kc = 16 * (tid & 7);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int code = static_cast<int>((wb >> (8 * (e % 4) + 2 * (e / 4))) & 3u);
                sb[buf][(kc + e) * LP + t] = bf16_bits(static_cast<float>(code - 1));
            }
        } else {
            // A transposed: row n = 16*(tid%8) + e, t = tid/8
            const int t = tid >> 3, nc = 16 * (tid & 7);
#pragma unroll
            for (int e = 0; e < 16; ++e) sa[buf][(nc + e) * LP + t] = va[e];
            // B transposed: column k = 16*(tid%8) + e, t = tid/8
#pragma unroll
            for (int e = 0; e < 16; ++e) sb[buf][(nc + e) * LP + t] = vb[e];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nsteps = t_end > t_begin ? static_cast<int>((t_end - t_begin + BT - 1) / BT) : 0;
    if (nsteps > 0) {
        load_step(t_begin);
        store_step(0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps) load_step(t_begin + static_cast<int64_t>(st + 1) * BT);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wr * 64 + i * 32 + r32;
                av[i] = *reinterpret_cast<const bf16x8 *>(&sa[buf][row * LP + 16 * ks + 8 * g]);
                const int col = wc * 64 + i * 32 + r32;
                bv[i] = *reinterpret_cast<const bf16x8 *>(&sb[buf][col * LP + 16 * ks + 8 * g]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (st + 1 < nsteps) store_step(buf ^ 1);
        __syncthreads();
    }
    // C block (i, j): lane holds rows 8*(e/4) + 4*g + e%4, column r32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = s0 + wc * 64 + j * 32 + r32;
            if (col >= S) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = r0 + wr * 64 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < R) {
                    float *o = p.out + row * S + col;
                    if constexpr (MODE == 0) *o = acc[i][j][e] * p.scale;
                    else atomicAdd(o, acc[i][j][e] * p.scale);
                }
            }
        }
}

// dx and dgamma from g: workgroup per RPW rows, thread per columns c = tid + 256 j.
//   r = (mean x^2 + eps)^(-1/2), dot = sum_c g*gamma*x, dx = r*gamma*g - x*r^3/K*dot;
//   dgamma[c] += sum over the workgroup's rows of g*x*r (fp32 atomics into a zeroed array).
constexpr int RPW = 16;
template <bool XBF16>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const void *x, const float *gsrc, const float *gamma,
                                                       float eps, int64_t M, int32_t K, float *dx,
                                                       float *dgamma) {
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
                if (dx) dx[m * K + c] = r * gm * gv - xv * c3;
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

// out[c] += sum over rows [r0, r1) of src[r][c] (bf16 or fp32), thread per column, rows split
// over blockIdx.y (fp32 atomics into a zeroed array).
template <bool BF16>
__global__ __launch_bounds__(256) void col_sum_kernel(const void *src, int64_t R, int32_t C, int32_t rows_per,
                                                      float *out) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * rows_per;
    const int64_t r1 = r0 + rows_per < R ? r0 + rows_per : R;
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) s += load_act<BF16>(src, r * C + c);
    atomicAdd(&out[c], s);
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ------------------------------------------------------------------ MLGRU backward
constexpr int kBC = 16;           // tokens per chunk (the forward's chunk)
constexpr int kJD = 16;           // channels per thread in phase 1 (D <= 4096)

__device__ __forceinline__ float silu_grad(float z) {
    const float s = sigmoidf_(z);
    return s * (1.0f + z * (1.0f - s));
}

// Phase 1: workgroup per (chunk, b), thread per channels d = tid + 256 j.
template <bool IFGBF16, bool DOBF16>
__global__ __launch_bounds__(256) void mlgru_bwd_rows_kernel(MlgruBwdArgs p) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = blockIdx.x, b = blockIdx.y;
    const int D = p.D;
    const int64_t t0 = static_cast<int64_t>(c) * kBC;
    const int64_t t1 = t0 + kBC < p.T ? t0 + kBC : p.T;
    const int nj = D / 256 + (D % 256 ? 1 : 0);
    float h[kJD], gw_part[kJD];
    const int64_t crow = static_cast<int64_t>(b) * p.n_chunks + c;
#pragma unroll
    for (int j = 0; j < kJD; ++j) {
        const int d = tid + 256 * j;
        gw_part[j] = 0.0f;
        h[j] = 0.0f;
        if (j < nj && d < D)
            h[j] = c == 0 ? (p.h0 ? p.h0[static_cast<int64_t>(b) * D + d] : 0.0f) : p.hin[crow * D + d];
    }
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t row = static_cast<int64_t>(b) * p.T + t;
        float hs = 0.0f, sd = 0.0f;
        float dn[kJD];
#pragma unroll
        for (int j = 0; j < kJD; ++j) {
            const int d = tid + 256 * j;
            dn[j] = 0.0f;
            if (j < nj && d < D) {
                const float iv = load_act<IFGBF16>(p.ifg, row * 3 * D + d);
                const float fv = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d);
                const float lb = p.f_lower ? p.f_lower[d] : 0.0f;
                const float f = fmaf(1.0f - lb, sigmoidf_(fv + (p.f_bias ? p.f_bias[d] : 0.0f)), lb);
                h[j] = f * h[j] + (1.0f - f) * siluf_(iv);
                if (p.gate_mode == 0) {
                    const float gv = load_act<IFGBF16>(p.ifg, row * 3 * D + 2 * D + d);
                    const float dov = load_act<DOBF16>(p.dout, row * D + d);
                    dn[j] = dov * (p.gnorm_w ? p.gnorm_w[d] : 1.0f) * siluf_(gv);
                    hs = fmaf(h[j], h[j], hs);
                    sd = fmaf(dn[j], h[j], sd);
                }
            }
        }
        float rho = 0.0f, k3 = 0.0f;
        if (p.gate_mode == 0) {
            hs = wave_sum(hs);
            sd = wave_sum(sd);
            if (lane == 0) {
                red[0][wave] = hs;
                red[1][wave] = sd;
            }
            __syncthreads();
            hs = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
            sd = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
            __syncthreads();
            rho = 1.0f / sqrtf(hs / static_cast<float>(D) + p.eps);
            k3 = rho * rho * rho / static_cast<float>(D) * sd;
        }
#pragma unroll
        for (int j = 0; j < kJD; ++j) {
            const int d = tid + 256 * j;
            if (j < nj && d < D) {
                const float gv = load_act<IFGBF16>(p.ifg, row * 3 * D + 2 * D + d);
                const float dov = load_act<DOBF16>(p.dout, row * D + d);
                float dho, dg;
                if (p.gate_mode == 0) {
                    const float w = p.gnorm_w ? p.gnorm_w[d] : 1.0f;
                    const float nrm = h[j] * rho;
                    dg = dov * nrm * w * silu_grad(gv);
                    gw_part[j] = fmaf(dov * nrm, siluf_(gv), gw_part[j]);
                    dho = rho * dn[j] - h[j] * k3;
                } else {
                    const float s = sigmoidf_(gv);
                    dg = dov * h[j] * s * (1.0f - s);
                    dho = dov * s;
                }
                if (t == p.T - 1 && p.dh_last) dho += p.dh_last[static_cast<int64_t>(b) * D + d];
                p.d_ifg[row * 3 * D + 2 * D + d] = dg;
                p.dho[row * D + d] = dho;
            }
        }
    }
    // the chunk's reverse scan from zero (this thread re-reads its own dh_out values)
#pragma unroll
    for (int j = 0; j < kJD; ++j) {
        const int d = tid + 256 * j;
        if (j < nj && d < D) {
            const float lb = p.f_lower ? p.f_lower[d] : 0.0f;
            const float fb = p.f_bias ? p.f_bias[d] : 0.0f;
            float G = 0.0f, fnext = 0.0f, prod = 1.0f, f = 0.0f;
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t row = static_cast<int64_t>(b) * p.T + t;
                G = p.dho[row * D + d] + fnext * G;
                const float fv = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d);
                f = fmaf(1.0f - lb, sigmoidf_(fv + fb), lb);
                if (t > t0) prod *= f;
                fnext = f;
            }
            p.cb[crow * D + d] = G;       // local G at the chunk's first token
            p.cp[crow * D + d] = prod;    // prod of f over the chunk after its first token
            p.cf0[crow * D + d] = f;      // f at the chunk's first token
            p.gw_part[crow * D + d] = gw_part[j];
        }
    }
}

// Phase 2: thread per (b, d): G entering chunk c from the right (true G at chunk c+1's first
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

// Phase 3: thread per (b, chunk, d): rerun the chunk forward (state, f, c per token in
// registers), then walk it backwards with the carried G.
template <bool IFGBF16>
__global__ __launch_bounds__(256) void mlgru_bwd_out_kernel(MlgruBwdArgs p) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int D = p.D;
    if (i >= p.B * p.n_chunks * D) return;
    const int64_t crow = i / D, d = i % D;
    const int64_t b = crow / p.n_chunks, c = crow % p.n_chunks;
    const int64_t t0 = c * kBC;
    const int n = static_cast<int>(t0 + kBC < p.T ? kBC : p.T - t0);
    const float lb = p.f_lower ? p.f_lower[d] : 0.0f;
    const float fb = p.f_bias ? p.f_bias[d] : 0.0f;
    float hprev[kBC], fz[kBC], cv[kBC], iv[kBC];
    float h = c == 0 ? (p.h0 ? p.h0[b * D + d] : 0.0f) : p.hin[crow * D + d];
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        hprev[k] = fz[k] = cv[k] = iv[k] = 0.0f;
        if (k < n) {
            const int64_t row = b * p.T + t0 + k;
            iv[k] = load_act<IFGBF16>(p.ifg, row * 3 * D + d);
            fz[k] = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d) + fb;
        }
    }
    float fnext = c + 1 < p.n_chunks ? p.cf0[(crow + 1) * D + d] : 0.0f;
    float G = p.cg[crow * D + d];
    float dfb = 0.0f;
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        if (k < n) {
            const float f = fmaf(1.0f - lb, sigmoidf_(fz[k]), lb);
            hprev[k] = h;
            cv[k] = siluf_(iv[k]);
            h = f * h + (1.0f - f) * cv[k];
        }
    }
#pragma unroll
    for (int k = kBC - 1; k >= 0; --k) {
        if (k < n) {
            const int64_t row = b * p.T + t0 + k;
            const float sz = sigmoidf_(fz[k]);
            const float f = fmaf(1.0f - lb, sz, lb);
            G = p.dho[row * D + d] + fnext * G;
            p.d_ifg[row * 3 * D + d] = (1.0f - f) * G * silu_grad(iv[k]);
            const float dz = (hprev[k] - cv[k]) * G * (1.0f - lb) * sz * (1.0f - sz);
            p.d_ifg[row * 3 * D + D + d] = dz;
            dfb += dz;
            fnext = f;
        }
    }
    p.fb_part[crow * D + d] = dfb;
}

}  // namespace

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    if (n <= 0 || !p) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_col_sum(const void *src, int bf16, int64_t R, int32_t C, float *out, hipStream_t s) {
    if (R <= 0 || C <= 0) return hipSuccess;
    // about 64 rows per workgroup, at most 4096 row splits
    int64_t splits = (R + 63) / 64;
    if (splits > 4096) splits = 4096;
    const int32_t rows_per = static_cast<int32_t>((R + splits - 1) / splits);
    splits = (R + rows_per - 1) / rows_per;
    const dim3 grid(static_cast<unsigned>((C + 255) / 256), static_cast<unsigned>(splits));
    if (bf16) hipLaunchKernelGGL((col_sum_kernel<true>), grid, dim3(256), 0, s, src, R, C, rows_per, out);
    else hipLaunchKernelGGL((col_sum_kernel<false>), grid, dim3(256), 0, s, src, R, C, rows_per, out);
    return hipGetLastError();
}

hipError_t launch_bitlinear_bwd(const BitlinearBwdArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    hipError_t e;
    // g = s_w * dy T
    timing_begin(FAM_BWD_G, s);
    {
        BwdGemmArgs g{};
        g.dy = a.dy;
        g.dy_bf16 = a.dy_bf16;
        g.packed = a.packed;
        g.M = a.M;
        g.N = a.N;
        g.K = a.K;
        g.scale = a.scale;
        g.out = a.g;
        const dim3 grid(static_cast<unsigned>((a.K + BS - 1) / BS), static_cast<unsigned>((a.M + BR - 1) / BR));
        if (a.dy_bf16) hipLaunchKernelGGL((bwd_gemm_kernel<0, true>), grid, dim3(GT), 0, s, g);
        else hipLaunchKernelGGL((bwd_gemm_kernel<0, false>), grid, dim3(GT), 0, s, g);
    }
    timing_end(FAM_BWD_G, s);
    if (a.dgamma && (e = launch_fill_zero(a.dgamma, a.K, s)) != hipSuccess) return e;
    {
        const dim3 grid(static_cast<unsigned>((a.M + RPW - 1) / RPW));
        if (a.x_bf16) hipLaunchKernelGGL((bwd_rows_kernel<true>), grid, dim3(256), 0, s, a.x, a.g, a.gamma, a.eps, a.M, a.K, a.dx, a.dgamma);
        else hipLaunchKernelGGL((bwd_rows_kernel<false>), grid, dim3(256), 0, s, a.x, a.g, a.gamma, a.eps, a.M, a.K, a.dx, a.dgamma);
    }
    if (a.dw) {
        if ((e = launch_fill_zero(a.dw, static_cast<int64_t>(a.N) * a.K, s)) != hipSuccess) return e;
        BwdGemmArgs g{};
        g.dy = a.dy;
        g.dy_bf16 = a.dy_bf16;
        g.q = a.q;
        g.a = a.a;
        g.M = a.M;
        g.N = a.N;
        g.K = a.K;
        g.scale = 1.0f;
        g.out = a.dw;
        const int64_t tiles = static_cast<int64_t>((a.K + BS - 1) / BS) * ((a.N + BR - 1) / BR);
        // split the tokens so that about 1024 workgroups run, each over >= 8 steps
        int64_t splits = (1024 + tiles - 1) / tiles;
        const int64_t max_splits = (a.M + 8 * BT - 1) / (8 * BT);
        if (splits > max_splits) splits = max_splits;
        if (splits < 1) splits = 1;
        int64_t per = (a.M + splits - 1) / splits;
        per = (per + BT - 1) / BT * BT;
        splits = (a.M + per - 1) / per;
        g.t_per_split = static_cast<int32_t>(per);
        const dim3 grid(static_cast<unsigned>((a.K + BS - 1) / BS), static_cast<unsigned>((a.N + BR - 1) / BR),
                        static_cast<unsigned>(splits));
        timing_begin(FAM_BWD_DW, s);
        if (a.dy_bf16) hipLaunchKernelGGL((bwd_gemm_kernel<1, true>), grid, dim3(GT), 0, s, g);
        else hipLaunchKernelGGL((bwd_gemm_kernel<1, false>), grid, dim3(GT), 0, s, g);
        timing_end(FAM_BWD_DW, s);
    }
    if (a.db) {
        if ((e = launch_fill_zero(a.db, a.N, s)) != hipSuccess) return e;
        if ((e = launch_col_sum(a.dy, a.dy_bf16, a.M, a.N, a.db, s)) != hipSuccess) return e;
    }
    return hipGetLastError();
}

hipError_t launch_mlgru_bwd(const MlgruBwdArgs &a, hipStream_t s) {
    if (a.B <= 0) return hipSuccess;
    hipError_t e;
    timing_begin(FAM_BWD_SCAN, s);
    const dim3 g1(static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(a.B));
    if (a.ifg_bf16) {
        if (a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_rows_kernel<true, true>), g1, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((mlgru_bwd_rows_kernel<true, false>), g1, dim3(256), 0, s, a);
    } else {
        if (a.dout_bf16) hipLaunchKernelGGL((mlgru_bwd_rows_kernel<false, true>), g1, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((mlgru_bwd_rows_kernel<false, false>), g1, dim3(256), 0, s, a);
    }
    const int64_t nc = a.B * a.D;
    hipLaunchKernelGGL(mlgru_bwd_carry_kernel, dim3(static_cast<unsigned>((nc + 255) / 256)), dim3(256), 0, s, a);
    const int64_t n3 = a.B * a.n_chunks * a.D;
    const dim3 g3(static_cast<unsigned>((n3 + 255) / 256));
    if (a.ifg_bf16) hipLaunchKernelGGL((mlgru_bwd_out_kernel<true>), g3, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((mlgru_bwd_out_kernel<false>), g3, dim3(256), 0, s, a);
    const int64_t R = a.B * a.n_chunks;
    if (a.dgnorm_w) {
        if ((e = launch_fill_zero(a.dgnorm_w, a.D, s)) != hipSuccess) return e;
        if ((e = launch_col_sum(a.gw_part, 0, R, a.D, a.dgnorm_w, s)) != hipSuccess) return e;
    }
    if (a.df_bias) {
        if ((e = launch_fill_zero(a.df_bias, a.D, s)) != hipSuccess) return e;
        if ((e = launch_col_sum(a.fb_part, 0, R, a.D, a.df_bias, s)) != hipSuccess) return e;
    }
    timing_end(FAM_BWD_SCAN, s);
    return hipGetLastError();
}

}  // namespace mmf
