// gemv_decode.hip -- decode-regime BitLinear for a few tokens: streams the 2-bit packed
// ternary weights from HBM once per token group and reduces with cross-lane shuffles.
//
// DataCamp "MatMul-free language models", sections "Replacing MatMul with ternary
// operations" (products by -1/0/+1 are sign-matched adds) and "From optimised GPU to
// custom FPGA" (token generation is limited by moving the weights); Hysen Labs
// "MatMul-Free LM", section "FusedBitLinear" (norm + quantize + accumulate in one kernel).
//
// With one token per step the weights (0.25 byte each) are read once and used once, so
// the kernel is HBM-bound.  Design:
//   - prologue: the workgroup RMS/absmax-quantizes its token group (<= 8 rows) straight
//     into LDS (the same arithmetic as the standalone quantizer, so the int8 codes are
//     identical), or copies rows that are already quantized;
//   - each wave owns 8 weight rows, 8 lanes per row; lane j of a row reads 16-byte chunks
//     j, j+8, ... (64 k each), so one load instruction moves 8 rows x 128 contiguous bytes;
//   - each packed word unpacks to four dwords of int8 codes (code = q+1) consumed by
//     v_dot4_i32_i8 against the LDS-resident int8 activations; the code offset is removed
//     with the row sum of the activations (acc = sum q_x*code - sum q_x, exact);
//   - the 8 partial sums of a row are combined with 3 xor-shuffle steps, after which lane j
//     of the row writes token j (fused rescale, bias, residual or SiLU(gate)*up).
// LDS layout of a token row: chunk c (64 bytes) at byte 64c + 16*(c/2), which puts the
// eight chunks read by one instruction on disjoint bank quads.
#include "mmf_internal.h"

namespace mmf {

namespace {

__device__ __forceinline__ int chunk_off(int c) { return c * 64 + (c >> 1) * 16; }

template <bool BF16>
__device__ __forceinline__ void load8v(const void *x, int64_t idx, float v[8]) {
    if constexpr (BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + idx);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + idx);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + idx + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ __forceinline__ int dot16(const v4i q[4], const v4i c[4], int acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = __builtin_amdgcn_sdot4(q[i].x, c[i].x, acc, false);
        acc = __builtin_amdgcn_sdot4(q[i].y, c[i].y, acc, false);
        acc = __builtin_amdgcn_sdot4(q[i].z, c[i].z, acc, false);
        acc = __builtin_amdgcn_sdot4(q[i].w, c[i].w, acc, false);
    }
    return acc;
}

// XIN: 0 = pre-quantized input, 1 = fp32 activations, 2 = bf16 activations.
template <int EPI, int XIN, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemv_dot4_kernel(GemvArgs p) {
    extern __shared__ __attribute__((aligned(16))) int8_t qs[];
    __shared__ float red_a[4][kGemvTokens], red_b[4][kGemvTokens];
    __shared__ float s_a[kGemvTokens];
    __shared__ int s_rs[kGemvTokens];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.K, NC = K / 64;
    const int rowb = chunk_off(NC);  // bytes per token row in LDS (NC is even or padded)
    const int TG = p.tokens_per_group;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * TG;
    const int mt = static_cast<int>(p.M - t0 < TG ? p.M - t0 : TG);
    const bool cap_blk = blockIdx.x == 0;

    // ---------------------------------------------------------------- prologue
    if constexpr (XIN != 0) {
        constexpr bool BF = XIN == 2;
        float pm[kGemvTokens], ps[kGemvTokens];
#pragma unroll
        for (int t = 0; t < kGemvTokens; ++t) { pm[t] = 0.f; ps[t] = 0.f; }
#pragma unroll
        for (int t = 0; t < kGemvTokens; ++t) {
            if (t >= mt) break;
            for (int k0 = tid * 8; k0 < K; k0 += 2048) {
                float v[8];
                load8v<BF>(p.x, (t0 + t) * K + k0, v);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pj = p.gamma ? v[j] * p.gamma[k0 + j] : v[j];
                    pm[t] = fmaxf(pm[t], fabsf(pj));
                    ps[t] += v[j] * v[j];
                }
            }
            pm[t] = wave_max(pm[t]);
            ps[t] = wave_sum(ps[t]);
            if (lane == 0) { red_a[wave][t] = pm[t]; red_b[wave][t] = ps[t]; }
        }
        __syncthreads();
        float sc[kGemvTokens];
        int qsum[kGemvTokens];
#pragma unroll
        for (int t = 0; t < kGemvTokens; ++t) {
            const float mx = fmaxf(fmaxf(red_a[0][t], red_a[1][t]), fmaxf(red_a[2][t], red_a[3][t]));
            const float me = fmaxf(mx, 1e-5f);
            sc[t] = 127.0f / me;
            qsum[t] = 0;
            if (tid == 0 && t < mt) {
                const float ss = (red_b[0][t] + red_b[1][t]) + (red_b[2][t] + red_b[3][t]);
                s_a[t] = me / 127.0f * (1.0f / sqrtf(ss / static_cast<float>(K) + p.eps));
            }
        }
#pragma unroll
        for (int t = 0; t < kGemvTokens; ++t) {
            if (t >= mt) break;
            const int64_t tok = t0 + t;
            const bool capt = cap_blk && p.cap.row0 <= tok && tok < p.cap.row1;
            for (int k0 = tid * 8; k0 < K; k0 += 2048) {
                float v[8];
                load8v<BF>(p.x, tok * K + k0, v);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pj = p.gamma ? v[j] * p.gamma[k0 + j] : v[j];
                    float r = rintf(pj * sc[t]);
                    r = fminf(fmaxf(r, -127.0f), 127.0f);
                    const int qi = static_cast<int>(r);
                    qsum[t] += qi;
                    const uint32_t byte = static_cast<uint32_t>(qi) & 0xFFu;
                    if (j < 4) lo |= byte << (8 * j);
                    else hi |= byte << (8 * (j - 4));
                }
                const int c = k0 >> 6;
                *reinterpret_cast<uint2 *>(qs + t * rowb + chunk_off(c) + (k0 & 63)) = make_uint2(lo, hi);
                if (capt) {
                    const int64_t cr = tok - p.cap.row0;
                    if (p.cap.x_in)
#pragma unroll
                        for (int j = 0; j < 8; ++j) p.cap.x_in[cr * K + k0 + j] = v[j];
                    if (p.cap.q) *reinterpret_cast<uint2 *>(p.cap.q + cr * K + k0) = make_uint2(lo, hi);
                }
            }
            qsum[t] = wave_sum_i(qsum[t]);
        }
        __syncthreads();  // red_a reuse below
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < kGemvTokens; ++t) red_a[wave][t] = __int_as_float(qsum[t]);
        }
        __syncthreads();
        if (tid < mt) {
            s_rs[tid] = (__float_as_int(red_a[0][tid]) + __float_as_int(red_a[1][tid])) +
                        (__float_as_int(red_a[2][tid]) + __float_as_int(red_a[3][tid]));
            const int64_t tok = t0 + tid;
            if (cap_blk && p.cap.a && p.cap.row0 <= tok && tok < p.cap.row1)
                p.cap.a[tok - p.cap.row0] = s_a[tid];
        }
    } else {
        for (int t = 0; t < mt; ++t)
            for (int k0 = tid * 16; k0 < K; k0 += 4096) {
                const uint4 v = *reinterpret_cast<const uint4 *>(p.q + (t0 + t) * K + k0);
                *reinterpret_cast<uint4 *>(qs + t * rowb + chunk_off(k0 >> 6) + (k0 & 63)) = v;
            }
        if (tid < mt) {
            s_a[tid] = p.a[t0 + tid];
            s_rs[tid] = p.rowsum[t0 + tid];
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- main loop
    const int slot = lane >> 3, j = lane & 7;
    const int r = blockIdx.x * 32 + wave * 8 + slot;
    const bool rvalid = r < p.rows_total;
    int sg = 0, n = r;
    if constexpr (EPI != EPI_GLU) {
        while (sg + 1 < p.nseg && n >= p.seg[sg].n) { n -= p.seg[sg].n; ++sg; }
    }
    const int nn = rvalid ? n : 0;
    const uint32_t *w0 = p.seg[sg].packed + static_cast<int64_t>(nn) * (K / 16);
    const uint32_t *w1 = EPI == EPI_GLU ? p.seg[1].packed + static_cast<int64_t>(nn) * (K / 16) : nullptr;

    int acc0[kGemvTokens], acc1[kGemvTokens];
#pragma unroll
    for (int t = 0; t < kGemvTokens; ++t) { acc0[t] = 0; acc1[t] = 0; }

    for (int c = j; c < NC; c += 8) {
        const uint4 wa = *reinterpret_cast<const uint4 *>(w0 + c * 4);
        v4i ca[4] = {unpack_codes(wa.x), unpack_codes(wa.y), unpack_codes(wa.z), unpack_codes(wa.w)};
        v4i cb[4];
        if constexpr (EPI == EPI_GLU) {
            const uint4 wb = *reinterpret_cast<const uint4 *>(w1 + c * 4);
            cb[0] = unpack_codes(wb.x); cb[1] = unpack_codes(wb.y);
            cb[2] = unpack_codes(wb.z); cb[3] = unpack_codes(wb.w);
        }
#pragma unroll
        for (int t = 0; t < kGemvTokens; ++t) {
            if (t >= mt) break;
            const v4i *qp = reinterpret_cast<const v4i *>(qs + t * rowb + chunk_off(c));
            const v4i qv[4] = {qp[0], qp[1], qp[2], qp[3]};
            acc0[t] = dot16(qv, ca, acc0[t]);
            if constexpr (EPI == EPI_GLU) acc1[t] = dot16(qv, cb, acc1[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < kGemvTokens; ++t) {
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) {
            acc0[t] += __shfl_xor(acc0[t], o, 64);
            if constexpr (EPI == EPI_GLU) acc1[t] += __shfl_xor(acc1[t], o, 64);
        }
    }
    // lane j of the row writes token j
    int my0 = 0, my1 = 0;
#pragma unroll
    for (int t = 0; t < kGemvTokens; ++t)
        if (t == j) { my0 = acc0[t]; my1 = acc1[t]; }
    if (!rvalid || j >= mt) return;
    const int64_t tok = t0 + j;
    const int32_t rs = s_rs[j];
    const float at = s_a[j];
    const bool capr = p.cap.row0 <= tok && tok < p.cap.row1;
    const int64_t crow = tok - p.cap.row0;
    if constexpr (EPI == EPI_GLU) {
        const int32_t ag = my0 - rs, au = my1 - rs;
        float yg = static_cast<float>(ag) * (p.seg[0].scale * at);
        float yu = static_cast<float>(au) * (p.seg[1].scale * at);
        if (p.seg[0].bias) yg += p.seg[0].bias[n];
        if (p.seg[1].bias) yu += p.seg[1].bias[n];
        const float mv = siluf_(yg) * yu;
        store_act<OUT_BF16>(p.out, tok * p.ldo + n, mv);
        if (capr) {
            if (p.cap.acc) {
                int32_t *cp = p.cap.acc + crow * p.cap.acc_ld;
                cp[p.seg[0].cap_col0 + n] = ag;
                cp[p.seg[1].cap_col0 + n] = au;
            }
            if (p.cap.y_out) p.cap.y_out[crow * p.ldo + n] = OUT_BF16 ? round_to_bf16(mv) : mv;
        }
    } else {
        const Seg &S = p.seg[sg];
        const int32_t av = my0 - rs;
        float y = static_cast<float>(av) * (S.scale * at);
        if (S.bias) y += S.bias[n];
        if constexpr (EPI == EPI_RESID) y = load_act<OUT_BF16>(p.resid, tok * p.ldr + S.out_col0 + n) + y;
        store_act<OUT_BF16>(p.out, tok * p.ldo + S.out_col0 + n, y);
        if (capr) {
            if (p.cap.acc) p.cap.acc[crow * p.cap.acc_ld + S.cap_col0 + n] = av;
            if (p.cap.y_out) p.cap.y_out[crow * p.ldo + S.out_col0 + n] = OUT_BF16 ? round_to_bf16(y) : y;
        }
    }
}

template <int EPI, int XIN>
void launch3(const GemvArgs &a, dim3 grid, size_t lds, hipStream_t s) {
    if (a.out_bf16) hipLaunchKernelGGL((gemv_dot4_kernel<EPI, XIN, true>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((gemv_dot4_kernel<EPI, XIN, false>), grid, dim3(256), lds, s, a);
}

template <int EPI>
void launch2(const GemvArgs &a, dim3 grid, size_t lds, hipStream_t s) {
    if (!a.x) launch3<EPI, 0>(a, grid, lds, s);
    else if (a.x_bf16) launch3<EPI, 2>(a, grid, lds, s);
    else launch3<EPI, 1>(a, grid, lds, s);
}

}  // namespace

// Bytes of LDS per token row for a given K.
size_t gemv_lds_row_bytes(int K) {
    const int nc = K / 64;
    return static_cast<size_t>(nc * 64 + (nc >> 1) * 16 + 16);
}

hipError_t launch_gemv(const GemvArgs &a_in, hipStream_t s) {
    if (a_in.M <= 0) return hipSuccess;
    GemvArgs a = a_in;
    const size_t rowb = gemv_lds_row_bytes(a.K);
    int tg = static_cast<int>((64 * 1024) / rowb);
    if (tg > kGemvTokens) tg = kGemvTokens;
    if (tg < 1) tg = 1;
    a.tokens_per_group = tg;
    const dim3 grid(static_cast<unsigned>((a.rows_total + 31) / 32),
                    static_cast<unsigned>((a.M + tg - 1) / tg));
    const size_t lds = rowb * tg;
    timing_begin(FAM_GEMV, s);
    switch (a.epi) {
        case EPI_STORE: launch2<EPI_STORE>(a, grid, lds, s); break;
        case EPI_RESID: launch2<EPI_RESID>(a, grid, lds, s); break;
        default: launch2<EPI_GLU>(a, grid, lds, s); break;
    }
    timing_end(FAM_GEMV, s);
    return hipGetLastError();
}

}  // namespace mmf
