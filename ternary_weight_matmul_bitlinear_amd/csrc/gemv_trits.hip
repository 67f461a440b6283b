// gemv_trits.hip -- decode-regime BitLinear over base-3 packed ternary weights: five weights
// per byte (1.6 bits each) instead of four (2 bits), for the few-token regime where the
// weight stream is the traffic.
//
// HackerPapers page on arXiv 2406.02528 "Scalable MatMul-free Language Modeling" (HN
// discussion list): the weights are ternary digits, trits, and 3^5 = 243 <= 256 puts five in
// a byte.  DataCamp "MatMul-free language models", section "From optimised GPU to custom
// FPGA": token generation is limited by moving the weights.
//
// Format (host_ternary.cpp): codes c = q + 1; byte j of 4-byte word w of a row holds the
// codes of k = 20w + 4i + j, i = 0..4, as the base-3 number v = sum_i c_i 3^(4-i), stored as
// b = ceil(256 v / 243); rows are padded with q = 0 to 16-byte chunks of 80 weights.
//
// Unpacking: b / 256 is v / 243 rounded up by less than 1/256, so multiplying by 3 moves the
// next base-3 digit into the integer part: t_0 = b, digit_i = (3 t_i) >> 8, t_{i+1} =
// (3 t_i) & 255, exact for all five digits (the rounding, scaled by 3^5 / 256 < 1, never
// crosses a digit boundary).  A word's four bytes sit in two registers of two 16-bit lanes
// (bytes 0,2 and 1,3), so each round is one packed 16-bit multiply, one packed shift and one
// mask per register, and digit i of the four bytes is exactly the int8x4 code vector of
// k = 20w + 4i .. 20w + 4i + 3: one v_dot4_i32_i8 against the activation codes.  The codes
// (0, 1, 2) are multiplied as they are and the token's code sum is removed once per row:
// acc = sum q_x*c - sum q_x (exact in int32).
//
// Layout: 16 lanes per weight row, 4 rows per wave, 16 rows per workgroup; lane j holds the
// row's 16-byte chunks j, j+16, ... (NCH of them), all requested at kernel entry; the
// workgroup quantizes up to four token rows into LDS meanwhile (the arithmetic of every
// other quantizer of the library, so the int8 codes are identical), padded with zero codes
// to the chunk grid.
#include "mmf_internal.h"

namespace mmf {

namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr int kTritTG = 4;   // token rows per workgroup

template <bool BF16>
__device__ __forceinline__ void load4v(const void *x, int64_t i, float (&v)[4]) {
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + i);
        v[0] = __uint_as_float(u.x << 16);
        v[1] = __uint_as_float(u.x & 0xFFFF0000u);
        v[2] = __uint_as_float(u.y << 16);
        v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + i);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
}

// The 20 code vectors of one 16-byte chunk (4 words x 5 digits), index 5w + i.
__device__ __forceinline__ void chunk_codes(const uint4 &ch, int (&cd)[20]) {
    const uint32_t wd[4] = {ch.x, ch.y, ch.z, ch.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t lo = wd[w] & 0x00FF00FFu, hi = (wd[w] >> 8) & 0x00FF00FFu;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const u16x2 l3 = __builtin_bit_cast(u16x2, lo) * static_cast<unsigned short>(3);
            const u16x2 h3 = __builtin_bit_cast(u16x2, hi) * static_cast<unsigned short>(3);
            const uint32_t dl = __builtin_bit_cast(uint32_t, l3 >> static_cast<unsigned short>(8));
            const uint32_t dh = __builtin_bit_cast(uint32_t, h3 >> static_cast<unsigned short>(8));
            lo = __builtin_bit_cast(uint32_t, l3) & 0x00FF00FFu;
            hi = __builtin_bit_cast(uint32_t, h3) & 0x00FF00FFu;
            cd[5 * w + i] = static_cast<int>(dl | (dh << 8));
        }
    }
}

template <bool XBF16, bool OBF16, int NCH>
__global__ __launch_bounds__(256) void gemv_trits_kernel(TritArgs p) {
    extern __shared__ __attribute__((aligned(16))) int8_t xq[];   // [kTritTG][Kpad] int8 codes
    __shared__ float red_m[4][kTritTG], red_s[4][kTritTG];
    __shared__ int red_q[4][kTritTG];
    __shared__ float s_a[kTritTG];
    __shared__ int s_rs[kTritTG];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.K, RB = p.row_bytes, NCHK = RB / 16, Kpad = RB * 5;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTritTG;
    const int mt = static_cast<int>(p.M - t0 < kTritTG ? p.M - t0 : kTritTG);

    // ---- weight chunks of this lane's row, requested first (clamped, masked below)
    const int slot = lane >> 4, j = lane & 15;
    const int r = blockIdx.x * 16 + wave * 4 + slot;
    const int rr = r < p.N ? r : p.N - 1;
    uint4 wv[NCH];
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
        const int c = j + 16 * it < NCHK ? j + 16 * it : NCHK - 1;
        wv[it] = *reinterpret_cast<const uint4 *>(p.packed + static_cast<int64_t>(rr) * RB + 16 * c);
    }

    // ---- quantize the token group: pass 1 row max |x*gamma| and sum x^2
    float pm[kTritTG], ps[kTritTG];
#pragma unroll
    for (int t = 0; t < kTritTG; ++t) {
        pm[t] = 0.f;
        ps[t] = 0.f;
        if (t < mt) {
            const int64_t base = (t0 + t) * K;
            for (int k = tid * 4; k < K; k += 1024) {
                float v[4];
                load4v<XBF16>(p.x, base + k, v);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pv = p.gamma ? v[e] * p.gamma[k + e] : v[e];
                    pm[t] = fmaxf(pm[t], fabsf(pv));
                    ps[t] = fmaf(v[e], v[e], ps[t]);
                }
            }
        }
    }
    {
        const float rm = wave_reduce_multi<kTritTG, true>(pm);
        const float rs = wave_reduce_multi<kTritTG, false>(ps);
        if ((lane & 15) == 0) {
            red_m[wave][lane >> 4] = rm;
            red_s[wave][lane >> 4] = rs;
        }
    }
    __syncthreads();
    float sc[kTritTG];
#pragma unroll
    for (int t = 0; t < kTritTG; ++t) {
        const float m = fmaxf(fmaxf(red_m[0][t], red_m[1][t]), fmaxf(red_m[2][t], red_m[3][t]));
        const float me = fmaxf(m, 1e-5f);
        sc[t] = 127.0f / me;
        if (tid == 0) {
            const float s2 = (red_s[0][t] + red_s[1][t]) + (red_s[2][t] + red_s[3][t]);
            s_a[t] = me / 127.0f * (1.0f / sqrtf(s2 * (1.0f / static_cast<float>(K)) + p.eps));
        }
    }
    // pass 2: int8 codes into LDS (zero codes past K and for absent tokens), code sums
    int qs[kTritTG];
    const bool cap_blk = blockIdx.x == 0;
#pragma unroll
    for (int t = 0; t < kTritTG; ++t) {
        qs[t] = 0;
        const int64_t row = t0 + t;
        const bool capr = cap_blk && t < mt && p.cap.row0 <= row && row < p.cap.row1;
        for (int k = tid * 4; k < Kpad; k += 1024) {
            uint32_t pk = 0;
            if (t < mt && k < K) {
                float v[4];
                load4v<XBF16>(p.x, row * K + k, v);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pv = p.gamma ? v[e] * p.gamma[k + e] : v[e];
                    float q = rintf(pv * sc[t]);
                    q = fminf(fmaxf(q, -127.0f), 127.0f);
                    const int qi = static_cast<int>(q);
                    qs[t] += qi;
                    pk |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * e);
                }
                if (capr) {
                    const int64_t cr = row - p.cap.row0;
                    if (p.cap.x_in)
                        *reinterpret_cast<float4 *>(p.cap.x_in + cr * K + k) = make_float4(v[0], v[1], v[2], v[3]);
                    if (p.cap.q) *reinterpret_cast<uint32_t *>(p.cap.q + cr * K + k) = pk;
                }
            }
            *reinterpret_cast<uint32_t *>(xq + t * Kpad + k) = pk;
        }
    }
    {
        const int rq = wave_reduce_multi<kTritTG, false>(qs);
        if ((lane & 15) == 0) red_q[wave][lane >> 4] = rq;
    }
    __syncthreads();
    if (tid < kTritTG) {
        s_rs[tid] = (red_q[0][tid] + red_q[1][tid]) + (red_q[2][tid] + red_q[3][tid]);
        const int64_t row = t0 + tid;
        if (cap_blk && tid < mt && p.cap.a && p.cap.row0 <= row && row < p.cap.row1)
            p.cap.a[row - p.cap.row0] = s_a[tid];
    }

    // ---- dot products: codes of a chunk extracted once, used for every token
    int acc[kTritTG];
#pragma unroll
    for (int t = 0; t < kTritTG; ++t) acc[t] = 0;
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
        const int c = j + 16 * it;
        if (c < NCHK) {
            int cd[20];
            chunk_codes(wv[it], cd);
#pragma unroll
            for (int t = 0; t < kTritTG; ++t) {
                if (t < mt) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(xq + t * Kpad + 80 * c);
#pragma unroll
                    for (int u = 0; u < 5; ++u) {
                        const uint4 xv = xp[u];
                        acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(xv.x), cd[4 * u], acc[t], false);
                        acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(xv.y), cd[4 * u + 1], acc[t], false);
                        acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(xv.z), cd[4 * u + 2], acc[t], false);
                        acc[t] = __builtin_amdgcn_sdot4(static_cast<int>(xv.w), cd[4 * u + 3], acc[t], false);
                    }
                }
            }
        }
    }
    __syncthreads();   // LDS reads done before the row sums are read below (same slots)
#pragma unroll
    for (int t = 0; t < kTritTG; ++t) {
        int v = acc[t];
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 4, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 1, 64);
        acc[t] = v;
    }
    // lane j < mt of the row stores token j
    if (r < p.N && j < mt) {
        int a = acc[0];
#pragma unroll
        for (int t = 1; t < kTritTG; ++t)
            if (t == j) a = acc[t];
        const int exact = a - s_rs[j];
        float y = static_cast<float>(exact) * p.scale * s_a[j];
        if (p.bias) y += p.bias[r];
        const int64_t row = t0 + j;
        if constexpr (OBF16) static_cast<uint16_t *>(p.out)[row * p.N + r] = f32_to_bf16_bits(y);
        else static_cast<float *>(p.out)[row * p.N + r] = y;
        if (p.cap.row0 <= row && row < p.cap.row1) {
            const int64_t cr = row - p.cap.row0;
            if (p.cap.acc) p.cap.acc[cr * p.N + r] = exact;
            if (p.cap.y_out) p.cap.y_out[cr * p.N + r] = OBF16 ? round_to_bf16(y) : y;
        }
    }
}

template <bool XBF16, bool OBF16>
hipError_t launch_trits_x(const TritArgs &a, hipStream_t s) {
    const int nchk = a.row_bytes / 16;
    const int per_lane = (nchk + 15) / 16;
    const dim3 grid(static_cast<unsigned>((a.N + 15) / 16), static_cast<unsigned>((a.M + kTritTG - 1) / kTritTG));
    const size_t lds = static_cast<size_t>(kTritTG) * a.row_bytes * 5;
    if (per_lane <= 1) hipLaunchKernelGGL((gemv_trits_kernel<XBF16, OBF16, 1>), grid, dim3(256), lds, s, a);
    else if (per_lane <= 2) hipLaunchKernelGGL((gemv_trits_kernel<XBF16, OBF16, 2>), grid, dim3(256), lds, s, a);
    else if (per_lane <= 4) hipLaunchKernelGGL((gemv_trits_kernel<XBF16, OBF16, 4>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((gemv_trits_kernel<XBF16, OBF16, 8>), grid, dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_trits(const TritArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    timing_begin(FAM_GEMV, s);
    hipError_t e;
    if (a.x_bf16) e = a.out_bf16 ? launch_trits_x<true, true>(a, s) : launch_trits_x<true, false>(a, s);
    else e = a.out_bf16 ? launch_trits_x<false, true>(a, s) : launch_trits_x<false, false>(a, s);
    timing_end(FAM_GEMV, s);
    return e;
}

}  // namespace mmf
