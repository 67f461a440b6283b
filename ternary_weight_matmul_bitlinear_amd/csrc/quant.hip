// quant.hip -- per-token activation quantization (RMSNorm + absmax int8) for gfx950.
//
// DataCamp "MatMul-free language models", section "Core components: MLGRU and GLU":
// activations are RMS-normalised before they are quantized.  Hysen Labs "MatMul-Free LM",
// section "FusedBitLinear": norm, quantization and accumulation belong to one BitLinear.
// Per row x[0..K) with gain gamma:
//   p = fl32(x*gamma), m = max(max|p|, 1e-5), s = fl32(127/m),
//   q = clamp(rint(fl32(p*s)), -127, 127), a = m/127 * 1/sqrt(mean(x^2) + eps).
// The RMSNorm factor cancels in p*s, so q does not depend on any fp reduction order; it
// enters only a.  Each multiply is a single fp32 rounding (no contraction: there is no add
// to fuse), the division is IEEE, rint rounds half to even.
//
// Layout: one wave per row, 4 rows per 256-thread workgroup; each lane handles 8
// consecutive elements per step (one 16-byte bf16 load or two 16-byte fp32 loads), so a
// wave streams 512 contiguous elements of its row per step.  The row is read twice (max,
// then quantize); the second pass hits L1/L2.  HBM-bound: K*(bytes_in + 1) bytes per row.
#include "mmf_internal.h"

namespace mmf {

template <bool BF16>
__device__ __forceinline__ void load8(const void *x, int64_t idx, float v[8]) {
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

template <bool BF16, bool GAMMA>
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= p.M) return;
    const int K = p.K;
    const int64_t base = row * K;

    float mx = 0.0f, ss = 0.0f;
    for (int k0 = lane * 8; k0 < K; k0 += 512) {
        float v[8];
        load8<BF16>(p.x, base + k0, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pj = GAMMA ? v[j] * p.gamma[k0 + j] : v[j];
            mx = fmaxf(mx, fabsf(pj));
            ss += v[j] * v[j];
        }
    }
    mx = wave_max(mx);
    ss = wave_sum(ss);
    const float me = fmaxf(mx, 1e-5f);
    const float s = 127.0f / me;

    const bool cap = p.cap.row0 <= row && row < p.cap.row1;
    const int64_t crow = row - p.cap.row0;
    int qsum = 0;
    for (int k0 = lane * 8; k0 < K; k0 += 512) {
        float v[8];
        load8<BF16>(p.x, base + k0, v);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pj = GAMMA ? v[j] * p.gamma[k0 + j] : v[j];
            float r = rintf(pj * s);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const int qi = static_cast<int>(r);
            qsum += qi;
            const uint32_t byte = static_cast<uint32_t>(qi) & 0xFFu;
            if (j < 4) lo |= byte << (8 * j);
            else hi |= byte << (8 * (j - 4));
        }
        *reinterpret_cast<uint2 *>(p.q + base + k0) = make_uint2(lo, hi);
        if (cap) {
            if (p.cap.x_in) {
#pragma unroll
                for (int j = 0; j < 8; ++j) p.cap.x_in[crow * K + k0 + j] = v[j];
            }
            if (p.cap.q)
                *reinterpret_cast<uint2 *>(p.cap.q + crow * K + k0) = make_uint2(lo, hi);
        }
    }
    qsum = wave_sum_i(qsum);
    if (lane == 0) {
        const float r = 1.0f / sqrtf(ss / static_cast<float>(K) + p.eps);
        const float a = me / 127.0f * r;
        p.a[row] = a;
        p.rowsum[row] = qsum;
        if (cap && p.cap.a) p.cap.a[crow] = a;
    }
}

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.M + 3) / 4)), block(256);
    timing_begin(FAM_QUANT, s);
    if (a.x_bf16) {
        if (a.gamma) hipLaunchKernelGGL((quant_rows_kernel<true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((quant_rows_kernel<true, false>), grid, block, 0, s, a);
    } else {
        if (a.gamma) hipLaunchKernelGGL((quant_rows_kernel<false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((quant_rows_kernel<false, false>), grid, block, 0, s, a);
    }
    timing_end(FAM_QUANT, s);
    return hipGetLastError();
}

}  // namespace mmf
