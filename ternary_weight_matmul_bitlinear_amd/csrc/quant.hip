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
// Layout: one wave per row at a time, rows strided over the waves of the grid.  A lane
// holds 8 consecutive elements per 512-element chunk of the row (one 16-byte bf16 load or
// two 16-byte fp32 loads per chunk), NC chunks per row, kept in registers between the max
// pass and the quantize pass, so the row is read from HBM once; the next row's loads are
// issued before the current row is reduced.  bf16 rows without a gain at the model widths
// use quant_rows256_kernel instead, whose waits never drain earlier stores.
// HBM-bound: K*(bytes_in + 1) bytes per row.
#include "mmf_internal.h"

namespace mmf {

namespace {

template <bool BF16> struct Chunk;
template <> struct Chunk<true> { uint4 u; };
template <> struct Chunk<false> { float4 a, b; };

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void *x, int64_t idx, Chunk<BF16> &c) {
    if constexpr (BF16) c.u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + idx);
    else {
        c.a = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + idx);
        c.b = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + idx + 4);
    }
}

template <bool BF16>
__device__ __forceinline__ void unpack_chunk(const Chunk<BF16> &c, float v[8]) {
    if constexpr (BF16) {
        const uint32_t w[4] = {c.u.x, c.u.y, c.u.z, c.u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        v[0] = c.a.x; v[1] = c.a.y; v[2] = c.a.z; v[3] = c.a.w;
        v[4] = c.b.x; v[5] = c.b.y; v[6] = c.b.z; v[7] = c.b.w;
    }
}

// NC = chunks of 512 elements per row held per lane (K <= 512*NC).
template <bool BF16, bool GAMMA, int NC>
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs p) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    const int K = p.K;

    // prefetch the next row only while both rows fit comfortably in registers
    constexpr bool PF = NC * (BF16 ? 4 : 8) <= 64;
    Chunk<BF16> cur[NC], nxt[PF ? NC : 1];
    auto fetch = [&](int64_t row, Chunk<BF16> *c) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int k0 = lane * 8 + 512 * i;
            if (k0 < K) load_chunk<BF16>(p.x, row * K + k0, c[i]);
        }
    };
    int64_t row = wave_id;
    if (PF && row < p.M) fetch(row, cur);
    for (; row < p.M; row += nwaves) {
        const int64_t next = row + nwaves;
        if constexpr (PF) {
            if (next < p.M) fetch(next, nxt);
        } else {
            fetch(row, cur);
        }

        float mx = 0.0f, ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int k0 = lane * 8 + 512 * i;
            if (k0 < K) {
                float v[8];
                unpack_chunk<BF16>(cur[i], v);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pj = GAMMA ? v[j] * p.gamma[k0 + j] : v[j];
                    mx = fmaxf(mx, fabsf(pj));
                    ss += v[j] * v[j];
                }
            }
        }
        mx = wave_max(mx);
        ss = wave_sum(ss);
        const float me = fmaxf(mx, 1e-5f);
        const float s = 127.0f / me;

        const bool cap = p.cap.row0 <= row && row < p.cap.row1;
        const int64_t crow = row - p.cap.row0;
        int qsum = 0;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int k0 = lane * 8 + 512 * i;
            if (k0 < K) {
                float v[8];
                unpack_chunk<BF16>(cur[i], v);
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
                *reinterpret_cast<uint2 *>(p.q + row * K + k0) = make_uint2(lo, hi);
                if (cap) {
                    if (p.cap.x_in) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) p.cap.x_in[crow * K + k0 + j] = v[j];
                    }
                    if (p.cap.q) *reinterpret_cast<uint2 *>(p.cap.q + crow * K + k0) = make_uint2(lo, hi);
                }
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
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < NC; ++i) cur[i] = nxt[i];
        }
    }
}

// bf16 rows without a gain at the model widths: lane l holds EPL consecutive elements
// EPL*l + 64*EPL*c of chunk c (EPL = 8: one 16-byte load and one 8-byte store per chunk, for
// widths that are multiples of 512; EPL = 4: 8-byte loads and 4-byte stores otherwise), NC
// chunks, R rows per wave with all of their loads issued before the first row is reduced.
// Every global access after the row loads is unconditional (the rows of a partial last
// wave are clamped to the last row and rewrite its identical results; the scale and code
// sum are stored by all lanes), so each wait covers only the loads of the row it precedes
// and never the earlier rows' stores.  CAP adds the stage-capture stores (tests only).
template <int NC, int R, bool CAP, int EPL>
__global__ __launch_bounds__(256) void quant_rows256_kernel(QuantArgs p) {
    constexpr int NWD = EPL / 2;  // 32-bit words (bf16 pairs) per lane per chunk
    typedef uint32_t raw_t __attribute__((ext_vector_type(NWD)));
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int K = p.K;
    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = wave_id * R + r;
        rows[r] = row < p.M ? row : p.M - 1;
    }
    raw_t raw[R][NC];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c)
            raw[r][c] = *reinterpret_cast<const raw_t *>(static_cast<const uint16_t *>(p.x) + rows[r] * K + lane * EPL + 64 * EPL * c);
    __builtin_amdgcn_sched_barrier(0);  // all row loads are issued here, not next to their use
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float v[NC][EPL];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int w = 0; w < NWD; ++w) {
                v[c][2 * w] = __uint_as_float(raw[r][c][w] << 16);
                v[c][2 * w + 1] = __uint_as_float(raw[r][c][w] & 0xFFFF0000u);
            }
        float mx = 0.0f, ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                mx = fmaxf(mx, fabsf(v[c][j]));
                ss += v[c][j] * v[c][j];
            }
        mx = wave_max(mx);
        ss = wave_sum(ss);
        const float me = fmaxf(mx, 1e-5f);
        const float sc = 127.0f / me;
        const int64_t row = rows[r];
        int qsum = 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            uint32_t pk[EPL / 4];
#pragma unroll
            for (int d = 0; d < EPL / 4; ++d) {
                pk[d] = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float q = rintf(v[c][4 * d + j] * sc);
                    q = fminf(fmaxf(q, -127.0f), 127.0f);
                    const int qi = static_cast<int>(q);
                    qsum += qi;
                    pk[d] |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * j);
                }
            }
            const int64_t k0 = lane * EPL + 64 * EPL * c;
            if constexpr (EPL == 8) *reinterpret_cast<uint2 *>(p.q + row * K + k0) = make_uint2(pk[0], pk[1]);
            else *reinterpret_cast<uint32_t *>(p.q + row * K + k0) = pk[0];
            if constexpr (CAP) {
                if (p.cap.row0 <= row && row < p.cap.row1) {
                    const int64_t crow = row - p.cap.row0;
#pragma unroll
                    for (int d = 0; d < EPL / 4; ++d) {
                        if (p.cap.x_in)
                            *reinterpret_cast<float4 *>(p.cap.x_in + crow * K + k0 + 4 * d) =
                                make_float4(v[c][4 * d], v[c][4 * d + 1], v[c][4 * d + 2], v[c][4 * d + 3]);
                        if (p.cap.q) *reinterpret_cast<uint32_t *>(p.cap.q + crow * K + k0 + 4 * d) = pk[d];
                    }
                }
            }
        }
        qsum = wave_sum_i(qsum);
        const float a = me / 127.0f * (1.0f / sqrtf(ss / static_cast<float>(K) + p.eps));
        p.a[row] = a;
        p.rowsum[row] = qsum;
        if constexpr (CAP) {
            if (lane == 0 && p.cap.a && p.cap.row0 <= row && row < p.cap.row1) p.cap.a[row - p.cap.row0] = a;
        }
    }
}

template <int NC, int R, int EPL>
void launch_rows256_r(const QuantArgs &a, hipStream_t s) {
    const int64_t waves = (a.M + R - 1) / R;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    if (a.cap.row1 > a.cap.row0) hipLaunchKernelGGL((quant_rows256_kernel<NC, R, true, EPL>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((quant_rows256_kernel<NC, R, false, EPL>), grid, dim3(256), 0, s, a);
}

// The model widths: D = 1024, 2048, 2560 and F = 5632 (16-byte loads), F = 2816, 6912 (8-byte
// loads), one row per wave (more rows per wave measured slower or equal).
bool launch_rows256(const QuantArgs &a, hipStream_t s) {
    if (!a.x_bf16 || a.gamma || a.K % 256 != 0) return false;
    if (a.K % 512 == 0) {
        switch (a.K / 512) {
            case 2: launch_rows256_r<2, 1, 8>(a, s); return true;
            case 4: launch_rows256_r<4, 1, 8>(a, s); return true;
            case 5: launch_rows256_r<5, 1, 8>(a, s); return true;
            case 11: launch_rows256_r<11, 1, 8>(a, s); return true;
            default: return false;
        }
    }
    switch (a.K / 256) {
        case 11: launch_rows256_r<11, 1, 4>(a, s); return true;
        case 27: launch_rows256_r<27, 1, 4>(a, s); return true;
        default: return false;
    }
}

template <bool BF16, bool GAMMA>
void launch_nc(const QuantArgs &a, dim3 grid, hipStream_t s) {
    const int nc = (a.K + 511) / 512;
    if (nc <= 2) hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 2>), grid, dim3(256), 0, s, a);
    else if (nc <= 4) hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 4>), grid, dim3(256), 0, s, a);
    else if (nc <= 8) hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 8>), grid, dim3(256), 0, s, a);
    else if (nc <= 16) hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 16>), grid, dim3(256), 0, s, a);
    else if (nc <= 32) hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 32>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((quant_rows_kernel<BF16, GAMMA, 64>), grid, dim3(256), 0, s, a);
}
}  // namespace

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    // enough waves to keep every CU busy; each wave walks rows with a stride
    const int64_t wg_needed = (a.M + 3) / 4;
    const int64_t wg_cap = 256 * 8;
    const dim3 grid(static_cast<unsigned>(wg_needed < wg_cap ? wg_needed : wg_cap));
    timing_begin(FAM_QUANT, s);
    if (launch_rows256(a, s)) {
    } else if (a.x_bf16) {
        if (a.gamma) launch_nc<true, true>(a, grid, s);
        else launch_nc<true, false>(a, grid, s);
    } else {
        if (a.gamma) launch_nc<false, true>(a, grid, s);
        else launch_nc<false, false>(a, grid, s);
    }
    timing_end(FAM_QUANT, s);
    return hipGetLastError();
}

}  // namespace mmf
