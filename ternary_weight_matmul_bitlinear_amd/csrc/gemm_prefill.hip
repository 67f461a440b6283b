// gemm_prefill.hip -- prefill-regime BitLinear: int8 activations x 2-bit ternary weights
// on the gfx950 int8 matrix cores (v_mfma_i32_32x32x32_i8).
//
// DataCamp "MatMul-free language models", section "Replacing MatMul with ternary
// operations": with weights in {-1,0,1} every product is a negate/drop/keep of an int8
// activation, so the layer output is an exact signed integer sum.  At thousands of tokens
// that sum is a dense contraction, so it runs on MFMA: the packed weights are unpacked in
// registers to int8 codes c = q + 1 in {0,1,2}, multiplied on the matrix cores, and the
// offset is removed once per row: acc = sum_k q_x*c - sum_k q_x (exact in int32).
//
// Tiling (256 threads = 4 waves as 2x2, tile 128 x 128 x 64):
//   - A (int8 activations) tile 128 rows x 64 k staged in LDS with an 80-byte row pitch
//     (conflict-free 16-byte reads: 8 consecutive rows land on disjoint bank quads);
//   - B (packed weights) tile 128 rows x 4 words staged in LDS with a 24-byte pitch
//     (conflict-free 8-byte reads); one packed word is exactly the 16-code B operand of a
//     lane, so B travels 2 bits per weight all the way to the registers;
//   - each wave owns 64 x 64 of the output = 2 x 2 MFMA blocks of 32 x 32; per 64-deep k
//     step a lane issues 8 MFMAs;
//   - lane l (r = l % 32, g = l / 32) feeds, for MFMA half ks in {0,1}, activation bytes
//     k = 32g + 16ks + [0,16) of row r and packed word 2g + ks of weight row r, so A and B
//     agree on every (lane group, byte) -> k pairing;
//   - double-buffered LDS with the next tile prefetched into registers during the MFMAs.
// Epilogues (fused, in registers): y = acc*s_w*a (+bias) stored in fp32/bf16; the same plus
// a residual; or SiLU(gate)*up when the tile pairs 64 gate rows with the same 64 up rows.
#include "mmf_internal.h"

namespace mmf {

namespace {
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int A_PITCH = 80;  // bytes
constexpr int B_PITCH = 24;  // bytes

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_ternary_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) int8_t smA[2][BM * A_PITCH];
    __shared__ __attribute__((aligned(16))) int8_t smB[2][BN * B_PITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int K = p.K, KW = K / 16;  // words per packed row

    // ---- tile coordinates
    const int mt = blockIdx.x / p.tiles_n_total;
    int nt = blockIdx.x % p.tiles_n_total;
    int sg = 0;
    while (sg + 1 < p.nseg && nt >= p.tiles_n[sg]) { nt -= p.tiles_n[sg]; ++sg; }
    const int64_t m0 = static_cast<int64_t>(mt) * BM;

    // ---- global source pointers (clamped in-bounds; out-of-range rows are never stored)
    const int arow = tid >> 1, ahalf = tid & 1;
    const int64_t ag = m0 + arow < p.M ? m0 + arow : p.M - 1;
    const int8_t *aptr = p.A + ag * K + ahalf * 32;
    const uint32_t *bptr = nullptr;
    if (tid < BN) {
        if constexpr (EPI == EPI_GLU) {
            const int sub = (tid & 63) >> 5;
            const int f = nt * 64 + 32 * (tid >> 6) + (tid & 31);
            const Seg &S = p.seg[sub];
            bptr = S.packed + static_cast<int64_t>(f < S.n ? f : S.n - 1) * KW;
        } else {
            const Seg &S = p.seg[sg];
            const int n = nt * BN + tid;
            bptr = S.packed + static_cast<int64_t>(n < S.n ? n : S.n - 1) * KW;
        }
    }

    uint4 ra0, ra1, rb = make_uint4(0, 0, 0, 0);
    auto gload = [&](int kt) {
        ra0 = *reinterpret_cast<const uint4 *>(aptr + kt * BK);
        ra1 = *reinterpret_cast<const uint4 *>(aptr + kt * BK + 16);
        if (tid < BN) rb = *reinterpret_cast<const uint4 *>(bptr + kt * 4);
    };
    auto sstore = [&](int buf) {
        int8_t *da = smA[buf] + arow * A_PITCH + ahalf * 32;
        *reinterpret_cast<uint4 *>(da) = ra0;
        *reinterpret_cast<uint4 *>(da + 16) = ra1;
        if (tid < BN) {
            uint2 *db = reinterpret_cast<uint2 *>(smB[buf] + tid * B_PITCH);
            db[0] = make_uint2(rb.x, rb.y);
            db[1] = make_uint2(rb.z, rb.w);
        }
    };

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    const int g = lane >> 5, r32 = lane & 31;
    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        v4i av[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const int8_t *pa = smA[cur] + (wm * 64 + mi * 32 + r32) * A_PITCH + g * 32;
            av[mi][0] = *reinterpret_cast<const v4i *>(pa);
            av[mi][1] = *reinterpret_cast<const v4i *>(pa + 16);
        }
        uint2 bw[2];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
            bw[ni] = *reinterpret_cast<const uint2 *>(smB[cur] + (wn * 64 + ni * 32 + r32) * B_PITCH + g * 8);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const v4i bv = unpack_codes(ks ? bw[ni].y : bw[ni].x);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][ks], bv, acc[mi][ni], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds C[row][col] for col = r32 of each 32-wide block and
    //      rows 8*(e/4) + 4*g + (e%4) of each 32-tall block.
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t row = m0 + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (row >= p.M) continue;
            const int32_t rs = p.rowsum[row];
            const float arow_s = p.a[row];
            const bool capr = p.cap.row0 <= row && row < p.cap.row1;
            const int64_t crow = row - p.cap.row0;
            if constexpr (EPI == EPI_GLU) {
                const int f = nt * 64 + 32 * wn + r32;
                if (f >= p.seg[0].n) continue;
                const int32_t ag_ = acc[mi][0][e] - rs, au = acc[mi][1][e] - rs;
                float yg = static_cast<float>(ag_) * (p.seg[0].scale * arow_s);
                float yu = static_cast<float>(au) * (p.seg[1].scale * arow_s);
                if (p.seg[0].bias) yg += p.seg[0].bias[f];
                if (p.seg[1].bias) yu += p.seg[1].bias[f];
                const float mv = siluf_(yg) * yu;
                store_act<OUT_BF16>(p.out, row * p.ldo + f, mv);
                if (capr) {
                    if (p.cap.acc) {
                        int32_t *c = p.cap.acc + crow * p.cap.acc_ld;
                        c[p.seg[0].cap_col0 + f] = ag_;
                        c[p.seg[1].cap_col0 + f] = au;
                    }
                    if (p.cap.y_out) p.cap.y_out[crow * p.ldo + f] = OUT_BF16 ? round_to_bf16(mv) : mv;
                }
            } else {
                const Seg &S = p.seg[sg];
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int n = nt * BN + wn * 64 + ni * 32 + r32;
                    if (n >= S.n) continue;
                    const int32_t av_ = acc[mi][ni][e] - rs;
                    float y = static_cast<float>(av_) * (S.scale * arow_s);
                    if (S.bias) y += S.bias[n];
                    const int64_t oi = row * p.ldo + S.out_col0 + n;
                    if constexpr (EPI == EPI_RESID)
                        y = load_act<OUT_BF16>(p.resid, row * p.ldr + S.out_col0 + n) + y;
                    store_act<OUT_BF16>(p.out, oi, y);
                    if (capr) {
                        if (p.cap.acc) p.cap.acc[crow * p.cap.acc_ld + S.cap_col0 + n] = av_;
                        if (p.cap.y_out) p.cap.y_out[crow * p.ldo + S.out_col0 + n] = OUT_BF16 ? round_to_bf16(y) : y;
                    }
                }
            }
        }
    }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &a, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    timing_begin(a.family, s);
    if (a.out_bf16) hipLaunchKernelGGL((gemm_ternary_kernel<EPI, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_ternary_kernel<EPI, false>), grid, block, 0, s, a);
    timing_end(a.family, s);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm(const GemmArgs &a_in, hipStream_t s) {
    if (a_in.M <= 0) return hipSuccess;
    GemmArgs a = a_in;
    a.tiles_n_total = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const int w = a.epi == EPI_GLU ? 64 : BN;
        a.tiles_n[i] = (a.seg[i].n + w - 1) / w;
        if (a.epi == EPI_GLU && i == 1) a.tiles_n[i] = 0;  // up rows ride with the gate tile
        a.tiles_n_total += a.tiles_n[i];
    }
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    const dim3 grid(static_cast<unsigned>(tiles_m * a.tiles_n_total));
    switch (a.epi) {
        case EPI_STORE: return launch_epi<EPI_STORE>(a, grid, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, grid, s);
        default: return launch_epi<EPI_GLU>(a, grid, s);
    }
}

}  // namespace mmf
