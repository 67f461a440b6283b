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
// Tiling (256 threads = 4 waves as 2 (M) x 2 (N); workgroup tile 128 x 256 x 64; two
// workgroups per CU so one's epilogue overlaps the other's MFMA loop):
//   - each wave owns 64 x 128 of the output = 2 x 4 MFMA blocks of 32 x 32 (128 int32
//     accumulators per lane).  A (int8, 1 byte per k) costs 4x the LDS bytes of B (2 bits
//     per k), so the wave tile is wide in N: 384 LDS bytes per 64K-op MFMA;
//   - A tile 128 rows x 64 k in LDS with an 80-byte row pitch (16-byte reads of 8
//     consecutive rows hit disjoint bank quads); B tile 256 rows x 4 packed words with a
//     24-byte pitch (conflict-free 8-byte reads).  One packed word is exactly the 16-code
//     B operand of a lane, so weights travel at 2 bits each all the way to the registers;
//   - lane l (r = l % 32, g = l / 32) feeds, for MFMA half ks in {0,1}, activation bytes
//     k = 32g + 16ks + [0,16) of row r and packed word 2g + ks of weight row r, so A and B
//     agree on every (lane group, byte) -> k pairing;
//   - double-buffered LDS, next k-tile prefetched into registers during the MFMAs;
//   - workgroups are dispatched round-robin over the 8 XCDs; tile ids are remapped so each
//     XCD owns a contiguous run of tiles (N fastest), i.e. a few M-tiles of activations and
//     all weight tiles, which stay in that XCD's L2.
// Epilogues (fused, in registers): y = acc*s_w*a (+bias) stored in fp32/bf16; the same plus
// a residual; or SiLU(gate)*up when the tile pairs 128 gate rows with the same 128 up rows.
#include "mmf_internal.h"

namespace mmf {

namespace {
constexpr int BM = 128, BN = 256, BK = 64;
constexpr int NT = 256;      // threads
constexpr int A_PITCH = 80;  // bytes
constexpr int B_PITCH = 24;  // bytes
constexpr int MI = 2, NI = 4;
constexpr int EP_PITCH = 36;  // floats per staged epilogue row (32 + 4 pad)
static_assert(NT / 64 * 32 * EP_PITCH * 4 <= 2 * BM * A_PITCH, "epilogue staging must fit in the A tiles");

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NT, 2) void gemm_ternary_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) int8_t smA[2][BM * A_PITCH];
    __shared__ __attribute__((aligned(16))) int8_t smB[2][BN * B_PITCH];
    __shared__ int32_t s_rs[BM];  // per-row activation code sum and scale of this tile
    __shared__ float s_a[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int K = p.K, KW = K / 16;  // words per packed row

    // ---- XCD-aware tile id: XCD x (= blockIdx % 8) owns a contiguous range of tiles
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int qx = nwg >> 3, rx = nwg & 7, xcd = bid & 7, idx = bid >> 3;
    const int tile = (xcd < rx ? xcd * (qx + 1) : rx * (qx + 1) + (xcd - rx) * qx) + idx;
    const int mt = tile / p.tiles_n_total;
    int nt = tile % p.tiles_n_total;
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
            // tile column c: wave half wn = c / 128, block ni = (c % 128) / 32, lane j = c % 32
            const int c = tid, cwn = c >> 7, cni = (c & 127) >> 5;
            const int sub = cni >> 1;  // 0: gate, 1: up
            const int f = nt * 128 + 64 * cwn + 32 * (cni & 1) + (c & 31);
            const Seg &S = p.seg[sub];
            bptr = S.packed + static_cast<int64_t>(f < S.n ? f : S.n - 1) * KW;
        } else {
            const Seg &S = p.seg[sg];
            const int n = nt * BN + tid;
            bptr = S.packed + static_cast<int64_t>(n < S.n ? n : S.n - 1) * KW;
        }
    }

    if (tid < BM) {
        const int64_t r = m0 + tid < p.M ? m0 + tid : p.M - 1;
        s_rs[tid] = p.rowsum[r];
        s_a[tid] = p.a[r];
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

    v16i acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
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
        v4i av[MI][2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int8_t *pa = smA[cur] + (wm * 64 + mi * 32 + r32) * A_PITCH + g * 32;
            av[mi][0] = *reinterpret_cast<const v4i *>(pa);
            av[mi][1] = *reinterpret_cast<const v4i *>(pa + 16);
        }
        uint2 bw[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            bw[ni] = *reinterpret_cast<const uint2 *>(smB[cur] + (wn * 128 + ni * 32 + r32) * B_PITCH + g * 8);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const v4i bv = unpack_codes(ks ? bw[ni].y : bw[ni].x);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][ks], bv, acc[mi][ni], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  A lane holds C[row][col] for col = r32 of each 32-wide block and rows
    //      8*(e/4) + 4*g + (e%4) of each 32-tall block.  Final fp32 values are computed in
    //      that layout (rescale, bias, SiLU(gate)*up), staged one 32 x 32 block at a time in
    //      LDS (per-wave region, 36-float pitch), and read back as 8 consecutive columns of
    //      one row per lane, so the residual loads and the output stores are 16-byte
    //      accesses covering whole row segments.
    float *stg = reinterpret_cast<float *>(&smA[0][0]) + wave * (32 * EP_PITCH);
    constexpr int NOB = EPI == EPI_GLU ? 2 : NI;  // output blocks per 32-row slab
    // 16-byte accesses need 8-element-aligned row strides and column offsets
    const bool vec_ok = (p.ldo % 8 == 0) && (EPI != EPI_RESID || p.ldr % 8 == 0) &&
                        (EPI == EPI_GLU || p.seg[sg].out_col0 % 8 == 0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        int32_t rs_e[16];
        float a_e[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int lr = wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            rs_e[e] = s_rs[lr];
            a_e[e] = s_a[lr];
        }
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) {
            // global column of this lane's value and of the block's first column
            int col_lane, col0;
            if constexpr (EPI == EPI_GLU) {
                col0 = nt * 128 + 64 * wn + 32 * ob;
            } else {
                col0 = nt * BN + wn * 128 + ob * 32;
            }
            col_lane = col0 + r32;
            const Seg &S = p.seg[EPI == EPI_GLU ? 0 : sg];
            const int ncols = S.n;
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if constexpr (EPI == EPI_GLU) {
                    const int32_t ag_ = acc[mi][ob][e] - rs_e[e], au = acc[mi][ob + 2][e] - rs_e[e];
                    float yg = static_cast<float>(ag_) * (p.seg[0].scale * a_e[e]);
                    float yu = static_cast<float>(au) * (p.seg[1].scale * a_e[e]);
                    if (p.seg[0].bias && col_lane < ncols) yg += p.seg[0].bias[col_lane];
                    if (p.seg[1].bias && col_lane < ncols) yu += p.seg[1].bias[col_lane];
                    v[e] = siluf_(yg) * yu;
                } else {
                    const int32_t av_ = acc[mi][ob][e] - rs_e[e];
                    v[e] = static_cast<float>(av_) * (S.scale * a_e[e]);
                    if (S.bias && col_lane < ncols) v[e] += S.bias[col_lane];
                }
            }
            if (p.cap.acc) {  // integer accumulators of captured rows (rare; test protocol)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 64 + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    if (row < p.M && col_lane < ncols && p.cap.row0 <= row && row < p.cap.row1) {
                        int32_t *c = p.cap.acc + (row - p.cap.row0) * p.cap.acc_ld;
                        if constexpr (EPI == EPI_GLU) {
                            c[p.seg[0].cap_col0 + col_lane] = acc[mi][ob][e] - rs_e[e];
                            c[p.seg[1].cap_col0 + col_lane] = acc[mi][ob + 2][e] - rs_e[e];
                        } else {
                            c[S.cap_col0 + col_lane] = acc[mi][ob][e] - rs_e[e];
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) stg[(8 * (e >> 2) + 4 * g + (e & 3)) * EP_PITCH + r32] = v[e];
            __syncthreads();
            // lane l: rows l/4 and l/4 + 16 of the block, columns 8*(l%4) .. +7
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rr = (lane >> 2) + 16 * i, cc = 8 * (lane & 3);
                const int64_t row = m0 + wm * 64 + mi * 32 + rr;
                const int col = col0 + cc;  // column inside the segment
                const float4 lo = *reinterpret_cast<const float4 *>(stg + rr * EP_PITCH + cc);
                const float4 hi = *reinterpret_cast<const float4 *>(stg + rr * EP_PITCH + cc + 4);
                float o[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                if (row >= p.M || col >= ncols) continue;
                const int ocol = (EPI == EPI_GLU ? 0 : S.out_col0) + col;
                const bool full = vec_ok && col + 8 <= ncols;
                if constexpr (EPI == EPI_RESID) {
                    const int64_t ri = row * p.ldr + ocol;
                    if (full) {
                        if constexpr (OUT_BF16) {
                            const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.resid) + ri);
                            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                o[2 * j] += __uint_as_float(w[j] << 16);
                                o[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
                            }
                        } else {
                            const float4 r0 = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.resid) + ri);
                            const float4 r1 = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.resid) + ri + 4);
                            o[0] += r0.x; o[1] += r0.y; o[2] += r0.z; o[3] += r0.w;
                            o[4] += r1.x; o[5] += r1.y; o[6] += r1.z; o[7] += r1.w;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (col + j < ncols) o[j] += load_act<OUT_BF16>(p.resid, ri + j);
                    }
                }
                if constexpr (OUT_BF16) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) o[j] = round_to_bf16(o[j]);
                }
                const int64_t oi = row * p.ldo + ocol;
                if (full) {
                    if constexpr (OUT_BF16) {
                        uint32_t w[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            w[j] = (__float_as_uint(o[2 * j]) >> 16) | (__float_as_uint(o[2 * j + 1]) & 0xFFFF0000u);
                        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + oi) = make_uint4(w[0], w[1], w[2], w[3]);
                    } else {
                        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
                        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + oi + 4) = make_float4(o[4], o[5], o[6], o[7]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (col + j < ncols) store_act<OUT_BF16>(p.out, oi + j, o[j]);
                }
                if (p.cap.y_out && p.cap.row0 <= row && row < p.cap.row1) {
                    float *cy = p.cap.y_out + (row - p.cap.row0) * p.ldo + ocol;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (col + j < ncols) cy[j] = o[j];
                }
            }
            __syncthreads();
        }
    }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &a, dim3 grid, hipStream_t s) {
    const dim3 block(NT);
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
        const int w = a.epi == EPI_GLU ? 128 : BN;
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
