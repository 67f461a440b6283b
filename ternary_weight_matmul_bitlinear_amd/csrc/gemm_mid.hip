// gemm_mid.hip -- BitLinear for a few dozen token rows (up to 64): int8 MFMA against ternary
// weights that are streamed from HBM exactly once, with the k range split over the waves of
// a workgroup.
//
// DataCamp "MatMul-free language models", section "Replacing MatMul with ternary
// operations": with weights in {-1,0,1} the layer output is an exact signed integer sum of
// int8 activations; the packed codes c = q + 1 are multiplied on the matrix cores and the
// offset is removed once per row, acc = sum_k q_x*c - sum_k q_x (exact in int32).
//
// Between one-token decode and thousands of prefill tokens: with tens of rows every weight
// is still read once (the weights dominate the traffic), but the dot4 decode kernel spends
// one VALU lane-op per 4 codes per token and becomes ALU-bound, while the prefill tiles
// (128 rows) leave most workgroups idle.  Here:
//   - one 256-thread workgroup owns 32 weight rows (for the GLU, 32 gate rows and the 32 up
//     rows of the same features) and all M <= 64 token rows as one or two 32-row MFMA
//     blocks (MB = 1 up to 32 rows);
//   - its four waves take interleaved k-tiles of 128 (kt = wave, wave + 4, ...), so the
//     four waves together read whole 128-byte lines of every weight row;
//   - lane l (r = l % 32, g = l / 32) holds, per k-tile, the 16-byte packed piece (words
//     4g..4g+3) of weight row r: word 4g + ks is exactly the 16-code B operand of MFMA step
//     ks, paired with activation bytes 64g + 16ks + [0,16) of token row r.  All weight
//     pieces of a wave are requested at kernel entry;
//   - every workgroup reads all M x K activations (L2 resident), so their fetch sets the
//     time: they are loaded as whole 128-byte row segments (8 lanes per row, up to four
//     k-tiles ahead) and moved into the MFMA layout through a wave-private LDS buffer.  The
//     MFMA layout fetched directly (32 rows per load, 16 bytes each) costs one cache-line
//     access per lane and ran at about 30 GB/s per CU;
//   - the four partial accumulators are summed through LDS and the fused epilogue (rescale,
//     bias, residual, or SiLU(gate)*up) stores 8 consecutive outputs of one row per thread.
// KTW (k-tiles per wave) is a template parameter so every load is unconditional: k-tiles
// past the end re-read the last tile with zero weight codes.
#include "mmf_internal.h"

namespace mmf {

namespace {

constexpr int MID_NT = 256;
constexpr int MID_KT = 128;  // k per tile

// Keeps the compiler from moving LDS accesses of this wave across the point (the hardware
// completes one wave's LDS instructions in issue order, so program order is enough).
__device__ __forceinline__ void lds_order() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

template <int EPI, bool OUT_BF16, int KTW, int MB>
__global__ __launch_bounds__(MID_NT) void gemm_mid_kernel(GemmArgs p) {
    constexpr int NB = EPI == EPI_GLU ? 2 : 1;  // 32-row weight blocks per workgroup
    // MB: 32-row token blocks (M <= 32 * MB)
    constexpr int PITCH = NB * 32 + 4;         // int32 per LDS row of a partial tile
    // the k loop stages activation tiles in LDS (two buffers of MB * 4 KB per wave); the
    // partial tiles of the reduction reuse the same memory afterwards
    constexpr int STG_BYTES = 4 * 2 * MB * 32 * MID_KT;
    constexpr int RED_BYTES = 4 * MB * 32 * PITCH * 4;
    __shared__ __attribute__((aligned(16))) int8_t lds[STG_BYTES > RED_BYTES ? STG_BYTES : RED_BYTES];
    auto red = reinterpret_cast<int32_t (*)[MB * 32][PITCH]>(lds);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, g = lane >> 5;
    const int K = p.K, KW = K / 16;
    const int nk = (K + MID_KT - 1) / MID_KT;
    const bool ragged = (K % MID_KT) != 0;

    // ---- this workgroup's weight rows: block nb of segment sg starting at row n0
    int blk = blockIdx.x, sg = 0;
    if constexpr (EPI != EPI_GLU) {
        while (sg + 1 < p.nseg && blk >= p.tiles_n[sg]) { blk -= p.tiles_n[sg]; ++sg; }
    }
    const int n0 = blk * 32;
    const uint32_t *wrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const Seg &S = p.seg[EPI == EPI_GLU ? nb : sg];
        const int n = n0 + r32 < S.n ? n0 + r32 : S.n - 1;  // clamped rows are never stored
        wrow[nb] = S.packed + static_cast<int64_t>(n) * KW;
    }

    // ---- activation tiles (MB*32 rows x 128 bytes) are fetched with whole 128-byte row
    //      segments per 8 lanes: load j of lane l reads token row 8j + l/8, 16-byte chunk
    //      (l%8) ^ (row%8), and stores it to LDS slot 16l of the wave's buffer, i.e. chunk c
    //      of row r sits at r*128 + 16*(c ^ r%8), so the fragment reads of 8 consecutive rows
    //      (same chunk) hit 8 different bank groups.  Rows past M re-read row M-1 (never
    //      stored); the upper half of a ragged last tile re-reads the lower half (in bounds,
    //      multiplied by zero codes).
    constexpr int AL = MB * 32 / 8;  // 16-byte loads per lane per activation tile
    uint32_t a_goff[AL];             // byte offset of this lane's chunk inside a k-tile
    int a_chunk[AL];
#pragma unroll
    for (int j = 0; j < AL; ++j) {
        const int row = 8 * j + (lane >> 3), c = (lane & 7) ^ (row & 7);
        const int64_t m = row < p.M ? row : p.M - 1;
        a_goff[j] = static_cast<uint32_t>(m * K + 16 * c);
        a_chunk[j] = c;
    }
    auto tile_of = [&](int i) __attribute__((always_inline)) {
        const int kt0 = wave + 4 * i;
        return kt0 < nk ? kt0 : nk - 1;
    };
    // packed weights: all pieces of this wave requested up front
    uint4 bw[KTW][NB];
    auto load_b = [&](int i) __attribute__((always_inline)) {
        const int kt = tile_of(i);
        const int word = kt * 8 + (ragged && kt == nk - 1 ? 0 : 4 * g);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bw[i][nb] = *reinterpret_cast<const uint4 *>(wrow[nb] + word);
    };
    // raw activation tiles run PD k-tiles ahead of the MFMAs
    constexpr int PD = KTW < 4 ? KTW : 4;
    v4i araw[PD][AL];  // vector type (a struct copy of uint4 would keep the array in scratch)
    auto load_a = [&](int i, v4i (&dst)[AL]) __attribute__((always_inline)) {
        const int kt = tile_of(i);
        const bool cut = ragged && kt == nk - 1;
        const int8_t *base = p.A + static_cast<int64_t>(kt) * MID_KT;
#pragma unroll
        for (int j = 0; j < AL; ++j)
            dst[j] = *reinterpret_cast<const v4i *>(base + (cut && a_chunk[j] >= 4 ? a_goff[j] - 64 : a_goff[j]));
    };
    int8_t *stg = lds + wave * (2 * MB * 32 * MID_KT);
    auto put_a = [&](int buf, const v4i (&src)[AL]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < AL; ++j)
            *reinterpret_cast<v4i *>(stg + buf * (MB * 32 * MID_KT) + j * 1024 + 16 * lane) = src[j];
    };
    // MFMA fragment of step ks: token row mb*32 + r32, bytes 64g + 16ks + [0,16) of the tile
    int f_off[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int row = mb * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) f_off[mb][ks] = row * MID_KT + 16 * ((4 * g + ks) ^ (row & 7));
    }
    auto get_a = [&](int buf, v4i (&dst)[MB][4]) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                dst[mb][ks] = *reinterpret_cast<const v4i *>(stg + buf * (MB * 32 * MID_KT) + f_off[mb][ks]);
    };

    v16i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0;

    load_a(0, araw[0]);
#pragma unroll
    for (int i = 0; i < KTW; ++i) load_b(i);
#pragma unroll
    for (int i = 1; i < PD; ++i) load_a(i, araw[i]);
    // epilogue operands of this thread (token row tid/4, columns 8*(tid%4) .. +7 of the
    // block), requested with the prologue so that their latency is not paid after the k loop
    const int e_row = (tid >> 2) < p.M ? (tid >> 2) : static_cast<int>(p.M) - 1;
    const Seg &S = p.seg[EPI == EPI_GLU ? 0 : sg];
    const int col = n0 + 8 * (tid & 3);  // first column (feature) inside the segment
    const int ocol = (EPI == EPI_GLU ? 0 : S.out_col0) + col;
    const bool vec = col + 8 <= S.n && (p.ldo % 8 == 0) && (ocol % 8 == 0) && (EPI != EPI_RESID || p.ldr % 8 == 0);
    const int32_t rs = p.rowsum[e_row];
    const float a = p.a[e_row];
    v4i rv[OUT_BF16 ? 1 : 2] = {};
    if constexpr (EPI == EPI_RESID) {
        if (vec) {
            const int64_t ri = static_cast<int64_t>(e_row) * p.ldr + ocol;
            if constexpr (OUT_BF16) {
                rv[0] = *reinterpret_cast<const v4i *>(static_cast<const uint16_t *>(p.resid) + ri);
            } else {
                rv[0] = *reinterpret_cast<const v4i *>(static_cast<const float *>(p.resid) + ri);
                rv[OUT_BF16 ? 0 : 1] = *reinterpret_cast<const v4i *>(static_cast<const float *>(p.resid) + ri + 4);
            }
        }
    }
    // keep every load above issued here: the scheduler would otherwise sink them next to
    // their first use and serialize the memory latency
    __builtin_amdgcn_sched_barrier(0);
    // LDS accesses of one wave complete in order, so its own buffers need no barrier
    put_a(0, araw[0]);
    if (PD < KTW) load_a(PD, araw[0]);
    lds_order();
    v4i av[2][MB][4];
    get_a(0, av[0]);
#pragma unroll
    for (int i = 0; i < KTW; ++i) {
        // the next tile goes to the other buffer and its fragments are read before this
        // tile's MFMAs, so the LDS latency hides behind them
        if (i + 1 < KTW) {
            lds_order();  // after the reads of the buffer's previous tile
            put_a((i + 1) & 1, araw[(i + 1) % PD]);
            if (i + 1 + PD < KTW) load_a(i + 1 + PD, araw[(i + 1) % PD]);
            lds_order();
            get_a((i + 1) & 1, av[(i + 1) & 1]);
        }
        const int kt0 = wave + 4 * i;
        // code mask: zero for tiles past the end and for the upper half of a ragged last tile
        const bool live = kt0 < nk && !(ragged && kt0 == nk - 1 && g);
        const uint32_t msk = live ? 0x03030303u : 0u;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t w[4] = {bw[i][nb].x, bw[i][nb].y, bw[i][nb].z, bw[i][nb].w};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const v4i b = v4i{static_cast<int>(w[ks] & msk), static_cast<int>((w[ks] >> 2) & msk),
                                  static_cast<int>((w[ks] >> 4) & msk), static_cast<int>((w[ks] >> 6) & msk)};
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[i & 1][mb][ks], b, acc[mb][nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // every wave is done with its staging buffers before they hold partials

    // ---- sum the four waves' partial tiles.  Lane l holds C[row][col] for col = nb*32 + l%32
    //      and rows mb*32 + 8*(e/4) + 4*g + (e%4).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                red[wave][mb * 32 + 8 * (e >> 2) + 4 * g + (e & 3)][nb * 32 + r32] = acc[mb][nb][e];
    __syncthreads();

    // ---- epilogue: thread -> row tid/4, columns 8*(tid%4) .. +7 of the 32-column block
    const int row_l = tid >> 2, c8 = 8 * (tid & 3);
    const int64_t row = row_l;  // equal to e_row from here on
    if (row_l >= MB * 32 || row >= p.M) return;
    int32_t v[NB][8];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[nb][j] = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int4 lo = *reinterpret_cast<const int4 *>(&red[w][row_l][nb * 32 + c8]);
            const int4 hi = *reinterpret_cast<const int4 *>(&red[w][row_l][nb * 32 + c8 + 4]);
            v[nb][0] += lo.x; v[nb][1] += lo.y; v[nb][2] += lo.z; v[nb][3] += lo.w;
            v[nb][4] += hi.x; v[nb][5] += hi.y; v[nb][6] += hi.z; v[nb][7] += hi.w;
        }
    }
    const int ncols = S.n;
    if (col >= ncols) return;
    float o[8];
    if constexpr (EPI == EPI_GLU) {
        const float sa_g = p.seg[0].scale * a, sa_u = p.seg[1].scale * a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cj = col + j < ncols ? col + j : ncols - 1;
            const float bg = p.seg[0].bias ? p.seg[0].bias[cj] : 0.0f;
            const float bu = p.seg[1].bias ? p.seg[1].bias[cj] : 0.0f;
            const float yg = static_cast<float>(v[0][j] - rs) * sa_g + bg;
            const float yu = static_cast<float>(v[1][j] - rs) * sa_u + bu;
            o[j] = siluf_(yg) * yu;
        }
    } else {
        const float sa = S.scale * a;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cj = col + j < ncols ? col + j : ncols - 1;
            const float bb = S.bias ? S.bias[cj] : 0.0f;
            o[j] = static_cast<float>(v[0][j] - rs) * sa + bb;
        }
    }
    if (p.cap.acc && p.cap.row0 <= row && row < p.cap.row1) {  // test protocol (rare)
        int32_t *c = p.cap.acc + (row - p.cap.row0) * p.cap.acc_ld;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (col + j >= ncols) continue;
            if constexpr (EPI == EPI_GLU) {
                c[p.seg[0].cap_col0 + col + j] = v[0][j] - rs;
                c[p.seg[1].cap_col0 + col + j] = v[1][j] - rs;
            } else {
                c[S.cap_col0 + col + j] = v[0][j] - rs;
            }
        }
    }
    if constexpr (EPI == EPI_RESID) {
        if (vec) {
            if constexpr (OUT_BF16) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = static_cast<uint32_t>(rv[0][j]);
                    o[2 * j] += __uint_as_float(w << 16);
                    o[2 * j + 1] += __uint_as_float(w & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[j] += __int_as_float(rv[0][j]);
                    o[4 + j] += __int_as_float(rv[OUT_BF16 ? 0 : 1][j]);
                }
            }
        } else {
            const int64_t ri = row * p.ldr + ocol;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < ncols) o[j] += load_act<OUT_BF16>(p.resid, ri + j);
        }
    }
    const int64_t oi = row * p.ldo + ocol;
    if constexpr (OUT_BF16) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(o[2 * j], o[2 * j + 1]);
        if (vec) {
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + oi) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < ncols) static_cast<uint16_t *>(p.out)[oi + j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // the stored (rounded) values, for the capture
            o[2 * j] = __uint_as_float(w[j] << 16);
            o[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        if (vec) {
            *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + oi) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + oi + 4) = make_float4(o[4], o[5], o[6], o[7]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (col + j < ncols) static_cast<float *>(p.out)[oi + j] = o[j];
        }
    }
    if (p.cap.y_out && p.cap.row0 <= row && row < p.cap.row1) {
        float *cy = p.cap.y_out + (row - p.cap.row0) * p.ldo + ocol;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (col + j < ncols) cy[j] = o[j];
    }
}

template <int EPI, bool OUT_BF16, int MB>
bool launch_ktw(const GemmArgs &a, dim3 grid, hipStream_t s) {
    const int nk = (a.K + MID_KT - 1) / MID_KT;
    const int ktw = (nk + 3) / 4;
    if (ktw <= 2) hipLaunchKernelGGL((gemm_mid_kernel<EPI, OUT_BF16, 2, MB>), grid, dim3(MID_NT), 0, s, a);
    else if (ktw <= 4) hipLaunchKernelGGL((gemm_mid_kernel<EPI, OUT_BF16, 4, MB>), grid, dim3(MID_NT), 0, s, a);
    else if (ktw <= 8) hipLaunchKernelGGL((gemm_mid_kernel<EPI, OUT_BF16, 8, MB>), grid, dim3(MID_NT), 0, s, a);
    else if constexpr (EPI != EPI_GLU) {  // (the GLU's two weight blocks would not fit)
        if (ktw <= 12) hipLaunchKernelGGL((gemm_mid_kernel<EPI, OUT_BF16, 12, MB>), grid, dim3(MID_NT), 0, s, a);
        else if (ktw <= 16) hipLaunchKernelGGL((gemm_mid_kernel<EPI, OUT_BF16, 16, MB>), grid, dim3(MID_NT), 0, s, a);
        else return false;
    } else {
        return false;
    }
    return true;
}

template <int EPI, bool OUT_BF16>
bool launch_mb(const GemmArgs &a, dim3 grid, hipStream_t s) {
    return a.M <= 32 ? launch_ktw<EPI, OUT_BF16, 1>(a, grid, s) : launch_ktw<EPI, OUT_BF16, 2>(a, grid, s);
}

template <int EPI>
bool launch_mid_epi(const GemmArgs &a, dim3 grid, hipStream_t s) {
    return a.out_bf16 ? launch_mb<EPI, true>(a, grid, s) : launch_mb<EPI, false>(a, grid, s);
}
}  // namespace

bool mid_gemm_supported(const GemmArgs &a) {
    const int nk = (a.K + MID_KT - 1) / MID_KT;
    const int ktw = (nk + 3) / 4;
    return a.M >= 1 && a.M <= kMidMaxM && (ktw <= 8 || (ktw <= 16 && a.epi != EPI_GLU));
}

hipError_t launch_gemm_mid(const GemmArgs &a_in, hipStream_t s) {
    if (a_in.M <= 0) return hipSuccess;
    GemmArgs a = a_in;
    a.tiles_n_total = 0;
    for (int i = 0; i < a.nseg; ++i) {
        a.tiles_n[i] = (a.seg[i].n + 31) / 32;
        if (a.epi == EPI_GLU && i == 1) a.tiles_n[i] = 0;  // up rows ride with the gate block
        a.tiles_n_total += a.tiles_n[i];
    }
    const dim3 grid(static_cast<unsigned>(a.tiles_n_total));
    timing_begin(a.family, s);
    bool ok;
    switch (a.epi) {
        case EPI_STORE: ok = launch_mid_epi<EPI_STORE>(a, grid, s); break;
        case EPI_RESID: ok = launch_mid_epi<EPI_RESID>(a, grid, s); break;
        default: ok = launch_mid_epi<EPI_GLU>(a, grid, s); break;
    }
    timing_end(a.family, s);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace mmf
