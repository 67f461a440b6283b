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
// Tiling (256 threads = 4 waves as 2 (M) x 2 (N); workgroup tile 128 x 256, k-tiles of
// 128; two workgroups per CU so one's epilogue overlaps the other's MFMA loop):
//   - each wave owns 64 x 128 of the output = 2 x 4 MFMA blocks of 32 x 32 (128 int32
//     accumulators per lane).  A (int8, 1 byte per k) costs 4x the LDS bytes of B (2 bits
//     per k), so the wave tile is wide in N;
//   - k-tiles stream from global memory straight into LDS (global_load_lds_dwordx4, no
//     register staging) through a ring of 3 stages, so two tiles are in flight while the
//     third is multiplied; one barrier per k-tile;
//   - the direct loads write each wave's 1 KB in lane order, so bank spreading is done by
//     choosing what each lane fetches: A row r keeps its eight 16-byte chunks in slots
//     permuted by (r ^ r/8) & 7, B row r keeps its two 16-byte halves swapped when
//     (r/4 ^ r/8) is odd; the 16-byte fragment reads of 8 (or 16) consecutive lanes then
//     fall on distinct banks;
//   - lane l (r = l % 32, g = l / 32) feeds MFMA step ks in {0..3} of a k-tile with
//     packed word 4g + ks of weight row r (one word is exactly 16 codes, the B operand)
//     and activation bytes k = 64g + 16ks + [0,16) of row r, so A and B agree on every
//     (lane, byte) -> k pairing.  A ragged last k-tile (K % 128 == 64) zeroes the B
//     operand of the upper lane half;
//   - workgroups are dispatched round-robin over the 8 XCDs; tile ids are remapped so each
//     XCD owns a contiguous run of tiles, walked in groups of 8 M-tiles (N-tile by N-tile,
//     the group's M-tiles side by side): the activation tiles of a group stay in that XCD's
//     L2 while each weight tile is read once per group.
// Epilogues (fused, in registers): y = acc*s_w*a (+bias) stored in fp32/bf16; the same plus
// a residual; or SiLU(gate)*up when the tile pairs 128 gate rows with the same 128 up rows.
#include "mmf_internal.h"

#include <type_traits>


namespace mmf {

namespace {
constexpr int BM = 128, BN = 256, BK = 128;
constexpr int NT = 256;                   // threads
constexpr int STAGES = 3;
constexpr int A_BYTES = BM * BK;          // 16 KB per stage
constexpr int B_BYTES = BN * BK / 4;      // 8 KB per stage
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int A_LOADS = A_BYTES / (NT * 16);  // direct 16-byte loads per thread per stage
constexpr int B_LOADS = B_BYTES / (NT * 16);
constexpr int WN = 2, WM = 4 / WN;  // waves along N and along M
constexpr int MI = BM / 32 / WM, NI = BN / 32 / WN;  // 32 x 32 MFMA blocks per wave
constexpr int EP_PITCH = 36;  // floats per staged epilogue row (32 + 4 pad)
static_assert(A_LOADS == 4 && B_LOADS == 2, "load split");
static_assert(NT / 64 * 32 * EP_PITCH * 4 <= STAGES * STAGE_BYTES, "epilogue staging must fit");

__device__ __forceinline__ int swz_a(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_b(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// Barrier without the memory fence of __syncthreads (whose release semantics would wait for
// every outstanding direct-to-LDS load); ordering of the LDS ring is explicit via vmcnt.
__device__ __forceinline__ void barrier_nofence() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Two packed words -> their 32 codes (two B operands).
__device__ __forceinline__ void unpack_codes_x2(uint32_t w0, uint32_t w1, v4i &c0, v4i &c1) {
    c0 = unpack_codes(w0);
    c1 = unpack_codes(w1);
}

template <int EPI, bool OUT_BF16>
__global__ __launch_bounds__(NT, 2) void gemm_ternary_kernel(GemmArgs p) {
    constexpr bool GLU = EPI == EPI_GLU || EPI == EPI_GLU_KEEP;
    __shared__ __attribute__((aligned(16))) int8_t smem[STAGES * STAGE_BYTES];
    __shared__ int32_t s_rs[BM];  // per-row activation code sum and scale of this tile
    __shared__ float s_a[BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int K = p.K, KW = K / 16;  // words per packed row

    // ---- XCD-aware tile id: XCD x (= blockIdx % 8) owns a contiguous range of tiles, and
    //      tiles run in groups of GM M-tiles: N-tile by N-tile, the GM M-tiles of a group
    //      side by side.  The ~64 tiles an XCD runs at once then share GM activation tiles
    //      (GM x 128 rows, kept in its L2 while the group walks N) and a few weight tiles, so
    //      every weight tile is fetched once per group instead of once per M-tile.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int qx = nwg >> 3, rx = nwg & 7, xcd = bid & 7, idx = bid >> 3;
    const int tile = (xcd < rx ? xcd * (qx + 1) : rx * (qx + 1) + (xcd - rx) * qx) + idx;
    constexpr int GM = 8;
    const int ntn = p.tiles_n_total, n_mt = static_cast<int>((p.M + BM - 1) / BM);
    const int grp = tile / (GM * ntn), in_g = tile % (GM * ntn);
    const int gm = n_mt - grp * GM < GM ? n_mt - grp * GM : GM;   // M-tiles in this group
    const int mt = grp * GM + in_g % gm;
    int nt = in_g / gm;
    int sg = 0;
    while (sg + 1 < p.nseg && nt >= p.tiles_n[sg]) { nt -= p.tiles_n[sg]; ++sg; }
    const int64_t m0 = static_cast<int64_t>(mt) * BM;

    // ---- direct-load sources.  Load i of this thread fills 16-byte LDS slot
    //      s = (wave*L + i)*64 + lane of the stage from a wave-uniform base plus a 32-bit lane
    //      offset fixed for the whole k loop.  Rows beyond M / N are clamped in-bounds (their
    //      outputs are never stored); in a ragged last k-tile the upper half is re-read from
    //      the lower half (in-bounds) and multiplied by zero codes.
    const int8_t *a_base = p.A + m0 * K;
    uint32_t a_off_g[A_LOADS];
    bool a_hi[A_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const int s = (wave * A_LOADS + i) * 64 + lane;
        const int row = s >> 3, c = (s & 7) ^ swz_a(row);
        const int64_t r = m0 + row < p.M ? row : p.M - 1 - m0;
        a_off_g[i] = static_cast<uint32_t>(r * K + 16 * c);
        a_hi[i] = c >= 4;
    }
    const uint32_t *b_base[B_LOADS];
    uint32_t b_off_g[B_LOADS];
    bool b_hi[B_LOADS];
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
        const int s = (wave * B_LOADS + i) * 64 + lane;
        const int row = s >> 1, h = (s & 1) ^ swz_b(row);
        int r;
        if constexpr (GLU) {
            // tile column c: wave wn = c / (32 NI), block ni = (c / 32) % NI, lane j = c % 32;
            // the first NI/2 blocks of a wave are gate rows, the last NI/2 the same up rows;
            // the 32 rows of one load share the block, hence the matrix (gate or up)
            const int blk = wave * B_LOADS + i;
            const int cwn = blk / NI, cni = blk % NI;
            const Seg &S = p.seg[cni / (NI / 2)];
            const int f = nt * 128 + 16 * NI * cwn + 32 * (cni % (NI / 2)) + (row & 31);
            r = f < S.n ? f : S.n - 1;
            b_base[i] = S.packed;
        } else {
            const Seg &S = p.seg[sg];
            const int n = nt * BN + row;
            r = n < S.n ? n : S.n - 1;
            b_base[i] = S.packed;
        }
        b_off_g[i] = static_cast<uint32_t>((r * KW + 4 * h) * 4);
        b_hi[i] = h != 0;
    }
    const int nk = (K + BK - 1) / BK;
    const bool ragged = (K % BK) != 0;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    auto issue = [&](int kt, int st) {
        const uint32_t dst = lds0 + st * STAGE_BYTES;
        const bool cut = ragged && kt == nk - 1;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const uint32_t off = cut && a_hi[i] ? a_off_g[i] - 64 : a_off_g[i];
            dma16(a_base + kt * BK, off, dst + (wave * A_LOADS + i) * 1024);
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const uint32_t off = cut && b_hi[i] ? b_off_g[i] - 16 : b_off_g[i];
            dma16(b_base[i] + kt * (BK / 16), off, dst + A_BYTES + (wave * B_LOADS + i) * 1024);
        }
    };

    // per-row code sums and scales, needed only by the epilogue: requested before the first
    // k-tiles so that the two latencies overlap, written to LDS after the k loop
    // (every thread loads, threads past BM a duplicate row, so there is no branch)
    int32_t rs_t;
    float a_t;
    {
        const int64_t rr = m0 + (tid & (BM - 1));
        const int64_t r = rr < p.M ? rr : p.M - 1;
        rs_t = p.rowsum[r];
        a_t = p.a[r];
    }

    v16i acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

    const int g = lane >> 5, r32 = lane & 31;
    // fragment offsets inside a stage: A row (wm*64 + mi*32 + r32), logical chunk 4g + ks;
    // B row (wn*128 + ni*32 + r32), half g (its swizzle does not depend on ni)
    int a_off[MI][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * (32 * MI) + mi * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a_off[mi][ks] = row * BK + 16 * ((4 * g + ks) ^ swz_a(row));
    }
    const int brow = wn * (32 * NI) + r32;
    const int b_off = A_BYTES + brow * 32 + 16 * (g ^ swz_b(brow));

    // one k-tile: wait for it, free the oldest stage, refill it, multiply.  ST is static so
    // every LDS address is a fixed register plus an immediate.
    auto step = [&](int kt, auto st_c) {
        constexpr int ST = decltype(st_c)::value;
        // tile kt has landed once at most the next tile's loads are outstanding
        if (kt + 1 < nk) wait_vmcnt<A_LOADS + B_LOADS>();
        else wait_vmcnt<0>();
        barrier_nofence();  // every wave's part of tile kt is in LDS; stage kt-1 is free
        if (kt + 2 < nk) issue(kt + 2, (ST + 2) % STAGES);
        const int8_t *sa = smem + ST * STAGE_BYTES;
        // fragment reads in the order of first use (packed B words, then A for k-steps 0-1,
        // then A for k-steps 2-3), so the first MFMAs wait only for the reads they consume
        uint4 bw[NI];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bw[ni] = *reinterpret_cast<const uint4 *>(sa + b_off + ni * 1024);
        v4i av[MI][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) av[mi][ks] = *reinterpret_cast<const v4i *>(sa + a_off[mi][ks]);
        if (ragged && kt == nk - 1 && g) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) bw[ni] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            v4i bv[NI][2];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const uint32_t w0 = half ? bw[ni].z : bw[ni].x, w1 = half ? bw[ni].w : bw[ni].y;
                unpack_codes_x2(w0, w1, bv[ni][0], bv[ni][1]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[mi][2 * half + kk], bv[ni][kk], acc[mi][ni], 0, 0, 0);
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    issue(0, 0);
    if (nk > 1) issue(1, 1);
    for (int kt = 0; kt < nk; kt += 3) {
        step(kt, S0{});
        if (kt + 1 < nk) step(kt + 1, S1{});
        if (kt + 2 < nk) step(kt + 2, S2{});
    }
    if (tid < BM) {
        s_rs[tid] = rs_t;
        s_a[tid] = a_t;
    }
    __syncthreads();  // all waves are done with the ring before it is reused for staging

    // ---- epilogue.  A lane holds C[row][col] for col = r32 of each 32-wide block and rows
    //      8*(e/4) + 4*g + (e%4) of each 32-tall block.  Final fp32 values are computed in
    //      that layout (rescale, bias, SiLU(gate)*up), staged one 32 x 32 block at a time in
    //      LDS (per-wave region, 36-float pitch), and read back as 8 consecutive columns of
    //      one row per lane, so the residual loads and the output stores are 16-byte
    //      accesses covering whole row segments.  The staging region is private to the
    //      wave, so only wave-level ordering is needed.
    float *stg = reinterpret_cast<float *>(smem) + wave * (32 * EP_PITCH);
    constexpr int NOB = GLU ? NI / 2 : NI;  // output blocks per 32-row slab
    // 16-byte accesses need 8-element-aligned row strides and column offsets
    const bool vec_ok = (p.ldo % 8 == 0) && (EPI != EPI_RESID || p.ldr % 8 == 0) &&
                        (GLU || p.seg[sg].out_col0 % 8 == 0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        // residuals of this 32-row slab (bf16: all its blocks; fp32: loaded per block), issued
        // before the values are computed so that their latency overlaps the rescale
        constexpr int RB = EPI == EPI_RESID ? (OUT_BF16 ? NI : 1) : 1;
        uint4 rvb[RB][2][OUT_BF16 ? 1 : 2];
        auto load_resid = [&](int ob, uint4 (&dst)[2][OUT_BF16 ? 1 : 2]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rr = (lane >> 2) + 16 * i, cc = 8 * (lane & 3);
                const int64_t row = m0 + wm * (32 * MI) + mi * 32 + rr;
                const int col = nt * BN + wn * (32 * NI) + ob * 32 + cc;
                if (row < p.M && vec_ok && col + 8 <= p.seg[sg].n) {
                    const int64_t ri = row * p.ldr + p.seg[sg].out_col0 + col;
                    if constexpr (OUT_BF16) {
                        dst[i][0] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.resid) + ri);
                    } else {
                        dst[i][0] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p.resid) + ri);
                        dst[i][OUT_BF16 ? 0 : 1] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p.resid) + ri + 4);
                    }
                }
            }
        };
        if constexpr (EPI == EPI_RESID && OUT_BF16) {
#pragma unroll
            for (int ob = 0; ob < NI; ++ob) load_resid(ob, rvb[ob]);
        }
        int32_t rs_e[16];
        float a_e[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int lr = wm * (32 * MI) + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            rs_e[e] = s_rs[lr];
            a_e[e] = s_a[lr];
        }
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) {
            // global column of this lane's value and of the block's first column
            int col0;
            if constexpr (GLU) {
                col0 = nt * 128 + 16 * NI * wn + 32 * ob;
            } else {
                col0 = nt * BN + wn * (32 * NI) + ob * 32;
            }
            const int col_lane = col0 + r32;
            const Seg &S = p.seg[GLU ? 0 : sg];
            const int ncols = S.n;
            if constexpr (EPI == EPI_RESID && !OUT_BF16) load_resid(ob, rvb[0]);
            float v[16];
            if constexpr (GLU) {
                const float sg0 = p.seg[0].scale, su = p.seg[1].scale;
                const float bg = p.seg[0].bias && col_lane < ncols ? p.seg[0].bias[col_lane] : 0.0f;
                const float bu = p.seg[1].bias && col_lane < ncols ? p.seg[1].bias[col_lane] : 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int32_t ag_ = acc[mi][ob][e] - rs_e[e], au = acc[mi][ob + NI / 2][e] - rs_e[e];
                    const float yg = static_cast<float>(ag_) * (sg0 * a_e[e]) + bg;
                    const float yu = static_cast<float>(au) * (su * a_e[e]) + bu;
                    v[e] = siluf_(yg) * yu;
                    if constexpr (EPI == EPI_GLU_KEEP) {
                        const int64_t row = m0 + wm * (32 * MI) + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                        if (row < p.M && col_lane < ncols) {
                            p.keep[row * 2 * ncols + col_lane] = f32_to_bf16_bits(yg);
                            p.keep[row * 2 * ncols + ncols + col_lane] = f32_to_bf16_bits(yu);
                        }
                    }
                }
            } else {
                const float bb = S.bias && col_lane < ncols ? S.bias[col_lane] : 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int32_t av_ = acc[mi][ob][e] - rs_e[e];
                    v[e] = static_cast<float>(av_) * (S.scale * a_e[e]) + bb;
                }
            }
            if (p.cap.acc) {  // integer accumulators of captured rows (rare; test protocol)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * (32 * MI) + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                    if (row < p.M && col_lane < ncols && p.cap.row0 <= row && row < p.cap.row1) {
                        int32_t *c = p.cap.acc + (row - p.cap.row0) * p.cap.acc_ld;
                        if constexpr (GLU) {
                            c[p.seg[0].cap_col0 + col_lane] = acc[mi][ob][e] - rs_e[e];
                            c[p.seg[1].cap_col0 + col_lane] = acc[mi][ob + NI / 2][e] - rs_e[e];
                        } else {
                            c[S.cap_col0 + col_lane] = acc[mi][ob][e] - rs_e[e];
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) stg[(8 * (e >> 2) + 4 * g + (e & 3)) * EP_PITCH + r32] = v[e];
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
            // lane l: rows l/4 and l/4 + 16 of the block, columns 8*(l%4) .. +7
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rr = (lane >> 2) + 16 * i, cc = 8 * (lane & 3);
                const int64_t row = m0 + wm * (32 * MI) + mi * 32 + rr;
                const int col = col0 + cc;  // column inside the segment
                const float4 lo = *reinterpret_cast<const float4 *>(stg + rr * EP_PITCH + cc);
                const float4 hi = *reinterpret_cast<const float4 *>(stg + rr * EP_PITCH + cc + 4);
                float o[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                if (row >= p.M || col >= ncols) continue;
                const int ocol = (GLU ? 0 : S.out_col0) + col;
                const bool full = vec_ok && col + 8 <= ncols;
                if constexpr (EPI == EPI_RESID) {
                    const int64_t ri = row * p.ldr + ocol;
                    if (full) {
                        if constexpr (OUT_BF16) {
                            const uint4 u = rvb[ob][i][0];
                            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                o[2 * j] += __uint_as_float(w[j] << 16);
                                o[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
                            }
                        } else {
                            const float4 r0 = __builtin_bit_cast(float4, rvb[0][i][0]);
                            const float4 r1 = __builtin_bit_cast(float4, rvb[0][i][OUT_BF16 ? 0 : 1]);
                            o[0] += r0.x; o[1] += r0.y; o[2] += r0.z; o[3] += r0.w;
                            o[4] += r1.x; o[5] += r1.y; o[6] += r1.z; o[7] += r1.w;
                        }
                    } else {
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
                    if (full) {
                        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + oi) = make_uint4(w[0], w[1], w[2], w[3]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (col + j < ncols)
                                static_cast<uint16_t *>(p.out)[oi + j] = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {  // the stored (rounded) values, for the capture
                        o[2 * j] = __uint_as_float(w[j] << 16);
                        o[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
                    }
                } else {
                    if (full) {
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
            __builtin_amdgcn_wave_barrier();
            asm volatile("" ::: "memory");
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
    const bool glu = a.epi == EPI_GLU || a.epi == EPI_GLU_KEEP;
    for (int i = 0; i < a.nseg; ++i) {
        const int w = glu ? 128 : BN;
        a.tiles_n[i] = (a.seg[i].n + w - 1) / w;
        if (glu && i == 1) a.tiles_n[i] = 0;  // up rows ride with the gate tile
        a.tiles_n_total += a.tiles_n[i];
    }
    const int64_t tiles_m = (a.M + BM - 1) / BM;
    const dim3 grid(static_cast<unsigned>(tiles_m * a.tiles_n_total));
    switch (a.epi) {
        case EPI_STORE: return launch_epi<EPI_STORE>(a, grid, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, grid, s);
        case EPI_GLU_KEEP: return launch_epi<EPI_GLU_KEEP>(a, grid, s);
        default: return launch_epi<EPI_GLU>(a, grid, s);
    }
}

}  // namespace mmf
