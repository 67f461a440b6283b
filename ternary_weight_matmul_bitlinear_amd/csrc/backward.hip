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
//   phase 3 (workgroup per 64 channels, runs of chunks folded and composed): carry G
//     backwards across chunks; dh0 = f_0 G_0;
//   phase 4 (as phase 2): walk the chunk backwards with the carried G:
//     di = (1-f) G silu'(i), df_pre = (h_{t-1} - c) G (1-lb) sigma'(z).
// Per-chunk partial sums of dgnorm_w and df_bias are reduced by a column-sum kernel.
#include "mmf_internal.h"

#include <type_traits>

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
// The contraction may be cut into segments of seg_steps steps with a scale of their own (the
// weight scales of linears that share an input, stacked along t): the accumulators are
// multiplied by seg_ratio[j] = scale_j / scale_(j+1) when segment j + 1 begins, and by
// `scale` (the last segment's) at the end.  The output rows may be cut into up to three
// matrices of c_rows rows each (C, C1, C2; a NULL one is not written).
struct NtGemmArgs {
    const void *A;
    int32_t a_bf16;
    const uint16_t *B;
    int64_t R;
    int32_t S;
    int64_t T;              // contraction length
    int64_t lda, ldb;       // row strides in elements
    float scale;
    float *C;               // [R][S] (or its first c_rows rows)
    int64_t t_per_split;    // multiple of BT (T when not split)
    int32_t atomic;         // 0: C = v; 1: C += v with fp32 atomics (split); 2: C += v
    int32_t seg_steps;      // contraction steps per segment (0: one segment)
    float seg_ratio[2];
    int64_t c_rows;         // rows per output matrix (0: all in C)
    float *C1, *C2;
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
    // a new contraction segment begins at step st: rescale what was accumulated so far
    auto seg_edge = [&](int st) {
        if (p.seg_steps && st > 0 && st % p.seg_steps == 0) {
            const float r = p.seg_ratio[st / p.seg_steps - 1];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] *= r;
        }
    };
    for (int st = 0; st < nsteps; st += 2) {
        if (st + 2 < nsteps) load_step(tstep(st + 2), ra0, rb0);
        seg_edge(st);
        compute(0);
        if (st + 1 < nsteps) store_step(1, ra1, rb1);
        lds_barrier();
        if (st + 1 < nsteps) {
            if (st + 3 < nsteps) load_step(tstep(st + 3), ra1, rb1);
            seg_edge(st + 1);
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
                int64_t row = r0 + wr * 64 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < p.R) {
                    float *cm = p.C;
                    if (p.c_rows) {
                        if (row >= 2 * p.c_rows) {
                            cm = p.C2;
                            row -= 2 * p.c_rows;
                        } else if (row >= p.c_rows) {
                            cm = p.C1;
                            row -= p.c_rows;
                        }
                        if (!cm) continue;
                    }
                    float *o = cm + row * p.S + col;
                    if (p.atomic == 1) atomicAdd(o, acc[i][j][e] * p.scale);
                    else if (p.atomic == 2) *o += acc[i][j][e] * p.scale;
                    else *o = acc[i][j][e] * p.scale;
                }
            }
        }
}

// The same product for bf16 A, fed by direct-to-LDS 16-byte loads (no register staging)
// into two LDS buffers of 64-deep contraction steps: tile kt + 1 is requested while tile kt
// is multiplied.  One workgroup of 8 waves per CU, tiles of 256 x 256 (4 x 2 waves, each
// 64 x 128 = 2 x 4 MFMA blocks: 6 operand reads per 8 MFMAs, 64 KB of operands per 256
// MFMAs).  The loads, not the matrix cores, set the pace (the texture data path is busy
// most of the time), so the tile is as large as the accumulators allow and each step reads
// whole 128-byte lines of every row (32-deep steps, half lines, took 13 % longer even with a
// 4-buffer ring).  An LDS tile row is 64 bf16 = 128 bytes, eight 16-byte chunks, chunk c of
// row r stored at c ^ dswz(r) (the same swizzle as the int8 GEMM's activation tile).  A load
// fills 64 consecutive 16-byte slots of a buffer (8 rows): lane slot s holds row s / 8,
// stored chunk s % 8.  Requires T and the split length to be multiples of 64 and 16-byte
// aligned rows; rows past R or S are read from row R-1 / S-1 (their outputs are not stored).
constexpr int DGT = 512;                                 // threads (8 waves)
constexpr int DR = 256, DS = 256, DT = 64, DSTAGES = 2;
constexpr int DA_BYTES = DR * DT * 2;                    // 32 KB
constexpr int DB_BYTES = DS * DT * 2;                    // 32 KB
constexpr int DSTAGE = DA_BYTES + DB_BYTES;
constexpr int DA_LOADS = DA_BYTES / (DGT * 16), DB_LOADS = DB_BYTES / (DGT * 16);
static_assert(DA_LOADS == 4 && DB_LOADS == 4, "load split");

__device__ __forceinline__ int dswz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ void barrier_only() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(DGT, 1) void nt_gemm_dma_kernel(NtGemmArgs p) {
    __shared__ __attribute__((aligned(16))) char smem[DSTAGES * DSTAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int r32 = lane & 31, g = lane >> 5;
    int rt, st;
    {   // grouped, XCD-aware tile order (as in the staged kernel above), groups of 4 row tiles
        const int n_rt = static_cast<int>((p.R + DR - 1) / DR), n_st = (p.S + DS - 1) / DS;
        const int nwg = gridDim.x, bid = blockIdx.x;
        const int qx = nwg >> 3, rx = nwg & 7, xcd = bid & 7, idx = bid >> 3;
        const int tile = (xcd < rx ? xcd * (qx + 1) : rx * (qx + 1) + (xcd - rx) * qx) + idx;
        constexpr int GM = 4;
        const int grp = tile / (GM * n_st), in_g = tile % (GM * n_st);
        const int gm = n_rt - grp * GM < GM ? n_rt - grp * GM : GM;
        rt = grp * GM + in_g % gm;
        st = in_g / gm;
    }
    const int64_t r0 = static_cast<int64_t>(rt) * DR;
    const int s0 = st * DS;
    const int64_t t_begin = static_cast<int64_t>(blockIdx.z) * p.t_per_split;
    const int64_t t_end = t_begin + p.t_per_split < p.T ? t_begin + p.t_per_split : p.T;
    const int n = t_end > t_begin ? static_cast<int>((t_end - t_begin) / DT) : 0;

    // per-lane byte offsets of the loads from the wave-uniform step bases
    uint32_t a_off[DA_LOADS], b_off[DB_LOADS];
#pragma unroll
    for (int i = 0; i < DA_LOADS; ++i) {
        const int sl = (wave * DA_LOADS + i) * 64 + lane, row = sl >> 3, c = (sl & 7) ^ dswz(row);
        const int64_t rr = r0 + row < p.R ? row : p.R - 1 - r0;
        a_off[i] = static_cast<uint32_t>((rr * p.lda + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < DB_LOADS; ++i) {
        const int sl = (wave * DB_LOADS + i) * 64 + lane, row = sl >> 3, c = (sl & 7) ^ dswz(row);
        const int64_t rr = s0 + row < p.S ? row : p.S - 1 - s0;
        b_off[i] = static_cast<uint32_t>((rr * p.ldb + 8 * c) * 2);
    }
    const uint16_t *a_row0 = static_cast<const uint16_t *>(p.A) + r0 * p.lda;
    const uint16_t *b_row0 = p.B + static_cast<int64_t>(s0) * p.ldb;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(smem));
    auto issue = [&](int kt, int sg) {
        const int64_t t = t_begin + static_cast<int64_t>(kt) * DT;
        const uint32_t dst = lds0 + sg * DSTAGE;
#pragma unroll
        for (int i = 0; i < DA_LOADS; ++i) dma16(a_row0 + t, a_off[i], dst + (wave * DA_LOADS + i) * 1024);
#pragma unroll
        for (int i = 0; i < DB_LOADS; ++i) dma16(b_row0 + t, b_off[i], dst + DA_BYTES + (wave * DB_LOADS + i) * 1024);
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // fragment offsets in a stage: A row wr*64 + mi*32 + r32, B row wc*128 + ni*32 + r32,
    // logical chunk 2 ks + g
    int fa[2][4], fb[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
            const int row = wr * 64 + mi * 32 + r32;
            fa[mi][ks] = row * 128 + 16 * ((2 * ks + g) ^ dswz(row));
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int row = wc * 128 + ni * 32 + r32;
            fb[ni][ks] = DA_BYTES + row * 128 + 16 * ((2 * ks + g) ^ dswz(row));
        }
    }
    auto step = [&](int kt, auto sc) {
        constexpr int SG = decltype(sc)::value;
        wait_vmcnt<0>();  // this wave's part of tile kt has landed (nothing later is in flight)
        barrier_only();   // every wave's part of tile kt is in LDS; the stage of kt - 1 is free
        if (kt + 1 < n) issue(kt + 1, (SG + 1) % DSTAGES);
        if (p.seg_steps && kt > 0 && (kt * DT) % (p.seg_steps * BT) == 0) {
            const float r = p.seg_ratio[kt * DT / (p.seg_steps * BT) - 1];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] *= r;
        }
        const char *sb = smem + SG * DSTAGE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 av[2], bv[4];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) av[mi] = *reinterpret_cast<const bf16x8 *>(sb + fa[mi][ks]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bv[ni] = *reinterpret_cast<const bf16x8 *>(sb + fb[ni][ks]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mi], bv[ni], acc[mi][ni], 0, 0, 0);
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (n > 0) issue(0, 0);
    int kt = 0;
    for (; kt + 2 <= n; kt += 2) {
        step(kt, S0{});
        step(kt + 1, S1{});
    }
    if (kt < n) step(kt, S0{});

    // C block (mi, ni): lane holds rows 8*(e/4) + 4*g + e%4, column r32
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int col = s0 + wc * 128 + ni * 32 + r32;
            if (col >= p.S) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int64_t row = r0 + wr * 64 + mi * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
                if (row < p.R) {
                    float *cm = p.C;
                    if (p.c_rows) {
                        if (row >= 2 * p.c_rows) {
                            cm = p.C2;
                            row -= 2 * p.c_rows;
                        } else if (row >= p.c_rows) {
                            cm = p.C1;
                            row -= p.c_rows;
                        }
                        if (!cm) continue;
                    }
                    float *o = cm + row * p.S + col;
                    const float v = acc[mi][ni][e] * p.scale;
                    if (p.atomic == 1) atomicAdd(o, v);
                    else if (p.atomic == 2) *o += v;
                    else *o = v;
                }
            }
        }
}

// The direct-load kernel takes the product when A is bf16, the contraction and the split
// are multiples of its step (64), rows are 16-byte aligned and a tile's loads stay within 32-bit
// offsets.
static bool dma_ok(const NtGemmArgs &a) {
    return a.a_bf16 && a.T % DT == 0 && a.t_per_split % DT == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
           reinterpret_cast<uintptr_t>(a.A) % 16 == 0 && reinterpret_cast<uintptr_t>(a.B) % 16 == 0 &&
           static_cast<int64_t>(DS) * (a.lda > a.ldb ? a.lda : a.ldb) * 2 < (int64_t(1) << 31);
}

static dim3 dma_grid(const NtGemmArgs &a, int64_t splits) {
    return dim3(static_cast<unsigned>(((a.R + DR - 1) / DR) * ((a.S + DS - 1) / DS)), 1, static_cast<unsigned>(splits));
}

__device__ __forceinline__ float silu_grad(float z) {
    const float s = sigmoidf_(z);
    return s * (1.0f + z * (1.0f - s));
}

// W^T as bf16 values -1/0/1: out[k][n] (row stride ldo) for the packed [N][K/16] matrix
// (N % 8 == 0); up to seven matrices per launch (blockIdx.z).  A workgroup takes 64 rows n x 32 words (512 k) of the packed matrix: the
// words are read row by row as 16-byte vectors into LDS, then every output row k is
// written as 64 consecutive n (eight 16-byte stores).
__global__ __launch_bounds__(256) void expand_wt_kernel(ExpandJobs jobs) {
    __shared__ uint32_t wl[64][33];
    const int tid = threadIdx.x;
    const uint32_t *packed = jobs.packed[blockIdx.z];
    const int32_t N = jobs.N[blockIdx.z], K = jobs.K[blockIdx.z];
    uint16_t *out = jobs.out[blockIdx.z];
    const int64_t ldo = jobs.ldo[blockIdx.z];
    const int KW = K / 16;
    const int n0 = blockIdx.x * 64, kw0 = blockIdx.y * 32;
    if (n0 >= N || kw0 >= KW) return;   // (the grid covers the largest matrix of the launch)
#pragma unroll
    for (int it = 0; it < 2; ++it) {   // 64 rows x 8 vectors of 4 words
        const int v = tid + 256 * it, r = v >> 3, c4 = 4 * (v & 7);
        const int n = n0 + r;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (n < N) {
            const uint32_t *src = packed + static_cast<int64_t>(n) * KW + kw0 + c4;
            if (kw0 + c4 + 4 <= KW && (KW & 3) == 0) {
                const uint4 u = *reinterpret_cast<const uint4 *>(src);
                w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (kw0 + c4 + e < KW) w[e] = src[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) wl[r][c4 + e] = w[e];
    }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {   // 512 rows k x 8 chunks of 8 n
        const int v = tid + 256 * it, kl = v >> 3, nc = v & 7;
        const int kwl = kl >> 4, j = kl & 15;
        const int k = 16 * (kw0 + kwl) + j, n = n0 + 8 * nc;
        if (k >= K || n >= N) continue;
        const int sh = 8 * (j & 3) + 2 * (j >> 2);
        uint16_t c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t code = (wl[8 * nc + e][kwl] >> sh) & 3u;
            c[e] = code == 2 ? 0x3F80u : (code == 0 ? 0xBF80u : 0u);
        }
        *reinterpret_cast<uint4 *>(out + static_cast<int64_t>(k) * ldo + n) =
            make_uint4(c[0] | (uint32_t(c[1]) << 16), c[2] | (uint32_t(c[3]) << 16),
                       c[4] | (uint32_t(c[5]) << 16), c[6] | (uint32_t(c[7]) << 16));
    }
}

// Column sums folded into a transpose: out[j][c - j*cols] += sum_m src[m][c] for the columns
// of segment j (up to three outputs; a NULL one is skipped), fp32 atomics into zeroed arrays.
struct ColSums {
    float *o[3];
    int32_t cols;
};

// dst[c][m] = bf16(src[m][c] * (scale ? scale[m] : 1)) for m < M, 0 for M <= m < ldm (the
// padding of every destination row), and the column sums of the unscaled src (if any output
// is given).  src [M][lds]: bf16, fp32 or int8 codes (SRC 0/1/2).  A workgroup takes 64
// columns and 256 rows as four 64 x 64 tiles through LDS: rows are read as 16-byte vectors
// (when `vec`: every row 16-byte aligned) and columns written as 32-byte runs.
template <int SRC>
__global__ __launch_bounds__(256) void transpose_kernel(const void *src, int64_t lds, int32_t vec,
                                                        const float *scale, int64_t M, int32_t C,
                                                        int64_t ldm, uint16_t *dst, ColSums cs) {
    constexpr int ES = SRC == 0 ? 2 : (SRC == 1 ? 4 : 1);   // bytes per element
    constexpr int EV = 16 / ES;                              // elements per 16-byte vector
    constexpr int VR = 64 / EV;                              // vectors per tile row
    constexpr int NV = 64 * VR / 256;                        // vectors per thread per tile
    __shared__ float tile[64][65];
    __shared__ float sc[64];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * 64;
    const bool sums = cs.o[0] || cs.o[1] || cs.o[2];
    float csum = 0.0f;
#pragma unroll 1
    for (int tm = 0; tm < 4; ++tm) {
        const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 256 + 64 * tm;
        if (m0 >= ldm) break;
        if (tid < 64) {
            const int64_t m = m0 + tid;
            sc[tid] = m < M ? (scale ? scale[m] : 1.0f) : 0.0f;
        }
        const bool full = vec && m0 + 64 <= M && c0 + 64 <= C;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int v = tid + 256 * j, r = v / VR, cc = (v % VR) * EV;
            const int64_t m = m0 + r;
            float f[EV];
            if (full) {
                const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const char *>(src) +
                                                                 (m * lds + c0 + cc) * ES);
                const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    if constexpr (SRC == 0) f[e] = bf16_bits_to_f32(static_cast<uint16_t>(u[e / 2] >> (16 * (e % 2))));
                    else if constexpr (SRC == 1) f[e] = __uint_as_float(u[e]);
                    else f[e] = static_cast<float>(static_cast<int8_t>(u[e / 4] >> (8 * (e % 4))));
                }
            } else {
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const int c = c0 + cc + e;
                    f[e] = 0.0f;
                    if (m < M && c < C) {
                        const int64_t idx = m * lds + c;
                        if constexpr (SRC == 0) f[e] = bf16_bits_to_f32(static_cast<const uint16_t *>(src)[idx]);
                        else if constexpr (SRC == 1) f[e] = static_cast<const float *>(src)[idx];
                        else f[e] = static_cast<float>(static_cast<const int8_t *>(src)[idx]);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < EV; ++e) tile[r][cc + e] = f[e];
        }
        __syncthreads();
        {
            const int cl = tid >> 2, mm = 16 * (tid & 3);
            const int c = c0 + cl;
            uint16_t v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float t = tile[mm + e][cl];
                csum += t;
                v[e] = bf16_bits(t * sc[mm + e]);
            }
            if (c < C) store16(dst + static_cast<int64_t>(c) * ldm + m0 + mm, v);
        }
        __syncthreads();
    }
    if (sums) {
        csum += __shfl_xor(csum, 1);
        csum += __shfl_xor(csum, 2);
        const int c = c0 + (tid >> 2);
        if ((tid & 3) == 0 && c < C) {
            const int j = c / cs.cols;
            if (j < 3 && cs.o[j]) atomicAdd(&cs.o[j][c - j * cs.cols], csum);
        }
    }
}

// dx and dgamma from g, workgroup per row (rows blockIdx.x, + gridDim.x, ...), thread per
// four consecutive columns c = 4 tid + 1024 j (K % 4 == 0, K <= 8192), the row's x and g held
// in registers between the two passes:
//   r = (mean x^2 + eps)^(-1/2), dot = sum_c g*gamma*x, d = r*gamma*g - x*r^3/K*dot
//   (+ a residual gradient res [M][K], bf16 for RES 1, fp32 for RES 2);
//   OUT 0: dx = d (fp32); OUT 1: also a bf16 copy dx_bf16; OUT 2: d is the gradient at the
//   GLU's gated product m = SiLU(gate)*up (K = F) and is carried through it: dgu [M][2F] bf16
//   gets dgate = d*up*silu'(gate) at column c and dup = d*SiLU(gate) at F + c, gate | up from
//   the pre-activations gu [M][2F] bf16;
//   dgamma: each workgroup's sum over its rows of g*x*r into dg_part[blockIdx.x][K], then
//   summed over the workgroups by the column-sum kernel (one fp32 atomic per column per 768
//   workgroups contended more than the two launches cost).
constexpr int RV = 8;   // float4 chunks per thread (K <= 8192)

template <bool XBF16>
__device__ __forceinline__ float4 load4(const void *p, int64_t i) {
    if constexpr (XBF16) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    } else {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    }
}

template <bool XBF16, int RES, int OUT>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdRowsArgs p) {
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.K;
    float4 dg[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j) dg[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int64_t m = blockIdx.x; m < p.M; m += gridDim.x) {
        float4 xv[RV], gv[RV];
        float ss = 0.0f, dot = 0.0f;
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            const int c = 4 * tid + 1024 * j;
            xv[j] = gv[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (c < K) {
                xv[j] = load4<XBF16>(p.x, m * K + c);
                gv[j] = *reinterpret_cast<const float4 *>(p.g + m * K + c);
                const float4 gm = p.gamma ? *reinterpret_cast<const float4 *>(p.gamma + c)
                                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                ss = fmaf(xv[j].x, xv[j].x, fmaf(xv[j].y, xv[j].y, fmaf(xv[j].z, xv[j].z, fmaf(xv[j].w, xv[j].w, ss))));
                dot = fmaf(gv[j].x * gm.x, xv[j].x, fmaf(gv[j].y * gm.y, xv[j].y,
                      fmaf(gv[j].z * gm.z, xv[j].z, fmaf(gv[j].w * gm.w, xv[j].w, dot))));
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
        const float r = 1.0f / sqrtf(ss / static_cast<float>(K) + p.eps);
        const float c3 = r * r * r / static_cast<float>(K) * dot;
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            const int c = 4 * tid + 1024 * j;
            if (c < K) {
                const float4 gm = p.gamma ? *reinterpret_cast<const float4 *>(p.gamma + c)
                                          : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                float d[4] = {r * gm.x * gv[j].x - xv[j].x * c3, r * gm.y * gv[j].y - xv[j].y * c3,
                              r * gm.z * gv[j].z - xv[j].z * c3, r * gm.w * gv[j].w - xv[j].w * c3};
                if constexpr (RES != 0) {
                    const float4 rv = load4<RES == 1>(p.res, m * K + c);
                    d[0] += rv.x;
                    d[1] += rv.y;
                    d[2] += rv.z;
                    d[3] += rv.w;
                }
                if constexpr (OUT == 2) {
                    const float4 ga = load4<true>(p.gu, m * 2 * K + c);
                    const float4 up = load4<true>(p.gu, m * 2 * K + K + c);
                    const float gg[4] = {ga.x, ga.y, ga.z, ga.w}, uu[4] = {up.x, up.y, up.z, up.w};
                    float dga[4], dup[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dga[e] = d[e] * uu[e] * silu_grad(gg[e]);
                        dup[e] = d[e] * siluf_(gg[e]);
                    }
                    *reinterpret_cast<uint2 *>(p.dgu + m * 2 * K + c) =
                        make_uint2(pack_bf16x2(dga[0], dga[1]), pack_bf16x2(dga[2], dga[3]));
                    *reinterpret_cast<uint2 *>(p.dgu + m * 2 * K + K + c) =
                        make_uint2(pack_bf16x2(dup[0], dup[1]), pack_bf16x2(dup[2], dup[3]));
                } else {
                    if (p.dx) *reinterpret_cast<float4 *>(p.dx + m * K + c) = make_float4(d[0], d[1], d[2], d[3]);
                    if constexpr (OUT == 1)
                        *reinterpret_cast<uint2 *>(p.dx_bf16 + m * K + c) =
                            make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
                }
                dg[j].x = fmaf(gv[j].x * xv[j].x, r, dg[j].x);
                dg[j].y = fmaf(gv[j].y * xv[j].y, r, dg[j].y);
                dg[j].z = fmaf(gv[j].z * xv[j].z, r, dg[j].z);
                dg[j].w = fmaf(gv[j].w * xv[j].w, r, dg[j].w);
            }
        }
    }
    if (p.dgamma) {
#pragma unroll
        for (int j = 0; j < RV; ++j) {
            const int c = 4 * tid + 1024 * j;
            if (c < K) *reinterpret_cast<float4 *>(p.dg_part + static_cast<int64_t>(blockIdx.x) * K + c) = dg[j];
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

// Several arrays zeroed by one launch: blockIdx.y picks the array, the workgroups along x
// stride over it.
__global__ __launch_bounds__(256) void fill_zero_many_kernel(ZeroJobs j) {
    float *p = j.p[blockIdx.y];
    const int64_t n = j.n[blockIdx.y];
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = 0.0f;
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
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
__global__ __launch_bounds__(512) void mlgru_bwd_carry_kernel(MlgruBwdArgs p) {
    // G at the first token of chunk c: G_c = cb_c + m_c G_(c+1), m_c = cp_c f0_(c+1) (zero for
    // the last chunk).  Workgroup per (b, 64 channels), wave s owns the s-th of 8 runs of
    // consecutive chunks: it folds its run, right to left, into one affine map G -> A G + B
    // (lane = channel), the maps are composed through LDS (from the last run backwards) to give
    // the G entering every run from the right, and each wave walks its run again storing the
    // G carried into each chunk (cg) -- the two-level scheme of the forward's carry pass.
    constexpr int RUNS = 8;
    __shared__ float sA[RUNS][64], sB[RUNS][64];
    const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
    const int D = p.D, nc = p.n_chunks;
    const int d = blockIdx.x * 64 + lane;
    const bool live = d < D;
    const int64_t b = blockIdx.y, row0 = b * nc;
    const int L = (nc + RUNS - 1) / RUNS;
    const int c0 = s * L < nc ? s * L : nc, c1 = c0 + L < nc ? c0 + L : nc;
    // the run's m and cb are requested U chunks at a time ahead of the dependent chain; a run
    // of at most U chunks (2048 tokens and fewer at 16 tokens per chunk) stays in registers
    // for the second walk
    constexpr int U = 16;
    float mv[U], bv[U];
    auto load_batch = [&](int ce) {   // chunks ce - u, u < U, clamped to the run
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = ce - u >= c0 ? ce - u : c0;
            mv[u] = c + 1 < nc ? p.cp[(row0 + c) * D + d] * p.cf0[(row0 + c + 1) * D + d] : 0.0f;
            bv[u] = p.cb[(row0 + c) * D + d];
        }
    };
    const bool one_batch = c1 - c0 <= U;
    float A = 1.0f, Bv = 0.0f;
    if (live)
        for (int ce = c1 - 1; ce >= c0; ce -= U) {
            load_batch(ce);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ce - u >= c0) {
                    Bv = fmaf(mv[u], Bv, bv[u]);
                    A *= mv[u];
                }
        }
    sA[s][lane] = A;
    sB[s][lane] = Bv;
    __syncthreads();
    if (!live) return;
    float G = 0.0f;   // entering the last chunk of run s from the right
    for (int j = RUNS - 1; j > s; --j) G = fmaf(sA[j][lane], G, sB[j][lane]);
    for (int ce = c1 - 1; ce >= c0; ce -= U) {
        if (!one_batch) load_batch(ce);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ce - u >= c0) {
                p.cg[(row0 + ce - u) * D + d] = G;
                G = fmaf(mv[u], G, bv[u]);
            }
    }
    if (s == 0 && p.dh0) p.dh0[b * D + d] = p.cf0[row0 * D + d] * G;
}

// Phases 2 and 4: thread per (b, chunk, d).  Rerun the chunk forward (state before each
// token, f, c, i in registers), form the gradient at h from the output gate (gate mode 0
// with the per-token rho and k3 of phase 1), then walk the chunk backwards:
//   PASS 0: from zero (G_t = dh_t + f_{t+1} G_{t+1}) -> the chunk's first-token G, the
//           product of f after the first token, f at the first token; dg and the chunk's
//           partial sum of the g_norm weight gradient;
//   PASS 1: from the carried G (phase 3) -> di, df_pre and the chunk's partial sum of df.
__device__ __forceinline__ void store_grad(const MlgruBwdArgs &p, int64_t i, float v) {
    if (p.d_ifg_bf16) store_act<true>(p.d_ifg, i, v);
    else store_act<false>(p.d_ifg, i, v);
}

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
    // per token: hprev, sigma of the forget pre-activation (taken once), i, and the gradient
    // at h (caching sigma(i) too costs a wave of occupancy, which this latency-bound pass
    // needs more than the sigmoids it saves)
    float hprev[kBC], sz[kBC], iv[kBC], dh[kBC];
    float h = c == 0 ? (p.h0 ? p.h0[b * D + d] : 0.0f) : p.hin[crow * D + d];
    float gwp = 0.0f;
#pragma unroll
    for (int k = 0; k < kBC; ++k) {
        hprev[k] = sz[k] = iv[k] = dh[k] = 0.0f;
        if (k < n) {
            const int64_t row = b * p.T + t0 + k;
            iv[k] = load_act<IFGBF16>(p.ifg, row * 3 * D + d);
            const float fzk = load_act<IFGBF16>(p.ifg, row * 3 * D + D + d) + fb;
            const float gv = load_act<IFGBF16>(p.ifg, row * 3 * D + 2 * D + d);
            const float dov = load_act<DOBF16>(p.dout, row * D + d);
            sz[k] = sigmoidf_(fzk);
            const float f = fmaf(1.0f - lb, sz[k], lb);
            hprev[k] = h;
            h = f * h + (1.0f - f) * siluf_(iv[k]);
            float dho, dg;
            if (p.gate_mode == 0) {
                const float rho = p.stats[2 * row], k3 = p.stats[2 * row + 1];
                const float sgg = sigmoidf_(gv);
                const float nrm = h * rho, sg = gv * sgg;
                dho = rho * (dov * gw * sg) - h * k3;
                dg = dov * nrm * gw * (sgg * (1.0f + gv * (1.0f - sgg)));
                gwp = fmaf(dov * nrm, sg, gwp);
            } else {
                const float s = sigmoidf_(gv);
                dg = dov * h * s * (1.0f - s);
                dho = dov * s;
            }
            if (t0 + k == p.T - 1 && p.dh_last) dho += p.dh_last[b * D + d];
            dh[k] = dho;
            if constexpr (PASS == 0) store_grad(p, row * 3 * D + 2 * D + d, dg);
        }
    }
    if constexpr (PASS == 0) {
        float G = 0.0f, fnext = 0.0f, prod = 1.0f, f = 0.0f;
#pragma unroll
        for (int k = kBC - 1; k >= 0; --k) {
            if (k < n) {
                G = dh[k] + fnext * G;
                f = fmaf(1.0f - lb, sz[k], lb);
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
                const float f = fmaf(1.0f - lb, sz[k], lb);
                const float si = sigmoidf_(iv[k]);
                const float cv = iv[k] * si;
                G = dh[k] + fnext * G;
                store_grad(p, row * 3 * D + d, (1.0f - f) * G * (si * (1.0f + iv[k] * (1.0f - si))));
                const float dz = (hprev[k] - cv) * G * (1.0f - lb) * sz[k] * (1.0f - sz[k]);
                store_grad(p, row * 3 * D + D + d, dz);
                dfb += dz;
                fnext = f;
            }
        }
        p.fb_part[crow * D + d] = dfb;
    }
}

}  // namespace

hipError_t launch_fill_zero_many(const ZeroJobs &j, hipStream_t s) {
    ZeroJobs c{};
    int nj = 0;
    int64_t mx = 0;
    for (int i = 0; i < j.count && i < ZeroJobs::kMax; ++i)
        if (j.p[i] && j.n[i] > 0) {
            c.p[nj] = j.p[i];
            c.n[nj] = j.n[i];
            mx = std::max(mx, j.n[i]);
            ++nj;
        }
    if (!nj) return hipSuccess;
    c.count = nj;
    const int64_t wg = std::min<int64_t>((mx + 255) / 256, 2048);
    hipLaunchKernelGGL(fill_zero_many_kernel, dim3(static_cast<unsigned>(wg), static_cast<unsigned>(nj)), dim3(256), 0, s, c);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t s) {
    if (n <= 0 || !p) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_col_sum(const void *src, int bf16, int64_t lds, int64_t R, int32_t C, float *out,
                          hipStream_t s) {
    if (R <= 0 || C <= 0) return hipSuccess;
    // about 16 rows per workgroup (the partial sums of a few hundred to a few thousand
    // workgroups), at most 256 row splits (so at most 256 atomics per column for long sums)
    int64_t splits = (R + 15) / 16;
    if (splits > 256) splits = 256;
    const int32_t rows_per = static_cast<int32_t>((R + splits - 1) / splits);
    splits = (R + rows_per - 1) / rows_per;
    const dim3 grid(static_cast<unsigned>((C + 255) / 256), static_cast<unsigned>(splits));
    if (bf16) hipLaunchKernelGGL((col_sum_kernel<true>), grid, dim3(256), 0, s, src, lds, R, C, rows_per, out);
    else hipLaunchKernelGGL((col_sum_kernel<false>), grid, dim3(256), 0, s, src, lds, R, C, rows_per, out);
    return hipGetLastError();
}

hipError_t launch_expand_wt(const ExpandJobs &j, hipStream_t s) {
    if (j.count <= 0) return hipSuccess;
    int32_t mn = 0, mk = 0;
    for (int i = 0; i < j.count; ++i) {
        mn = std::max(mn, j.N[i]);
        mk = std::max(mk, j.K[i]);
    }
    const dim3 ge(static_cast<unsigned>((mn + 63) / 64), static_cast<unsigned>((mk / 16 + 31) / 32),
                  static_cast<unsigned>(j.count));
    hipLaunchKernelGGL(expand_wt_kernel, ge, dim3(256), 0, s, j);
    return hipGetLastError();
}

hipError_t bwd_launch_g(const void *dy, int dy_bf16, int64_t ldy, const uint32_t *const *packed,
                        const float *scales, int nseg, int32_t N, int32_t K, int64_t M, uint16_t *wt,
                        int expanded, float *g, hipStream_t s) {
    if (M <= 0 || nseg < 1 || nseg > 3) return hipSuccess;
    const int64_t ldb = static_cast<int64_t>(nseg) * N;
    if (!expanded) {
        ExpandJobs ej{};
        for (int j = 0; j < nseg; ++j) {
            ej.packed[j] = packed[j];
            ej.N[j] = N;
            ej.K[j] = K;
            ej.out[j] = wt + static_cast<int64_t>(j) * N;
            ej.ldo[j] = ldb;
        }
        ej.count = nseg;
        hipError_t e = launch_expand_wt(ej, s);
        if (e != hipSuccess) return e;
    }
    // one launch over the stacked contraction when every segment boundary is a step boundary
    // and the scale ratios are finite
    bool one = N % BT == 0;
    for (int j = 0; j < nseg; ++j) one = one && scales[j] > 0.0f && scales[j] < 3.0e38f;
    const dim3 grid(static_cast<unsigned>(((K + BS - 1) / BS) * ((M + BR - 1) / BR)), 1, 1);
    const int nl = nseg == 1 || one ? 1 : nseg;
    timing_begin(FAM_BWD_G, s);
    for (int l = 0; l < nl; ++l) {
        NtGemmArgs ga{};
        ga.a_bf16 = dy_bf16;
        ga.R = M;
        ga.S = K;
        ga.lda = ldy;
        ga.ldb = ldb;
        ga.C = g;
        if (nl == 1) {
            ga.A = dy;
            ga.B = wt;
            ga.T = ldb;
            ga.scale = scales[nseg - 1];
            ga.seg_steps = nseg > 1 ? N / BT : 0;
            for (int j = 0; j + 1 < nseg; ++j) ga.seg_ratio[j] = scales[j] / scales[j + 1];
        } else {   // one launch per linear, added into g
            ga.A = static_cast<const char *>(dy) + static_cast<int64_t>(l) * N * (dy_bf16 ? 2 : 4);
            ga.B = wt + static_cast<int64_t>(l) * N;
            ga.T = N;
            ga.scale = scales[l];
            ga.atomic = l > 0 ? 2 : 0;
        }
        ga.t_per_split = ga.T;
        if (dma_ok(ga)) hipLaunchKernelGGL(nt_gemm_dma_kernel, dma_grid(ga, 1), dim3(DGT), 0, s, ga);
        else if (dy_bf16) hipLaunchKernelGGL((nt_gemm_kernel<true>), grid, dim3(GT), 0, s, ga);
        else hipLaunchKernelGGL((nt_gemm_kernel<false>), grid, dim3(GT), 0, s, ga);
    }
    timing_end(FAM_BWD_G, s);
    return hipGetLastError();
}

// one workgroup per row up to 768 of them (each then takes every 768th row): the row kernels
// hold 135-155 VGPRs, three 256-thread workgroups per CU, so 768 is one full wave on 256 CUs
static int64_t rows_grid(int64_t M) { return M < 768 ? M : 768; }

size_t bwd_rows_part_bytes(int64_t M, int32_t K) {
    return M > 0 ? static_cast<size_t>(rows_grid(M)) * K * 4 : 0;
}

hipError_t bwd_launch_rows(const BwdRowsArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    hipError_t e;
    const BwdRowsArgs &p = a;
    if (p.dgamma && !a.dgamma_zeroed && (e = launch_fill_zero(p.dgamma, a.K, s)) != hipSuccess) return e;
    const int64_t nwg = rows_grid(a.M);
    const dim3 grid(static_cast<unsigned>(nwg));
    const int rk = a.res ? (a.res_bf16 ? 1 : 2) : 0;
    const int ok = a.dgu ? 2 : (a.dx_bf16 ? 1 : 0);
#define MMF_ROWS(XB, RK, OK) hipLaunchKernelGGL((bwd_rows_kernel<XB, RK, OK>), grid, dim3(256), 0, s, p)
#define MMF_ROWS_OK(XB, RK) \
    if (ok == 2) MMF_ROWS(XB, RK, 2); else if (ok == 1) MMF_ROWS(XB, RK, 1); else MMF_ROWS(XB, RK, 0);
    if (a.x_bf16) {
        if (rk == 1) { MMF_ROWS_OK(true, 1) }
        else if (rk == 2) { MMF_ROWS_OK(true, 2) }
        else { MMF_ROWS_OK(true, 0) }
    } else {
        if (rk == 1) { MMF_ROWS_OK(false, 1) }
        else if (rk == 2) { MMF_ROWS_OK(false, 2) }
        else { MMF_ROWS_OK(false, 0) }
    }
#undef MMF_ROWS_OK
#undef MMF_ROWS
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.dgamma) return launch_col_sum(p.dg_part, 0, a.K, nwg, a.K, p.dgamma, s);
    return hipSuccess;
}

template <int SRC>
static void launch_transpose(const void *src, int64_t lds, const float *scale, int64_t M, int32_t C,
                             int64_t ldm, uint16_t *dst, const ColSums &cs, hipStream_t s) {
    constexpr int ES = SRC == 0 ? 2 : (SRC == 1 ? 4 : 1);
    const int vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && (lds * ES) % 16 == 0;
    const dim3 gt(static_cast<unsigned>((C + 63) / 64), static_cast<unsigned>((ldm + 255) / 256));
    hipLaunchKernelGGL((transpose_kernel<SRC>), gt, dim3(256), 0, s, src, lds, vec, scale, M, C, ldm, dst, cs);
}

hipError_t bwd_launch_qT(const int8_t *q, int64_t M, int32_t K, int64_t ldm, uint16_t *qT, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    launch_transpose<2>(q, static_cast<int64_t>(K), nullptr, M, K, ldm, qT, ColSums{}, s);
    return hipGetLastError();
}

hipError_t bwd_launch_dw(const void *dy, int dy_bf16, int64_t ldy, const float *a, int64_t M, int nseg,
                         int32_t N, int32_t K, int64_t ldm, const uint16_t *qT, uint16_t *dyaT,
                         float *const *dw, float *const *db, int zeroed, hipStream_t s) {
    hipError_t e;
    bool any_dw = false;
    for (int j = 0; j < nseg; ++j) {
        if (db[j] && !zeroed && (e = launch_fill_zero(db[j], N, s)) != hipSuccess) return e;
        any_dw = any_dw || dw[j];
    }
    if (M <= 0) {
        for (int j = 0; j < nseg; ++j)
            if (dw[j] && !zeroed && (e = launch_fill_zero(dw[j], static_cast<int64_t>(N) * K, s)) != hipSuccess) return e;
        return hipSuccess;
    }
    if (!any_dw) {   // the bias gradients alone: column sums
        for (int j = 0; j < nseg; ++j) {
            const void *src = static_cast<const char *>(dy) + static_cast<int64_t>(j) * N * (dy_bf16 ? 2 : 4);
            if (db[j] && (e = launch_col_sum(src, dy_bf16, ldy, M, N, db[j], s)) != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int32_t R = nseg * N;
    ColSums cs{};
    for (int j = 0; j < nseg; ++j) cs.o[j] = db[j];
    cs.cols = N;
    if (dy_bf16) launch_transpose<0>(dy, ldy, a, M, R, ldm, dyaT, cs, s);
    else launch_transpose<1>(dy, ldy, a, M, R, ldm, dyaT, cs, s);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    NtGemmArgs ga{};
    ga.A = dyaT;
    ga.a_bf16 = 1;
    ga.B = qT;
    ga.R = R;
    ga.S = K;
    ga.T = ldm;
    ga.lda = ldm;
    ga.ldb = ldm;
    ga.scale = 1.0f;
    ga.C = dw[0];
    if (nseg > 1) {
        ga.c_rows = N;
        ga.C1 = dw[1];
        ga.C2 = nseg > 2 ? dw[2] : nullptr;
    }
    ga.t_per_split = ldm;
    const bool dma = dma_ok(ga);
    const int64_t tiles = dma ? static_cast<int64_t>((K + DS - 1) / DS) * ((R + DR - 1) / DR)
                              : static_cast<int64_t>((K + BS - 1) / BS) * ((R + BR - 1) / BR);
    // split the tokens over workgroups (fp32 atomics) when there are too few tiles for 256
    // CUs x 2: the smallest split count, each split >= 8 steps, whose last wave of workgroups
    // is at least 85 % full (or the best of those tried)
    const int64_t slots = dma ? 256 : 512;   // co-resident workgroups on 256 CUs
    const int64_t max_splits = std::min<int64_t>(64, std::max<int64_t>(1, (ldm + 8 * BT - 1) / (8 * BT)));
    int64_t splits = 1;
    double best = -1.0;
    for (int64_t sp = 1; sp <= max_splits; ++sp) {
        const int64_t wg = tiles * sp, waves = (wg + slots - 1) / slots;
        const double fill = static_cast<double>(wg) / static_cast<double>(waves * slots);
        if (wg < slots && sp < max_splits) continue;   // not yet one full wave
        if (fill > best + 1e-9) {
            best = fill;
            splits = sp;
        }
        if (fill >= 0.85) break;
    }
    int64_t per = (ldm + splits - 1) / splits;
    per = (per + BT - 1) / BT * BT;
    splits = (ldm + per - 1) / per;
    ga.t_per_split = per;
    ga.atomic = splits > 1 || zeroed ? 1 : 0;   // onto zeros: atomics are exact adds to 0 and then sums
    if (splits > 1 && !zeroed)
        for (int j = 0; j < nseg; ++j)
            if (dw[j] && (e = launch_fill_zero(dw[j], static_cast<int64_t>(N) * K, s)) != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>(tiles), 1, static_cast<unsigned>(splits));
    timing_begin(FAM_BWD_DW, s);
    if (dma) hipLaunchKernelGGL(nt_gemm_dma_kernel, grid, dim3(DGT), 0, s, ga);
    else hipLaunchKernelGGL((nt_gemm_kernel<true>), grid, dim3(GT), 0, s, ga);
    timing_end(FAM_BWD_DW, s);
    return hipGetLastError();
}

hipError_t launch_bitlinear_bwd(const BitlinearBwdArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    hipError_t e;
    if ((e = bwd_launch_g(a.dy, a.dy_bf16, a.N, &a.packed, &a.scale, 1, a.N, a.K, a.M, a.wt, 0, a.g, s)) != hipSuccess) return e;
    BwdRowsArgs r{};
    r.x = a.x;
    r.x_bf16 = a.x_bf16;
    r.g = a.g;
    r.gamma = a.gamma;
    r.eps = a.eps;
    r.M = a.M;
    r.K = a.K;
    r.dx = a.dx;
    r.dgamma = a.dgamma;
    r.dg_part = a.dg_part;
    if ((a.dx || a.dgamma) && (e = bwd_launch_rows(r, s)) != hipSuccess) return e;
    if (a.dw && (e = bwd_launch_qT(a.q, a.M, a.K, a.ldm, a.qT, s)) != hipSuccess) return e;
    float *dw = a.dw, *db = a.db;
    if (a.dw || a.db)
        if ((e = bwd_launch_dw(a.dy, a.dy_bf16, a.N, a.a, a.M, 1, a.N, a.K, a.ldm, a.qT, a.dyaT, &dw, &db, 0, s)) != hipSuccess) return e;
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
    hipLaunchKernelGGL(mlgru_bwd_carry_kernel, dim3(static_cast<unsigned>((a.D + 63) / 64), static_cast<unsigned>(a.B)),
                       dim3(512), 0, s, a);
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
