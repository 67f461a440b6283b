// gemv_decode.hip -- decode-regime BitLinear for a few tokens: streams the 2-bit packed
// ternary weights from HBM once per token group and reduces with cross-lane shuffles.
//
// DataCamp "MatMul-free language models", sections "Replacing MatMul with ternary
// operations" (products by -1/0/+1 are sign-matched adds) and "From optimised GPU to
// custom FPGA" (token generation is limited by moving the weights); Hysen Labs
// "MatMul-Free LM", section "FusedBitLinear" (norm + quantize + accumulate in one kernel).
//
// With a few tokens per step the weights (0.25 byte each) are read once and used once, and
// one BitLinear moves only a few MB, about one memory latency's worth of HBM bandwidth, so
// the kernel is built to have every weight byte in flight as early as possible:
//   - 16 lanes per weight row, 4 rows per wave, 16 rows per workgroup (32 for one token and
//     rows of 8192 or more, so the row is quantized half as often); lane j of a row
//     holds 16-byte chunks j, j+16, ... (64 k each) of the row in registers, and all of
//     them are requested at kernel entry;
//   - loads return in issue order, so for one token (up to four token rows run one per row
//     of the grid, the weight rows re-read for the next token coming from the same XCD's
//     L2) the activation row (or the pre-quantized codes with their scale and code
//     sum) is requested first, held in registers, and the weight and residual requests
//     that follow are unconditional (clamped addresses) so every wait is exact; the number
//     of chunks per lane is a template parameter (1, 2, 4, 6 or 8), so a short row neither
//     holds nor requests unused chunks;
//   - meanwhile the workgroup RMS/absmax-quantizes its token group (<= TG rows) into LDS
//     (the same arithmetic as the standalone quantizer, so the int8 codes are identical),
//     or copies rows that are already quantized; for o_proj of a decode step (one token
//     per sequence, one sequence per row of the grid) the prologue first runs the MLGRU
//     step and g_norm from the i|f|g pre-activations and the carried state (XIN 3);
//   - each packed word gives four dwords of 2-bit codes c = q + 1 ((w >> 2a) & 0x03030303),
//     which one v_perm_b32 each maps to signed int8 weights (code 0,1,2 -> -1,0,+1),
//     consumed by v_dot4_i32_i8 against the LDS-resident activations: the int32 result is
//     the exact ternary product.  For one token and rows of 8192 or more the permute is
//     skipped: the codes are multiplied as they are and the offset is removed once per
//     token with the row's code sum (acc = sum q_x*c - sum q_x), which the prologue adds to
//     its reductions;
//   - the 16 partial sums of a row are reduced for all tokens at once (halving exchanges),
//     after which one lane per token writes the output (fused rescale, bias, residual or
//     SiLU(gate)*up).
// LDS layout: chunk c (64 k) of all TG token rows together, token t at byte
// c*(64*TG + 16) + 64*t: token offsets are immediates, and the 16-byte pad puts the sixteen
// chunks read by one instruction on distinct bank quads.
#include "mmf_internal.h"

#include <type_traits>

namespace mmf {

namespace {

constexpr int LPR = 16;          // lanes per weight row
constexpr int RPW = 64 / LPR;    // rows per wave
// rows per workgroup: NW waves of RPW rows (4 waves, or 8 for one token with K >= 8192:
// the activation row is then quantized once per 32 rows instead of once per 16)
constexpr int CB = 8;            // 64-k chunks held per lane per pass (K <= 8192 in one pass)
constexpr int kStreamRows = 16384;  // one token and at least this many rows: streaming kernel

__host__ __device__ __forceinline__ int chunk_stride(int tg) { return 64 * tg + 16; }

// 2-bit codes (0,1,2) in each byte of (w >> 2a) & 0x03030303 -> signed ternary int8 x 4.
__device__ __forceinline__ v4i signed_codes(uint32_t w) {
    constexpr uint32_t kTab = 0x000100FFu;  // byte v of the table = value of code v
    v4i r;
    r.x = static_cast<int>(__builtin_amdgcn_perm(0u, kTab, w & 0x03030303u));
    r.y = static_cast<int>(__builtin_amdgcn_perm(0u, kTab, (w >> 2) & 0x03030303u));
    r.z = static_cast<int>(__builtin_amdgcn_perm(0u, kTab, (w >> 4) & 0x03030303u));
    r.w = static_cast<int>(__builtin_amdgcn_perm(0u, kTab, (w >> 6) & 0x03030303u));
    return r;
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4 &u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}

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

// XIN: 0 = pre-quantized input, 1 = fp32 activations, 2 = bf16 activations, 3 = one MLGRU
// step computed from the i|f|g pre-activations and the carried state (o_proj of one token
// per grid row, i.e. per sequence of a decode step; activations in the output dtype).
// TG: token rows per workgroup (1, 4, 8 or 16; up to four rows, one per grid row).
// NW: waves per workgroup.
// NI: 64-k chunks held per lane per pass (CB, or for one token the fewest of 1, 2, 4, 6, 8
// that cover the row, so short rows neither hold nor request unused chunks).
template <int EPI, int XIN, bool OUT_BF16, int TG, int NW, int NI>
__global__ __launch_bounds__(64 * NW) void gemv_dot4_kernel(GemvArgs p) {
    constexpr int NT = 64 * NW;
    // long rows (8 waves): codes multiplied as they are, offset removed per token with the
    // row's code sum (fewer VALU per code); otherwise codes mapped to signed weights, which
    // needs no code sum (no extra reduction before the dot products)
    constexpr bool UNS = NW == 8;
    extern __shared__ __attribute__((aligned(16))) int8_t qs[];
    __shared__ float red_m[NW][TG], red_s[NW][TG], red_h[NW];
    __shared__ int red_q[NW][TG];
    __shared__ float s_a[TG];
    __shared__ int s_rs[TG];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = p.K, NC = K / 64;
    constexpr int CS = 64 * TG + 16;      // bytes per chunk of all token rows in LDS
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * TG;
    const int mt = static_cast<int>(p.M - t0 < TG ? p.M - t0 : TG);
    const bool cap_blk = blockIdx.x == 0;

    // ---------------------------------------------------------------- weight rows
    const int slot = lane / LPR, j = lane % LPR;
    const int r = blockIdx.x * (NW * RPW) + wave * RPW + slot;
    const bool rvalid = r < p.rows_total;
    int sg = 0, n = r;
    if constexpr (EPI != EPI_GLU) {
        while (sg + 1 < p.nseg && n >= p.seg[sg].n) { n -= p.seg[sg].n; ++sg; }
        // segment boundaries are multiples of the 4 rows of a wave (checked at launch), so the
        // segment is wave-uniform and its fields come from scalar loads
        sg = __builtin_amdgcn_readfirstlane(sg);
    }
    const int nn = rvalid ? n : 0;
    const uint32_t *w0 = p.seg[sg].packed + static_cast<int64_t>(nn) * (K / 16);
    const uint32_t *w1 = EPI == EPI_GLU ? p.seg[1].packed + static_cast<int64_t>(nn) * (K / 16) : nullptr;
    // One token: its activation row (bf16 to quantize, or pre-quantized codes) is requested
    // before the weights.  Loads return in issue order, so a row fetched after the weights
    // could only be quantized once every weight chunk had arrived; fetched first, the
    // quantization overlaps the weight latency.  The weight and residual loads after it are
    // unconditional (clamped addresses, unused values masked), which keeps the wait for the
    // row exact.
    constexpr bool EARLY = TG == 1 && XIN != 1;
    constexpr int KEEP = TG == 1 ? (NW == 8 ? 4 : 3) : 0;
    const bool keep = KEEP > 0 && K <= 8 * NT * KEEP;      // bf16 row held in registers
    const bool qearly = EARLY && XIN == 0 && K <= 32 * NT;  // code row held in registers
    uint4 xr[EARLY && XIN == 2 ? KEEP : 1];
    uint4 qr[2];
    // (requested whether or not the row fits the registers: clamped, in bounds, and unused
    // when it does not; a conditional load here would make the compiler park it in scratch)
    if constexpr (EARLY && XIN == 2) {
#pragma unroll
        for (int it = 0; it < KEEP; ++it) {
            const int k0 = tid * 8 + 8 * NT * it;
            xr[it] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + t0 * K + (k0 < K ? k0 : K - 8));
        }
    }
    // one MLGRU step (XIN 3): the token's i, f, g pre-activations, carried state, forget-gate
    // bias and g_norm gain for this thread's KF groups of 8 channels
    constexpr int KF = XIN == 3 ? (NI <= 2 ? 1 : 2) : 1;
    using RawAct = typename std::conditional<OUT_BF16, uint4, float4[2]>::type;
    RawAct ri[KF], rf[KF], rg[KF];
    float4 rh[KF][2], rb[KF][2], rl[KF][2], rw[KF][2];
    if constexpr (XIN == 3) {
        auto ld_act = [&](int64_t e, RawAct &dst) __attribute__((always_inline)) {
            if constexpr (OUT_BF16) {
                dst = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + e);
            } else {
                dst[0] = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.x) + e);
                dst[1] = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.x) + e + 4);
            }
        };
        auto ld_par = [&](const float *src, int k, float4 (&dst)[2], float dflt) __attribute__((always_inline)) {
            if (src) {
                dst[0] = *reinterpret_cast<const float4 *>(src + k);
                dst[1] = *reinterpret_cast<const float4 *>(src + k + 4);
            } else {
                dst[0] = dst[1] = make_float4(dflt, dflt, dflt, dflt);
            }
        };
#pragma unroll
        for (int it = 0; it < KF; ++it) {
            int k0 = tid * 8 + 8 * NT * it;
            k0 = k0 < K ? k0 : K - 8;
            const int64_t base = t0 * 3 * static_cast<int64_t>(K) + k0;
            ld_act(base, ri[it]);
            ld_act(base + K, rf[it]);
            ld_act(base + 2 * K, rg[it]);
            ld_par(p.h_prev ? p.h_prev + t0 * K : nullptr, k0, rh[it], 0.0f);
            ld_par(p.f_bias, k0, rb[it], 0.0f);
            ld_par(p.f_lower, k0, rl[it], 0.0f);
            ld_par(p.gnorm_w, k0, rw[it], 1.0f);
        }
    }
    float a_early = 0.f;
    int rs_early = 0;
    if constexpr (EARLY && XIN == 0) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int k0 = tid * 16 + 16 * NT * it;
            qr[it] = *reinterpret_cast<const uint4 *>(p.q + t0 * K + (k0 < K ? k0 : K - 16));
        }
        a_early = p.a[t0];
        rs_early = p.rowsum[t0];
    }
    if constexpr (EARLY) __builtin_amdgcn_sched_barrier(0);
    uint4 wa[NI], wb[NI];
    auto load_pass = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if constexpr (EARLY) {
                // every slot is requested (slots past the row end re-read its last chunk)
                int c = base + j + LPR * i;
                c = c < NC ? c : NC - 1;
                wa[i] = *reinterpret_cast<const uint4 *>(w0 + c * 4);
                if constexpr (EPI == EPI_GLU) wb[i] = *reinterpret_cast<const uint4 *>(w1 + c * 4);
            } else {
                const int c = base + j + LPR * i;
                if (c < NC && rvalid) {
                    wa[i] = *reinterpret_cast<const uint4 *>(w0 + c * 4);
                    if constexpr (EPI == EPI_GLU) wb[i] = *reinterpret_cast<const uint4 *>(w1 + c * 4);
                }
            }
        }
    };
    load_pass(0);  // the first pass of weights is in flight during the prologue
    // residual of this lane's output (lane j of a row writes token j / (16 / TG)), requested
    // now so that its latency overlaps the rest of the kernel
    constexpr int STRIDE = LPR / TG;
    const int tj = j / STRIDE;
    float resid_v = 0.f;
    if constexpr (EPI == EPI_RESID) {
        if constexpr (EARLY) {
            resid_v = load_act<OUT_BF16>(p.resid, t0 * p.ldr + p.seg[sg].out_col0 + nn);
        } else {
            if (rvalid && j % STRIDE == 0 && tj < mt)
                resid_v = load_act<OUT_BF16>(p.resid, (t0 + tj) * p.ldr + p.seg[sg].out_col0 + n);
        }
    }
    if constexpr (EARLY) __builtin_amdgcn_sched_barrier(0);

    // ---------------------------------------------------------------- prologue
    if constexpr (XIN != 0) {
        // two straight-line passes over all TG token slots (slots past the group end read
        // the group's last row and are never stored), so the loads of every token are in
        // flight together
        constexpr bool BF = XIN == 2;
        float pm[TG], ps[TG];
        // one token: its row (<= KEEP x 8 values per thread) stays in registers between the
        // two passes
        float xk[KEEP > 0 ? KEEP : 1][8];
        if constexpr (XIN == 3) {
            // DataCamp "MatMul-free language models", "Core components: MLGRU and GLU";
            // Hysen Labs "MatMul-Free LM", "HGRN attention" (g_norm):
            //   f = sigmoid(f_pre + b_f), h_t = f*h_{t-1} + (1-f)*SiLU(i_pre),
            //   o = RMSNorm_D(h_t)*gnorm_w * g*sigmoid(g)  (gate mode 1: sigmoid(g)*h_t);
            // o is then quantized below as o_proj's input.  Workgroup 0 writes h_t.
            auto cvt8 = [&](const RawAct &r, float (&v)[8]) __attribute__((always_inline)) {
                if constexpr (OUT_BF16) {
                    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] = __uint_as_float(w[e] << 16);
                        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                    }
                } else {
                    v[0] = r[0].x; v[1] = r[0].y; v[2] = r[0].z; v[3] = r[0].w;
                    v[4] = r[1].x; v[5] = r[1].y; v[6] = r[1].z; v[7] = r[1].w;
                }
            };
            auto f8 = [](const float4 (&r)[2], float (&v)[8]) __attribute__((always_inline)) {
                v[0] = r[0].x; v[1] = r[0].y; v[2] = r[0].z; v[3] = r[0].w;
                v[4] = r[1].x; v[5] = r[1].y; v[6] = r[1].z; v[7] = r[1].w;
            };
            float hsum[1] = {0.f};
#pragma unroll
            for (int it = 0; it < KF; ++it) {
                const int k0 = tid * 8 + 8 * NT * it;
                float iv[8], fv[8], hv[8], bv[8], lv[8];
                cvt8(ri[it], iv);
                cvt8(rf[it], fv);
                f8(rh[it], hv);
                f8(rb[it], bv);
                f8(rl[it], lv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = fmaf(1.0f - lv[e], sigmoidf_(fv[e] + bv[e]), lv[e]);
                    hv[e] = f * hv[e] + (1.0f - f) * siluf_(iv[e]);
                }
                if (k0 < K) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        hsum[0] = fmaf(hv[e], hv[e], hsum[0]);
                        xk[it][e] = hv[e];
                    }
                    if (blockIdx.x == 0 && p.h_new) {
                        float *hd = p.h_new + t0 * K + k0;
                        *reinterpret_cast<float4 *>(hd) = make_float4(hv[0], hv[1], hv[2], hv[3]);
                        *reinterpret_cast<float4 *>(hd + 4) = make_float4(hv[4], hv[5], hv[6], hv[7]);
                    }
                }
            }
            const float hw = wave_reduce_multi<1, false>(hsum);
            if (lane == 0) red_h[wave] = hw;
            __syncthreads();
            float htot = red_h[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) htot += red_h[w];
            const float r = 1.0f / sqrtf(htot * (1.0f / static_cast<float>(K)) + p.g_eps);
#pragma unroll
            for (int it = 0; it < KF; ++it) {
                const int k0 = tid * 8 + 8 * NT * it;
                if (k0 < K) {
                    float gv[8], gw[8];
                    cvt8(rg[it], gv);
                    f8(rw[it], gw);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        xk[it][e] = p.gate_mode == 0 ? xk[it][e] * r * gw[e] * siluf_(gv[e])
                                                     : sigmoidf_(gv[e]) * xk[it][e];
                    // g_norm's output is materialised in the activation dtype before it is
                    // quantized as o_proj's input
                    if constexpr (OUT_BF16) {
#pragma unroll
                        for (int e = 0; e < 8; e += 2) round_bf16_pair(xk[it][e], xk[it][e + 1]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            const int64_t tok = t0 + (t < mt ? t : mt - 1);
            pm[t] = 0.f;
            ps[t] = 0.f;
            if (keep) {
#pragma unroll
                for (int it = 0; it < KEEP; ++it) {
                    const int k0 = tid * 8 + 8 * NT * it;
                    if (k0 < K) {
                        if constexpr (XIN == 3) {
                            // xk holds the gated MLGRU output
                        } else if constexpr (EARLY) {
                            const uint32_t w[4] = {xr[it].x, xr[it].y, xr[it].z, xr[it].w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                xk[it][2 * e] = __uint_as_float(w[e] << 16);
                                xk[it][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                            }
                        } else {
                            load8v<BF>(p.x, tok * K + k0, xk[it]);
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float pj = p.gamma ? xk[it][e] * p.gamma[k0 + e] : xk[it][e];
                            pm[t] = fmaxf(pm[t], fabsf(pj));
                            ps[t] += xk[it][e] * xk[it][e];
                        }
                    }
                }
                continue;
            }
            for (int k0 = tid * 8; k0 < K; k0 += 8 * NT) {
                float v[8];
                load8v<BF>(p.x, tok * K + k0, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pj = p.gamma ? v[e] * p.gamma[k0 + e] : v[e];
                    pm[t] = fmaxf(pm[t], fabsf(pj));
                    ps[t] += v[e] * v[e];
                }
            }
        }
        {
            constexpr int SH = 6 - (TG == 1 ? 0 : TG == 4 ? 2 : TG == 8 ? 3 : 4);
            const float rm = wave_reduce_multi<TG, true>(pm);
            const float rs = wave_reduce_multi<TG, false>(ps);
            if ((lane & ((1 << SH) - 1)) == 0) {
                red_m[wave][lane >> SH] = rm;
                red_s[wave][lane >> SH] = rs;
            }
        }
        __syncthreads();
        float sc[TG];
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            float mx = red_m[0][t];
#pragma unroll
            for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red_m[w][t]);
            sc[t] = 127.0f / fmaxf(mx, 1e-5f);
        }
        const bool cap_any = cap_blk && (p.cap.x_in || p.cap.q) && p.cap.row0 < t0 + mt && t0 < p.cap.row1;
        int qsum[TG];  // this thread's share of each token's code sum
#pragma unroll
        for (int t = 0; t < TG; ++t) qsum[t] = 0;
        auto quant8 = [&](int t, int k0, const float (&v)[8]) __attribute__((always_inline)) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pj = p.gamma ? v[e] * p.gamma[k0 + e] : v[e];
                float rq = rintf(pj * sc[t]);
                rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                if constexpr (UNS) qsum[t] += static_cast<int>(rq);
                const uint32_t byte = static_cast<uint32_t>(static_cast<int>(rq)) & 0xFFu;
                if (e < 4) lo |= byte << (8 * e);
                else hi |= byte << (8 * (e - 4));
            }
            *reinterpret_cast<uint2 *>(qs + (k0 >> 6) * CS + 64 * t + (k0 & 63)) = make_uint2(lo, hi);
            const int64_t tok = t0 + t;
            if (cap_any && t < mt && p.cap.row0 <= tok && tok < p.cap.row1) {  // test protocol
                const int64_t cr = tok - p.cap.row0;
                if (p.cap.x_in)
#pragma unroll
                    for (int e = 0; e < 8; ++e) p.cap.x_in[cr * K + k0 + e] = v[e];
                if (p.cap.q) *reinterpret_cast<uint2 *>(p.cap.q + cr * K + k0) = make_uint2(lo, hi);
            }
        };
        if (keep) {
#pragma unroll
            for (int it = 0; it < KEEP; ++it) {
                const int k0 = tid * 8 + 8 * NT * it;
                if (k0 < K) quant8(0, k0, xk[it]);
            }
        } else {
            for (int k0 = tid * 8; k0 < K; k0 += 8 * NT) {
                float v[TG][8];
#pragma unroll
                for (int t = 0; t < TG; ++t) load8v<BF>(p.x, (t0 + (t < mt ? t : mt - 1)) * K + k0, v[t]);
#pragma unroll
                for (int t = 0; t < TG; ++t) quant8(t, k0, v[t]);
            }
        }
        if constexpr (UNS) {
            // code sums: reduced here, summed over the waves after the barrier below
            constexpr int SH = 6 - (TG == 1 ? 0 : TG == 4 ? 2 : TG == 8 ? 3 : 4);
            const int rq = wave_reduce_multi<TG, false, int>(qsum);
            if ((lane & ((1 << SH) - 1)) == 0) red_q[wave][lane >> SH] = rq;
        }
        if (tid < mt) {
            const int t = tid;
            float mx = red_m[0][t], ss = red_s[0][t];
#pragma unroll
            for (int w = 1; w < NW; ++w) { mx = fmaxf(mx, red_m[w][t]); ss += red_s[w][t]; }
            const float me = fmaxf(mx, 1e-5f);
            s_a[t] = me / 127.0f * (1.0f / sqrtf(ss / static_cast<float>(K) + p.eps));
            const int64_t tok = t0 + t;
            if (cap_blk && p.cap.a && p.cap.row0 <= tok && tok < p.cap.row1) p.cap.a[tok - p.cap.row0] = s_a[t];
        }
    } else {
        if (qearly) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int k0 = tid * 16 + 16 * NT * it;
                // stored field by field: a whole-struct copy keeps qr in scratch memory
                if (k0 < K)
                    *reinterpret_cast<uint4 *>(qs + (k0 >> 6) * CS + (k0 & 63)) =
                        make_uint4(qr[it].x, qr[it].y, qr[it].z, qr[it].w);
            }
        } else for (int k0 = tid * 16; k0 < K; k0 += 16 * NT) {
            uint4 v[TG];  // every token's 16 bytes requested before any is stored
#pragma unroll
            for (int t = 0; t < TG; ++t)
                v[t] = *reinterpret_cast<const uint4 *>(p.q + (t0 + (t < mt ? t : mt - 1)) * K + k0);
#pragma unroll
            for (int t = 0; t < TG; ++t) *reinterpret_cast<uint4 *>(qs + (k0 >> 6) * CS + 64 * t + (k0 & 63)) = v[t];
        }
        if (tid < mt) {
            s_a[tid] = EARLY ? a_early : p.a[t0 + tid];
            s_rs[tid] = EARLY ? rs_early : p.rowsum[t0 + tid];
        }
    }
    __syncthreads();
    if constexpr (XIN != 0 && UNS) {
        if (tid < mt) {
            int q = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) q += red_q[w][tid];
            s_rs[tid] = q;
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- dot products
    int acc0[TG], acc1[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) { acc0[t] = 0; acc1[t] = 0; }
    for (int base = 0; base < NC; base += LPR * NI) {
        if (base > 0) load_pass(base);
        const int niter = (NC - base + LPR - 1) / LPR;  // chunk slots in use (uniform)
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (i >= niter) break;
            // chunk slots past the row end read as weight 0 against chunk 0 and add nothing
            const int c = base + j + LPR * i;
            const bool cv = c < NC && rvalid;
            const uint32_t z = UNS ? 0u : 0x55555555u;  // a zero contribution either way
            auto codes = [&](uint32_t w) __attribute__((always_inline)) {
                return UNS ? unpack_codes(w) : signed_codes(w);
            };
            const v4i ca[4] = {codes(cv ? wa[i].x : z), codes(cv ? wa[i].y : z),
                               codes(cv ? wa[i].z : z), codes(cv ? wa[i].w : z)};
            v4i cb[4];
            if constexpr (EPI == EPI_GLU) {
                cb[0] = codes(cv ? wb[i].x : z); cb[1] = codes(cv ? wb[i].y : z);
                cb[2] = codes(cv ? wb[i].z : z); cb[3] = codes(cv ? wb[i].w : z);
            }
            const int8_t *qc = qs + (cv ? c : 0) * CS;
            // every token slot is multiplied (slots past the group end hold stale values and
            // their sums are never stored), so the loop has no token-dependent branches; the
            // activations of up to 4 tokens are read before their dot products
            constexpr int TB = TG < 4 ? TG : 4;
#pragma unroll
            for (int t0b = 0; t0b < TG; t0b += TB) {
                v4i qv[TB][4];
#pragma unroll
                for (int u = 0; u < TB; ++u) {
                    const v4i *qp = reinterpret_cast<const v4i *>(qc + 64 * (t0b + u));
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) qv[u][q4] = qp[q4];
                }
#pragma unroll
                for (int u = 0; u < TB; ++u) {
                    acc0[t0b + u] = dot16(qv[u], ca, acc0[t0b + u]);
                    if constexpr (EPI == EPI_GLU) acc1[t0b + u] = dot16(qv[u], cb, acc1[t0b + u]);
                }
            }
        }
    }
    // the 16 partial sums of the row, for every token at once: lane j of the row ends with
    // token j / (16 / TG)
    int my0 = wave_reduce_multi<TG, false, int, LPR>(acc0);
    int my1 = 0;
    if constexpr (EPI == EPI_GLU) my1 = wave_reduce_multi<TG, false, int, LPR>(acc1);
    if (p.copy_n > 0 && blockIdx.y == 0) {  // side copy (after the weights are consumed)
        const int64_t i = (static_cast<int64_t>(blockIdx.x) * NT + tid) * 4;
        if (i < p.copy_n)
            *reinterpret_cast<float4 *>(p.copy_dst + i) = *reinterpret_cast<const float4 *>(p.copy_src + i);
    }
    if (!rvalid || j % STRIDE != 0) return;
    if (tj >= mt) return;
    if constexpr (UNS) {
        my0 -= s_rs[tj];
        if constexpr (EPI == EPI_GLU) my1 -= s_rs[tj];
    }
    const int64_t tok = t0 + tj;
    const float at = s_a[tj];
    const bool capr = p.cap.row0 <= tok && tok < p.cap.row1;
    const int64_t crow = tok - p.cap.row0;
    if constexpr (EPI == EPI_GLU) {
        float yg = static_cast<float>(my0) * (p.seg[0].scale * at);
        float yu = static_cast<float>(my1) * (p.seg[1].scale * at);
        if (p.seg[0].bias) yg += p.seg[0].bias[n];
        if (p.seg[1].bias) yu += p.seg[1].bias[n];
        const float mv = siluf_(yg) * yu;
        store_act<OUT_BF16>(p.out, tok * p.ldo + n, mv);
        if (capr) {
            if (p.cap.acc) {
                int32_t *cp = p.cap.acc + crow * p.cap.acc_ld;
                cp[p.seg[0].cap_col0 + n] = my0;
                cp[p.seg[1].cap_col0 + n] = my1;
            }
            if (p.cap.y_out) p.cap.y_out[crow * p.ldo + n] = OUT_BF16 ? round_to_bf16(mv) : mv;
        }
    } else {
        const Seg &S = p.seg[sg];
        float y = static_cast<float>(my0) * (S.scale * at);
        if (S.bias) y += S.bias[n];
        if constexpr (EPI == EPI_RESID) y = resid_v + y;
        store_act<OUT_BF16>(p.out, tok * p.ldo + S.out_col0 + n, y);
        if (capr) {
            if (p.cap.acc) p.cap.acc[crow * p.cap.acc_ld + S.cap_col0 + n] = my0;
            if (p.cap.y_out) p.cap.y_out[crow * p.ldo + S.out_col0 + n] = OUT_BF16 ? round_to_bf16(y) : y;
        }
    }
}

// One token and many weight rows (the LM head, larger matrices): a grid of a few workgroups
// per CU quantizes the activation row once into LDS and then streams blocks of 16 rows,
// requesting the next block's weights before the current block's dot products, so the
// prologue is paid once per workgroup instead of once per 16 rows and every workgroup keeps
// two blocks of weights in flight.  Same arithmetic as the kernel above (one token, bf16
// activations, plain store epilogue, one segment); the codes are multiplied unmapped and
// the row's code sum is subtracted once per output.
template <bool OUT_BF16, int NI>
__global__ __launch_bounds__(256) void gemv_stream_kernel(GemvArgs p) {
    constexpr int NW = 4, NT = 64 * NW, RB = NW * RPW;  // 16 rows per block
    constexpr int NS = (NI + 1) / 2;                    // 8-value slices of the row per thread
    constexpr int CS = 64 + 16;                         // LDS bytes per 64-k chunk
    extern __shared__ __attribute__((aligned(16))) int8_t qs[];
    __shared__ float red_m[NW], red_s[NW];
    __shared__ int red_q[NW];
    __shared__ float s_a;
    __shared__ int s_rs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = lane / LPR, j = lane % LPR;
    const int K = p.K, NC = K / 64;
    const int nrb = (p.rows_total + RB - 1) / RB;
    const Seg &S0 = p.seg[0];

    // the activation row is requested first (loads return in issue order)
    uint4 xr[NS];
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
        const int k0 = tid * 8 + 8 * NT * s4;
        xr[s4] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + (k0 < K ? k0 : K - 8));
    }
    // a block's weights: every slot requested (rows and chunks past the end clamped)
    auto wload = [&](int rb, uint4 (&w)[NI]) __attribute__((always_inline)) {
        int r = rb * RB + wave * RPW + slot;
        r = r < p.rows_total ? r : p.rows_total - 1;
        const uint32_t *wr = S0.packed + static_cast<int64_t>(r) * (K / 16);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            int c = j + LPR * i;
            c = c < NC ? c : NC - 1;
            w[i] = *reinterpret_cast<const uint4 *>(wr + c * 4);
        }
    };
    uint4 wa[NI], wb[NI];
    int rb = blockIdx.x;
    wload(rb, wa);
    __builtin_amdgcn_sched_barrier(0);

    // prologue: RMS/absmax quantization of the row into LDS (the quantizer's arithmetic)
    float xv[NS][8];
    float pm[1] = {0.f}, ps[1] = {0.f};
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
        const int k0 = tid * 8 + 8 * NT * s4;
        bf16x8_to_f32(xr[s4], xv[s4]);
        if (k0 < K) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pj = p.gamma ? xv[s4][e] * p.gamma[k0 + e] : xv[s4][e];
                pm[0] = fmaxf(pm[0], fabsf(pj));
                ps[0] += xv[s4][e] * xv[s4][e];
            }
        }
    }
    {
        const float rm = wave_reduce_multi<1, true>(pm);
        const float rs = wave_reduce_multi<1, false>(ps);
        if (lane == 0) {
            red_m[wave] = rm;
            red_s[wave] = rs;
        }
    }
    __syncthreads();
    float mx = red_m[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red_m[w]);
    const float sc = 127.0f / fmaxf(mx, 1e-5f);
    const bool cap0 = blockIdx.x == 0 && p.cap.row0 <= 0 && 0 < p.cap.row1;
    int qsum[1] = {0};  // the row's code sum: codes are multiplied unmapped (c = q_w + 1)
#pragma unroll
    for (int s4 = 0; s4 < NS; ++s4) {
        const int k0 = tid * 8 + 8 * NT * s4;
        if (k0 < K) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pj = p.gamma ? xv[s4][e] * p.gamma[k0 + e] : xv[s4][e];
                float rq = rintf(pj * sc);
                rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                qsum[0] += static_cast<int>(rq);
                const uint32_t byte = static_cast<uint32_t>(static_cast<int>(rq)) & 0xFFu;
                if (e < 4) lo |= byte << (8 * e);
                else hi |= byte << (8 * (e - 4));
            }
            *reinterpret_cast<uint2 *>(qs + (k0 >> 6) * CS + (k0 & 63)) = make_uint2(lo, hi);
            if (cap0) {  // test protocol
                const int64_t cr = -p.cap.row0;
                if (p.cap.x_in)
#pragma unroll
                    for (int e = 0; e < 8; ++e) p.cap.x_in[cr * K + k0 + e] = xv[s4][e];
                if (p.cap.q) *reinterpret_cast<uint2 *>(p.cap.q + cr * K + k0) = make_uint2(lo, hi);
            }
        }
    }
    {
        const int rq = wave_reduce_multi<1, false, int>(qsum);
        if (lane == 0) red_q[wave] = rq;
    }
    __syncthreads();
    if (tid == 0) {
        float ss = red_s[0];
        int qt = red_q[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            ss += red_s[w];
            qt += red_q[w];
        }
        const float me = fmaxf(mx, 1e-5f);
        s_a = me / 127.0f * (1.0f / sqrtf(ss / static_cast<float>(K) + p.eps));
        s_rs = qt;
        if (cap0 && p.cap.a) p.cap.a[-p.cap.row0] = s_a;
    }
    __syncthreads();
    const float at = s_a;
    const int row_sum = s_rs;

    // dot products of one block against the LDS-resident codes, 16-lane reduction, store
    auto block = [&](int rbk, const uint4 (&w)[NI]) __attribute__((always_inline)) {
        const int r = rbk * RB + wave * RPW + slot;
        int acc[1] = {0};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int c = j + LPR * i;
            const bool cv = c < NC;
            // chunks past the row end (clamped re-reads) count as code 0
            const v4i ca[4] = {unpack_codes(cv ? w[i].x : 0u), unpack_codes(cv ? w[i].y : 0u),
                               unpack_codes(cv ? w[i].z : 0u), unpack_codes(cv ? w[i].w : 0u)};
            const v4i *qp = reinterpret_cast<const v4i *>(qs + (cv ? c : 0) * CS);
            const v4i qv[4] = {qp[0], qp[1], qp[2], qp[3]};
            acc[0] = dot16(qv, ca, acc[0]);
        }
        const int tot = wave_reduce_multi<1, false, int, LPR>(acc) - row_sum;
        if (r < p.rows_total && j == 0) {
            float y = static_cast<float>(tot) * (S0.scale * at);
            if (S0.bias) y += S0.bias[r];
            store_act<OUT_BF16>(p.out, S0.out_col0 + r, y);
            if (p.cap.row0 <= 0 && 0 < p.cap.row1) {
                const int64_t cr = -p.cap.row0;
                if (p.cap.acc) p.cap.acc[cr * p.cap.acc_ld + S0.cap_col0 + r] = tot;
                if (p.cap.y_out) p.cap.y_out[cr * p.ldo + S0.out_col0 + r] = OUT_BF16 ? round_to_bf16(y) : y;
            }
        }
    };
    // two register sets of weights: the next block (or, past the end, the current one again)
    // is requested unconditionally before the current block is multiplied
    while (true) {
        const int rn = rb + static_cast<int>(gridDim.x);
        wload(rn < nrb ? rn : rb, wb);
        block(rb, wa);
        rb = rn;
        if (rb >= nrb) break;
        const int rn2 = rb + static_cast<int>(gridDim.x);
        wload(rn2 < nrb ? rn2 : rb, wa);
        block(rb, wb);
        rb = rn2;
        if (rb >= nrb) break;
    }
}

template <bool OUT_BF16>
void launch_stream(const GemvArgs &a, size_t lds, unsigned grid, hipStream_t s) {
    const int groups = (a.K / 64 + LPR - 1) / LPR;
    if (groups <= 1) hipLaunchKernelGGL((gemv_stream_kernel<OUT_BF16, 1>), dim3(grid), dim3(256), lds, s, a);
    else if (groups <= 2) hipLaunchKernelGGL((gemv_stream_kernel<OUT_BF16, 2>), dim3(grid), dim3(256), lds, s, a);
    else if (groups <= 4) hipLaunchKernelGGL((gemv_stream_kernel<OUT_BF16, 4>), dim3(grid), dim3(256), lds, s, a);
    else if (groups <= 6) hipLaunchKernelGGL((gemv_stream_kernel<OUT_BF16, 6>), dim3(grid), dim3(256), lds, s, a);
    else hipLaunchKernelGGL((gemv_stream_kernel<OUT_BF16, 8>), dim3(grid), dim3(256), lds, s, a);
}

template <int EPI, int XIN, int TG, int NW, int NI>
void launch5(const GemvArgs &a, size_t lds, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((a.rows_total + NW * RPW - 1) / (NW * RPW)),
                    static_cast<unsigned>((a.M + TG - 1) / TG));
    if (a.out_bf16) hipLaunchKernelGGL((gemv_dot4_kernel<EPI, XIN, true, TG, NW, NI>), grid, dim3(64 * NW), lds, s, a);
    else hipLaunchKernelGGL((gemv_dot4_kernel<EPI, XIN, false, TG, NW, NI>), grid, dim3(64 * NW), lds, s, a);
}

template <int EPI, int XIN, int TG>
void launch4(const GemvArgs &a, size_t lds, hipStream_t s) {
    if constexpr (TG == 1) {
        if (a.K >= 8192) {
            launch5<EPI, XIN, TG, 8, CB>(a, lds, s);
            return;
        }
        // one pass (K < 8192): chunks per lane = ceil(K / 64 / 16)
        const int groups = (a.K / 64 + LPR - 1) / LPR;
        if (groups <= 1) launch5<EPI, XIN, TG, 4, 1>(a, lds, s);
        else if (groups <= 2) launch5<EPI, XIN, TG, 4, 2>(a, lds, s);
        else if (groups <= 4) launch5<EPI, XIN, TG, 4, 4>(a, lds, s);
        else if (groups <= 6) launch5<EPI, XIN, TG, 4, 6>(a, lds, s);
        else launch5<EPI, XIN, TG, 4, CB>(a, lds, s);
        return;
    }
    launch5<EPI, XIN, TG, 4, CB>(a, lds, s);
}

template <int EPI, int XIN>
void launch3(const GemvArgs &a, size_t lds, hipStream_t s) {
    switch (a.tokens_per_group) {
        case 1: launch4<EPI, XIN, 1>(a, lds, s); break;
        case 4: launch4<EPI, XIN, 4>(a, lds, s); break;
        case 8: launch4<EPI, XIN, 8>(a, lds, s); break;
        default: launch4<EPI, XIN, 16>(a, lds, s); break;
    }
}

template <int EPI>
void launch2(const GemvArgs &a, size_t lds, hipStream_t s) {
    if constexpr (EPI == EPI_RESID) {
        if (a.mlgru) {  // one token per grid row (sequence), K <= 4096 (checked by launch_gemv): 1, 2 or 4 chunks per lane
            const int groups = (a.K / 64 + LPR - 1) / LPR;
            if (groups <= 1) launch5<EPI, 3, 1, 4, 1>(a, lds, s);
            else if (groups <= 2) launch5<EPI, 3, 1, 4, 2>(a, lds, s);
            else launch5<EPI, 3, 1, 4, 4>(a, lds, s);
            return;
        }
    }
    if (!a.x) launch3<EPI, 0>(a, lds, s);
    else if (a.x_bf16) launch3<EPI, 2>(a, lds, s);
    else launch3<EPI, 1>(a, lds, s);
}

}  // namespace

// Bytes of LDS for tg token rows of length K.
size_t gemv_lds_bytes(int K, int tg) { return static_cast<size_t>(K / 64) * chunk_stride(tg); }

hipError_t launch_gemv(const GemvArgs &a_in, hipStream_t s) {
    if (a_in.M <= 0) return hipSuccess;
    if (a_in.epi != EPI_GLU)
        for (int i = 0; i + 1 < a_in.nseg; ++i)
            if (a_in.seg[i].n % RPW != 0) return hipErrorInvalidValue;  // segment not wave-aligned
    if (a_in.mlgru && (a_in.epi != EPI_RESID || a_in.M > 4 || a_in.K > 4096 || !a_in.x ||
                       a_in.x_bf16 != a_in.out_bf16))
        return hipErrorInvalidValue;  // the fused MLGRU step: one token per grid row, <= 4 rows, D <= 4096
    // the side copy: 4 floats per thread of grid row 0, at least 16 threads per weight row
    if (a_in.copy_n % 4 != 0 || a_in.copy_n > 64LL * a_in.rows_total) return hipErrorInvalidValue;
    GemvArgs a = a_in;
    if (a.M == 1 && a.epi == EPI_STORE && a.nseg == 1 && a.x && a.x_bf16 && !a.mlgru &&
        a.copy_n == 0 && a.K <= 8192 && a.rows_total >= kStreamRows) {
        // one token, many rows: persistent streaming over 16-row blocks, 2 workgroups per CU
        static const int cus = [] {
            int dev = 0, n = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
                n = 256;
            return n;
        }();
        const int nrb = (a.rows_total + 15) / 16;
        const unsigned grid = static_cast<unsigned>(nrb < 2 * cus ? nrb : 2 * cus);
        a.tokens_per_group = 1;
        timing_begin(FAM_GEMV, s);
        if (a.out_bf16) launch_stream<true>(a, gemv_lds_bytes(a.K, 1), grid, s);
        else launch_stream<false>(a, gemv_lds_bytes(a.K, 1), grid, s);
        timing_end(FAM_GEMV, s);
        return hipGetLastError();
    }
    // token rows per workgroup: up to 4 rows, one per row of the grid (each token takes the
    // one-token kernel with its early activation fetch; the weight rows it re-reads for the
    // next token come from the same XCD's L2); above, groups of 8 or 16 rows within 64 KB of
    // LDS (reached when the decode regime is forced; by default the k-split MFMA kernel runs)
    int tg = a.M <= 4 ? 1 : a.M <= 8 ? 8 : 16;
    while (tg > 1 && gemv_lds_bytes(a.K, tg) > 64 * 1024) tg = tg == 16 ? 8 : tg == 8 ? 4 : 1;
    a.tokens_per_group = tg;
    const size_t lds = gemv_lds_bytes(a.K, tg);
    timing_begin(FAM_GEMV, s);
    switch (a.epi) {
        case EPI_STORE: launch2<EPI_STORE>(a, lds, s); break;
        case EPI_RESID: launch2<EPI_RESID>(a, lds, s); break;
        default: launch2<EPI_GLU>(a, lds, s); break;
    }
    timing_end(FAM_GEMV, s);
    return hipGetLastError();
}

}  // namespace mmf
