// scan.hip -- MLGRU token mixer for gfx950: fused gates, chunked time-parallel scan,
// RMSNorm-swish output gate and (optionally) the int8 quantization of o_proj's input.
//
// DataCamp "MatMul-free language models", section "Core components: MLGRU and GLU": the
// hidden state carries memory from token to token and gates in (0,1) decide what flows.
// Hysen Labs "MatMul-Free LM", section "HGRN attention": the recurrence needs only the
// current token and the previous state (linear in T); its output passes g_norm, an RMSNorm
// fused with a swish gate, before o_proj.  Per (b, d):
//   f = lb + (1 - lb)*sigmoid(f_pre + b_f), c = SiLU(i_pre), h_t = f*h_{t-1} + (1-f)*c,
//   o_t = RMSNorm_D(h_t)*gnorm_w * g*sigmoid(g)   (or sigmoid(g)*h_t).
// lb is the optional per-layer lower bound of HGRN's forget gate (0 without one): the same
// page names the Hierarchical Gated Recurrent Network; the bound follows HGRN's design.
//
// The recurrence is elementwise in d, so it is parallel over B*D channels; to fill 256
// CUs at long T it is also chunked over time (16-token chunks):
//   phase 1 (thread per chunk and 4 channels): local scan from 0 -> end state hloc and
//     prod(f);
//   phase 2 (per channel block, 8 runs of chunks composed through LDS): carry across
//     chunks, h_in[c+1] = prod_c*h_in[c] + hloc_c;
//   phase 3 (workgroup per chunk, W = D/512 waves per token row, 8 channels per lane):
//     rerun the recurrence from h_in in registers tile by tile, then the per-token RMSNorm
//     over D, the gate and either a store of o or its int8 quantization for o_proj (q, a,
//     row sum); the reductions over D of a tile share one LDS exchange each.
// Phases 1 and 3 read the pre-activations once each and evaluate three sigmoids per
// element; at the 370M shape they are bound by vector ALU issue, not by HBM.  With one
// chunk (decode, short T) phases 1 and 2 are skipped.  Shapes outside the row layout
// (D not a multiple of 64, other chunk lengths) use the channel-quad kernels.
#include "mmf_internal.h"

namespace mmf {

namespace {

// Channels go in quads (4 consecutive d): one 8-byte bf16 or 16-byte fp32 access.
template <bool BF16>
__device__ __forceinline__ float4 load4(const void *p, int64_t i) {
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    }
}

__device__ __forceinline__ float4 ld4f(const float *p) { return *reinterpret_cast<const float4 *>(p); }

// Raw (unconverted) quad of activations: 8 bytes of bf16 or 16 bytes of fp32.
template <bool BF16> struct RawQuad;
template <> struct RawQuad<true> { using T = uint2; };
template <> struct RawQuad<false> { using T = float4; };

template <bool BF16>
__device__ __forceinline__ typename RawQuad<BF16>::T load_raw4(const void *p, int64_t i) {
    if constexpr (BF16) return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
    else return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
}
__device__ __forceinline__ void cvt4(uint2 u, float (&v)[4]) {
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ void cvt4(float4 u, float (&v)[4]) {
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}
__device__ __forceinline__ void st4f(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

// Forget gate with HGRN's per-layer lower bound lb (0 without one; fma(1, s, 0) = s, so the
// unbounded gate is unchanged): f = lb + (1 - lb)*sigmoid(f_pre + b_f).
__device__ __forceinline__ float gate_step(float h, float ip, float fp, float fb, float lb,
                                           float *f_out) {
    const float f = fmaf(1.0f - lb, sigmoidf_(fp + fb), lb);
    *f_out = f;
    return f * h + (1.0f - f) * siluf_(ip);
}

// Phase 1: thread per (b, chunk, channel quad): local scan from 0 over the chunk.
template <bool BF16>
__global__ __launch_bounds__(256) void scan_local_kernel(ScanArgs p) {
    const int qd = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int D = p.D;
    if (4 * qd >= D) return;
    const int d = 4 * qd;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int nt = static_cast<int>((t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T) - t_beg);
    const float4 fb = p.f_bias ? ld4f(p.f_bias + d) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 lb = p.f_lower ? ld4f(p.f_lower + d) : make_float4(0.f, 0.f, 0.f, 0.f);
    float h[4] = {0.f, 0.f, 0.f, 0.f}, pf[4] = {1.f, 1.f, 1.f, 1.f};
    const float fbv[4] = {fb.x, fb.y, fb.z, fb.w}, lbv[4] = {lb.x, lb.y, lb.z, lb.w};
    const int64_t base = (b * p.T + t_beg) * 3 * D + d;
#pragma unroll 8
    for (int t = 0; t < nt; ++t) {
        const float4 ip = load4<BF16>(p.ifg, base + static_cast<int64_t>(t) * 3 * D);
        const float4 fp = load4<BF16>(p.ifg, base + static_cast<int64_t>(t) * 3 * D + D);
        const float iv[4] = {ip.x, ip.y, ip.z, ip.w}, fv[4] = {fp.x, fp.y, fp.z, fp.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f;
            h[e] = gate_step(h[e], iv[e], fv[e], fbv[e], lbv[e], &f);
            pf[e] *= f;
        }
    }
    const int64_t o = (b * p.n_chunks + c) * D + d;
    st4f(p.hloc + o, make_float4(h[0], h[1], h[2], h[3]));
    st4f(p.pf + o, make_float4(pf[0], pf[1], pf[2], pf[3]));
}

// Phase 2: thread per (b, channel): carry across chunks (loads batched ahead of the chain).
__global__ __launch_bounds__(256) void scan_carry_kernel(ScanArgs p) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    const int64_t b = blockIdx.y;
    if (d >= p.D) return;
    const int D = p.D;
    float carry = p.h0 ? p.h0[b * D + d] : 0.0f;
    constexpr int U = 16;
    for (int c0 = 0; c0 < p.n_chunks; c0 += U) {
        float pf[U], hl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u < p.n_chunks ? c0 + u : p.n_chunks - 1;
            const int64_t o = (b * p.n_chunks + c) * D + d;
            pf[u] = p.pf[o];
            hl[u] = p.hloc[o];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c < p.n_chunks) {
                p.hin[(b * p.n_chunks + c) * D + d] = carry;
                carry = pf[u] * carry + hl[u];
            }
        }
    }
}

// Workgroup-wide version: per-wave totals through LDS (red[4][N]); returns all N totals.
template <int N, bool MAX, typename T>
__device__ __forceinline__ void block_reduce_multi(T (&v)[N], T (*red)[N], T (&out)[N]) {
    constexpr int SH = N == 8 ? 3 : 4;  // value index of lane l is l >> SH
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T r = wave_reduce_multi<N, MAX>(v);
    if ((lane & ((1 << SH) - 1)) == 0) red[wave][lane >> SH] = r;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const T a = red[0][i], b = red[1][i], c = red[2][i], d = red[3][i];
        out[i] = MAX ? ((a > b ? a : b) > (c > d ? c : d) ? (a > b ? a : b) : (c > d ? c : d))
                     : (a + b) + (c + d);
    }
}

// Phase 3: workgroup per (b, chunk); each thread owns JQ channel quads (D <= 1024*JQ) and
// walks the chunk in tiles of TS tokens: the recurrence runs in registers, the per-token
// reductions over D (sum h^2; max |p| and sum o^2; sum q) are multi-value wave butterflies
// plus one LDS exchange each, and the next tile's pre-activations are loaded before the
// current tile's reductions.
template <bool IN_BF16, int QUANT, bool OUT_BF16, int JQ, int TS>
__global__ __launch_bounds__(256) void scan_out_kernel(ScanArgs p) {
    __shared__ float red_ss[4][TS], red_mx[4][TS], red_s2[4][TS];
    __shared__ int red_q[4][TS];
    const int c = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = p.D;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int64_t t_end = t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T;
    const float inv_d = 1.0f / static_cast<float>(D);

    float h[JQ][4], fb[JQ][4], lb[JQ][4], gw[JQ][4], qg[JQ][4];
    bool dv[JQ];
#pragma unroll
    for (int j = 0; j < JQ; ++j) {
        const int d = 4 * (tid + 256 * j);
        dv[j] = d < D;
        float4 hv = make_float4(0.f, 0.f, 0.f, 0.f), fv = hv, lv = hv, g1 = make_float4(1.f, 1.f, 1.f, 1.f), q1 = g1;
        if (dv[j]) {
            if (p.n_chunks > 1) hv = ld4f(p.hin + (b * p.n_chunks + c) * D + d);
            else if (p.h0) hv = ld4f(p.h0 + b * D + d);
            if (p.f_bias) fv = ld4f(p.f_bias + d);
            if (p.f_lower) lv = ld4f(p.f_lower + d);
            if (p.gnorm_w) g1 = ld4f(p.gnorm_w + d);
            if (QUANT && p.q_gamma) q1 = ld4f(p.q_gamma + d);
        }
        h[j][0] = hv.x; h[j][1] = hv.y; h[j][2] = hv.z; h[j][3] = hv.w;
        fb[j][0] = fv.x; fb[j][1] = fv.y; fb[j][2] = fv.z; fb[j][3] = fv.w;
        lb[j][0] = lv.x; lb[j][1] = lv.y; lb[j][2] = lv.z; lb[j][3] = lv.w;
        gw[j][0] = g1.x; gw[j][1] = g1.y; gw[j][2] = g1.z; gw[j][3] = g1.w;
        qg[j][0] = q1.x; qg[j][1] = q1.y; qg[j][2] = q1.z; qg[j][3] = q1.w;
    }

    using Raw = typename RawQuad<IN_BF16>::T;
    Raw ip[TS][JQ], fp[TS][JQ], gp[TS][JQ];
    auto fetch = [&](int64_t tt) {
        const int nt = static_cast<int>(t_end - tt < TS ? t_end - tt : TS);
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
            for (int j = 0; j < JQ; ++j) {
                const int d = 4 * (tid + 256 * j);
                if (t < nt && dv[j]) {
                    const int64_t base = (b * p.T + tt + t) * 3 * D + d;
                    ip[t][j] = load_raw4<IN_BF16>(p.ifg, base);
                    fp[t][j] = load_raw4<IN_BF16>(p.ifg, base + D);
                    gp[t][j] = load_raw4<IN_BF16>(p.ifg, base + 2 * D);
                }
            }
    };
    if (t_beg < t_end) fetch(t_beg);

    for (int64_t tt = t_beg; tt < t_end; tt += TS) {
        const int nt = static_cast<int>(t_end - tt < TS ? t_end - tt : TS);
        // ---- recurrence (registers)
        float o[TS][JQ][4], ss[TS];
        Raw gs[TS][JQ];  // g of this tile, kept raw while the next tile is fetched
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            ss[t] = 0.f;
#pragma unroll
            for (int j = 0; j < JQ; ++j) {
                float iv[4], fv[4];
                cvt4(ip[t][j], iv);
                cvt4(fp[t][j], fv);
                gs[t][j] = gp[t][j];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (t < nt && dv[j]) {
                        float f;
                        h[j][e] = gate_step(h[j][e], iv[e], fv[e], fb[j][e], lb[j][e], &f);
                    }
                    o[t][j][e] = h[j][e];
                    ss[t] += (t < nt && dv[j]) ? h[j][e] * h[j][e] : 0.f;
                }
            }
        }
        if (tt + TS < t_end) fetch(tt + TS);  // next tile in flight during the reductions

        // ---- g_norm + gate
        if (p.gate_mode == 0) {
            float tot[TS];
            block_reduce_multi<TS, false>(ss, red_ss, tot);
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const float r = 1.0f / sqrtf(tot[t] * inv_d + p.eps);
#pragma unroll
                for (int j = 0; j < JQ; ++j) {
                    float gv[4];
                    cvt4(gs[t][j], gv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[t][j][e] = o[t][j][e] * r * gw[j][e] * siluf_(gv[e]);
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < TS; ++t)
#pragma unroll
                for (int j = 0; j < JQ; ++j) {
                    float gv[4];
                    cvt4(gs[t][j], gv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[t][j][e] = sigmoidf_(gv[e]) * o[t][j][e];
                }
        }

        if constexpr (QUANT == 0) {
#pragma unroll
            for (int t = 0; t < TS; ++t)
#pragma unroll
                for (int j = 0; j < JQ; ++j) {
                    const int d = 4 * (tid + 256 * j);
                    if (t < nt && dv[j]) {
                        const int64_t oi = (b * p.T + tt + t) * D + d;
                        if constexpr (OUT_BF16) {
                            const uint32_t lo = f32_to_bf16_bits(o[t][j][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(o[t][j][1])) << 16);
                            const uint32_t hi = f32_to_bf16_bits(o[t][j][2]) | (static_cast<uint32_t>(f32_to_bf16_bits(o[t][j][3])) << 16);
                            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + oi) = make_uint2(lo, hi);
                        } else {
                            st4f(static_cast<float *>(p.out) + oi, make_float4(o[t][j][0], o[t][j][1], o[t][j][2], o[t][j][3]));
                        }
                    }
                }
        } else {
            // ---- int8 quantization of o (with o_proj's gain) for o_proj; o is first
            // materialised in the activation dtype, as g_norm's output
            if constexpr (IN_BF16) {
#pragma unroll
                for (int t = 0; t < TS; ++t)
#pragma unroll
                    for (int j = 0; j < JQ; ++j) {
                        round_bf16_pair(o[t][j][0], o[t][j][1]);
                        round_bf16_pair(o[t][j][2], o[t][j][3]);
                    }
            }
            float mx[TS], s2[TS], mxt[TS], s2t[TS];
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                mx[t] = 0.f;
                s2[t] = 0.f;
#pragma unroll
                for (int j = 0; j < JQ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (t < nt && dv[j]) {
                            const float pv = p.q_gamma ? o[t][j][e] * qg[j][e] : o[t][j][e];
                            mx[t] = fmaxf(mx[t], fabsf(pv));
                            s2[t] += o[t][j][e] * o[t][j][e];
                        }
                    }
            }
            {
                const float rm = wave_reduce_multi<TS, true>(mx);
                const float rs = wave_reduce_multi<TS, false>(s2);
                constexpr int SH = TS == 8 ? 3 : 4;
                const int lane = tid & 63, wave = tid >> 6;
                if ((lane & ((1 << SH) - 1)) == 0) {
                    red_mx[wave][lane >> SH] = rm;
                    red_s2[wave][lane >> SH] = rs;
                }
                __syncthreads();
#pragma unroll
                for (int t = 0; t < TS; ++t) {
                    mxt[t] = fmaxf(fmaxf(red_mx[0][t], red_mx[1][t]), fmaxf(red_mx[2][t], red_mx[3][t]));
                    s2t[t] = (red_s2[0][t] + red_s2[1][t]) + (red_s2[2][t] + red_s2[3][t]);
                }
            }
            int qs[TS];
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const float me = fmaxf(mxt[t], 1e-5f);
                const float sc = 127.0f / me;
                const int64_t row = b * p.T + tt + t;
                const bool capr = t < nt && p.cap.row0 <= row && row < p.cap.row1;
                const int64_t cr = row - p.cap.row0;
                qs[t] = 0;
#pragma unroll
                for (int j = 0; j < JQ; ++j) {
                    const int d = 4 * (tid + 256 * j);
                    if (t < nt && dv[j]) {
                        uint32_t packed = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float pv = p.q_gamma ? o[t][j][e] * qg[j][e] : o[t][j][e];
                            float rq = rintf(pv * sc);
                            rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                            const int qi = static_cast<int>(rq);
                            qs[t] += qi;
                            packed |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * e);
                        }
                        *reinterpret_cast<uint32_t *>(p.q + row * D + d) = packed;
                        if (capr) {
                            if (p.cap.x_in) st4f(p.cap.x_in + cr * D + d, make_float4(o[t][j][0], o[t][j][1], o[t][j][2], o[t][j][3]));
                            if (p.cap.q) *reinterpret_cast<uint32_t *>(p.cap.q + cr * D + d) = packed;
                        }
                    }
                }
            }
            int qtot[TS];
            block_reduce_multi<TS, false>(qs, red_q, qtot);
            if (tid < nt) {
                int qv = 0;
                float me = 0.f, s2v = 0.f;
#pragma unroll
                for (int t = 0; t < TS; ++t)
                    if (t == tid) { qv = qtot[t]; me = fmaxf(mxt[t], 1e-5f); s2v = s2t[t]; }
                const int64_t row = b * p.T + tt + tid;
                const float a = me / 127.0f * (1.0f / sqrtf(s2v * inv_d + p.q_eps));
                p.a[row] = a;
                p.rowsum[row] = qv;
                if (p.cap.a && p.cap.row0 <= row && row < p.cap.row1) p.cap.a[row - p.cap.row0] = a;
            }
        }
        __syncthreads();  // the reduction slots are reused by the next tile
    }
    if (c == p.n_chunks - 1 && p.h_out) {
#pragma unroll
        for (int j = 0; j < JQ; ++j) {
            const int d = 4 * (tid + 256 * j);
            if (dv[j]) st4f(p.h_out + b * D + d, make_float4(h[j][0], h[j][1], h[j][2], h[j][3]));
        }
    }
}

template <bool BF16, int CPL> struct RawVec {
    static constexpr int NW = BF16 ? CPL / 2 : CPL;  // 32-bit words
    uint32_t w[NW];
};

template <bool BF16, int CPL>
__device__ __forceinline__ void load_vec(const void *base, int64_t elem, RawVec<BF16, CPL> &r) {
    constexpr int NW = RawVec<BF16, CPL>::NW;
    const uint32_t *p = reinterpret_cast<const uint32_t *>(static_cast<const char *>(base) + elem * (BF16 ? 2 : 4));
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < NW; k += 4) {
            const uint4 u = *reinterpret_cast<const uint4 *>(p + k);
            r.w[k] = u.x; r.w[k + 1] = u.y; r.w[k + 2] = u.z; r.w[k + 3] = u.w;
        }
    } else if constexpr (NW == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = u.x; r.w[1] = u.y;
    } else {
        r.w[0] = p[0];
    }
}

template <bool BF16, int CPL>
__device__ __forceinline__ void cvt_vec(const RawVec<BF16, CPL> &r, float (&v)[CPL]) {
    if constexpr (BF16) {
#pragma unroll
        for (int k = 0; k < CPL / 2; ++k) {
            v[2 * k] = __uint_as_float(r.w[k] << 16);
            v[2 * k + 1] = __uint_as_float(r.w[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) v[k] = __uint_as_float(r.w[k]);
    }
}

template <int CPL>
__device__ __forceinline__ void load_f32(const float *p, float (&v)[CPL], float dflt) {
    if (!p) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) v[k] = dflt;
        return;
    }
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int k = 0; k < CPL; k += 4) {
            const float4 u = *reinterpret_cast<const float4 *>(p + k);
            v[k] = u.x; v[k + 1] = u.y; v[k + 2] = u.z; v[k + 3] = u.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) v[k] = p[k];
    }
}

template <int CPL>
__device__ __forceinline__ void store_f32(float *p, const float (&v)[CPL]) {
    if constexpr (CPL % 4 == 0) {
#pragma unroll
        for (int k = 0; k < CPL; k += 4) *reinterpret_cast<float4 *>(p + k) = make_float4(v[k], v[k + 1], v[k + 2], v[k + 3]);
    } else {
#pragma unroll
        for (int k = 0; k < CPL; ++k) p[k] = v[k];
    }
}

// Row-wide reduction of TS per-token values: wave butterflies (lane l ends with value
// index l >> SH), then with W > 1 an exchange through LDS slot buffer red[W][TS].
template <int TS, int W, bool MAX, typename T>
__device__ __forceinline__ void row_reduce(T (&v)[TS], T (*red)[TS], T (&out)[TS]) {
    constexpr int SH = TS == 8 ? 3 : (TS == 4 ? 4 : 5);
    const int lane = threadIdx.x & 63;
    const T r = wave_reduce_multi<TS, MAX>(v);
    if constexpr (W == 1) {
#pragma unroll
        for (int t = 0; t < TS; ++t) out[t] = __shfl(r, t << SH, 64);
    } else {
        const int wave = threadIdx.x >> 6;
        if ((lane & ((1 << SH) - 1)) == 0) red[wave][lane >> SH] = r;
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            T acc = red[0][t];
#pragma unroll
            for (int w = 1; w < W; ++w) acc = MAX ? (acc > red[w][t] ? acc : red[w][t]) : acc + red[w][t];
            out[t] = acc;
        }
    }
}

template <bool IN_BF16, int QUANT, bool OUT_BF16, int CPL, int W, int TS>
__global__ __launch_bounds__(64 * W) void scan_row_kernel(ScanArgs p) {
    __shared__ float red_ss[2][W][TS], red_mx[2][W][TS], red_s2[2][W][TS];
    __shared__ int red_q[2][W][TS];
    const int c = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = p.D;
    const int d0 = tid * CPL;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int64_t t_end = t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T;
    const float inv_d = 1.0f / static_cast<float>(D);

    float h[CPL], fb[CPL], lb[CPL], gw[CPL], qg[CPL];
    if (p.n_chunks > 1) load_f32<CPL>(p.hin + (b * p.n_chunks + c) * D + d0, h, 0.0f);
    else load_f32<CPL>(p.h0 ? p.h0 + b * D + d0 : nullptr, h, 0.0f);
    load_f32<CPL>(p.f_bias ? p.f_bias + d0 : nullptr, fb, 0.0f);
    load_f32<CPL>(p.f_lower ? p.f_lower + d0 : nullptr, lb, 0.0f);
    load_f32<CPL>(p.gnorm_w ? p.gnorm_w + d0 : nullptr, gw, 1.0f);
    load_f32<CPL>(QUANT && p.q_gamma ? p.q_gamma + d0 : nullptr, qg, 1.0f);

    using Raw = RawVec<IN_BF16, CPL>;
    Raw ip[TS], fp[TS], gp[TS];
    const int64_t D3 = 3 * static_cast<int64_t>(D);
    auto fetch = [&](int64_t tt) __attribute__((always_inline)) {
        const int nt = static_cast<int>(t_end - tt < TS ? t_end - tt : TS);
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            if (t < nt) {
                const int64_t base = (b * p.T + tt + t) * D3 + d0;
                load_vec<IN_BF16, CPL>(p.ifg, base, ip[t]);
                load_vec<IN_BF16, CPL>(p.ifg, base + D, fp[t]);
                load_vec<IN_BF16, CPL>(p.ifg, base + 2 * D, gp[t]);
            }
        }
    };
    if (t_beg < t_end) fetch(t_beg);

    int par = 0;
    for (int64_t tt = t_beg; tt < t_end; tt += TS, par ^= 1) {
        const int nt = static_cast<int>(t_end - tt < TS ? t_end - tt : TS);
        float o[TS][CPL], ss[TS];
        Raw gs[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            float iv[CPL], fv[CPL];
            cvt_vec<IN_BF16, CPL>(ip[t], iv);
            cvt_vec<IN_BF16, CPL>(fp[t], fv);
            gs[t] = gp[t];
            ss[t] = 0.f;
            if (t < nt) {
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    float f;
                    h[k] = gate_step(h[k], iv[k], fv[k], fb[k], lb[k], &f);
                    ss[t] = fmaf(h[k], h[k], ss[t]);
                }
            }
#pragma unroll
            for (int k = 0; k < CPL; ++k) o[t][k] = h[k];
        }
        if (tt + TS < t_end) fetch(tt + TS);  // next tile in flight during the reductions

        if (p.gate_mode == 0) {
            float tot[TS];
            row_reduce<TS, W, false>(ss, red_ss[par], tot);
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const float r = 1.0f / sqrtf(tot[t] * inv_d + p.eps);
                float gv[CPL];
                cvt_vec<IN_BF16, CPL>(gs[t], gv);
#pragma unroll
                for (int k = 0; k < CPL; ++k) o[t][k] = o[t][k] * r * gw[k] * siluf_(gv[k]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                float gv[CPL];
                cvt_vec<IN_BF16, CPL>(gs[t], gv);
#pragma unroll
                for (int k = 0; k < CPL; ++k) o[t][k] = sigmoidf_(gv[k]) * o[t][k];
            }
        }

        if constexpr (QUANT == 0) {
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                if (t >= nt) continue;
                const int64_t oi = (b * p.T + tt + t) * D + d0;
                if constexpr (OUT_BF16) {
                    uint32_t w[CPL / 2 > 0 ? CPL / 2 : 1];
#pragma unroll
                    for (int k = 0; k < CPL / 2; ++k) w[k] = pack_bf16x2(o[t][2 * k], o[t][2 * k + 1]);
                    uint32_t *dst = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.out) + oi);
                    if constexpr (CPL == 8) *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
                    else if constexpr (CPL == 4) *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
                    else {
#pragma unroll
                        for (int k = 0; k < CPL / 2; ++k) dst[k] = w[k];
                    }
                } else {
                    store_f32<CPL>(static_cast<float *>(p.out) + oi, o[t]);
                }
            }
        } else {
            // ---- int8 quantization of o (with o_proj's gain) for o_proj; o is first
            // materialised in the activation dtype, as g_norm's output
            if constexpr (IN_BF16) {
                static_assert(CPL % 2 == 0, "channels per lane come in pairs");
#pragma unroll
                for (int t = 0; t < TS; ++t)
#pragma unroll
                    for (int k = 0; k < CPL; k += 2) round_bf16_pair(o[t][k], o[t][k + 1]);
            }
            float mx[TS], s2[TS], mxt[TS], s2t[TS];
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                mx[t] = 0.f;
                s2[t] = 0.f;
                if (t < nt) {
#pragma unroll
                    for (int k = 0; k < CPL; ++k) {
                        mx[t] = fmaxf(mx[t], fabsf(o[t][k] * qg[k]));
                        s2[t] = fmaf(o[t][k], o[t][k], s2[t]);
                    }
                }
            }
            row_reduce<TS, W, true>(mx, red_mx[par], mxt);
            row_reduce<TS, W, false>(s2, red_s2[par], s2t);
            int qs[TS];
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                qs[t] = 0;
                if (t >= nt) continue;
                const float me = fmaxf(mxt[t], 1e-5f);
                const float sc = 127.0f / me;
                const int64_t row = b * p.T + tt + t;
                uint32_t pk[CPL / 4 > 0 ? CPL / 4 : 1] = {};
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    float rq = rintf((o[t][k] * qg[k]) * sc);
                    rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                    const int qi = static_cast<int>(rq);
                    qs[t] += qi;
                    pk[k >> 2] |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * (k & 3));
                }
                int8_t *qd = p.q + row * D + d0;
                if constexpr (CPL == 8) *reinterpret_cast<uint2 *>(qd) = make_uint2(pk[0], pk[1]);
                else if constexpr (CPL == 4) *reinterpret_cast<uint32_t *>(qd) = pk[0];
                else {
#pragma unroll
                    for (int k = 0; k < CPL; ++k) qd[k] = static_cast<int8_t>((pk[k >> 2] >> (8 * (k & 3))) & 0xFF);
                }
                if (p.cap.row0 <= row && row < p.cap.row1) {
                    const int64_t cr = row - p.cap.row0;
                    if (p.cap.x_in) store_f32<CPL>(p.cap.x_in + cr * D + d0, o[t]);
                    if (p.cap.q) {
#pragma unroll
                        for (int k = 0; k < CPL; ++k) p.cap.q[cr * D + d0 + k] = static_cast<int8_t>((pk[k >> 2] >> (8 * (k & 3))) & 0xFF);
                    }
                }
            }
            int qtot[TS];
            row_reduce<TS, W, false>(qs, red_q[par], qtot);
            if (tid < nt) {
                int qv = 0;
                float me = 0.f, s2v = 0.f;
#pragma unroll
                for (int t = 0; t < TS; ++t)
                    if (t == tid) { qv = qtot[t]; me = fmaxf(mxt[t], 1e-5f); s2v = s2t[t]; }
                const int64_t row = b * p.T + tt + tid;
                const float a = me / 127.0f * (1.0f / sqrtf(s2v * inv_d + p.q_eps));
                p.a[row] = a;
                p.rowsum[row] = qv;
                if (p.cap.a && p.cap.row0 <= row && row < p.cap.row1) p.cap.a[row - p.cap.row0] = a;
            }
        }
    }
    if (c == p.n_chunks - 1 && p.h_out) store_f32<CPL>(p.h_out + b * D + d0, h);
}

// Output pass over whole 16-token chunks of bf16 pre-activations, quantizing for o_proj (the
// prefill block path).  Same arithmetic as scan_row_kernel with 4-token tiles, but the four
// tiles of the chunk are unrolled and every global access is unconditional, so each wait
// on a tile's loads counts exactly the accesses issued after them: the next tile's loads
// stay in flight across this tile's stores instead of a wait that drains both.  The
// per-token scale and code sum are stored by every lane (lane l writes token l % 4; equal
// values to the same address).  CAP adds the stage-capture stores (tests only).
template <int W, bool CAP>
__global__ __launch_bounds__(64 * W) void scan_row16_kernel(ScanArgs p) {
    constexpr int CPL = 8, TS = 4, NTILE = kScanChunk / TS;
    __shared__ float red_ss[2][W][TS], red_mx[2][W][TS], red_s2[2][W][TS];
    __shared__ int red_q[2][W][TS];
    const int c = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = p.D;
    const int d0 = tid * CPL;
    const int64_t t_beg = static_cast<int64_t>(c) * kScanChunk;
    const float inv_d = 1.0f / static_cast<float>(D);
    const int64_t D3 = 3 * static_cast<int64_t>(D);

    // per-channel parameters first: the waits for them then never cover tile loads
    float h[CPL], fb[CPL], lb[CPL], gw[CPL], qg[CPL];
    if (p.n_chunks > 1) load_f32<CPL>(p.hin + (b * p.n_chunks + c) * D + d0, h, 0.0f);
    else load_f32<CPL>(p.h0 ? p.h0 + b * D + d0 : nullptr, h, 0.0f);
    load_f32<CPL>(p.f_bias ? p.f_bias + d0 : nullptr, fb, 0.0f);
    load_f32<CPL>(p.f_lower ? p.f_lower + d0 : nullptr, lb, 0.0f);
    load_f32<CPL>(p.gnorm_w ? p.gnorm_w + d0 : nullptr, gw, 1.0f);
    load_f32<CPL>(p.q_gamma ? p.q_gamma + d0 : nullptr, qg, 1.0f);

    using Raw = RawVec<true, CPL>;
    Raw ip[TS], fp[TS], gp[TS];
    auto fetch = [&](int64_t tt) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            const int64_t base = (b * p.T + tt + t) * D3 + d0;
            load_vec<true, CPL>(p.ifg, base, ip[t]);
            load_vec<true, CPL>(p.ifg, base + D, fp[t]);
            load_vec<true, CPL>(p.ifg, base + 2 * D, gp[t]);
        }
    };
    fetch(t_beg);

#pragma unroll
    for (int k = 0; k < NTILE; ++k) {
        const int64_t tt = t_beg + k * TS;
        const int par = k & 1;
        float o[TS][CPL], ss[TS];
        Raw gs[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            float iv[CPL], fv[CPL];
            cvt_vec<true, CPL>(ip[t], iv);
            cvt_vec<true, CPL>(fp[t], fv);
            gs[t] = gp[t];
            ss[t] = 0.f;
#pragma unroll
            for (int kk = 0; kk < CPL; ++kk) {
                float f;
                h[kk] = gate_step(h[kk], iv[kk], fv[kk], fb[kk], lb[kk], &f);
                ss[t] = fmaf(h[kk], h[kk], ss[t]);
                o[t][kk] = h[kk];
            }
        }
        if (k + 1 < NTILE) fetch(tt + TS);  // next tile in flight during this tile's tail

        if (p.gate_mode == 0) {
            float tot[TS];
            row_reduce<TS, W, false>(ss, red_ss[par], tot);
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                const float r = 1.0f / sqrtf(tot[t] * inv_d + p.eps);
                float gv[CPL];
                cvt_vec<true, CPL>(gs[t], gv);
#pragma unroll
                for (int kk = 0; kk < CPL; ++kk) o[t][kk] = o[t][kk] * r * gw[kk] * siluf_(gv[kk]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < TS; ++t) {
                float gv[CPL];
                cvt_vec<true, CPL>(gs[t], gv);
#pragma unroll
                for (int kk = 0; kk < CPL; ++kk) o[t][kk] = sigmoidf_(gv[kk]) * o[t][kk];
            }
        }
        // g_norm's output is materialised in the activation dtype (bf16) before o_proj
        // quantizes it
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
            for (int kk = 0; kk < CPL; kk += 2) round_bf16_pair(o[t][kk], o[t][kk + 1]);

        float mx[TS], s2[TS], mxt[TS], s2t[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            mx[t] = 0.f;
            s2[t] = 0.f;
#pragma unroll
            for (int kk = 0; kk < CPL; ++kk) {
                mx[t] = fmaxf(mx[t], fabsf(o[t][kk] * qg[kk]));
                s2[t] = fmaf(o[t][kk], o[t][kk], s2[t]);
            }
        }
        row_reduce<TS, W, true>(mx, red_mx[par], mxt);
        row_reduce<TS, W, false>(s2, red_s2[par], s2t);
        int qs[TS];
#pragma unroll
        for (int t = 0; t < TS; ++t) {
            const float me = fmaxf(mxt[t], 1e-5f);
            const float sc = 127.0f / me;
            const int64_t row = b * p.T + tt + t;
            uint32_t pk[2] = {0u, 0u};
            qs[t] = 0;
#pragma unroll
            for (int kk = 0; kk < CPL; ++kk) {
                float rq = rintf((o[t][kk] * qg[kk]) * sc);
                rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                const int qi = static_cast<int>(rq);
                qs[t] += qi;
                pk[kk >> 2] |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * (kk & 3));
            }
            *reinterpret_cast<uint2 *>(p.q + row * D + d0) = make_uint2(pk[0], pk[1]);
            if constexpr (CAP) {
                if (p.cap.row0 <= row && row < p.cap.row1) {
                    const int64_t cr = row - p.cap.row0;
                    if (p.cap.x_in) store_f32<CPL>(p.cap.x_in + cr * D + d0, o[t]);
                    if (p.cap.q) *reinterpret_cast<uint2 *>(p.cap.q + cr * D + d0) = make_uint2(pk[0], pk[1]);
                }
            }
        }
        int qtot[TS];
        row_reduce<TS, W, false>(qs, red_q[par], qtot);
        const int tl = tid & (TS - 1);
        int qv = qtot[0];
        float me = mxt[0], s2v = s2t[0];
#pragma unroll
        for (int t = 1; t < TS; ++t)
            if (t == tl) { qv = qtot[t]; me = mxt[t]; s2v = s2t[t]; }
        me = fmaxf(me, 1e-5f);
        const int64_t row = b * p.T + tt + tl;
        const float a = me / 127.0f * (1.0f / sqrtf(s2v * inv_d + p.q_eps));
        p.a[row] = a;
        p.rowsum[row] = qv;
        if constexpr (CAP) {
            if (p.cap.a && p.cap.row0 <= row && row < p.cap.row1) p.cap.a[row - p.cap.row0] = a;
        }
    }
    if (c == p.n_chunks - 1 && p.h_out) store_f32<CPL>(p.h_out + b * D + d0, h);
}

// Phase 1, row layout: thread per (b, chunk, group of CPL channels); the chunk's CH tokens
// of i and f are all loaded before the local scan runs (one 16-byte load per token and
// pre-activation), so the whole chunk is in flight at once.
template <bool BF16, int CPL, int CH>
__global__ __launch_bounds__(256) void scan_local_row_kernel(ScanArgs p) {
    const int G = p.D / CPL;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= p.B * p.n_chunks * G) return;
    const int gi = static_cast<int>(idx % G);
    const int64_t bc = idx / G;
    const int c = static_cast<int>(bc % p.n_chunks);
    const int64_t b = bc / p.n_chunks;
    const int D = p.D, d0 = gi * CPL;
    const int64_t t_beg = static_cast<int64_t>(c) * CH;
    const int nt = static_cast<int>(p.T - t_beg < CH ? p.T - t_beg : CH);
    const int64_t D3 = 3 * static_cast<int64_t>(D);
    float fb[CPL], lb[CPL], h[CPL], pf[CPL];
    load_f32<CPL>(p.f_bias ? p.f_bias + d0 : nullptr, fb, 0.0f);
    load_f32<CPL>(p.f_lower ? p.f_lower + d0 : nullptr, lb, 0.0f);
    // every load is issued (a ragged last chunk re-reads its last token), so the wait before
    // token t covers only the loads of tokens up to t
    using Raw = RawVec<BF16, CPL>;
    Raw iv[CH], fv[CH];
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        const int tc = t < nt ? t : nt - 1;
        const int64_t base = (b * p.T + t_beg + tc) * D3 + d0;
        load_vec<BF16, CPL>(p.ifg, base, iv[t]);
        load_vec<BF16, CPL>(p.ifg, base + D, fv[t]);
    }
#pragma unroll
    for (int k = 0; k < CPL; ++k) { h[k] = 0.f; pf[k] = 1.f; }
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        if (t < nt) {
            float i4[CPL], f4[CPL];
            cvt_vec<BF16, CPL>(iv[t], i4);
            cvt_vec<BF16, CPL>(fv[t], f4);
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                float f;
                h[k] = gate_step(h[k], i4[k], f4[k], fb[k], lb[k], &f);
                pf[k] *= f;
            }
        }
    }
    const int64_t o = (b * p.n_chunks + c) * D + d0;
    store_f32<CPL>(p.hloc + o, h);
    store_f32<CPL>(p.pf + o, pf);
}

// Phase 2, two-level: workgroup per (b, 64 channels), wave s owns the s-th of 8 runs of
// consecutive chunks.  Each wave folds its run into one affine map h -> A*h + B (lane =
// channel), the maps are composed through LDS to give the state entering every run, and
// each wave walks its run again writing the state entering each chunk.  Loads are batched
// U chunks ahead of the dependent multiply-add chain.
__global__ __launch_bounds__(512) void scan_carry2_kernel(ScanArgs p) {
    constexpr int RUNS = 8, U = 16;
    __shared__ float sA[RUNS][64], sB[RUNS][64];
    const int lane = threadIdx.x & 63, s = threadIdx.x >> 6;
    const int d = blockIdx.x * 64 + lane;
    const int64_t b = blockIdx.y;
    const int D = p.D, nc = p.n_chunks;
    const int L = (nc + RUNS - 1) / RUNS;
    const int c0 = s * L, c1 = c0 + L < nc ? c0 + L : nc;
    const int64_t row0 = b * nc;
    float A = 1.f, Bv = 0.f;
    // a run of at most U chunks (2048 tokens and fewer at 16 tokens per chunk) stays in
    // registers for the second walk instead of being read again
    float pf[U], hl[U];
    const bool one_batch = c1 - c0 <= U;
    for (int c = c0; c < c1; c += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u < c1 ? c + u : c1 - 1;
            pf[u] = p.pf[(row0 + cc) * D + d];
            hl[u] = p.hloc[(row0 + cc) * D + d];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c + u < c1) {
                Bv = pf[u] * Bv + hl[u];
                A *= pf[u];
            }
        }
    }
    sA[s][lane] = A;
    sB[s][lane] = Bv;
    __syncthreads();
    float h = p.h0 ? p.h0[b * D + d] : 0.0f;
    for (int j = 0; j < s; ++j) h = sA[j][lane] * h + sB[j][lane];
    for (int c = c0; c < c1; c += U) {
        if (!one_batch) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c + u < c1 ? c + u : c1 - 1;
                pf[u] = p.pf[(row0 + cc) * D + d];
                hl[u] = p.hloc[(row0 + cc) * D + d];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c + u < c1) {
                p.hin[(row0 + c + u) * D + d] = h;
                h = pf[u] * h + hl[u];
            }
        }
    }
}

__global__ void copy_state_kernel(const float *h0, float *h_out, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) h_out[i] = h0 ? h0[i] : 0.0f;
}

template <bool IN_BF16, int QUANT, bool OUT_BF16, int TS>
void launch_out_ts(const ScanArgs &a, dim3 grid, hipStream_t s) {
    const int jq = (a.D + 1023) / 1024;
    if (jq <= 1) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, 1, TS>), grid, dim3(256), 0, s, a);
    else if (jq == 2) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, 2, TS>), grid, dim3(256), 0, s, a);
    else if (jq == 3) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, 3, TS>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, 4, TS>), grid, dim3(256), 0, s, a);
}

// Token tile of 4: larger tiles amortize the reductions further but the replicated
// per-token values push the kernel past 128 registers (measured slower at 8).
template <bool IN_BF16, int QUANT, bool OUT_BF16>
void launch_out_q(const ScanArgs &a, dim3 grid, hipStream_t s) {
    launch_out_ts<IN_BF16, QUANT, OUT_BF16, 4>(a, grid, s);
}

// Row-layout output pass: W waves per token row, CPL channels per lane (ragged chunks,
// fp32 pre-activations, unquantized output).  Tiles of 2 tokens at 8 channels per lane (4 at
// 4): larger tiles amortize the reductions further but their registers halve the waves per
// SIMD where more than two waves per SIMD are resident.
template <bool IN_BF16, int QUANT, bool OUT_BF16, int CPL, int W>
void launch_row(const ScanArgs &a, dim3 grid, hipStream_t s) {
    constexpr int TS = CPL >= 8 ? 2 : 4;
    hipLaunchKernelGGL((scan_row_kernel<IN_BF16, QUANT, OUT_BF16, CPL, W, TS>), grid, dim3(64 * W), 0, s, a);
}

template <bool IN_BF16, int QUANT, bool OUT_BF16>
bool launch_row_q(const ScanArgs &a, dim3 grid, hipStream_t s) {
    const int D = a.D;
    if (D % 512 == 0) {
        switch (D / 512) {
            case 1: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 1>(a, grid, s); return true;
            case 2: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 2>(a, grid, s); return true;
            case 3: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 3>(a, grid, s); return true;
            case 4: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 4>(a, grid, s); return true;
            case 5: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 5>(a, grid, s); return true;
            case 6: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 6>(a, grid, s); return true;
            case 7: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 7>(a, grid, s); return true;
            case 8: launch_row<IN_BF16, QUANT, OUT_BF16, 8, 8>(a, grid, s); return true;
            default: return false;
        }
    }
    if (D % 256 == 0) {
        switch (D / 256) {
            case 1: launch_row<IN_BF16, QUANT, OUT_BF16, 4, 1>(a, grid, s); return true;
            case 3: launch_row<IN_BF16, QUANT, OUT_BF16, 4, 3>(a, grid, s); return true;
            case 4: launch_row<IN_BF16, QUANT, OUT_BF16, 4, 4>(a, grid, s); return true;
            case 5: launch_row<IN_BF16, QUANT, OUT_BF16, 4, 5>(a, grid, s); return true;
            default: return false;
        }
    }
    return false;
}

template <bool CAP>
bool launch_row16(const ScanArgs &a, dim3 grid, hipStream_t s) {
    switch (a.D / 512) {
        case 1: hipLaunchKernelGGL((scan_row16_kernel<1, CAP>), grid, dim3(64), 0, s, a); return true;
        case 2: hipLaunchKernelGGL((scan_row16_kernel<2, CAP>), grid, dim3(128), 0, s, a); return true;
        case 3: hipLaunchKernelGGL((scan_row16_kernel<3, CAP>), grid, dim3(192), 0, s, a); return true;
        case 4: hipLaunchKernelGGL((scan_row16_kernel<4, CAP>), grid, dim3(256), 0, s, a); return true;
        case 5: hipLaunchKernelGGL((scan_row16_kernel<5, CAP>), grid, dim3(320), 0, s, a); return true;
        case 6: hipLaunchKernelGGL((scan_row16_kernel<6, CAP>), grid, dim3(384), 0, s, a); return true;
        case 7: hipLaunchKernelGGL((scan_row16_kernel<7, CAP>), grid, dim3(448), 0, s, a); return true;
        case 8: hipLaunchKernelGGL((scan_row16_kernel<8, CAP>), grid, dim3(512), 0, s, a); return true;
        default: return false;
    }
}

// whole 16-token chunks of bf16 pre-activations quantized for o_proj
bool launch_row16_q(const ScanArgs &a, dim3 grid, hipStream_t s) {
    if (!a.ifg_bf16 || a.chunk != kScanChunk || a.T % kScanChunk != 0 || a.D % 512 != 0) return false;
    return a.cap.row1 > a.cap.row0 ? launch_row16<true>(a, grid, s) : launch_row16<false>(a, grid, s);
}

template <bool IN_BF16>
void launch_out(const ScanArgs &a, dim3 grid, hipStream_t s) {
    if (a.q) {
        if (IN_BF16 && launch_row16_q(a, grid, s)) return;
        if (!launch_row_q<IN_BF16, 1, false>(a, grid, s)) launch_out_q<IN_BF16, 1, false>(a, grid, s);
    } else if (a.out_bf16) {
        if (!launch_row_q<IN_BF16, 0, true>(a, grid, s)) launch_out_q<IN_BF16, 0, true>(a, grid, s);
    } else {
        if (!launch_row_q<IN_BF16, 0, false>(a, grid, s)) launch_out_q<IN_BF16, 0, false>(a, grid, s);
    }
}
}  // namespace

hipError_t launch_scan_carries(const ScanArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    if (a.n_chunks > 1) {
        if (a.chunk == kScanChunk && a.D % 64 == 0) {
            // row layout: 4 channels per thread (8-byte bf16 or 16-byte fp32 loads; with 8 per
            // thread the 370M block had half the waves in flight and phase 1 took 3 us longer),
            // runs of chunks for the carry
            const int cpl = 4;
            const int64_t n = a.B * a.n_chunks * (a.D / cpl);
            const dim3 g1(static_cast<unsigned>((n + 255) / 256));
            if (a.ifg_bf16) hipLaunchKernelGGL((scan_local_row_kernel<true, 4, kScanChunk>), g1, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((scan_local_row_kernel<false, 4, kScanChunk>), g1, dim3(256), 0, s, a);
            const dim3 g2(static_cast<unsigned>(a.D / 64), static_cast<unsigned>(a.B));
            hipLaunchKernelGGL(scan_carry2_kernel, g2, dim3(512), 0, s, a);
        } else {
            const dim3 g1(static_cast<unsigned>((a.D / 4 + 255) / 256), static_cast<unsigned>(a.n_chunks),
                          static_cast<unsigned>(a.B));
            if (a.ifg_bf16) hipLaunchKernelGGL((scan_local_kernel<true>), g1, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((scan_local_kernel<false>), g1, dim3(256), 0, s, a);
            const dim3 g2(static_cast<unsigned>((a.D + 255) / 256), static_cast<unsigned>(a.B));
            hipLaunchKernelGGL(scan_carry_kernel, g2, dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    timing_begin(FAM_SCAN, s);
    launch_scan_carries(a, s);
    const dim3 g3(static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(a.B));
    if (a.ifg_bf16) launch_out<true>(a, g3, s);
    else launch_out<false>(a, g3, s);
    timing_end(FAM_SCAN, s);
    return hipGetLastError();
}

hipError_t launch_copy_state(const float *h0, float *h_out, int64_t n, hipStream_t s) {
    if (n <= 0 || !h_out) return hipSuccess;
    hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, s, h0, h_out, n);
    return hipGetLastError();
}

// Ternary embedding gather: thread per (token, packed word) writes 16 values.
template <bool BF16>
__global__ void embedding_kernel(const uint32_t *packed, float scale, int64_t vocab, int32_t D,
                                 const int32_t *ids, int64_t m, void *x) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int W = D / 16;
    if (i >= m * W) return;
    const int64_t t = i / W;
    const int j = static_cast<int>(i % W);
    const int32_t id = ids[t];
    const bool ok = id >= 0 && id < vocab;
    const uint32_t w = ok ? packed[static_cast<int64_t>(id) * W + j] : 0x55555555u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int a = k >> 2, bb = k & 3;
        const int code = static_cast<int>((w >> (8 * bb + 2 * a)) & 3u);
        const float v = static_cast<float>(code - 1) * scale;
        store_act<BF16>(x, t * D + 16 * j + k, v);
    }
}

hipError_t launch_embedding(const uint32_t *packed, float scale, int64_t vocab, int32_t D,
                            const int32_t *ids, int64_t m, void *x, int bf16, hipStream_t s) {
    if (m <= 0) return hipSuccess;
    const int64_t n = m * (D / 16);
    const dim3 grid(static_cast<unsigned>((n + 255) / 256));
    timing_begin(FAM_EMBED, s);
    if (bf16) hipLaunchKernelGGL((embedding_kernel<true>), grid, dim3(256), 0, s, packed, scale, vocab, D, ids, m, x);
    else hipLaunchKernelGGL((embedding_kernel<false>), grid, dim3(256), 0, s, packed, scale, vocab, D, ids, m, x);
    timing_end(FAM_EMBED, s);
    return hipGetLastError();
}

}  // namespace mmf
