// scan.hip -- MLGRU token mixer for gfx950: fused gates, chunked time-parallel scan,
// RMSNorm-swish output gate and (optionally) the int8 quantization of o_proj's input.
//
// DataCamp "MatMul-free language models", section "Core components: MLGRU and GLU": the
// hidden state carries memory from token to token and gates in (0,1) decide what flows.
// Hysen Labs "MatMul-Free LM", section "HGRN attention": the recurrence needs only the
// current token and the previous state (linear in T); its output passes g_norm, an RMSNorm
// fused with a swish gate, before o_proj.  Per (b, d):
//   f = sigmoid(f_pre + b_f), c = SiLU(i_pre), h_t = f*h_{t-1} + (1-f)*c,
//   o_t = RMSNorm_D(h_t)*gnorm_w * g*sigmoid(g)   (or sigmoid(g)*h_t).
//
// The recurrence is elementwise in d, so it is parallel over B*D channels; to fill 256
// CUs at long T it is also chunked over time.  All phases are HBM-bound:
//   phase 1 (per chunk, channel quad): local scan from 0 -> end state hloc and prod(f);
//   phase 2 (per channel): carry across chunks, h_in[c+1] = prod_c*h_in[c] + hloc_c;
//   phase 3 (workgroup per chunk): rerun the recurrence from h_in for a tile of tokens,
//     parking h in LDS, then one wave per token does the RMSNorm over D, the gate and
//     either a store of o or its int8 quantization for o_proj (q, a, row sum) with
//     wave-only reductions: two barriers per token tile instead of two per token.
// With one chunk (decode, short T) phases 1 and 2 are skipped.
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
__device__ __forceinline__ void st4f(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

__device__ __forceinline__ float gate_step(float h, float ip, float fp, float fb, float *f_out) {
    const float f = sigmoidf_(fp + fb);
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
    float h[4] = {0.f, 0.f, 0.f, 0.f}, pf[4] = {1.f, 1.f, 1.f, 1.f};
    const float fbv[4] = {fb.x, fb.y, fb.z, fb.w};
    const int64_t base = (b * p.T + t_beg) * 3 * D + d;
#pragma unroll 8
    for (int t = 0; t < nt; ++t) {
        const float4 ip = load4<BF16>(p.ifg, base + static_cast<int64_t>(t) * 3 * D);
        const float4 fp = load4<BF16>(p.ifg, base + static_cast<int64_t>(t) * 3 * D + D);
        const float iv[4] = {ip.x, ip.y, ip.z, ip.w}, fv[4] = {fp.x, fp.y, fp.z, fp.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float f;
            h[e] = gate_step(h[e], iv[e], fv[e], fbv[e], &f);
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

// Phase 3: workgroup per (b, chunk), tokens in tiles of TS.  JQ = channel quads per
// thread in the recurrence (D <= 1024*JQ); per token row a lane holds NV = 4*JQ float4.
template <bool IN_BF16, int QUANT, bool OUT_BF16, int TS, int JQ>
__global__ __launch_bounds__(256) void scan_out_kernel(ScanArgs p) {
    extern __shared__ __attribute__((aligned(16))) float hs[];  // [TS][D]
    const int c = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = p.D;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int64_t t_end = t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T;
    const float inv_d = 1.0f / static_cast<float>(D);

    float h[JQ][4], fb[JQ][4];
#pragma unroll
    for (int j = 0; j < JQ; ++j) {
        const int d = 4 * (tid + 256 * j);
        float4 hv = make_float4(0.f, 0.f, 0.f, 0.f), fv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (d < D) {
            if (p.n_chunks > 1) hv = ld4f(p.hin + (b * p.n_chunks + c) * D + d);
            else if (p.h0) hv = ld4f(p.h0 + b * D + d);
            if (p.f_bias) fv = ld4f(p.f_bias + d);
        }
        h[j][0] = hv.x; h[j][1] = hv.y; h[j][2] = hv.z; h[j][3] = hv.w;
        fb[j][0] = fv.x; fb[j][1] = fv.y; fb[j][2] = fv.z; fb[j][3] = fv.w;
    }

    for (int64_t tt = t_beg; tt < t_end; tt += TS) {
        const int nt = static_cast<int>(t_end - tt < TS ? t_end - tt : TS);
        // ---- recurrence for the tile (all loads of the tile issued before the chain)
        float4 ip[TS][JQ], fp[TS][JQ];
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
            for (int j = 0; j < JQ; ++j) {
                const int d = 4 * (tid + 256 * j);
                if (t < nt && d < D) {
                    const int64_t base = (b * p.T + tt + t) * 3 * D + d;
                    ip[t][j] = load4<IN_BF16>(p.ifg, base);
                    fp[t][j] = load4<IN_BF16>(p.ifg, base + D);
                }
            }
#pragma unroll
        for (int t = 0; t < TS; ++t)
#pragma unroll
            for (int j = 0; j < JQ; ++j) {
                const int d = 4 * (tid + 256 * j);
                if (t < nt && d < D) {
                    const float iv[4] = {ip[t][j].x, ip[t][j].y, ip[t][j].z, ip[t][j].w};
                    const float fv[4] = {fp[t][j].x, fp[t][j].y, fp[t][j].z, fp[t][j].w};
                    float f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[j][e] = gate_step(h[j][e], iv[e], fv[e], fb[j][e], &f);
                    st4f(hs + t * D + d, make_float4(h[j][0], h[j][1], h[j][2], h[j][3]));
                }
            }
        __syncthreads();

        // ---- one wave per token: g_norm, gate, then store or quantize
        constexpr int NV = JQ * 4;
        for (int t = wave; t < nt; t += 4) {
            const int64_t row = b * p.T + tt + t;
            const float *hr = hs + t * D;
            float4 hv[NV], gv[NV];
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = 4 * (lane + 64 * k);
                if (d < D) {
                    hv[k] = ld4f(hr + d);
                    gv[k] = load4<IN_BF16>(p.ifg, row * 3 * D + 2 * D + d);
                    ss += hv[k].x * hv[k].x + hv[k].y * hv[k].y + hv[k].z * hv[k].z + hv[k].w * hv[k].w;
                }
            }
            float r = 0.f;
            if (p.gate_mode == 0) r = 1.0f / sqrtf(wave_sum(ss) * inv_d + p.eps);
            float ov[NV][4];
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = 4 * (lane + 64 * k);
                if (d < D) {
                    const float hvv[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
                    const float g[4] = {gv[k].x, gv[k].y, gv[k].z, gv[k].w};
                    const float4 gw = p.gnorm_w ? ld4f(p.gnorm_w + d) : make_float4(1.f, 1.f, 1.f, 1.f);
                    const float gwa[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ov[k][e] = p.gate_mode == 0 ? hvv[e] * r * gwa[e] * siluf_(g[e]) : sigmoidf_(g[e]) * hvv[e];
                    }
                }
            }
            if constexpr (QUANT == 0) {
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const int d = 4 * (lane + 64 * k);
                    if (d < D) {
                        if constexpr (OUT_BF16) {
                            const uint32_t lo = f32_to_bf16_bits(ov[k][0]) | (static_cast<uint32_t>(f32_to_bf16_bits(ov[k][1])) << 16);
                            const uint32_t hi = f32_to_bf16_bits(ov[k][2]) | (static_cast<uint32_t>(f32_to_bf16_bits(ov[k][3])) << 16);
                            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + row * D + d) = make_uint2(lo, hi);
                        } else {
                            st4f(static_cast<float *>(p.out) + row * D + d, make_float4(ov[k][0], ov[k][1], ov[k][2], ov[k][3]));
                        }
                    }
                }
            } else {
                float pv[NV][4];
                float mx = 0.f, s2 = 0.f;
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const int d = 4 * (lane + 64 * k);
                    if (d < D) {
                        const float4 qg = p.q_gamma ? ld4f(p.q_gamma + d) : make_float4(1.f, 1.f, 1.f, 1.f);
                        const float qga[4] = {qg.x, qg.y, qg.z, qg.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pv[k][e] = p.q_gamma ? ov[k][e] * qga[e] : ov[k][e];
                            mx = fmaxf(mx, fabsf(pv[k][e]));
                            s2 += ov[k][e] * ov[k][e];
                        }
                    }
                }
                mx = wave_max(mx);
                s2 = wave_sum(s2);
                const float me = fmaxf(mx, 1e-5f);
                const float sc = 127.0f / me;
                const bool capr = p.cap.row0 <= row && row < p.cap.row1;
                const int64_t cr = row - p.cap.row0;
                int qsum = 0;
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    const int d = 4 * (lane + 64 * k);
                    if (d < D) {
                        uint32_t packed = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float rq = rintf(pv[k][e] * sc);
                            rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                            const int qi = static_cast<int>(rq);
                            qsum += qi;
                            packed |= (static_cast<uint32_t>(qi) & 0xFFu) << (8 * e);
                        }
                        *reinterpret_cast<uint32_t *>(p.q + row * D + d) = packed;
                        if (capr) {
                            if (p.cap.x_in) st4f(p.cap.x_in + cr * D + d, make_float4(ov[k][0], ov[k][1], ov[k][2], ov[k][3]));
                            if (p.cap.q) *reinterpret_cast<uint32_t *>(p.cap.q + cr * D + d) = packed;
                        }
                    }
                }
                qsum = wave_sum_i(qsum);
                if (lane == 0) {
                    const float a = me / 127.0f * (1.0f / sqrtf(s2 * inv_d + p.q_eps));
                    p.a[row] = a;
                    p.rowsum[row] = qsum;
                    if (capr && p.cap.a) p.cap.a[cr] = a;
                }
            }
        }
        __syncthreads();
    }
    if (c == p.n_chunks - 1 && p.h_out) {
#pragma unroll
        for (int j = 0; j < JQ; ++j) {
            const int d = 4 * (tid + 256 * j);
            if (d < D) st4f(p.h_out + b * D + d, make_float4(h[j][0], h[j][1], h[j][2], h[j][3]));
        }
    }
}

__global__ void copy_state_kernel(const float *h0, float *h_out, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) h_out[i] = h0 ? h0[i] : 0.0f;
}

template <bool IN_BF16, int QUANT, bool OUT_BF16, int TS>
void launch_out_ts(const ScanArgs &a, dim3 grid, hipStream_t s) {
    const size_t lds = static_cast<size_t>(TS) * a.D * 4;
    const int jq = (a.D + 1023) / 1024;
    if (jq <= 1) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, TS, 1>), grid, dim3(256), lds, s, a);
    else if (jq == 2) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, TS, 2>), grid, dim3(256), lds, s, a);
    else if (jq == 3) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, TS, 3>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((scan_out_kernel<IN_BF16, QUANT, OUT_BF16, TS, 4>), grid, dim3(256), lds, s, a);
}

// Token tile: the LDS tile TS x D fp32 stays at or under 64 KB.
template <bool IN_BF16, int QUANT, bool OUT_BF16>
void launch_out_q(const ScanArgs &a, dim3 grid, hipStream_t s) {
    if (a.D <= 1024) launch_out_ts<IN_BF16, QUANT, OUT_BF16, 16>(a, grid, s);
    else if (a.D <= 2048) launch_out_ts<IN_BF16, QUANT, OUT_BF16, 8>(a, grid, s);
    else launch_out_ts<IN_BF16, QUANT, OUT_BF16, 4>(a, grid, s);
}

template <bool IN_BF16>
void launch_out(const ScanArgs &a, dim3 grid, hipStream_t s) {
    if (a.q) launch_out_q<IN_BF16, 1, false>(a, grid, s);
    else if (a.out_bf16) launch_out_q<IN_BF16, 0, true>(a, grid, s);
    else launch_out_q<IN_BF16, 0, false>(a, grid, s);
}
}  // namespace

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    timing_begin(FAM_SCAN, s);
    if (a.n_chunks > 1) {
        const dim3 g1(static_cast<unsigned>((a.D / 4 + 255) / 256), static_cast<unsigned>(a.n_chunks),
                      static_cast<unsigned>(a.B));
        if (a.ifg_bf16) hipLaunchKernelGGL((scan_local_kernel<true>), g1, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((scan_local_kernel<false>), g1, dim3(256), 0, s, a);
        const dim3 g2(static_cast<unsigned>((a.D + 255) / 256), static_cast<unsigned>(a.B));
        hipLaunchKernelGGL(scan_carry_kernel, g2, dim3(256), 0, s, a);
    }
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
