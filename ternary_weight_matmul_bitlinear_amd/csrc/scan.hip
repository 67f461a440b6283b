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
// CUs at long T it is also chunked over time (HBM-bound throughout):
//   phase 1 (per chunk, channel): local scan from 0 -> end state hloc and prod(f);
//   phase 2 (per channel): carry across chunks, h_in[c+1] = prod_c*h_in[c] + hloc_c;
//   phase 3 (per chunk, one workgroup owning all D channels of a token): rerun the
//     recurrence from h_in, then per token the RMSNorm over D (workgroup reduction), the
//     swish gate, and either a store of o or its int8 quantization for o_proj (a second
//     reduction for max|o| and sum(o^2)), writing q, a and the row sum.
// With one chunk (decode, short T) phases 1 and 2 are skipped.
#include "mmf_internal.h"

namespace mmf {

namespace {
constexpr int JMAX = 16;  // channels per thread in phase 3 (D <= 4096)

template <bool BF16>
__global__ __launch_bounds__(256) void scan_local_kernel(ScanArgs p) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int64_t b = blockIdx.z;
    if (d >= p.D) return;
    const int D = p.D;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int64_t t_end = t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T;
    const float fb = p.f_bias ? p.f_bias[d] : 0.0f;
    float h = 0.0f, pf = 1.0f;
#pragma unroll 4
    for (int64_t t = t_beg; t < t_end; ++t) {
        const int64_t base = (b * p.T + t) * 3 * D;
        const float ip = load_act<BF16>(p.ifg, base + d);
        const float fp = load_act<BF16>(p.ifg, base + D + d);
        const float f = sigmoidf_(fp + fb);
        const float cc = siluf_(ip);
        h = f * h + (1.0f - f) * cc;
        pf *= f;
    }
    const int64_t o = (b * p.n_chunks + c) * D + d;
    p.hloc[o] = h;
    p.pf[o] = pf;
}

__global__ __launch_bounds__(256) void scan_carry_kernel(ScanArgs p) {
    const int d = blockIdx.x * 256 + threadIdx.x;
    const int64_t b = blockIdx.y;
    if (d >= p.D) return;
    const int D = p.D;
    float carry = p.h0 ? p.h0[b * D + d] : 0.0f;
    for (int c = 0; c < p.n_chunks; ++c) {
        const int64_t o = (b * p.n_chunks + c) * D + d;
        p.hin[o] = carry;
        carry = p.pf[o] * carry + p.hloc[o];
    }
}

struct Red2 { float a, b; };

// Workgroup reductions (4 waves); `slot` alternates between calls so one barrier suffices.
__device__ __forceinline__ float block_sum(float v, float (*red)[4], int slot) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[slot][threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
}
__device__ __forceinline__ Red2 block_max_sum(float m, float s, float (*rm)[4], float (*rs)[4],
                                              int slot) {
    m = wave_max(m);
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) {
        rm[slot][threadIdx.x >> 6] = m;
        rs[slot][threadIdx.x >> 6] = s;
    }
    __syncthreads();
    Red2 r;
    r.a = fmaxf(fmaxf(rm[slot][0], rm[slot][1]), fmaxf(rm[slot][2], rm[slot][3]));
    r.b = (rs[slot][0] + rs[slot][1]) + (rs[slot][2] + rs[slot][3]);
    return r;
}

// QUANT: 0 = store o (OUT_BF16 selects dtype), 1 = quantize o for o_proj.
template <bool IN_BF16, int QUANT, bool OUT_BF16>
__global__ __launch_bounds__(256) void scan_out_kernel(ScanArgs p) {
    __shared__ float red_s[2][4], red_m[2][4], red_q[2][4];
    __shared__ int rsum[kScanChunk][4];
    const int c = blockIdx.x;
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = p.D;
    const int64_t t_beg = static_cast<int64_t>(c) * p.chunk;
    const int64_t t_end = t_beg + p.chunk < p.T ? t_beg + p.chunk : p.T;
    const float inv_d = 1.0f / static_cast<float>(D);

    float h[JMAX], fb[JMAX], gw[JMAX], qg[JMAX];
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
        const int d = tid + 256 * j;
        h[j] = 0.f; fb[j] = 0.f; gw[j] = 1.f; qg[j] = 1.f;
        if (d < D) {
            if (p.n_chunks > 1) h[j] = p.hin[(b * p.n_chunks + c) * D + d];
            else if (p.h0) h[j] = p.h0[b * D + d];
            if (p.f_bias) fb[j] = p.f_bias[d];
            if (p.gnorm_w) gw[j] = p.gnorm_w[d];
            if (QUANT && p.q_gamma) qg[j] = p.q_gamma[d];
        }
    }

    // software prefetch of the next token's pre-activations
    float ni[JMAX], nf[JMAX], ng[JMAX];
    auto fetch = [&](int64_t t) {
        const int64_t base = (b * p.T + t) * 3 * D;
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            const int d = tid + 256 * j;
            if (d < D) {
                ni[j] = load_act<IN_BF16>(p.ifg, base + d);
                nf[j] = load_act<IN_BF16>(p.ifg, base + D + d);
                ng[j] = load_act<IN_BF16>(p.ifg, base + 2 * D + d);
            }
        }
    };
    if (t_beg < t_end) fetch(t_beg);

    int slot = 0;
    for (int64_t t = t_beg; t < t_end; ++t) {
        float gi[JMAX];
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            const int d = tid + 256 * j;
            gi[j] = ng[j];
            if (d < D) {
                const float f = sigmoidf_(nf[j] + fb[j]);
                const float cc = siluf_(ni[j]);
                h[j] = f * h[j] + (1.0f - f) * cc;
                ss += h[j] * h[j];
            }
        }
        if (t + 1 < t_end) fetch(t + 1);
        const int64_t row = b * p.T + t;

        float o[JMAX];
        if (p.gate_mode == 0) {
            const float tot = block_sum(ss, red_s, slot);
            const float r = 1.0f / sqrtf(tot * inv_d + p.eps);
#pragma unroll
            for (int j = 0; j < JMAX; ++j) o[j] = h[j] * r * gw[j] * siluf_(gi[j]);
        } else {
#pragma unroll
            for (int j = 0; j < JMAX; ++j) o[j] = sigmoidf_(gi[j]) * h[j];
        }
        if (p.round_bf16) {
#pragma unroll
            for (int j = 0; j < JMAX; ++j) o[j] = round_to_bf16(o[j]);
        }
        if constexpr (QUANT == 0) {
#pragma unroll
            for (int j = 0; j < JMAX; ++j) {
                const int d = tid + 256 * j;
                if (d < D) store_act<OUT_BF16>(p.out, row * D + d, o[j]);
            }
        } else {
            float mx = 0.f, s2 = 0.f;
#pragma unroll
            for (int j = 0; j < JMAX; ++j) {
                const int d = tid + 256 * j;
                if (d < D) {
                    const float pj = o[j] * qg[j];
                    mx = fmaxf(mx, fabsf(pj));
                    s2 += o[j] * o[j];
                }
            }
            const Red2 rr = block_max_sum(mx, s2, red_m, red_q, slot);
            const float me = fmaxf(rr.a, 1e-5f);
            const float sc = 127.0f / me;
            const bool capr = p.cap.row0 <= row && row < p.cap.row1;
            const int64_t cr = row - p.cap.row0;
            int qsum = 0;
#pragma unroll
            for (int j = 0; j < JMAX; ++j) {
                const int d = tid + 256 * j;
                if (d < D) {
                    const float pj = o[j] * qg[j];
                    float rq = rintf(pj * sc);
                    rq = fminf(fmaxf(rq, -127.0f), 127.0f);
                    const int qi = static_cast<int>(rq);
                    qsum += qi;
                    p.q[row * D + d] = static_cast<int8_t>(qi);
                    if (capr) {
                        if (p.cap.x_in) p.cap.x_in[cr * D + d] = o[j];
                        if (p.cap.q) p.cap.q[cr * D + d] = static_cast<int8_t>(qi);
                    }
                }
            }
            qsum = wave_sum_i(qsum);
            if (lane == 0) rsum[t - t_beg][wave] = qsum;
            if (tid == 0) {
                const float a = me / 127.0f * (1.0f / sqrtf(rr.b * inv_d + p.q_eps));
                p.a[row] = a;
                if (capr && p.cap.a) p.cap.a[cr] = a;
            }
        }
        slot ^= 1;
    }
    if constexpr (QUANT != 0) {
        __syncthreads();
        const int nt = static_cast<int>(t_end - t_beg);
        if (tid < nt)
            p.rowsum[b * p.T + t_beg + tid] = (rsum[tid][0] + rsum[tid][1]) + (rsum[tid][2] + rsum[tid][3]);
    }
    if (c == p.n_chunks - 1 && p.h_out) {
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            const int d = tid + 256 * j;
            if (d < D) p.h_out[b * D + d] = h[j];
        }
    }
}

__global__ void copy_state_kernel(const float *h0, float *h_out, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) h_out[i] = h0 ? h0[i] : 0.0f;
}

template <bool IN_BF16>
void launch_out(const ScanArgs &a, dim3 grid, hipStream_t s) {
    if (a.q) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, 1, false>), grid, dim3(256), 0, s, a);
    else if (a.out_bf16) hipLaunchKernelGGL((scan_out_kernel<IN_BF16, 0, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_out_kernel<IN_BF16, 0, false>), grid, dim3(256), 0, s, a);
}
}  // namespace

hipError_t launch_scan(const ScanArgs &a, hipStream_t s) {
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    const unsigned dblk = static_cast<unsigned>((a.D + 255) / 256);
    timing_begin(FAM_SCAN, s);
    if (a.n_chunks > 1) {
        const dim3 g1(dblk, static_cast<unsigned>(a.n_chunks), static_cast<unsigned>(a.B));
        if (a.ifg_bf16) hipLaunchKernelGGL((scan_local_kernel<true>), g1, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((scan_local_kernel<false>), g1, dim3(256), 0, s, a);
        const dim3 g2(dblk, static_cast<unsigned>(a.B));
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
        const int a = (k & 15) >> 2, bb = k & 3;
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
