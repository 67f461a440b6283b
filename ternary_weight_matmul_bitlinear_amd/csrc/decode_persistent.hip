// decode_persistent.hip -- one decode step of a whole stack (embedding, L blocks, head) for
// one sequence in a single cooperative launch.
//
// DataCamp "MatMul-free language models", section "From optimised GPU to custom FPGA":
// generating a token is limited by moving the weights; Hysen Labs "MatMul-Free LM",
// sections "HGRN attention" (block: RMSNorm -> i/f/g -> recurrence -> g_norm -> o_proj) and
// "Installation and model initialization" (hidden 2048, 32000-entry embedding, 24 layers).
//
// With one token each BitLinear moves only 1-16 MB of 2-bit weights, about one memory
// latency's worth of HBM bandwidth, and the step is a chain of 4L + 1 dependent stages
// (i|f|g; MLGRU step + g_norm + o_proj + residual; gate|up + SiLU product; down + residual;
// then the head).  Here every workgroup of one co-resident grid owns a slice of every
// stage's weight rows and keeps the chain inside the kernel:
//   - the slice of the next stage is requested into registers as soon as the current stage's
//     outputs are stored, and the small vectors the next stage reads (its quantizer's gain,
//     for the MLGRU step the state, forget bias and bound and the g_norm weight) are copied
//     into LDS by direct loads at the same point, with that stage's bias values; so the HBM
//     latency of all of them overlaps the wait for the other workgroups, and no dependent
//     global load is left between a wait and the stage's outputs;
//   - a stage's outputs go to an exchange area as 64-bit words holding two bf16 values and
//     the launch's tag in the upper half; a word is written with one 64-bit store and read
//     with one 64-bit load, both relaxed device-scope atomics, so a reader that sees the
//     current tag also sees both values -- no fence, no counter, one memory round trip from
//     the last producer's store to the consumers;
//   - every workgroup reads the whole input vector of a stage, quantizes it into LDS (the
//     same arithmetic as the launch-per-stage kernels) and multiplies its rows; the MLGRU
//     step and g_norm are recomputed by every workgroup from the i|f|g vector and the state;
//     workgroup 0 writes the new state once every workgroup has read the old one (it has
//     seen all of the stage's outputs);
//   - every wait is bounded: past the deadline, or once another workgroup has reported a
//     timeout through the error word, the workgroup stops and the kernel ends; the caller
//     reads the error word (stack_decode_status).
// The tag is one more than the epoch word, which the last workgroup to finish increments,
// so the next launch on the same exchange area expects a new tag; the area is cleared once
// (stack_decode_init), so no stale word carries a current tag.
#include "mmf_internal.h"

namespace mmf {

namespace {

constexpr int kPT = 256;       // threads per workgroup
// weight units (64 weights, one 16-byte load) per thread for each stage's slice: registers
// hold only the slice of the next stage while a wait is pending
constexpr int kUIfg = 6, kUO = 2, kUGu = 10, kUDn = 6, kUHd = 16;
constexpr int kPMaxU = kUHd;
constexpr int kPMaxW = 16;     // exchange words (two values) per thread per input vector
constexpr int kPMaxWD = 8;     // the same for hidden-size vectors (D <= 4096)
constexpr int kPMaxK = 8192;   // widest BitLinear input
constexpr int kPMaxD = 4096;   // widest hidden size
constexpr int kPMaxRows = 128; // rows of one stage slice
static_assert(kPMaxRows <= 2 * kPT, "an epilogue handles its rows in one pass");

__device__ __forceinline__ uint64_t xch_load(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xch_store(uint64_t *p, uint32_t vals, uint32_t tag) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | vals, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ctl_load(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Red {   // block-reduction scratch
    float f[4][4];
    int i[4];
};

// max and sum of two per-thread floats over the workgroup (4 waves)
__device__ __forceinline__ void block_max_sum(float mx, float sm, Red &r, float &omx, float &osm) {
    mx = wave_max(mx);
    sm = wave_sum(sm);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        r.f[0][wave] = mx;
        r.f[1][wave] = sm;
    }
    __syncthreads();
    omx = fmaxf(fmaxf(r.f[0][0], r.f[0][1]), fmaxf(r.f[0][2], r.f[0][3]));
    osm = (r.f[1][0] + r.f[1][1]) + (r.f[1][2] + r.f[1][3]);
    __syncthreads();
}
__device__ __forceinline__ float block_sum(float v, Red &r) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) r.f[2][wave] = v;
    __syncthreads();
    const float t = (r.f[2][0] + r.f[2][1]) + (r.f[2][2] + r.f[2][3]);
    __syncthreads();
    return t;
}
__device__ __forceinline__ int block_sum_i(int v, Red &r) {
    v = wave_sum_i(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) r.i[wave] = v;
    __syncthreads();
    const int t = (r.i[0] + r.i[1]) + (r.i[2] + r.i[3]);
    __syncthreads();
    return t;
}

// A stage's weight slice: virtual rows [0, nr) of this workgroup, each a row of one of up to
// three [N][K] packed matrices: i|f|g (virtual row r0 + v of the concatenated 3D rows), one
// matrix (o, down, head), or gate|up pairs (v < np: gate row p0 + v, else up row p0 + v - np).
struct Slice {
    const uint32_t *m0, *m1, *m2;
    int K, N;        // K of the input, rows per matrix
    int r0, nr;      // first concatenated row (or pair p0) and virtual rows
    int pairs;       // 1: gate|up pairs (nr = 2 * pairs count)
    // The matrix is chosen by adding address differences, not by selecting among the fields:
    // a select of two field loads is folded into one load at a lane-dependent offset, which
    // sends the whole struct to scratch memory, and every scratch reload then waits for the
    // weight loads issued before it.
    __device__ __forceinline__ const uint32_t *row(int v) const {
        const intptr_t a0 = reinterpret_cast<intptr_t>(m0);
        const intptr_t d1 = reinterpret_cast<intptr_t>(m1) - a0, d2 = reinterpret_cast<intptr_t>(m2) - a0;
        int r;
        intptr_t a;
        if (pairs) {
            const int np = nr / 2;
            a = a0 + (v < np ? 0 : d1);
            r = r0 + (v < np ? v : v - np);
        } else {
            const int c = r0 + v;
            a = a0 + (c < N ? 0 : (c < 2 * N ? d1 : d2));
            r = c < N ? c : (c < 2 * N ? c - N : c - 2 * N);
        }
        return reinterpret_cast<const uint32_t *>(a) + static_cast<int64_t>(r) * (K / 16);
    }
};

template <int NU>
__device__ __forceinline__ void prefetch(const Slice &s, uint4 (&wv)[NU]) {
    // every register of the array is written (zero past the slice), so no earlier contents
    // stay live across the waits; units past the slice issue no load
    const int upr = s.K / 64, U = s.nr * upr;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = threadIdx.x + kPT * i;
        wv[i] = make_uint4(0u, 0u, 0u, 0u);
        if (u < U) wv[i] = *reinterpret_cast<const uint4 *>(s.row(u / upr) + 4 * (u % upr));
    }
}

// racc[v] += sum over this thread's units of row v (codes multiplied unmapped: the token's
// code sum is removed once per row in the epilogue)
template <int NU>
__device__ __forceinline__ void dot_slice(const Slice &s, const uint4 (&wv)[NU],
                                          const int8_t *xq, int *racc) {
    const int upr = s.K / 64, U = s.nr * upr;
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const int u = threadIdx.x + kPT * i;
        if (u < U) {
            const int v = u / upr, kb = u % upr;
            const uint32_t w[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            const v4i *xp = reinterpret_cast<const v4i *>(xq + 64 * kb);
            int acc = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4i x = xp[q];             // k = 64 kb + 16 q .. + 15
                const v4i c = unpack_codes(w[q]);
                acc = __builtin_amdgcn_sdot4(x.x, c.x, acc, false);
                acc = __builtin_amdgcn_sdot4(x.y, c.y, acc, false);
                acc = __builtin_amdgcn_sdot4(x.z, c.z, acc, false);
                acc = __builtin_amdgcn_sdot4(x.w, c.w, acc, false);
            }
            atomicAdd(&racc[v], acc);
        }
    }
}

}  // namespace

struct PState {   // per-workgroup LDS
    alignas(16) int8_t xq[kPMaxK];
    uint16_t xs[kPMaxD];    // the layer's input x (bf16 bits), for the o_proj residual
    uint16_t y1s[kPMaxD];   // the layer's y1 (bf16 bits), for the down residual
    int racc[kPMaxRows];
    alignas(16) float gain[kPMaxK + 256];      // the next quantizer's gain (+ 1 KB of slack)
    alignas(16) float vb[4][kPMaxD + 256];     // MLGRU step: h, forget bias, lower bound, g_norm weight
    Red red;
    float a;
    int rs;
};

namespace {

// Copy n floats (n % 4 == 0, src 16-byte aligned; nothing when src is NULL) into LDS at dst
// with direct 16-byte loads, 1 KB per wave instruction.  The copy lands asynchronously;
// wait_words (or an explicit vmcnt wait and barrier) orders it before the reads.  Lanes past
// the end re-read the last 16 bytes into dst's 1 KB of slack.
__device__ __forceinline__ void stage_vec(const float *src, int n, float *dst) {
    if (!src) return;
    const int bytes = 4 * n, chunks = (bytes + 1023) >> 10;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst));
    for (int c = wave; c < chunks; c += kPT / 64) {
        uint32_t off = static_cast<uint32_t>(c * 1024 + 16 * lane);
        off = off < static_cast<uint32_t>(bytes) ? off : static_cast<uint32_t>(bytes - 16);
        dma16(src, off, lds + static_cast<uint32_t>(c) * 1024u);
    }
}

// Bounded wait until every word of NB lists of n_words exchange words (list b at base + b *
// stride) carries the tag; word tid + 256 j of list b returns its value half in
// vals[b * NW + j].  The lists are polled together, so one memory round trip serves all.
// false (for the whole workgroup) on a timeout or a reported error.  Every direct-to-LDS copy
// issued before it has landed when it returns.
template <int NW, int NB = 1>
__device__ __forceinline__ bool wait_words(const uint64_t *base, int n_words, uint32_t tag,
                                           uint32_t *vals, const PersistArgs &p,
                                           int trace_slot = -1, int64_t stride = 0) {
    static_assert(NW * NB <= 32, "pending mask");
    const uint64_t t_in = __builtin_amdgcn_s_memrealtime();
    uint32_t pending = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            vals[b * NW + j] = 0u;
            if (static_cast<int>(threadIdx.x) + kPT * j < n_words) pending |= 1u << (b * NW + j);
        }
    }
    const uint64_t deadline = __builtin_amdgcn_s_memrealtime() + p.spin_ticks;
    bool ok = true;
    while (pending) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                if (pending & (1u << (b * NW + j))) {
                    const uint64_t w = xch_load(base + b * stride + threadIdx.x + kPT * j);
                    if (static_cast<uint32_t>(w >> 32) == tag) {
                        vals[b * NW + j] = static_cast<uint32_t>(w);
                        pending &= ~(1u << (b * NW + j));
                    }
                }
            }
        }
        if (!pending) break;
        if (__builtin_amdgcn_s_memrealtime() > deadline || ctl_load(p.ctl + 2) != 0) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(p.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmcnt<0>();   // this thread's direct-to-LDS copies have landed
    const bool all_ok = !__syncthreads_or(!ok);
    if (p.trace && trace_slot >= 0 && blockIdx.x == 0 && threadIdx.x == 0) {
        p.trace[2 * trace_slot] = t_in;
        p.trace[2 * trace_slot + 1] = __builtin_amdgcn_s_memrealtime();
    }
    return all_ok;
}

// Quantize the vector held as bf16 pairs in vals (word w = tid + 256 j holds elements 2w,
// 2w+1) with gain gamma into st.xq; sets st.a and st.rs.  Same arithmetic as the row
// quantizers: p = x*gamma, m = max|p| floored at 1e-5, q = rint(p * (127/m)) clamped,
// a = m/127 / sqrt(mean x^2 + eps).
template <int NW>
__device__ __forceinline__ void quantize_words(const uint32_t (&vals)[NW], int n, const float *gamma,
                                               float eps, PState &st) {
    float mx = 0.f, ss = 0.f;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int w = threadIdx.x + kPT * j;
        if (2 * w < n) {
            const float v0 = __uint_as_float(vals[j] << 16), v1 = __uint_as_float(vals[j] & 0xFFFF0000u);
            const float p0 = gamma ? v0 * gamma[2 * w] : v0, p1 = gamma ? v1 * gamma[2 * w + 1] : v1;
            mx = fmaxf(mx, fmaxf(fabsf(p0), fabsf(p1)));
            ss += v0 * v0;
            ss += v1 * v1;
        }
    }
    float m, s2;
    block_max_sum(mx, ss, st.red, m, s2);
    const float me = fmaxf(m, 1e-5f);
    const float sc = 127.0f / me;
    int qs = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int w = threadIdx.x + kPT * j;
        if (2 * w < n) {
            const float v0 = __uint_as_float(vals[j] << 16), v1 = __uint_as_float(vals[j] & 0xFFFF0000u);
            const float p0 = gamma ? v0 * gamma[2 * w] : v0, p1 = gamma ? v1 * gamma[2 * w + 1] : v1;
            const float q0 = fminf(fmaxf(rintf(p0 * sc), -127.0f), 127.0f);
            const float q1 = fminf(fmaxf(rintf(p1 * sc), -127.0f), 127.0f);
            qs += static_cast<int>(q0) + static_cast<int>(q1);
            st.xq[2 * w] = static_cast<int8_t>(q0);
            st.xq[2 * w + 1] = static_cast<int8_t>(q1);
        }
    }
    const int rs = block_sum_i(qs, st.red);
    if (threadIdx.x == 0) {
        st.a = me / 127.0f * (1.0f / sqrtf(s2 / static_cast<float>(n) + eps));
        st.rs = rs;
    }
    __syncthreads();
}

// rows [lo, hi) of n split over G workgroups, in units of `unit` rows
__device__ __forceinline__ void split(int n, int unit, int &lo, int &hi) {
    const int nu = n / unit, g = blockIdx.x, G = gridDim.x;
    lo = static_cast<int>(static_cast<int64_t>(g) * nu / G) * unit;
    hi = static_cast<int>(static_cast<int64_t>(g + 1) * nu / G) * unit;
}

// NWD / NWF: exchange words per thread of a hidden-size / GLU-size vector (two values each);
// the launch picks the smallest instance that covers D and F
template <int NWD, int NWF>
__global__ __launch_bounds__(kPT) void decode_persistent_kernel(PersistArgs p) {
    __shared__ PState st;
    const int tid = threadIdx.x;
    const int D = p.D, F = p.F, L = p.L;
    if (p.trace && blockIdx.x == 0 && tid == 0) p.trace[0] = p.trace[1] = __builtin_amdgcn_s_memrealtime();
    const uint32_t tag = ctl_load(p.ctl) + 1u;
    if (ctl_load(p.ctl + 2) != 0) return;   // an earlier launch timed out: nothing runs
    const int64_t lstride = static_cast<int64_t>(D / 2) * 5 + F / 2;   // exchange words per layer
    auto X = [&](int l) { return p.xch + l * lstride; };               // [D/2], layer input
    auto IFG = [&](int l) { return p.xch + l * lstride + D / 2; };     // [3D/2]
    auto Y1 = [&](int l) { return p.xch + l * lstride + 2 * D; };      // [D/2]
    auto M = [&](int l) { return p.xch + l * lstride + (5 * D) / 2; }; // [F/2]

    uint4 w_ifg[kUIfg], w_o[kUO], w_gu[kUGu], w_dn[kUDn], w_hd[kUHd];
    uint32_t vals[NWD], mvals[NWF];
    float hnew[NWD][2];

    // slices of this workgroup (the same for every layer)
    int ifg0, ifg1, o0, o1, gu0, gu1, dn0, dn1, hd0, hd1;
    split(3 * D, 2, ifg0, ifg1);
    split(D, 2, o0, o1);
    split(F, 2, gu0, gu1);          // GLU hidden values (gate|up pairs)
    split(D, 2, dn0, dn1);
    split(p.V, 1, hd0, hd1);
    auto slice_ifg = [&](const PLayer &ly) {
        return Slice{ly.w[0], ly.w[1], ly.w[2], D, D, ifg0, ifg1 - ifg0, 0};
    };
    auto slice_o = [&](const PLayer &ly) { return Slice{ly.w[3], ly.w[3], ly.w[3], D, D, o0, o1 - o0, 0}; };
    auto slice_gu = [&](const PLayer &ly) {
        return Slice{ly.w[4], ly.w[5], ly.w[5], D, F, gu0, 2 * (gu1 - gu0), 1};
    };
    auto slice_dn = [&](const PLayer &ly) { return Slice{ly.w[6], ly.w[6], ly.w[6], F, D, dn0, dn1 - dn0, 0}; };
    const Slice slice_hd{p.head, p.head, p.head, D, p.V, hd0, hd1 - hd0, 0};

    auto clear_acc = [&](int nr) {
        for (int v = tid; v < nr; v += kPT) st.racc[v] = 0;
    };
    // bias values of this thread's epilogue rows (v = 2 tid + e), read before the stage's wait
    float bp[4];
    auto bias_ifg = [&](const PLayer &ly) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = 0.0f;
        if (2 * tid < ifg1 - ifg0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = ifg0 + 2 * tid + e, seg = r / D;
                if (ly.b[seg]) bp[e] = ly.b[seg][r % D];
            }
        }
    };
    auto bias_rows = [&](const float *b, int r0, int nr) {   // o, down
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = 0.0f;
        if (b && 2 * tid < nr) {
            bp[0] = b[r0 + 2 * tid];
            bp[1] = b[r0 + 2 * tid + 1];
        }
    };
    auto bias_gu = [&](const PLayer &ly) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = 0.0f;
        if (2 * tid < gu1 - gu0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (ly.b[4]) bp[e] = ly.b[4][gu0 + 2 * tid + e];
                if (ly.b[5]) bp[2 + e] = ly.b[5][gu0 + 2 * tid + e];
            }
        }
    };
    auto bias_head = [&]() {
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = 0.0f;
        if (p.head_bias && tid < hd1 - hd0) bp[0] = p.head_bias[hd0 + tid];
    };

    prefetch(slice_ifg(p.layers[0]), w_ifg);
    stage_vec(p.layers[0].g_x, D, st.gain);
    bias_ifg(p.layers[0]);
    // ---- embedding: x0 = s_E * q_E[id], rounded to bf16 (every workgroup builds it)
    {
        const int id = p.ids[0];
        const bool idv = id >= 0 && id < p.vocab;
        const uint32_t *er = p.emb + static_cast<int64_t>(idv ? id : 0) * (D / 16);
#pragma unroll
        for (int j = 0; j < NWD; ++j) {
            const int w = tid + kPT * j;
            if (2 * w < D) {
                uint32_t pr = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = 2 * w + e;
                    const uint32_t code = (er[k / 16] >> (8 * (k % 4) + 2 * ((k % 16) / 4))) & 3u;
                    const float v = idv ? static_cast<float>(static_cast<int>(code) - 1) * p.emb_scale : 0.0f;
                    pr |= static_cast<uint32_t>(f32_to_bf16_bits(v)) << (16 * e);
                }
                vals[j] = pr;
            }
        }
    }
    wait_vmcnt<0>();   // layer 0 has no wait: land its gain copy here
    __syncthreads();

    for (int l = 0; l < L; ++l) {
        const PLayer &ly = p.layers[l];
        // ================= stage A: i|f|g = BitLinear(x)
        if (l > 0 && !wait_words<NWD>(X(l), D / 2, tag, vals, p, 4 * l)) return;
#pragma unroll
        for (int j = 0; j < NWD; ++j) {
            const int w = tid + kPT * j;
            if (2 * w < D) *reinterpret_cast<uint32_t *>(st.xs + 2 * w) = vals[j];
        }
        clear_acc(ifg1 - ifg0);
        quantize_words(vals, D, ly.g_x ? st.gain : nullptr, ly.e_x, st);
        {
            const Slice s = slice_ifg(ly);
            dot_slice(s, w_ifg, st.xq, st.racc);
            __syncthreads();
            const float a = st.a;
            const int rs = st.rs;
            const int v = 2 * tid;
            if (v < s.nr) {
                uint32_t pr = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int seg = (ifg0 + v + e) / D;
                    const float y = static_cast<float>(st.racc[v + e] - rs) * (ly.s[seg] * a) + bp[e];
                    pr |= static_cast<uint32_t>(f32_to_bf16_bits(y)) << (16 * e);
                }
                xch_store(IFG(l) + (ifg0 + v) / 2, pr, tag);
            }
        }
        // next: o_proj's slice, its gain, the MLGRU step's vectors, o's bias values
        prefetch(slice_o(ly), w_o);
        stage_vec(ly.g_o, D, st.gain);
        stage_vec(p.h_state + static_cast<int64_t>(l) * D, D, st.vb[0]);
        stage_vec(ly.f_bias, D, st.vb[1]);
        stage_vec(ly.f_lower, D, st.vb[2]);
        stage_vec(ly.gnorm_w, D, st.vb[3]);
        bias_rows(ly.b[3], o0, o1 - o0);

        // ================= stage B: MLGRU step, g_norm, o_proj + residual
        {
            // thread word w covers channels 2w, 2w+1: i at IFG[w], f at IFG[D/2 + w], g at
            // IFG[D + w]; the three lists are polled together
            uint32_t vifg[3 * NWD];
            if (!wait_words<NWD, 3>(IFG(l), D / 2, tag, vifg, p, 4 * l + 1, D / 2)) return;
            const uint32_t *vi = vifg, *vf = vifg + NWD, *vg = vifg + 2 * NWD;
            float hsum = 0.f;
#pragma unroll
            for (int j = 0; j < NWD; ++j) {
                const int w = tid + kPT * j;
                hnew[j][0] = hnew[j][1] = 0.f;
                if (2 * w < D) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int d = 2 * w + e;
                        const float iv = __uint_as_float(e ? vi[j] & 0xFFFF0000u : vi[j] << 16);
                        const float fv = __uint_as_float(e ? vf[j] & 0xFFFF0000u : vf[j] << 16);
                        const float fb = ly.f_bias ? st.vb[1][d] : 0.0f;
                        const float lb = ly.f_lower ? st.vb[2][d] : 0.0f;
                        const float f = fmaf(1.0f - lb, sigmoidf_(fv + fb), lb);
                        const float h = f * st.vb[0][d] + (1.0f - f) * siluf_(iv);
                        hnew[j][e] = h;
                        hsum = fmaf(h, h, hsum);
                    }
                }
            }
            const float htot = block_sum(hsum, st.red);
            const float r = 1.0f / sqrtf(htot * (1.0f / static_cast<float>(D)) + ly.g_eps);
            // g_norm output, materialised in bf16, held as pairs in vals for the quantizer
#pragma unroll
            for (int j = 0; j < NWD; ++j) {
                const int w = tid + kPT * j;
                if (2 * w < D) {
                    float o[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int d = 2 * w + e;
                        const float gv = __uint_as_float(e ? vg[j] & 0xFFFF0000u : vg[j] << 16);
                        const float gw = ly.gnorm_w ? st.vb[3][d] : 1.0f;
                        o[e] = ly.gate_mode == 0 ? hnew[j][e] * r * gw * siluf_(gv) : sigmoidf_(gv) * hnew[j][e];
                    }
                    vals[j] = pack_bf16x2(o[0], o[1]);
                }
            }
        }
        clear_acc(o1 - o0);
        quantize_words(vals, D, ly.g_o ? st.gain : nullptr, ly.e_o, st);
        {
            const Slice s = slice_o(ly);
            dot_slice(s, w_o, st.xq, st.racc);
            __syncthreads();
            const float a = st.a;
            const int rs = st.rs;
            const int v = 2 * tid;
            if (v < s.nr) {
                uint32_t pr = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int n = o0 + v + e;
                    float y = static_cast<float>(st.racc[v + e] - rs) * (ly.s[3] * a) + bp[e];
                    y = __uint_as_float(static_cast<uint32_t>(st.xs[n]) << 16) + y;
                    pr |= static_cast<uint32_t>(f32_to_bf16_bits(y)) << (16 * e);
                }
                xch_store(Y1(l) + (o0 + v) / 2, pr, tag);
            }
        }
        prefetch(slice_gu(ly), w_gu);
        stage_vec(ly.g_gu, D, st.gain);
        bias_gu(ly);

        // ================= stage C: gate|up, SiLU(gate) * up
        if (!wait_words<NWD>(Y1(l), D / 2, tag, vals, p, 4 * l + 2)) return;
        if (blockIdx.x == 0) {   // every workgroup has read the old state: store the new one
            float *hd = p.h_state + static_cast<int64_t>(l) * D;
#pragma unroll
            for (int j = 0; j < NWD; ++j) {
                const int w = tid + kPT * j;
                if (2 * w < D) *reinterpret_cast<float2 *>(hd + 2 * w) = make_float2(hnew[j][0], hnew[j][1]);
            }
        }
#pragma unroll
        for (int j = 0; j < NWD; ++j) {
            const int w = tid + kPT * j;
            if (2 * w < D) *reinterpret_cast<uint32_t *>(st.y1s + 2 * w) = vals[j];
        }
        clear_acc(2 * (gu1 - gu0));
        quantize_words(vals, D, ly.g_gu ? st.gain : nullptr, ly.e_gu, st);
        {
            const Slice s = slice_gu(ly);
            dot_slice(s, w_gu, st.xq, st.racc);
            __syncthreads();
            const float a = st.a;
            const int rs = st.rs, np = s.nr / 2;
            const int v = 2 * tid;
            if (v < np) {
                uint32_t pr = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float yg = static_cast<float>(st.racc[v + e] - rs) * (ly.s[4] * a) + bp[e];
                    const float yu = static_cast<float>(st.racc[np + v + e] - rs) * (ly.s[5] * a) + bp[2 + e];
                    pr |= static_cast<uint32_t>(f32_to_bf16_bits(siluf_(yg) * yu)) << (16 * e);
                }
                xch_store(M(l) + (gu0 + v) / 2, pr, tag);
            }
        }
        prefetch(slice_dn(ly), w_dn);
        stage_vec(ly.g_down, F, st.gain);
        bias_rows(ly.b[6], dn0, dn1 - dn0);

        // ================= stage D: down + residual -> next layer's input
        if (!wait_words<NWF>(M(l), F / 2, tag, mvals, p, 4 * l + 3)) return;
        clear_acc(dn1 - dn0);
        quantize_words(mvals, F, ly.g_down ? st.gain : nullptr, ly.e_down, st);
        {
            const Slice s = slice_dn(ly);
            dot_slice(s, w_dn, st.xq, st.racc);
            __syncthreads();
            const float a = st.a;
            const int rs = st.rs;
            const int v = 2 * tid;
            if (v < s.nr) {
                uint32_t pr = 0;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int n = dn0 + v + e;
                    float y = static_cast<float>(st.racc[v + e] - rs) * (ly.s[6] * a) + bp[e];
                    y = __uint_as_float(static_cast<uint32_t>(st.y1s[n]) << 16) + y;
                    pr |= static_cast<uint32_t>(f32_to_bf16_bits(y)) << (16 * e);
                }
                xch_store(X(l + 1) + (dn0 + v) / 2, pr, tag);
                if (l == L - 1 && p.y) *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.y) + dn0 + v) = pr;
            }
        }
        if (l + 1 < L) {
            prefetch(slice_ifg(p.layers[l + 1]), w_ifg);
            stage_vec(p.layers[l + 1].g_x, D, st.gain);
            bias_ifg(p.layers[l + 1]);
        } else {
            prefetch(slice_hd, w_hd);
            stage_vec(p.head_gamma, D, st.gain);
            bias_head();
        }
    }

    // ================= head: logits = BitLinear(x_L)
    if (p.logits) {
        if (!wait_words<NWD>(X(L), D / 2, tag, vals, p, 4 * L)) return;
        clear_acc(hd1 - hd0);
        quantize_words(vals, D, p.head_gamma ? st.gain : nullptr, p.head_eps, st);
        dot_slice(slice_hd, w_hd, st.xq, st.racc);
        __syncthreads();
        const float a = st.a;
        const int rs = st.rs;
        if (tid < hd1 - hd0) p.logits[hd0 + tid] = static_cast<float>(st.racc[tid] - rs) * (p.head_scale * a) + bp[0];
    }
    if (p.trace && blockIdx.x == 0 && tid == 0) {   // end of this workgroup's work
        p.trace[2 * (4 * L + 1)] = __builtin_amdgcn_s_memrealtime();
        p.trace[2 * (4 * L + 1) + 1] = 0;
    }
    // ---- the last workgroup to finish moves the epoch on (the next launch's tag)
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(p.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {
            __hip_atomic_store(p.ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p.ctl, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

int persist_max_units(int rows, int K) { return (rows * (K / 64) + kPT - 1) / kPT; }
void persist_stage_units(int (&u)[5]) {
    u[0] = kUIfg; u[1] = kUO; u[2] = kUGu; u[3] = kUDn; u[4] = kUHd;
}
int persist_limits(int *max_units, int *max_words, int *max_k, int *max_d, int *max_rows) {
    *max_units = kPMaxU;
    *max_words = kPMaxW;
    *max_k = kPMaxK;
    *max_d = kPMaxD;
    *max_rows = kPMaxRows;
    return kPT;
}

namespace {
using PersistKernel = void (*)(PersistArgs);
// the instance for hidden size D and GLU size F
PersistKernel persist_kernel(int D, int F) {
    if (D <= 2 * kPT * 4 && F <= 2 * kPT * 12) return decode_persistent_kernel<4, 12>;
    return decode_persistent_kernel<kPMaxWD, kPMaxW>;
}
}  // namespace

hipError_t launch_decode_persistent(const PersistArgs &a, int grid, hipStream_t s) {
    timing_begin(FAM_GEMV, s);
    void *args[] = {const_cast<PersistArgs *>(&a)};
    const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void *>(persist_kernel(a.D, a.F)),
                                                    dim3(grid), dim3(kPT), args, 0, s);
    timing_end(FAM_GEMV, s);
    return e;
}

int persist_occupancy(int D, int F, int *blocks_per_cu) {
    return static_cast<int>(hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, reinterpret_cast<const void *>(persist_kernel(D, F)), kPT, 0));
}

}  // namespace mmf
