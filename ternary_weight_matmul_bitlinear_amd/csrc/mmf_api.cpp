// mmf_api.cpp -- C ABI of libmmf: argument validation, workspace carving, regime choice and
// the launch sequences of BitLinear, MLGRU, GLU, block and stack forward passes.
//
// Hysen Labs "MatMul-Free LM", sections "FusedBitLinear" and "HGRN attention": a block is
// RMSNorm -> i/f/g BitLinears -> gated recurrence -> g_norm -> o_proj, each BitLinear
// normalising, quantizing and accumulating its input.  DataCamp "MatMul-free language
// models", section "Core components: MLGRU and GLU": the GLU channel mixer follows.
// Residuals are pre-norm: y1 = x + o_proj(...), y = y1 + GLU(y1).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>
#include <atomic>
#include <algorithm>

#include "mmf_internal.h"

namespace mmf {

// ------------------------------------------------------------------ error state
static thread_local std::string g_err;

int set_error(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

static int hip_error(hipError_t e, const char *where) {
    return set_error(MMF_EHIP, "%s: %s", where, hipGetErrorString(e));
}

// ------------------------------------------------------------------ device check
static std::mutex g_dev_mu;
static std::vector<int> g_dev_ok;  // -1 unknown, 0 not gfx950, 1 gfx950

static int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "hipGetDevice");
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (dev < static_cast<int>(g_dev_ok.size()) && g_dev_ok[dev] >= 0)
            return g_dev_ok[dev] ? MMF_OK : set_error(MMF_EDEVICE, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_error(e, "hipGetDeviceProperties");
    const int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    {
        std::lock_guard<std::mutex> lk(g_dev_mu);
        if (dev >= static_cast<int>(g_dev_ok.size())) g_dev_ok.resize(dev + 1, -1);
        g_dev_ok[dev] = ok;
    }
    return ok ? MMF_OK : set_error(MMF_EDEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
}

// ------------------------------------------------------------------ regime knob
static std::atomic<int> g_regime{0};
// Token rows up to which the weight-streaming decode kernel is used.
constexpr int64_t kDecodeMaxM = 4;

static bool use_decode(int64_t m) {
    const int r = g_regime.load();
    if (r == 1) return true;
    if (r >= 2) return false;
    return m <= kDecodeMaxM;
}

// ------------------------------------------------------------------ timing
struct TimingFamily {
    std::vector<hipEvent_t> ev;  // pairs (start, stop)
    size_t used = 0;
    int64_t launches = 0;
};
static std::mutex g_tmu;
static bool g_timing = false;
static uint32_t g_timing_mask = 0xFFFFFFFFu;  // families that record events while enabled
static TimingFamily g_fam[FAM_COUNT];
static const char *kFamNames[FAM_COUNT] = {"quant", "gemm_ifg", "gemm_o", "gemm_gateup",
                                           "gemm_down", "gemm", "gemv", "scan", "embed"};
static thread_local hipEvent_t t_pending = nullptr;

void timing_begin(int family, hipStream_t s) {
    if (!g_timing || !((g_timing_mask >> family) & 1u)) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    TimingFamily &f = g_fam[family];
    if (f.used + 2 > f.ev.size()) {
        for (int i = 0; i < 64; ++i) {
            // timing-only events: no system-scope fence (cache writeback and invalidate) when
            // they are recorded, so they perturb the timed stream as little as possible
            hipEvent_t e;
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
            f.ev.push_back(e);
        }
    }
    t_pending = f.ev[f.used];
    hipEventRecord(t_pending, s);
}

void timing_end(int family, hipStream_t s) {
    if (!g_timing || !t_pending) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    TimingFamily &f = g_fam[family];
    hipEventRecord(f.ev[f.used + 1], s);
    f.used += 2;
    f.launches += 1;
    t_pending = nullptr;
}

// ------------------------------------------------------------------ helpers
static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }
static bool valid_dt(int dt) { return dt == MMF_F32 || dt == MMF_BF16; }
static size_t dt_size(int dt) { return dt == MMF_BF16 ? 2 : 4; }

struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(size_t bytes) {
        T *p = reinterpret_cast<T *>(base ? base + off : nullptr);
        off += align_up(bytes);
        return p;
    }
};

static int check_linear(const mmf_bitlinear *w, const char *name) {
    if (!w) return set_error(MMF_EINVAL, "%s: NULL descriptor", name);
    if (!w->packed) return set_error(MMF_EINVAL, "%s: NULL packed weights", name);
    if (w->K <= 0 || w->N <= 0) return set_error(MMF_ESHAPE, "%s: K=%d N=%d", name, w->K, w->N);
    if (w->K % 64) return set_error(MMF_ESHAPE, "%s: K=%d is not a multiple of 64", name, w->K);
    if (w->K > 32768) return set_error(MMF_ESHAPE, "%s: K=%d exceeds 32768", name, w->K);
    if (!aligned16(w->packed)) return set_error(MMF_EALIGN, "%s: packed weights not 16-byte aligned", name);
    if (!(w->eps >= 0.0f)) return set_error(MMF_EINVAL, "%s: eps must be >= 0", name);
    return MMF_OK;
}

static CapDev cap_of(const mmf_stage_capture *c, int32_t acc_ld) {
    CapDev d;
    if (!c) return d;
    d.row0 = c->row0;
    d.row1 = c->row1;
    d.x_in = c->x_in;
    d.q = c->q;
    d.a = c->a;
    d.acc = c->acc;
    d.y_out = c->y_out;
    d.acc_ld = acc_ld;
    return d;
}

static int check_cap(const mmf_stage_capture *c, const char *name) {
    if (!c) return MMF_OK;
    if (c->row0 < 0 || c->row1 < c->row0) return set_error(MMF_EINVAL, "%s capture: bad window [%lld, %lld)", name, (long long)c->row0, (long long)c->row1);
    return MMF_OK;
}

static Seg seg_of(const mmf_bitlinear &w, int32_t out_col0, int32_t cap_col0) {
    Seg s;
    s.packed = w.packed;
    s.bias = w.bias;
    s.scale = w.scale;
    s.n = w.N;
    s.out_col0 = out_col0;
    s.cap_col0 = cap_col0;
    return s;
}

// Quantize rows of x into the int8 scratch (prefill path).
struct QBuf {
    int8_t *q;
    float *a;
    int32_t *rs;
};

static hipError_t quantize(const void *x, bool bf16, const float *gamma, float eps, int64_t M,
                           int32_t K, const QBuf &qb, const mmf_stage_capture *cap,
                           hipStream_t s) {
    QuantArgs qa{};
    qa.x = x;
    qa.x_bf16 = bf16;
    qa.gamma = gamma;
    qa.eps = eps;
    qa.M = M;
    qa.K = K;
    qa.q = qb.q;
    qa.a = qb.a;
    qa.rowsum = qb.rs;
    qa.cap = cap_of(cap, 0);
    qa.cap.acc = nullptr;
    qa.cap.y_out = nullptr;
    return launch_quant(qa, s);
}

// Prefill GEMM from quantized rows.
static hipError_t gemm(const QBuf &qb, int64_t M, int32_t K, const Seg *segs, int nseg, int epi,
                       void *out, int32_t ldo, bool out_bf16, const void *resid, int32_t ldr,
                       const mmf_stage_capture *cap, int32_t cap_ld, int family, hipStream_t s) {
    GemmArgs ga{};
    ga.A = qb.q;
    ga.rowsum = qb.rs;
    ga.a = qb.a;
    ga.M = M;
    ga.K = K;
    for (int i = 0; i < nseg; ++i) ga.seg[i] = segs[i];
    ga.nseg = nseg;
    ga.epi = epi;
    ga.out = out;
    ga.ldo = ldo;
    ga.out_bf16 = out_bf16;
    ga.resid = resid;
    ga.ldr = ldr;
    ga.cap = cap_of(cap, cap_ld);
    ga.cap.x_in = nullptr;
    ga.cap.q = nullptr;
    ga.cap.a = nullptr;
    ga.family = family;
    // up to kMidMaxM rows: the k-split kernel that reads the weights once (regime 3 forces
    // the 128-row tiles at any M)
    if (g_regime.load() != 3 && M <= kMidMaxM && mid_gemm_supported(ga)) return launch_gemm_mid(ga, s);
    return launch_gemm(ga, s);
}

// Extras of a decode GEMV: the fused MLGRU step of o_proj and a side copy of the state.
struct GemvExtra {
    const float *h_prev = nullptr;
    float *h_new = nullptr;
    const float *f_bias = nullptr;
    const float *gnorm_w = nullptr;
    float g_eps = 0.f;
    int32_t gate_mode = 0;
    bool mlgru = false;
    const float *copy_src = nullptr;
    float *copy_dst = nullptr;
    int32_t copy_n = 0;
};

// Decode GEMV, from raw activations (x != NULL) or from quantized rows.
static hipError_t gemv(const void *x, bool x_bf16, const float *gamma, float eps, const QBuf *qb,
                       int64_t M, int32_t K, const Seg *segs, int nseg, int epi, void *out,
                       int32_t ldo, bool out_bf16, const void *resid, int32_t ldr,
                       const mmf_stage_capture *cap, int32_t cap_ld, hipStream_t s,
                       const GemvExtra *ex = nullptr) {
    GemvArgs ga{};
    if (ex) {
        ga.mlgru = ex->mlgru;
        ga.h_prev = ex->h_prev;
        ga.h_new = ex->h_new;
        ga.f_bias = ex->f_bias;
        ga.gnorm_w = ex->gnorm_w;
        ga.g_eps = ex->g_eps;
        ga.gate_mode = ex->gate_mode;
        ga.copy_src = ex->copy_src;
        ga.copy_dst = ex->copy_dst;
        ga.copy_n = ex->copy_n;
    }
    ga.x = x;
    ga.x_bf16 = x_bf16;
    ga.gamma = gamma;
    ga.eps = eps;
    if (qb) {
        ga.q = qb->q;
        ga.a = qb->a;
        ga.rowsum = qb->rs;
    }
    ga.M = M;
    ga.K = K;
    int rows = 0;
    for (int i = 0; i < nseg; ++i) {
        ga.seg[i] = segs[i];
        rows += segs[i].n;
    }
    ga.nseg = nseg;
    ga.rows_total = epi == EPI_GLU ? segs[0].n : rows;
    ga.epi = epi;
    ga.out = out;
    ga.ldo = ldo;
    ga.out_bf16 = out_bf16;
    ga.resid = resid;
    ga.ldr = ldr;
    ga.cap = cap_of(cap, cap_ld);
    if (!x) {  // x_in/q/a were recorded by the producer of the quantized rows
        ga.cap.x_in = nullptr;
        ga.cap.q = nullptr;
        ga.cap.a = nullptr;
    }
    return launch_gemv(ga, s);
}

static size_t qbuf_bytes(int64_t M, int64_t K) {
    return align_up(static_cast<size_t>(M) * K) + 2 * align_up(static_cast<size_t>(M) * 4);
}
static QBuf take_qbuf(Carver &c, int64_t M, int64_t K) {
    QBuf q;
    q.q = c.take<int8_t>(static_cast<size_t>(M) * K);
    q.a = c.take<float>(static_cast<size_t>(M) * 4);
    q.rs = c.take<int32_t>(static_cast<size_t>(M) * 4);
    return q;
}

static int64_t scan_chunks(int64_t T) { return (T + kScanChunk - 1) / kScanChunk; }
static size_t scan_bytes(int64_t B, int64_t T, int64_t D) {
    const int64_t nc = scan_chunks(T);
    if (nc <= 1) return 0;
    return 3 * align_up(static_cast<size_t>(B * nc * D) * 4);
}

}  // namespace mmf

using namespace mmf;

// =================================================================== C ABI
extern "C" {

int mmf_abi_version(void) { return MMF_ABI_VERSION; }

const char *mmf_last_error(void) { return g_err.c_str(); }

int mmf_set_regime(int regime) {
    if (regime < 0 || regime > 3) return set_error(MMF_EINVAL, "mmf_set_regime: %d", regime);
    return g_regime.exchange(regime);
}

int mmf_timing_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return MMF_OK;
}

int mmf_timing_families(uint32_t mask) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing_mask = mask;
    return MMF_OK;
}

int mmf_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &f : g_fam) {
        f.used = 0;
        f.launches = 0;
    }
    return MMF_OK;
}

int mmf_timing_count(void) { return FAM_COUNT; }

const char *mmf_timing_name(int i) { return (i >= 0 && i < FAM_COUNT) ? kFamNames[i] : nullptr; }

int mmf_timing_query(const char *family, int64_t *launches, double *total_ms) {
    if (!family || !launches || !total_ms) return set_error(MMF_EINVAL, "mmf_timing_query: NULL argument");
    std::lock_guard<std::mutex> lk(g_tmu);
    for (int i = 0; i < FAM_COUNT; ++i) {
        if (std::strcmp(family, kFamNames[i])) continue;
        double tot = 0.0;
        for (size_t k = 0; k + 1 < g_fam[i].used; k += 2) {
            float ms = 0.f;
            hipError_t e = hipEventElapsedTime(&ms, g_fam[i].ev[k], g_fam[i].ev[k + 1]);
            if (e != hipSuccess) return hip_error(e, "hipEventElapsedTime");
            tot += ms;
        }
        *launches = g_fam[i].launches;
        *total_ms = tot;
        return MMF_OK;
    }
    return set_error(MMF_EINVAL, "mmf_timing_query: unknown family '%s'", family);
}

// ------------------------------------------------------------------ BitLinear
size_t bitlinear_workspace_bytes(const mmf_bitlinear *w, int64_t m) {
    if (!w || m <= 0 || w->K <= 0) return 0;
    return qbuf_bytes(m, w->K);
}

int bitlinear_forward(const mmf_bitlinear *w, const void *x, mmf_dtype x_dt, int64_t m, void *y,
                      mmf_dtype y_dt, void *ws, size_t ws_bytes, const mmf_stage_capture *cap,
                      hipStream_t stream) {
    int rc = check_linear(w, "bitlinear_forward");
    if (rc) return rc;
    if (!valid_dt(x_dt) || !valid_dt(y_dt)) return set_error(MMF_EDTYPE, "bitlinear_forward: dtype %d/%d", x_dt, y_dt);
    if (m < 0) return set_error(MMF_ESHAPE, "bitlinear_forward: m=%lld", (long long)m);
    if ((rc = check_cap(cap, "bitlinear_forward"))) return rc;
    if (m == 0) return MMF_OK;
    if (!x || !y) return set_error(MMF_EINVAL, "bitlinear_forward: NULL x or y");
    if (!aligned16(x) || !aligned16(y)) return set_error(MMF_EALIGN, "bitlinear_forward: x or y not 16-byte aligned");
    const bool decode = use_decode(m);
    const size_t need = bitlinear_workspace_bytes(w, m);
    if (!decode) {
        if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "bitlinear_forward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
        if (!aligned16(ws)) return set_error(MMF_EALIGN, "bitlinear_forward: workspace not 16-byte aligned");
    }
    if ((rc = check_device())) return rc;
    const Seg seg = seg_of(*w, 0, 0);
    hipError_t e;
    if (decode) {
        e = gemv(x, x_dt == MMF_BF16, w->norm_w, w->eps, nullptr, m, w->K, &seg, 1, EPI_STORE, y,
                 w->N, y_dt == MMF_BF16, nullptr, 0, cap, w->N, stream);
        if (e != hipSuccess) return hip_error(e, "bitlinear_forward decode launch");
        return MMF_OK;
    }
    Carver c(ws);
    const QBuf qb = take_qbuf(c, m, w->K);
    e = quantize(x, x_dt == MMF_BF16, w->norm_w, w->eps, m, w->K, qb, cap, stream);
    if (e != hipSuccess) return hip_error(e, "bitlinear_forward quantize launch");
    e = gemm(qb, m, w->K, &seg, 1, EPI_STORE, y, w->N, y_dt == MMF_BF16, nullptr, 0, cap, w->N,
             FAM_GEMM_OTHER, stream);
    if (e != hipSuccess) return hip_error(e, "bitlinear_forward gemm launch");
    return MMF_OK;
}

// ------------------------------------------------------------------ MLGRU
size_t mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D) {
    if (B <= 0 || T <= 0 || D <= 0) return 0;
    return scan_bytes(B, T, D);
}

static int check_scan_shape(int64_t B, int64_t T, int64_t D, const char *who) {
    if (B < 0 || T < 0 || D <= 0) return set_error(MMF_ESHAPE, "%s: B=%lld T=%lld D=%lld", who, (long long)B, (long long)T, (long long)D);
    if (D % 64 || D > 4096) return set_error(MMF_ESHAPE, "%s: D=%lld must be a multiple of 64 and <= 4096", who, (long long)D);
    return MMF_OK;
}

int mlgru_scan(const mmf_mlgru_args *a, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!a) return set_error(MMF_EINVAL, "mlgru_scan: NULL args");
    int rc = check_scan_shape(a->B, a->T, a->D, "mlgru_scan");
    if (rc) return rc;
    if (!valid_dt(a->ifg_dt) || !valid_dt(a->out_dt)) return set_error(MMF_EDTYPE, "mlgru_scan: dtype");
    if (a->gate_mode != MMF_GATE_SWISH_RMSNORM && a->gate_mode != MMF_GATE_SIGMOID) return set_error(MMF_EINVAL, "mlgru_scan: gate_mode %d", a->gate_mode);
    if (!(a->eps >= 0.0f)) return set_error(MMF_EINVAL, "mlgru_scan: eps");
    const int64_t M = a->B * a->T;
    if (M > 0 && (!a->ifg || !a->out)) return set_error(MMF_EINVAL, "mlgru_scan: NULL ifg or out");
    if (M > 0 && (!aligned16(a->ifg) || !aligned16(a->out))) return set_error(MMF_EALIGN, "mlgru_scan: ifg/out not 16-byte aligned");
    if ((a->h0 && !aligned16(a->h0)) || (a->h_out && !aligned16(a->h_out)) ||
        (a->f_bias && !aligned16(a->f_bias)) || (a->gnorm_w && !aligned16(a->gnorm_w)))
        return set_error(MMF_EALIGN, "mlgru_scan: h0/h_out/f_bias/gnorm_w not 16-byte aligned");
    const size_t need = mlgru_workspace_bytes(a->B, a->T, a->D);
    if (need && (!ws || ws_bytes < need)) return set_error(MMF_EWORKSPACE, "mlgru_scan: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if ((rc = check_device())) return rc;
    hipError_t e;
    if (M == 0) {  // h_T = h_0
        if (a->B > 0 && a->h_out && a->h_out != a->h0) {
            e = launch_copy_state(a->h0, a->h_out, a->B * a->D, stream);
            if (e != hipSuccess) return hip_error(e, "mlgru_scan copy launch");
        }
        return MMF_OK;
    }
    ScanArgs s{};
    s.ifg = a->ifg;
    s.ifg_bf16 = a->ifg_dt == MMF_BF16;
    s.f_bias = a->f_bias;
    s.h0 = a->h0;
    s.h_out = a->h_out;
    s.gnorm_w = a->gnorm_w;
    s.eps = a->eps;
    s.gate_mode = a->gate_mode;
    s.B = a->B;
    s.T = a->T;
    s.D = static_cast<int32_t>(a->D);
    s.chunk = kScanChunk;
    s.n_chunks = static_cast<int32_t>(scan_chunks(a->T));
    Carver c(ws);
    if (s.n_chunks > 1) {
        const size_t n = static_cast<size_t>(a->B * s.n_chunks * a->D) * 4;
        s.hloc = c.take<float>(n);
        s.pf = c.take<float>(n);
        s.hin = c.take<float>(n);
    }
    s.out = a->out;
    s.out_bf16 = a->out_dt == MMF_BF16;
    e = launch_scan(s, stream);
    if (e != hipSuccess) return hip_error(e, "mlgru_scan launch");
    return MMF_OK;
}

// ------------------------------------------------------------------ GLU
static int check_glu(const mmf_bitlinear *gate, const mmf_bitlinear *up, const mmf_bitlinear *down,
                     const char *who) {
    int rc;
    if ((rc = check_linear(gate, "gate")) || (rc = check_linear(up, "up")) || (rc = check_linear(down, "down"))) return rc;
    if (gate->K != up->K || gate->N != up->N || down->K != gate->N || down->N != gate->K)
        return set_error(MMF_ESHAPE, "%s: gate [%d,%d] up [%d,%d] down [%d,%d] do not chain", who, gate->N, gate->K, up->N, up->K, down->N, down->K);
    if (gate->norm_w != up->norm_w || gate->eps != up->eps)
        return set_error(MMF_EINVAL, "%s: gate and up must share norm_w and eps", who);
    return MMF_OK;
}

size_t glu_workspace_bytes(const mmf_bitlinear *gate, const mmf_bitlinear *down, int64_t m) {
    if (!gate || !down || m <= 0) return 0;
    const int64_t D = gate->K, F = gate->N;
    return qbuf_bytes(m, std::max(D, F)) + align_up(static_cast<size_t>(m * F) * 4);
}

int glu_forward(const mmf_bitlinear *gate, const mmf_bitlinear *up, const mmf_bitlinear *down,
                const void *x, mmf_dtype dt, int64_t m, const void *residual, void *y, void *ws,
                size_t ws_bytes, const mmf_capture *cap, hipStream_t stream) {
    int rc = check_glu(gate, up, down, "glu_forward");
    if (rc) return rc;
    if (!valid_dt(dt)) return set_error(MMF_EDTYPE, "glu_forward: dtype %d", dt);
    if (m < 0) return set_error(MMF_ESHAPE, "glu_forward: m=%lld", (long long)m);
    if (cap && ((rc = check_cap(&cap->gateup, "gateup")) || (rc = check_cap(&cap->down, "down")))) return rc;
    if (m == 0) return MMF_OK;
    if (!x || !y) return set_error(MMF_EINVAL, "glu_forward: NULL x or y");
    if (!aligned16(x) || !aligned16(y) || (residual && !aligned16(residual))) return set_error(MMF_EALIGN, "glu_forward: x/y/residual not 16-byte aligned");
    const size_t need = glu_workspace_bytes(gate, down, m);
    if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "glu_forward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "glu_forward: workspace not 16-byte aligned");
    if ((rc = check_device())) return rc;
    const int32_t D = gate->K, F = gate->N;
    const bool bf = dt == MMF_BF16;
    Carver c(ws);
    const QBuf qb = take_qbuf(c, m, std::max(D, F));
    void *mact = c.take<char>(static_cast<size_t>(m * F) * 4);
    const Seg gu[2] = {seg_of(*gate, 0, 0), seg_of(*up, 0, F)};
    const Seg dn = seg_of(*down, 0, 0);
    const int epi_dn = residual ? EPI_RESID : EPI_STORE;
    const mmf_stage_capture *cg = cap ? &cap->gateup : nullptr, *cd = cap ? &cap->down : nullptr;
    hipError_t e;
    // the GLU hidden m is stored in the activation dtype between the two kernels
    if (use_decode(m)) {
        e = gemv(x, bf, gate->norm_w, gate->eps, nullptr, m, D, gu, 2, EPI_GLU, mact, F, bf, nullptr, 0, cg, 2 * F, stream);
        if (e == hipSuccess)
            e = gemv(mact, bf, down->norm_w, down->eps, nullptr, m, F, &dn, 1, epi_dn, y, D, bf, residual, D, cd, D, stream);
    } else {
        e = quantize(x, bf, gate->norm_w, gate->eps, m, D, qb, cg, stream);
        if (e == hipSuccess)
            e = gemm(qb, m, D, gu, 2, EPI_GLU, mact, F, bf, nullptr, 0, cg, 2 * F, FAM_GEMM_GATEUP, stream);
        if (e == hipSuccess) e = quantize(mact, bf, down->norm_w, down->eps, m, F, qb, cd, stream);
        if (e == hipSuccess)
            e = gemm(qb, m, F, &dn, 1, epi_dn, y, D, bf, residual, D, cd, D, FAM_GEMM_DOWN, stream);
    }
    if (e != hipSuccess) return hip_error(e, "glu_forward launch");
    return MMF_OK;
}

// ------------------------------------------------------------------ block
static int check_block(const mmf_block *w, const char *who) {
    if (!w) return set_error(MMF_EINVAL, "%s: NULL block", who);
    int rc;
    if ((rc = check_linear(&w->i, "i")) || (rc = check_linear(&w->f, "f")) || (rc = check_linear(&w->g, "g")) ||
        (rc = check_linear(&w->o, "o")))
        return rc;
    if ((rc = check_glu(&w->gate, &w->up, &w->down, who))) return rc;
    const int32_t D = w->i.K;
    const mmf_bitlinear *sq[4] = {&w->i, &w->f, &w->g, &w->o};
    for (auto *l : sq)
        if (l->K != D || l->N != D) return set_error(MMF_ESHAPE, "%s: i/f/g/o must be [D][D] with D=%d", who, D);
    if (w->gate.K != D) return set_error(MMF_ESHAPE, "%s: gate/up K=%d != D=%d", who, w->gate.K, D);
    if (D > 4096) return set_error(MMF_ESHAPE, "%s: D=%d exceeds 4096", who, D);
    if (w->f.norm_w != w->i.norm_w || w->g.norm_w != w->i.norm_w || w->f.eps != w->i.eps || w->g.eps != w->i.eps)
        return set_error(MMF_EINVAL, "%s: i, f, g must share norm_w and eps", who);
    if (w->gate_mode != MMF_GATE_SWISH_RMSNORM && w->gate_mode != MMF_GATE_SIGMOID) return set_error(MMF_EINVAL, "%s: gate_mode %d", who, w->gate_mode);
    if (!(w->eps >= 0.0f)) return set_error(MMF_EINVAL, "%s: eps", who);
    // per-channel vectors are read 16 bytes at a time
    if ((w->f_bias && !aligned16(w->f_bias)) || (w->gnorm_w && !aligned16(w->gnorm_w)) ||
        (w->o.norm_w && !aligned16(w->o.norm_w)))
        return set_error(MMF_EALIGN, "%s: f_bias/gnorm_w/o.norm_w not 16-byte aligned", who);
    return MMF_OK;
}

size_t block_workspace_bytes(const mmf_block *w, int64_t B, int64_t T) {
    if (!w || B <= 0 || T <= 0) return 0;
    const int64_t M = B * T, D = w->i.K, F = w->gate.N;
    return qbuf_bytes(M, std::max(D, F)) + align_up(static_cast<size_t>(M * std::max(3 * D, F)) * 4) +
           align_up(static_cast<size_t>(M * D) * 4) + scan_bytes(B, T, D) +
           (M == 1 ? align_up(static_cast<size_t>(D) * 4) : 0);  // new state of a fused step
}

int block_forward(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                  float *h_state, void *y, void *ws, size_t ws_bytes, const mmf_capture *cap,
                  hipStream_t stream) {
    int rc = check_block(w, "block_forward");
    if (rc) return rc;
    if (!valid_dt(dt)) return set_error(MMF_EDTYPE, "block_forward: dtype %d", dt);
    if (B < 0 || T < 0) return set_error(MMF_ESHAPE, "block_forward: B=%lld T=%lld", (long long)B, (long long)T);
    if (cap && ((rc = check_cap(&cap->ifg, "ifg")) || (rc = check_cap(&cap->o, "o")) ||
                (rc = check_cap(&cap->gateup, "gateup")) || (rc = check_cap(&cap->down, "down"))))
        return rc;
    const int64_t M = B * T;
    if (M == 0) return MMF_OK;  // h_T = h_0 already in place
    if (!x || !y) return set_error(MMF_EINVAL, "block_forward: NULL x or y");
    if (!aligned16(x) || !aligned16(y)) return set_error(MMF_EALIGN, "block_forward: x/y not 16-byte aligned");
    if (h_state && !aligned16(h_state)) return set_error(MMF_EALIGN, "block_forward: h_state not 16-byte aligned");
    const size_t need = block_workspace_bytes(w, B, T);
    if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "block_forward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "block_forward: workspace not 16-byte aligned");
    if ((rc = check_device())) return rc;

    const int32_t D = w->i.K, F = w->gate.N;
    const bool bf = dt == MMF_BF16;
    Carver c(ws);
    const QBuf qb = take_qbuf(c, M, std::max(D, F));
    void *act = c.take<char>(static_cast<size_t>(M * std::max(3 * D, F)) * 4);  // ifg, then m
    void *y1 = c.take<char>(static_cast<size_t>(M * D) * 4);
    const Seg ifg[3] = {seg_of(w->i, 0, 0), seg_of(w->f, D, D), seg_of(w->g, 2 * D, 2 * D)};
    const Seg so = seg_of(w->o, 0, 0);
    const Seg gu[2] = {seg_of(w->gate, 0, 0), seg_of(w->up, 0, F)};
    const Seg dn = seg_of(w->down, 0, 0);
    const mmf_stage_capture *c_ifg = cap ? &cap->ifg : nullptr, *c_o = cap ? &cap->o : nullptr,
                            *c_gu = cap ? &cap->gateup : nullptr, *c_dn = cap ? &cap->down : nullptr;
    const bool decode = use_decode(M);

    // 1-2: i|f|g projections of x
    hipError_t e;
    if (decode) {
        e = gemv(x, bf, w->i.norm_w, w->i.eps, nullptr, M, D, ifg, 3, EPI_STORE, act, 3 * D, bf, nullptr, 0, c_ifg, 3 * D, stream);
    } else {
        e = quantize(x, bf, w->i.norm_w, w->i.eps, M, D, qb, c_ifg, stream);
        if (e == hipSuccess) e = gemm(qb, M, D, ifg, 3, EPI_STORE, act, 3 * D, bf, nullptr, 0, c_ifg, 3 * D, FAM_GEMM_IFG, stream);
    }
    if (e != hipSuccess) return hip_error(e, "block_forward ifg launch");

    if (decode && M == 1) {
        // one token: the MLGRU step, g_norm and o_proj's quantization run in the o_proj
        // kernel's prologue (every workgroup recomputes the D-wide step; workgroup 0 writes
        // the new state to the workspace, and the gate|up kernel, which runs after every
        // reader of the old state has finished, copies it into h_state)
        float *h_tmp = h_state ? c.take<float>(static_cast<size_t>(D) * 4) : nullptr;
        GemvExtra eo;
        eo.mlgru = true;
        eo.h_prev = h_state;
        eo.h_new = h_tmp;
        eo.f_bias = w->f_bias;
        eo.gnorm_w = w->gnorm_w;
        eo.g_eps = w->eps;
        eo.gate_mode = w->gate_mode;
        e = gemv(act, bf, w->o.norm_w, w->o.eps, nullptr, M, D, &so, 1, EPI_RESID, y1, D, bf, x, D, c_o, D, stream, &eo);
        if (e != hipSuccess) return hip_error(e, "block_forward o_proj launch");
        GemvExtra eg;
        if (h_state) {
            eg.copy_src = h_tmp;
            eg.copy_dst = h_state;
            eg.copy_n = D;
        }
        e = gemv(y1, bf, w->gate.norm_w, w->gate.eps, nullptr, M, D, gu, 2, EPI_GLU, act, F, bf, nullptr, 0, c_gu, 2 * F, stream, &eg);
        if (e == hipSuccess)
            e = gemv(act, bf, w->down.norm_w, w->down.eps, nullptr, M, F, &dn, 1, EPI_RESID, y, D, bf, y1, D, c_dn, D, stream);
        if (e != hipSuccess) return hip_error(e, "block_forward glu launch");
        return MMF_OK;
    }

    // 3: MLGRU + g_norm, quantized from fp32 for o_proj
    ScanArgs s{};
    s.ifg = act;
    s.ifg_bf16 = bf;
    s.f_bias = w->f_bias;
    s.h0 = h_state;
    s.h_out = h_state;
    s.gnorm_w = w->gnorm_w;
    s.eps = w->eps;
    s.gate_mode = w->gate_mode;
    s.B = B;
    s.T = T;
    s.D = D;
    s.chunk = kScanChunk;
    s.n_chunks = static_cast<int32_t>(scan_chunks(T));
    if (s.n_chunks > 1) {
        const size_t n = static_cast<size_t>(B * s.n_chunks * D) * 4;
        s.hloc = c.take<float>(n);
        s.pf = c.take<float>(n);
        s.hin = c.take<float>(n);
    }
    s.q = qb.q;
    s.a = qb.a;
    s.rowsum = qb.rs;
    s.q_gamma = w->o.norm_w;
    s.q_eps = w->o.eps;
    s.cap = cap_of(c_o, 0);
    s.cap.acc = nullptr;
    s.cap.y_out = nullptr;
    e = launch_scan(s, stream);
    if (e != hipSuccess) return hip_error(e, "block_forward scan launch");

    // 4: o_proj + residual x -> y1
    if (decode) e = gemv(nullptr, bf, nullptr, 0.f, &qb, M, D, &so, 1, EPI_RESID, y1, D, bf, x, D, c_o, D, stream);
    else e = gemm(qb, M, D, &so, 1, EPI_RESID, y1, D, bf, x, D, c_o, D, FAM_GEMM_O, stream);
    if (e != hipSuccess) return hip_error(e, "block_forward o_proj launch");

    // 5-8: GLU with residual y1 -> y
    // the GLU hidden m is stored in the activation dtype between the two kernels
    if (decode) {
        e = gemv(y1, bf, w->gate.norm_w, w->gate.eps, nullptr, M, D, gu, 2, EPI_GLU, act, F, bf, nullptr, 0, c_gu, 2 * F, stream);
        if (e == hipSuccess)
            e = gemv(act, bf, w->down.norm_w, w->down.eps, nullptr, M, F, &dn, 1, EPI_RESID, y, D, bf, y1, D, c_dn, D, stream);
    } else {
        e = quantize(y1, bf, w->gate.norm_w, w->gate.eps, M, D, qb, c_gu, stream);
        if (e == hipSuccess) e = gemm(qb, M, D, gu, 2, EPI_GLU, act, F, bf, nullptr, 0, c_gu, 2 * F, FAM_GEMM_GATEUP, stream);
        if (e == hipSuccess) e = quantize(act, bf, w->down.norm_w, w->down.eps, M, F, qb, c_dn, stream);
        if (e == hipSuccess) e = gemm(qb, M, F, &dn, 1, EPI_RESID, y, D, bf, y1, D, c_dn, D, FAM_GEMM_DOWN, stream);
    }
    if (e != hipSuccess) return hip_error(e, "block_forward glu launch");
    return MMF_OK;
}

// ------------------------------------------------------------------ embedding
int embedding_forward(const uint32_t *packed, float scale, int64_t vocab, int64_t D,
                      const int32_t *ids, int64_t m, void *x, mmf_dtype dt, hipStream_t stream) {
    if (!packed) return set_error(MMF_EINVAL, "embedding_forward: NULL packed");
    if (vocab <= 0 || D <= 0 || D % 64 || m < 0) return set_error(MMF_ESHAPE, "embedding_forward: vocab=%lld D=%lld m=%lld", (long long)vocab, (long long)D, (long long)m);
    if (!valid_dt(dt)) return set_error(MMF_EDTYPE, "embedding_forward: dtype %d", dt);
    if (m == 0) return MMF_OK;
    if (!ids || !x) return set_error(MMF_EINVAL, "embedding_forward: NULL ids or x");
    if (!aligned16(packed) || !aligned16(x)) return set_error(MMF_EALIGN, "embedding_forward: packed/x not 16-byte aligned");
    int rc = check_device();
    if (rc) return rc;
    hipError_t e = launch_embedding(packed, scale, vocab, static_cast<int32_t>(D), ids, m, x, dt == MMF_BF16, stream);
    if (e != hipSuccess) return hip_error(e, "embedding_forward launch");
    return MMF_OK;
}

// ------------------------------------------------------------------ stack
size_t stack_workspace_bytes(const mmf_stack *s, int64_t B, int64_t T) {
    if (!s || s->n_layers <= 0 || !s->blocks || B <= 0 || T <= 0) return 0;
    const int64_t M = B * T, D = s->blocks[0].i.K;
    size_t blk = 0;
    for (int l = 0; l < s->n_layers; ++l) blk = std::max(blk, block_workspace_bytes(&s->blocks[l], B, T));
    if (s->head) blk = std::max(blk, bitlinear_workspace_bytes(s->head, M));
    return 2 * align_up(static_cast<size_t>(M * D) * 4) + blk;
}

int stack_forward(const mmf_stack *s, const int32_t *ids, const void *x, mmf_dtype dt, int64_t B,
                  int64_t T, float *h_state, void *y, float *logits, void *ws, size_t ws_bytes,
                  hipStream_t stream) {
    if (!s || !s->blocks || s->n_layers <= 0) return set_error(MMF_EINVAL, "stack_forward: empty stack");
    if (!valid_dt(dt)) return set_error(MMF_EDTYPE, "stack_forward: dtype %d", dt);
    if (B < 0 || T < 0) return set_error(MMF_ESHAPE, "stack_forward: B=%lld T=%lld", (long long)B, (long long)T);
    int rc;
    const int32_t D = s->blocks[0].i.K;
    for (int l = 0; l < s->n_layers; ++l) {
        if ((rc = check_block(&s->blocks[l], "stack_forward"))) return rc;
        if (s->blocks[l].i.K != D) return set_error(MMF_ESHAPE, "stack_forward: layer %d has D=%d, not %d", l, s->blocks[l].i.K, D);
    }
    if (s->head) {
        if ((rc = check_linear(s->head, "head"))) return rc;
        if (s->head->K != D) return set_error(MMF_ESHAPE, "stack_forward: head K=%d != D=%d", s->head->K, D);
    }
    if (logits && !s->head) return set_error(MMF_EINVAL, "stack_forward: logits requested without a head");
    if (ids && !s->embed_packed) return set_error(MMF_EINVAL, "stack_forward: ids given without an embedding");
    if (!ids && !x) return set_error(MMF_EINVAL, "stack_forward: neither ids nor x");
    if (!y && !logits) return set_error(MMF_EINVAL, "stack_forward: neither y nor logits");
    const int64_t M = B * T;
    if (M == 0) return MMF_OK;
    if ((x && !aligned16(x)) || (y && !aligned16(y)) || (logits && !aligned16(logits))) return set_error(MMF_EALIGN, "stack_forward: x/y/logits not 16-byte aligned");
    if (h_state && !aligned16(h_state)) return set_error(MMF_EALIGN, "stack_forward: h_state not 16-byte aligned");
    const size_t need = stack_workspace_bytes(s, B, T);
    if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "stack_forward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "stack_forward: workspace not 16-byte aligned");
    if ((rc = check_device())) return rc;

    Carver c(ws);
    void *buf[2] = {c.take<char>(static_cast<size_t>(M * D) * 4), c.take<char>(static_cast<size_t>(M * D) * 4)};
    char *bws = c.base + c.off;
    const size_t bws_bytes = ws_bytes - c.off;
    const void *cur = x;
    if (ids) {
        rc = embedding_forward(s->embed_packed, s->embed_scale, s->vocab, D, ids, M, buf[0], dt, stream);
        if (rc) return rc;
        cur = buf[0];
    }
    for (int l = 0; l < s->n_layers; ++l) {
        // block_forward reads x before it writes y, so y may alias x
        void *dst = (l == s->n_layers - 1 && y) ? y : buf[(l + 1) & 1];
        float *hs = h_state ? h_state + static_cast<int64_t>(l) * B * D : nullptr;
        rc = block_forward(&s->blocks[l], cur, dt, B, T, hs, dst, bws, bws_bytes, nullptr, stream);
        if (rc) return rc;
        cur = dst;
    }
    if (logits) {
        rc = bitlinear_forward(s->head, cur, dt, M, logits, MMF_F32, bws, bws_bytes, nullptr, stream);
        if (rc) return rc;
    }
    return MMF_OK;
}

}  // extern "C"
