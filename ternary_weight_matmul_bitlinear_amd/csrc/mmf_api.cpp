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

// One-token decode steps of up to this many sequences run the MLGRU step, g_norm and
// o_proj's quantization inside the o_proj launch (one token per workgroup row of its grid).
constexpr int64_t kFusedStepMaxB = 4;

static bool fused_step(int64_t B, int64_t T, int64_t D, int64_t F) {
    // (the gate|up launch's side copy of the new state covers 64 floats per GLU row)
    return T == 1 && B >= 1 && B <= kFusedStepMaxB && D <= 4096 && B * D <= 64 * F && use_decode(B);
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
                                           "gemm_down", "gemm", "gemv", "scan", "embed", "bwd_g", "bwd_dw", "bwd_scan"};
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
                       const mmf_stage_capture *cap, int32_t cap_ld, int family, hipStream_t s,
                       uint16_t *keep = nullptr) {
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
    ga.keep = keep;
    // up to kMidMaxM rows: the k-split kernel that reads the weights once (regime 3 forces
    // the 128-row tiles at any M; only these keep the GLU's pre-activations)
    if (g_regime.load() != 3 && M <= kMidMaxM && epi != EPI_GLU_KEEP && mid_gemm_supported(ga))
        return launch_gemm_mid(ga, s);
    return launch_gemm(ga, s);
}

// Extras of a decode GEMV: the fused MLGRU step of o_proj and a side copy of the state.
struct GemvExtra {
    const float *h_prev = nullptr;
    float *h_new = nullptr;
    const float *f_bias = nullptr;
    const float *f_lower = nullptr;
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
        ga.f_lower = ex->f_lower;
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

// ------------------------------------------------------------ static scratch
// Device scratch of the no-allocation entry point: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes the array's name to a kernel
// (on the host it is only a stand-in symbol); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::mutex g_scr_mu;
static std::vector<void *> g_scr_ptr;  // per device; nullptr until looked up

static int scratch_for_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if (dev >= static_cast<int>(g_scr_ptr.size())) g_scr_ptr.resize(dev + 1, nullptr);
    if (!g_scr_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress(scratch)");
        if (!p) return set_error(MMF_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scr_ptr[dev] = p;
    }
    *out = g_scr_ptr[dev];
    return MMF_OK;
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

// --------------------------------------------------- BitLinear, base-3 packed weights
int bitlinear_forward_trits(const mmf_bitlinear_trits *w, const void *x, mmf_dtype x_dt,
                            int64_t m, void *y, mmf_dtype y_dt, const mmf_stage_capture *cap,
                            hipStream_t stream) {
    if (!w) return set_error(MMF_EINVAL, "bitlinear_forward_trits: NULL descriptor");
    if (!w->packed) return set_error(MMF_EINVAL, "bitlinear_forward_trits: NULL packed weights");
    if (w->K <= 0 || w->N <= 0 || w->K % 64 || w->K > 10240)
        return set_error(MMF_ESHAPE, "bitlinear_forward_trits: K=%d N=%d (K must be a positive multiple of 64, at most 10240)", w->K, w->N);
    if (!valid_dt(x_dt) || !valid_dt(y_dt)) return set_error(MMF_EDTYPE, "bitlinear_forward_trits: dtype %d/%d", x_dt, y_dt);
    if (m < 0 || m > 16) return set_error(MMF_ESHAPE, "bitlinear_forward_trits: m=%lld (decode regime: 0..16 token rows)", (long long)m);
    if (!(w->eps >= 0.0f)) return set_error(MMF_EINVAL, "bitlinear_forward_trits: eps must be >= 0");
    int rc;
    if ((rc = check_cap(cap, "bitlinear_forward_trits"))) return rc;
    if (m == 0) return MMF_OK;
    if (!x || !y) return set_error(MMF_EINVAL, "bitlinear_forward_trits: NULL x or y");
    if (!aligned16(x) || !aligned16(y) || !aligned16(w->packed))
        return set_error(MMF_EALIGN, "bitlinear_forward_trits: x, y or packed not 16-byte aligned");
    if ((rc = check_device())) return rc;
    TritArgs a{};
    a.x = x;
    a.x_bf16 = x_dt == MMF_BF16;
    a.gamma = w->norm_w;
    a.eps = w->eps;
    a.M = m;
    a.K = w->K;
    a.row_bytes = static_cast<int32_t>(mmf_trit_row_bytes(w->K));
    a.packed = w->packed;
    a.scale = w->scale;
    a.bias = w->bias;
    a.N = w->N;
    a.out = y;
    a.out_bf16 = y_dt == MMF_BF16;
    a.cap = cap_of(cap, w->N);
    const hipError_t e = launch_gemv_trits(a, stream);
    if (e != hipSuccess) return hip_error(e, "bitlinear_forward_trits launch");
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
        (a->f_bias && !aligned16(a->f_bias)) || (a->gnorm_w && !aligned16(a->gnorm_w)) ||
        (a->f_lower && !aligned16(a->f_lower)))
        return set_error(MMF_EALIGN, "mlgru_scan: h0/h_out/f_bias/f_lower/gnorm_w not 16-byte aligned");
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
    s.f_lower = a->f_lower;
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
        (w->o.norm_w && !aligned16(w->o.norm_w)) || (w->f_lower && !aligned16(w->f_lower)))
        return set_error(MMF_EALIGN, "%s: f_bias/f_lower/gnorm_w/o.norm_w not 16-byte aligned", who);
    return MMF_OK;
}

size_t block_workspace_bytes(const mmf_block *w, int64_t B, int64_t T) {
    if (!w || B <= 0 || T <= 0) return 0;
    const int64_t M = B * T, D = w->i.K, F = w->gate.N;
    return qbuf_bytes(M, std::max(D, F)) + align_up(static_cast<size_t>(M * std::max(3 * D, F)) * 4) +
           align_up(static_cast<size_t>(M * D) * 4) + scan_bytes(B, T, D) +
           (T == 1 && B <= kFusedStepMaxB ? align_up(static_cast<size_t>(M * D) * 4) : 0);  // new state of a fused step
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

    if (fused_step(B, T, D, F)) {
        // one token per sequence, up to kFusedStepMaxB sequences: the MLGRU step, g_norm and
        // o_proj's quantization run in the o_proj kernel's prologue (the workgroups of grid row
        // b take sequence b; each recomputes its D-wide step; workgroup (0, b) writes the new
        // state to the workspace, and the gate|up kernel, which runs after every reader of the
        // old state has finished, copies it into h_state)
        float *h_tmp = h_state ? c.take<float>(static_cast<size_t>(M * D) * 4) : nullptr;
        GemvExtra eo;
        eo.mlgru = true;
        eo.h_prev = h_state;
        eo.h_new = h_tmp;
        eo.f_bias = w->f_bias;
        eo.f_lower = w->f_lower;
        eo.gnorm_w = w->gnorm_w;
        eo.g_eps = w->eps;
        eo.gate_mode = w->gate_mode;
        e = gemv(act, bf, w->o.norm_w, w->o.eps, nullptr, M, D, &so, 1, EPI_RESID, y1, D, bf, x, D, c_o, D, stream, &eo);
        if (e != hipSuccess) return hip_error(e, "block_forward o_proj launch");
        GemvExtra eg;
        if (h_state) {
            eg.copy_src = h_tmp;
            eg.copy_dst = h_state;
            eg.copy_n = static_cast<int32_t>(M * D);
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
    s.f_lower = w->f_lower;
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

size_t block_scratch_bytes(void) { return kScratchBytes; }

int block_forward_noalloc(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                          float *h_state, void *y, hipStream_t stream) {
    int rc = check_block(w, "block_forward_noalloc");
    if (rc) return rc;
    if (B < 0 || T < 0) return set_error(MMF_ESHAPE, "block_forward_noalloc: B=%lld T=%lld", (long long)B, (long long)T);
    if (B * T == 0) return MMF_OK;
    const size_t need = block_workspace_bytes(w, B, T);
    if (need > kScratchBytes)
        return set_error(MMF_EWORKSPACE, "block_forward_noalloc: B*T=%lld needs %zu bytes of scratch, more than the %zu-byte static scratch",
                         (long long)(B * T), need, kScratchBytes);
    void *ws = nullptr;
    if ((rc = check_device()) || (rc = scratch_for_current_device(&ws))) return rc;
    // every byte of the workspace a block_forward call reads was written earlier in the same
    // call, so the scratch needs no clearing between calls
    return block_forward(w, x, dt, B, T, h_state, y, ws, kScratchBytes, nullptr, stream);
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

// --------------------------------------------- one-launch decode step (one sequence)
namespace {
struct DecodeLayout {
    size_t trace, table, xch, total;   // byte offsets of the stamps, layer table, exchange area
};
DecodeLayout decode_layout(const mmf_stack *s) {
    const int64_t D = s->blocks[0].i.K, F = s->blocks[0].gate.N, L = s->n_layers;
    DecodeLayout d;
    d.trace = 256;
    d.table = d.trace + align_up(static_cast<size_t>(4 * L + 2) * 16);
    d.xch = d.table + align_up(static_cast<size_t>(L) * sizeof(PLayer));
    d.total = d.xch + align_up(static_cast<size_t>(L + 1) * static_cast<size_t>(D / 2 * 5 + F / 2) * 8);
    return d;
}
int decode_grid(const mmf_stack *s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    int per_cu = 0;
    if (persist_occupancy(s->blocks[0].i.K, s->blocks[0].gate.N, &per_cu) != 0 || per_cu < 1) return 0;
    return prop.multiProcessorCount;   // one workgroup per CU
}
int check_decode_stack(const mmf_stack *s, int grid, const char *who) {
    if (!s || !s->blocks || s->n_layers <= 0) return set_error(MMF_EINVAL, "%s: empty stack", who);
    if (!s->embed_packed || !s->head) return set_error(MMF_EINVAL, "%s: the stack needs an embedding and a head", who);
    int rc;
    const int32_t D = s->blocks[0].i.K, F = s->blocks[0].gate.N;
    for (int l = 0; l < s->n_layers; ++l) {
        if ((rc = check_block(&s->blocks[l], who))) return rc;
        if (s->blocks[l].i.K != D || s->blocks[l].gate.N != F)
            return set_error(MMF_ESHAPE, "%s: layer %d has D=%d F=%d, not %d/%d", who, l, s->blocks[l].i.K, s->blocks[l].gate.N, D, F);
    }
    if ((rc = check_linear(s->head, "head"))) return rc;
    if (s->head->K != D) return set_error(MMF_ESHAPE, "%s: head K=%d != D=%d", who, s->head->K, D);
    // the kernel copies these vectors into LDS with 16-byte direct loads
    for (int l = 0; l < s->n_layers; ++l) {
        const mmf_block &b = s->blocks[l];
        const void *v[7] = {b.i.norm_w, b.o.norm_w, b.gate.norm_w, b.down.norm_w, b.f_bias, b.f_lower, b.gnorm_w};
        for (const void *q : v)
            if (q && !aligned16(q)) return set_error(MMF_EALIGN, "%s: layer %d: a gain, forget bias/bound or g_norm weight is not 16-byte aligned", who, l);
    }
    if (s->head->norm_w && !aligned16(s->head->norm_w)) return set_error(MMF_EALIGN, "%s: head gain not 16-byte aligned", who);
    int mu, mw, mk, md, mr;
    persist_limits(&mu, &mw, &mk, &md, &mr);
    const int G = grid > 0 ? grid : 1;
    auto per_wg = [&](int n, int unit) { return ((n / unit + G - 1) / G) * unit; };
    const int V = s->head->N;
    if (D > md || F > mk || D % 4 || F % 4)
        return set_error(MMF_ESHAPE, "%s: D=%d F=%d outside the one-launch limits (D <= %d, F <= %d)", who, D, F, md, mk);
    if (per_wg(V, 1) > mr || 2 * per_wg(F, 2) > mr || per_wg(3 * D, 2) > mr)
        return set_error(MMF_ESHAPE, "%s: more than %d rows per workgroup at %d workgroups", who, mr, G);
    const int need[5] = {persist_max_units(per_wg(3 * D, 2), D), persist_max_units(per_wg(D, 2), D),
                         persist_max_units(2 * per_wg(F, 2), D), persist_max_units(per_wg(D, 2), F),
                         persist_max_units(per_wg(V, 1), D)};
    int have[5];
    persist_stage_units(have);
    for (int k = 0; k < 5; ++k)
        if (need[k] > have[k])
            return set_error(MMF_ESHAPE, "%s: stage %d needs %d weight units per thread, more than %d, at %d workgroups", who, k, need[k], have[k], G);
    (void)mu;
    return MMF_OK;
}
}  // namespace

extern "C" {

size_t stack_decode_workspace_bytes(const mmf_stack *s) {
    if (!s || !s->blocks || s->n_layers <= 0) return 0;
    return decode_layout(s).total;
}

int stack_decode_init(const mmf_stack *s, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if (!s || !s->blocks || s->n_layers <= 0) return set_error(MMF_EINVAL, "stack_decode_init: empty stack");
    if ((rc = check_device())) return rc;
    const int G = decode_grid(s);
    if (G <= 0) return set_error(MMF_EHIP, "stack_decode_init: no occupancy for the one-launch decode kernel");
    if ((rc = check_decode_stack(s, G, "stack_decode_init"))) return rc;
    const DecodeLayout lay = decode_layout(s);
    if (!ws || ws_bytes < lay.total) return set_error(MMF_EWORKSPACE, "stack_decode_init: workspace %zu < %zu", ws ? ws_bytes : 0, lay.total);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "stack_decode_init: workspace not 16-byte aligned");
    std::vector<PLayer> tab(s->n_layers);
    for (int l = 0; l < s->n_layers; ++l) {
        const mmf_block &b = s->blocks[l];
        const mmf_bitlinear *m[7] = {&b.i, &b.f, &b.g, &b.o, &b.gate, &b.up, &b.down};
        PLayer &t = tab[l];
        for (int k = 0; k < 7; ++k) {
            t.w[k] = m[k]->packed;
            t.s[k] = m[k]->scale;
            t.b[k] = m[k]->bias;
        }
        t.g_x = b.i.norm_w; t.e_x = b.i.eps;
        t.g_o = b.o.norm_w; t.e_o = b.o.eps;
        t.g_gu = b.gate.norm_w; t.e_gu = b.gate.eps;
        t.g_down = b.down.norm_w; t.e_down = b.down.eps;
        t.f_bias = b.f_bias;
        t.f_lower = b.f_lower;
        t.gnorm_w = b.gnorm_w;
        t.g_eps = b.eps;
        t.gate_mode = b.gate_mode;
    }
    char *base = static_cast<char *>(ws);
    hipError_t e = hipMemsetAsync(base, 0, lay.total, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(base + lay.table, tab.data(), tab.size() * sizeof(PLayer), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);   // the host table is a local
    if (e != hipSuccess) return hip_error(e, "stack_decode_init");
    return MMF_OK;
}

int stack_decode_step(const mmf_stack *s, const int32_t *ids, float *h_state, float *logits,
                      void *y, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc;
    if (!s || !s->blocks || s->n_layers <= 0) return set_error(MMF_EINVAL, "stack_decode_step: empty stack");
    if (!ids || !h_state) return set_error(MMF_EINVAL, "stack_decode_step: NULL ids or h_state");
    if (!logits && !y) return set_error(MMF_EINVAL, "stack_decode_step: neither logits nor y");
    if ((y && !aligned16(y)) || (logits && !aligned16(logits)) || !aligned16(h_state))
        return set_error(MMF_EALIGN, "stack_decode_step: y/logits/h_state not 16-byte aligned");
    const DecodeLayout lay = decode_layout(s);
    if (!ws || ws_bytes < lay.total) return set_error(MMF_EWORKSPACE, "stack_decode_step: workspace %zu < %zu", ws ? ws_bytes : 0, lay.total);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "stack_decode_step: workspace not 16-byte aligned");
    if ((rc = check_device())) return rc;
    const int G = decode_grid(s);
    if (G <= 0) return set_error(MMF_EHIP, "stack_decode_step: no occupancy for the one-launch decode kernel");
    if ((rc = check_decode_stack(s, G, "stack_decode_step"))) return rc;
    char *base = static_cast<char *>(ws);
    PersistArgs a{};
    a.layers = reinterpret_cast<const PLayer *>(base + lay.table);
    a.L = s->n_layers;
    a.D = s->blocks[0].i.K;
    a.F = s->blocks[0].gate.N;
    a.V = s->head->N;
    a.emb = s->embed_packed;
    a.emb_scale = s->embed_scale;
    a.vocab = s->vocab;
    a.head = s->head->packed;
    a.head_scale = s->head->scale;
    a.head_bias = s->head->bias;
    a.head_gamma = s->head->norm_w;
    a.head_eps = s->head->eps;
    a.ids = ids;
    a.h_state = h_state;
    a.logits = logits;
    a.y = y;
    a.xch = reinterpret_cast<uint64_t *>(base + lay.xch);
    a.ctl = reinterpret_cast<uint32_t *>(base);
    a.trace = reinterpret_cast<uint64_t *>(base + lay.trace);
    a.spin_ticks = 20000000;   // 0.2 s per wait (100 MHz counter)
    const hipError_t e = launch_decode_persistent(a, G, stream);
    if (e != hipSuccess) return hip_error(e, "stack_decode_step launch");
    return MMF_OK;
}

int stack_decode_status(const void *ws, hipStream_t stream) {
    if (!ws) return set_error(MMF_EINVAL, "stack_decode_status: NULL workspace");
    uint32_t ctl[3] = {0, 0, 0};
    hipError_t e = hipMemcpyAsync(ctl, ws, sizeof ctl, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_error(e, "stack_decode_status");
    if (ctl[2]) return set_error(MMF_EHIP, "stack_decode_step: a stage wait timed out (re-initialise the workspace)");
    return MMF_OK;
}

// ------------------------------------------------------------------ backward
size_t bitlinear_backward_workspace_bytes(const mmf_bitlinear *w, int64_t m) {
    if (!w || w->K <= 0 || w->N <= 0 || m <= 0) return 0;
    const size_t K = static_cast<size_t>(w->K), N = static_cast<size_t>(w->N), M = static_cast<size_t>(m);
    const size_t ldm = (M + 63) / 64 * 64;
    return align_up(M * K) + align_up(M * 4) + align_up(M * 4) + align_up(M * K * 4) +
           align_up(K * N * 2) + align_up(N * ldm * 2) + align_up(K * ldm * 2) +
           align_up(bwd_rows_part_bytes(m, w->K));
}

int bitlinear_backward(const mmf_bitlinear *w, const void *x, mmf_dtype x_dt, int64_t m,
                       const void *dy, mmf_dtype dy_dt, float *dx, float *dgamma, float *dw,
                       float *db, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_linear(w, "bitlinear_backward");
    if (rc) return rc;
    if (!valid_dt(x_dt) || !valid_dt(dy_dt)) return set_error(MMF_EDTYPE, "bitlinear_backward: dtype %d/%d", x_dt, dy_dt);
    if (m < 0) return set_error(MMF_ESHAPE, "bitlinear_backward: m=%lld", (long long)m);
    if (w->N % 8) return set_error(MMF_ESHAPE, "bitlinear_backward: N=%d is not a multiple of 8", w->N);
    if (w->K > 8192) return set_error(MMF_ESHAPE, "bitlinear_backward: K=%d exceeds 8192", w->K);
    if (m == 0) {   // every gradient is an empty sum
        hipError_t e = hipSuccess;
        if (dgamma) e = launch_fill_zero(dgamma, w->K, stream);
        if (e == hipSuccess && dw) e = launch_fill_zero(dw, static_cast<int64_t>(w->N) * w->K, stream);
        if (e == hipSuccess && db) e = launch_fill_zero(db, w->N, stream);
        return e == hipSuccess ? MMF_OK : hip_error(e, "bitlinear_backward fill");
    }
    if (!x || !dy) return set_error(MMF_EINVAL, "bitlinear_backward: NULL x or dy");
    if (!aligned16(x) || !aligned16(dy) || (dx && !aligned16(dx)) || (dw && !aligned16(dw)) ||
        (w->norm_w && !aligned16(w->norm_w)))
        return set_error(MMF_EALIGN, "bitlinear_backward: x/dy/dx/dw/norm_w not 16-byte aligned");
    const size_t need = bitlinear_backward_workspace_bytes(w, m);
    if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "bitlinear_backward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "bitlinear_backward: workspace not 16-byte aligned");
    if ((rc = check_device())) return rc;
    Carver c(ws);
    QBuf qb;
    qb.q = c.take<int8_t>(static_cast<size_t>(m) * w->K);
    qb.a = c.take<float>(static_cast<size_t>(m) * 4);
    qb.rs = c.take<int32_t>(static_cast<size_t>(m) * 4);
    float *g = c.take<float>(static_cast<size_t>(m) * w->K * 4);
    const int64_t ldm = (m + 63) / 64 * 64;
    uint16_t *wt = c.take<uint16_t>(static_cast<size_t>(w->K) * w->N * 2);
    uint16_t *dyaT = c.take<uint16_t>(static_cast<size_t>(w->N) * ldm * 2);
    uint16_t *qT = c.take<uint16_t>(static_cast<size_t>(w->K) * ldm * 2);
    float *dg_part = c.take<float>(bwd_rows_part_bytes(m, w->K));
    hipError_t e = quantize(x, x_dt == MMF_BF16, w->norm_w, w->eps, m, w->K, qb, nullptr, stream);
    if (e != hipSuccess) return hip_error(e, "bitlinear_backward quant launch");
    BitlinearBwdArgs a{};
    a.x = x;
    a.x_bf16 = x_dt == MMF_BF16;
    a.gamma = w->norm_w;
    a.eps = w->eps;
    a.M = m;
    a.K = w->K;
    a.N = w->N;
    a.packed = w->packed;
    a.scale = w->scale;
    a.dy = dy;
    a.dy_bf16 = dy_dt == MMF_BF16;
    a.q = qb.q;
    a.a = qb.a;
    a.g = g;
    a.wt = wt;
    a.ldm = ldm;
    a.dyaT = dyaT;
    a.qT = qT;
    a.dg_part = dg_part;
    a.dx = dx;
    a.dgamma = dgamma;
    a.dw = dw;
    a.db = db;
    e = launch_bitlinear_bwd(a, stream);
    if (e != hipSuccess) return hip_error(e, "bitlinear_backward launch");
    return MMF_OK;
}

size_t mlgru_backward_workspace_bytes(int64_t B, int64_t T, int64_t D) {
    if (B <= 0 || T <= 0 || D <= 0) return 0;
    const size_t cn = static_cast<size_t>(B * scan_chunks(T) * D) * 4;
    return scan_bytes(B, T, D) + align_up(static_cast<size_t>(B * T) * 8) + 6 * align_up(cn);
}

}  // extern "C"

// d_ifg in bf16 (d_ifg_bf16) for the block backward's own use
static int mlgru_backward_impl(const mmf_mlgru_args *a, const void *dout, mmf_dtype dout_dt,
                               const float *dh_last, void *d_ifg, bool d_ifg_bf16, float *dh0,
                               float *dgnorm_w, float *df_bias, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
    if (!a) return set_error(MMF_EINVAL, "mlgru_backward: NULL args");
    int rc = check_scan_shape(a->B, a->T, a->D, "mlgru_backward");
    if (rc) return rc;
    if (!valid_dt(a->ifg_dt) || !valid_dt(dout_dt)) return set_error(MMF_EDTYPE, "mlgru_backward: dtype");
    if (a->gate_mode != MMF_GATE_SWISH_RMSNORM && a->gate_mode != MMF_GATE_SIGMOID) return set_error(MMF_EINVAL, "mlgru_backward: gate_mode %d", a->gate_mode);
    if (!(a->eps >= 0.0f)) return set_error(MMF_EINVAL, "mlgru_backward: eps");
    const int64_t M = a->B * a->T;
    if (M > 0 && (!a->ifg || !dout || !d_ifg)) return set_error(MMF_EINVAL, "mlgru_backward: NULL ifg, dout or d_ifg");
    if ((a->h0 && !aligned16(a->h0)) || (a->f_bias && !aligned16(a->f_bias)) ||
        (a->gnorm_w && !aligned16(a->gnorm_w)) || (a->f_lower && !aligned16(a->f_lower)) ||
        (M > 0 && (!aligned16(a->ifg) || !aligned16(dout) || !aligned16(d_ifg))))
        return set_error(MMF_EALIGN, "mlgru_backward: a pointer is not 16-byte aligned");
    if ((rc = check_device())) return rc;
    hipError_t e = hipSuccess;
    if (M == 0) {   // dh0 = dh_last; the parameter gradients are empty sums
        if (dh0 && a->B > 0) e = launch_copy_state(dh_last, dh0, a->B * a->D, stream);
        if (e == hipSuccess && dgnorm_w) e = launch_fill_zero(dgnorm_w, a->D, stream);
        if (e == hipSuccess && df_bias) e = launch_fill_zero(df_bias, a->D, stream);
        return e == hipSuccess ? MMF_OK : hip_error(e, "mlgru_backward fill");
    }
    const size_t need = mlgru_backward_workspace_bytes(a->B, a->T, a->D);
    if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "mlgru_backward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
    if (!aligned16(ws)) return set_error(MMF_EALIGN, "mlgru_backward: workspace not 16-byte aligned");
    const int32_t nc = static_cast<int32_t>(scan_chunks(a->T));
    const size_t cn = static_cast<size_t>(a->B * nc * a->D) * 4;
    Carver c(ws);
    ScanArgs s{};
    s.ifg = a->ifg;
    s.ifg_bf16 = a->ifg_dt == MMF_BF16;
    s.f_bias = a->f_bias;
    s.f_lower = a->f_lower;
    s.h0 = a->h0;
    s.B = a->B;
    s.T = a->T;
    s.D = static_cast<int32_t>(a->D);
    s.chunk = kScanChunk;
    s.n_chunks = nc;
    {
        Carver sc(c.take<char>(scan_bytes(a->B, a->T, a->D)));
        if (nc > 1) {
            s.hloc = sc.take<float>(cn);
            s.pf = sc.take<float>(cn);
            s.hin = sc.take<float>(cn);
        }
    }
    MlgruBwdArgs b{};
    b.ifg = a->ifg;
    b.ifg_bf16 = s.ifg_bf16;
    b.f_bias = a->f_bias;
    b.f_lower = a->f_lower;
    b.h0 = a->h0;
    b.gnorm_w = a->gnorm_w;
    b.eps = a->eps;
    b.gate_mode = a->gate_mode;
    b.B = a->B;
    b.T = a->T;
    b.D = static_cast<int32_t>(a->D);
    b.n_chunks = nc;
    b.hin = s.hin;
    b.dout = dout;
    b.dout_bf16 = dout_dt == MMF_BF16;
    b.dh_last = dh_last;
    b.d_ifg = d_ifg;
    b.d_ifg_bf16 = d_ifg_bf16;
    b.dh0 = dh0;
    b.dgnorm_w = dgnorm_w;
    b.df_bias = df_bias;
    b.stats = c.take<float>(static_cast<size_t>(M) * 8);
    b.cb = c.take<float>(cn);
    b.cp = c.take<float>(cn);
    b.cf0 = c.take<float>(cn);
    b.cg = c.take<float>(cn);
    b.gw_part = c.take<float>(cn);
    b.fb_part = c.take<float>(cn);
    e = launch_scan_carries(s, stream);
    if (e == hipSuccess) e = launch_mlgru_bwd(b, stream);
    if (e != hipSuccess) return hip_error(e, "mlgru_backward launch");
    return MMF_OK;
}

extern "C" {

int mlgru_backward(const mmf_mlgru_args *a, const void *dout, mmf_dtype dout_dt, const float *dh_last,
                   float *d_ifg, float *dh0, float *dgnorm_w, float *df_bias, void *ws,
                   size_t ws_bytes, hipStream_t stream) {
    return mlgru_backward_impl(a, dout, dout_dt, dh_last, d_ifg, false, dh0, dgnorm_w, df_bias, ws,
                               ws_bytes, stream);
}

size_t block_backward_workspace_bytes(const mmf_block *w, int64_t B, int64_t T) {
    if (!w || B <= 0 || T <= 0) return 0;
    const int64_t M = B * T, D = w->i.K, F = w->gate.N, KN = std::max(D, F);
    const int64_t ldm = (M + 63) / 64 * 64;
    auto f4 = [](int64_t n) { return align_up(static_cast<size_t>(n) * 4); };
    auto h2 = [](int64_t n) { return align_up(static_cast<size_t>(n) * 2); };
    return 3 * qbuf_bytes(M, D) + qbuf_bytes(M, F) +                       // q of x, o, y1, m
           f4(M * 3 * D) + 2 * f4(M * D) + h2(M * 2 * F) + f4(M * F) +     // ifg, o, y1, gate|up (bf16), m
           scan_bytes(B, T, D) +                                           // forward chunk carries
           f4(M * KN) + h2(M * 2 * F) + f4(M * D) + h2(M * D) + f4(M * D) + h2(M * 3 * D) +
                                                              // g, dgu, dy1 (+ bf16), do, d_ifg
           h2(F * D) + h2(2 * F * D) + h2(D * D) + h2(3 * D * D) +         // bf16 W^T of all seven
           h2(KN * ldm) + h2(std::max(3 * D, 2 * F) * ldm) +               // q^T, (dy a)^T
           align_up(bwd_rows_part_bytes(M, static_cast<int32_t>(KN))) +   // dgamma partials
           mlgru_backward_workspace_bytes(B, T, D);
}

int block_backward(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                   const float *h0, const void *dy, mmf_dtype dy_dt, const float *dh_last, float *dx,
                   float *dh0, const mmf_block_grads *gr, void *ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_block(w, "block_backward");
    if (rc) return rc;
    if (!valid_dt(dt) || !valid_dt(dy_dt)) return set_error(MMF_EDTYPE, "block_backward: dtype %d/%d", dt, dy_dt);
    if (B < 0 || T < 0) return set_error(MMF_ESHAPE, "block_backward: B=%lld T=%lld", (long long)B, (long long)T);
    const int32_t D = w->i.K, F = w->gate.N;
    if (F % 8 || F > 8192) return set_error(MMF_ESHAPE, "block_backward: F=%d must be a multiple of 8 and <= 8192", F);
    // the row kernels read the gains 16 bytes at a time
    if ((w->i.norm_w && !aligned16(w->i.norm_w)) || (w->gate.norm_w && !aligned16(w->gate.norm_w)) ||
        (w->down.norm_w && !aligned16(w->down.norm_w)))
        return set_error(MMF_EALIGN, "block_backward: i/gate/down norm_w not 16-byte aligned");
    const int64_t M = B * T;
    static const mmf_block_grads none{};
    const mmf_block_grads &G = gr ? *gr : none;
    if ((h0 && !aligned16(h0)) || (dh_last && !aligned16(dh_last)) || (dh0 && !aligned16(dh0)) ||
        (M > 0 && (!aligned16(x) || !aligned16(dy) || !aligned16(dx))))
        return set_error(MMF_EALIGN, "block_backward: x/dy/dx/h0/dh_last/dh0 not 16-byte aligned");
    if (M > 0 && (!x || !dy || !dx)) return set_error(MMF_EINVAL, "block_backward: NULL x, dy or dx");
    const mmf_bitlinear *lin[7] = {&w->i, &w->f, &w->g, &w->o, &w->gate, &w->up, &w->down};
    if (M > 0) {
        const size_t need = block_backward_workspace_bytes(w, B, T);
        if (!ws || ws_bytes < need) return set_error(MMF_EWORKSPACE, "block_backward: workspace %zu < %zu", ws ? ws_bytes : 0, need);
        if (!aligned16(ws)) return set_error(MMF_EALIGN, "block_backward: workspace not 16-byte aligned");
    }
    if ((rc = check_device())) return rc;
    hipError_t e = hipSuccess;
    if (M == 0) {   // dh0 = dh_last; every parameter gradient is an empty sum
        if (dh0 && B > 0) e = launch_copy_state(dh_last, dh0, B * D, stream);
        for (int k = 0; k < 7 && e == hipSuccess; ++k) {
            if (G.dw[k]) e = launch_fill_zero(G.dw[k], static_cast<int64_t>(lin[k]->N) * lin[k]->K, stream);
            if (e == hipSuccess && G.db[k]) e = launch_fill_zero(G.db[k], lin[k]->N, stream);
        }
        const int32_t gk[4] = {D, D, D, F};
        for (int k = 0; k < 4 && e == hipSuccess; ++k)
            if (G.dgamma[k]) e = launch_fill_zero(G.dgamma[k], gk[k], stream);
        if (e == hipSuccess && G.dgnorm_w) e = launch_fill_zero(G.dgnorm_w, D, stream);
        if (e == hipSuccess && G.df_bias) e = launch_fill_zero(G.df_bias, D, stream);
        return e == hipSuccess ? MMF_OK : hip_error(e, "block_backward fill");
    }
    const bool bf = dt == MMF_BF16, dyb = dy_dt == MMF_BF16;
    const int64_t ldm = (M + 63) / 64 * 64, KN = std::max(D, F);
    Carver c(ws);
    const QBuf qx = take_qbuf(c, M, D), qo = take_qbuf(c, M, D), qy = take_qbuf(c, M, D), qm = take_qbuf(c, M, F);
    void *ifg = c.take<char>(static_cast<size_t>(M * 3 * D) * 4);
    void *o = c.take<char>(static_cast<size_t>(M * D) * 4);
    void *y1 = c.take<char>(static_cast<size_t>(M * D) * 4);
    uint16_t *gu = c.take<uint16_t>(static_cast<size_t>(M * 2 * F) * 2);
    void *m = c.take<char>(static_cast<size_t>(M * F) * 4);
    char *scan_ws = c.take<char>(scan_bytes(B, T, D));
    float *g = c.take<float>(static_cast<size_t>(M * KN) * 4);
    uint16_t *dgu = c.take<uint16_t>(static_cast<size_t>(M * 2 * F) * 2);
    float *dy1 = c.take<float>(static_cast<size_t>(M * D) * 4);
    uint16_t *dy1b = c.take<uint16_t>(static_cast<size_t>(M * D) * 2);
    float *dO = c.take<float>(static_cast<size_t>(M * D) * 4);
    uint16_t *d_ifg = c.take<uint16_t>(static_cast<size_t>(M * 3 * D) * 2);
    // the seven W^T in bf16, stacked per contraction: down [F][D], gate|up [D][2F], o [D][D],
    // i|f|g [D][3D]
    uint16_t *wt_dn = c.take<uint16_t>(static_cast<size_t>(F) * D * 2);
    uint16_t *wt_gu = c.take<uint16_t>(static_cast<size_t>(D) * 2 * F * 2);
    uint16_t *wt_o = c.take<uint16_t>(static_cast<size_t>(D) * D * 2);
    uint16_t *wt_ifg = c.take<uint16_t>(static_cast<size_t>(D) * 3 * D * 2);
    uint16_t *qT = c.take<uint16_t>(static_cast<size_t>(KN * ldm) * 2);
    uint16_t *dyaT = c.take<uint16_t>(static_cast<size_t>(std::max(3 * D, 2 * F) * ldm) * 2);
    float *dg_part = c.take<float>(bwd_rows_part_bytes(M, static_cast<int32_t>(KN)));
    const size_t mws_bytes = mlgru_backward_workspace_bytes(B, T, D);
    void *mws = c.take<char>(mws_bytes);
#define MMF_TRY(expr, what) do { if ((e = (expr)) != hipSuccess) return hip_error(e, "block_backward " what); } while (0)

    // ---- forward, recomputed: i|f|g, the MLGRU with its gate (o stored), o_proj + x -> y1,
    //      m = SiLU(gate)*up from the gate|up GEMM's GLU epilogue, which also keeps the gate
    //      and up pre-activations in bf16 for the product's backward
    const Seg sifg[3] = {seg_of(w->i, 0, 0), seg_of(w->f, D, D), seg_of(w->g, 2 * D, 2 * D)};
    const Seg so = seg_of(w->o, 0, 0);
    const Seg sgu[2] = {seg_of(w->gate, 0, 0), seg_of(w->up, F, F)};
    MMF_TRY(quantize(x, bf, w->i.norm_w, w->i.eps, M, D, qx, nullptr, stream), "quant x");
    MMF_TRY(gemm(qx, M, D, sifg, 3, EPI_STORE, ifg, 3 * D, bf, nullptr, 0, nullptr, 0, FAM_GEMM_IFG, stream), "ifg");
    {
        ScanArgs sa{};
        sa.ifg = ifg;
        sa.ifg_bf16 = bf;
        sa.f_bias = w->f_bias;
        sa.f_lower = w->f_lower;
        sa.h0 = h0;
        sa.gnorm_w = w->gnorm_w;
        sa.eps = w->eps;
        sa.gate_mode = w->gate_mode;
        sa.B = B;
        sa.T = T;
        sa.D = D;
        sa.chunk = kScanChunk;
        sa.n_chunks = static_cast<int32_t>(scan_chunks(T));
        if (sa.n_chunks > 1) {
            Carver sc(scan_ws);
            const size_t n = static_cast<size_t>(B * sa.n_chunks * D) * 4;
            sa.hloc = sc.take<float>(n);
            sa.pf = sc.take<float>(n);
            sa.hin = sc.take<float>(n);
        }
        sa.out = o;
        sa.out_bf16 = bf;
        MMF_TRY(launch_scan(sa, stream), "scan");
    }
    MMF_TRY(quantize(o, bf, w->o.norm_w, w->o.eps, M, D, qo, nullptr, stream), "quant o");
    MMF_TRY(gemm(qo, M, D, &so, 1, EPI_RESID, y1, D, bf, x, D, nullptr, 0, FAM_GEMM_O, stream), "o_proj");
    MMF_TRY(quantize(y1, bf, w->gate.norm_w, w->gate.eps, M, D, qy, nullptr, stream), "quant y1");
    MMF_TRY(gemm(qy, M, D, sgu, 2, EPI_GLU_KEEP, m, F, bf, nullptr, 0, nullptr, 0, FAM_GEMM_OTHER, stream, gu),
            "gate|up");
    MMF_TRY(quantize(m, bf, w->down.norm_w, w->down.eps, M, F, qm, nullptr, stream), "quant m");

    // Backward.  Each BitLinear: g = s_w dy T on the matrix cores, then the row kernel (dx,
    // dgamma from g and the normalisation's input); dW and db from the transposed (dy a) and
    // q.  Linears that share an input (gate | up; i | f | g) are one contraction over their
    // stacked dy, with one row kernel and one dW launch.  Gradients that feed a contraction are
    // kept in bf16 (dgate|dup, dy1's copy, d_ifg); those added as residuals stay fp32.
    auto rows = [&](const void *xin, const mmf_bitlinear &l, int32_t K) {
        BwdRowsArgs r{};
        r.x = xin;
        r.x_bf16 = bf;
        r.g = g;
        r.gamma = l.norm_w;
        r.eps = l.eps;
        r.M = M;
        r.K = K;
        r.dgamma_zeroed = 1;
        r.dg_part = dg_part;
        return r;
    };
    // the seven ternary matrices expanded to bf16 W^T by one launch
    {
        ExpandJobs ej{};
        auto job = [&](const mmf_bitlinear &l, uint16_t *out, int64_t ldo) {
            ej.packed[ej.count] = l.packed;
            ej.N[ej.count] = l.N;
            ej.K[ej.count] = l.K;
            ej.out[ej.count] = out;
            ej.ldo[ej.count++] = ldo;
        };
        job(w->down, wt_dn, D);
        job(w->gate, wt_gu, 2 * F);
        job(w->up, wt_gu + F, 2 * F);
        job(w->o, wt_o, D);
        job(w->i, wt_ifg, 3 * D);
        job(w->f, wt_ifg + D, 3 * D);
        job(w->g, wt_ifg + 2 * D, 3 * D);
        MMF_TRY(launch_expand_wt(ej, stream), "expand");
    }
    // every output that is accumulated (gains, biases, weights) zeroed by one launch
    {
        ZeroJobs z{};
        const int32_t gk[4] = {D, D, D, F};
        for (int k = 0; k < 4; ++k) {
            z.p[z.count] = G.dgamma[k];
            z.n[z.count++] = gk[k];
        }
        for (int k = 0; k < 7; ++k) {
            z.p[z.count] = G.db[k];
            z.n[z.count++] = lin[k]->N;
            z.p[z.count] = G.dw[k];
            z.n[z.count++] = static_cast<int64_t>(lin[k]->N) * lin[k]->K;
        }
        MMF_TRY(launch_fill_zero_many(z, stream), "zero");
    }
    // ---- down (its dx, the gradient at m, is carried through m = SiLU(gate)*up in the row kernel)
    {
        const uint32_t *pk[1] = {w->down.packed};
        const float sc[1] = {w->down.scale};
        MMF_TRY(bwd_launch_g(dy, dyb, D, pk, sc, 1, D, F, M, wt_dn, 1, g, stream), "down g");
        BwdRowsArgs r = rows(m, w->down, F);
        r.gu = gu;
        r.dgu = dgu;
        r.dgamma = G.dgamma[3];
        MMF_TRY(bwd_launch_rows(r, stream), "down rows");
        if (G.dw[6]) MMF_TRY(bwd_launch_qT(qm.q, M, F, ldm, qT, stream), "down qT");
        MMF_TRY(bwd_launch_dw(dy, dyb, D, qm.a, M, 1, D, F, ldm, qT, dyaT, &G.dw[6], &G.db[6], 1, stream), "down dw");
    }
    // ---- gate | up: dy1 = dy + gate^T(dgate) + up^T(dup)
    {
        const uint32_t *pk[2] = {w->gate.packed, w->up.packed};
        const float sc[2] = {w->gate.scale, w->up.scale};
        MMF_TRY(bwd_launch_g(dgu, 1, 2 * F, pk, sc, 2, F, D, M, wt_gu, 1, g, stream), "gate|up g");
        BwdRowsArgs r = rows(y1, w->gate, D);
        r.dx = dy1;
        r.dx_bf16 = dy1b;
        r.res = dy;
        r.res_bf16 = dyb;
        r.dgamma = G.dgamma[2];
        MMF_TRY(bwd_launch_rows(r, stream), "gate|up rows");
        if (G.dw[4] || G.dw[5]) MMF_TRY(bwd_launch_qT(qy.q, M, D, ldm, qT, stream), "gate|up qT");
        MMF_TRY(bwd_launch_dw(dgu, 1, 2 * F, qy.a, M, 2, F, D, ldm, qT, dyaT, &G.dw[4], &G.db[4], 1, stream), "gate|up dw");
    }
    // ---- o_proj: do = o^T(dy1)
    {
        const uint32_t *pk[1] = {w->o.packed};
        const float sc[1] = {w->o.scale};
        MMF_TRY(bwd_launch_g(dy1b, 1, D, pk, sc, 1, D, D, M, wt_o, 1, g, stream), "o g");
        BwdRowsArgs r = rows(o, w->o, D);
        r.dx = dO;
        r.dgamma = G.dgamma[1];
        MMF_TRY(bwd_launch_rows(r, stream), "o rows");
        if (G.dw[3]) MMF_TRY(bwd_launch_qT(qo.q, M, D, ldm, qT, stream), "o qT");
        MMF_TRY(bwd_launch_dw(dy1b, 1, D, qo.a, M, 1, D, D, ldm, qT, dyaT, &G.dw[3], &G.db[3], 1, stream), "o dw");
    }
#undef MMF_TRY
    // ---- the MLGRU with its output gate
    {
        mmf_mlgru_args ma{};
        ma.ifg = ifg;
        ma.ifg_dt = dt;
        ma.f_bias = w->f_bias;
        ma.h0 = h0;
        ma.gnorm_w = w->gnorm_w;
        ma.eps = w->eps;
        ma.gate_mode = w->gate_mode;
        ma.out_dt = dt;
        ma.B = B;
        ma.T = T;
        ma.D = D;
        ma.f_lower = w->f_lower;
        if ((rc = mlgru_backward_impl(&ma, dO, MMF_F32, dh_last, d_ifg, true, dh0, G.dgnorm_w, G.df_bias, mws,
                                      mws_bytes, stream)))
            return rc;
    }
    // ---- i | f | g: dx = dy1 + i^T(d_i) + f^T(d_f) + g^T(d_g)
#define MMF_TRY(expr, what) do { if ((e = (expr)) != hipSuccess) return hip_error(e, "block_backward " what); } while (0)
    {
        const uint32_t *pk[3] = {w->i.packed, w->f.packed, w->g.packed};
        const float sc[3] = {w->i.scale, w->f.scale, w->g.scale};
        MMF_TRY(bwd_launch_g(d_ifg, 1, 3 * D, pk, sc, 3, D, D, M, wt_ifg, 1, g, stream), "ifg g");
        BwdRowsArgs r = rows(x, w->i, D);
        r.dx = dx;
        r.res = dy1;
        r.res_bf16 = 0;
        r.dgamma = G.dgamma[0];
        MMF_TRY(bwd_launch_rows(r, stream), "ifg rows");
        if (G.dw[0] || G.dw[1] || G.dw[2]) MMF_TRY(bwd_launch_qT(qx.q, M, D, ldm, qT, stream), "ifg qT");
        MMF_TRY(bwd_launch_dw(d_ifg, 1, 3 * D, qx.a, M, 3, D, D, ldm, qT, dyaT, &G.dw[0], &G.db[0], 1, stream), "ifg dw");
    }
#undef MMF_TRY
    return MMF_OK;
}

}  // extern "C"
