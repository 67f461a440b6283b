/*
 * mmf_oracle.c -- plain, slow CPU oracle of the MatMul-free LM block forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or load this
 * file; only the tests, the package's smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [DC-ternary] DataCamp blog "MatMul-free language models" (zh), section
 *                "Replacing MatMul with ternary operations" (用三值运算取代 MatMul):
 *                BitLinear weights restricted to {-1,0,1}; absmean quantization scales the
 *                matrix by the mean absolute value of its elements and rounds each element
 *                to the nearest of -1, 0, 1; products by -1/0/1 become negate/drop/keep.
 *   [DC-core]    same page, section "Core components: MLGRU and GLU" (核心组件：MLGRU 与 GLU):
 *                RMSNorm normalises activations before they are quantized; MLGRU keeps a
 *                hidden state updated token by token through element-wise gates in (0,1);
 *                the MatMul-free GLU applies two BitLinears, SiLU on one branch, an
 *                element-wise product and a third BitLinear.
 *   [HL-fbl]     Hysen Labs project page "MatMul-Free LM: 用三元权重和门控循环把矩阵乘法请出语言模型",
 *                section "FusedBitLinear": each projection RMS-normalises its input, then
 *                quantizes and accumulates against the ternary weights.
 *   [HL-hgrn]    same page, section "HGRN attention: gated recurrence replaces softmax":
 *                block input -> RMSNorm -> i/f/g projections -> recurrence -> g_norm
 *                (RMSNorm fused with a swish gate) -> o_proj.
 *   [DC-train]   DataCamp page, section "Replacing MatMul with ternary operations": the
 *                weights are trained in full precision and ternarized during training;
 *                section "From optimised GPU to custom FPGA": fused training kernels.
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   R1  activations: per-token symmetric absmax int8 in [-127,127]; the RMSNorm factor r
 *       cancels in the absmax ratio, so q is computed from x*gamma and r enters only the
 *       dequantization scale a = r*max|x*gamma|/127.
 *   R2  both quantizers round half to even (rintf in the default rounding mode).
 *   R3  guards: absmean scale and row absmax are floored at 1e-5.
 *   R4  absmean sum: per row in double (k ascending), rows summed in double (n ascending).
 *   R5  MLGRU: f = sigmoid(f_pre + b_f), c = SiLU(i_pre), h_t = f*h_{t-1} + (1-f)*c;
 *       i_proj feeds the candidate, f_proj the forget gate, g_proj the output gate.
 *   R6  output gate: o = RMSNorm_D(h)*gamma_g * g*sigmoid(g) (default) or sigmoid(g)*h.
 *   R7  block: pre-norm residuals y1 = x + o_proj(...), y2 = y1 + GLU(y1); one RMSNorm per
 *       BitLinear input; y1 and y2 rounded once to the residual dtype.
 *   R8  every tensor that one of the pages' modules hands to the next is materialised in
 *       the activation dtype (bf16 for bf16 workloads, fp32 otherwise), as the pages' model
 *       runs in half precision (Hysen Labs, section on the official generation example:
 *       the model is moved to the GPU in half precision).  The modules are the ones the
 *       pages name: the i, f and g projections (their outputs feed the recurrence), g_norm
 *       (Hysen Labs, "HGRN attention": a module of its own whose output feeds o_proj),
 *       the MatMul-free GLU's gated product (DataCamp, "Core components": formed from the
 *       two branches, then passed to the third BitLinear), and the residual stream y1, y2.
 *       The recurrent state h is carried in fp32 and is not rounded.
 *   R12 HGRN's hierarchical forget-gate lower bound (Hysen Labs, "HGRN attention", names
 *       the Hierarchical Gated Recurrent Network but not its formula; the formula is read
 *       from HGRN's published design and its parity is unpinned by the pages): layer l has
 *       a per-channel bound lb_l in [0,1) that grows with depth, made from per-layer logits
 *       G[L][D] as an exclusive cumulative softmax over the layers, lb_l[d] =
 *       sum_{j<l} exp(G[j][d]) / sum_j exp(G[j][d]) (layer 0 is unbounded); the forget gate
 *       becomes f = lb + (1 - lb)*sigmoid(f_pre + b_f).
 *   R14 backward ([DC-train]; the pages do not say how a gradient crosses the quantizers):
 *       the straight-through estimator -- the activation quantizer passes the gradient of
 *       its dequantized output x_hat = q*a unchanged to x*gamma*r (the RMS-normalised input
 *       it approximates), and the ternarizer passes the gradient of W_hat = s_w*T unchanged
 *       to the latent weights.  Everything else (RMSNorm, the gates, the recurrence,
 *       g_norm) is differentiated exactly.
 *
 * Floating point: every non-quantizer computation is fp64.  The quantizers (ternarize,
 * activation quant) are defined in fp32 so that both sides take each integer decision in
 * the same precision.  Build with -ffp-contract=off and without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_ABI_VERSION 1

int orc_abi_version(void) { return ORC_ABI_VERSION; }
int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* A ternary linear layer as the oracle sees it: q in {-1,0,1}, row n = output feature. */
typedef struct orc_linear {
    const int8_t *q;      /* [n, k] */
    float scale;          /* absmean scale s (dequantized weight = q*s) */
    const float *gamma;   /* [k] RMSNorm gain of the input, or NULL for ones */
    const float *bias;    /* [n] or NULL */
    int64_t n, k;
} orc_linear;

/* ---------------------------------------------------------------- helpers (fp64) */

static double sigmoid_d(double z) { return 1.0 / (1.0 + exp(-z)); }
static double silu_d(double z) { return z * sigmoid_d(z); }

/* Round a double to the nearest bfloat16 value (ties to even), returned as a double.
 * One rounding: the value is scaled by an exact power of two so that the bf16 unit in the
 * last place becomes 1, rounded to an integer, and scaled back. */
double orc_round_bf16(double d) {
    if (d == 0.0 || !isfinite(d)) return d;
    int e;
    frexp(d, &e);                 /* d = m * 2^e, 0.5 <= |m| < 1 */
    int ulp = e - 8;              /* bf16 keeps 8 significant bits */
    if (ulp < -133) ulp = -133;   /* subnormal range: fixed ulp 2^-133 */
    double r = ldexp(nearbyint(ldexp(d, -ulp)), ulp);
    if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, d);
    return r;
}

/* -------------------------------------------------------- O1 absmean ternarization
 * [DC-ternary]: scale by the mean absolute value of the whole matrix, round each element
 * to the nearest integer in {-1,0,1}.  Readings R2, R3, R4.
 */
int orc_ternarize(const float *w, int64_t n, int64_t k, int8_t *q, float *scale) {
    if (!w || !q || !scale || n <= 0 || k <= 0) return -1;
    double total = 0.0;
    for (int64_t r = 0; r < n; ++r) {
        double row = 0.0;
        for (int64_t c = 0; c < k; ++c) row += fabs((double)w[r * k + c]);
        total += row;
    }
    float mean_abs = (float)(total / ((double)n * (double)k));
    float s = mean_abs > 1e-5f ? mean_abs : 1e-5f;
    for (int64_t i = 0; i < n * k; ++i) {
        float v = rintf(w[i] / s);
        if (v > 1.0f) v = 1.0f;
        if (v < -1.0f) v = -1.0f;
        q[i] = (int8_t)v;
    }
    *scale = s;
    return 0;
}

/* ------------------------------------------------------------- O2 2-bit packing
 * Storage format for the ternary weights (the pages only say "trits"): code = q + 1 in
 * {0,1,2}; a row of k values is stored as k/16 little-endian 32-bit words; element
 * k = 16*j + 4*a + b lives in word j at bits [8*b + 2*a, 8*b + 2*a + 1].
 */
int orc_pack(const int8_t *q, int64_t n, int64_t k, uint32_t *packed) {
    if (!q || !packed || n <= 0 || k <= 0 || k % 16) return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < k / 16; ++j) {
            uint32_t word = 0;
            for (int a = 0; a < 4; ++a)
                for (int b = 0; b < 4; ++b) {
                    int v = q[r * k + 16 * j + 4 * a + b];
                    if (v < -1 || v > 1) return -1;
                    word |= (uint32_t)(v + 1) << (8 * b + 2 * a);
                }
            packed[r * (k / 16) + j] = word;
        }
    return 0;
}

int orc_unpack(const uint32_t *packed, int64_t n, int64_t k, int8_t *q) {
    if (!q || !packed || n <= 0 || k <= 0 || k % 16) return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t kk = 0; kk < k; ++kk) {
            int64_t j = kk / 16, a = (kk % 16) / 4, b = kk % 4;
            uint32_t code = (packed[r * (k / 16) + j] >> (8 * b + 2 * a)) & 3u;
            if (code == 3u) return -2;
            q[r * k + kk] = (int8_t)((int)code - 1);
        }
    return 0;
}

/* ------------------------------------------- base-3 "trit" packing (1.6 bits)
 * HackerPapers page on arXiv 2406.02528 (HN discussion list): the weights are ternary digits,
 * "trits", with values in {-1, 0, 1}.  Five trits fit in a byte (3^5 = 243 <= 256).
 * Format (a reading; the pages give none): codes c = q + 1 in {0,1,2}; a row is cut into
 * words of 4 bytes = 20 trits; byte j (0..3) of word w holds the codes of
 * k = 20w + 4i + j for i = 0..4 as the base-3 number v = sum_i c_i * 3^(4-i) (i = 0 most
 * significant), stored as b = ceil(256*v/243); a row is padded with code 1 (q = 0) to whole
 * 16-byte chunks of 80 trits.  The oracle decodes by the definition: v = floor(243*b/256)
 * (exact inverse, as 243/256 < 1) and base-3 digits by repeated division.
 */
int64_t orc_trit_row_bytes(int64_t k) { return 16 * ((k + 79) / 80); }

static int64_t trit_pos(int64_t byte_in_row, int i) {   /* k of digit i of a row byte */
    int64_t w = byte_in_row / 4, j = byte_in_row % 4;
    return 20 * w + 4 * i + j;
}

int orc_pack_trits(const int8_t *q, int64_t n, int64_t k, uint8_t *packed) {
    if (!q || !packed || n <= 0 || k <= 0) return -1;
    int64_t rb = orc_trit_row_bytes(k);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t by = 0; by < rb; ++by) {
            int v = 0;
            for (int i = 0; i < 5; ++i) {
                int64_t kk = trit_pos(by, i);
                int c = 1;                               /* padding: q = 0 */
                if (kk < k) {
                    int qq = q[r * k + kk];
                    if (qq < -1 || qq > 1) return -1;
                    c = qq + 1;
                }
                v = 3 * v + c;
            }
            packed[r * rb + by] = (uint8_t)((256 * v + 242) / 243);   /* ceil(256 v / 243) */
        }
    return 0;
}

int orc_unpack_trits(const uint8_t *packed, int64_t n, int64_t k, int8_t *q) {
    if (!q || !packed || n <= 0 || k <= 0) return -1;
    int64_t rb = orc_trit_row_bytes(k);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t by = 0; by < rb; ++by) {
            int b = packed[r * rb + by];
            int v = (243 * b) / 256;
            if ((256 * v + 242) / 243 != b) return -2;   /* not the encoding of any v */
            int c[5];
            for (int i = 4; i >= 0; --i) { c[i] = v % 3; v /= 3; }
            for (int i = 0; i < 5; ++i) {
                int64_t kk = trit_pos(by, i);
                if (kk < k) q[r * k + kk] = (int8_t)(c[i] - 1);
                else if (c[i] != 1) return -2;           /* padding must be q = 0 */
            }
        }
    return 0;
}

/* ------------------------------------------------- O3 activation quantization
 * [DC-core] RMSNorm before quantization; [HL-fbl] norm -> quantize -> accumulate.
 * Per row: p = fl32(x*gamma); m = max|p| floored at 1e-5; s = fl32(127/m);
 * q = clamp(rne(fl32(p*s)), -127, 127); r = 1/sqrt(mean x^2 + eps) (fp64);
 * a = r*m/127 (fp64).  Readings R1, R2, R3.
 */
void orc_act_quant(const float *x, int64_t m, int64_t k, const float *gamma, double eps,
                   int8_t *q, double *a, int32_t *rowsum) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        const float *xr = x + row * k;
        float mx = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            float p = gamma ? xr[c] * gamma[c] : xr[c];
            float ap = fabsf(p);
            if (ap > mx) mx = ap;
        }
        float me = mx > 1e-5f ? mx : 1e-5f;
        float s = 127.0f / me;
        int32_t sum = 0;
        double ss = 0.0;
        for (int64_t c = 0; c < k; ++c) {
            float p = gamma ? xr[c] * gamma[c] : xr[c];
            float v = rintf(p * s);
            if (v > 127.0f) v = 127.0f;
            if (v < -127.0f) v = -127.0f;
            int8_t qi = (int8_t)v;
            if (q) q[row * k + c] = qi;
            sum += qi;
            ss += (double)xr[c] * (double)xr[c];
        }
        double r = 1.0 / sqrt(ss / (double)k + eps);
        if (a) a[row] = r * (double)me / 127.0;
        if (rowsum) rowsum[row] = sum;
    }
}

/* ------------------------------------------------------- O4 ternary accumulate
 * [DC-ternary]: multiplying by -1/0/1 is negate/drop/keep, so the product with the
 * weight matrix is a signed sum of int8 activations.  Exact in int32.
 */
void orc_accumulate(const int8_t *qx, const int8_t *qw, int64_t m, int64_t n, int64_t k,
                    int32_t *acc) {
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row)
        for (int64_t col = 0; col < n; ++col) {
            const int8_t *xr = qx + row * k, *wr = qw + col * k;
            int32_t s = 0;
            for (int64_t c = 0; c < k; ++c) {
                if (wr[c] > 0) s += xr[c];
                else if (wr[c] < 0) s -= xr[c];
            }
            acc[row * n + col] = s;
        }
}

/* ---------------------------------------------------------------- O5 BitLinear
 * y[m, n] = acc[m, n] * s_w * a[m] + bias[n], fp64.  Optional outputs: q_x, a, acc.
 */
int orc_bitlinear(const float *x, int64_t m, const orc_linear *w, double eps, double *y,
                  int8_t *q_out, double *a_out, int32_t *acc_out) {
    if (!x || !w || !y || m < 0 || w->n <= 0 || w->k <= 0) return -1;
    if (m == 0) return 0;
    int64_t k = w->k, n = w->n;
    int8_t *q = q_out ? q_out : (int8_t *)malloc((size_t)(m * k));
    double *a = a_out ? a_out : (double *)malloc(sizeof(double) * (size_t)m);
    int32_t *acc = acc_out ? acc_out : (int32_t *)malloc(sizeof(int32_t) * (size_t)(m * n));
    if (!q || !a || !acc) return -3;
    orc_act_quant(x, m, k, w->gamma, eps, q, a, NULL);
    orc_accumulate(q, w->q, m, n, k, acc);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row)
        for (int64_t col = 0; col < n; ++col)
            y[row * n + col] = (double)acc[row * n + col] * (double)w->scale * a[row] +
                               (w->bias ? (double)w->bias[col] : 0.0);
    if (!q_out) free(q);
    if (!a_out) free(a);
    if (!acc_out) free(acc);
    return 0;
}

/* ------------------------------------------------------- O6 gated recurrence
 * [DC-core]: the hidden state is the memory; gates in (0,1) decide what flows.
 * h_t = f_t*h_{t-1} + (1-f_t)*c_t per (b, d), t ascending.  f, c given (post-activation).
 * Layout [B, T, D]; h0 [B, D] or NULL (zeros); h_seq [B, T, D] and h_last [B, D] optional.
 */
void orc_gated_recurrence(const double *f, const double *c, int64_t B, int64_t T, int64_t D,
                          const double *h0, double *h_seq, double *h_last) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            double h = h0 ? h0[b * D + d] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t i = (b * T + t) * D + d;
                h = f[i] * h + (1.0 - f[i]) * c[i];
                if (h_seq) h_seq[i] = h;
            }
            if (h_last) h_last[b * D + d] = h;
        }
}

/* ----------------------------------------------------- O6 + O7 MLGRU with output gate
 * ifg: [B, T, 3D] pre-activations, segments i | f | g along the last axis.
 * [HL-hgrn] i/f/g projections, recurrence, g_norm = RMSNorm fused with a swish gate.
 * Readings R5, R6, R12 (f_lower [D] or NULL).  gate_mode 0: out = h*rsqrt(mean_D h^2 + eps)*gnorm_w * g*sigmoid(g);
 * gate_mode 1: out = sigmoid(g)*h.  h_last [B, D] receives h_T.
 */
int orc_mlgru(const double *ifg, int64_t B, int64_t T, int64_t D, const float *f_bias,
              const float *f_lower, const double *h0, const float *gnorm_w, double eps,
              int gate_mode, double *out, double *h_last) {
    if (!ifg || !out || B <= 0 || T < 0 || D <= 0 || (gate_mode != 0 && gate_mode != 1))
        return -1;
    int64_t M = B * T;
    double *f = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *c = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    if (!f || !c || !h) return -3;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < M; ++row)
        for (int64_t d = 0; d < D; ++d) {
            const double *r = ifg + row * 3 * D;
            double sg = sigmoid_d(r[D + d] + (f_bias ? (double)f_bias[d] : 0.0));
            double lb = f_lower ? (double)f_lower[d] : 0.0;   /* reading R12 */
            f[row * D + d] = lb + (1.0 - lb) * sg;
            c[row * D + d] = silu_d(r[d]);
        }
    orc_gated_recurrence(f, c, B, T, D, h0, h, h_last);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < M; ++row) {
        const double *g = ifg + row * 3 * D + 2 * D;
        const double *hr = h + row * D;
        if (gate_mode == 0) {
            double ss = 0.0;
            for (int64_t d = 0; d < D; ++d) ss += hr[d] * hr[d];
            double r = 1.0 / sqrt(ss / (double)D + eps);
            for (int64_t d = 0; d < D; ++d)
                out[row * D + d] =
                    hr[d] * r * (gnorm_w ? (double)gnorm_w[d] : 1.0) * silu_d(g[d]);
        } else {
            for (int64_t d = 0; d < D; ++d) out[row * D + d] = sigmoid_d(g[d]) * hr[d];
        }
    }
    free(f);
    free(c);
    free(h);
    return 0;
}

/* ------------------------------------------- B1 BitLinear backward (reading R14)
 * Forward (O3-O5): y = x_hat W_hat^T + b, x_hat[m,c] = q[m,c]*a[m], W_hat = s_w*T.  With
 * the straight-through estimator, x_hat stands for u = x*gamma*r (r = (mean_c x^2 +
 * eps)^(-1/2) per row) and W_hat for the latent weights.  Given dy [m, n]:
 *   g[m,c]     = sum_n dy[m,n] W_hat[n,c]            gradient at u
 *   dw[n,c]    = sum_m dy[m,n] x_hat[m,c]            gradient of the latent weights
 *   db[n]      = sum_m dy[m,n]
 *   dgamma[c]  = sum_m g[m,c] x[m,c] r[m]
 *   dx[m,c]    = r gamma_c g[m,c] - x[m,c] r^3 / k * sum_j g[m,j] gamma_j x[m,j]
 * (u_j = gamma_j x_j r and dr/dx_c = -x_c r^3 / k).  gamma NULL means gamma = 1.  Every
 * output may be NULL.  fp64.
 */
int orc_bitlinear_backward(const float *x, int64_t m, const orc_linear *w, double eps,
                           const double *dy, double *dx, double *dgamma, double *dw,
                           double *db) {
    if (!x || !w || !dy || m < 0 || w->n <= 0 || w->k <= 0) return -1;
    const int64_t k = w->k, n = w->n;
    int8_t *q = (int8_t *)malloc((size_t)(m * k + 1));
    double *a = (double *)malloc(sizeof(double) * (size_t)(m + 1));
    double *g = (double *)malloc(sizeof(double) * (size_t)(m * k + 1));
    double *r = (double *)malloc(sizeof(double) * (size_t)(m + 1));
    if (!q || !a || !g || !r) return -3;
    orc_act_quant(x, m, k, w->gamma, eps, q, a, NULL);
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < m; ++row) {
        double ss = 0.0;
        for (int64_t c = 0; c < k; ++c) ss += (double)x[row * k + c] * (double)x[row * k + c];
        r[row] = 1.0 / sqrt(ss / (double)k + eps);
        for (int64_t c = 0; c < k; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j) acc += dy[row * n + j] * (double)w->q[j * k + c];
            g[row * k + c] = acc * (double)w->scale;
        }
    }
    if (dw) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j)
            for (int64_t c = 0; c < k; ++c) {
                double acc = 0.0;
                for (int64_t row = 0; row < m; ++row)
                    acc += dy[row * n + j] * (double)q[row * k + c] * a[row];
                dw[j * k + c] = acc;
            }
    }
    if (db)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t row = 0; row < m; ++row) acc += dy[row * n + j];
            db[j] = acc;
        }
    if (dgamma)
        for (int64_t c = 0; c < k; ++c) {
            double acc = 0.0;
            for (int64_t row = 0; row < m; ++row) acc += g[row * k + c] * (double)x[row * k + c] * r[row];
            dgamma[c] = acc;
        }
    if (dx) {
#pragma omp parallel for schedule(static)
        for (int64_t row = 0; row < m; ++row) {
            const float *xr = x + row * k;
            double dot = 0.0;
            for (int64_t c = 0; c < k; ++c)
                dot += g[row * k + c] * (w->gamma ? (double)w->gamma[c] : 1.0) * (double)xr[c];
            const double r1 = r[row], r3 = r1 * r1 * r1;
            for (int64_t c = 0; c < k; ++c)
                dx[row * k + c] = r1 * (w->gamma ? (double)w->gamma[c] : 1.0) * g[row * k + c] -
                                  (double)xr[c] * r3 / (double)k * dot;
        }
    }
    free(q);
    free(a);
    free(g);
    free(r);
    return 0;
}

/* ------------------------------------ B2 MLGRU + output gate backward (reading R14)
 * Forward: orc_mlgru.  Given dout [B,T,D] (gradient at the gated output) and dh_last [B,D]
 * (gradient at the final state, or NULL), returns d_ifg [B,T,3D] (gradients of the i | f | g
 * pre-activations), and, each optional, dh0 [B,D], dgnorm_w [D], df_bias [D].
 *   gate_mode 0: n = h*rho, rho = (mean_D h^2 + eps)^(-1/2), out = n*w*silu(g):
 *     dg = dout*n*w*silu'(g);  dn = dout*w*silu(g);  dgnorm_w += dout*n*silu(g);
 *     dh_out = rho*dn - h*rho^3/D * sum_D(dn*h)
 *   gate_mode 1: out = sigmoid(g)*h: dg = dout*h*sigmoid'(g);  dh_out = dout*sigmoid(g)
 *   reverse recurrence, t descending: G_t = dh_out_t + f_{t+1}*G_{t+1} (dh_last joins at the
 *     last step); dc = (1-f_t)*G_t;  df = (h_{t-1} - c_t)*G_t;  di = dc*silu'(i);
 *     dz = df*(1-lb)*sigmoid(z)*(1-sigmoid(z)), z = f_pre + b_f (= the f_pre gradient, and
 *     summed over tokens, df_bias);  dh0 = f_0*G_0.
 * silu'(z) = sigmoid(z)*(1 + z*(1 - sigmoid(z))).  fp64.
 */
int orc_mlgru_backward(const double *ifg, int64_t B, int64_t T, int64_t D, const float *f_bias,
                       const float *f_lower, const double *h0, const float *gnorm_w, double eps,
                       int gate_mode, const double *dout, const double *dh_last, double *d_ifg,
                       double *dh0, double *dgnorm_w, double *df_bias) {
    if (!ifg || !dout || !d_ifg || B <= 0 || T < 0 || D <= 0 || (gate_mode != 0 && gate_mode != 1))
        return -1;
    const int64_t M = B * T;
    double *f = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *c = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *h = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *dho = (double *)malloc(sizeof(double) * (size_t)(M * D + 1));
    double *gw_part = (double *)calloc((size_t)(M * D + 1), sizeof(double));
    if (!f || !c || !h || !dho || !gw_part) return -3;
    for (int64_t row = 0; row < M; ++row)
        for (int64_t d = 0; d < D; ++d) {   /* the forward's gates (O6), recomputed */
            const double *r = ifg + row * 3 * D;
            const double zf = r[D + d] + (f_bias ? (double)f_bias[d] : 0.0);
            const double lbd = f_lower ? (double)f_lower[d] : 0.0;
            f[row * D + d] = lbd + (1.0 - lbd) * sigmoid_d(zf);
            c[row * D + d] = silu_d(r[d]);
        }
    orc_gated_recurrence(f, c, B, T, D, h0, h, NULL);
    /* output gate backward, token by token */
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < M; ++row) {
        const double *g = ifg + row * 3 * D + 2 * D, *hr = h + row * D, *dor = dout + row * D;
        double *dg = d_ifg + row * 3 * D + 2 * D;
        if (gate_mode == 0) {
            double ss = 0.0;
            for (int64_t d = 0; d < D; ++d) ss += hr[d] * hr[d];
            const double rho = 1.0 / sqrt(ss / (double)D + eps);
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                const double w = gnorm_w ? (double)gnorm_w[d] : 1.0;
                const double sgm = sigmoid_d(g[d]);
                const double n = hr[d] * rho;
                dg[d] = dor[d] * n * w * sgm * (1.0 + g[d] * (1.0 - sgm));
                gw_part[row * D + d] = dor[d] * n * silu_d(g[d]);
                const double dn = dor[d] * w * silu_d(g[d]);
                dho[row * D + d] = dn;   /* finished below */
                dot += dn * hr[d];
            }
            for (int64_t d = 0; d < D; ++d)
                dho[row * D + d] = rho * dho[row * D + d] - hr[d] * rho * rho * rho / (double)D * dot;
        } else {
            for (int64_t d = 0; d < D; ++d) {
                const double sgm = sigmoid_d(g[d]);
                dg[d] = dor[d] * hr[d] * sgm * (1.0 - sgm);
                dho[row * D + d] = dor[d] * sgm;
            }
        }
    }
    /* reverse recurrence, per (b, d) */
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t d = 0; d < D; ++d) {
            double G = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t i = (b * T + t) * D + d;
                G = dho[i] + (t == T - 1 ? (dh_last ? dh_last[b * D + d] : 0.0)
                                         : f[(b * T + t + 1) * D + d] * G);
                const double hp = t > 0 ? h[i - D] : (h0 ? h0[b * D + d] : 0.0);
                const double *r = ifg + (b * T + t) * 3 * D;
                const double si = sigmoid_d(r[d]);
                d_ifg[(b * T + t) * 3 * D + d] = (1.0 - f[i]) * G * si * (1.0 + r[d] * (1.0 - si));
                const double z = r[D + d] + (f_bias ? (double)f_bias[d] : 0.0), sz = sigmoid_d(z);
                const double lb = f_lower ? (double)f_lower[d] : 0.0;
                d_ifg[(b * T + t) * 3 * D + D + d] = (hp - c[i]) * G * (1.0 - lb) * sz * (1.0 - sz);
            }
            if (dh0) dh0[b * D + d] = T > 0 ? f[(b * T) * D + d] * G : (dh_last ? dh_last[b * D + d] : 0.0);
        }
    if (dgnorm_w)
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t row = 0; row < M; ++row) acc += gw_part[row * D + d];
            dgnorm_w[d] = gate_mode == 0 ? acc : 0.0;
        }
    if (df_bias)
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t row = 0; row < M; ++row) acc += d_ifg[row * 3 * D + D + d];
            df_bias[d] = acc;
        }
    free(f);
    free(c);
    free(h);
    free(dho);
    free(gw_part);
    return 0;
}

/* Round a double activation to the activation dtype (reading R8): bf16 or fp32. */
static void to_act(const double *src, float *dst, int64_t n, int act_bf16) {
    for (int64_t i = 0; i < n; ++i)
        dst[i] = act_bf16 ? (float)orc_round_bf16(src[i]) : (float)src[i];
}

/* Per-BitLinear stage record of a block run (every pointer optional). */
typedef struct orc_stage {
    float *x_in;   /* [M, K] fp32 stage input as quantized */
    int8_t *q;     /* [M, K] */
    double *a;     /* [M] */
    int32_t *acc;  /* [M, N]; for a group of projections sharing one input, N is the
                      sum of their widths and the projections sit side by side */
} orc_stage;

/* Several BitLinears applied to one input x [M, K]: outs[p] = BitLinear_p(x) [M, n_p].
 * The input is quantized once per projection (identically, as the gain is shared). */
static int group_bitlinear(const float *x, int64_t M, int np, const orc_linear *const *w,
                           double eps, double *const *outs, orc_stage *st) {
    int64_t K = w[0]->k, ntot = 0;
    for (int p = 0; p < np; ++p) ntot += w[p]->n;
    int8_t *q = (int8_t *)malloc((size_t)(M * K));
    double *a = (double *)malloc(sizeof(double) * (size_t)M);
    if (!q || !a) return -3;
    int64_t off = 0;
    for (int p = 0; p < np; ++p) {
        int64_t n = w[p]->n;
        int32_t *acc = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M * n));
        if (!acc) return -3;
        int rc = orc_bitlinear(x, M, w[p], eps, outs[p], q, a, acc);
        if (rc) return rc;
        if (st && st->acc)
            for (int64_t r = 0; r < M; ++r)
                memcpy(st->acc + r * ntot + off, acc + r * n, sizeof(int32_t) * (size_t)n);
        off += n;
        free(acc);
    }
    if (st) {
        if (st->x_in) memcpy(st->x_in, x, sizeof(float) * (size_t)(M * K));
        if (st->q) memcpy(st->q, q, (size_t)(M * K));
        if (st->a) memcpy(st->a, a, sizeof(double) * (size_t)M);
    }
    free(q);
    free(a);
    return 0;
}

/* ------------------------------------------------------------------ O8 GLU
 * [DC-core]: two BitLinears on the input, SiLU on one branch, element-wise product, a
 * third BitLinear.  x [M, D] -> y [M, D] (fp64, no residual).  m_out [M, F] receives the
 * stage input of the down projection, rounded to the activation dtype (optional; R8).
 */
static int glu_impl(const float *x, int64_t M, const orc_linear *gate, const orc_linear *up,
                    const orc_linear *down, double eps, int act_bf16, double *y, float *m_out,
                    orc_stage *st_gu, orc_stage *st_down) {
    if (gate->n != up->n || gate->k != up->k || down->k != gate->n || down->n != gate->k)
        return -1;
    int64_t F = gate->n;
    double *yg = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *yu = (double *)malloc(sizeof(double) * (size_t)(M * F));
    float *mm = (float *)malloc(sizeof(float) * (size_t)(M * F));
    if (!yg || !yu || !mm) return -3;
    const orc_linear *gu[2] = {gate, up};
    double *outs[2] = {yg, yu};
    int rc = group_bitlinear(x, M, 2, gu, eps, outs, st_gu);
    if (rc) return rc;
    for (int64_t i = 0; i < M * F; ++i) yg[i] = silu_d(yg[i]) * yu[i];
    to_act(yg, mm, M * F, act_bf16);
    if (m_out) memcpy(m_out, mm, sizeof(float) * (size_t)(M * F));
    if (st_down && st_down->x_in) memcpy(st_down->x_in, mm, sizeof(float) * (size_t)(M * F));
    rc = orc_bitlinear(mm, M, down, eps, y, st_down ? st_down->q : NULL,
                       st_down ? st_down->a : NULL, st_down ? st_down->acc : NULL);
    free(yg);
    free(yu);
    free(mm);
    return rc;
}

int orc_glu(const float *x, int64_t M, const orc_linear *gate, const orc_linear *up,
            const orc_linear *down, double eps, int act_bf16, double *y, float *m_out) {
    if (!x || !gate || !up || !down || !y || M < 0) return -1;
    if (M == 0) return 0;
    return glu_impl(x, M, gate, up, down, eps, act_bf16, y, m_out, NULL, NULL);
}

/* ---------------------------------------------------------------- O9 block
 * [HL-hgrn] block: RMSNorm -> i/f/g BitLinears -> MLGRU -> g_norm -> o_proj; then the GLU
 * of [DC-core].  Reading R7 (pre-norm residuals).
 * x [B, T, D] fp32 holding values exact in the residual dtype; y [B, T, D] receives y2
 * (rounded to the residual dtype); h0 [B, D] or NULL; h_last [B, D] optional;
 * ifg_out [B, T, 3D] and y1_out [B, T, D] optional.  Stage records (optional): i|f|g
 * (N = 3D), o, gate|up (N = 2F), down.
 */
int orc_block(const float *x, int64_t B, int64_t T, const orc_linear *wi,
              const orc_linear *wf, const orc_linear *wg, const orc_linear *wo,
              const orc_linear *wgate, const orc_linear *wup, const orc_linear *wdown,
              const float *f_bias, const float *f_lower, const float *gnorm_w, double eps,
              int gate_mode, int resid_bf16, const double *h0, double *h_last, double *y,
              double *ifg_out, float *y1_out, orc_stage *st_ifg, orc_stage *st_o,
              orc_stage *st_gu, orc_stage *st_down) {
    if (!x || !wi || !wf || !wg || !wo || !wgate || !wup || !wdown || !y) return -1;
    int64_t D = wi->k, F = wgate->n, M = B * T;
    if (wf->k != D || wg->k != D || wi->n != D || wf->n != D || wg->n != D) return -1;
    if (wo->k != D || wo->n != D || wup->n != F || wgate->k != D || wup->k != D) return -1;
    if (wdown->k != F || wdown->n != D) return -1;
    if (M == 0) return 0;
    double *yi = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *yf = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *yg = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *ifg = (double *)malloc(sizeof(double) * (size_t)(M * 3 * D));
    double *o = (double *)malloc(sizeof(double) * (size_t)(M * D));
    float *o32 = (float *)malloc(sizeof(float) * (size_t)(M * D));
    double *yo = (double *)malloc(sizeof(double) * (size_t)(M * D));
    float *y1 = (float *)malloc(sizeof(float) * (size_t)(M * D));
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *glu = (double *)malloc(sizeof(double) * (size_t)(M * D));
    if (!yi || !yf || !yg || !ifg || !o || !o32 || !yo || !y1 || !tmp || !glu) return -3;

    /* i, f, g projections of x. */
    const orc_linear *proj[3] = {wi, wf, wg};
    double *outs[3] = {yi, yf, yg};
    int rc = group_bitlinear(x, M, 3, proj, eps, outs, st_ifg);
    if (rc) return rc;
    for (int64_t r = 0; r < M; ++r)
        for (int64_t d = 0; d < D; ++d) {
            ifg[r * 3 * D + d] = yi[r * D + d];
            ifg[r * 3 * D + D + d] = yf[r * D + d];
            ifg[r * 3 * D + 2 * D + d] = yg[r * D + d];
        }
    if (resid_bf16)
        for (int64_t i = 0; i < M * 3 * D; ++i) ifg[i] = orc_round_bf16(ifg[i]);
    if (ifg_out) memcpy(ifg_out, ifg, sizeof(double) * (size_t)(M * 3 * D));

    /* MLGRU + output gate, then o_proj with the residual. */
    rc = orc_mlgru(ifg, B, T, D, f_bias, f_lower, h0, gnorm_w, eps, gate_mode, o, h_last);
    if (rc) return rc;
    to_act(o, o32, M * D, resid_bf16);
    if (st_o && st_o->x_in) memcpy(st_o->x_in, o32, sizeof(float) * (size_t)(M * D));
    rc = orc_bitlinear(o32, M, wo, eps, yo, st_o ? st_o->q : NULL, st_o ? st_o->a : NULL,
                       st_o ? st_o->acc : NULL);
    if (rc) return rc;
    for (int64_t i = 0; i < M * D; ++i) tmp[i] = (double)x[i] + yo[i];
    to_act(tmp, y1, M * D, resid_bf16);
    if (y1_out) memcpy(y1_out, y1, sizeof(float) * (size_t)(M * D));

    /* GLU with the residual. */
    rc = glu_impl(y1, M, wgate, wup, wdown, eps, resid_bf16, glu, NULL, st_gu, st_down);
    if (rc) return rc;
    for (int64_t i = 0; i < M * D; ++i) tmp[i] = (double)y1[i] + glu[i];
    for (int64_t i = 0; i < M * D; ++i)
        y[i] = resid_bf16 ? orc_round_bf16(tmp[i]) : (double)(float)tmp[i];

    free(yi); free(yf); free(yg); free(ifg); free(o); free(o32); free(yo); free(y1);
    free(tmp); free(glu);
    return 0;
}

/* ------------------------------------------------- B3 block backward (reading R14)
 * The gradients of orc_block: the forward is rerun with the same roundings (R8), then the
 * chain of B1/B2 and the GLU's elementwise product is walked backwards:
 *   dy1 = dy;  dm = down^T(dy) (B1 on the down input m);
 *   dgate = dm*u*silu'(g), dup = dm*silu(g) (g, u: the gate and up pre-activations);
 *   dy1 += gate^T(dgate) + up^T(dup) (B1 on y1);  do = o^T(dy1) (B1 on the g_norm output);
 *   d_ifg, dh0 = B2(do, dh_last);  dx = dy1 + sum_k k^T(d_ifg_k) for k = i, f, g (B1 on x).
 * dy [B, T, D] and dh_last [B, D] (or NULL) fp64; dx [B, T, D], dh0 [B, D]; per BitLinear
 * (order i, f, g, o, gate, up, down) optional dw [N, K], db [N], dgamma [K]; dgnorm_w,
 * df_bias [D] optional.  fp64.
 */
int orc_block_backward(const float *x, int64_t B, int64_t T, const orc_linear *const *w7,
                       const float *f_bias, const float *f_lower, const float *gnorm_w, double eps,
                       int gate_mode, int resid_bf16, const double *h0, const double *dy,
                       const double *dh_last, double *dx, double *dh0, double *const *dw,
                       double *const *db, double *const *dgamma, double *dgnorm_w,
                       double *df_bias) {
    if (!x || !w7 || !dy || !dx) return -1;
    for (int k = 0; k < 7; ++k)
        if (!w7[k]) return -1;
    const int64_t D = w7[0]->k, F = w7[4]->n, M = B * T;
    if (M == 0) return 0;
    double *ifg = (double *)malloc(sizeof(double) * (size_t)(M * 3 * D));
    double *o = (double *)malloc(sizeof(double) * (size_t)(M * D));
    float *o32 = (float *)malloc(sizeof(float) * (size_t)(M * D));
    double *yo = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(M * D));
    float *y1 = (float *)malloc(sizeof(float) * (size_t)(M * D));
    double *gp = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *up = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *mv = (double *)malloc(sizeof(double) * (size_t)(M * F));
    float *m32 = (float *)malloc(sizeof(float) * (size_t)(M * F));
    double *dm = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *dg = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *du = (double *)malloc(sizeof(double) * (size_t)(M * F));
    double *dy1 = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *dpart = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *dout = (double *)malloc(sizeof(double) * (size_t)(M * D));
    double *d_ifg = (double *)malloc(sizeof(double) * (size_t)(M * 3 * D));
    double *dseg = (double *)malloc(sizeof(double) * (size_t)(M * D));
    if (!ifg || !o || !o32 || !yo || !tmp || !y1 || !gp || !up || !mv || !m32 || !dm || !dg ||
        !du || !dy1 || !dpart || !dout || !d_ifg || !dseg)
        return -3;
    /* forward, as orc_block computes it */
    {
        double *outs[3];
        double *yi = (double *)malloc(sizeof(double) * (size_t)(M * D * 3));
        if (!yi) return -3;
        outs[0] = yi; outs[1] = yi + M * D; outs[2] = yi + 2 * M * D;
        int rc = group_bitlinear(x, M, 3, w7, eps, outs, NULL);
        if (rc) return rc;
        for (int64_t r = 0; r < M; ++r)
            for (int64_t c = 0; c < 3 * D; ++c) {
                const double v = outs[c / D][r * D + c % D];
                ifg[r * 3 * D + c] = resid_bf16 ? orc_round_bf16(v) : v;
            }
        free(yi);
    }
    int rc = orc_mlgru(ifg, B, T, D, f_bias, f_lower, h0, gnorm_w, eps, gate_mode, o, NULL);
    if (rc) return rc;
    to_act(o, o32, D * M, resid_bf16);
    if ((rc = orc_bitlinear(o32, M, w7[3], eps, yo, NULL, NULL, NULL))) return rc;
    for (int64_t i = 0; i < M * D; ++i) tmp[i] = yo[i] + (double)x[i];   /* y1 before rounding */
    to_act(tmp, y1, M * D, resid_bf16);
    {
        double *outs[2] = {gp, up};
        if ((rc = group_bitlinear(y1, M, 2, w7 + 4, eps, outs, NULL))) return rc;
    }
    for (int64_t i = 0; i < M * F; ++i) mv[i] = silu_d(gp[i]) * up[i];
    to_act(mv, m32, M * F, resid_bf16);
    /* backward */
    if ((rc = orc_bitlinear_backward(m32, M, w7[6], eps, dy, dm, dgamma ? dgamma[6] : NULL,
                                     dw ? dw[6] : NULL, db ? db[6] : NULL)))
        return rc;
    for (int64_t i = 0; i < M * F; ++i) {
        const double sg = sigmoid_d(gp[i]);
        dg[i] = dm[i] * up[i] * sg * (1.0 + gp[i] * (1.0 - sg));
        du[i] = dm[i] * gp[i] * sg;
    }
    memcpy(dy1, dy, sizeof(double) * (size_t)(M * D));
    for (int k = 4; k <= 5; ++k) {
        if ((rc = orc_bitlinear_backward(y1, M, w7[k], eps, k == 4 ? dg : du, dpart,
                                         dgamma ? dgamma[k] : NULL, dw ? dw[k] : NULL,
                                         db ? db[k] : NULL)))
            return rc;
        for (int64_t i = 0; i < M * D; ++i) dy1[i] += dpart[i];
    }
    if ((rc = orc_bitlinear_backward(o32, M, w7[3], eps, dy1, dout, dgamma ? dgamma[3] : NULL,
                                     dw ? dw[3] : NULL, db ? db[3] : NULL)))
        return rc;
    if ((rc = orc_mlgru_backward(ifg, B, T, D, f_bias, f_lower, h0, gnorm_w, eps, gate_mode, dout,
                                 dh_last, d_ifg, dh0, dgnorm_w, df_bias)))
        return rc;
    memcpy(dx, dy1, sizeof(double) * (size_t)(M * D));
    for (int k = 0; k < 3; ++k) {
        for (int64_t r = 0; r < M; ++r)
            for (int64_t d = 0; d < D; ++d) dseg[r * D + d] = d_ifg[r * 3 * D + k * D + d];
        if ((rc = orc_bitlinear_backward(x, M, w7[k], eps, dseg, dpart, dgamma ? dgamma[k] : NULL,
                                         dw ? dw[k] : NULL, db ? db[k] : NULL)))
            return rc;
        for (int64_t i = 0; i < M * D; ++i) dx[i] += dpart[i];
    }
    free(ifg); free(o); free(o32); free(yo); free(tmp); free(y1); free(gp); free(up); free(mv);
    free(m32); free(dm); free(dg); free(du); free(dy1); free(dpart); free(dout); free(d_ifg);
    free(dseg);
    return 0;
}

/* ----------------------------------------- HGRN forget-gate lower bounds (R12)
 * G [L, D] per-layer logits -> lb [L, D]: for each channel, a softmax over the L layers
 * (fp64; the largest logit is subtracted first so exp cannot overflow), accumulated over
 * the layers before l.  lb_0 = 0 and lb grows with l, staying below 1.
 */
int orc_hgrn_lower_bounds(const float *G, int64_t L, int64_t D, float *lb) {
    if (!G || !lb || L <= 0 || D <= 0) return -1;
    for (int64_t d = 0; d < D; ++d) {
        double mx = (double)G[d];
        for (int64_t l = 1; l < L; ++l)
            if ((double)G[l * D + d] > mx) mx = (double)G[l * D + d];
        double tot = 0.0;
        for (int64_t l = 0; l < L; ++l) tot += exp((double)G[l * D + d] - mx);
        double acc = 0.0;
        for (int64_t l = 0; l < L; ++l) {
            lb[l * D + d] = (float)(acc / tot);
            acc += exp((double)G[l * D + d] - mx);
        }
    }
    return 0;
}

/* ------------------------------------------------------ ternary embedding gather
 * Embedding rows are ternary like every other weight matrix: x[t] = s_E * q_E[id[t]],
 * rounded to the residual dtype.
 */
int orc_embedding(const int8_t *qe, float scale, int64_t vocab, int64_t D, const int32_t *ids,
                  int64_t M, int resid_bf16, float *x) {
    for (int64_t t = 0; t < M; ++t) {
        if (ids[t] < 0 || ids[t] >= vocab) return -1;
        for (int64_t d = 0; d < D; ++d) {
            double v = (double)qe[(int64_t)ids[t] * D + d] * (double)scale;
            x[t * D + d] = resid_bf16 ? (float)orc_round_bf16(v) : (float)v;
        }
    }
    return 0;
}

/* Vector form of orc_round_bf16 for the test harness. */
void orc_round_bf16_array(const double *src, double *dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = orc_round_bf16(src[i]);
}
