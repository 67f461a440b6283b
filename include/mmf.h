/*
 * mmf.h -- C ABI of libmmf, a gfx950 (MI355X) implementation of the forward pass of one
 * MatMul-free language-model block: ternary BitLinear -> MLGRU token mixer -> GLU.
 *
 * Sources (cited by page title and section):
 *   [DC-ternary] DataCamp blog "MatMul-free language models", section "Replacing MatMul with
 *                ternary operations": BitLinear with weights in {-1,0,1}; absmean
 *                quantization of each weight matrix; products become add/subtract.
 *   [DC-core]    same page, section "Core components: MLGRU and GLU": RMSNorm before
 *                activation quantization; MLGRU hidden state updated token by token through
 *                gates in (0,1); MatMul-free GLU = two BitLinears, SiLU on one branch,
 *                element-wise product, a third BitLinear.
 *   [DC-gpu]     same page, section "From optimised GPU to custom FPGA": fused kernels
 *                avoid memory round trips; token generation is limited by moving weights.
 *   [HL-fbl]     Hysen Labs project page "MatMul-Free LM", section "FusedBitLinear": each
 *                projection RMS-normalises its input, quantizes it and accumulates it against
 *                the ternary weights inside one fused kernel.
 *   [HL-hgrn]    same page, section "HGRN attention": block input -> RMSNorm -> i/f/g
 *                projections -> gated recurrence -> g_norm (RMSNorm fused with a swish gate)
 *                -> o_proj.
 *   [HL-init]    same page, section "Installation and model initialization": the default
 *                configuration has hidden size 2048, a 32000-entry embedding and 24 layers.
 *
 * Arithmetic, shared by every entry point:
 *   - activation quantization of a row x[0..K) with gain gamma: p = fl32(x*gamma),
 *     m = max(max|p|, 1e-5), s = fl32(127/m), q = clamp(rint(fl32(p*s)), -127, 127)
 *     (round half to even), a = m/127 * rsqrt(mean(x^2) + eps).  The RMSNorm factor cancels
 *     in the absmax ratio, so it enters only the dequantization scale a;
 *   - accumulation acc[m][n] = sum_k q_x[m][k] * q_w[n][k] in int32 (exact);
 *   - rescale y = acc * s_w * a[m] (+ bias[n]) in fp32;
 *   - MLGRU: f = sigmoid(f_pre + b_f), c = SiLU(i_pre), h_t = f*h_{t-1} + (1-f)*c (fp32
 *     state); output gate o = RMSNorm_D(h)*gnorm_w * g*sigmoid(g) (MMF_GATE_SWISH_RMSNORM)
 *     or sigmoid(g)*h (MMF_GATE_SIGMOID);
 *   - GLU: SiLU(gate(x)) * up(x), then down;
 *   - block: y1 = x + o_proj(MLGRU(x)); y = y1 + GLU(y1).  Every tensor one module hands
 *     to the next -- the i/f/g projections, the g_norm output, the GLU's gated product, y1
 *     and y -- is materialised in the activation dtype (bf16 or fp32); the state h is fp32.
 *
 * Packed ternary weights: a matrix [N][K] (row n = output feature, K % 64 == 0) is stored
 * as N*K/16 uint32 words, row-major; element k = 16*j + 4*a + b of a row sits in word j at
 * bits 8*b + 2*a .. 8*b + 2*a + 1 as code = q + 1 (0 -> -1, 1 -> 0, 2 -> +1; 3 invalid).
 * One fp32 scale per matrix (absmean is per matrix).
 *
 * Conventions for every entry point below:
 *   - tensor pointers are DEVICE pointers owned by the caller (unless marked host) and must
 *     stay valid until the work queued on the stream has finished;
 *   - the library never allocates or frees device memory inside a forward call; all
 *     scratch comes from the caller's workspace `ws` (size from the *_workspace_bytes call);
 *   - nothing synchronises the stream; work is queued on `stream` (NULL = null stream);
 *   - arguments are validated before anything is queued: on a non-zero return nothing was
 *     queued and mmf_last_error() (thread-local) says why.  Device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI;
 *   - x, y, packed weights and workspaces must be 16-byte aligned;
 *   - every entry point is thread-safe; calls that share a workspace must be ordered.
 */
#ifndef MMF_H
#define MMF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMF_ABI_VERSION 2

/* Status codes. */
#define MMF_OK 0
#define MMF_EINVAL (-1)     /* NULL where required, bad enum, invalid packed code */
#define MMF_ESHAPE (-2)     /* K % 64 != 0, mismatched dims, negative sizes */
#define MMF_EALIGN (-3)     /* a pointer is not 16-byte aligned */
#define MMF_EDTYPE (-4)     /* unsupported dtype */
#define MMF_EWORKSPACE (-5) /* workspace NULL or smaller than required */
#define MMF_EHIP (-6)       /* a HIP call failed (message carries hipGetErrorString) */
#define MMF_EDEVICE (-7)    /* current device is not gfx950 */

typedef enum mmf_dtype { MMF_F32 = 0, MMF_BF16 = 1 } mmf_dtype;

typedef enum mmf_gate_mode {
    MMF_GATE_SWISH_RMSNORM = 0, /* g_norm: RMSNorm_D(h) * gnorm_w * g * sigmoid(g) */
    MMF_GATE_SIGMOID = 1        /* sigmoid(g) * h */
} mmf_gate_mode;

/* One BitLinear ([DC-ternary], [HL-fbl]). */
typedef struct mmf_bitlinear {
    const uint32_t *packed; /* device [N][K/16] packed ternary codes */
    float scale;            /* absmean scale s_w of the matrix */
    const float *norm_w;    /* device [K] RMSNorm gain of the input, or NULL (ones) */
    const float *bias;      /* device [N] or NULL */
    float eps;              /* RMSNorm epsilon of the input (1e-6 if unsure) */
    int32_t K, N;
} mmf_bitlinear;

/* One block ([HL-hgrn], [DC-core]).  i, f, g, o: [D][D]; gate, up: [F][D]; down: [D][F].
 * i, f, g must share norm_w (same pointer or all NULL) and eps, as must gate and up: each
 * group quantizes its shared input once.  f_bias, f_lower, gnorm_w and o.norm_w are read 16
 * bytes at a time and must be 16-byte aligned (MMF_EALIGN).
 * f_lower is HGRN's per-layer lower bound on the forget gate: [HL-hgrn] names the
 * Hierarchical Gated Recurrent Network, and, following HGRN's published design (a reading:
 * the pages give no formula), the gate becomes f = lb + (1 - lb)*sigmoid(f_pre + b_f), with
 * lb in [0, 1] growing with depth (mmf_hgrn_lower_bounds builds it); NULL = no bound. */
typedef struct mmf_block {
    mmf_bitlinear i, f, g, o, gate, up, down;
    const float *f_bias;  /* device [D] forget-gate bias, or NULL (zeros) */
    const float *gnorm_w; /* device [D] g_norm gain, or NULL (ones) */
    float eps;            /* g_norm epsilon */
    int32_t gate_mode;    /* mmf_gate_mode */
    const float *f_lower; /* device [D] forget-gate lower bound, or NULL (none) */
} mmf_block;

/* Optional record of one BitLinear stage for token rows [row0, row1) (device buffers,
 * any may be NULL): the fp32 input exactly as quantized, its int8 codes, its scale a, the
 * int32 accumulators acc = sum_k q_x * q_w, and the stage output exactly as stored for
 * the next kernel, widened to fp32 (i|f|g: the pre-activations; o: y1 = x + o_proj;
 * gate|up: the GLU hidden SiLU(gate)*up; down: the block output).  For a group of
 * projections sharing an input (i|f|g, gate|up) acc has the group's concatenated width
 * (3D or 2F) in that order; y_out has the width of the stored output (3D, D, F, D). */
typedef struct mmf_stage_capture {
    int64_t row0, row1;
    float *x_in;   /* [rows][K] */
    int8_t *q;     /* [rows][K] */
    float *a;      /* [rows] */
    int32_t *acc;  /* [rows][N] */
    float *y_out;  /* [rows][N_out] */
} mmf_stage_capture;

typedef struct mmf_capture {
    mmf_stage_capture ifg, o, gateup, down;
} mmf_capture;

/* ------------------------------------------------------------------ library state */

/* ABI version (MMF_ABI_VERSION). */
int mmf_abi_version(void);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char *mmf_last_error(void);

/* Test knob, process-wide: 0 = choose the BitLinear kernel by token count (default: the
 * weight-streaming dot4 kernel for few rows, the k-split MFMA kernel up to 64 rows, the
 * 128-row MFMA tiles above), 1 = force the weight-streaming kernel, 2 = force the MFMA
 * kernels (k-split up to 64 rows, tiles above), 3 = force the 128-row MFMA tiles.
 * Returns the previous value, or MMF_EINVAL for another value. */
int mmf_set_regime(int regime);

/* Per-kernel launch timing with HIP events recorded on the launch stream around every
 * launch of the named kernel family.  enable: 1 on, 0 off (events are kept).  After the
 * stream has been synchronised, mmf_timing_query returns the number of timed launches and
 * their summed duration in ms for a family name (see mmf_timing_name); reset clears them. */
int mmf_timing_enable(int enable);
/* Restrict timing to the families whose bit (1 << i, i as in mmf_timing_name) is set in
 * mask; the default is every family.  Events cost a few microseconds of queue time each,
 * so timing only the kernel of interest keeps the measured stream close to an untimed one. */
int mmf_timing_families(uint32_t mask);
int mmf_timing_reset(void);
int mmf_timing_query(const char *family, int64_t *launches, double *total_ms);
/* Name of family i (0 <= i < mmf_timing_count()), or NULL. */
const char *mmf_timing_name(int i);
int mmf_timing_count(void);

/* --------------------------------------------------------- host weight preparation */

/* Absmean ternarization [DC-ternary], on HOST memory: s = max(mean|w|, 1e-5) with the mean
 * summed in double per row (k ascending) and over rows (n ascending);
 * q = clamp(rint(w / s), -1, 1) (fp32 division, ties to even).  w [n][k] host fp32,
 * q_out [n][k] host int8, *scale_out host.  MMF_EINVAL on NULL, MMF_ESHAPE on n,k <= 0. */
int mmf_ternary_quantize(const float *w, int64_t n, int64_t k, int8_t *q_out,
                         float *scale_out);

/* Pack q [n][k] in {-1,0,1} (host) into the 2-bit format (host, [n][k/16] words).
 * MMF_ESHAPE unless k % 16 == 0; MMF_EINVAL on a value outside {-1,0,1}. */
int mmf_ternary_pack(const int8_t *q, int64_t n, int64_t k, uint32_t *packed);

/* Unpack (host -> host).  MMF_EINVAL on code 3 anywhere. */
int mmf_ternary_unpack(const uint32_t *packed, int64_t n, int64_t k, int8_t *q);

/* HGRN forget-gate lower bounds of an L-layer stack, on HOST memory (reading of [HL-hgrn],
 * see mmf_block.f_lower): per channel d a softmax of the per-layer logits g[0..L)[d] over
 * the layers, summed over the layers before l: lb[l][d] = sum_{j<l} e^g[j][d] / sum_j
 * e^g[j][d] (sums in double, largest logit subtracted first), so lb[0] = 0 and lb grows
 * with depth.  g, lb: [L][D] fp32.  MMF_EINVAL on NULL, MMF_ESHAPE on L, D <= 0. */
int mmf_hgrn_lower_bounds(const float *g, int64_t L, int64_t D, float *lb);

/* Base-3 packing ("trits", five ternary weights per byte, 1.6 bits each): the HackerPapers
 * page on arXiv 2406.02528 (HN discussion list) calls the weights ternary digits, trits;
 * 3^5 = 243 <= 256.  Format (a reading): codes c = q + 1; byte j of 4-byte word w of a row
 * holds k = 20w + 4i + j (i = 0..4, i = 0 most significant) as v = sum_i c_i 3^(4-i),
 * stored as b = ceil(256 v / 243); rows are padded with q = 0 to 16-byte chunks of 80
 * weights, mmf_trit_row_bytes(k) = 16 * ceil(k / 80) bytes.  Host memory.  Pack: MMF_EINVAL
 * on a value outside {-1,0,1}; unpack: MMF_EINVAL on a byte no group packs to or non-zero
 * padding. */
int64_t mmf_trit_row_bytes(int64_t k);
int mmf_ternary_pack_trits(const int8_t *q, int64_t n, int64_t k, uint8_t *packed);
int mmf_ternary_unpack_trits(const uint8_t *packed, int64_t n, int64_t k, int8_t *q);

/* ------------------------------------------------------------------- forward calls */

/* Scratch bytes bitlinear_forward needs for m token rows of w. */
size_t bitlinear_workspace_bytes(const mmf_bitlinear *w, int64_t m);

/* y[m][N] = BitLinear(x[m][K]) [HL-fbl]: RMSNorm + int8 quantization of each row of x,
 * ternary accumulation, rescale (+ bias).  x dtype x_dt, y dtype y_dt.  m == 0 is a no-op.
 * The regime (weight-streaming decode kernel vs int8-MFMA prefill kernel) is chosen from m.
 * cap (nullable) records the stage for its row window. */
int bitlinear_forward(const mmf_bitlinear *w, const void *x, mmf_dtype x_dt, int64_t m,
                      void *y, mmf_dtype y_dt, void *ws, size_t ws_bytes,
                      const mmf_stage_capture *cap, hipStream_t stream);

/* A BitLinear with base-3 packed weights (see mmf_ternary_pack_trits). */
typedef struct mmf_bitlinear_trits {
    const uint8_t *packed;  /* device [N][mmf_trit_row_bytes(K)], 16-byte aligned */
    float scale;            /* absmean scale s_w of the matrix */
    const float *norm_w;    /* device [K] RMSNorm gain of the input, or NULL (ones) */
    const float *bias;      /* device [N] or NULL */
    float eps;
    int32_t K, N;           /* K % 64 == 0, K <= 10240 */
} mmf_bitlinear_trits;

/* y[m][N] = BitLinear(x[m][K]) [HL-fbl] in the decode regime (0 <= m <= 16 token rows)
 * over base-3 packed weights: the same quantization, exact int32 accumulation and rescale
 * as bitlinear_forward, with 20 % fewer weight bytes streamed.  No workspace.  cap as for
 * bitlinear_forward (acc and y_out rows have stride N). */
int bitlinear_forward_trits(const mmf_bitlinear_trits *w, const void *x, mmf_dtype x_dt,
                            int64_t m, void *y, mmf_dtype y_dt, const mmf_stage_capture *cap,
                            hipStream_t stream);

/* MLGRU token mixer + output gate [DC-core], [HL-hgrn], without the o_proj. */
typedef struct mmf_mlgru_args {
    const void *ifg;       /* device [B][T][3D]: pre-activations i | f | g (ifg_dt) */
    mmf_dtype ifg_dt;
    const float *f_bias;   /* [D] or NULL */
    const float *h0;       /* [B][D] fp32 initial state, or NULL (zeros) */
    float *h_out;          /* [B][D] fp32 final state h_T, or NULL; may equal h0 */
    const float *gnorm_w;  /* [D] or NULL; every pointer 16-byte aligned (MMF_EALIGN) */
    float eps;
    int32_t gate_mode;     /* mmf_gate_mode */
    void *out;             /* [B][T][D] gated output (out_dt) */
    mmf_dtype out_dt;
    int64_t B, T, D;       /* D % 64 == 0, D <= 4096 */
    const float *f_lower;  /* [D] forget-gate lower bound (see mmf_block), or NULL */
} mmf_mlgru_args;

size_t mlgru_workspace_bytes(int64_t B, int64_t T, int64_t D);

/* Chunked scan: parallel over (b, d), chunked over T with a carry pass between chunks. */
int mlgru_scan(const mmf_mlgru_args *args, void *ws, size_t ws_bytes, hipStream_t stream);

/* GLU channel mixer [DC-core]: y = down(SiLU(gate(x)) * up(x)) (+ residual if non-NULL).
 * x, residual, y: [m][D] of dtype dt.  gate, up: [F][D]; down: [D][F]. */
size_t glu_workspace_bytes(const mmf_bitlinear *gate, const mmf_bitlinear *down, int64_t m);
int glu_forward(const mmf_bitlinear *gate, const mmf_bitlinear *up,
                const mmf_bitlinear *down, const void *x, mmf_dtype dt, int64_t m,
                const void *residual, void *y, void *ws, size_t ws_bytes,
                const mmf_capture *cap, hipStream_t stream);

/* One block [HL-hgrn]: x [B][T][D] (dt) -> y [B][T][D] (dt).  h_state: [B][D] fp32 state,
 * 16-byte aligned, read as h_0 and overwritten with h_T (NULL: h_0 = 0, h_T dropped).
 * T == 1 with h_state is one decode step; with B <= 4 too (and D <= 4096) the MLGRU step runs
 * inside the o_proj launch and h_T passes through the workspace before it reaches h_state
 * (written by a later launch of the same call, so h_state holds h_0 until the call's work
 * completes).
 * cap (nullable) records each BitLinear stage.  The workspace holds the quantized rows, the
 * projections, the scan's chunk summaries and (B*T == 1) one D-float state row. */
size_t block_workspace_bytes(const mmf_block *w, int64_t B, int64_t T);
int block_forward(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                  float *h_state, void *y, void *ws, size_t ws_bytes,
                  const mmf_capture *cap, hipStream_t stream);

/* block_forward without a caller workspace and without any device allocation, for callers
 * that cannot allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The scratch is a static device array of block_scratch_bytes() bytes
 * (32 MiB), one per GPU, reserved when the library is loaded onto it and held until the
 * process ends; the call fails with MMF_EWORKSPACE, queueing nothing, when
 * block_workspace_bytes(w, B, T) exceeds it (for example above 850 token rows at hidden
 * 2048 / GLU 5632).  Same arguments and results as block_forward without capture.  Every
 * call on one GPU uses that GPU's scratch: calls that may overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller. */
size_t block_scratch_bytes(void);
int block_forward_noalloc(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                          float *h_state, void *y, hipStream_t stream);

/* Ternary embedding gather of the 32000-entry embedding [HL-init], read as a ternary
 * matrix like every other weight matrix [DC-ternary] (a reading: the pages do not say how
 * the embedding is stored): x[t][:] = s_E * q_E[ids[t]][:], rounded to dt.
 * packed [vocab][D/16]; ids device int32 [m]; an id outside [0, vocab) yields a zero row. */
int embedding_forward(const uint32_t *packed, float scale, int64_t vocab, int64_t D,
                      const int32_t *ids, int64_t m, void *x, mmf_dtype dt,
                      hipStream_t stream);

/* A stack of blocks [HL-hgrn] with optional ternary embedding (ids -> x) and head
 * (x_L -> logits, a BitLinear whose input RMSNorm is the final norm). */
typedef struct mmf_stack {
    const mmf_block *blocks;      /* HOST array of n_layers block descriptors */
    int32_t n_layers;
    const uint32_t *embed_packed; /* device [vocab][D/16] or NULL */
    float embed_scale;
    int64_t vocab;
    const mmf_bitlinear *head;    /* HOST pointer to the head descriptor, or NULL */
} mmf_stack;

size_t stack_workspace_bytes(const mmf_stack *s, int64_t B, int64_t T);

/* ids [B*T] (device int32) when the stack has an embedding, else x [B][T][D] (dt).
 * h_state [n_layers][B][D] fp32 in/out or NULL.  y [B][T][D] (dt) receives x_L (nullable
 * when logits are requested); logits [B*T][vocab] fp32 (nullable; needs a head). */
int stack_forward(const mmf_stack *s, const int32_t *ids, const void *x, mmf_dtype dt,
                  int64_t B, int64_t T, float *h_state, void *y, float *logits, void *ws,
                  size_t ws_bytes, hipStream_t stream);

/* One decode step of a stack for ONE sequence in a single cooperative launch: embedding of
 * ids[0], every block (state h_state [n_layers][D] fp32, read and written), the head
 * (logits [vocab] fp32, nullable) and the last hidden row y [D] (bf16, nullable), with the
 * arithmetic of stack_forward (bf16 activations).  Generating a token is limited by moving
 * the weights ([DC-gpu], section "From optimised GPU to custom FPGA"), and with one token
 * every BitLinear is a short dependent stage: here each workgroup of a co-resident grid
 * streams a slice of every stage's weights and the stages hand their outputs over through
 * the workspace instead of through kernel launches.
 * The workspace (stack_decode_workspace_bytes) belongs to one stack: stack_decode_init
 * writes its layer table and clears it (synchronising the stream; call it once, and again
 * after a timeout); consecutive steps on one workspace must be ordered.  Needs an
 * embedding and a head; limits: D <= 4096, F <= 8192, at most 128 rows of a stage per
 * workgroup (one workgroup per CU), else MMF_ESHAPE (use stack_forward).  Every wait of
 * the kernel is bounded (0.2 s); a timeout ends the kernel and is reported by
 * stack_decode_status, which synchronises the stream.  Workspace layout (for inspection):
 * bytes [0, 12) hold the epoch, a counter and the timeout flag (uint32 each); bytes
 * [256, 256 + 16 * (4 * n_layers + 2)) hold 100 MHz stamps (uint64 pairs) taken by workgroup
 * 0 in the last step: the kernel's start (twice), then for every layer the start and end
 * of its waits for the layer input (zero for layer 0), i|f|g, y1 and the GLU hidden, then
 * the head's wait, then the end of its work (and a zero); the last
 * align_up((n_layers + 1) * S * 8, 256) bytes, S = 5*D/2 + F/2, are the exchange words of
 * the last step: word l*S + j (1 <= l <= n_layers, j < D/2) holds layer l's input elements
 * 2j, 2j+1 as bf16 in its low 32 bits (layer n_layers: the head's input). */
size_t stack_decode_workspace_bytes(const mmf_stack *s);
int stack_decode_init(const mmf_stack *s, void *ws, size_t ws_bytes, hipStream_t stream);
int stack_decode_step(const mmf_stack *s, const int32_t *ids, float *h_state, float *logits,
                      void *y, void *ws, size_t ws_bytes, hipStream_t stream);
int stack_decode_status(const void *ws, hipStream_t stream);

/* ------------------------------------------------------------------ backward
 * Gradients for training the latent weights.  DataCamp "MatMul-free language models",
 * section "Replacing MatMul with ternary operations": the weights are trained in full
 * precision and ternarized during training; section "From optimised GPU to custom FPGA":
 * fused training kernels.  The pages do not say how a gradient crosses the quantizers; here
 * it passes straight through both: the activation quantizer's dequantized output q*a stands
 * for u = x*gamma*r (r = (mean x^2 + eps)^(-1/2)) and W_hat = s_w*T for the latent weights.
 *
 * bitlinear_backward: x [m][K] (x_dt, the forward input), dy [m][N] (dy_dt, gradient at the
 * BitLinear output).  Outputs (fp32, each may be NULL):
 *   dx [m][K]     = r*gamma*g - x*r^3/K * sum_K(g*gamma*x),  g = s_w * dy T
 *   dgamma [K]    = sum_m g*x*r       (gradient of w->norm_w; ones when it is NULL)
 *   dw [N][K]     = sum_m dy[m][n] * q[m][k] * a[m]   (latent weights)
 *   db [N]        = sum_m dy
 * g and dw run on bf16 matrix cores with fp32 accumulation: dy is rounded to bf16 (exact
 * for bf16 dy) and, for dw, the product dy*a is.  dgamma, dw and db are summed with fp32
 * atomics (the order of the sum varies between runs).  Needs N % 8 == 0, K <= 8192, every
 * pointer 16-byte aligned.  Workspace: bitlinear_backward_workspace_bytes (q, a, g, a bf16
 * copy of the ternary matrix transposed, bf16 transposes of dy*a and q, and per-workgroup
 * partial sums of dgamma; about m*(7K + 2N) + 2KN + 3072K bytes). */
size_t bitlinear_backward_workspace_bytes(const mmf_bitlinear *w, int64_t m);
int bitlinear_backward(const mmf_bitlinear *w, const void *x, mmf_dtype x_dt, int64_t m,
                       const void *dy, mmf_dtype dy_dt, float *dx, float *dgamma, float *dw,
                       float *db, void *ws, size_t ws_bytes, hipStream_t stream);

/* mlgru_backward: the forward's arguments (args->out, h_out, out_dt unused), dout [B][T][D]
 * (dout_dt, gradient at the gated output), dh_last [B][D] fp32 (gradient at h_T) or NULL.
 * Outputs (fp32): d_ifg [B][T][3D] gradients of the i | f | g pre-activations; dh0 [B][D],
 * dgnorm_w [D] (zero in gate mode MMF_GATE_SIGMOID), df_bias [D], each may be NULL:
 *   gate 0: dg = dout*n*w*silu'(g), dh = rho*dn - h*rho^3/D*sum_D(dn*h), dn = dout*w*silu(g),
 *           n = h*rho; gate 1: dg = dout*h*sigmoid'(g), dh = dout*sigmoid(g);
 *   G_t = dh_t + f_{t+1} G_{t+1} (+ dh_last at the last token), di = (1-f_t) G_t silu'(i),
 *   df_pre = (h_{t-1} - c_t) G_t (1-lb) sigmoid'(f_pre + b_f), dh0 = f_0 G_0.
 * fp32 throughout; dgnorm_w and df_bias are summed over 16-token chunks with fp32 atomics.
 * Same shape limits as mlgru_scan.  Workspace: mlgru_backward_workspace_bytes. */
size_t mlgru_backward_workspace_bytes(int64_t B, int64_t T, int64_t D);
int mlgru_backward(const mmf_mlgru_args *args, const void *dout, mmf_dtype dout_dt,
                   const float *dh_last, float *d_ifg, float *dh0, float *dgnorm_w,
                   float *df_bias, void *ws, size_t ws_bytes, hipStream_t stream);

/* block_backward: every gradient of block_forward (same arguments: x [B][T][D] of dtype dt,
 * h0 the initial state or NULL), given dy [B][T][D] (dy_dt, gradient at the block output)
 * and dh_last [B][D] fp32 (gradient at the final state) or NULL.  The forward is recomputed
 * (prefill kernels; the gate|up GEMM also keeps the gate and up pre-activations in bf16),
 * then: down's BitLinear
 * backward gives dm; the GLU product gives dgate = dm*up*silu'(gate), dup = dm*SiLU(gate);
 * gate and up share one contraction for the input gradient (dy1 = dy + gate^T dgate +
 * up^T dup), o_proj gives the gradient at the g_norm output, the MLGRU backward d_ifg, dh0,
 * dgnorm_w, df_bias, and i, f, g one contraction for dx = dy1 + sum_k k^T d_k.  Outputs fp32:
 * dx [B][T][D], dh0 [B][D] or NULL, and the parameter gradients in grads (any pointer NULL =
 * not wanted; grads itself may be NULL): dw[k] [N][K] and db[k] [N] per BitLinear (order i, f,
 * g, o, gate, up, down), dgamma[0..3] [K] for the norm gains of x (i|f|g), the g_norm output
 * (o), y1 (gate|up) and m (down), dgnorm_w [D], df_bias [D].  Needs F % 8 == 0 and F <= 8192;
 * same block limits as block_forward.  Gradients that feed a contraction pass between the
 * stages in bf16 (dgate|dup, dy1's copy, d_ifg), those added as residuals in fp32; every
 * accumulated output (dw, db, dgamma) is zeroed by the call and summed with fp32 atomics
 * (the order of the sums varies between runs).  Workspace: block_backward_workspace_bytes
 * (the recomputed activations, the gradients between the stages, bf16 operand copies). */
typedef struct mmf_block_grads {
    float *dw[7];
    float *db[7];
    float *dgamma[4];
    float *dgnorm_w;
    float *df_bias;
} mmf_block_grads;
size_t block_backward_workspace_bytes(const mmf_block *w, int64_t B, int64_t T);
int block_backward(const mmf_block *w, const void *x, mmf_dtype dt, int64_t B, int64_t T,
                   const float *h0, const void *dy, mmf_dtype dy_dt, const float *dh_last, float *dx,
                   float *dh0, const mmf_block_grads *grads, void *ws, size_t ws_bytes,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MMF_H */
