/*
 * dflash.h -- C ABI of libdflash.so, the MI355X (gfx950) hot path of the DFlash
 * KV-injection block drafter: context projection, per-layer context K/V,
 * drafter layers, LM-head argmax and greedy block verification.
 *
 * The method (page "@mlx-bun/inference 0.0.0-stage -> 1.0.0", dflash.ts, the
 * header comment on Eq 2 and Eq 3):
 *   Eq 2  H_ctx = RMSNorm(W_c [H^l1; ...; H^lm])  over every context row.
 *   Eq 3  draft layer i: K_i = [W_K n_ctx ; W_K n_d], V_i = [W_V n_ctx ; W_V n_d],
 *         Q_i = W_Q n_d, with n_ctx, n_d the layer's attn_norm of H_ctx and H_d;
 *         the gamma block rows attend bidirectionally over [context ++ block].
 *   Greedy verify (page "Inco Hacks Native: DFlash 2 Speculation", section 3):
 *         accepted = longest draft prefix equal to the target argmax,
 *         committed = accepted + 1.
 *
 * Conventions for every call below
 *   - All tensor pointers are DEVICE pointers unless a comment says "host".
 *   - Matrices are row-major [out, in]: the reduction axis is contiguous.
 *     A product is y[m, n] = sum_k x[m, k] * W[n, k].
 *   - Weight formats (dflash_weight.dtype):
 *       DFLASH_F32      float  [rows, cols]
 *       DFLASH_BF16     bfloat16 bits (uint16) [rows, cols]
 *       DFLASH_INT4G64  codes: uint32 [rows, cols/8], 8 codes per word, low
 *                       nibble = lowest column; scales, biases: bfloat16
 *                       [rows, cols/64]; w[n, k] = scale[n, k/64] * q + bias[n, k/64].
 *     Norm gains, mask_emb and block_pos are float for DFLASH_F32 models and
 *     bfloat16 otherwise. Weight data and norm gains are read as 16-byte
 *     vectors: they must be 16-byte aligned, else the call is DECLINED.
 *   - Rounding contract (bf16 and int4 models; f32 models never round):
 *     accumulation is fp32; the input of every weight product is rounded to
 *     bf16 (nearest-even), as are the Q/K/V projections, the attention output,
 *     the gated-FFN product, the out-projection result Y and the K/V cache.
 *     The residual stream H_d and H_ctx stay fp32; logits stay fp32 and are
 *     never materialised.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream), performs no host synchronisation and allocates nothing. The
 *     caller owns every buffer (weights, KV cache, workspace, outputs) and
 *     keeps it alive until the stream has passed the call. The library keeps
 *     no pointer after return and holds no per-model state; calls are
 *     thread-safe. Calls that share a workspace must be ordered on one stream.
 *   - Return value: DFLASH_OK, or
 *       DFLASH_DECLINED  a valid request this library will not serve (no
 *                        gfx950 device, unsupported head dim / dtype / shape,
 *                        or the kill switch DFLASH_DISABLE=1 in the
 *                        environment). Nothing is enqueued or written; the
 *                        caller falls back to plain decoding. (An acceleration
 *                        path may decline a request but must never fail one:
 *                        page "A Refusal Is Not A Failure", section "The rule
 *                        it earned".)
 *       DFLASH_EINVAL    null pointer, inconsistent dims or sizes.
 *       DFLASH_ENOSPC    workspace or KV capacity too small.
 *       DFLASH_EHIP      a kernel launch failed; the stream state is undefined.
 *     Validation happens on the host before anything is enqueued.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_OK        0
#define DFLASH_DECLINED  1
#define DFLASH_EINVAL   (-1)
#define DFLASH_ENOSPC   (-2)
#define DFLASH_EHIP     (-3)

enum { DFLASH_F32 = 0, DFLASH_BF16 = 1, DFLASH_INT4G64 = 2 };
enum { DFLASH_ACT_GELU_TANH = 0, DFLASH_ACT_SILU = 1 };

/* Drafter geometry. d must equal hq*hd and hq must be a multiple of hkv
 * (query head h reads key/value head h / (hq/hkv)). hd is 64 or 128; d is at
 * most 8192 (wider drafters are DECLINED).
 * gamma = block query rows = drafted tokens (the verify width is gamma+1); at
 * most 32 (the block's keys form one 32-key attention unit), and
 * (hq/hkv)*gamma query rows per kv head at most 48 (40 for f32 models): larger
 * blocks are DECLINED.
 *
 * The DFlash2 variant (page "Inco Hacks Native: DFlash 2 Speculation",
 * section 1: a sliding-window drafter) adds two fields; zero in both gives the
 * plain drafter. The pages fix neither, so both are parameters:
 *   window      attend to the last `window` context keys of each sequence
 *               (the block's own keys always); 0 = the whole context.
 *   rope_theta  rotary positions on Q and K: dims i and i + hd/2 of a head
 *               turn by the angle position * rope_theta^(-2i/hd); context row
 *               t sits at position t, block row k at position len + k (len =
 *               the sequence's context length when the block is drafted).
 *               Context keys are turned when appended; 0 = no rotation. */
typedef struct {
    int32_t H;       /* target hidden size (tap width and LM-head width)   */
    int32_t m;       /* number of tapped target layers                      */
    int32_t d;       /* drafter width                                        */
    int32_t nl;      /* drafter layers                                       */
    int32_t hq;      /* query heads                                          */
    int32_t hkv;     /* key/value heads                                      */
    int32_t hd;      /* head dim                                             */
    int32_t F;       /* FFN inner width                                      */
    int32_t V;       /* vocabulary                                           */
    int32_t gamma;   /* block rows                                           */
    float   eps;     /* RMSNorm epsilon                                      */
    int32_t act;     /* DFLASH_ACT_*: activation of the gate branch          */
    int32_t wdtype;  /* DFLASH_F32 / DFLASH_BF16 / DFLASH_INT4G64            */
    int32_t window;  /* context keys attended, counted from the end; 0 = all */
    float   rope_theta; /* rotary base; 0 = no rotary positions              */
} dflash_dims;

typedef struct {
    int32_t     dtype;   /* DFLASH_F32 / DFLASH_BF16 / DFLASH_INT4G64 */
    int32_t     rows;    /* outputs N                                  */
    int32_t     cols;    /* reduction K                                */
    const void* data;    /* see the weight formats above               */
    const void* scales;  /* int4 only, else NULL                       */
    const void* biases;  /* int4 only, else NULL                       */
} dflash_weight;

/* One drafter layer (page 3, #layer). */
typedef struct {
    const void*   attn_norm;  /* [d]                                              */
    dflash_weight w_qkv;      /* [(hq + 2 hkv) hd, d]: Q rows, then K rows, then V */
    dflash_weight w_o;        /* [d, hq hd]                                       */
    const void*   ffn_norm;   /* [d]                                              */
    dflash_weight w_gate_up;  /* [2F, d]: gate rows (activated) then up rows      */
    dflash_weight w_down;     /* [d, F]                                           */
} dflash_layer;

/* The drafter plus the two tables it borrows from the target (it has no
 * embedding or head of its own: page "A Refusal Is Not A Failure"). */
typedef struct {
    dflash_dims          dims;
    dflash_weight        w_c;        /* [d, m H]  Eq 2 projection                 */
    const void*          ctx_norm;   /* [d]                                       */
    dflash_weight        tok_proj;   /* [d, H]    anchor embedding -> width d     */
    const void*          mask_emb;   /* [gamma-1, d]                              */
    const void*          block_pos;  /* [gamma, d]                                */
    const void*          out_norm;   /* [d]                                       */
    dflash_weight        out_proj;   /* [H, d]                                    */
    dflash_weight        embed_in;   /* [V, H]    target input embedding          */
    dflash_weight        lm_head;    /* [V, H]    target LM head                  */
    const dflash_layer*  layers;     /* HOST array of nl layers                   */
} dflash_model;

/* Retained per-layer context K/V of B sequences, element type `dtype`
 * (DFLASH_F32 for f32 models, DFLASH_BF16 otherwise):
 *   k: [nl][B][hkv][cap][hd]         (row-major keys)
 *   v: [nl][B][hkv][cap/32][hd][32]  (DFLASH_BF16: values in 32-key chunks,
 *                                     head-dim major inside a chunk, so the
 *                                     attention's value operand is 8
 *                                     consecutive keys of one dim and a chunk's
 *                                     values are one contiguous run)
 *      [nl][B][hkv][hd][cap]         (DFLASH_F32: head-dim major)
 * cap must be a multiple of 32 for DFLASH_BF16 caches.
 * len: device int32 [B], rows held per sequence. */
typedef struct {
    void*    k;
    void*    v;
    int32_t* len;
    int32_t  B;
    int32_t  cap;
    int32_t  dtype;
} dflash_kv;

/* Workspace bytes needed by any call below for up to B sequences and a
 * context capacity of cap rows (the per-call requirement never exceeds it).
 * Returns 0 for invalid dims. */
size_t dflash_workspace_bytes(const dflash_dims* dims, int32_t B, int32_t cap);

/* DFLASH_OK if this library would serve models of these dims on the current
 * device, DFLASH_DECLINED if not, DFLASH_EINVAL if the dims are inconsistent. */
int dflash_query(const dflash_dims* dims);

/* Static description of a status code. */
const char* dflash_status_string(int status);

/* Number of successful enqueues since load (all calls together): evidence
 * that the accelerated path really ran. */
uint64_t dflash_invocations(void);

/* Instrumentation: launch tracing. Between dflash_trace_begin and
 * dflash_trace_end, every launch of the chosen kinds (a bit mask) makes each of
 * its workgroups write the device wall clock at its start and end into the
 * stamp buffer: launch j takes entries [offset_j, offset_j + 2 W_j) of
 * `stamps` (device memory of `capacity` uint64 entries), workgroup w writing
 * its start to entry offset_j + 2w and its end to offset_j + 2w + 1, in ticks
 * of dflash_wall_clock_hz(); the launch's duration is max(end) - min(start).
 * The stamp pointer is a kernel argument, so launches captured into a graph
 * while tracing is on rewrite their entries on every replay. Launches beyond
 * the capacity are not traced. Process-wide setting: concurrent calls share
 * the buffer. Tracing changes no result. */
enum { DFLASH_TRACE_LM_HEAD = 1,      /* LM-head argmax projections                 */
       DFLASH_TRACE_ATTENTION = 2,    /* block attention (not the partial merge)    */
       DFLASH_TRACE_PROJECTIONS = 4   /* every other projection launch: context
                                         projection, K/V append, block init, layer
                                         and out projections                        */ };
typedef struct {
    char    kernel[64];      /* kernel name with its template arguments, e.g.
                                "skinny_kernel<7, 5>"                              */
    int32_t kind;            /* one DFLASH_TRACE_* bit                              */
    int32_t workgroups;      /* W: stamp pairs the launch writes                    */
    int64_t offset;          /* first stamp entry of the launch                     */
    double  bytes;           /* algorithmic HBM bytes known on the host: weights,
                                activation rows and outputs (attention: Q, the
                                block's keys and values, and O)                    */
    double  ctx_row_bytes;   /* attention: bytes per held context row (keys and
                                values), which the caller multiplies by the held
                                row count (it lives on the device); else 0          */
} dflash_trace_record;

/* Start tracing the launches of `kinds` into `stamps`; NULL or capacity 0 switches tracing off. */
void dflash_trace_begin(int32_t kinds, uint64_t* stamps, int64_t capacity);
/* Stop tracing; copy the records of the traced launches (in enqueue order, at
 * most `capacity` of them) to `records` (host memory) and return how many
 * launches were traced. */
int32_t dflash_trace_end(dflash_trace_record* records, int32_t capacity);

/* Launch shape of the LM-head argmax over M rows of activations in y_dtype
 * (DFLASH_F32 / DFLASH_BF16) against a V x H head of weight format dtype
 * (DFLASH_F32 / DFLASH_BF16 / DFLASH_INT4G64): returns the workgroups per
 * launch and stores the number of launches in *launches (GEMV launches of up to
 * 8 rows, or, for a bf16 head with bf16 rows, 16 or more of them and H a
 * multiple of 128, matrix-core launches of up to 128 rows). 0 for invalid
 * arguments (launches may be NULL). */
int32_t dflash_lm_head_workgroups(int32_t V, int32_t H, int32_t dtype, int32_t M, int32_t y_dtype, int32_t* launches);

/* Tick rate of the wall clock the stamps use, for the current device, in Hz:
 * measured on the first call per device (two readings of the device clock
 * about 100 ms apart on the host's steady clock; the call allocates 16 bytes
 * of device memory for it, synchronises the device and sleeps), then cached;
 * 0 on failure. Not to be called while a stream is being captured. */
double dflash_wall_clock_hz(void);
/* The rate the runtime reports for that clock (hipDeviceAttributeWallClockRate),
 * in Hz, 0 when it reports none; for comparison with the measured rate. */
double dflash_wall_clock_hz_reported(void);

/* Eq 2 (page 3, #buildContext): h_ctx[r] = RMSNorm(sum_j T_j[r] W_c[:, jH:(j+1)H]^T; ctx_norm).
 *   taps:   HOST array of m device pointers; tap j is [n, H] with row stride
 *           tap_ld elements, float for f32 models, bfloat16 otherwise.
 *   n:      rows (>= 0; 0 enqueues nothing).
 *   h_ctx:  float [n, d] output.
 * Workspace: optional; a workspace of dflash_workspace_bytes(dims, B, cap)
 * bytes with B*(gamma+1) >= n serves every use below, and ws may be NULL.
 * For n <= 8 rows with a workspace the long reduction is split across more
 * workgroups (partial sums in ws, added in a fixed order). For bf16 models
 * with 16 <= n <= 128 rows (a round's rows), H a multiple of 128 and a
 * 16-byte aligned workspace, the projection runs on matrix cores with
 * split-K partial sums in ws. Otherwise, from 64 rows on, bf16 models run it
 * as a matrix-core GEMM (prefill; no workspace needed), and as GEMVs below. */
int dflash_context_project(const dflash_model* M, const void* const* taps, int64_t tap_ld, int32_t n,
                           float* h_ctx, void* ws, size_t ws_bytes, void* stream);

/* Eq 3, context half (page 3, projectContextRows): for every layer i and
 * every appended row, K = bf16(bf16(RMSNorm(h_ctx; attn_norm_i)) W_K_i^T) and
 * V likewise, written to kv at rows len[b], len[b]+1, ...; then
 * len[b] += appended rows.
 *   h_ctx:       float [n, d]; rows of sequence b are row_offsets[b] ..
 *                row_offsets[b+1]-1 (device int32 [B+1], non-decreasing).
 *   counts:      device int32 [B] or NULL. If given, only the first
 *                min(counts[b], rows of b) rows of b are appended (the verified
 *                rows of a round); NULL appends all rows.
 *   Rows that would pass cap are not written and len[b] stops at cap (the
 *   caller sizes cap; see dflash_workspace_bytes).
 * Workspace: optional (ws may be NULL; dflash_workspace_bytes(dims, B, cap)
 * serves every use below). For bf16 models, d a multiple of 128 and a
 * 16-byte aligned workspace: 16 <= n <= 128 rows (a round's rows) run on
 * matrix cores, all layers in one launch (each layer's normalised rows and
 * split-K partial sums in ws, B*(gamma+1) >= n); n >= 64 rows otherwise run
 * as one matrix-core GEMM over all layers (per-row RMS factors in ws, at
 * least 4n bytes; B*cap rows always fit). With a workspace of at least
 * dflash_kv_prefill_workspace_bytes(dims, n) bytes and h_ctx 16-byte aligned,
 * that GEMM first writes every layer's bf16 normalised rows into ws and then
 * reads them as plain bf16 tiles (the same values, fewer bytes per tile).
 * Everything else runs as GEMVs. */
int dflash_ctx_kv_append(const dflash_model* M, const float* h_ctx, int32_t n, const int32_t* row_offsets,
                         const int32_t* counts, const dflash_kv* kv, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes with which dflash_ctx_kv_append of n >= 64 rows stages
 * every layer's normalised rows as bf16 before its matrix-core GEMM
 * (layers * n * d * 2, rounded up to 256); 0 for invalid dims or n <= 0. */
size_t dflash_kv_prefill_workspace_bytes(const dflash_dims* dims, int32_t n);

/* Workspace bytes with which, for an int4-g64 model (Eq 2 and the context
 * half of Eq 3 on a prompt's rows: page 3, #buildContext and
 * projectContextRows), dflash_context_project and dflash_ctx_kv_append of
 * n >= 64 rows run on matrix cores (ws and h_ctx 16-byte aligned): the call
 * first expands its int4 weights in ws into bf16 high and low parts
 * (w = scale * q + bias formed in fp32; high = bf16(w), low = bf16(w - high),
 * which together hold w to about 16 bits), [N, 2K] per matrix, then runs one
 * bf16 GEMM of [A | A] against [W_high | W_low]: W_c [d, m*H] for the
 * projection (d * 2*m*H * 2 bytes), every layer's K and V rows [2*hkv*hd, d]
 * plus 4n bytes of row RMS factors for the append. Returns the larger of the
 * two (256-byte rounded); 0 for dims that are invalid or not int4, n < 64, or
 * widths that are not multiples of 64. With a smaller workspace the int4
 * calls run on the GEMV paths. */
size_t dflash_int4_prefill_workspace_bytes(const dflash_dims* dims, int32_t n);

/* One drafter layer on the block (page 3, #layer, Eq 3), in place:
 *   n = RMSNorm(H; attn_norm), Q/K_b/V_b = n W^T,
 *   O = softmax(hd^-1/2 Q [K_ctx[0:len[b]] ; K_b]^T) [V_ctx ; V_b]  (no mask),
 *   H += O W_o^T, n2 = RMSNorm(H; ffn_norm), H += (act(n2 W_gate^T) * n2 W_up^T) W_down^T.
 *   h_block: float [B, gamma, d], read and written.
 *   kv:      read only (never written by this call).
 * Workspace: dflash_workspace_bytes(dims, B, kv->cap). */
int dflash_draft_layer(const dflash_model* M, int32_t layer, float* h_block, const dflash_kv* kv, int32_t B,
                       void* ws, size_t ws_bytes, void* stream);

/* Block init + every layer + out projection + LM-head argmax (page 3,
 * forwardRows with a retained context, greedy; #buildBlock, #backbone,
 * #baseLogits):
 *   H_d[b, 0] = E_in[anchor[b]] tok_proj^T + block_pos[0],
 *   H_d[b, k] = mask_emb[k-1] + block_pos[k]   (k >= 1),
 *   ... layers ..., Y = bf16(bf16(RMSNorm(H_d; out_norm)) out_proj^T),
 *   draft_ids[b, k] = argmax_v Y[b, k] . lm_head[v]  (lowest index on ties).
 *   anchor_ids: device int32 [B], each in [0, V).
 *   draft_ids:  device int32 [B, gamma] output.
 *   y_out:      optional [B, gamma, H] output (float for f32 models, bfloat16
 *               otherwise); NULL to skip.
 *   max_logit:  optional float [B, gamma] output (the winning logit); NULL to skip.
 * Workspace: dflash_workspace_bytes(dims, B, kv->cap). */
int dflash_draft_forward(const dflash_model* M, const int32_t* anchor_ids, const dflash_kv* kv, int32_t B,
                         int32_t* draft_ids, void* y_out, float* max_logit, void* ws, size_t ws_bytes,
                         void* stream);

/* The DSpark heads (page 3, #markov and #confidence; initialised there with
 * markov.w2 = 0 and conf.w = 0): bf16 for bf16 and int4 models, float for f32
 * models.
 *   w1:     [V, r]  markov.w1, the sequential head's token table
 *   w2t:    [V, r]  markov.w2 (the page's [r, V] matrix) transposed: row v holds
 *           column v, so the Markov bias of token v is e1 . w2t[v]
 *   conf_w: [d + r] conf.w over [block row; e1];  conf_b: [1] conf.b
 * r must be a multiple of 8 and w1, w2t 16-byte aligned, else DECLINED. */
typedef struct {
    int32_t     r;
    const void* w1;
    const void* w2t;
    const void* conf_w;
    const void* conf_b;
} dflash_dspark_head;

/* Workspace bytes of dflash_draft_forward_dspark for up to B sequences and a
 * context capacity of cap rows (0 for invalid arguments). */
size_t dflash_dspark_workspace_bytes(const dflash_dims* dims, int32_t r, int32_t B, int32_t cap);

/* Greedy drafting with the DSpark sequential (Markov) head and confidence
 * head, and confidence-scheduled draft-length pruning (page 3: forwardRows with
 * #markov and #confidence; DflashDraftOpts.thresholds / minConf, Alg 1):
 *   block = RMSNorm(H_d; out_norm) after every layer (#backbone), Y as in
 *   dflash_draft_forward, base = Y . lm_head^T (fp32, #baseLogits); then for
 *   k = 0 .. gamma-1, previous = the anchor (k = 0) or draft k-1:
 *     e1 = w1[previous]
 *     draft_ids[b, k] = argmax_v base[b, k, v] + e1 . w2t[v]  (lowest index on ties)
 *     conf[b, k] = sigmoid([block[b, k]; e1] . conf_w + conf_b)
 *   lengths[b] = the first k >= 1 with conf[b, k] < thresholds[k] (min_conf
 *   when thresholds is NULL), else gamma: the row's draft is cut there and
 *   position 0 is always kept. Every step runs for every row (no host
 *   synchronisation); positions at or past lengths[b] are not proposed.
 *   min_conf <= 0 with thresholds NULL never cuts (a confidence is positive).
 *   thresholds: device float [gamma] or NULL.  conf: device float [B, gamma]
 *   or NULL.  lengths: device int32 [B] or NULL.  y_out: as in
 *   dflash_draft_forward.  Other arguments as in dflash_draft_forward; EINVAL
 *   for a NULL head pointer or min_conf NaN.
 * Workspace: dflash_dspark_workspace_bytes(dims, r, B, kv->cap). */
int dflash_draft_forward_dspark(const dflash_model* M, const dflash_dspark_head* head, const int32_t* anchor_ids,
                                const dflash_kv* kv, int32_t B, const float* thresholds, float min_conf,
                                int32_t* draft_ids, float* conf, int32_t* lengths, void* y_out, void* ws,
                                size_t ws_bytes, void* stream);

/* One drafting round in one call (page 3, forwardRows with a retained
 * context: the new rows projected by Eq 2, their per-layer K/V appended, then
 * the block drafted; projectContextRows notes that the context half is
 * independent of the block and can be retained): the same results as
 *   dflash_context_project(taps, n) -> h_ctx;
 *   dflash_ctx_kv_append(h_ctx, row_offsets, counts);
 *   dflash_draft_forward(anchor_ids)
 * with these arguments. Where a layer's block rows and the new context rows fit
 * one projection pass (the GEMV path: bf16 or f32 weights, d <= 2048 and
 * B*gamma + n <= 16 rows), the context rows' K/V come out of that layer's own
 * Q|K|V pass, so each layer's K/V weights are read once per round; otherwise
 * the calls run one after the other.
 *   taps, tap_ld, n:        as in dflash_context_project (n <= B*(gamma+1)).
 *   row_offsets, counts:    as in dflash_ctx_kv_append.
 *   the rest:               as in dflash_draft_forward.
 * Workspace: dflash_round_workspace_bytes(dims, B, kv->cap). */
int dflash_draft_round(const dflash_model* M, const void* const* taps, int64_t tap_ld, int32_t n,
                       const int32_t* row_offsets, const int32_t* counts, const dflash_kv* kv, int32_t B,
                       const int32_t* anchor_ids, int32_t* draft_ids, void* y_out, float* max_logit, void* ws,
                       size_t ws_bytes, void* stream);
size_t dflash_round_workspace_bytes(const dflash_dims* dims, int32_t B, int32_t cap);

/* Greedy ids under a borrowed LM head (page 3, #baseLogits and the argmax
 * step of forwardRows): ids[r] = argmax_v y[r] . E_out[v], lowest index on
 * ties; logits are fp32 accumulations and are never materialised.
 *   E_out: HOST pointer to the weight descriptor, [V, H].
 *   y:     [M, H], element type y_dtype (DFLASH_F32 or DFLASH_BF16); rounded
 *          to bf16 before the product unless E_out is f32.
 *   ids:   device int32 [M];  max_logit: optional float [M].
 * Workspace: at least dflash_lm_head_workspace_bytes(E_out->rows, M); with
 * dflash_lm_head_workspace_bytes_for(E_out, y_dtype, M) bytes (more where the
 * head has a matrix-core path: int4-g64 heads over at most 16 bf16 rows, whose
 * split partial logits then live in the workspace) the fastest path runs. The
 * ids are the same either way (the argmax of the same products); the head
 * sums them in another order, so max_logit may differ in the last bits. */
int dflash_lm_head_argmax(const dflash_weight* E_out, const void* y, int32_t y_dtype, int32_t M, int32_t* ids,
                          float* max_logit, void* ws, size_t ws_bytes, void* stream);
size_t dflash_lm_head_workspace_bytes(int32_t V, int32_t M);
size_t dflash_lm_head_workspace_bytes_for(const dflash_weight* E_out, int32_t y_dtype, int32_t M);

/* Greedy block verification (page "Inco Hacks Native: DFlash 2
 * Speculation", sections 1 and 3: block = 1 verify + gamma proposals;
 * e.g. accepted=7 committed=8, accepted=5 committed=6 at block 8):
 *   t[b, j] = argmax_v target_logits[b, j, v]  (j = 0..gamma, lowest index on ties)
 *   accepted[b] = largest a <= gamma with draft_ids[b, k] == t[b, k] for all k < a
 *   committed[b] = accepted[b] + 1
 *   ids[b, j] = t[b, j] for j <= accepted[b], else -1
 *   next_anchor[b] = t[b, accepted[b]]  (optional; NULL to skip)
 *   target_logits: float [B, gamma+1, V]; draft_ids: int32 [B, gamma].
 * Workspace: at least dflash_verify_workspace_bytes(B, gamma, V). */
int dflash_verify_greedy(const float* target_logits, const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V,
                         int32_t* accepted, int32_t* committed, int32_t* ids, int32_t* next_anchor, void* ws,
                         size_t ws_bytes, void* stream);
size_t dflash_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V);

/* dflash_verify_greedy for a pruned block (page 3, Alg 1: sequence b proposes
 * only its first lengths[b] drafts): accepted[b] = largest a <= lengths[b]
 * with draft_ids[b, k] == t[b, k] for all k < a; committed, ids and
 * next_anchor follow from it as in dflash_verify_greedy.
 *   lengths: device int32 [B], each clamped to [0, gamma] (not NULL: EINVAL).
 * Workspace: at least dflash_verify_workspace_bytes(B, gamma, V). */
int dflash_verify_greedy_lengths(const float* target_logits, const int32_t* draft_ids, const int32_t* lengths,
                                 int32_t B, int32_t gamma, int32_t V, int32_t* accepted, int32_t* committed,
                                 int32_t* ids, int32_t* next_anchor, void* ws, size_t ws_bytes, void* stream);

/* Greedy verification from the target's hidden states (the DFlash2 variant:
 * page "Inco Hacks Native: DFlash 2 Speculation", section 3, the target
 * verifies the block). The target hands over its final hidden rows (after its
 * own final norm) at the gamma+1 verify positions; the borrowed LM head scores
 * them and the greedy rule of dflash_verify_greedy decides:
 *   t[b, j] = argmax_v target_hidden[b, j] . E_out[v]   (lowest index on ties)
 * then accepted, committed, ids and next_anchor exactly as there (lengths:
 * optional, as in dflash_verify_greedy_lengths; NULL = gamma for every row).
 *   target_hidden: device [B, gamma+1, H], bf16 (bf16 and int4 models) or
 *                  fp32 (fp32 models), 16-byte aligned; E_out is the model's
 *                  lm_head. No logits are materialised.
 * Workspace: at least dflash_verify_hidden_workspace_bytes(dims, B). */
int dflash_verify_from_hidden(const dflash_model* model, const void* target_hidden, int32_t B,
                              const int32_t* draft_ids, const int32_t* lengths, int32_t* accepted,
                              int32_t* committed, int32_t* ids, int32_t* next_anchor, void* ws, size_t ws_bytes,
                              void* stream);
size_t dflash_verify_hidden_workspace_bytes(const dflash_dims* dims, int32_t B);

/* For callers that cannot allocate (code under HIP graph capture, serving
 * loops or harnesses that forbid hipMalloc): dflash_verify_greedy without a
 * workspace argument. Same arguments, outputs and checks otherwise. Its
 * partial results live in a device array the library holds, one per device,
 * of dflash_verify_noalloc_max_bytes() bytes (1 MiB) from the library's load to
 * the end of the process; a request whose dflash_verify_workspace_bytes(B,
 * gamma, V) exceeds it returns DFLASH_ENOSPC before anything is enqueued. The
 * call allocates nothing. Calls that overlap on one device share that array and
 * race; order them on one stream. */
int dflash_verify_greedy_noalloc(const float* target_logits, const int32_t* draft_ids, int32_t B, int32_t gamma,
                                 int32_t V, int32_t* accepted, int32_t* committed, int32_t* ids,
                                 int32_t* next_anchor, void* stream);
size_t dflash_verify_noalloc_max_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
