// C ABI of libdflash.so (declared in include/dflash.h): argument validation on
// the host, workspace layout, and the kernel sequence of each call.
#include <atomic>
#include <chrono>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/dflash.h"
#include "attention.hpp"
#include "gemm.hpp"
#include "gemv.hpp"
#include "head.hpp"
#include "i4mm.hpp"
#include "rope.hpp"
#include "skinny.hpp"
#include "trace.hpp"

using namespace dfl;

namespace dfl {
int api_gate();
void api_count_invocation();
}  // namespace dfl


namespace {

std::atomic<uint64_t> g_invocations{0};

// launch tracing (dflash_trace_begin / dflash_trace_end)
struct TraceState {
    std::mutex mu;
    std::atomic<int> kinds{0};
    uint64_t* stamps = nullptr;
    int64_t capacity = 0, cursor = 0;
    std::vector<dflash_trace_record> records;
};
TraceState g_trace;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool kill_switch() {
    const char* e = std::getenv("DFLASH_DISABLE");
    return e && e[0] && std::strcmp(e, "0") != 0;
}

// gfx950 present on the current device (checked per call; the properties
// query is cached per device id)
bool device_supported() {
    static std::mutex mu;
    static int cached[64];
    static bool init = false;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lk(mu);
    if (!init) {
        for (int& c : cached) c = -1;
        init = true;
    }
    if (cached[dev] < 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
        cached[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    }
    return cached[dev] == 1;
}

int gate() { return (kill_switch() || !device_supported()) ? DFLASH_DECLINED : DFLASH_OK; }

int check_dims(const dflash_dims* d) {
    if (!d) return DFLASH_EINVAL;
    if (d->H <= 0 || d->m <= 0 || d->d <= 0 || d->nl < 0 || d->hq <= 0 || d->hkv <= 0 || d->hd <= 0 || d->F <= 0 ||
        d->V <= 0 || d->gamma <= 0)
        return DFLASH_EINVAL;
    if (d->d != d->hq * d->hd || d->hq % d->hkv != 0) return DFLASH_EINVAL;
    if (!(d->eps >= 0.0f) || d->eps > 1.0f) return DFLASH_EINVAL;
    if (d->window < 0 || !(d->rope_theta >= 0.0f) || d->rope_theta > 1e30f) return DFLASH_EINVAL;
    if (d->hd != 64 && d->hd != 128) return DFLASH_DECLINED;
    if (d->wdtype != DFLASH_F32 && d->wdtype != DFLASH_BF16 && d->wdtype != DFLASH_INT4G64) return DFLASH_DECLINED;
    if (d->act != DFLASH_ACT_GELU_TANH && d->act != DFLASH_ACT_SILU) return DFLASH_DECLINED;
    if (d->nl > kMaxLayers || d->m > kMaxTaps) return DFLASH_DECLINED;
    if (d->gamma > kAttnMaxGamma) return DFLASH_DECLINED;  // the block's keys form one 32-key unit
    if (d->d > 8192) return DFLASH_DECLINED;  // the row norms hold a row in one workgroup's registers
    if ((d->hq / d->hkv) * d->gamma > attention_max_rows(d->wdtype == DFLASH_F32)) return DFLASH_DECLINED;
    const int q = d->wdtype == DFLASH_INT4G64 ? 64 : 8;
    if (d->H % q || d->d % q || d->F % q) return DFLASH_DECLINED;
    return DFLASH_OK;
}

int wtype_of(int dtype) { return dtype == DFLASH_F32 ? W_F32 : (dtype == DFLASH_BF16 ? W_BF16 : W_I4); }

// the rotary frequencies of (hd, theta), formed once per thread for the last pair asked for
const RopeFreq& rope_freqs(int hd, float theta) {
    thread_local RopeFreq f{};
    thread_local int f_hd = -1;
    thread_local float f_theta = -1.0f;
    if (hd != f_hd || theta != f_theta) {
        f = rope_freq(hd, theta);
        f_hd = hd;
        f_theta = theta;
    }
    return f;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_weight(const dflash_weight& w, int rows, int cols, int want_dtype /* -1: any */) {
    if (!w.data) return DFLASH_EINVAL;
    if (!aligned16(w.data)) return DFLASH_DECLINED;  // rows are read as 16-byte vectors
    if (w.dtype != DFLASH_F32 && w.dtype != DFLASH_BF16 && w.dtype != DFLASH_INT4G64) return DFLASH_EINVAL;
    if (want_dtype >= 0 && w.dtype != want_dtype) return DFLASH_EINVAL;
    if (w.rows != rows || w.cols != cols) return DFLASH_EINVAL;
    if (w.dtype == DFLASH_INT4G64) {
        if (!w.scales || !w.biases) return DFLASH_EINVAL;
        if (cols % 64) return DFLASH_DECLINED;
    } else if (cols % 8) {
        return DFLASH_DECLINED;
    }
    return DFLASH_OK;
}

#define DFL_TRY(expr)                     \
    do {                                  \
        const int rc_ = (expr);           \
        if (rc_ != DFLASH_OK) return rc_; \
    } while (0)
#define DFL_HIP(expr)                                    \
    do {                                                 \
        if ((expr) != hipSuccess) return DFLASH_EHIP;    \
    } while (0)

int check_model(const dflash_model* M) {
    if (!M) return DFLASH_EINVAL;
    DFL_TRY(check_dims(&M->dims));
    const dflash_dims& d = M->dims;
    const int wd = d.wdtype;
    if (!M->ctx_norm || !M->block_pos || !M->out_norm || (d.gamma > 1 && !M->mask_emb)) return DFLASH_EINVAL;
    if (d.nl > 0 && !M->layers) return DFLASH_EINVAL;
    if (!aligned16(M->ctx_norm) || !aligned16(M->out_norm)) return DFLASH_DECLINED;  // gains: 16-byte vectors
    DFL_TRY(check_weight(M->w_c, d.d, d.m * d.H, wd));
    DFL_TRY(check_weight(M->tok_proj, d.d, d.H, wd));
    DFL_TRY(check_weight(M->out_proj, d.H, d.d, wd));
    DFL_TRY(check_weight(M->embed_in, d.V, d.H, -1));
    DFL_TRY(check_weight(M->lm_head, d.V, d.H, -1));
    for (int i = 0; i < d.nl; ++i) {
        const dflash_layer& L = M->layers[i];
        if (!L.attn_norm || !L.ffn_norm) return DFLASH_EINVAL;
        if (!aligned16(L.attn_norm) || !aligned16(L.ffn_norm)) return DFLASH_DECLINED;
        DFL_TRY(check_weight(L.w_qkv, (d.hq + 2 * d.hkv) * d.hd, d.d, wd));
        DFL_TRY(check_weight(L.w_o, d.d, d.hq * d.hd, wd));
        DFL_TRY(check_weight(L.w_gate_up, 2 * d.F, d.d, wd));
        DFL_TRY(check_weight(L.w_down, d.d, d.F, wd));
    }
    return DFLASH_OK;
}

int check_kv(const dflash_kv* kv, const dflash_dims& d, int B) {
    if (!kv || !kv->k || !kv->v || !kv->len) return DFLASH_EINVAL;
    if (kv->B < B || B <= 0 || kv->cap <= 0) return DFLASH_EINVAL;
    const int want = d.wdtype == DFLASH_F32 ? DFLASH_F32 : DFLASH_BF16;
    if (kv->dtype != want) return DFLASH_EINVAL;
    if (kv->dtype == DFLASH_BF16 && kv->cap % 32) return DFLASH_EINVAL;  // 32-key chunks of the value rows
    return DFLASH_OK;
}

WeightPtr wptr(const dflash_weight& w) {
    WeightPtr p;
    p.data = w.data;
    p.scales = static_cast<const uint16_t*>(w.scales);
    p.biases = static_cast<const uint16_t*>(w.biases);
    return p;
}


// output rows from which a projection's GEMV takes 4 weight rows per wavefront: bf16 and
// fp32 weights from 4096 (wide drafter 628 -> 660 blocks/s), int4 weights (ALU-bound
// products) from 16384 (4096 cost the int4 wide drafter 8%)
#ifndef DFL_RPW4_N
#define DFL_RPW4_N 4096
#endif
#ifndef DFL_RPW4_N_I4
#define DFL_RPW4_N_I4 16384
#endif
int rpw_for(int N, int wdtype) {
    const int n4 = wdtype == DFLASH_INT4G64 ? DFL_RPW4_N_I4 : DFL_RPW4_N;
    return N >= n4 ? 4 : (N >= 2048 ? 2 : 1);
}
// workgroup cap of the per-layer projections (row tiles beyond it are looped over)
#ifndef DFL_SMALL_WGS
#define DFL_SMALL_WGS 512
#endif
// row counts from which the context projection and the K/V append run as
// matrix-core GEMMs (prefill) instead of GEMVs
#ifndef DFL_GEMM_MIN_ROWS
#define DFL_GEMM_MIN_ROWS 64
#endif
// LM-head workgroups; each loops over row tiles of 16 vocabulary rows (768: three
// workgroups per CU at the head kernel's register budget, all resident at once)
#ifndef DFL_LM_WGS
#define DFL_LM_WGS 768
#endif
constexpr int kLmWgs = DFL_LM_WGS;
// weight rows per wavefront and workgroups of an int4 LM head (its products are
// ALU-bound: two rows per wavefront keep two wavefronts per SIMD)
#ifndef DFL_LM_RPW_I4
#define DFL_LM_RPW_I4 2
#endif
#ifndef DFL_LM_WGS_I4
#define DFL_LM_WGS_I4 512
#endif
// weight rows per wavefront of a bf16 / fp32 LM head
#ifndef DFL_LM_RPW
#define DFL_LM_RPW 4
#endif
// One argmax partial per LM-head workgroup. Row tiles of 4 * rpw vocabulary rows; a
// head whose rows (H) stage in one pass runs persistent workgroups (kLmWgs, or one
// per CU for long rows), a longer one a workgroup per tile.
int lm_rpw(int wtype) { return wtype == W_I4 ? DFL_LM_RPW_I4 : DFL_LM_RPW; }
int lm_tiles(int V, int wtype) { return (V + 4 * lm_rpw(wtype) - 1) / (4 * lm_rpw(wtype)); }
// argmax partials per row, enough for any head layout
int lm_tiles_max(int V) {
    const int r = DFL_LM_RPW_I4 < DFL_LM_RPW ? DFL_LM_RPW_I4 : DFL_LM_RPW;
    return (V + 4 * r - 1) / (4 * r);
}
int lm_wgs(int wtype) { return wtype == W_I4 ? DFL_LM_WGS_I4 : kLmWgs; }
int lm_nblocks(int V, int H, int wtype, int rows) {
    return gemv_head_grid(wtype, H, lm_tiles(V, wtype), lm_wgs(wtype), rows);
}
// split-K of the context projection for few rows: K ranges of at most 2048
#ifndef DFL_CTX_SPLIT_K
#define DFL_CTX_SPLIT_K 2048
#endif
#ifndef DFL_KV_WGS
#define DFL_KV_WGS DFL_SMALL_WGS  // workgroup cap of the context K/V append, all layers together
#endif
// (int4 weights: staging the activations costs ALU work as well, so wider K ranges)
#ifndef DFL_CTX_SPLIT_K_I4
#define DFL_CTX_SPLIT_K_I4 8192
#endif
int ctx_splits(const dflash_dims& d) {
    const int w = d.wdtype == DFLASH_INT4G64 ? DFL_CTX_SPLIT_K_I4 : DFL_CTX_SPLIT_K;
    return (d.m * d.H + w - 1) / w;
}
// block row counts from which the projections of a bf16 drafter run on matrix
// cores (one pass over each weight matrix) instead of 8-row GEMV passes
#ifndef DFL_SKINNY_MIN_ROWS
#define DFL_SKINNY_MIN_ROWS 16
#endif
// long rows of a bf16 / int4 drafter: RMSNorm once per row into bf16 rows (norm_rows)
// instead of two passes over the fp32 row in every GEMV workgroup's prologue
bool prenorm(const dflash_dims& d) { return d.wdtype != DFLASH_F32 && d.d > kRegNormMaxK; }
// ... and from this many on drafters with long rows (d, or the head's H, above the register
// norm's limit): there an 8-row GEMV pass over the long weight rows costs more than one
// matrix-core pass for all rows (Wide, 7 rows: 675 -> 723 blocks/s); on short rows the
// GEMVs' latency is lower (Default, 5 rows: 3,335 against 2,665 on matrix cores)
#ifndef DFL_SKINNY_MIN_ROWS_WIDE
#define DFL_SKINNY_MIN_ROWS_WIDE 4
#endif
int skinny_min_rows(const dflash_dims& d) { return prenorm(d) ? DFL_SKINNY_MIN_ROWS_WIDE : DFL_SKINNY_MIN_ROWS; }
// split-K of the plain-prologue GEMVs (residual, store and gated epilogues): K ranges
// of at most this many elements for the 8-row kernels (twice as many for the 4-row
// int4 kernel), which stage once within the normal LDS budget with several
// workgroups per CU; a reduce kernel adds the partial sums in split order and applies
// the epilogue
#ifndef DFL_GEMV_SPLIT_K
#define DFL_GEMV_SPLIT_K 4096
#endif
void gemv_split(const dflash_dims& d, int K, int rows, int* nsplit, int* kslice) {
    const int lim = DFL_GEMV_SPLIT_K * (8 / gemv_maxm(wtype_of(d.wdtype), rows < 8 ? rows : 8));
    int ns = d.wdtype == DFLASH_F32 ? 1 : (K + lim - 1) / lim;
    int ks = K;
    if (ns > 1) {
        ks = ((K + ns - 1) / ns + 511) / 512 * 512;
        ns = (K + ks - 1) / ks;
    }
    *nsplit = ns;
    *kslice = ks;
}

bool lm_head_skinny(int wdtype, int y_f32, int rows, int H) {
    return wdtype == DFLASH_BF16 && !y_f32 && H % kSkinnyK == 0 &&
           rows >= (H > kRegNormMaxK ? DFL_SKINNY_MIN_ROWS_WIDE : DFL_SKINNY_MIN_ROWS);
}
bool skinny_ok(const dflash_dims& d, int rows) {
    return d.wdtype == DFLASH_BF16 && rows >= skinny_min_rows(d) && d.d % kSkinnyK == 0 && d.F % kSkinnyK == 0 &&
           d.H % kSkinnyK == 0;
}
// fp32 split-K partials of the skinny launches of a forward (rows in launches of kSkinnyRows)
// Split-K of the gated (gate/up) matrix-core projection: gate/up tiles alone give about
// one workgroup per CU at the wide width (2F = 34816 rows: 272 tiles), where the kernel
// holds two per CU; split, the K ranges write partial sums over the 2F gate and up rows
// and an ordered reduce applies the activation.
#ifndef DFL_SK_GATED_WGS
#define DFL_SK_GATED_WGS 512
#endif
void skinny_gated_split(int n2, int K, int* nsplit, int* kslice) {
    const int tiles = skinny_tiles(SK_PARTIAL, n2), chunks = K / kSkinnyK;
    int sp = tiles >= DFL_SK_GATED_WGS ? 1 : (DFL_SK_GATED_WGS + tiles - 1) / tiles;
    sp = sp < 1 ? 1 : (sp > chunks ? chunks : sp);
    const int per = chunks > 0 ? (chunks + sp - 1) / sp : 1;
    *kslice = per * kSkinnyK;
    *nsplit = chunks > 0 ? (chunks + per - 1) / per : 1;
}

size_t skinny_part_bytes(const dflash_dims& d, int rows) {
    const int r = rows < kSkinnyRows ? rows : kSkinnyRows;
    const int qkv_rows = (d.hq + 2 * d.hkv) * d.hd;
    const int shapes[5][3] = {{SK_STORE, qkv_rows, d.d}, {SK_RESID, d.d, d.hq * d.hd}, {SK_RESID, d.d, d.F},
                              {SK_STORE, d.H, d.d}, {SK_STORE, d.d, d.H}};
    size_t most = 0;
    for (const auto& sh : shapes) {
        int ns = 1, ks = 0;
        skinny_split(sh[0], sh[1], sh[2], 1, &ns, &ks);
        const size_t b = ns > 1 ? (size_t)ns * r * sh[1] * 4 : 0;
        if (b > most) most = b;
    }
    int ns = 1, ks = 0;
    skinny_gated_split(2 * d.F, d.d, &ns, &ks);
    size_t g = ns > 1 ? (size_t)ns * r * 2 * d.F * 4 : 0;
    const size_t bal = skinny_gated_balanced_floats(r) * 4;  // the balanced gated launch's tail partials
    if (bal > g) g = bal;
    return g > most ? g : most;
}

// Workspace of the matrix-core paths for n context rows (a round's appended
// block rows); 0 when those paths do not apply. Context projection: split-K
// partial sums [nsplit][n][d]. K/V append: each layer's normalised rows, bf16
// [nl][n][d], then the split-K partials [nl][nsplit][n][2 hkv hd].
bool ctx_skinny_rows(const dflash_dims& d, int n) {
    return d.wdtype == DFLASH_BF16 && n >= skinny_min_rows(d) && n <= kSkinnyRows;
}
size_t ctx_project_skinny_bytes(const dflash_dims& d, int n) {
    if (!ctx_skinny_rows(d, n) || d.H % kSkinnyK || d.m > kMaxTaps) return 0;
    int ns = 1, ks = 0;
    skinny_split(SK_PARTIAL, d.d, d.m * d.H, 1, &ns, &ks);
    return (size_t)ns * n * d.d * 4;
}
size_t kv_append_norm_bytes(const dflash_dims& d, int n) { return align_up((size_t)d.nl * n * d.d * 2); }
// the GEMV append of up to 8 pre-normalised rows over K ranges beyond one pass of the
// 8-row kernel's normal LDS budget splits K (two ranges at width 5120: half the staging,
// twice the resident workgroups); its fp32 partials [nl][nsplit][n][2 hkv hd] follow the
// normalised rows in the workspace
int kv_append_gemv_split(const dflash_dims& d, int n, int* kslice) {
    int ns = 1, ks = d.d;
    if (d.wdtype == DFLASH_BF16 && prenorm(d) && n >= 1 && n <= 8 && d.d > kStageBytes / (8 * 2))
        gemv_split(d, d.d, n, &ns, &ks);
    *kslice = ks;
    return ns;
}
size_t kv_append_split_bytes(const dflash_dims& d, int n) {
    int ks = 0;
    const int ns = kv_append_gemv_split(d, n, &ks);
    return kv_append_norm_bytes(d, n) + (ns > 1 ? align_up((size_t)d.nl * ns * n * 2 * d.hkv * d.hd * 4) : 0);
}
// int4 context projection of n <= 16 rows on matrix cores: split partials [ns][n][d] (0: not
// served there; the K ranges must not straddle a tap buffer)
size_t ctx_i4_bytes(const dflash_dims& d, int n) {
    if (d.wdtype != DFLASH_INT4G64 || !i4mm_ok(d.m * d.H, n)) return 0;
    int ns = 1, ks = 0;
    i4mm_split(d.m * d.H, &ns, &ks);
    if (d.H % ks) return 0;
    return align_up((size_t)ns * n * d.d * 4);
}
// int4 K/V append of n <= 16 pre-normalised rows on matrix cores: the normalised rows, then
// split partials [nl][ns][n][2 hkv hd] (0: not served there)
size_t kv_i4_bytes(const dflash_dims& d, int n) {
    if (d.wdtype != DFLASH_INT4G64 || !prenorm(d) || d.nl < 1 || !i4mm_ok(d.d, n)) return 0;
    int ns = 1, ks = 0;
    i4mm_split(d.d, &ns, &ks);
    return kv_append_norm_bytes(d, n) + align_up((size_t)d.nl * ns * n * 2 * d.hkv * d.hd * 4);
}

// int4 prefill (n >= DFL_GEMM_MIN_ROWS rows) on matrix cores: the call expands its int4
// weights into bf16 high and low parts in ws ([N, 2K], one bf16 GEMM against [A | A]); the
// context projection expands W_c [d, m H], the K/V append every layer's K and V rows
// [2 hkv hd, d] and keeps the per-row RMS factors after them. 0: not served there.
size_t i4_prefill_proj_bytes(const dflash_dims& d, int n) {
    if (d.wdtype != DFLASH_INT4G64 || n < DFL_GEMM_MIN_ROWS || d.H % 64 || d.m > kMaxTaps) return 0;
    return align_up((size_t)d.d * 2 * d.m * d.H * 2);
}
size_t i4_prefill_kv_bytes(const dflash_dims& d, int n) {
    if (d.wdtype != DFLASH_INT4G64 || n < DFL_GEMM_MIN_ROWS || d.d % 64 || d.nl < 1) return 0;
    return align_up((size_t)d.nl * 2 * d.hkv * d.hd * 2 * d.d * 2) + align_up((size_t)n * 4);
}

size_t kv_append_skinny_bytes(const dflash_dims& d, int n) {
    if (!ctx_skinny_rows(d, n) || d.d % kSkinnyK || d.nl < 1) return 0;
    const int N = 2 * d.hkv * d.hd;
    int ns = 1, ks = 0;
    skinny_split(SK_KV, N, d.d, d.nl, &ns, &ks);
    return kv_append_norm_bytes(d, n) + (ns > 1 ? (size_t)d.nl * ns * n * N * 4 : 0);
}

struct Ws {
    float* hd;
    float* qkv;
    float* part;
    float* o;
    float* a;
    float* y;
    float* lmv;
    int32_t* lmi;
    float* ctxp;   // split-K partials of the context projection [splits][B*(gamma+1)][d]
    uint16_t* vt;  // block values, head-dim major [B][hkv][hd][32] (bf16 models)
    uint16_t* an;  // normalised block rows, bf16 [B*gamma][d] (matrix-core path, long rows)
    float* skp;    // matrix-core path: split-K partial sums
    float* rsp;    // GEMV path: split-K partial sums of the residual projections
    float* i4h;    // int4 LM head on matrix cores: split-K partial logits [splits][B*gamma][V] (else null)
    size_t i4h_bytes;
    bool skinny;   // the block projections run on matrix cores
    size_t total;
    int nsplit;  // attention workgroups per (sequence, kv head)
    int nparts;  // attention partials per (sequence, head)
};

Ws ws_layout(const dflash_dims& d, int B, int cap, void* base) {
    Ws w{};
    const size_t rows = (size_t)B * d.gamma;
    const int qkv_rows = (d.hq + 2 * d.hkv) * d.hd;
    attention_splits(attn_span(cap, d.window), d.gamma, d.wdtype == DFLASH_F32, B * d.hkv, (d.hq / d.hkv) * d.gamma,
                     d.hd, &w.nsplit, &w.nparts);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const size_t o_hd = take(rows * d.d * 4);
    const size_t o_qkv = take(rows * qkv_rows * 4);
    const size_t o_part = take((size_t)B * d.hq * w.nparts * d.gamma * (d.hd + 2) * 4);
    const size_t o_o = take(rows * d.hq * d.hd * 4);
    const size_t o_a = take(rows * d.F * 4);
    const size_t o_y = take(rows * d.H * 4);
    const size_t nb = lm_tiles_max(d.V);  // enough for any head layout
    const size_t o_lmv = take(rows * nb * 4);
    const size_t o_lmi = take(rows * nb * 4);
    const size_t o_ctxp = take((size_t)ctx_splits(d) * B * (d.gamma + 1) * d.d * 4);
    const size_t o_vt = take((size_t)B * d.hkv * d.hd * 32 * 2);
    w.skinny = skinny_ok(d, (int)rows);
    const size_t o_an = take((w.skinny || prenorm(d)) ? rows * d.d * 2 : 0);
    const size_t o_skp = take(w.skinny ? skinny_part_bytes(d, (int)rows) : 0);
    size_t rsp_bytes = 0;
    if (!w.skinny) {
        // O and down (N = d), QKV (K = d), out (N = H, K = d) and gate/up (2F rows, K = d),
        // when their rows are pre-normalised (plain prologue)
        const int shapes[5][2] = {{d.hq * d.hd, d.d}, {d.F, d.d}, {d.d, qkv_rows}, {d.d, d.H}, {d.d, 2 * d.F}};
        for (int q = 0; q < 5; ++q) {
            if (q >= 2 && !prenorm(d)) break;
            int ns = 1, ks = 0;
            // int4 weights of up to 16 rows: always partial sums (matrix-core K ranges)
            const bool i4 = d.wdtype == DFLASH_INT4G64 && i4mm_ok(shapes[q][0], (int)rows);
            if (i4)
                i4mm_split(shapes[q][0], &ns, &ks);
            else
                gemv_split(d, shapes[q][0], (int)rows, &ns, &ks);
            const size_t b = (size_t)ns * rows * shapes[q][1] * 4;
            if ((ns > 1 || i4) && b > rsp_bytes) rsp_bytes = b;
        }
    }
    const size_t o_rsp = take(rsp_bytes);
    size_t i4h_bytes = 0;
    if (d.wdtype == DFLASH_INT4G64 && i4mm_ok(d.H, (int)rows)) {
        int ns = 1, ks = 0;
        i4mm_split(d.H, &ns, &ks);
        i4h_bytes = (size_t)ns * rows * d.V * 4;
    }
    const size_t o_i4h = take(i4h_bytes);
    w.i4h_bytes = i4h_bytes;
    w.total = off;
    // the context append of up to B*cap rows keeps one float per row at the base; the
    // matrix-core context paths of a round's B*(gamma+1) rows use the base as well
    if (w.total < (size_t)B * cap * 4) w.total = align_up((size_t)B * cap * 4);
    const int nr = B * (d.gamma + 1);
    const size_t ctx_need = align_up(ctx_project_skinny_bytes(d, nr)), kv_need = align_up(kv_append_skinny_bytes(d, nr));
    if (w.total < ctx_need) w.total = ctx_need;
    if (w.total < kv_need) w.total = kv_need;
    if (prenorm(d) && w.total < kv_append_norm_bytes(d, nr)) w.total = kv_append_norm_bytes(d, nr);
    if (prenorm(d) && w.total < kv_append_split_bytes(d, nr < 8 ? nr : 8))
        w.total = kv_append_split_bytes(d, nr < 8 ? nr : 8);
    if (w.total < ctx_i4_bytes(d, nr)) w.total = ctx_i4_bytes(d, nr);
    if (w.total < kv_i4_bytes(d, nr)) w.total = kv_i4_bytes(d, nr);
    char* c = static_cast<char*>(base);
    if (c) {
        w.hd = reinterpret_cast<float*>(c + o_hd);
        w.qkv = reinterpret_cast<float*>(c + o_qkv);
        w.part = reinterpret_cast<float*>(c + o_part);
        w.o = reinterpret_cast<float*>(c + o_o);
        w.a = reinterpret_cast<float*>(c + o_a);
        w.y = reinterpret_cast<float*>(c + o_y);
        w.lmv = reinterpret_cast<float*>(c + o_lmv);
        w.lmi = reinterpret_cast<int32_t*>(c + o_lmi);
        w.ctxp = reinterpret_cast<float*>(c + o_ctxp);
        w.vt = reinterpret_cast<uint16_t*>(c + o_vt);
        w.an = reinterpret_cast<uint16_t*>(c + o_an);
        w.skp = reinterpret_cast<float*>(c + o_skp);
        w.rsp = reinterpret_cast<float*>(c + o_rsp);
        w.i4h = i4h_bytes ? reinterpret_cast<float*>(c + o_i4h) : nullptr;
    }
    return w;
}

// ---------------------------------------------------------------------------
// GEMV helpers; activation rows are processed in chunks of up to 8 (32 for
// long row counts of the context projection and append)

GemvParams base_params(const dflash_dims& d) {
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.gain_f32 = d.wdtype == DFLASH_F32 ? 1 : 0;
    p.eps = d.eps;
    p.round_out = d.wdtype == DFLASH_F32 ? 0 : 1;
    p.src_f32 = d.wdtype == DFLASH_F32 ? 1 : 0;  // rounded activations travel as bf16
    p.max_wgs = DFL_SMALL_WGS;
    return p;
}

hipError_t gemv_rows(int wtype, int pro, int epi, GemvParams p, int rows, hipStream_t s, int layers = 1,
                     int maxm_long = 8) {
    // the bf16 block init of at most 4 sequences over rows longer than the 8-row kernel
    // stages in its normal LDS budget (H 5120) stages 4 rows: half the LDS keeps it in
    // that budget, at three persistent workgroups per CU instead of one
    const bool init4 = wtype == W_BF16 && pro == PRO_GATHER && epi == EPI_BLOCKINIT && rows <= 4 &&
                       p.K > kStageBytes / (8 * 2);
    const int maxm = rows > 8 ? maxm_long : init4 ? 4 : gemv_maxm(wtype, rows);
    for (int r0 = 0; r0 < rows; r0 += maxm) {
        GemvParams q = p;
        q.M = rows - r0 < maxm ? rows - r0 : maxm;
        if (pro == PRO_NORM || (pro == PRO_PLAIN && p.src_f32)) q.x = p.x + (int64_t)r0 * p.x_ld;
        if (pro == PRO_PLAIN && !p.src_f32)
            q.x = reinterpret_cast<const float*>(reinterpret_cast<const uint16_t*>(p.x) + (int64_t)r0 * p.x_ld);
        if (pro == PRO_TAPS) {
            const size_t esz = p.src_f32 ? 4 : 2;
            for (int j = 0; j < kMaxTaps; ++j)
                if (p.taps[j]) q.taps[j] = static_cast<const char*>(p.taps[j]) + (size_t)r0 * p.tap_ld * esz;
        }
        if (pro == PRO_GATHER) q.ids = p.ids + r0;
        if (epi == EPI_RESID || (epi == EPI_STORE && !p.out_bf16) || (epi == EPI_GATED && !p.round_out))
            q.out = p.out + (int64_t)r0 * p.out_ld;
        if ((epi == EPI_STORE && p.out_bf16) || (epi == EPI_GATED && p.round_out))
            q.out = reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)r0 * p.out_ld);
        if (epi == EPI_KV || (epi == EPI_STORE && p.vt)) q.row_base = p.row_base + r0;
        if (epi == EPI_BLOCKINIT) q.seq_base = p.seq_base + r0;
        if (epi == EPI_ARGMAX) {
            q.part_val = p.part_val + (int64_t)r0 * p.nblocks;
            q.part_idx = p.part_idx + (int64_t)r0 * p.nblocks;
            if (p.base) q.base = p.base + (int64_t)r0 * p.base_ld;
        }
        const hipError_t e = launch_gemv(wtype, pro, epi, maxm, q, layers, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// A plain-prologue GEMV with a residual (out += x W^T, fp32) or store epilogue (p's
// out fields): one launch, or split-K partials into part and the ordered reduce that
// applies the epilogue (long K ranges). With norm_gain, a split residual reduce also
// writes bf16(RMSNorm(out; norm_gain)) to norm_dst (the next projection's rows) and
// sets *normed; otherwise *normed is cleared.
hipError_t gemv_plain(const dflash_dims& d, int wt, int epi, GemvParams p, int rows, float* part, hipStream_t s,
                      const void* norm_gain = nullptr, uint16_t* norm_dst = nullptr, bool* normed = nullptr) {
    int ns = 1, ks = p.K;
    // int4 weights of up to 16 bf16 rows: matrix-core K ranges, then the same ordered reduce
    const bool i4 = wt == W_I4 && !p.src_f32 && i4mm_ok(p.K, rows) && part;
    if (i4)
        i4mm_split(p.K, &ns, &ks);
    else
        gemv_split(d, p.K, rows, &ns, &ks);
    if (normed) *normed = false;
    if (ns <= 1 && !i4) return gemv_rows(wt, PRO_PLAIN, epi, p, rows, s);
    SkinnyParams r;
    std::memset(&r, 0, sizeof(r));
    r.M = rows;
    r.N = epi == EPI_GATED ? p.F : p.N;  // gated: F outputs from the 2F gate and up rows
    r.act = p.act;
    r.nsplit = ns;
    r.part = part;
    r.out = p.out;
    r.out_ld = p.out_ld;
    r.out_bf16 = epi == EPI_STORE ? p.out_bf16 : 0;
    r.vt = epi == EPI_STORE ? p.vt : nullptr;
    r.vt_col = p.vt_col;
    r.row_base = p.row_base;
    r.gamma = p.gamma;
    r.hkv = p.hkv;
    r.hd = p.hd;
    hipError_t e;
    if (i4) {
        I4Params q;
        std::memset(&q, 0, sizeof(q));
        q.codes[0] = static_cast<const uint32_t*>(p.w[0].data);
        q.scales[0] = p.w[0].scales;
        q.biases[0] = p.w[0].biases;
        q.layers = 1;
        q.N = p.N;
        q.K = p.K;
        q.a = reinterpret_cast<const uint16_t*>(p.x);
        q.a_ld = p.x_ld;
        q.M = rows;
        q.nsplit = ns;
        q.kslice = ks;
        q.part = part;
        e = launch_i4mm(q, s);
    } else {
        p.ksplit = ns;
        p.kslice = ks;
        p.max_wgs = DFL_SMALL_WGS / ns > 0 ? DFL_SMALL_WGS / ns : 1;
        p.rpw = rpw_for(p.N, d.wdtype);
        p.out = part;
        p.out_ld = p.N;
        p.split_stride = (int64_t)rows * p.N;
        p.round_out = 0;
        p.out_bf16 = 0;
        p.vt = nullptr;
        e = gemv_rows(wt, PRO_PLAIN, EPI_STORE, p, rows, s);
    }
    if (e != hipSuccess) return e;
    if (epi == EPI_RESID && norm_gain && norm_dst && normed) {
        *normed = true;
        return launch_resid_norm(part, ns, rows, p.N, static_cast<float*>(r.out), r.out_ld, norm_gain,
                                 d.wdtype == DFLASH_F32, d.eps, norm_dst, d.d, s);
    }
    return launch_split_reduce(epi == EPI_RESID ? SK_RESID : (epi == EPI_GATED ? SK_GATED : SK_STORE), r, s);
}

// matrix-core projections of `rows` block rows, in launches of up to kSkinnyRows
hipError_t skinny_rows(int epi, SkinnyParams p, int rows, hipStream_t s) {
    skinny_split(epi, p.N, p.K, p.layers, &p.nsplit, &p.kslice);
    p.nblocks = skinny_tiles(epi, p.N);
    const size_t out_esz = (epi == SK_GATED || (epi == SK_STORE && p.out_bf16)) ? 2 : 4;
    for (int r0 = 0; r0 < rows; r0 += kSkinnyRows) {
        SkinnyParams q = p;
        q.M = rows - r0 < kSkinnyRows ? rows - r0 : kSkinnyRows;
        q.a = p.a + (int64_t)r0 * p.a_ld;
        q.row_base = p.row_base + r0;
        if (p.out) q.out = static_cast<char*>(p.out) + (size_t)r0 * p.out_ld * out_esz;
        if (epi == SK_ARGMAX) {
            q.part_val = p.part_val + (int64_t)r0 * p.nblocks;
            q.part_idx = p.part_idx + (int64_t)r0 * p.nblocks;
            if (p.base) q.base = p.base + (int64_t)r0 * p.base_ld;
        }
        const hipError_t e = launch_skinny(epi, q, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// the gated projection: one launch with the activation epilogue, or (split K) partial
// sums over the 2F gate and up rows and the gated reduce, per launch of kSkinnyRows rows
hipError_t skinny_gated(SkinnyParams p, int rows, hipStream_t s) {
    int ns = 1, ks = p.K;
    skinny_gated_split(p.N, p.K, &ns, &ks);
    for (int r0 = 0; r0 < rows; r0 += kSkinnyRows) {
        const int m = rows - r0 < kSkinnyRows ? rows - r0 : kSkinnyRows;
        if (p.part && skinny_gated_balanced(m, p.N, p.K)) {
            // 5+ row tiles and more column tiles than CUs: whole tiles spread over the CUs on
            // the direct-to-LDS kernel, the remainder split in K (partials in p.part)
            SkinnyParams q = p;
            q.M = m;
            q.a = p.a + (int64_t)r0 * p.a_ld;
            q.out = static_cast<uint16_t*>(p.out) + (size_t)r0 * p.out_ld;
            q.nblocks = skinny_tiles(SK_GATED, p.N);
            const hipError_t e = launch_skinny_gated_balanced(q, s);
            if (e != hipSuccess) return e;
            continue;
        }
        if (ns <= 1) {
            SkinnyParams q = p;
            q.M = m;
            q.a = p.a + (int64_t)r0 * p.a_ld;
            q.out = static_cast<uint16_t*>(p.out) + (size_t)r0 * p.out_ld;
            const hipError_t e = skinny_rows(SK_GATED, q, m, s);
            if (e != hipSuccess) return e;
            continue;
        }
        SkinnyParams q = p;
        q.M = m;
        q.a = p.a + (int64_t)r0 * p.a_ld;
        q.nsplit = ns;
        q.kslice = ks;
        q.nblocks = skinny_tiles(SK_PARTIAL, p.N);
        q.out = nullptr;
        hipError_t e = launch_skinny(SK_PARTIAL, q, s);
        if (e != hipSuccess) return e;
        SkinnyParams r = q;
        r.N = p.F;
        r.out = static_cast<uint16_t*>(p.out) + (size_t)r0 * p.out_ld;
        e = launch_split_reduce(SK_GATED, r, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

SkinnyParams skinny_params(const dflash_weight& W, const uint16_t* a, int64_t a_ld, int N, int K, float* part) {
    SkinnyParams p;
    std::memset(&p, 0, sizeof(p));
    p.a = a;
    p.a_ld = a_ld;
    p.w[0] = static_cast<const uint16_t*>(W.data);
    p.layers = 1;
    p.N = N;
    p.K = K;
    p.part = part;
    return p;
}

hipError_t norm_rows(const float* x, int rows, int K, const void* gain, float eps, uint16_t* dst, hipStream_t s) {
    NormRowsParams q;
    std::memset(&q, 0, sizeof(q));
    q.x = x;
    q.x_ld = K;
    q.rows = rows;
    q.K = K;
    q.layers = 1;
    q.eps = eps;
    q.gain[0] = gain;
    q.dst = dst;
    q.dst_ld = K;
    return launch_norm_rows(q, s);
}

// H += a W^T on matrix cores (p's out = H). Split K with norm_gain: the partial sums,
// then one kernel per row that adds them in split order and also writes
// bf16(RMSNorm(H; norm_gain)) to norm_dst (the next projection's rows), *normed set;
// otherwise the residual epilogue alone, *normed cleared
hipError_t skinny_resid(const dflash_dims& d, SkinnyParams p, int rows, hipStream_t s, const void* norm_gain,
                        uint16_t* norm_dst, bool* normed) {
    int ns = 1, ks = p.K;
    skinny_split(SK_RESID, p.N, p.K, 1, &ns, &ks);
    *normed = false;
    if (ns <= 1 || !norm_gain || !norm_dst || (p.N % 4) || p.N > kNormMaxK) return skinny_rows(SK_RESID, p, rows, s);
    float* h = static_cast<float*>(p.out);
    for (int r0 = 0; r0 < rows; r0 += kSkinnyRows) {
        SkinnyParams q = p;
        q.M = rows - r0 < kSkinnyRows ? rows - r0 : kSkinnyRows;
        q.a = p.a + (int64_t)r0 * p.a_ld;
        q.nsplit = ns;
        q.kslice = ks;
        q.nblocks = skinny_tiles(SK_PARTIAL, p.N);
        q.out = nullptr;
        hipError_t e = launch_skinny(SK_PARTIAL, q, s);
        if (e != hipSuccess) return e;
        e = launch_resid_norm(p.part, ns, q.M, p.N, h + (int64_t)r0 * p.out_ld, p.out_ld, norm_gain,
                              d.wdtype == DFLASH_F32, d.eps, norm_dst + (int64_t)r0 * d.d, d.d, s);
        if (e != hipSuccess) return e;
    }
    *normed = true;
    return hipSuccess;
}

// a draft layer's projections on matrix cores (bf16 drafter, 16 or more block
// rows), with the rounding points of the GEMV path: bf16 normalised rows, Q/K/V,
// O and A. skinny_qkv: before the attention (an_ready: w.an already holds the
// normalised rows); skinny_out_ffn: after it
int skinny_qkv(const dflash_model* M, int i, float* h, int rows, const Ws& w, hipStream_t s, bool an_ready) {
    const dflash_dims& d = M->dims;
    const dflash_layer& L = M->layers[i];
    const int qkv_rows = (d.hq + 2 * d.hkv) * d.hd;
    {  // [Q | K_b | V_b] = bf16(RMSNorm(H; attn_norm)) W_qkv^T, V_b head-dim major
        if (!an_ready) DFL_HIP(norm_rows(h, rows, d.d, L.attn_norm, d.eps, w.an, s));
        SkinnyParams p = skinny_params(L.w_qkv, w.an, d.d, qkv_rows, d.d, w.skp);
        p.out = w.qkv;
        p.out_ld = qkv_rows;
        p.out_bf16 = 1;
        p.vt = w.vt;
        p.vt_col = (d.hq + d.hkv) * d.hd;
        p.gamma = d.gamma;
        p.hkv = d.hkv;
        p.hd = d.hd;
        DFL_HIP(skinny_rows(SK_STORE, p, rows, s));
    }
    return DFLASH_OK;
}

// next_gain / an_ready: as for run_layer
int skinny_out_ffn(const dflash_model* M, int i, float* h, int rows, const Ws& w, hipStream_t s,
                   const void* next_gain, bool* an_ready) {
    const dflash_dims& d = M->dims;
    const dflash_layer& L = M->layers[i];
    bool ffn_ready = false;
    {  // H += O W_o^T (a split reduce also writes the FFN's normalised rows)
        SkinnyParams p = skinny_params(L.w_o, reinterpret_cast<const uint16_t*>(w.o), d.hq * d.hd, d.d,
                                       d.hq * d.hd, w.skp);
        p.out = h;
        p.out_ld = d.d;
        DFL_HIP(skinny_resid(d, p, rows, s, L.ffn_norm, w.an, &ffn_ready));
    }
    {  // A = bf16(act(n2 W_gate^T) * (n2 W_up^T)), n2 = bf16(RMSNorm(H; ffn_norm))
        if (!ffn_ready) DFL_HIP(norm_rows(h, rows, d.d, L.ffn_norm, d.eps, w.an, s));
        SkinnyParams p = skinny_params(L.w_gate_up, w.an, d.d, 2 * d.F, d.d, w.skp);
        p.F = d.F;
        p.act = d.act;
        p.out = w.a;
        p.out_ld = d.F;
        DFL_HIP(skinny_gated(p, rows, s));
    }
    {  // H += A W_down^T (a split reduce also writes the next projection's normalised rows)
        SkinnyParams p = skinny_params(L.w_down, reinterpret_cast<const uint16_t*>(w.a), d.F, d.d, d.F, w.skp);
        p.out = h;
        p.out_ld = d.d;
        DFL_HIP(skinny_resid(d, p, rows, s, next_gain, w.an, an_ready));
    }
    return DFLASH_OK;
}

// next_gain: the RMSNorm gain of the projection that follows the layer (the next
// layer's attn_norm or out_norm; null when none follows in this call); *an_ready says
// on entry whether w.an already holds this layer's normalised input rows (bf16) and on
// return whether it holds the next projection's
// The round's new context rows for the one-pass layers: their K/V are produced by each
// layer's own Q|K|V pass (rows of h_ctx, sequence b's rows row_offsets[b] ..; the first
// counts[b] of them stored at len_old[b] + i, the lengths before the round)
struct CtxRows {
    const float* h_ctx;
    int n;
    const int32_t* row_offsets;
    const int32_t* counts;
    const int32_t* len_old;
};

// the fused pass applies: GEMV path with the in-register RMSNorm prologue, and the block rows
// plus the context rows within one 16-row launch
bool fused_qkv_ok(const dflash_dims& d, const Ws& w, int rows, int n) {
    // rotary keys turn after their rows are written, at the pre-round lengths: kept to the
    // separate append
    return !w.skinny && !prenorm(d) && d.wdtype != DFLASH_INT4G64 && d.d <= kRegNormMaxK && n > 0 &&
           rows + n <= 16 && d.rope_theta == 0.0f;
}

// the end of a K/V append: with rotary positions the new keys turn at the positions they
// were written to (the lengths before the append), then the lengths advance
int append_done(const dflash_model* M, const dflash_kv* kv, const int32_t* row_offsets, const int32_t* counts, int n,
                hipStream_t s) {
    const dflash_dims& d = M->dims;
    if (d.rope_theta > 0.0f && d.nl > 0)
        DFL_HIP(launch_rope_cache(kv->k, kv->dtype == DFLASH_F32, d.nl, (int64_t)kv->B * d.hkv * kv->cap * d.hd, kv->B,
                                  d.hkv, kv->cap, d.hd, row_offsets, counts, kv->len, n, rope_freqs(d.hd, d.rope_theta),
                                  s));
    DFL_HIP(launch_advance_len(kv->len, row_offsets, counts, kv->B, kv->cap, s));
    return DFLASH_OK;
}

int run_layer(const dflash_model* M, int i, float* h, const dflash_kv* kv, int B, const Ws& w, hipStream_t s,
              const void* next_gain, bool* an_ready, const CtxRows* ctx = nullptr) {
    const dflash_dims& d = M->dims;
    const dflash_layer& L = M->layers[i];
    const int wt = wtype_of(d.wdtype);
    const int rows = B * d.gamma;
    const int qkv_rows = (d.hq + 2 * d.hkv) * d.hd;

    if (w.skinny) {
        DFL_TRY(skinny_qkv(M, i, h, rows, w, s, *an_ready));
    } else {  // n = RMSNorm(H; attn_norm); [Q | K_b | V_b] = n W_qkv^T
        GemvParams p = base_params(d);
        p.w[0] = wptr(L.w_qkv);
        p.N = qkv_rows;
        p.K = d.d;
        p.rpw = rpw_for(p.N, d.wdtype);
        p.x = h;
        p.x_ld = d.d;
        p.gain[0] = L.attn_norm;
        int pro = PRO_NORM;
        if (prenorm(d)) {
            if (!*an_ready) DFL_HIP(norm_rows(h, rows, d.d, L.attn_norm, d.eps, w.an, s));
            p.x = reinterpret_cast<const float*>(w.an);  // bf16 rows (src_f32 = 0)
            pro = PRO_PLAIN;
        }
        p.out = w.qkv;
        p.out_ld = qkv_rows;
        if (d.wdtype != DFLASH_F32) {
            // bf16 models (Q, K_b, V_b are bf16 by the rounding contract): Q and K_b row-major,
            // V_b head-dim major: the layout of one 32-key chunk of the value cache
            p.out_bf16 = 1;
            p.vt = w.vt;
            p.vt_col = (d.hq + d.hkv) * d.hd;
            p.row_base = 0;
            p.gamma = d.gamma;
            p.hkv = d.hkv;
            p.hd = d.hd;
        }
        if (ctx && fused_qkv_ok(d, w, rows, ctx->n)) {
            // one pass over the layer's Q|K|V rows: the block rows' Q, K_b, V_b as above, and
            // the round's context rows' K, V into this layer's cache
            p.x2 = ctx->h_ctx;
            p.M1 = rows;
            p.M = rows + ctx->n;
            p.kv_col0 = d.hq * d.hd;
            p.out_bf16 = d.wdtype != DFLASH_F32;
            p.vt_col = (d.hq + d.hkv) * d.hd;
            p.row_base = 0;
            p.kcache = kv->k;
            p.vcache = kv->v;
            p.len = ctx->len_old;
            p.row_offsets = ctx->row_offsets;
            p.counts = ctx->counts;
            p.B = kv->B;
            p.cap = kv->cap;
            p.kv_f32 = kv->dtype == DFLASH_F32;
            p.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
            const size_t esz = kv->dtype == DFLASH_F32 ? 4 : 2;
            // this layer's caches: the launch's grid.y is 1, so layer 0 of the pointers
            p.kcache = static_cast<char*>(kv->k) + (size_t)i * p.layer_stride * esz;
            p.vcache = static_cast<char*>(kv->v) + (size_t)i * p.layer_stride * esz;
            p.hkv = d.hkv;
            p.hd = d.hd;
            p.gamma = d.gamma;
            DFL_HIP(launch_gemv(wt, PRO_NORM, EPI_QKVKV, 16, p, 1, s));
        } else if (pro == PRO_PLAIN) {
            DFL_HIP(gemv_plain(d, wt, EPI_STORE, p, rows, w.rsp, s));
        } else {
            DFL_HIP(gemv_rows(wt, pro, EPI_STORE, p, rows, s));
        }
    }
    if (d.rope_theta > 0.0f)  // block row k of sequence b at position len[b] + k
        DFL_HIP(launch_rope_block(w.qkv, d.wdtype == DFLASH_F32, qkv_rows, kv->len, B, d.gamma, d.hq, d.hkv, d.hd,
                                  rope_freqs(d.hd, d.rope_theta), s));
    {  // O = softmax(Q [K_ctx; K_b]^T / sqrt(hd)) [V_ctx; V_b]
        AttnParams a;
        std::memset(&a, 0, sizeof(a));
        a.qkv = w.qkv;
        a.qkv_ld = qkv_rows;
        const size_t esz = kv->dtype == DFLASH_F32 ? 4 : 2;
        const size_t layer_bytes = (size_t)kv->B * d.hkv * kv->cap * d.hd * esz;
        a.kcache = static_cast<const char*>(kv->k) + (size_t)i * layer_bytes;
        a.vcache = static_cast<const char*>(kv->v) + (size_t)i * layer_bytes;
        a.len = kv->len;
        a.B = B;
        a.hq = d.hq;
        a.hkv = d.hkv;
        a.hd = d.hd;
        a.gamma = d.gamma;
        a.cap = kv->cap;
        a.window = d.window;
        a.nsplit = w.nsplit;
        a.nparts = w.nparts;
        a.kv_f32 = kv->dtype == DFLASH_F32;
        a.scale = 1.0f / sqrtf((float)d.hd);
        a.part = w.part;
        a.vblk = w.vt;
        a.out = w.o;
        a.out_ld = d.hq * d.hd;
        a.round_out = d.wdtype == DFLASH_F32 ? 0 : 1;
        DFL_HIP(launch_attention(a, s));
    }
    *an_ready = false;
    if (w.skinny) return skinny_out_ffn(M, i, h, rows, w, s, next_gain, an_ready);
    const bool pn = prenorm(d);
    bool ffn_ready = false;
    {  // H += O W_o^T
        GemvParams p = base_params(d);
        p.w[0] = wptr(L.w_o);
        p.N = d.d;
        p.K = d.hq * d.hd;
        p.rpw = rpw_for(p.N, d.wdtype);
        p.x = w.o;
        p.x_ld = d.hq * d.hd;
        p.out = h;
        p.out_ld = d.d;
        // a split reduce also writes the FFN's normalised rows
        DFL_HIP(gemv_plain(d, wt, EPI_RESID, p, rows, w.rsp, s, pn ? L.ffn_norm : nullptr, w.an, &ffn_ready));
    }
    {  // A = act(n2 W_gate^T) * (n2 W_up^T), n2 = RMSNorm(H; ffn_norm)
        GemvParams p = base_params(d);
        p.w[0] = wptr(L.w_gate_up);
        p.N = 2 * d.F;
        p.F = d.F;
        p.K = d.d;
        p.rpw = d.F >= 8192 ? 4 : 2;
        p.act = d.act;
        p.x = h;
        p.x_ld = d.d;
        p.gain[0] = L.ffn_norm;
        p.out = w.a;
        p.out_ld = d.F;
        int pro = PRO_NORM;
        if (pn) {
            if (!ffn_ready) DFL_HIP(norm_rows(h, rows, d.d, L.ffn_norm, d.eps, w.an, s));
            p.x = reinterpret_cast<const float*>(w.an);
            pro = PRO_PLAIN;
        }
        if (pro == PRO_PLAIN)
            DFL_HIP(gemv_plain(d, wt, EPI_GATED, p, rows, w.rsp, s));
        else
            DFL_HIP(gemv_rows(wt, pro, EPI_GATED, p, rows, s));
    }
    {  // H += A W_down^T
        GemvParams p = base_params(d);
        p.w[0] = wptr(L.w_down);
        p.N = d.d;
        p.K = d.F;
        p.rpw = rpw_for(p.N, d.wdtype);
        p.x = w.a;
        p.x_ld = d.F;
        p.out = h;
        p.out_ld = d.d;
        // a split reduce also writes the next projection's normalised rows
        DFL_HIP(gemv_plain(d, wt, EPI_RESID, p, rows, w.rsp, s, pn ? next_gain : nullptr, w.an, an_ready));
    }
    return DFLASH_OK;
}

int lm_head(const dflash_weight& E, const void* y, int y_f32, int rows, int H, int V, int32_t* ids, float* maxl,
            float* pv, int32_t* pi, hipStream_t s, float* i4part = nullptr, size_t i4part_bytes = 0) {
    if (E.dtype == DFLASH_INT4G64 && !y_f32 && i4mm_ok(H, rows) && i4part) {
        // int4 head on matrix cores: split-K partial logits, then the ordered split argmax
        int ns = 1, ks = 0;
        i4mm_split(H, &ns, &ks);
        if ((size_t)ns * rows * V * 4 <= i4part_bytes) {
            I4Params q;
            std::memset(&q, 0, sizeof(q));
            q.codes[0] = static_cast<const uint32_t*>(E.data);
            q.scales[0] = static_cast<const uint16_t*>(E.scales);
            q.biases[0] = static_cast<const uint16_t*>(E.biases);
            q.layers = 1;
            q.N = V;
            q.K = H;
            q.a = static_cast<const uint16_t*>(y);
            q.a_ld = H;
            q.M = rows;
            q.nsplit = ns;
            q.kslice = ks;
            q.part = i4part;
            DFL_HIP(launch_i4mm(q, s));
            const int nb = i4_argmax_blocks(V);
            DFL_HIP(launch_i4_split_argmax(i4part, ns, rows, V, pv, pi, nb, s));
            DFL_HIP(launch_argmax_merge(pv, pi, nb, rows, ids, maxl, s));
            return DFLASH_OK;
        }
    }
    if (lm_head_skinny(E.dtype, y_f32, rows, H)) {
        // matrix cores: one pass over the head for all rows, a (max, index) partial per row and tile
        SkinnyParams p = skinny_params(E, static_cast<const uint16_t*>(y), H, V, H, nullptr);
        p.part_val = pv;
        p.part_idx = pi;
        DFL_HIP(skinny_rows(SK_ARGMAX, p, rows, s));
        DFL_HIP(launch_argmax_merge(pv, pi, skinny_tiles(SK_ARGMAX, V), rows, ids, maxl, s));
        return DFLASH_OK;
    }
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.w[0] = wptr(E);
    p.N = V;
    p.K = H;
    p.rpw = lm_rpw(wtype_of(E.dtype));
    p.max_wgs = lm_wgs(wtype_of(E.dtype));
    p.taps[0] = y;
    p.tap_ld = H;
    p.H = H;
    p.src_f32 = y_f32;
    p.nblocks = lm_nblocks(V, H, wtype_of(E.dtype), rows < 8 ? rows : 8);
    p.part_val = pv;
    p.part_idx = pi;
    DFL_HIP(gemv_rows(wtype_of(E.dtype), PRO_TAPS, EPI_ARGMAX, p, rows, s));
    DFL_HIP(launch_argmax_merge(pv, pi, p.nblocks, rows, ids, maxl, s));
    return DFLASH_OK;
}

// block init and every layer: H_d in w.hd; *an_ready says whether w.an holds the out
// projection's normalised rows
int forward_backbone(const dflash_model* M, const int32_t* anchor_ids, const dflash_kv* kv, int B, const Ws& w,
                     hipStream_t s, bool* an_ready, const CtxRows* ctx = nullptr) {
    const dflash_dims& d = M->dims;
    const int wt = wtype_of(d.wdtype);
    bool an_init = false;
    const bool init_sk = w.skinny && d.wdtype == DFLASH_BF16 && M->embed_in.dtype == DFLASH_BF16 &&
                         M->tok_proj.dtype == DFLASH_BF16 && B >= DFL_SKINNY_MIN_ROWS && d.H % kSkinnyK == 0 &&
                         (int64_t)d.gamma * d.d >= d.H;
    if (init_sk) {
        // 16 or more sequences on matrix cores: the anchors' embeddings gathered into w.an
        // (B rows of H; it holds B * gamma rows of d), their tok_proj product as row 0 of each
        // block, the block positions added and the mask rows written
        DFL_HIP(launch_gather_rows(static_cast<const uint16_t*>(M->embed_in.data), M->embed_in.rows, anchor_ids, B,
                                   d.H, w.an, s));
        SkinnyParams p = skinny_params(M->tok_proj, w.an, d.H, d.d, d.H, w.skp);
        if (B <= kSkinnyRows && d.d % 4 == 0 && d.d <= kNormMaxK) {
            // the product's split partials, then one kernel for the block rows and the first
            // layer's RMSNorm (the norm of the out projection when there are no layers)
            int ns = 1, ks = 0;
            skinny_split(SK_PARTIAL, d.d, d.H, 1, &ns, &ks);
            DFL_HIP(skinny_rows(SK_PARTIAL, p, B, s));
            DFL_HIP(launch_block_norm(w.skp, ns, B, d.gamma, d.d, w.hd, static_cast<const uint16_t*>(M->block_pos),
                                      static_cast<const uint16_t*>(M->mask_emb),
                                      d.nl > 0 ? M->layers[0].attn_norm : M->out_norm, 0, d.eps, w.an, s));
            an_init = true;
        } else {
            p.out = w.hd;
            p.out_ld = (int64_t)d.gamma * d.d;
            DFL_HIP(skinny_rows(SK_STORE, p, B, s));
            DFL_HIP(launch_block_fill(w.hd, B, d.gamma, d.d, M->block_pos, M->mask_emb, 0, s));
        }
    } else {  // block rows: E_in[anchor] tok_proj^T + block_pos[0]; mask_emb[k-1] + block_pos[k]
        GemvParams p = base_params(d);
        p.w[0] = wptr(M->tok_proj);
        p.N = d.d;
        p.K = d.H;
        p.rpw = rpw_for(p.N, d.wdtype);
        p.ids = anchor_ids;
        p.table = wptr(M->embed_in);
        p.table_type = wtype_of(M->embed_in.dtype);
        p.table_rows = M->embed_in.rows;
        p.out = w.hd;
        p.block_pos = M->block_pos;
        p.mask_emb = M->mask_emb;
        p.gamma = d.gamma;
        p.seq_base = 0;
        DFL_HIP(gemv_rows(wt, PRO_GATHER, EPI_BLOCKINIT, p, B, s));
    }
    *an_ready = an_init;  // w.an holds the next projection's normalised rows
    for (int i = 0; i < d.nl; ++i)
        DFL_TRY(run_layer(M, i, w.hd, kv, B, w, s, i + 1 < d.nl ? M->layers[i + 1].attn_norm : M->out_norm,
                          an_ready, ctx));
    return DFLASH_OK;
}

// Y = bf16(bf16(RMSNorm(H_d; out_norm)) out_proj^T) into y (fp32 throughout for fp32 models).
// rows_in: the normalised rows already computed (bf16, fp32 for fp32 models), or null
int forward_out(const dflash_model* M, int B, const Ws& w, hipStream_t s, bool an_ready, const void* rows_in,
                float* y) {
    const dflash_dims& d = M->dims;
    const int wt = wtype_of(d.wdtype);
    const int rows = B * d.gamma;
    if (w.skinny) {
        const uint16_t* a = static_cast<const uint16_t*>(rows_in);
        if (!a) {
            if (!an_ready) DFL_HIP(norm_rows(w.hd, rows, d.d, M->out_norm, d.eps, w.an, s));
            a = w.an;
        }
        SkinnyParams p = skinny_params(M->out_proj, a, d.d, d.H, d.d, w.skp);
        p.out = y;
        p.out_ld = d.H;
        p.out_bf16 = 1;
        DFL_HIP(skinny_rows(SK_STORE, p, rows, s));
        return DFLASH_OK;
    }
    GemvParams p = base_params(d);
    p.w[0] = wptr(M->out_proj);
    p.N = d.H;
    p.K = d.d;
    p.rpw = rpw_for(p.N, d.wdtype);
    p.x = w.hd;
    p.x_ld = d.d;
    p.gain[0] = M->out_norm;
    p.out = y;
    p.out_ld = d.H;
    p.out_bf16 = d.wdtype == DFLASH_F32 ? 0 : 1;
    if (rows_in) {
        p.x = static_cast<const float*>(rows_in);  // bf16 rows unless fp32 model (src_f32)
        DFL_HIP(gemv_plain(d, wt, EPI_STORE, p, rows, w.rsp, s));
    } else if (prenorm(d)) {
        if (!an_ready) DFL_HIP(norm_rows(w.hd, rows, d.d, M->out_norm, d.eps, w.an, s));
        p.x = reinterpret_cast<const float*>(w.an);
        DFL_HIP(gemv_plain(d, wt, EPI_STORE, p, rows, w.rsp, s));
    } else {
        DFL_HIP(gemv_rows(wt, PRO_NORM, EPI_STORE, p, rows, s));
    }
    return DFLASH_OK;
}

// the borrowed head's logits of `rows` rows, fp32 [rows, V] (matrix cores for 16 or more bf16
// rows; part holds their split-K partial sums for a short vocabulary)
int lm_head_store(const dflash_weight& E, const void* y, int y_f32, int rows, int H, int V, float* out, float* part,
                  hipStream_t s) {
    if (lm_head_skinny(E.dtype, y_f32, rows, H)) {
        SkinnyParams p = skinny_params(E, static_cast<const uint16_t*>(y), H, V, H, part);
        p.out = out;
        p.out_ld = V;
        p.out_bf16 = 0;
        DFL_HIP(skinny_rows(SK_STORE, p, rows, s));
        return DFLASH_OK;
    }
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.w[0] = wptr(E);
    p.N = V;
    p.K = H;
    p.rpw = rpw_for(V, E.dtype);
    p.max_wgs = DFL_SMALL_WGS;
    p.taps[0] = y;
    p.tap_ld = H;
    p.H = H;
    p.src_f32 = y_f32;
    p.out = out;
    p.out_ld = V;
    DFL_HIP(gemv_rows(wtype_of(E.dtype), PRO_TAPS, EPI_STORE, p, rows, s));
    return DFLASH_OK;
}

// one Markov step: per row m < B, the (max, lowest index) over v of
// base[m * base_ld + v] + e1[m] . w2t[v], as partials [B][*nblocks]
int markov_argmax(const dflash_weight& w2t, const void* e1, int f32, int B, int r, int V, const float* base,
                  int64_t base_ld, float* pv, int32_t* pi, int* nblocks, hipStream_t s) {
    if (lm_head_skinny(w2t.dtype, f32, B, r)) {
        SkinnyParams p = skinny_params(w2t, static_cast<const uint16_t*>(e1), r, V, r, nullptr);
        p.part_val = pv;
        p.part_idx = pi;
        p.base = base;
        p.base_ld = base_ld;
        *nblocks = skinny_tiles(SK_ARGMAX, V);
        DFL_HIP(skinny_rows(SK_ARGMAX, p, B, s));
        return DFLASH_OK;
    }
    GemvParams p;
    std::memset(&p, 0, sizeof(p));
    p.w[0] = wptr(w2t);
    p.N = V;
    p.K = r;
    p.rpw = lm_rpw(wtype_of(w2t.dtype));
    p.max_wgs = lm_wgs(wtype_of(w2t.dtype));
    p.taps[0] = e1;
    p.tap_ld = r;
    p.H = r;
    p.src_f32 = f32;
    p.nblocks = lm_nblocks(V, r, wtype_of(w2t.dtype), B < 8 ? B : 8);
    p.part_val = pv;
    p.part_idx = pi;
    p.base = base;
    p.base_ld = base_ld;
    *nblocks = p.nblocks;
    DFL_HIP(gemv_rows(wtype_of(w2t.dtype), PRO_TAPS, EPI_ARGMAX, p, B, s));
    return DFLASH_OK;
}

// workspace of the round: the forward's own (which the context projection and a separate
// append also use), then the new rows' H_ctx [B (gamma + 1)][d] fp32 and the lengths before
// the round [B]
struct Round {
    Ws fw;
    float* h_ctx;
    int32_t* len_old;
    size_t total;
};
Round round_layout(const dflash_dims& d, int B, int cap, void* wsp) {
    Round rd{};
    char* c = static_cast<char*>(wsp);
    rd.fw = ws_layout(d, B, cap, wsp);
    size_t off = align_up(rd.fw.total);
    rd.h_ctx = c ? reinterpret_cast<float*>(c + off) : nullptr;
    off += align_up((size_t)B * (d.gamma + 1) * d.d * 4);
    rd.len_old = c ? reinterpret_cast<int32_t*>(c + off) : nullptr;
    off += align_up((size_t)B * 4);
    rd.total = off;
    return rd;
}

// workspace of the DSpark forward: the forward's own, then the base logits [B gamma][V] fp32,
// the block rows [B gamma][d] (4 bytes each), the Markov operand rows [B][r] (4 bytes each),
// the step partials [B][tiles] (value, index), pruning lengths [B] when the caller passes
// none, and the split-K partials of a matrix-core head store over a short vocabulary
struct Dspark {
    Ws fw;
    float* base;
    void* hout;
    void* e1;
    float* pv;
    int32_t* pi;
    int32_t* lens;
    float* skp;
    size_t total;
};
Dspark dspark_layout(const dflash_dims& d, int r, int B, int cap, void* wsp) {
    Dspark ds{};
    char* c = static_cast<char*>(wsp);
    ds.fw = ws_layout(d, B, cap, wsp);
    size_t off = align_up(ds.fw.total);
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return c ? c + o : nullptr;
    };
    const size_t rows = (size_t)B * d.gamma;
    ds.base = reinterpret_cast<float*>(take(rows * d.V * 4));
    ds.hout = take(rows * d.d * 4);
    ds.e1 = take((size_t)B * r * 4);
    const size_t nb = lm_tiles_max(d.V);
    ds.pv = reinterpret_cast<float*>(take((size_t)B * nb * 4));
    ds.pi = reinterpret_cast<int32_t*>(take((size_t)B * nb * 4));
    ds.lens = reinterpret_cast<int32_t*>(take((size_t)B * 4));
    int ns = 1, ks = 0;
    skinny_split(SK_STORE, d.V, d.H, 1, &ns, &ks);
    const size_t r0 = rows < (size_t)kSkinnyRows ? rows : (size_t)kSkinnyRows;
    ds.skp = reinterpret_cast<float*>(take(ns > 1 ? (size_t)ns * r0 * d.V * 4 : 0));
    ds.total = off;
    return ds;
}

}  // namespace

int dfl::api_gate() { return gate(); }
void dfl::api_count_invocation() { g_invocations++; }

uint64_t* dfl::trace_launch(int kind, const char* name, int64_t workgroups, double bytes, double ctx_row_bytes) {
    static_assert(TRACE_LM_HEAD == DFLASH_TRACE_LM_HEAD && TRACE_ATTENTION == DFLASH_TRACE_ATTENTION &&
                      TRACE_PROJECTIONS == DFLASH_TRACE_PROJECTIONS,
                  "trace kinds");
    if (!(g_trace.kinds.load(std::memory_order_relaxed) & kind)) return nullptr;
    std::lock_guard<std::mutex> lk(g_trace.mu);
    if (!(g_trace.kinds.load() & kind) || !g_trace.stamps || g_trace.cursor + 2 * workgroups > g_trace.capacity)
        return nullptr;
    dflash_trace_record r;
    std::memset(&r, 0, sizeof(r));
    std::strncpy(r.kernel, name, sizeof(r.kernel) - 1);
    r.kind = kind;
    r.workgroups = (int32_t)workgroups;
    r.offset = g_trace.cursor;
    r.bytes = bytes;
    r.ctx_row_bytes = ctx_row_bytes;
    g_trace.records.push_back(r);
    uint64_t* slice = g_trace.stamps + g_trace.cursor;
    g_trace.cursor += 2 * workgroups;
    return slice;
}

// ===========================================================================

extern "C" {

size_t dflash_workspace_bytes(const dflash_dims* dims, int32_t B, int32_t cap) {
    if (check_dims(dims) == DFLASH_EINVAL || B <= 0 || cap < 0) return 0;
    return ws_layout(*dims, B, cap, nullptr).total;
}

int dflash_query(const dflash_dims* dims) {
    DFL_TRY(check_dims(dims));
    return gate();
}

const char* dflash_status_string(int status) {
    switch (status) {
        case DFLASH_OK: return "ok";
        case DFLASH_DECLINED: return "declined: request not served by this library (fall back to plain decoding)";
        case DFLASH_EINVAL: return "invalid argument";
        case DFLASH_ENOSPC: return "workspace or KV capacity too small";
        case DFLASH_EHIP: return "HIP launch failure";
    }
    return "unknown status";
}

uint64_t dflash_invocations(void) { return g_invocations.load(); }

void dflash_trace_begin(int32_t kinds, uint64_t* stamps, int64_t capacity) {
    std::lock_guard<std::mutex> lk(g_trace.mu);
    const bool on = stamps && capacity > 0 && kinds > 0;
    g_trace.stamps = on ? stamps : nullptr;
    g_trace.capacity = on ? capacity : 0;
    g_trace.cursor = 0;
    g_trace.records.clear();
    g_trace.kinds.store(on ? (kinds & (DFLASH_TRACE_LM_HEAD | DFLASH_TRACE_ATTENTION | DFLASH_TRACE_PROJECTIONS)) : 0);
}

int32_t dflash_trace_end(dflash_trace_record* records, int32_t capacity) {
    std::lock_guard<std::mutex> lk(g_trace.mu);
    const int32_t n = (int32_t)g_trace.records.size();
    for (int32_t i = 0; i < n && i < capacity && records; ++i) records[i] = g_trace.records[i];
    g_trace.kinds.store(0);
    g_trace.stamps = nullptr;
    g_trace.capacity = g_trace.cursor = 0;
    g_trace.records.clear();
    return n;
}

int32_t dflash_lm_head_workgroups(int32_t V, int32_t H, int32_t dtype, int32_t M, int32_t y_dtype, int32_t* launches) {
    if (V <= 0 || H <= 0 || M <= 0 || (dtype != DFLASH_F32 && dtype != DFLASH_BF16 && dtype != DFLASH_INT4G64) ||
        (y_dtype != DFLASH_F32 && y_dtype != DFLASH_BF16))
        return 0;
    if (lm_head_skinny(dtype, y_dtype == DFLASH_F32, M, H)) {
        if (launches) *launches = (M + kSkinnyRows - 1) / kSkinnyRows;
        return skinny_tiles(SK_ARGMAX, V);
    }
    if (launches) *launches = (M + 7) / 8;
    return lm_nblocks(V, H, wtype_of(dtype), M < 8 ? M : 8);
}

// The rate is measured: two readings of the device clock 100 ms apart on the host's steady
// clock (the runtime's reported rate has disagreed with the counter on some devices). Once
// per device and process; the readings run on the null stream and synchronise the device.
double dflash_wall_clock_hz(void) {
    static std::mutex mu;
    static double rate[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0.0;
    std::lock_guard<std::mutex> lock(mu);
    if (rate[dev] > 0.0) return rate[dev];
    uint64_t* buf = nullptr;
    if (hipMalloc(&buf, 2 * sizeof(uint64_t)) != hipSuccess) return 0.0;
    uint64_t ticks[2] = {0, 0};
    double secs = 0.0;
    bool ok = launch_wall_clock(buf, nullptr) == hipSuccess && hipDeviceSynchronize() == hipSuccess;
    const auto t0 = std::chrono::steady_clock::now();
    if (ok) {
        std::this_thread::sleep_for(std::chrono::milliseconds(100));
        secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        ok = launch_wall_clock(buf + 1, nullptr) == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
             hipMemcpy(ticks, buf, sizeof(ticks), hipMemcpyDeviceToHost) == hipSuccess;
    }
    (void)hipFree(buf);
    if (!ok || ticks[1] <= ticks[0] || secs <= 0.0) return 0.0;
    rate[dev] = (double)(ticks[1] - ticks[0]) / secs;
    return rate[dev];
}

double dflash_wall_clock_hz_reported(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0.0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
    return 1000.0 * khz;
}

int dflash_context_project(const dflash_model* M, const void* const* taps, int64_t tap_ld, int32_t n, float* h_ctx,
                           void* ws, size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (n < 0 || !taps || (n > 0 && !h_ctx) || tap_ld < d.H) return DFLASH_EINVAL;
    for (int j = 0; j < d.m; ++j)
        if (!taps[j]) return DFLASH_EINVAL;
    for (int j = 0; j < d.m; ++j)
        if ((reinterpret_cast<uintptr_t>(taps[j]) & 15) || (tap_ld % 8)) return DFLASH_DECLINED;
    DFL_TRY(gate());
    if (n == 0) return DFLASH_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    GemvParams p = base_params(d);
    p.w[0] = wptr(M->w_c);
    p.N = d.d;
    p.K = d.m * d.H;
    p.rpw = rpw_for(p.N, d.wdtype);
    for (int j = 0; j < d.m; ++j) p.taps[j] = taps[j];
    p.tap_ld = tap_ld;
    p.H = d.H;
    p.src_f32 = d.wdtype == DFLASH_F32;
    p.out = h_ctx;
    p.out_ld = d.d;
    p.round_out = 0;  // P stays fp32; the norm follows
    const int splits = ctx_splits(d);
    const size_t part_bytes = (size_t)splits * n * d.d * 4;
    const size_t sk_bytes = ctx_project_skinny_bytes(d, n);
    if (sk_bytes > 0 && ws && aligned16(ws) && ws_bytes >= sk_bytes) {
        // a round's rows: P = [T_1 .. T_m] W_c^T on matrix cores, split-K partials in ws,
        // added in split order by the norm
        SkinnyParams q;
        std::memset(&q, 0, sizeof(q));
        q.M = n;
        q.N = d.d;
        q.K = d.m * d.H;
        for (int j = 0; j < d.m; ++j) q.a_seg[j] = static_cast<const uint16_t*>(taps[j]);
        q.a = q.a_seg[0];
        q.a_ld = tap_ld;
        q.seg_k = d.H;
        q.w[0] = static_cast<const uint16_t*>(M->w_c.data);
        q.layers = 1;
        q.part = static_cast<float*>(ws);
        skinny_split(SK_PARTIAL, q.N, q.K, 1, &q.nsplit, &q.kslice);
        DFL_HIP(launch_skinny(SK_PARTIAL, q, s));
        DFL_HIP(launch_rownorm(q.part, q.nsplit, (int64_t)n * d.d, h_ctx, n, d.d, M->ctx_norm, 0, d.eps, s));
    } else if (n >= DFL_GEMM_MIN_ROWS && d.wdtype == DFLASH_BF16 && d.H % 64 == 0 && d.m <= kMaxTaps) {
        // prefill: P = [T_1 .. T_m] W_c^T on matrix cores, then the norm in place
        GemmParams g;
        std::memset(&g, 0, sizeof(g));
        g.M = n;
        g.N = d.d;
        g.K = d.m * d.H;
        for (int j = 0; j < d.m; ++j) g.a[j] = static_cast<const uint16_t*>(taps[j]);
        g.a_ld = tap_ld;
        g.seg_k = d.H;
        g.b[0] = static_cast<const uint16_t*>(M->w_c.data);
        g.c = h_ctx;
        g.c_ld = d.d;
        DFL_HIP(launch_gemm(GEMM_A_TAPS, GEMM_EPI_F32, g, 1, s));
        DFL_HIP(launch_rownorm(h_ctx, 1, 0, h_ctx, n, d.d, M->ctx_norm, 0, d.eps, s));
    } else if (i4_prefill_proj_bytes(d, n) > 0 && ws && aligned16(ws) && ws_bytes >= i4_prefill_proj_bytes(d, n)) {
        // int4 prefill: W_c expanded into bf16 high and low parts [d, 2 m H] in ws, then
        // P = [T_1 .. T_m | T_1 .. T_m] [W_hi | W_lo]^T on matrix cores, then the norm in place
        uint16_t* wx = static_cast<uint16_t*>(ws);
        DFL_HIP(launch_i4_expand(static_cast<const uint32_t*>(M->w_c.data),
                                 static_cast<const uint16_t*>(M->w_c.scales),
                                 static_cast<const uint16_t*>(M->w_c.biases), d.m * d.H, 0, d.d, wx, s));
        GemmParams g;
        std::memset(&g, 0, sizeof(g));
        g.M = n;
        g.N = d.d;
        g.K = 2 * d.m * d.H;
        g.a_period = d.m * d.H;
        for (int j = 0; j < d.m; ++j) g.a[j] = static_cast<const uint16_t*>(taps[j]);
        g.a_ld = tap_ld;
        g.seg_k = d.H;
        g.b[0] = wx;
        g.c = h_ctx;
        g.c_ld = d.d;
        DFL_HIP(launch_gemm(GEMM_A_TAPS, GEMM_EPI_F32, g, 1, s));
        DFL_HIP(launch_rownorm(h_ctx, 1, 0, h_ctx, n, d.d, M->ctx_norm, 0, d.eps, s));
    } else if (M->w_c.dtype == DFLASH_INT4G64 && ctx_i4_bytes(d, n) > 0 && ws && aligned16(ws) &&
               ws_bytes >= ctx_i4_bytes(d, n)) {
        // int4 W_c, up to 16 rows: matrix-core K ranges (each inside one tap buffer), split
        // partials in ws added in split order by the norm
        I4Params q;
        std::memset(&q, 0, sizeof(q));
        q.codes[0] = static_cast<const uint32_t*>(M->w_c.data);
        q.scales[0] = static_cast<const uint16_t*>(M->w_c.scales);
        q.biases[0] = static_cast<const uint16_t*>(M->w_c.biases);
        q.layers = 1;
        q.N = d.d;
        q.K = d.m * d.H;
        for (int j = 0; j < d.m; ++j) q.a_seg[j] = static_cast<const uint16_t*>(taps[j]);
        q.seg_k = d.H;
        q.a_ld = tap_ld;
        q.M = n;
        i4mm_split(q.K, &q.nsplit, &q.kslice);
        q.part = static_cast<float*>(ws);
        DFL_HIP(launch_i4mm(q, s));
        // the K ranges' sums over many workgroups (split order), then the norm in place
        SkinnyParams r;
        std::memset(&r, 0, sizeof(r));
        r.M = n;
        r.N = d.d;
        r.nsplit = q.nsplit;
        r.part = q.part;
        r.out = h_ctx;
        r.out_ld = d.d;
        DFL_HIP(launch_split_reduce(SK_STORE, r, s));
        DFL_HIP(launch_rownorm(h_ctx, 1, 0, h_ctx, n, d.d, M->ctx_norm, 0, d.eps, s));
    } else if (n <= 8 && splits > 1 && ws && ws_bytes >= part_bytes) {
        // few rows: split the long reduction over more workgroups; partials in ws
        p.rpw = 4;
        p.kslice = (p.K + splits - 1) / splits;
        p.kslice = (p.kslice + 511) / 512 * 512;
        p.ksplit = (p.K + p.kslice - 1) / p.kslice;  // every range non-empty
        p.out = static_cast<float*>(ws);
        p.split_stride = (int64_t)n * d.d;
        DFL_HIP(gemv_rows(wtype_of(d.wdtype), PRO_TAPS, EPI_STORE, p, n, s));
        DFL_HIP(launch_rownorm(static_cast<float*>(ws), p.ksplit, (int64_t)n * d.d, h_ctx, n, d.d, M->ctx_norm,
                               d.wdtype == DFLASH_F32, d.eps, s));
    } else {
        DFL_HIP(gemv_rows(wtype_of(d.wdtype), PRO_TAPS, EPI_STORE, p, n, s, 1, 32));
        DFL_HIP(launch_rownorm(h_ctx, 1, 0, h_ctx, n, d.d, M->ctx_norm, d.wdtype == DFLASH_F32, d.eps, s));
    }
    g_invocations++;
    return DFLASH_OK;
}

int dflash_ctx_kv_append(const dflash_model* M, const float* h_ctx, int32_t n, const int32_t* row_offsets,
                         const int32_t* counts, const dflash_kv* kv, void* ws, size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (n < 0 || (n > 0 && !h_ctx) || !row_offsets || !kv) return DFLASH_EINVAL;
    DFL_TRY(check_kv(kv, d, kv->B));
    DFL_TRY(gate());
    if (n == 0) return DFLASH_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d.nl == 0) {  // no layer caches: only the held-row counts advance
        DFL_HIP(launch_advance_len(kv->len, row_offsets, counts, kv->B, kv->cap, s));
        g_invocations++;
        return DFLASH_OK;
    }
    const size_t sk_bytes = kv_append_skinny_bytes(d, n);
    if (sk_bytes > 0 && ws && aligned16(ws) && ws_bytes >= sk_bytes) {
        // a round's rows: every layer's bf16(RMSNorm(h_ctx; attn_norm_i)) into ws, then
        // [K | V] = those rows [W_K | W_V]^T for all layers in one matrix-core launch
        // (grid.z = layer), scattered into the cache
        uint16_t* an = static_cast<uint16_t*>(ws);
        NormRowsParams q;
        std::memset(&q, 0, sizeof(q));
        q.x = h_ctx;
        q.x_ld = d.d;
        q.rows = n;
        q.K = d.d;
        q.layers = d.nl;
        q.eps = d.eps;
        for (int i = 0; i < d.nl; ++i) q.gain[i] = M->layers[i].attn_norm;
        q.dst = an;
        q.dst_ld = d.d;
        q.dst_layer_stride = (int64_t)n * d.d;
        DFL_HIP(launch_norm_rows(q, s));
        SkinnyParams p;
        std::memset(&p, 0, sizeof(p));
        p.M = n;
        p.N = 2 * d.hkv * d.hd;
        p.K = d.d;
        p.a = an;
        p.a_ld = d.d;
        p.a_layer_stride = (int64_t)n * d.d;
        for (int i = 0; i < d.nl; ++i) p.w[i] = static_cast<const uint16_t*>(M->layers[i].w_qkv.data);
        p.w_row0 = (int64_t)d.hq * d.hd;  // the K and V rows of the fused QKV matrix
        p.layers = d.nl;
        p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + kv_append_norm_bytes(d, n));
        p.kcache = static_cast<uint16_t*>(kv->k);
        p.vcache = static_cast<uint16_t*>(kv->v);
        p.len = kv->len;
        p.row_offsets = row_offsets;
        p.counts = counts;
        p.B = kv->B;
        p.hkv = d.hkv;
        p.hd = d.hd;
        p.cap = kv->cap;
        p.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
        skinny_split(SK_KV, p.N, p.K, p.layers, &p.nsplit, &p.kslice);
        DFL_HIP(launch_skinny(SK_KV, p, s));
        DFL_TRY(append_done(M, kv, row_offsets, counts, n, s));
        g_invocations++;
        return DFLASH_OK;
    }
    if (i4_prefill_kv_bytes(d, n) > 0 && ws && aligned16(ws) && aligned16(h_ctx) && ws_bytes >= i4_prefill_kv_bytes(d, n)) {
        // int4 prefill: every layer's K and V rows expanded into bf16 high and low parts
        // [2 hkv hd, 2 d] in ws, the per-row RMS factors after them, then every layer's
        // [K | V] = [N | N] [W_hi | W_lo]^T (N = bf16(RMSNorm(h_ctx; attn_norm_i)) staged on
        // the fly) as one matrix-core GEMM over all layers, scattered into the cache
        const int kvr = 2 * d.hkv * d.hd;
        uint16_t* wx = static_cast<uint16_t*>(ws);
        const int64_t layer_elems = (int64_t)kvr * 2 * d.d;
        for (int i = 0; i < d.nl; ++i) {
            const dflash_weight& w = M->layers[i].w_qkv;
            DFL_HIP(launch_i4_expand(static_cast<const uint32_t*>(w.data), static_cast<const uint16_t*>(w.scales),
                                     static_cast<const uint16_t*>(w.biases), d.d, (int64_t)d.hq * d.hd, kvr,
                                     wx + i * layer_elems, s));
        }
        float* rinv = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)d.nl * layer_elems * 2));
        DFL_HIP(launch_row_rinv(h_ctx, d.d, n, d.d, d.eps, rinv, s));
        GemmParams g;
        std::memset(&g, 0, sizeof(g));
        g.M = n;
        g.N = kvr;
        g.K = 2 * d.d;
        g.a_period = d.d;
        g.x = h_ctx;
        g.a_ld = d.d;
        g.rinv = rinv;
        g.gain_f32 = 0;
        for (int i = 0; i < d.nl; ++i) {
            g.b[i] = wx + i * layer_elems;
            g.gain[i] = M->layers[i].attn_norm;
        }
        g.kcache = kv->k;
        g.vcache = kv->v;
        g.len = kv->len;
        g.row_offsets = row_offsets;
        g.counts = counts;
        g.B = kv->B;
        g.hkv = d.hkv;
        g.hd = d.hd;
        g.cap = kv->cap;
        g.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
        DFL_HIP(launch_gemm(GEMM_A_NORM, GEMM_EPI_KV, g, d.nl, s));
        DFL_TRY(append_done(M, kv, row_offsets, counts, n, s));
        g_invocations++;
        return DFLASH_OK;
    }
    if (n >= DFL_GEMM_MIN_ROWS && d.wdtype == DFLASH_BF16 && d.d % 64 == 0 && d.d <= kNormMaxK && ws &&
        aligned16(ws) && aligned16(h_ctx) && ws_bytes >= kv_append_norm_bytes(d, n)) {
        // prefill with room for every layer's normalised rows: bf16(RMSNorm(h_ctx; attn_norm_i))
        // into ws (each fp32 row read once for all layers), then every layer's [K | V] = those
        // rows [W_K | W_V]^T as one matrix-core GEMM over all layers (grid.z = layer) on plain
        // bf16 A tiles
        uint16_t* an = static_cast<uint16_t*>(ws);
        NormRowsParams q;
        std::memset(&q, 0, sizeof(q));
        q.x = h_ctx;
        q.x_ld = d.d;
        q.rows = n;
        q.K = d.d;
        q.layers = d.nl;
        q.eps = d.eps;
        for (int i = 0; i < d.nl; ++i) q.gain[i] = M->layers[i].attn_norm;
        q.dst = an;
        q.dst_ld = d.d;
        q.dst_layer_stride = (int64_t)n * d.d;
        q.all_layers = 1;
        DFL_HIP(launch_norm_rows(q, s));
        GemmParams g;
        std::memset(&g, 0, sizeof(g));
        g.M = n;
        g.N = 2 * d.hkv * d.hd;
        g.K = d.d;
        g.a[0] = an;
        g.a_ld = d.d;
        g.a_layer_stride = (int64_t)n * d.d;
        g.seg_k = d.d;
        for (int i = 0; i < d.nl; ++i) g.b[i] = static_cast<const uint16_t*>(M->layers[i].w_qkv.data);
        g.b_row0 = (int64_t)d.hq * d.hd;  // the K and V rows of the fused QKV matrix
        g.kcache = kv->k;
        g.vcache = kv->v;
        g.len = kv->len;
        g.row_offsets = row_offsets;
        g.counts = counts;
        g.B = kv->B;
        g.hkv = d.hkv;
        g.hd = d.hd;
        g.cap = kv->cap;
        g.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
        DFL_HIP(launch_gemm(GEMM_A_TAPS, GEMM_EPI_KV, g, d.nl, s));
        DFL_TRY(append_done(M, kv, row_offsets, counts, n, s));
        g_invocations++;
        return DFLASH_OK;
    }
    if (n >= DFL_GEMM_MIN_ROWS && d.wdtype == DFLASH_BF16 && d.d % 64 == 0 && ws && aligned16(ws) &&
        ws_bytes >= (size_t)n * 4) {
        // prefill: per-row RMS factors into ws, then every layer's [K | V] = bf16(N) [W_K | W_V]^T
        // on matrix cores (grid.z = layer), scattered into the cache
        float* rinv = static_cast<float*>(ws);
        DFL_HIP(launch_row_rinv(h_ctx, d.d, n, d.d, d.eps, rinv, s));
        GemmParams g;
        std::memset(&g, 0, sizeof(g));
        g.M = n;
        g.N = 2 * d.hkv * d.hd;
        g.K = d.d;
        g.x = h_ctx;
        g.a_ld = d.d;
        g.rinv = rinv;
        g.gain_f32 = 0;
        for (int i = 0; i < d.nl; ++i) {
            g.b[i] = static_cast<const uint16_t*>(M->layers[i].w_qkv.data);
            g.gain[i] = M->layers[i].attn_norm;
        }
        g.b_row0 = (int64_t)d.hq * d.hd;  // the K and V rows of the fused QKV matrix
        g.kcache = kv->k;
        g.vcache = kv->v;
        g.len = kv->len;
        g.row_offsets = row_offsets;
        g.counts = counts;
        g.B = kv->B;
        g.hkv = d.hkv;
        g.hd = d.hd;
        g.cap = kv->cap;
        g.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
        DFL_HIP(launch_gemm(GEMM_A_NORM, GEMM_EPI_KV, g, d.nl, s));
        DFL_TRY(append_done(M, kv, row_offsets, counts, n, s));
        g_invocations++;
        return DFLASH_OK;
    }
    GemvParams p = base_params(d);
    for (int i = 0; i < d.nl; ++i) {
        p.w[i] = wptr(M->layers[i].w_qkv);
        p.gain[i] = M->layers[i].attn_norm;
    }
    int pro = PRO_NORM;
    if (prenorm(d) && ws && aligned16(ws) && ws_bytes >= kv_append_norm_bytes(d, n)) {
        // long rows: every layer's bf16(RMSNorm(h_ctx; attn_norm_i)) once into ws (one
        // launch, grid.y = layer); the GEMV then stages layer y's plain rows
        NormRowsParams q;
        std::memset(&q, 0, sizeof(q));
        q.x = h_ctx;
        q.x_ld = d.d;
        q.rows = n;
        q.K = d.d;
        q.layers = d.nl;
        q.eps = d.eps;
        for (int i = 0; i < d.nl; ++i) q.gain[i] = M->layers[i].attn_norm;
        q.dst = static_cast<uint16_t*>(ws);
        q.dst_ld = d.d;
        q.dst_layer_stride = (int64_t)n * d.d;
        DFL_HIP(launch_norm_rows(q, s));
        pro = PRO_PLAIN;
    }
    p.w_row0 = (int64_t)d.hq * d.hd;  // the K and V rows of the fused QKV matrix
    p.max_wgs = DFL_KV_WGS / d.nl > 0 ? DFL_KV_WGS / d.nl : 1;  // per layer (grid.y)
    p.N = 2 * d.hkv * d.hd;
    p.K = d.d;
    p.rpw = rpw_for(p.N, d.wdtype);
    p.x = pro == PRO_PLAIN ? static_cast<const float*>(ws) : h_ctx;  // bf16 rows for PRO_PLAIN
    p.x_ld = d.d;
    p.x_layer_stride = pro == PRO_PLAIN ? (int64_t)n * d.d : 0;
    p.kcache = kv->k;
    p.vcache = kv->v;
    p.len = kv->len;
    p.row_offsets = row_offsets;
    p.counts = counts;
    p.row_base = 0;
    p.B = kv->B;
    p.hkv = d.hkv;
    p.hd = d.hd;
    p.cap = kv->cap;
    p.kv_f32 = kv->dtype == DFLASH_F32;
    p.layer_stride = (int64_t)kv->B * d.hkv * kv->cap * d.hd;
    bool i4w = true;  // every layer's K/V weights int4-g64
    for (int i = 0; i < d.nl; ++i) i4w = i4w && M->layers[i].w_qkv.dtype == DFLASH_INT4G64;
    int split_ks = 0;
    const int split_ns = pro == PRO_PLAIN ? kv_append_gemv_split(d, n, &split_ks) : 1;
    if (pro == PRO_PLAIN && i4w && !p.kv_f32 && kv_i4_bytes(d, n) > 0 && ws_bytes >= kv_i4_bytes(d, n)) {
        // int4, up to 16 rows: every layer's [K | V] on matrix cores (grid.y = layer) as split
        // partials, then one reduce over all layers adds them in order and scatters the rows
        float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kv_append_norm_bytes(d, n));
        I4Params q;
        std::memset(&q, 0, sizeof(q));
        for (int i = 0; i < d.nl; ++i) {
            q.codes[i] = static_cast<const uint32_t*>(M->layers[i].w_qkv.data);
            q.scales[i] = static_cast<const uint16_t*>(M->layers[i].w_qkv.scales);
            q.biases[i] = static_cast<const uint16_t*>(M->layers[i].w_qkv.biases);
        }
        q.w_row0 = (int64_t)d.hq * d.hd;  // the K and V rows of the fused QKV matrix
        q.layers = d.nl;
        q.N = p.N;
        q.K = d.d;
        q.a = static_cast<const uint16_t*>(ws);  // each layer's normalised rows
        q.a_ld = d.d;
        q.a_layer_stride = (int64_t)n * d.d;
        q.M = n;
        i4mm_split(q.K, &q.nsplit, &q.kslice);
        q.part = part;
        DFL_HIP(launch_i4mm(q, s));
        SkinnyParams r;
        std::memset(&r, 0, sizeof(r));
        r.M = n;
        r.N = p.N;
        r.layers = d.nl;
        r.nsplit = q.nsplit;
        r.part = part;
        r.kcache = static_cast<uint16_t*>(kv->k);
        r.vcache = static_cast<uint16_t*>(kv->v);
        r.len = kv->len;
        r.row_offsets = row_offsets;
        r.counts = counts;
        r.row_base = 0;
        r.B = kv->B;
        r.cap = kv->cap;
        r.hkv = d.hkv;
        r.hd = d.hd;
        r.layer_stride = p.layer_stride;
        DFL_HIP(launch_split_reduce(SK_KV, r, s));
    } else if (split_ns > 1 && !p.kv_f32 && ws_bytes >= kv_append_split_bytes(d, n)) {
        // K ranges write fp32 partials (one set per layer), then one reduce over all layers
        // adds them in split order and scatters the rows into the caches
        float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + kv_append_norm_bytes(d, n));
        GemvParams q = p;
        q.ksplit = split_ns;
        q.kslice = split_ks;
        q.max_wgs = p.max_wgs / split_ns > 0 ? p.max_wgs / split_ns : 1;
        q.out = part;
        q.out_ld = p.N;
        q.split_stride = (int64_t)n * p.N;  // layer y, range z at (y * split_ns + z) * split_stride
        q.round_out = 0;
        q.out_bf16 = 0;
        q.vt = nullptr;
        DFL_HIP(gemv_rows(wtype_of(d.wdtype), PRO_PLAIN, EPI_STORE, q, n, s, d.nl));
        SkinnyParams r;
        std::memset(&r, 0, sizeof(r));
        r.M = n;
        r.N = p.N;
        r.layers = d.nl;
        r.nsplit = split_ns;
        r.part = part;
        r.kcache = static_cast<uint16_t*>(kv->k);
        r.vcache = static_cast<uint16_t*>(kv->v);
        r.len = kv->len;
        r.row_offsets = row_offsets;
        r.counts = counts;
        r.row_base = 0;
        r.B = kv->B;
        r.cap = kv->cap;
        r.hkv = d.hkv;
        r.hd = d.hd;
        r.layer_stride = p.layer_stride;
        DFL_HIP(launch_split_reduce(SK_KV, r, s));
    } else {
        DFL_HIP(gemv_rows(wtype_of(d.wdtype), pro, EPI_KV, p, n, s, d.nl, 32));
    }
    DFL_TRY(append_done(M, kv, row_offsets, counts, n, s));
    g_invocations++;
    return DFLASH_OK;
}

int dflash_draft_layer(const dflash_model* M, int32_t layer, float* h_block, const dflash_kv* kv, int32_t B,
                       void* ws, size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (layer < 0 || layer >= d.nl || !h_block || B <= 0) return DFLASH_EINVAL;
    DFL_TRY(check_kv(kv, d, B));
    const Ws w = ws_layout(d, B, kv->cap, ws);
    if (!ws || ws_bytes < w.total) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    bool an_ready = false;
    DFL_TRY(run_layer(M, layer, h_block, kv, B, w, static_cast<hipStream_t>(stream), nullptr, &an_ready));
    g_invocations++;
    return DFLASH_OK;
}

int dflash_draft_forward(const dflash_model* M, const int32_t* anchor_ids, const dflash_kv* kv, int32_t B,
                         int32_t* draft_ids, void* y_out, float* max_logit, void* ws, size_t ws_bytes,
                         void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (!anchor_ids || !draft_ids || B <= 0) return DFLASH_EINVAL;
    DFL_TRY(check_kv(kv, d, B));
    const Ws w = ws_layout(d, B, kv->cap, ws);
    if (!ws || ws_bytes < w.total) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool an_ready = false;
    DFL_TRY(forward_backbone(M, anchor_ids, kv, B, w, s, &an_ready));
    // Y written straight into y_out when the caller wants it (bf16 for bf16/int4 models,
    // fp32 for fp32 models)
    float* y = y_out ? static_cast<float*>(y_out) : w.y;
    DFL_TRY(forward_out(M, B, w, s, an_ready, nullptr, y));
    DFL_TRY(lm_head(M->lm_head, y, d.wdtype == DFLASH_F32, B * d.gamma, d.H, d.V, draft_ids, max_logit, w.lmv, w.lmi,
                    s, w.i4h, w.i4h_bytes));
    g_invocations++;
    return DFLASH_OK;
}

size_t dflash_round_workspace_bytes(const dflash_dims* dims, int32_t B, int32_t cap) {
    if (check_dims(dims) == DFLASH_EINVAL || B <= 0 || cap < 0) return 0;
    return round_layout(*dims, B, cap, nullptr).total;
}

int dflash_draft_round(const dflash_model* M, const void* const* taps, int64_t tap_ld, int32_t n,
                       const int32_t* row_offsets, const int32_t* counts, const dflash_kv* kv, int32_t B,
                       const int32_t* anchor_ids, int32_t* draft_ids, void* y_out, float* max_logit, void* ws,
                       size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (n < 0 || !taps || !row_offsets || !anchor_ids || !draft_ids || B <= 0) return DFLASH_EINVAL;
    DFL_TRY(check_kv(kv, d, B));
    const Round rd = round_layout(d, B, kv->cap, ws);
    if (!ws || ws_bytes < rd.total || n > B * (d.gamma + 1)) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws& w = rd.fw;
    bool an_ready = false;
    if (n > 0) {
        // Eq 2 for the round's new rows (split partials, if any, in the forward's region)
        const int rc = dflash_context_project(M, taps, tap_ld, n, rd.h_ctx, ws, w.total, stream);
        if (rc != DFLASH_OK) return rc;
        g_invocations--;  // counted once, below
    }
    CtxRows ctx{rd.h_ctx, n, row_offsets, counts, rd.len_old};
    if (n > 0 && d.nl > 0 && fused_qkv_ok(d, w, B * d.gamma, n)) {
        // lengths advance first (the attention reads them); the layers store the new rows'
        // K/V at the saved lengths
        DFL_HIP(launch_advance_len(kv->len, row_offsets, counts, kv->B, kv->cap, s, rd.len_old));
        DFL_TRY(forward_backbone(M, anchor_ids, kv, B, w, s, &an_ready, &ctx));
    } else {
        if (n > 0) {
            const int rc = dflash_ctx_kv_append(M, rd.h_ctx, n, row_offsets, counts, kv, ws, w.total, stream);
            if (rc != DFLASH_OK) return rc;
            g_invocations--;
        }
        DFL_TRY(forward_backbone(M, anchor_ids, kv, B, w, s, &an_ready));
    }
    float* y = y_out ? static_cast<float*>(y_out) : w.y;
    DFL_TRY(forward_out(M, B, w, s, an_ready, nullptr, y));
    DFL_TRY(lm_head(M->lm_head, y, d.wdtype == DFLASH_F32, B * d.gamma, d.H, d.V, draft_ids, max_logit, w.lmv, w.lmi,
                    s, w.i4h, w.i4h_bytes));
    g_invocations++;
    return DFLASH_OK;
}

size_t dflash_dspark_workspace_bytes(const dflash_dims* dims, int32_t r, int32_t B, int32_t cap) {
    if (check_dims(dims) == DFLASH_EINVAL || r <= 0 || B <= 0 || cap < 0) return 0;
    return dspark_layout(*dims, r, B, cap, nullptr).total;
}

int dflash_draft_forward_dspark(const dflash_model* M, const dflash_dspark_head* head, const int32_t* anchor_ids,
                                const dflash_kv* kv, int32_t B, const float* thresholds, float min_conf,
                                int32_t* draft_ids, float* conf, int32_t* lengths, void* y_out, void* ws,
                                size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (!head || !anchor_ids || !draft_ids || B <= 0) return DFLASH_EINVAL;
    if (head->r <= 0 || !head->w1 || !head->w2t || !head->conf_w || !head->conf_b) return DFLASH_EINVAL;
    if (head->r % 8 || !aligned16(head->w1) || !aligned16(head->w2t)) return DFLASH_DECLINED;
    if (std::isnan(min_conf)) return DFLASH_EINVAL;
    DFL_TRY(check_kv(kv, d, B));
    const Dspark ds = dspark_layout(d, head->r, B, kv->cap, ws);
    if (!ws || ws_bytes < ds.total) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Ws& w = ds.fw;
    const bool f32 = d.wdtype == DFLASH_F32;
    const int rows = B * d.gamma;
    bool an_ready = false;
    DFL_TRY(forward_backbone(M, anchor_ids, kv, B, w, s, &an_ready));
    // the block rows RMSNorm(H_d; out_norm) (page 3, #backbone), kept for the confidence head:
    // bf16 for bf16/int4 models (the out projection's input), fp32 for fp32 models
    if (f32)
        DFL_HIP(launch_rownorm(w.hd, 1, 0, static_cast<float*>(ds.hout), rows, d.d, M->out_norm, 1, d.eps, s));
    else
        DFL_HIP(norm_rows(w.hd, rows, d.d, M->out_norm, d.eps, static_cast<uint16_t*>(ds.hout), s));
    float* y = y_out ? static_cast<float*>(y_out) : w.y;
    DFL_TRY(forward_out(M, B, w, s, false, ds.hout, y));
    // base logits of every block row, fp32 (page 3, #baseLogits)
    DFL_TRY(lm_head_store(M->lm_head, y, f32, rows, d.H, d.V, ds.base, ds.skp, s));
    // the sequential loop: step k merges step k-1's argmax, gathers w1[previous] and scores
    // base[:, k] + w1[previous] w2 over the vocabulary
    dflash_weight w2t;
    w2t.dtype = f32 ? DFLASH_F32 : DFLASH_BF16;
    w2t.rows = d.V;
    w2t.cols = head->r;
    w2t.data = head->w2t;
    w2t.scales = w2t.biases = nullptr;
    DsparkStepParams sp;
    std::memset(&sp, 0, sizeof(sp));
    sp.gamma = d.gamma;
    sp.B = B;
    sp.V = d.V;
    sp.r = head->r;
    sp.d = d.d;
    sp.f32 = f32;
    sp.anchors = anchor_ids;
    sp.part_val = ds.pv;
    sp.part_idx = ds.pi;
    sp.w1 = head->w1;
    sp.hout = ds.hout;
    sp.conf_w = head->conf_w;
    sp.conf_b = head->conf_b;
    sp.thresholds = thresholds;
    sp.min_conf = min_conf;
    sp.e1 = ds.e1;
    sp.ids = draft_ids;
    sp.conf = conf;
    sp.lengths = lengths ? lengths : ds.lens;
    for (int k = 0; k <= d.gamma; ++k) {
        sp.step = k;
        DFL_HIP(launch_dspark_step(sp, s));
        if (k == d.gamma) break;
        DFL_TRY(markov_argmax(w2t, ds.e1, f32, B, head->r, d.V, ds.base + (int64_t)k * d.V, (int64_t)d.gamma * d.V,
                              ds.pv, ds.pi, &sp.nblocks, s));
    }
    g_invocations++;
    return DFLASH_OK;
}

size_t dflash_lm_head_workspace_bytes(int32_t V, int32_t M) {
    if (V <= 0 || M <= 0) return 0;
    return 2 * align_up((size_t)M * lm_tiles_max(V) * 4);
}

int dflash_lm_head_argmax(const dflash_weight* E_out, const void* y, int32_t y_dtype, int32_t M, int32_t* ids,
                          float* max_logit, void* ws, size_t ws_bytes, void* stream) {
    if (!E_out || !y || !ids || M <= 0) return DFLASH_EINVAL;
    if (y_dtype != DFLASH_F32 && y_dtype != DFLASH_BF16) return DFLASH_EINVAL;
    DFL_TRY(check_weight(*E_out, E_out->rows, E_out->cols, -1));
    if (E_out->rows <= 0 || E_out->cols <= 0) return DFLASH_EINVAL;
    if (reinterpret_cast<uintptr_t>(y) & 15) return DFLASH_DECLINED;
    const size_t need = dflash_lm_head_workspace_bytes(E_out->rows, M);
    if (!ws || ws_bytes < need) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    char* c = static_cast<char*>(ws);
    float* pv = reinterpret_cast<float*>(c);
    int32_t* pi = reinterpret_cast<int32_t*>(c + need / 2);
    // an int4 head with room for its split partial logits past the GEMV need: matrix cores
    float* i4part = (ws_bytes > need && aligned16(c + need)) ? reinterpret_cast<float*>(c + need) : nullptr;
    DFL_TRY(lm_head(*E_out, y, y_dtype == DFLASH_F32, M, E_out->cols, E_out->rows, ids, max_logit, pv, pi,
                    static_cast<hipStream_t>(stream), i4part, i4part ? ws_bytes - need : 0));
    g_invocations++;
    return DFLASH_OK;
}

size_t dflash_lm_head_workspace_bytes_for(const dflash_weight* E_out, int32_t y_dtype, int32_t M) {
    if (!E_out || E_out->rows <= 0 || E_out->cols <= 0 || M <= 0) return 0;
    size_t n = dflash_lm_head_workspace_bytes(E_out->rows, M);
    if (E_out->dtype == DFLASH_INT4G64 && y_dtype == DFLASH_BF16 && i4mm_ok(E_out->cols, M)) {
        int ns = 1, ks = 0;
        i4mm_split(E_out->cols, &ns, &ks);
        n += align_up((size_t)ns * M * E_out->rows * 4);
    }
    return n;
}

size_t dflash_kv_prefill_workspace_bytes(const dflash_dims* dims, int32_t n) {
    if (check_dims(dims) == DFLASH_EINVAL || n <= 0) return 0;
    return kv_append_norm_bytes(*dims, n);
}

size_t dflash_int4_prefill_workspace_bytes(const dflash_dims* dims, int32_t n) {
    if (check_dims(dims) == DFLASH_EINVAL || n <= 0) return 0;
    const size_t a = i4_prefill_proj_bytes(*dims, n), b = i4_prefill_kv_bytes(*dims, n);
    return a > b ? a : b;
}

int dflash_verify_greedy_lengths(const float* target_logits, const int32_t* draft_ids, const int32_t* lengths,
                                 int32_t B, int32_t gamma, int32_t V, int32_t* accepted, int32_t* committed,
                                 int32_t* ids, int32_t* next_anchor, void* ws, size_t ws_bytes, void* stream) {
    if (!lengths) return DFLASH_EINVAL;
    if (!target_logits || !draft_ids || !accepted || !committed || !ids) return DFLASH_EINVAL;
    if (B <= 0 || gamma <= 0 || V <= 0) return DFLASH_EINVAL;
    if (gamma + 1 > 64) return DFLASH_DECLINED;
    if (reinterpret_cast<uintptr_t>(target_logits) & 15) return DFLASH_DECLINED;
    const size_t need = dflash_verify_workspace_bytes(B, gamma, V);
    if (!ws || ws_bytes < need) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    char* c = static_cast<char*>(ws);
    float* pv = reinterpret_cast<float*>(c);
    int32_t* pi = reinterpret_cast<int32_t*>(c + need / 2);
    DFL_HIP(launch_verify(target_logits, draft_ids, B, gamma, V, accepted, committed, ids, next_anchor, pv, pi,
                          static_cast<hipStream_t>(stream), lengths));
    g_invocations++;
    return DFLASH_OK;
}

// the int4 head's partial logits for `rows` rows on matrix cores (0: the GEMV head)
static size_t i4_head_bytes(const dflash_dims& d, int64_t rows) {
    if (d.wdtype != DFLASH_INT4G64 || rows > kI4Rows || !i4mm_ok(d.H, (int)rows)) return 0;
    int ns = 1, ks = 0;
    i4mm_split(d.H, &ns, &ks);
    return (size_t)ns * rows * d.V * 4;
}

size_t dflash_verify_hidden_workspace_bytes(const dflash_dims* dims, int32_t B) {
    if (check_dims(dims) == DFLASH_EINVAL || B <= 0) return 0;
    const size_t rows = (size_t)B * (dims->gamma + 1);
    return align_up(rows * 4) + 2 * align_up(rows * lm_tiles_max(dims->V) * 4) + align_up(i4_head_bytes(*dims, rows));
}

int dflash_verify_from_hidden(const dflash_model* M, const void* target_hidden, int32_t B, const int32_t* draft_ids,
                              const int32_t* lengths, int32_t* accepted, int32_t* committed, int32_t* ids,
                              int32_t* next_anchor, void* ws, size_t ws_bytes, void* stream) {
    DFL_TRY(check_model(M));
    const dflash_dims& d = M->dims;
    if (!target_hidden || !draft_ids || !accepted || !committed || !ids || B <= 0) return DFLASH_EINVAL;
    if (!aligned16(target_hidden)) return DFLASH_DECLINED;
    const size_t need = dflash_verify_hidden_workspace_bytes(&d, B);
    if (!ws || !aligned16(ws) || ws_bytes < need) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int rows = B * (d.gamma + 1);
    const size_t part = align_up((size_t)rows * lm_tiles_max(d.V) * 4);
    char* c = static_cast<char*>(ws);
    int32_t* tids = reinterpret_cast<int32_t*>(c);
    float* pv = reinterpret_cast<float*>(c + align_up((size_t)rows * 4));
    int32_t* pi = reinterpret_cast<int32_t*>(c + align_up((size_t)rows * 4) + part);
    float* i4part = reinterpret_cast<float*>(c + align_up((size_t)rows * 4) + 2 * part);
    // the target's greedy token of every verify row: its hidden row scored by the borrowed head
    DFL_TRY(lm_head(M->lm_head, target_hidden, d.wdtype == DFLASH_F32, rows, d.H, d.V, tids, nullptr, pv, pi, s,
                    i4part, i4_head_bytes(d, rows)));
    DFL_HIP(launch_verify_ids(tids, draft_ids, B, d.gamma, accepted, committed, ids, next_anchor, lengths, s));
    g_invocations++;
    return DFLASH_OK;
}

size_t dflash_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V) {
    if (B <= 0 || gamma <= 0 || V <= 0) return 0;
    return 2 * align_up((size_t)B * (gamma + 1) * verify_splits(V) * 4);
}

int dflash_verify_greedy(const float* target_logits, const int32_t* draft_ids, int32_t B, int32_t gamma, int32_t V,
                         int32_t* accepted, int32_t* committed, int32_t* ids, int32_t* next_anchor, void* ws,
                         size_t ws_bytes, void* stream) {
    if (!target_logits || !draft_ids || !accepted || !committed || !ids) return DFLASH_EINVAL;
    if (B <= 0 || gamma <= 0 || V <= 0) return DFLASH_EINVAL;
    if (gamma + 1 > 64) return DFLASH_DECLINED;
    if (reinterpret_cast<uintptr_t>(target_logits) & 15) return DFLASH_DECLINED;
    const size_t need = dflash_verify_workspace_bytes(B, gamma, V);
    if (!ws || ws_bytes < need) return DFLASH_ENOSPC;
    DFL_TRY(gate());
    char* c = static_cast<char*>(ws);
    float* pv = reinterpret_cast<float*>(c);
    int32_t* pi = reinterpret_cast<int32_t*>(c + need / 2);
    DFL_HIP(launch_verify(target_logits, draft_ids, B, gamma, V, accepted, committed, ids, next_anchor, pv, pi,
                          static_cast<hipStream_t>(stream)));
    g_invocations++;
    return DFLASH_OK;
}

}  // extern "C"
