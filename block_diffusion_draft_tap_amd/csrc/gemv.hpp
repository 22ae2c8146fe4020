// Skinny GEMV / small-M GEMM for the drafter's projections:
//   y[m, n] = sum_k x[m, k] * W[n, k]       (W row-major [N, K], K contiguous)
// for M <= MAXM activation rows. Each workgroup (4 wavefronts) owns a tile of
// 4*RPW weight rows and streams them over the whole K range once; every lane
// reads 16-byte weight chunks, the activations are staged once per workgroup
// in LDS (in K chunks) in the type the product uses (bf16 for bf16/int4
// weights, fp32 for fp32 weights), and partial sums are reduced across the
// wavefront at the end.
//
// Prologues build the activation rows while staging them:
//   PRO_PLAIN   x rows from an fp32 buffer
//   PRO_NORM    RMSNorm of fp32 rows with a gain: x * (mean x^2 + eps)^-1/2 * g
//   PRO_TAPS    concatenation of m tap buffers [rows, H] (Eq 2 input)
//   PRO_GATHER  rows of an embedding table selected by token ids
// Epilogues consume the reduced sums:
//   EPI_STORE      out[m, n] = y (optionally rounded to bf16)
//   EPI_RESID      out[m, n] += y                     (residual stream)
//   EPI_GATED      out[m, j] = act(y_gate[j]) * y_up[j]  (rows j and F+j)
//   EPI_KV         K/V rows written to the retained context cache
//   EPI_BLOCKINIT  block rows: anchor row + block_pos[0], mask rows
//   EPI_ARGMAX     per-workgroup (max, lowest index) of each row's outputs
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

enum WType { W_F32 = 0, W_BF16 = 1, W_I4 = 2 };
enum { PRO_PLAIN = 0, PRO_NORM = 1, PRO_TAPS = 2, PRO_GATHER = 3 };
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_GATED = 2, EPI_KV = 3, EPI_BLOCKINIT = 4, EPI_ARGMAX = 5, EPI_QKVKV = 6 };

constexpr int kMaxTaps = 8;
constexpr int kMaxLayers = 16;

struct WeightPtr {
    const void* data = nullptr;
    const uint16_t* scales = nullptr;
    const uint16_t* biases = nullptr;
};

struct GemvParams {
    // weights: per-layer pointers (grid.y selects the layer; entry 0 otherwise)
    WeightPtr w[kMaxLayers];
    int64_t w_row0;      // first weight row used (row offset into the matrix)
    int N;               // weight rows processed (outputs; for EPI_GATED 2F)
    int K;               // reduction length
    int M;               // active activation rows (<= MAXM)
    int rpw;             // weight rows per wavefront (1, 2 or 4; even for EPI_GATED)
    int ksplit;          // K ranges (grid.z); each writes its partial sums to out + z*split_stride
                         // (EPI_STORE fp32 over several layers: out + (y*ksplit + z)*split_stride)
    int kslice;          // K elements per range (multiple of 32)
    int64_t split_stride;
    int max_wgs;         // cap on workgroups; row tiles beyond it are looped over (0 = one per tile)

    // prologue
    const float* x;      // PRO_PLAIN / PRO_NORM: fp32 rows (PRO_PLAIN: bf16 rows when src_f32 = 0)
    int64_t x_ld;
    const float* x2;     // PRO_NORM with x2: rows m >= M1 come from x2 + (m - M1) * x_ld
    int M1;
    int64_t x_layer_stride;  // PRO_PLAIN: layer y's rows start at x + y * x_layer_stride elements
    const void* gain[kMaxLayers];  // PRO_NORM: per-layer gain vectors [K]
    int gain_f32;
    float eps;
    const void* taps[kMaxTaps];    // PRO_TAPS: tap j covers k in [j*H, (j+1)*H)
    int64_t tap_ld;
    int H;
    int src_f32;         // PRO_PLAIN / PRO_TAPS source element type (1 = fp32, 0 = bf16)
    const int32_t* ids;  // PRO_GATHER: table rows
    WeightPtr table;     // PRO_GATHER: embedding table [table_rows, K]
    int table_rows;      // ids are clamped to [0, table_rows)
    int table_type;      // WType of the table

    // epilogue
    float* out;
    int64_t out_ld;
    int round_out;       // EPI_STORE / EPI_GATED: round results to bf16 (EPI_GATED then stores bf16)
    int out_bf16;        // EPI_STORE: store bf16 values instead of fp32
    uint16_t* vt;        // EPI_STORE with out_bf16: outputs n >= vt_col go head-dim major to
    int vt_col;          //   vt[b][head][dim][32] (b = row / gamma, key = row % gamma; heads of hd)
                         //   instead of out; row_base is the global index of row 0
    int F;               // EPI_GATED: gate rows [0, F), up rows [F, 2F)
    int act;             // EPI_GATED: 0 gelu_tanh, 1 silu
    // EPI_KV
    void* kcache;        // [nl][B][hkv][cap][hd]
    void* vcache;
    const int32_t* len;
    const int32_t* row_offsets;  // [B+1]
    const int32_t* counts;       // [B] or null
    int row_base;        // global index of activation row 0 of this launch
    int B, hkv, hd, cap, kv_f32;
    int64_t layer_stride;  // elements per layer in the cache
    // EPI_QKVKV (one pass over a layer's fused Q|K|V rows): activation rows m < M1 are block
    // rows stored as EPI_STORE does (bf16 rows, values head-dim major through vt); rows
    // m >= M1 are context rows row_base + m - M1 whose key / value columns (n >= kv_col0)
    // go to the cache as EPI_KV does, at len[b] + i (len: the lengths before this round)
    int kv_col0;
    // EPI_BLOCKINIT
    const void* block_pos;  // [gamma, d]
    const void* mask_emb;   // [gamma-1, d]
    int gamma;
    int64_t seq_base;       // sequence index of activation row 0
    // EPI_ARGMAX
    float* part_val;     // [M][nblocks]
    int32_t* part_idx;
    int nblocks;
    const float* base;   // optional: the argmax runs over base[m * base_ld + n] + (row m . W[n])
    int64_t base_ld;
    uint64_t* stamps;    // set by the launcher when the launch is traced: (start, end) wall clock per workgroup
};

// Host-side launcher: picks the kernel for the weight type and the modes; maxm is
// the row capacity (4: int4 weights and M <= 4 only; 8; or 32 for the long-row
// paths).
hipError_t launch_gemv(int wtype, int pro, int epi, int maxm, const GemvParams& p, int layers, hipStream_t s);

// Grid of a launch with `rows` (<= 8) activation rows, reduction length K and
// ntiles row tiles under a persistent-workgroup cap (what the argmax partials
// are sized by): reductions that stage in one pass run persistent workgroups.
int gemv_head_grid(int wtype, int K, int ntiles, int max_wgs, int rows);

// Activation rows a launch of `rows` rows is compiled for: int4 weights, whose
// products are ALU-bound, take a 4-row kernel for up to 4 rows; everything else 8
inline int gemv_maxm(int wtype, int rows) { return (wtype == W_I4 && rows <= 4) ? 4 : 8; }

// LDS budget for staged activations per workgroup
constexpr int kStageBytes = 64 * 1024;
// PRO_NORM rows up to this length are normalised in registers in one round trip;
// longer rows take two passes over the fp32 row in every workgroup's prologue
constexpr int kRegNormMaxK = 2048;

}  // namespace dfl
