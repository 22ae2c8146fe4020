// Matrix-core projections of 16 to 128 activation rows (see skinny.hip):
//   y[m, n] = sum_k A[m, k] W[w_row0 + n, k]
// with bf16 A and W and fp32 accumulation, each weight row streamed once per
// launch; grid.z runs several layers' products in one launch.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gemv.hpp"

namespace dfl {

enum { SK_STORE = 0, SK_RESID = 1, SK_GATED = 2, SK_ARGMAX = 3, SK_KV = 4, SK_PARTIAL = 5 };

constexpr int kSkinnyRows = 128;  // activation rows per launch
constexpr int kSkinnyK = 128;     // K (and each split's K range) is a multiple of this
constexpr int kNormMaxK = 8192;   // longest row of the row-norm kernels

struct SkinnyParams {
    int M, N, K;          // SK_GATED: N = 2F weight rows (gate rows [0, F), up rows [F, 2F))
    // A: bf16 rows [M, K] at a + z * a_layer_stride (row stride a_ld); with seg_k > 0 the
    // columns come in segments of seg_k (a multiple of kSkinnyK): column k of row m is
    // a_seg[k / seg_k][m * a_ld + k % seg_k]
    const uint16_t* a;
    int64_t a_ld;
    int64_t a_layer_stride;
    const uint16_t* a_seg[kMaxTaps];
    int seg_k;
    // bf16 weights [*, K] of layer z; rows w_row0 .. w_row0 + N - 1 are used
    const uint16_t* w[kMaxLayers];
    int64_t w_row0;
    int layers;           // grid.z
    int F;                // SK_GATED
    int act;              // SK_GATED: 0 gelu_tanh, 1 silu
    // split-K: K ranges of kslice (grid.y). fp32 partial sums go to part
    // [layers][nsplit][M][N]; for SK_STORE / SK_RESID / SK_KV a second kernel adds them in
    // split order and applies the epilogue, for SK_PARTIAL the caller consumes them
    int nsplit, kslice;
    float* part;
    // SK_GATED on the direct-to-LDS kernel, balanced over the CUs (bal_main > 0): whole
    // tiles [0, bal_main) spread evenly over the workgroups, the remaining tiles split into
    // bal_items K ranges of bal_kslice (bal_splits per tile, at most one per workgroup) whose
    // partial sums go to bal_part [bal_splits][M][2 (F - bal_main 64)] (gate then up)
    int bal_main, bal_items, bal_splits, bal_kslice;
    float* bal_part;
    // SK_STORE: out[m, n] = y, fp32 or (out_bf16) bf16; with vt, bf16 columns n >= vt_col go
    //   head-dim major to vt[b][head][dim][32], b = (row_base + m) / gamma, key = its remainder
    // SK_RESID: out[m, n] += y (fp32)
    // SK_GATED: out[m, j] = bf16(act(y[m, j]) * y[m, F + j]) (bf16)
    void* out;
    int64_t out_ld;
    int out_bf16;
    uint16_t* vt;
    int vt_col, row_base, gamma, hkv, hd;
    // SK_ARGMAX: per row and workgroup tile, the (max, lowest index) of the row's outputs
    float* part_val;      // [M][nblocks]
    int32_t* part_idx;
    int nblocks;          // skinny_tiles(SK_ARGMAX, N)
    const float* base;    // SK_ARGMAX, optional: the argmax runs over base[m * base_ld + n] + y[m, n]
    int64_t base_ld;
    uint64_t* stamps;     // set by the launcher when the launch is traced: (start, end) wall clock per workgroup
    // SK_KV: columns [0, hkv*hd) are keys, [hkv*hd, 2*hkv*hd) values (bf16 caches). Row
    // r = row_base + m belongs to the sequence b with row_offsets[b] <= r < row_offsets[b+1]
    // and goes to cache position len[b] + (r - row_offsets[b]) when that index is below
    // counts[b] (all rows when counts is null) and the position below cap
    uint16_t* kcache;     // [layers][B][hkv][cap][hd]
    uint16_t* vcache;     // [layers][B][hkv][cap/32][hd][32]
    const int32_t* len;
    const int32_t* row_offsets;
    const int32_t* counts;
    int B, cap;
    int64_t layer_stride; // cache elements per layer
};

// workgroup tiles of a launch over N weight rows (the argmax partials per row)
int skinny_tiles(int epi, int N);
// split-K of a launch over `layers` products: the number of K ranges and their length
void skinny_split(int epi, int N, int K, int layers, int* nsplit, int* kslice);

// M in [1, kSkinnyRows], K a multiple of kSkinnyK; nsplit / kslice / nblocks as given by
// the functions above (part holds layers * nsplit * M * N floats when nsplit > 1 or
// for SK_PARTIAL)
hipError_t launch_skinny(int epi, const SkinnyParams& p, hipStream_t s);

// The gated product (N = 2F, one layer) balanced over the CUs on the direct-to-LDS kernel:
// whole column tiles spread evenly, the remaining tiles split into K ranges at most one per
// workgroup, their partial sums in part (at most skinny_gated_balanced_floats(M) floats)
// added in range order by the gated reduce. skinny_gated_balanced says whether a launch of
// M rows over N x K takes this path (5 to 8 row tiles, more column tiles than CUs).
bool skinny_gated_balanced(int M, int N, int K);
size_t skinny_gated_balanced_floats(int M);
hipError_t launch_skinny_gated_balanced(const SkinnyParams& p, hipStream_t s);

// The split-K sum and epilogue alone (SK_STORE / SK_RESID / SK_GATED, one layer; SK_KV,
// p.layers layers of partials [layers][nsplit][M][N] into bf16 caches): adds the nsplit
// fp32 partials part [nsplit][M][N] in split order and applies the epilogue (SK_GATED:
// N = F outputs from partials [nsplit][M][2F] of the gate and up rows); used for
// partials written by other kernels (N a multiple of 4)
hipError_t launch_split_reduce(int epi, const SkinnyParams& p, hipStream_t s);

// The residual split-K sum fused with the next RMSNorm: for each of the M rows,
// h[m] += sum_s part[s][m] (split order), then dst[m] = bf16(h[m] * (mean h[m]^2 +
// eps)^-1/2 * gain); one workgroup per row, N a multiple of 4 and at most 8192
hipError_t launch_resid_norm(const float* part, int nsplit, int M, int N, float* h, int64_t h_ld, const void* gain,
                             int gain_f32, float eps, uint16_t* dst, int64_t dst_ld, hipStream_t s);

// The block rows of B sequences (row r = b gamma + j, N values each) and their RMSNorm with
// `gain`: row j = 0 of sequence b is the sum of the split partials part[s][b] (nsplit
// partials [nsplit][B][N], split order) + block_pos[0], row j > 0 is mask_emb[j - 1] +
// block_pos[j] (bf16 tables [gamma][N], [gamma - 1][N]); h[r] = the row (fp32), dst[r] =
// bf16(row (mean row^2 + eps)^-1/2 gain). N a multiple of 4, at most 8192
hipError_t launch_block_norm(const float* part, int nsplit, int B, int gamma, int N, float* h,
                             const uint16_t* block_pos, const uint16_t* mask_emb, const void* gain, int gain_f32,
                             float eps, uint16_t* dst, hipStream_t s);

// dst + z * dst_layer_stride: rows r of bf16(x[r, k] * (mean_k x[r, k]^2 + eps)^-1/2 * gain[z][k])
// for rows of K fp32 values (K a multiple of 8, at most 8192), z < layers (grid.y)
struct NormRowsParams {
    const float* x;
    int64_t x_ld;
    int rows, K, layers, gain_f32;
    float eps;
    const void* gain[kMaxLayers];
    uint16_t* dst;
    int64_t dst_ld, dst_layer_stride;
    // 0: one layer per grid.y (more workgroups for a few rows); 1: each row read
    // once and written for every layer (long prefills)
    int all_layers;
};
hipError_t launch_norm_rows(const NormRowsParams& p, hipStream_t s);

}  // namespace dfl
