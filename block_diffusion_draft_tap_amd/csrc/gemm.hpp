// Matrix-core GEMM for the context prefill: C[m, n] = sum_k A[m, k] B[n, k]
// with bf16 operands and fp32 accumulation, for row counts where the
// projections are real contractions (see gemm.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gemv.hpp"

namespace dfl {

enum { GEMM_A_TAPS = 0, GEMM_A_NORM = 1 };
enum { GEMM_EPI_F32 = 0, GEMM_EPI_KV = 1 };

struct GemmParams {
    int M, N, K;  // K a multiple of 64
    // GEMM_A_TAPS: bf16 rows split along K into segments of seg_k columns
    // (a multiple of 64); segment j starts at a[j] + layer * a_layer_stride
    // (layer = grid.z), row stride a_ld elements
    const uint16_t* a[kMaxTaps];
    int64_t a_ld;
    int64_t a_layer_stride;
    int seg_k;
    // a_period > 0: A's column k is column k % a_period of the rows above (the K of a B
    // matrix that holds two parts of every weight, [W_hi | W_lo], against [A | A])
    int a_period;
    // GEMM_A_NORM: A[m, k] = bf16((x[m, k] * rinv[m]) * gain[k]) from fp32 rows
    // x (row stride a_ld); gain per layer (grid.z)
    const float* x;
    const float* rinv;
    const void* gain[kMaxLayers];
    int gain_f32;
    // B: bf16 weight rows [N, K]: row b_row0 + n of b[layer], row stride K
    const uint16_t* b[kMaxLayers];
    int64_t b_row0;
    // GEMM_EPI_F32: C fp32 [M, N], row stride c_ld
    float* c;
    int64_t c_ld;
    // GEMM_EPI_KV: columns [0, hkv*hd) are keys, [hkv*hd, 2*hkv*hd) values; row m
    // belongs to the sequence b with row_offsets[b] <= m < row_offsets[b+1] and
    // goes to cache position len[b] + (m - row_offsets[b]) when that row index is
    // below counts[b] (all rows when counts is null) and the position below cap
    void* kcache;  // [nl][B][hkv][cap][hd] bf16
    void* vcache;  // [nl][B][hkv][cap/32][hd][32] bf16
    const int32_t* len;
    const int32_t* row_offsets;
    const int32_t* counts;
    int B, hkv, hd, cap;
    int64_t layer_stride;  // cache elements per layer
};

// one launch per call; grid.z = layers (B, gain and the cache layer follow it)
hipError_t launch_gemm(int amode, int epi, const GemmParams& p, int layers, hipStream_t s);

// rinv[r] = (mean_k x[r, k]^2 + eps)^-1/2 for rows of K fp32 values
hipError_t launch_row_rinv(const float* x, int64_t ld, int rows, int K, float eps, float* rinv, hipStream_t s);

}  // namespace dfl
