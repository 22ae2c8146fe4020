// int4-g64 weights on matrix cores for up to 16 activation rows (see i4mm.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

constexpr int kI4Rows = 16;       // activation rows per launch (one MFMA row fragment)
constexpr int kI4Block = 128;     // K per block: two quantisation groups
constexpr int kI4MaxBlocks = 8;   // blocks per workgroup K range (1024 columns)
constexpr int kI4ArgChunk = 1024; // outputs per workgroup of the split argmax

constexpr int kI4MaxLayers = 16;  // weight sets of one launch (grid.y)
constexpr int kI4MaxSegs = 8;     // activation column segments

struct I4Params {
    // weights of layer z (grid.y): rows w_row0 .. w_row0 + N - 1 of [*, K] matrices
    const uint32_t* codes[kI4MaxLayers];   // [*, K/8], 8 codes per word, low nibble first
    const uint16_t* scales[kI4MaxLayers];  // bf16 [*, K/64]
    const uint16_t* biases[kI4MaxLayers];  // bf16 [*, K/64]
    int64_t w_row0;
    int layers;
    int N, K;                // K a multiple of 128
    // bf16 activation rows [M, K] of layer z at a + z * a_layer_stride (row stride a_ld, a
    // multiple of 8); with seg_k > 0 the columns come in segments of seg_k (a multiple of
    // kslice): column k of row m is a_seg[k / seg_k][m * a_ld + k % seg_k]
    const uint16_t* a;
    int64_t a_ld, a_layer_stride;
    const uint16_t* a_seg[kI4MaxSegs];
    int seg_k;
    int M;                   // 1 .. 16
    int nsplit, kslice;      // K ranges; kslice a multiple of 128, at most 1024
    float* part;             // fp32 partial sums [layers][nsplit][M][N]
    uint64_t* stamps;        // set by the launcher when the launch is traced
    uint32_t nib_mask, bf16_128;  // set by the launcher: the code unpack's constants
};

// whether a product of M rows over K columns runs here
bool i4mm_ok(int K, int M);
// K ranges of at most 1024 columns, balanced, multiples of 128
void i4mm_split(int K, int* nsplit, int* kslice);
// partial sums part[z][s][m][n] = sum over k in range s of a_z[m, k] w_z[w_row0 + n, k]
hipError_t launch_i4mm(I4Params p, hipStream_t s);
// per row m and chunk c of kI4ArgChunk outputs: the (max, lowest index) over n of
// sum_s part[s][m][n] (split order), into pv / pi [M][nblocks], nblocks = i4_argmax_blocks(N)
int i4_argmax_blocks(int N);
// rows row0 .. row0 + N - 1 of an int4-g64 matrix [*, K] expanded into bf16 [N, 2K]: columns
// [0, K) the high parts bf16(w), [K, 2K) the low parts bf16(w - bf16(w)), w = scale * q + bias
// formed in fp32 (exact but for the sum's rounding); high + low hold w to about 16 bits, so
// one bf16 matrix-core product over [A | A] reproduces the int4 product (the prefill GEMM)
hipError_t launch_i4_expand(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int K, int64_t row0,
                            int N, uint16_t* out, hipStream_t s);
hipError_t launch_i4_split_argmax(const float* part, int nsplit, int M, int N, float* pv, int32_t* pi, int nblocks,
                                  hipStream_t s);

}  // namespace dfl
