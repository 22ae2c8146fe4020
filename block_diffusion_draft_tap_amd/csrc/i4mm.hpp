// int4-g64 weights on matrix cores for up to 16 activation rows (see i4mm.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

constexpr int kI4Rows = 16;       // activation rows per launch (one MFMA row fragment)
constexpr int kI4Block = 128;     // K per block: two quantisation groups
constexpr int kI4MaxBlocks = 8;   // blocks per workgroup K range (1024 columns)
constexpr int kI4ArgChunk = 1024; // outputs per workgroup of the split argmax

struct I4Params {
    const uint32_t* codes;   // [N, K/8], 8 codes per word, low nibble first
    const uint16_t* scales;  // bf16 [N, K/64]
    const uint16_t* biases;  // bf16 [N, K/64]
    int N, K;                // K a multiple of 128
    const uint16_t* a;       // bf16 activation rows [M, K], row stride a_ld (a multiple of 8)
    int64_t a_ld;
    int M;                   // 1 .. 16
    int nsplit, kslice;      // K ranges (grid.y); kslice a multiple of 128, at most 1024
    float* part;             // fp32 partial sums [nsplit][M][N]
    uint64_t* stamps;        // set by the launcher when the launch is traced
};

// whether a product of M rows over K columns runs here
bool i4mm_ok(int K, int M);
// K ranges of at most 1024 columns, balanced, multiples of 128
void i4mm_split(int K, int* nsplit, int* kslice);
// partial sums part[s][m][n] = sum over k in range s of a[m, k] w[n, k]
hipError_t launch_i4mm(I4Params p, hipStream_t s);
// per row m and chunk c of kI4ArgChunk outputs: the (max, lowest index) over n of
// sum_s part[s][m][n] (split order), into pv / pi [M][nblocks], nblocks = i4_argmax_blocks(N)
int i4_argmax_blocks(int N);
hipError_t launch_i4_split_argmax(const float* part, int nsplit, int M, int N, float* pv, int32_t* pi, int nblocks,
                                  hipStream_t s);

}  // namespace dfl
