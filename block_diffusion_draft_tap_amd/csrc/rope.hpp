// Rotary positions of the DFlash2 variant (see rope.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

constexpr int kRopeMaxPairs = 64;  // hd / 2 for the supported head dims (64, 128)

// theta^(-2i/hd) for i < hd/2, computed on the host in double precision
struct RopeFreq {
    double invf[kRopeMaxPairs];
    int pairs;  // hd / 2
};
RopeFreq rope_freq(int hd, float theta);

// The block's Q and K_b rows in place: row b*gamma + k of qkv (Q heads at columns
// h*hd, kv heads at hq*hd + g*hd) turned at position len[b] + k. bf16 elements
// (rounded again after the turn) unless f32.
hipError_t launch_rope_block(void* qkv, int f32, int64_t qkv_ld, const int32_t* len, int B, int gamma, int hq,
                             int hkv, int hd, const RopeFreq& f, hipStream_t s);

// Keys just appended to the cache, in place, before the lengths advance: row m of
// the append (sequence b with row_offsets[b] <= m < row_offsets[b+1], i = m -
// row_offsets[b], kept when i < counts[b]) sits at position len[b] + i; its keys in
// every layer and kv head turn by that position. kcache [nl][B][hkv][cap][hd].
hipError_t launch_rope_cache(void* kcache, int f32, int nl, int64_t layer_stride, int B, int hkv, int cap, int hd,
                             const int32_t* row_offsets, const int32_t* counts, const int32_t* len, int n,
                             const RopeFreq& f, hipStream_t s);

}  // namespace dfl
