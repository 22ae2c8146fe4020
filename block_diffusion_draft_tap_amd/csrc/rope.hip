// Rotary positions of the DFlash2 variant (page "Inco Hacks Native: DFlash 2
// Speculation", section 1 names a sliding-window drafter; the rotation itself
// is this library's reading, the rotate-half layout of the Qwen family the
// drafter pairs with): dims i and i + hd/2 of a head turn by the angle
// pos * theta^(-2i/hd).
//
//   rope_block_kernel  the block's Q and K_b rows in place, block row k of
//                      sequence b at position len[b] + k
//   rope_cache_kernel  keys just written to the cache by an append, at the
//                      positions the append wrote them to
//
// The angle is formed and reduced to [-pi, pi] in double precision (positions
// reach 2^20 and more, where a float product alone would be off by a sizable
// fraction of a radian); its sine and cosine are then taken in float. The turn
// itself is float arithmetic on the stored (bf16 or fp32) values; bf16 results
// are rounded to nearest even, as every stored bf16 value is.
#include <cmath>

#include "common.hpp"
#include "rope.hpp"

namespace dfl {

RopeFreq rope_freq(int hd, float theta) {
    RopeFreq f{};
    f.pairs = hd / 2;
    for (int i = 0; i < f.pairs && i < kRopeMaxPairs; ++i)
        f.invf[i] = std::pow((double)theta, -2.0 * (double)i / (double)hd);
    return f;
}

__device__ __forceinline__ void rope_angle(int pos, double invf, float* c, float* s) {
    constexpr double kTwoPi = 6.283185307179586476925;
    double a = (double)pos * invf;
    a -= kTwoPi * rint(a * (1.0 / kTwoPi));
    sincosf((float)a, s, c);
}

template <bool F32>
__device__ __forceinline__ void rope_pair(void* base, int64_t i0, int64_t i1, float c, float s) {
    if constexpr (F32) {
        float* x = static_cast<float*>(base);
        const float a = x[i0], b = x[i1];
        x[i0] = a * c - b * s;
        x[i1] = b * c + a * s;
    } else {
        uint16_t* x = static_cast<uint16_t*>(base);
        const float a = bf16_bits_to_f32(x[i0]), b = bf16_bits_to_f32(x[i1]);
        x[i0] = (uint16_t)f32_to_bf16_bits(a * c - b * s);
        x[i1] = (uint16_t)f32_to_bf16_bits(b * c + a * s);
    }
}

// one workgroup per block row; thread t turns pair t % pairs of heads t / pairs,
// t / pairs + kBlock / pairs, ...
template <bool F32>
__global__ __launch_bounds__(kBlock) void rope_block_kernel(void* qkv, int64_t qkv_ld, const int32_t* len, int gamma,
                                                            int hq, int hkv, int hd, const RopeFreq f) {
    const int r = blockIdx.x;
    const int b = r / gamma, k = r - b * gamma;
    const int pairs = f.pairs;
    const int i = threadIdx.x % pairs;
    const int pos = max(len[b], 0) + k;
    float c, s;
    rope_angle(pos, f.invf[i], &c, &s);
    const int64_t row = (int64_t)r * qkv_ld;
    // heads 0 .. hq-1 are Q, hq .. hq+hkv-1 are K_b (columns hq*hd + g*hd)
    for (int h = threadIdx.x / pairs; h < hq + hkv; h += kBlock / pairs) {
        const int64_t col = row + (int64_t)h * hd + i;
        rope_pair<F32>(qkv, col, col + pairs, c, s);
    }
}

// one workgroup per appended row; thread t turns pair t % pairs of (layer, kv head)
// t / pairs, t / pairs + kBlock / pairs, ...
template <bool F32>
__global__ __launch_bounds__(kBlock) void rope_cache_kernel(void* kcache, int nl, int64_t layer_stride, int B, int hkv,
                                                            int cap, int hd, const int32_t* row_offsets,
                                                            const int32_t* counts, const int32_t* len,
                                                            const RopeFreq f) {
    const int m = blockIdx.x;
    // the row's sequence: the last b with row_offsets[b] <= m
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (row_offsets[mid] <= m) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rows_b = row_offsets[b + 1] - row_offsets[b];
    const int i_row = m - row_offsets[b];
    const int cnt = counts ? min(counts[b], rows_b) : rows_b;
    const int pos = len[b] + i_row;
    if (i_row < 0 || i_row >= cnt || pos < 0 || pos >= cap) return;  // not written by the append
    const int pairs = f.pairs;
    const int i = threadIdx.x % pairs;
    float c, s;
    rope_angle(pos, f.invf[i], &c, &s);
    for (int j = threadIdx.x / pairs; j < nl * hkv; j += kBlock / pairs) {
        const int layer = j / hkv, g = j - layer * hkv;
        const int64_t at = (int64_t)layer * layer_stride + (((int64_t)b * hkv + g) * cap + pos) * hd + i;
        rope_pair<F32>(kcache, at, at + pairs, c, s);
    }
}

hipError_t launch_rope_block(void* qkv, int f32, int64_t qkv_ld, const int32_t* len, int B, int gamma, int hq,
                             int hkv, int hd, const RopeFreq& f, hipStream_t s) {
    if (hd != 2 * f.pairs || f.pairs > kRopeMaxPairs || kBlock % f.pairs || B <= 0 || gamma <= 0)
        return hipErrorInvalidValue;
    (void)hipGetLastError();
    const dim3 grid((unsigned)(B * gamma));
    if (f32)
        hipLaunchKernelGGL((rope_block_kernel<true>), grid, dim3(kBlock), 0, s, qkv, qkv_ld, len, gamma, hq, hkv, hd,
                           f);
    else
        hipLaunchKernelGGL((rope_block_kernel<false>), grid, dim3(kBlock), 0, s, qkv, qkv_ld, len, gamma, hq, hkv,
                           hd, f);
    return hipGetLastError();
}

hipError_t launch_rope_cache(void* kcache, int f32, int nl, int64_t layer_stride, int B, int hkv, int cap, int hd,
                             const int32_t* row_offsets, const int32_t* counts, const int32_t* len, int n,
                             const RopeFreq& f, hipStream_t s) {
    if (hd != 2 * f.pairs || f.pairs > kRopeMaxPairs || kBlock % f.pairs || B <= 0 || nl <= 0)
        return hipErrorInvalidValue;
    if (n <= 0) return hipSuccess;
    (void)hipGetLastError();
    const dim3 grid((unsigned)n);
    if (f32)
        hipLaunchKernelGGL((rope_cache_kernel<true>), grid, dim3(kBlock), 0, s, kcache, nl, layer_stride, B, hkv, cap,
                           hd, row_offsets, counts, len, f);
    else
        hipLaunchKernelGGL((rope_cache_kernel<false>), grid, dim3(kBlock), 0, s, kcache, nl, layer_stride, B, hkv,
                           cap, hd, row_offsets, counts, len, f);
    return hipGetLastError();
}

}  // namespace dfl
