// Device helpers shared by the drafter kernels: bf16 bit conversions, bf16
// dot products, 64-lane wavefront reductions and the FFN activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

// native vectors: arrays of them stay in registers where arrays of the HIP vector
// structs may be kept in scratch memory
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 wavefronts per workgroup

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// c + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Larger value wins; equal values keep the lower index.
__device__ __forceinline__ void argmax_pick(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float v2 = __shfl_xor(v, o, kWave);
        int i2 = __shfl_xor(i, o, kWave);
        argmax_pick(v, i, v2, i2);
    }
}

// Sum NV per-lane values across the wavefront by recursive halving: at each
// step a lane keeps one half of its values and adds the partner's copy of that
// half, so the work shrinks with the value count. On return lanes 2v and 2v+1
// hold the full sum of value v (NV = 32), lanes 4v..4v+3 for NV = 16, and so
// on; for NV > 32 every lane holds value (lane >> (6 - log2 NV)).
template <int NV>
__device__ __forceinline__ float wave_sum_many(float (&v)[NV], int lane) {
    static_assert((NV & (NV - 1)) == 0 && NV >= 1 && NV <= 64, "power of two");
    int c = NV;
    int off = 32;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        if (c > 1) {
            const bool up = (lane & off) != 0;
            const int h = c >> 1;
#pragma unroll
            for (int i = 0; i < NV / 2; ++i) {
                if (i < h) {
                    float lo = v[i], hi = v[i + h];
                    float send = up ? lo : hi;
                    float keep = up ? hi : lo;
                    v[i] = keep + __shfl_xor(send, off, kWave);
                }
            }
            c = h;
        } else {
            v[0] += __shfl_xor(v[0], off, kWave);
        }
        off >>= 1;
    }
    return v[0];
}
// Which value index lane `lane` holds after wave_sum_many<NV>.
template <int NV>
__device__ __forceinline__ int wave_sum_many_index(int lane) {
    int idx = 0, off = 32, c = NV;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        if (c > 1) {
            c >>= 1;
            if (lane & off) idx += c;
        }
        off >>= 1;
    }
    return idx;
}

__device__ __forceinline__ float gelu_tanh(float x) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * x * (1.0f + tanhf(k0 * (x + 0.044715f * x * x * x)));
}
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Loads of data each launch reads once (weights, the K/V cache, target logits) carry the
// non-temporal hint, so the stream does not displace what the workgroups re-read from the
// caches (activation chunks, query tiles, partial sums)
#ifndef DFL_STREAM_NT
#define DFL_STREAM_NT 1
#endif
__device__ __forceinline__ u32x4 stream_load(const u32x4* p) {
#if DFL_STREAM_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
__device__ __forceinline__ f32x4 stream_load(const f32x4* p) {
#if DFL_STREAM_NT
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
    const u32x4 v = stream_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 stream_load(const float4* p) {
    const f32x4 v = stream_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float load_gain(const void* g, bool f32, int i) {
    return f32 ? static_cast<const float*>(g)[i] : bf16_bits_to_f32(static_cast<const uint16_t*>(g)[i]);
}

// gains i .. i+7 (i a multiple of 8) as one or two 16-byte loads
__device__ __forceinline__ void load_gain8(const void* g, bool f32, int i, float (&v)[8]) {
    if (f32) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(g) + i);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(g) + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(g) + i);
        v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
        v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
    }
}

// Offset of value (pos, dim) in one (sequence, kv head) slab of the value cache. bf16
// caches hold each 32-key chunk of all head dims contiguously ([cap/32][hd][32]): a key
// chunk's values are one contiguous run, read in 1 KB pieces. fp32 caches are head-dim
// major ([hd][cap]).
__host__ __device__ inline int64_t v_cache_off(int pos, int dim, int hd, int cap, bool f32) {
    return f32 ? (int64_t)dim * cap + pos : ((int64_t)(pos >> 5) * hd + dim) * 32 + (pos & 31);
}

}  // namespace dfl
