// Skinny GEMV family for the drafter projections (see gemv.hpp for the modes).
//
// Work split: a workgroup of 4 wavefronts owns a tile of 4*RPW consecutive
// weight rows (for the gated FFN: 2*RPW gate/up row pairs) and reads each of
// them exactly once over its K range. Lane l of a wavefront reads the 16-byte
// chunk at k = l*EPL + 64*EPL*i of each of its rows, so one wavefront
// instruction covers a contiguous 1 KiB (bf16) or 512 B (int4) run of a row.
// The activation rows are staged once per workgroup in LDS (in K chunks when
// the range is long) and read back as 16-byte vectors matching the weight
// chunk lane by lane. When the K range fits one chunk, a workgroup loops over
// several row tiles (persistent tiles) and stages the activations only once.
//
// Latency: the first PF weight iterations of a tile are loaded into registers
// before the activation prologue runs (and, across persistent tiles, before
// the previous tile's reduction), so the HBM latency overlaps the staging.
//
// Split K (grid.z): each range writes its partial sums to its own slice of
// the output; the consumer adds the slices in a fixed order.
//
// Products: bf16 weights use v_dot2 (two bf16 products per instruction into
// an fp32 accumulator); int4 weights are turned into bf16 (128 + q) pairs with
// two integer ops per pair and use the same v_dot2, with
//   sum_k x_k (s q_k + b) = s sum_k x_k (128 + q_k) + (b - 128 s) sum_k x_k
// evaluated per 32-element lane chunk (the activation sums are staged with
// the activations); fp32 weights use plain fp32 FMAs.
#include <cstdio>

#include "common.hpp"
#include "gemv.hpp"
#include "trace.hpp"

namespace dfl {


// weight iterations kept in flight per lane (register ring), for 1-2 and 4 rows per wavefront
#ifndef DFL_PF
#define DFL_PF 4
#endif
#ifndef DFL_PF_WIDE
#define DFL_PF_WIDE 2
#endif
// weight iterations in flight in the bf16 / fp32 LM head (argmax epilogue)
#ifndef DFL_PF_HEAD
#define DFL_PF_HEAD 2
#endif

template <int WT> struct WTraits;
template <> struct WTraits<W_F32> { typedef float X; static constexpr int EPL = 8; };
template <> struct WTraits<W_BF16> { typedef uint16_t X; static constexpr int EPL = 8; };
template <> struct WTraits<W_I4> { typedef uint16_t X; static constexpr int EPL = 32; };

// one lane's weight chunk of one row
template <int WT> struct WChunk;
template <> struct WChunk<W_BF16> { uint4 v; };
template <> struct WChunk<W_F32> { float4 a, b; };
template <> struct WChunk<W_I4> { uint4 c; float s, b; };

template <int WT>
__device__ __forceinline__ void wload(WChunk<WT>& w, const WeightPtr& W, int64_t row, int K, int k) {
    if constexpr (WT == W_BF16) {
        w.v = stream_load(reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W.data) + row * K + k));
    } else if constexpr (WT == W_F32) {
        const float* src = static_cast<const float*>(W.data) + row * K + k;
        w.a = stream_load(reinterpret_cast<const float4*>(src));
        w.b = stream_load(reinterpret_cast<const float4*>(src + 4));
    } else {
        w.c = stream_load(reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(W.data) + row * (K / 8) + k / 8));
        const int64_t g = row * (K / 64) + k / 64;
        w.s = bf16_bits_to_f32(W.scales[g]);
        w.b = bf16_bits_to_f32(W.biases[g]);
    }
}

// acc[r][m] += chunk(r) . x[m][kl .. kl+EPL)
template <int WT, int MAXM, int RPW>
__device__ __forceinline__ void wfma(const WChunk<WT> (&w)[RPW], const typename WTraits<WT>::X* xs, int KC, int kl,
                                     const float* xsum, float (&acc)[RPW][MAXM]) {
    if constexpr (WT == W_BF16) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)m * KC + kl);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                float a = acc[r][m];
                a = dot2_bf16(w[r].v.x, xv.x, a);
                a = dot2_bf16(w[r].v.y, xv.y, a);
                a = dot2_bf16(w[r].v.z, xv.z, a);
                a = dot2_bf16(w[r].v.w, xv.w, a);
                acc[r][m] = a;
            }
        }
    } else if constexpr (WT == W_F32) {
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            const float* xr = xs + (size_t)m * KC + kl;
            const float4 x0 = *reinterpret_cast<const float4*>(xr);
            const float4 x1 = *reinterpret_cast<const float4*>(xr + 4);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                float a = acc[r][m];
                a = fmaf(w[r].a.x, x0.x, a); a = fmaf(w[r].a.y, x0.y, a);
                a = fmaf(w[r].a.z, x0.z, a); a = fmaf(w[r].a.w, x0.w, a);
                a = fmaf(w[r].b.x, x1.x, a); a = fmaf(w[r].b.y, x1.y, a);
                a = fmaf(w[r].b.z, x1.z, a); a = fmaf(w[r].b.w, x1.w, a);
                acc[r][m] = a;
            }
        }
    } else {
        uint32_t pr[RPW][16];
        float bi[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            bi[r] = w[r].b - 128.0f * w[r].s;
            const uint32_t words[4] = {w[r].c.x, w[r].c.y, w[r].c.z, w[r].c.w};
#pragma unroll
            for (int wd = 0; wd < 4; ++wd)
#pragma unroll
                for (int j = 0; j < 4; ++j) pr[r][4 * wd + j] = ((words[wd] >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
        }
#pragma unroll
        for (int m = 0; m < MAXM; ++m) {
            float d[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) d[r] = 0.f;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)m * KC + kl + 8 * wd);
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    float a = d[r];
                    a = dot2_bf16(pr[r][4 * wd + 0], xv.x, a);
                    a = dot2_bf16(pr[r][4 * wd + 1], xv.y, a);
                    a = dot2_bf16(pr[r][4 * wd + 2], xv.z, a);
                    a = dot2_bf16(pr[r][4 * wd + 3], xv.w, a);
                    d[r] = a;
                }
            }
            const float xsm = xsum[m * (KC / 32) + kl / 32];
#pragma unroll
            for (int r = 0; r < RPW; ++r) acc[r][m] += w[r].s * d[r] + bi[r] * xsm;
        }
    }
}

// ---------------------------------------------------------------------------
// activation loaders: 8 consecutive elements k..k+7 of activation row m

__device__ __forceinline__ void load8_f32(const float* src, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8_bf16(const uint16_t* src, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
}
__device__ __forceinline__ void load8_weight_row(const WeightPtr& t, int type, int64_t row, int K, int k,
                                                 float (&v)[8]) {
    if (type == W_F32) {
        load8_f32(static_cast<const float*>(t.data) + row * K + k, v);
    } else if (type == W_BF16) {
        load8_bf16(static_cast<const uint16_t*>(t.data) + row * K + k, v);
    } else {
        const uint32_t c = static_cast<const uint32_t*>(t.data)[row * (K / 8) + k / 8];
        const int64_t g = row * (K / 64) + k / 64;
        const float s = bf16_bits_to_f32(t.scales[g]);
        const float b = bf16_bits_to_f32(t.biases[g]);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = s * (float)((c >> (4 * j)) & 15u) + b;
    }
}

// PRO_NORM source row m: below M1 from x, the rest from x2 (the fused QKV and context K/V pass)
__device__ __forceinline__ const float* norm_row(const GemvParams& p, int m) {
    return (p.x2 && m >= p.M1) ? p.x2 + (int64_t)(m - p.M1) * p.x_ld : p.x + (int64_t)m * p.x_ld;
}

template <int PRO>
__device__ __forceinline__ void load_x8(const GemvParams& p, int layer, int m, int k, const float* rinv,
                                        float (&v)[8]) {
    if (m >= p.M) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
        return;
    }
    if constexpr (PRO == PRO_PLAIN) {
        const int64_t off = (int64_t)layer * p.x_layer_stride + (int64_t)m * p.x_ld + k;
        if (p.src_f32)
            load8_f32(p.x + off, v);
        else
            load8_bf16(reinterpret_cast<const uint16_t*>(p.x) + off, v);
    } else if constexpr (PRO == PRO_NORM) {
        load8_f32(norm_row(p, m) + k, v);
        const float r = rinv[m];
        const void* g = p.gain[layer];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * r * load_gain(g, p.gain_f32, k + j);
    } else if constexpr (PRO == PRO_TAPS) {
        const int j = k / p.H, kk = k - j * p.H;
        if (p.src_f32)
            load8_f32(static_cast<const float*>(p.taps[j]) + (int64_t)m * p.tap_ld + kk, v);
        else
            load8_bf16(static_cast<const uint16_t*>(p.taps[j]) + (int64_t)m * p.tap_ld + kk, v);
    } else {  // PRO_GATHER
        const int id = min(max(p.ids[m], 0), p.table_rows - 1);
        load8_weight_row(p.table, p.table_type, (int64_t)id, p.K, k, v);
    }
}

// stage activation rows [0, MAXM) x [kc0, kc0 + kw) into LDS
template <int WT, int PRO, int MAXM>
__device__ __forceinline__ void stage(const GemvParams& p, int layer, int kc0, int kw, int KC,
                                      typename WTraits<WT>::X* xs, float* xsum, const float* rinv) {
    const int tid = threadIdx.x;
    if constexpr (WT == W_I4) {
        const int units = kw / 32;
        for (int u = tid; u < MAXM * units; u += kBlock) {
            const int m = u / units, c = u - m * units;
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[8];
                load_x8<PRO>(p, layer, m, kc0 + 32 * c + 8 * q, rinv, v);
                uint32_t b[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    b[j] = f32_to_bf16_bits(v[j]);
                    s += bf16_bits_to_f32(b[j]);
                }
                // pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7): the nibble pairing of a code word
                uint4 o;
                o.x = b[0] | (b[4] << 16);
                o.y = b[1] | (b[5] << 16);
                o.z = b[2] | (b[6] << 16);
                o.w = b[3] | (b[7] << 16);
                *reinterpret_cast<uint4*>(xs + (size_t)m * KC + 32 * c + 8 * q) = o;
            }
            xsum[m * (KC / 32) + c] = s;
        }
    } else {
        const int units = kw / 8;
#pragma unroll 4
        for (int u = tid; u < MAXM * units; u += kBlock) {
            const int m = u / units, c = u - m * units;
            float v[8];
            load_x8<PRO>(p, layer, m, kc0 + 8 * c, rinv, v);
            if constexpr (WT == W_BF16) {
                uint4 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                o.z = pack_bf16x2(v[4], v[5]);
                o.w = pack_bf16x2(v[6], v[7]);
                *reinterpret_cast<uint4*>(xs + (size_t)m * KC + 8 * c) = o;
            } else {
                float* d = xs + (size_t)m * KC + 8 * c;
                *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
    }
}

template <int EPI, int RPW>
__device__ __forceinline__ void tile_rows(const GemvParams& p, int tile, int wave, int64_t (&rows)[RPW]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        int64_t row;
        bool ok;
        if constexpr (EPI == EPI_GATED) {
            const int j = tile * 2 * RPW + wave * (RPW / 2) + r / 2;
            ok = j < p.F;
            row = (r & 1) ? (int64_t)p.F + j : (int64_t)j;
        } else {
            const int n = tile * 4 * RPW + wave * RPW + r;
            ok = n < p.N;
            row = n;
        }
        rows[r] = p.w_row0 + (ok ? row : 0);
    }
}

// ---------------------------------------------------------------------------

template <int WT, int PRO, int EPI, int MAXM, int RPW>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const GemvParams p, const int KC) {
    typedef typename WTraits<WT>::X X;
    constexpr int EPL = WTraits<WT>::EPL;
    constexpr int STEP = 64 * EPL;
    // weight iterations kept in flight
    constexpr int PF = (EPI == EPI_ARGMAX && WT != W_I4) ? DFL_PF_HEAD : (RPW >= 4 ? DFL_PF_WIDE : DFL_PF);
    extern __shared__ __align__(16) unsigned char smem[];
    X* xs = reinterpret_cast<X*>(smem);                                                 // [MAXM][KC]
    float* xsum = reinterpret_cast<float*>(smem + (size_t)MAXM * KC * sizeof(X));       // [MAXM][KC/32]
    float* red = xsum + (WT == W_I4 ? MAXM * (KC / 32) : 0);                            // [4*RPW][MAXM]
    float* rinv = red + 4 * RPW * MAXM;                                                 // [MAXM]

    const uint64_t t_start = trace_start(p.stamps);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int layer = blockIdx.y;
    const WeightPtr W = p.w[layer];
    const int K = p.K;
    const int kb = blockIdx.z * p.kslice;
    const int ke = min(K, kb + p.kslice);
    const int kw0 = min(KC, ke - kb);
    const bool single = (ke - kb) <= KC;
    const int ntiles = (EPI == EPI_GATED) ? (p.F + 2 * RPW - 1) / (2 * RPW) : (p.N + 4 * RPW - 1) / (4 * RPW);

    int tile = blockIdx.x;
    int64_t rows[RPW];
    tile_rows<EPI, RPW>(p, tile, wave, rows);

    // iterations of this lane in chunk 0
    const int nit = (kw0 > lane * EPL) ? (kw0 - lane * EPL + STEP - 1) / STEP : 0;

    // LM head over bf16 rows: the activation rows go out before the weights. Loads return
    // in issue order, so staged after the weight prefetch they would wait behind it and
    // hold back the first products; issued first, they land while the weights stream.
    // Up to kYB 16-byte chunks per thread; a longer head stages as below.
    constexpr bool kHeadY = EPI == EPI_ARGMAX && WT == W_BF16 && PRO == PRO_TAPS;
    constexpr int kYB = 8;
    u32x4 yreg[kHeadY ? kYB : 1];
    const int yunits = kw0 / 8;
    const bool yfast = kHeadY && !p.src_f32 && p.M > 0 && (kw0 % 8) == 0 && p.M * yunits <= kYB * kBlock;
    if constexpr (kHeadY) {
        if (yfast) {
            const uint16_t* y = static_cast<const uint16_t*>(p.taps[0]);
#pragma unroll
            for (int i = 0; i < kYB; ++i) {
                const int u = min(tid + i * kBlock, p.M * yunits - 1);
                const int m = u / yunits, c = u - m * yunits;
                yreg[i] = *reinterpret_cast<const u32x4*>(y + (int64_t)m * p.tap_ld + kb + 8 * c);
            }
        }
    }

    // first PF weight iterations of this tile, in flight before the prologue (after the
    // activation loads above, all PF go out, lanes past the K range re-reading its last
    // chunk: a fixed count lets the wait for the activations leave them in flight; a
    // head staged the usual way keeps the per-lane guard, measured faster there)
    WChunk<WT> pre[PF][RPW];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        if (kHeadY && yfast) {
            const int kk = min(kb + lane * EPL + i * STEP, ke - EPL);
#pragma unroll
            for (int r = 0; r < RPW; ++r) wload<WT>(pre[i][r], W, rows[r], K, kk);
        } else if (i < nit) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) wload<WT>(pre[i][r], W, rows[r], K, kb + lane * EPL + i * STEP);
        }
    }

    // EPI_RESID: this thread's first residual value (first tile, first epilogue slot) is
    // read now, alongside the weights, instead of after the reduction. Each output is
    // owned by one workgroup and the residual stream is not this launch's input.
    const int first_tile = tile;
    float rpre = 0.f;
    if constexpr (EPI == EPI_RESID) {
        if (tid < 4 * RPW * MAXM) {
            const int m = tid / (4 * RPW), n = tile * 4 * RPW + (tid - m * 4 * RPW);
            if (m < p.M && n < p.N) rpre = p.out[(int64_t)m * p.out_ld + n];
        }
    }

    // EPI_KV: sequence and cache position of each activation row, resolved once
    int* meta_b = reinterpret_cast<int*>(rinv + MAXM);
    int* meta_pos = meta_b + MAXM;
    if constexpr (EPI == EPI_KV || EPI == EPI_QKVKV) {
        if (tid < MAXM) {
            int b = 0, pos = -1;
            const int m0 = EPI == EPI_QKVKV ? p.M1 : 0;  // the first context row
            if (tid < p.M && tid >= m0) {
                const int gm = p.row_base + tid - m0;
                while (b + 1 < p.B && p.row_offsets[b + 1] <= gm) ++b;
                const int rows_b = p.row_offsets[b + 1] - p.row_offsets[b];
                const int i = gm - p.row_offsets[b];
                const int cnt = p.counts ? min(p.counts[b], rows_b) : rows_b;
                pos = p.len[b] + i;
                if (!(i >= 0 && i < cnt && pos < p.cap)) pos = -1;
            }
            meta_b[tid] = b;
            meta_pos[tid] = pos;
        }
    }

    constexpr bool kRegNorm = (PRO == PRO_NORM) && (WT != W_I4) && (MAXM == 8 || MAXM == 16);
    if (kHeadY && yfast) {
        // rows at or past M stay unwritten: their products land in accumulator slots that
        // never reach a result
        uint16_t* xb = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
        for (int i = 0; i < (kHeadY ? kYB : 1); ++i) {
            const int u = tid + i * kBlock;
            if (u < p.M * yunits) {
                const int m = u / yunits, c = u - m * yunits;
                *reinterpret_cast<u32x4*>(xb + (size_t)m * KC + 8 * c) = yreg[i];
            }
        }
        __syncthreads();
    } else if (kRegNorm && single && K <= kRegNormMaxK) {
        // one round trip: each wavefront loads whole rows and the matching gains
        // into registers, reduces the sum of squares with shuffles and writes the
        // normalised, rounded row to LDS
        constexpr int RW = MAXM / 4, UM = kRegNormMaxK / 512;
        float xr[RW][UM][8];
        float gr[UM][8];
#pragma unroll
        for (int u = 0; u < UM; ++u) {
            const int k = lane * 8 + u * 512;
            if (k < K) {
                load_gain8(p.gain[layer], p.gain_f32, k, gr[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) gr[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int m = wave + 4 * j;
#pragma unroll
            for (int u = 0; u < UM; ++u) {
                const int k = lane * 8 + u * 512;
                if (m < p.M && k < K) {
                    load8_f32(norm_row(p, m) + k, xr[j][u]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xr[j][u][e] = 0.f;
                }
            }
        }
        float rr[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            float ss = 0.f;
#pragma unroll
            for (int u = 0; u < UM; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += xr[j][u][e] * xr[j][u][e];
            ss = wave_sum(ss);
            rr[j] = 1.0f / sqrtf(ss / (float)K + p.eps);
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int m = wave + 4 * j;
#pragma unroll
            for (int u = 0; u < UM; ++u) {
                const int k = lane * 8 + u * 512;
                if (k < K) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (m < p.M) ? xr[j][u][e] * rr[j] * gr[u][e] : 0.f;
                    if constexpr (WT == W_BF16) {
                        uint4 o;
                        o.x = pack_bf16x2(v[0], v[1]);
                        o.y = pack_bf16x2(v[2], v[3]);
                        o.z = pack_bf16x2(v[4], v[5]);
                        o.w = pack_bf16x2(v[6], v[7]);
                        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(xs) + (size_t)m * KC + k) = o;
                    } else {
                        float* d = reinterpret_cast<float*>(xs) + (size_t)m * KC + k;
                        *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
                        *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
                    }
                }
            }
        }
        __syncthreads();
    } else {
        if constexpr (PRO == PRO_NORM) {
            for (int m = wave; m < p.M; m += 4) {
                const float* xr = norm_row(p, m);
                float s = 0.f;
                for (int k = lane * 4; k < K; k += 256) {
                    const float4 a = *reinterpret_cast<const float4*>(xr + k);
                    s += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
                }
                s = wave_sum(s);
                if (lane == 0) rinv[m] = 1.0f / sqrtf(s / (float)K + p.eps);
            }
            __syncthreads();
        }
        stage<WT, PRO, MAXM>(p, layer, kb, kw0, KC, xs, xsum, rinv);
        __syncthreads();
    }

    // per-workgroup running argmax over all of its tiles
    float amax = -INFINITY;
    int aidx = 0x7fffffff;

    while (true) {
        float acc[RPW][MAXM];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
            for (int m = 0; m < MAXM; ++m) acc[r][m] = 0.f;

        // chunk 0: a ring of PF register slots keeps PF weight iterations in
        // flight; the slot just consumed is refilled with iteration it + PF
        for (int base = 0; base < nit; base += PF) {
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int it = base + i;
                if (it < nit) {
                    wfma<WT, MAXM, RPW>(pre[i], xs, KC, lane * EPL + it * STEP, xsum, acc);
                    const int nx = it + PF;
                    if (nx < nit) {
#pragma unroll
                        for (int r = 0; r < RPW; ++r) wload<WT>(pre[i][r], W, rows[r], K, kb + lane * EPL + nx * STEP);
                    }
                }
            }
        }
        // further chunks (long K ranges; such launches have one tile per workgroup)
        for (int kc0 = kb + kw0; kc0 < ke; kc0 += KC) {
            const int kw = min(KC, ke - kc0);
            __syncthreads();
            stage<WT, PRO, MAXM>(p, layer, kc0, kw, KC, xs, xsum, rinv);
            __syncthreads();
            for (int k = kc0 + lane * EPL; k < kc0 + kw; k += STEP) {
                WChunk<WT> w[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r) wload<WT>(w[r], W, rows[r], K, k);
                wfma<WT, MAXM, RPW>(w, xs, KC, k - kc0, xsum, acc);
            }
        }

        // next tile's first iterations go out before this tile's reduction
        const int next = tile + (int)gridDim.x;
        const bool more = single && next < ntiles;
        if (more) {
            tile_rows<EPI, RPW>(p, next, wave, rows);
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                if (i < nit) {
#pragma unroll
                    for (int r = 0; r < RPW; ++r) wload<WT>(pre[i][r], W, rows[r], K, kb + lane * EPL + i * STEP);
                }
            }
        }

        // ---- reduce across the wavefront; sums land in red[wave*RPW + r][m]
        {
            constexpr int NV = RPW * MAXM;
            float vals[NV];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
#pragma unroll
                for (int m = 0; m < MAXM; ++m) vals[r * MAXM + m] = acc[r][m];
            const float tot = wave_sum_many<NV>(vals, lane);
            const int vi = wave_sum_many_index<NV>(lane);
            constexpr int SPAN = (NV >= 64) ? 1 : 64 / NV;
            if constexpr (EPI == EPI_ARGMAX) {
                // each lane keeps a running (max, lowest index) for its (row slot r, activation
                // row m) across the workgroup's tiles; the wavefronts are combined once at the end
                const int r = vi / MAXM, m = vi - r * MAXM;
                const int n = tile * 4 * RPW + wave * RPW + r;
                if ((lane % SPAN) == 0 && m < p.M && n < p.N)
                    argmax_pick(amax, aidx, p.base ? tot + p.base[(int64_t)m * p.base_ld + n] : tot, n);
            } else {
                if ((lane % SPAN) == 0) red[(wave * RPW) * MAXM + vi] = tot;
            }
        }
        if constexpr (EPI != EPI_ARGMAX) __syncthreads();

        // ---- epilogue of this tile (the argmax epilogue runs after the last tile)
        if constexpr (EPI == EPI_ARGMAX) {
        } else if constexpr (EPI == EPI_GATED) {
            for (int t = tid; t < 2 * RPW * MAXM; t += kBlock) {
                const int m = t / (2 * RPW), q = t - m * (2 * RPW);
                const int j = tile * 2 * RPW + q;
                if (m >= p.M || j >= p.F) continue;
                const float g = red[(2 * q) * MAXM + m], u = red[(2 * q + 1) * MAXM + m];
                const float y = (p.act == 0 ? gelu_tanh(g) : silu(g)) * u;
                if (p.round_out)
                    reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.out_ld + j] = (uint16_t)f32_to_bf16_bits(y);
                else
                    p.out[(int64_t)m * p.out_ld + j] = y;
            }
        } else {
            for (int t = tid; t < 4 * RPW * MAXM; t += kBlock) {
                const int m = t / (4 * RPW), u = t - m * (4 * RPW);
                const int n = tile * 4 * RPW + u;
                if (m >= p.M || n >= p.N) continue;
                const float y = red[u * MAXM + m];
                if constexpr (EPI == EPI_STORE) {
                    if (p.out_bf16) {
                        if (p.vt && n >= p.vt_col) {
                            const int row = p.row_base + m, bb = row / p.gamma, key = row - bb * p.gamma;
                            const int c = n - p.vt_col, head = c / p.hd, dim = c - head * p.hd;
                            p.vt[(((int64_t)bb * p.hkv + head) * p.hd + dim) * 32 + key] = (uint16_t)f32_to_bf16_bits(y);
                        } else {
                            uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + (int64_t)blockIdx.z * p.split_stride;
                            o[(int64_t)m * p.out_ld + n] = (uint16_t)f32_to_bf16_bits(y);
                        }
                    } else {
                        float* o = p.out + ((int64_t)layer * gridDim.z + blockIdx.z) * p.split_stride;
                        o[(int64_t)m * p.out_ld + n] = p.round_out ? round_bf16(y) : y;
                    }
                } else if constexpr (EPI == EPI_QKVKV) {
                    if (m < p.M1) {  // block row: Q | K_b | V_b
                        if (p.out_bf16) {
                            if (n >= p.vt_col) {
                                const int row = p.row_base + m, bb = row / p.gamma, key = row - bb * p.gamma;
                                const int c = n - p.vt_col, head = c / p.hd, dim = c - head * p.hd;
                                p.vt[(((int64_t)bb * p.hkv + head) * p.hd + dim) * 32 + key] =
                                    (uint16_t)f32_to_bf16_bits(y);
                            } else {
                                reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.out_ld + n] =
                                    (uint16_t)f32_to_bf16_bits(y);
                            }
                        } else {
                            p.out[(int64_t)m * p.out_ld + n] = y;
                        }
                    } else if (n >= p.kv_col0) {  // context row: its key or value into the cache
                        const int b = meta_b[m], pos = meta_pos[m];
                        if (pos >= 0) {
                            const int kvw = p.hkv * p.hd, c = n - p.kv_col0;
                            const int which = c / kvw;
                            const int head = (c - which * kvw) / p.hd;
                            const int dim = c - which * kvw - head * p.hd;
                            const int64_t hb = ((int64_t)b * p.hkv + head) * p.cap * p.hd;
                            const int64_t off = (int64_t)layer * p.layer_stride + hb +
                                                (which ? v_cache_off(pos, dim, p.hd, p.cap, p.kv_f32) : (int64_t)pos * p.hd + dim);
                            void* base = which ? p.vcache : p.kcache;
                            if (p.kv_f32)
                                static_cast<float*>(base)[off] = y;
                            else
                                static_cast<uint16_t*>(base)[off] = (uint16_t)f32_to_bf16_bits(y);
                        }
                    }
                } else if constexpr (EPI == EPI_RESID) {
                    float* o = p.out + (int64_t)m * p.out_ld + n;
                    *o = ((t == tid && tile == first_tile) ? rpre : *o) + y;
                } else if constexpr (EPI == EPI_BLOCKINIT) {
                    const int64_t b = p.seq_base + m;
                    const int d = p.N;
                    float* hb = p.out + b * (int64_t)p.gamma * d;
                    hb[n] = y + load_gain(p.block_pos, p.gain_f32, n);
                    for (int kk = 1; kk < p.gamma; ++kk)
                        hb[(int64_t)kk * d + n] = load_gain(p.mask_emb, p.gain_f32, (kk - 1) * d + n) +
                                                  load_gain(p.block_pos, p.gain_f32, kk * d + n);
                } else if constexpr (EPI == EPI_KV) {
                    const int b = meta_b[m], pos = meta_pos[m];
                    if (pos >= 0) {
                        const int kvw = p.hkv * p.hd;
                        const int which = n / kvw;
                        const int head = (n - which * kvw) / p.hd;
                        const int dim = n - which * kvw - head * p.hd;
                        // keys [B][hkv][cap][hd]; values in the value-cache layout (v_cache_off)
                        const int64_t hb = ((int64_t)b * p.hkv + head) * p.cap * p.hd;
                        const int64_t off = (int64_t)layer * p.layer_stride + hb +
                                            (which ? v_cache_off(pos, dim, p.hd, p.cap, p.kv_f32) : (int64_t)pos * p.hd + dim);
                        void* base = which ? p.vcache : p.kcache;
                        if (p.kv_f32)
                            static_cast<float*>(base)[off] = y;
                        else
                            static_cast<uint16_t*>(base)[off] = (uint16_t)f32_to_bf16_bits(y);
                    }
                }
            }
        }
        if (!more) break;
        tile = next;
        if constexpr (EPI != EPI_ARGMAX) __syncthreads();  // red[] is rewritten by the next tile
    }

    if constexpr (EPI == EPI_ARGMAX) {
        // combine the running (max, index) of every wavefront lane slot per activation row
        constexpr int NV = RPW * MAXM;
        constexpr int SPAN = (NV >= 64) ? 1 : 64 / NV;
        // the activation staging area (at least MAXM * 32 elements, >= 8 * NV bytes) is free once
        // every wavefront has finished its last tile
        __syncthreads();
        float* rv = reinterpret_cast<float*>(smem);               // [4][NV]
        int* ri = reinterpret_cast<int*>(smem) + 4 * NV;          // [4][NV]
        if ((lane % SPAN) == 0) {
            const int vi = wave_sum_many_index<NV>(lane);
            rv[wave * NV + vi] = amax;
            ri[wave * NV + vi] = aidx;
        }
        __syncthreads();
        if (tid < p.M) {
            float v = -INFINITY;
            int i = 0x7fffffff;
            for (int w = 0; w < 4; ++w)
                for (int r = 0; r < RPW; ++r) argmax_pick(v, i, rv[w * NV + r * MAXM + tid], ri[w * NV + r * MAXM + tid]);
            p.part_val[(int64_t)tid * p.nblocks + blockIdx.x] = v;
            p.part_idx[(int64_t)tid * p.nblocks + blockIdx.x] = i;
        }
    }
    trace_end(p.stamps, t_start);
}

// ---------------------------------------------------------------------------
// host dispatch

// LDS staging of the activation rows. Reductions up to the normal budget stage
// once and run the requested persistent grid; longer ones up to the wide budget
// (one workgroup per CU) stage once and run one persistent workgroup per CU;
// longer still, one workgroup per row tile stages chunk by chunk.
constexpr int kStageBytesWide = 136 * 1024;

static int num_cus() {
    static int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            return 256;
        return v;
    }();
    return n;
}

template <int WT, int MAXM>
static int stage_cols(int budget) {
    typedef typename WTraits<WT>::X X;
    return (budget / (MAXM * (int)sizeof(X))) / 512 * 512;
}

struct StagePlan {
    int KC;       // staged K elements per pass
    int max_wgs;  // persistent workgroup cap (0: one per tile)
};

template <int WT, int MAXM>
static StagePlan stage_plan(int kslice, int max_wgs) {
    const int kc = stage_cols<WT, MAXM>(kStageBytes);
    if (kslice <= kc) return {kc, max_wgs};
    const int kw = stage_cols<WT, MAXM>(kStageBytesWide);
    if (max_wgs > 0 && kslice <= kw) return {kw, max_wgs < num_cus() ? max_wgs : num_cus()};
    return {kc, max_wgs};
}

template <int WT, int MAXM>
static int head_grid_t(int K, int ntiles, int max_wgs) {
    const StagePlan sp = stage_plan<WT, MAXM>(K, max_wgs);
    return (sp.max_wgs > 0 && K <= sp.KC && ntiles > sp.max_wgs) ? sp.max_wgs : ntiles;
}

int gemv_head_grid(int wtype, int K, int ntiles, int max_wgs, int rows) {
    switch (wtype) {
        case W_F32: return head_grid_t<W_F32, 8>(K, ntiles, max_wgs);
        case W_BF16: return head_grid_t<W_BF16, 8>(K, ntiles, max_wgs);
        case W_I4:
            return gemv_maxm(W_I4, rows) == 4 ? head_grid_t<W_I4, 4>(K, ntiles, max_wgs)
                                              : head_grid_t<W_I4, 8>(K, ntiles, max_wgs);
    }
    return 0;
}

template <int WT, int PRO, int EPI, int MAXM, int RPW>
static hipError_t launch_one(const GemvParams& p, int layers, hipStream_t s) {
    typedef typename WTraits<WT>::X X;
    const int unit = (WT == W_I4) ? 32 : 8;
    GemvParams q = p;
    if (q.ksplit < 1) q.ksplit = 1;
    if (q.kslice <= 0 || q.ksplit == 1) q.kslice = q.K;
    const StagePlan sp = stage_plan<WT, MAXM>(q.kslice, q.max_wgs);
    q.max_wgs = sp.max_wgs;
    int KC = sp.KC;
    if (KC >= q.kslice) KC = q.kslice;
    KC = (KC + unit - 1) / unit * unit;
    size_t smem = (size_t)MAXM * KC * sizeof(X) + (WT == W_I4 ? (size_t)MAXM * (KC / 32) * 4 : 0) +
                  (size_t)4 * RPW * MAXM * 4 + (size_t)MAXM * 4 + (size_t)2 * MAXM * 4;
    // the argmax epilogue combines its wavefronts' (value, index) slots at the start of LDS
    if (EPI == EPI_ARGMAX && smem < (size_t)8 * 4 * RPW * MAXM) smem = (size_t)8 * 4 * RPW * MAXM;
    const int ntiles = (EPI == EPI_GATED) ? (q.F + 2 * RPW - 1) / (2 * RPW) : (q.N + 4 * RPW - 1) / (4 * RPW);
    int grid_x = ntiles;
    // persistent tiles only when the K range is staged once
    if (q.max_wgs > 0 && q.kslice <= KC && grid_x > q.max_wgs) grid_x = q.max_wgs;
    if (EPI == EPI_ARGMAX && q.nblocks != grid_x) return hipErrorInvalidValue;  // partial buffer layout
    dim3 grid(grid_x, layers, q.ksplit);
    {  // instrumentation: algorithmic bytes = weights + activation rows + outputs
        const double wb = WT == W_F32 ? 4.0 : (WT == W_BF16 ? 2.0 : 0.5 + 4.0 / 64);
        const double xb = q.src_f32 ? 4.0 : 2.0;
        const double nout = EPI == EPI_GATED ? q.F : (EPI == EPI_ARGMAX ? 0 : q.N);
        const double bytes = layers * ((double)q.N * q.K * wb + (double)q.M * q.K * xb + (double)q.M * nout * 4.0);
        char name[64];
        snprintf(name, sizeof name, "gemv_kernel<%d, %d, %d, %d, %d>", WT, PRO, EPI, MAXM, RPW);
        q.stamps = trace_launch(EPI == EPI_ARGMAX ? TRACE_LM_HEAD : TRACE_PROJECTIONS, name,
                                (int64_t)grid_x * layers * q.ksplit, bytes, 0.0);
    }
    // allow dynamic LDS beyond the 64 KiB default (gfx950 has 160 KiB per CU)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemv_kernel<WT, PRO, EPI, MAXM, RPW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL((gemv_kernel<WT, PRO, EPI, MAXM, RPW>), grid, dim3(kBlock), smem, s, q, KC);
    return hipGetLastError();
}

template <int WT, int PRO, int EPI, int MAXM>
static hipError_t launch_rpw(const GemvParams& p, int layers, hipStream_t s) {
    if constexpr (MAXM <= 8) {
        if (p.rpw >= 4) return launch_one<WT, PRO, EPI, MAXM, 4>(p, layers, s);
        if (p.rpw == 2 || EPI == EPI_GATED) return launch_one<WT, PRO, EPI, MAXM, 2>(p, layers, s);
        if constexpr (EPI != EPI_GATED) return launch_one<WT, PRO, EPI, MAXM, 1>(p, layers, s);
    } else {
        if (p.rpw >= 2 || EPI == EPI_GATED) return launch_one<WT, PRO, EPI, MAXM, 2>(p, layers, s);
        if constexpr (EPI != EPI_GATED) return launch_one<WT, PRO, EPI, MAXM, 1>(p, layers, s);
    }
    return hipErrorInvalidValue;
}

template <int PRO, int EPI, int MAXM>
static hipError_t launch_wt(int wtype, const GemvParams& p, int layers, hipStream_t s, int maxm) {
    if constexpr (MAXM == 8) {
        if (maxm == 4 && wtype == W_I4) return launch_rpw<W_I4, PRO, EPI, 4>(p, layers, s);
        if constexpr (PRO == PRO_GATHER && EPI == EPI_BLOCKINIT)
            if (maxm == 4 && wtype == W_BF16) return launch_rpw<W_BF16, PRO, EPI, 4>(p, layers, s);
    }
    switch (wtype) {
        case W_F32: return launch_rpw<W_F32, PRO, EPI, MAXM>(p, layers, s);
        case W_BF16: return launch_rpw<W_BF16, PRO, EPI, MAXM>(p, layers, s);
        case W_I4: return launch_rpw<W_I4, PRO, EPI, MAXM>(p, layers, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int wtype, int pro, int epi, int maxm, const GemvParams& p, int layers, hipStream_t s) {
    // 4-row kernels: int4 weights, and the bf16 block init (one anchor row per sequence)
    if (maxm == 4 && (p.M > 4 || !(wtype == W_I4 || (wtype == W_BF16 && pro == PRO_GATHER && epi == EPI_BLOCKINIT))))
        return hipErrorInvalidValue;
#define DFL_CASE(PRO, EPI)                                                                      \
    if (pro == PRO && epi == EPI) {                                                             \
        return maxm <= 8 ? launch_wt<PRO, EPI, 8>(wtype, p, layers, s, maxm)                          \
                         : launch_wt<PRO, EPI, 32>(wtype, p, layers, s, maxm);                        \
    }
    DFL_CASE(PRO_TAPS, EPI_STORE)
    DFL_CASE(PRO_NORM, EPI_KV)
    DFL_CASE(PRO_PLAIN, EPI_KV)
    if (pro == PRO_GATHER && epi == EPI_BLOCKINIT) return launch_wt<PRO_GATHER, EPI_BLOCKINIT, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_NORM && epi == EPI_STORE) return launch_wt<PRO_NORM, EPI_STORE, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_PLAIN && epi == EPI_RESID) return launch_wt<PRO_PLAIN, EPI_RESID, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_PLAIN && epi == EPI_STORE) return launch_wt<PRO_PLAIN, EPI_STORE, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_PLAIN && epi == EPI_GATED) return launch_wt<PRO_PLAIN, EPI_GATED, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_NORM && epi == EPI_GATED) return launch_wt<PRO_NORM, EPI_GATED, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_TAPS && epi == EPI_ARGMAX) return launch_wt<PRO_TAPS, EPI_ARGMAX, 8>(wtype, p, layers, s, maxm);
    if (pro == PRO_NORM && epi == EPI_QKVKV && maxm == 16 && wtype != W_I4)
        return launch_wt<PRO_NORM, EPI_QKVKV, 16>(wtype, p, layers, s, maxm);
#undef DFL_CASE
    return hipErrorInvalidValue;
}

}  // namespace dfl
