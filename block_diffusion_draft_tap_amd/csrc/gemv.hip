// Skinny GEMV family for the drafter projections (see gemv.hpp for the modes).
//
// Work split: a workgroup of 4 wavefronts owns 4*RPW consecutive weight rows
// (for the gated FFN: 2*RPW gate/up row pairs) and reads each of them exactly
// once over the full K range. Lane l of a wavefront reads the 16-byte chunk
// at k = l*EPL + 64*EPL*i of each of its rows, so a wavefront instruction
// covers one contiguous 1 KiB (bf16) or 512 B (int4) run of a row. The
// activation rows are staged in LDS once per K chunk and read back as 16-byte
// vectors that match the weight chunk lane by lane.
//
// Products: bf16 weights use v_dot2 (two bf16 products per instruction into
// an fp32 accumulator); int4 weights are turned into bf16 (128 + q) pairs with
// two integer ops per pair and use the same v_dot2, with
//   sum_k x_k (s q_k + b) = s sum_k x_k (128 + q_k) + (b - 128 s) sum_k x_k
// evaluated per 32-element lane chunk (the activation sums are staged with
// the activations); fp32 weights use plain fp32 FMAs.
#include "common.hpp"
#include "gemv.hpp"

namespace dfl {

template <int WT> struct WTraits;
template <> struct WTraits<W_F32> { typedef float X; static constexpr int EPL = 8; };
template <> struct WTraits<W_BF16> { typedef uint16_t X; static constexpr int EPL = 8; };
template <> struct WTraits<W_I4> { typedef uint16_t X; static constexpr int EPL = 32; };

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

template <int PRO>
__device__ __forceinline__ void load_x8(const GemvParams& p, int layer, int m, int k, const float* rinv,
                                        float (&v)[8]) {
    if (m >= p.M) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
        return;
    }
    if constexpr (PRO == PRO_PLAIN) {
        load8_f32(p.x + (int64_t)m * p.x_ld + k, v);
    } else if constexpr (PRO == PRO_NORM) {
        load8_f32(p.x + (int64_t)m * p.x_ld + k, v);
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

// ---------------------------------------------------------------------------

template <int WT, int PRO, int EPI, int MAXM, int RPW>
__global__ __launch_bounds__(kBlock) void gemv_kernel(const GemvParams p, const int KC) {
    typedef typename WTraits<WT>::X X;
    constexpr int EPL = WTraits<WT>::EPL;
    constexpr bool kBf = (WT != W_F32);
    extern __shared__ __align__(16) unsigned char smem[];
    X* xs = reinterpret_cast<X*>(smem);                                     // [MAXM][KC]
    float* xsum = reinterpret_cast<float*>(smem + (size_t)MAXM * KC * sizeof(X));  // [MAXM][KC/32]
    float* red = xsum + (WT == W_I4 ? MAXM * (KC / 32) : 0);                // [4*RPW][MAXM]
    float* rinv = red + 4 * RPW * MAXM;                                     // [MAXM]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int layer = blockIdx.y;
    const WeightPtr W = p.w[layer];
    const int K = p.K;

    // weight rows of this wavefront
    int64_t rows[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        int64_t row;
        bool ok;
        if constexpr (EPI == EPI_GATED) {
            const int j = blockIdx.x * 2 * RPW + wave * (RPW / 2) + r / 2;
            ok = j < p.F;
            row = (r & 1) ? (int64_t)p.F + j : (int64_t)j;
        } else {
            const int n = blockIdx.x * 4 * RPW + wave * RPW + r;
            ok = n < p.N;
            row = n;
        }
        rows[r] = p.w_row0 + (ok ? row : 0);
    }

    if constexpr (PRO == PRO_NORM) {
        for (int m = wave; m < p.M; m += 4) {
            const float* xr = p.x + (int64_t)m * p.x_ld;
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

    float acc[RPW][MAXM];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int m = 0; m < MAXM; ++m) acc[r][m] = 0.f;

    for (int kc0 = 0; kc0 < K; kc0 += KC) {
        const int kw = min(KC, K - kc0);
        __syncthreads();
        // ---- stage activation rows [0, MAXM) x [kc0, kc0+kw) into LDS
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
            for (int u = tid; u < MAXM * units; u += kBlock) {
                const int m = u / units, c = u - m * units;
                float v[8];
                load_x8<PRO>(p, layer, m, kc0 + 8 * c, rinv, v);
                if constexpr (kBf) {
                    uint4 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    o.z = pack_bf16x2(v[4], v[5]);
                    o.w = pack_bf16x2(v[6], v[7]);
                    *reinterpret_cast<uint4*>(xs + (size_t)m * KC + 8 * c) = o;
                } else {
                    float* d = reinterpret_cast<float*>(xs) + (size_t)m * KC + 8 * c;
                    *reinterpret_cast<float4*>(d) = make_float4(v[0], v[1], v[2], v[3]);
                    *reinterpret_cast<float4*>(d + 4) = make_float4(v[4], v[5], v[6], v[7]);
                }
            }
        }
        __syncthreads();

        // ---- stream the weight rows over this chunk
        for (int k = kc0 + lane * EPL; k < kc0 + kw; k += 64 * EPL) {
            const int kl = k - kc0;
            if constexpr (WT == W_BF16) {
                uint4 wv[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r)
                    wv[r] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W.data) + rows[r] * K + k);
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)m * KC + kl);
#pragma unroll
                    for (int r = 0; r < RPW; ++r) {
                        float a = acc[r][m];
                        a = dot2_bf16(wv[r].x, xv.x, a);
                        a = dot2_bf16(wv[r].y, xv.y, a);
                        a = dot2_bf16(wv[r].z, xv.z, a);
                        a = dot2_bf16(wv[r].w, xv.w, a);
                        acc[r][m] = a;
                    }
                }
            } else if constexpr (WT == W_F32) {
                float4 w0[RPW], w1[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const float* src = static_cast<const float*>(W.data) + rows[r] * K + k;
                    w0[r] = *reinterpret_cast<const float4*>(src);
                    w1[r] = *reinterpret_cast<const float4*>(src + 4);
                }
#pragma unroll
                for (int m = 0; m < MAXM; ++m) {
                    const float* xr = reinterpret_cast<const float*>(xs) + (size_t)m * KC + kl;
                    const float4 x0 = *reinterpret_cast<const float4*>(xr);
                    const float4 x1 = *reinterpret_cast<const float4*>(xr + 4);
#pragma unroll
                    for (int r = 0; r < RPW; ++r) {
                        float a = acc[r][m];
                        a = fmaf(w0[r].x, x0.x, a); a = fmaf(w0[r].y, x0.y, a);
                        a = fmaf(w0[r].z, x0.z, a); a = fmaf(w0[r].w, x0.w, a);
                        a = fmaf(w1[r].x, x1.x, a); a = fmaf(w1[r].y, x1.y, a);
                        a = fmaf(w1[r].z, x1.z, a); a = fmaf(w1[r].w, x1.w, a);
                        acc[r][m] = a;
                    }
                }
            } else {  // W_I4
                uint32_t pr[RPW][16];
                float sc[RPW], bi[RPW];
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    const uint4 cw = *reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(W.data) +
                                                                     rows[r] * (K / 8) + k / 8);
                    const int64_t g = rows[r] * (K / 64) + k / 64;
                    sc[r] = bf16_bits_to_f32(W.scales[g]);
                    bi[r] = bf16_bits_to_f32(W.biases[g]) - 128.0f * sc[r];
                    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            pr[r][4 * wd + j] = ((words[wd] >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
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
                    for (int r = 0; r < RPW; ++r) acc[r][m] += sc[r] * d[r] + bi[r] * xsm;
                }
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
        if ((lane % SPAN) == 0) red[(wave * RPW) * MAXM + vi] = tot;
    }
    __syncthreads();

    // ---- epilogue
    if constexpr (EPI == EPI_ARGMAX) {
        if (tid < p.M) {
            float best = -INFINITY;
            int bi = 0x7fffffff;
            for (int u = 0; u < 4 * RPW; ++u) {
                const int n = blockIdx.x * 4 * RPW + u;
                if (n < p.N) argmax_pick(best, bi, red[u * MAXM + tid], n);
            }
            p.part_val[(int64_t)tid * p.nblocks + blockIdx.x] = best;
            p.part_idx[(int64_t)tid * p.nblocks + blockIdx.x] = bi;
        }
    } else if constexpr (EPI == EPI_GATED) {
        for (int t = tid; t < 2 * RPW * MAXM; t += kBlock) {
            const int q = t / MAXM, m = t - q * MAXM;
            const int j = blockIdx.x * 2 * RPW + q;
            if (m >= p.M || j >= p.F) continue;
            const float g = red[(2 * q) * MAXM + m], u = red[(2 * q + 1) * MAXM + m];
            float y = (p.act == 0 ? gelu_tanh(g) : silu(g)) * u;
            if (p.round_out) y = round_bf16(y);
            p.out[(int64_t)m * p.out_ld + j] = y;
        }
    } else {
        for (int t = tid; t < 4 * RPW * MAXM; t += kBlock) {
            const int u = t / MAXM, m = t - u * MAXM;
            const int n = blockIdx.x * 4 * RPW + u;
            if (m >= p.M || n >= p.N) continue;
            const float y = red[t];
            if constexpr (EPI == EPI_STORE) {
                p.out[(int64_t)m * p.out_ld + n] = p.round_out ? round_bf16(y) : y;
            } else if constexpr (EPI == EPI_RESID) {
                p.out[(int64_t)m * p.out_ld + n] += y;
            } else if constexpr (EPI == EPI_BLOCKINIT) {
                const int64_t b = p.seq_base + m;
                const int d = p.N;
                float* hb = p.out + b * (int64_t)p.gamma * d;
                hb[n] = y + load_gain(p.block_pos, p.gain_f32, n);
                for (int kk = 1; kk < p.gamma; ++kk)
                    hb[(int64_t)kk * d + n] = load_gain(p.mask_emb, p.gain_f32, (kk - 1) * d + n) +
                                              load_gain(p.block_pos, p.gain_f32, kk * d + n);
            } else if constexpr (EPI == EPI_KV) {
                const int gm = p.row_base + m;
                int b = 0;
                while (b + 1 < p.B && p.row_offsets[b + 1] <= gm) ++b;
                const int rows_b = p.row_offsets[b + 1] - p.row_offsets[b];
                const int i = gm - p.row_offsets[b];
                const int cnt = p.counts ? min(p.counts[b], rows_b) : rows_b;
                const int pos = p.len[b] + i;
                if (i < cnt && pos < p.cap) {
                    const int kvw = p.hkv * p.hd;
                    const int which = n / kvw;
                    const int head = (n - which * kvw) / p.hd;
                    const int dim = n - which * kvw - head * p.hd;
                    const int64_t off = (int64_t)layer * p.layer_stride +
                                        (((int64_t)b * p.hkv + head) * p.cap + pos) * p.hd + dim;
                    void* base = which ? p.vcache : p.kcache;
                    if (p.kv_f32)
                        static_cast<float*>(base)[off] = y;
                    else
                        static_cast<uint16_t*>(base)[off] = (uint16_t)f32_to_bf16_bits(y);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host dispatch

template <int WT, int PRO, int EPI, int MAXM, int RPW>
static hipError_t launch_one(const GemvParams& p, int layers, hipStream_t s) {
    typedef typename WTraits<WT>::X X;
    const int unit = (WT == W_I4) ? 32 : 8;
    int KC = kStageBytes / (MAXM * (int)sizeof(X));
    KC = (KC / 512) * 512;
    if (KC >= p.K) KC = p.K;
    KC = (KC / unit) * unit;
    size_t smem = (size_t)MAXM * KC * sizeof(X) + (WT == W_I4 ? (size_t)MAXM * (KC / 32) * 4 : 0) +
                  (size_t)4 * RPW * MAXM * 4 + (size_t)MAXM * 4;
    int grid_x;
    if (EPI == EPI_GATED)
        grid_x = (p.F + 2 * RPW - 1) / (2 * RPW);
    else
        grid_x = (p.N + 4 * RPW - 1) / (4 * RPW);
    dim3 grid(grid_x, layers);
    // allow dynamic LDS beyond the 64 KiB default (gfx950 has 160 KiB per CU)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemv_kernel<WT, PRO, EPI, MAXM, RPW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((gemv_kernel<WT, PRO, EPI, MAXM, RPW>), grid, dim3(kBlock), smem, s, p, KC);
    return hipGetLastError();
}

template <int WT, int PRO, int EPI, int MAXM>
static hipError_t launch_rpw(const GemvParams& p, int layers, hipStream_t s) {
    if constexpr (MAXM == 8) {
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
static hipError_t launch_wt(int wtype, const GemvParams& p, int layers, hipStream_t s) {
    switch (wtype) {
        case W_F32: return launch_rpw<W_F32, PRO, EPI, MAXM>(p, layers, s);
        case W_BF16: return launch_rpw<W_BF16, PRO, EPI, MAXM>(p, layers, s);
        case W_I4: return launch_rpw<W_I4, PRO, EPI, MAXM>(p, layers, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int wtype, int pro, int epi, int maxm, const GemvParams& p, int layers, hipStream_t s) {
#define DFL_CASE(PRO, EPI)                                                                      \
    if (pro == PRO && epi == EPI) {                                                             \
        return maxm <= 8 ? launch_wt<PRO, EPI, 8>(wtype, p, layers, s)                          \
                         : launch_wt<PRO, EPI, 32>(wtype, p, layers, s);                        \
    }
    DFL_CASE(PRO_TAPS, EPI_STORE)
    DFL_CASE(PRO_NORM, EPI_KV)
    if (pro == PRO_GATHER && epi == EPI_BLOCKINIT) return launch_wt<PRO_GATHER, EPI_BLOCKINIT, 8>(wtype, p, layers, s);
    if (pro == PRO_NORM && epi == EPI_STORE) return launch_wt<PRO_NORM, EPI_STORE, 8>(wtype, p, layers, s);
    if (pro == PRO_PLAIN && epi == EPI_RESID) return launch_wt<PRO_PLAIN, EPI_RESID, 8>(wtype, p, layers, s);
    if (pro == PRO_NORM && epi == EPI_GATED) return launch_wt<PRO_NORM, EPI_GATED, 8>(wtype, p, layers, s);
    if (pro == PRO_TAPS && epi == EPI_ARGMAX) return launch_wt<PRO_TAPS, EPI_ARGMAX, 8>(wtype, p, layers, s);
#undef DFL_CASE
    return hipErrorInvalidValue;
}

}  // namespace dfl
