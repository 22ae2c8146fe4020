// Non-causal block attention over [retained context ++ block] (page 3,
// #layer, Eq 3; no mask inside the block: is_causal is false).
//
// Split-K over keys (flash-decoding): workgroup (b, kv head g, split s) reads
// its slice of the context K/V rows once and serves every query row that uses
// that kv head -- all hq/hkv query heads of the group times the gamma block
// rows -- so each context byte is fetched once per layer. Keys are processed
// in tiles of 64 staged in LDS. Scores: one key per lane, each wavefront owns
// a subset of query rows and keeps their running max and sum (online
// softmax, wavefront shuffles for the tile max and sum). P.V: one head-dim
// column per thread. The partial (o, m, l) of each split is merged by
// attn_merge_kernel with the usual log-sum-exp rescaling.
#include "attention.hpp"
#include "common.hpp"

namespace dfl {

constexpr int kTile = 64;

template <int HD, bool KVF32, int RMAX>
__global__ __launch_bounds__(kBlock) void attn_partial_kernel(const AttnParams p) {
    constexpr int HW = HD / 2;          // u32 words per bf16 row
    constexpr int KPAD = HW + 4;        // padded K row (words): breaks LDS bank aliasing
    constexpr int NPH = kBlock / HD;    // P.V phases (threads per head-dim column)
    constexpr int RPT = (RMAX + NPH - 1) / NPH;
    constexpr int RPWV = (RMAX + 3) / 4;  // softmax rows per wavefront

    // q: bf16 pairs (or fp32) [RMAX][HD]; K tile: bf16 pairs (or fp32) [64][padded]
    __shared__ __align__(16) uint32_t qs[RMAX * (KVF32 ? HD : HW)];
    __shared__ __align__(16) uint32_t ks[kTile * (KVF32 ? HD + 4 : KPAD)];
    __shared__ __align__(16) float vs[kTile * HD];
    __shared__ __align__(16) float ps[RMAX * kTile];
    __shared__ float alpha[RMAX];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.x % p.nsplit;
    const int bg = blockIdx.x / p.nsplit;
    const int g = bg % p.hkv, b = bg / p.hkv;
    const int qpg = p.hq / p.hkv;
    const int R = qpg * p.gamma;
    const int lenb = min(max(p.len[b], 0), p.cap);
    const int T = lenb + p.gamma;
    int C = (T + p.nsplit - 1) / p.nsplit;
    C = ((C + kTile - 1) / kTile) * kTile;
    const int start = s * C;
    const int end = min(T, start + C);

    const int64_t qkv_ld = p.qkv_ld;
    const float* qrow0 = p.qkv + (int64_t)b * p.gamma * qkv_ld;
    const int kcol = p.hq * HD + g * HD;
    const int vcol = p.hq * HD + p.hkv * HD + g * HD;
    const int64_t cache_base = ((int64_t)b * p.hkv + g) * p.cap * HD;

    // stage the group's query rows (already rounded to bf16 where the contract says so)
    for (int e = tid; e < R * HD; e += kBlock) {
        const int r = e / HD, dd = e - r * HD;
        const int h = g * qpg + r / p.gamma, i = r % p.gamma;
        const float v = qrow0[(int64_t)i * qkv_ld + h * HD + dd];
        if constexpr (KVF32) {
            qs[r * HD + dd] = __float_as_uint(v);
        } else {
            uint16_t* q16 = reinterpret_cast<uint16_t*>(qs);
            q16[r * HD + dd] = (uint16_t)f32_to_bf16_bits(v);
        }
    }

    float mrow[RPWV], lrow[RPWV];
#pragma unroll
    for (int j = 0; j < RPWV; ++j) { mrow[j] = -INFINITY; lrow[j] = 0.f; }
    float o[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) o[j] = 0.f;
    const int dcol = tid % HD, ph = tid / HD;

    for (int t0 = start; t0 < end; t0 += kTile) {
        __syncthreads();
        // ---- stage K and V rows t0 .. t0+63 (context rows, then block rows, then zeros)
        for (int e = tid; e < kTile * (HD / 8); e += kBlock) {
            const int key = e / (HD / 8), c8 = (e - key * (HD / 8)) * 8;
            const int kk = t0 + key;
            float kv8[8], vv8[8];
            if (kk < lenb) {
                const int64_t off = cache_base + (int64_t)kk * HD + c8;
                if constexpr (KVF32) {
                    const float* kp = static_cast<const float*>(p.kcache) + off;
                    const float* vp = static_cast<const float*>(p.vcache) + off;
#pragma unroll
                    for (int j = 0; j < 8; ++j) { kv8[j] = kp[j]; vv8[j] = vp[j]; }
                } else {
                    const uint4 ka = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.kcache) + off);
                    const uint4 va = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.vcache) + off);
                    const uint32_t kw4[4] = {ka.x, ka.y, ka.z, ka.w}, vw4[4] = {va.x, va.y, va.z, va.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kv8[2 * j] = bf16_lo(kw4[j]); kv8[2 * j + 1] = bf16_hi(kw4[j]);
                        vv8[2 * j] = bf16_lo(vw4[j]); vv8[2 * j + 1] = bf16_hi(vw4[j]);
                    }
                }
            } else if (kk < T) {
                const float* rowp = qrow0 + (int64_t)(kk - lenb) * qkv_ld;
#pragma unroll
                for (int j = 0; j < 8; ++j) { kv8[j] = rowp[kcol + c8 + j]; vv8[j] = rowp[vcol + c8 + j]; }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) { kv8[j] = 0.f; vv8[j] = 0.f; }
            }
            if constexpr (KVF32) {
#pragma unroll
                for (int j = 0; j < 8; ++j) ks[key * (HD + 4) + c8 + j] = __float_as_uint(kv8[j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) ks[key * KPAD + c8 / 2 + j] = pack_bf16x2(kv8[2 * j], kv8[2 * j + 1]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) vs[key * HD + c8 + j] = vv8[j];
        }
        __syncthreads();

        // ---- scores and online softmax: lane = key, wavefront `wave` owns rows wave, wave+4, ...
        {
            const int kk = t0 + lane;
            const bool valid = kk < end;
            if constexpr (KVF32) {
                float kr[HD];
#pragma unroll
                for (int j = 0; j < HD; ++j) kr[j] = __uint_as_float(ks[lane * (HD + 4) + j]);
#pragma unroll
                for (int j = 0; j < RPWV; ++j) {
                    const int r = wave + 4 * j;
                    if (r >= R) break;
                    float acc = 0.f;
#pragma unroll
                    for (int d = 0; d < HD; ++d) acc = fmaf(__uint_as_float(qs[r * HD + d]), kr[d], acc);
                    const float sc = valid ? acc * p.scale : -INFINITY;
                    const float mt = wave_max(sc);
                    const float mn = fmaxf(mrow[j], mt);
                    const float pv = valid ? expf(sc - mn) : 0.f;
                    const float al = expf(mrow[j] - mn);
                    lrow[j] = lrow[j] * al + wave_sum(pv);
                    mrow[j] = mn;
                    ps[r * kTile + lane] = pv;
                    if (lane == 0) alpha[r] = al;
                }
            } else {
                uint32_t kr[HW];
#pragma unroll
                for (int j = 0; j < HW; j += 4) {
                    const uint4 v4 = *reinterpret_cast<const uint4*>(&ks[lane * KPAD + j]);
                    kr[j] = v4.x; kr[j + 1] = v4.y; kr[j + 2] = v4.z; kr[j + 3] = v4.w;
                }
#pragma unroll
                for (int j = 0; j < RPWV; ++j) {
                    const int r = wave + 4 * j;
                    if (r >= R) break;
                    float acc = 0.f;
#pragma unroll
                    for (int w = 0; w < HW; w += 4) {
                        const uint4 q4 = *reinterpret_cast<const uint4*>(&qs[r * HW + w]);
                        acc = dot2_bf16(q4.x, kr[w], acc);
                        acc = dot2_bf16(q4.y, kr[w + 1], acc);
                        acc = dot2_bf16(q4.z, kr[w + 2], acc);
                        acc = dot2_bf16(q4.w, kr[w + 3], acc);
                    }
                    const float sc = valid ? acc * p.scale : -INFINITY;
                    const float mt = wave_max(sc);
                    const float mn = fmaxf(mrow[j], mt);
                    const float pv = valid ? expf(sc - mn) : 0.f;
                    const float al = expf(mrow[j] - mn);
                    lrow[j] = lrow[j] * al + wave_sum(pv);
                    mrow[j] = mn;
                    ps[r * kTile + lane] = pv;
                    if (lane == 0) alpha[r] = al;
                }
            }
        }
        __syncthreads();

        // ---- P.V: thread owns head-dim column dcol of rows ph, ph+NPH, ...
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = ph + NPH * j;
            if (r < R) o[j] *= alpha[r];
        }
        const int nk = min(kTile, end - t0);
        for (int key = 0; key < nk; key += 4) {
            const float v0 = vs[(key + 0) * HD + dcol];
            const float v1 = vs[(key + 1) * HD + dcol];
            const float v2 = vs[(key + 2) * HD + dcol];
            const float v3 = vs[(key + 3) * HD + dcol];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int r = ph + NPH * j;
                if (r < R) {
                    const float4 pp = *reinterpret_cast<const float4*>(&ps[r * kTile + key]);
                    float a = o[j];
                    a = fmaf(pp.x, v0, a);
                    a = fmaf(pp.y, v1, a);
                    a = fmaf(pp.z, v2, a);
                    a = fmaf(pp.w, v3, a);
                    o[j] = a;
                }
            }
        }
    }

    // ---- write this split's partials: [B][hq][nsplit][gamma][HD + 2]
    const int W = HD + 2;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = ph + NPH * j;
        if (r < R) {
            const int h = g * qpg + r / p.gamma, i = r % p.gamma;
            const int64_t base = ((((int64_t)b * p.hq + h) * p.nsplit + s) * p.gamma + i) * W;
            p.part[base + dcol] = o[j];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < RPWV; ++j) {
            const int r = wave + 4 * j;
            if (r < R) {
                const int h = g * qpg + r / p.gamma, i = r % p.gamma;
                const int64_t base = ((((int64_t)b * p.hq + h) * p.nsplit + s) * p.gamma + i) * W;
                p.part[base + HD] = mrow[j];
                p.part[base + HD + 1] = lrow[j];
            }
        }
    }
}

// One workgroup per (b, head, block row): combine the splits.
template <int HD>
__global__ __launch_bounds__(HD) void attn_merge_kernel(const AttnParams p) {
    const int row = blockIdx.x;  // (b*hq + h)*gamma + i
    const int i = row % p.gamma;
    const int bh = row / p.gamma;
    const int h = bh % p.hq, b = bh / p.hq;
    const int W = HD + 2;
    const float* base = p.part + ((int64_t)bh * p.nsplit * p.gamma + i) * W;
    const int64_t sstride = (int64_t)p.gamma * W;
    float M = -INFINITY;
    for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, base[s * sstride + HD]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
        const float ms = base[s * sstride + HD];
        if (ms == -INFINITY) continue;
        const float w = expf(ms - M);
        L += w * base[s * sstride + HD + 1];
        acc += w * base[s * sstride + threadIdx.x];
    }
    float y = acc / L;
    if (p.round_out) y = round_bf16(y);
    p.out[((int64_t)b * p.gamma + i) * p.out_ld + h * HD + threadIdx.x] = y;
}

template <int HD, bool KVF32>
static hipError_t launch_hd(const AttnParams& p, hipStream_t s) {
    const int R = (p.hq / p.hkv) * p.gamma;
    dim3 grid((unsigned)((int64_t)p.B * p.hkv * p.nsplit));
    if (R <= 8)
        hipLaunchKernelGGL((attn_partial_kernel<HD, KVF32, 8>), grid, dim3(kBlock), 0, s, p);
    else if (R <= 40)
        hipLaunchKernelGGL((attn_partial_kernel<HD, KVF32, 40>), grid, dim3(kBlock), 0, s, p);
    else
        return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3((unsigned)(p.B * p.hq * p.gamma)), dim3(HD), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
    if (p.hd == 128) return p.kv_f32 ? launch_hd<128, true>(p, s) : launch_hd<128, false>(p, s);
    if (p.hd == 64) return p.kv_f32 ? launch_hd<64, true>(p, s) : launch_hd<64, false>(p, s);
    return hipErrorInvalidValue;
}

int attention_max_rows() { return 40; }

}  // namespace dfl
