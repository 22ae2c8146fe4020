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

    // K/V rows of one 64-key tile, held in registers between the global loads
    // and the LDS stores so that the next tile's loads overlap this tile's math
    constexpr int UNITS = kTile * (HD / 8) / kBlock;
    float kst[UNITS][8], vst[UNITS][8];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int e = tid + u * kBlock;
            const int key = e / (HD / 8), c8 = (e - key * (HD / 8)) * 8;
            const int kk = t0 + key;
            if (kk < lenb) {
                const int64_t off = cache_base + (int64_t)kk * HD + c8;
                if constexpr (KVF32) {
                    const float* kp = static_cast<const float*>(p.kcache) + off;
                    const float* vp = static_cast<const float*>(p.vcache) + off;
#pragma unroll
                    for (int j = 0; j < 8; ++j) { kst[u][j] = kp[j]; vst[u][j] = vp[j]; }
                } else {
                    const uint4 ka = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.kcache) + off);
                    const uint4 va = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.vcache) + off);
                    const uint32_t kw4[4] = {ka.x, ka.y, ka.z, ka.w}, vw4[4] = {va.x, va.y, va.z, va.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kst[u][2 * j] = bf16_lo(kw4[j]); kst[u][2 * j + 1] = bf16_hi(kw4[j]);
                        vst[u][2 * j] = bf16_lo(vw4[j]); vst[u][2 * j + 1] = bf16_hi(vw4[j]);
                    }
                }
            } else if (kk < T) {
                const float* rowp = qrow0 + (int64_t)(kk - lenb) * qkv_ld;
#pragma unroll
                for (int j = 0; j < 8; ++j) { kst[u][j] = rowp[kcol + c8 + j]; vst[u][j] = rowp[vcol + c8 + j]; }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) { kst[u][j] = 0.f; vst[u][j] = 0.f; }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < UNITS; ++u) {
            const int e = tid + u * kBlock;
            const int key = e / (HD / 8), c8 = (e - key * (HD / 8)) * 8;
            if constexpr (KVF32) {
#pragma unroll
                for (int j = 0; j < 8; ++j) ks[key * (HD + 4) + c8 + j] = __float_as_uint(kst[u][j]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) ks[key * KPAD + c8 / 2 + j] = pack_bf16x2(kst[u][2 * j], kst[u][2 * j + 1]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) vs[key * HD + c8 + j] = vst[u][j];
        }
    };
    if (start < end) load_tile(start);

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
        store_tile();
        __syncthreads();
        if (t0 + kTile < end) load_tile(t0 + kTile);

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

// One workgroup per (b, head, block row): combine the splits. The split
// weights exp(m_s - M) are formed once in LDS; each thread group then adds a
// fixed subset of the splits and the groups are combined in a fixed order.
template <int HD>
__global__ __launch_bounds__(kBlock) void attn_merge_kernel(const AttnParams p) {
    constexpr int G = kBlock / HD;
    __shared__ float wts[64];
    __shared__ float part[G][HD];
    __shared__ float Lsh;
    const int row = blockIdx.x;  // (b*hq + h)*gamma + i
    const int i = row % p.gamma;
    const int bh = row / p.gamma;
    const int h = bh % p.hq, b = bh / p.hq;
    const int W = HD + 2;
    const float* base = p.part + ((int64_t)bh * p.nsplit * p.gamma + i) * W;
    const int64_t sstride = (int64_t)p.gamma * W;
    const int t = threadIdx.x;
    if (t < 64) {
        float ms = -INFINITY, ls = 0.f;
        if (t < p.nsplit) {
            ms = base[t * sstride + HD];
            ls = base[t * sstride + HD + 1];
        }
        const float M = wave_max(ms);
        const float w = (ms == -INFINITY) ? 0.f : expf(ms - M);
        const float L = wave_sum(w * ls);
        wts[t] = w;
        if (t == 0) Lsh = L;
    }
    __syncthreads();
    const int gi = t / HD, dcol = t % HD;
    float acc = 0.f;
#pragma unroll 8
    for (int sidx = gi; sidx < p.nsplit; sidx += G) acc += wts[sidx] * base[sidx * sstride + dcol];
    part[gi][dcol] = acc;
    __syncthreads();
    if (gi == 0) {
        float y = 0.f;
#pragma unroll
        for (int q = 0; q < G; ++q) y += part[q][dcol];
        y /= Lsh;
        const int64_t o = ((int64_t)b * p.gamma + i) * p.out_ld + h * HD + dcol;
        if (p.round_out)
            reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16_bits(y);
        else
            p.out[o] = y;
    }
}

template <int HD, bool KVF32>
static hipError_t launch_hd(const AttnParams& p, hipStream_t s) {
    const int R = (p.hq / p.hkv) * p.gamma;
    dim3 grid((unsigned)((int64_t)p.B * p.hkv * p.nsplit));
    (void)hipGetLastError();  // report only this launch's status
    if (R <= 8) {
        hipLaunchKernelGGL((attn_partial_kernel<HD, KVF32, 8>), grid, dim3(kBlock), 0, s, p);
    } else if (R <= 40) {
        hipLaunchKernelGGL((attn_partial_kernel<HD, KVF32, 40>), grid, dim3(kBlock), 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3((unsigned)(p.B * p.hq * p.gamma)), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
    if (p.hd == 128) return p.kv_f32 ? launch_hd<128, true>(p, s) : launch_hd<128, false>(p, s);
    if (p.hd == 64) return p.kv_f32 ? launch_hd<64, true>(p, s) : launch_hd<64, false>(p, s);
    return hipErrorInvalidValue;
}

int attention_max_rows() { return 40; }

}  // namespace dfl
