// Non-causal block attention over [retained context ++ block] (page 3,
// #layer, Eq 3; no mask inside the block: is_causal is false).
//
// Split-K over keys (flash-decoding). Every query row that reads a kv head --
// all hq/hkv query heads of the group times the gamma block rows -- is served
// by the same workgroup, so each context byte is fetched once per layer. Each
// split produces (o, running max m, running sum l) per row; attn_merge_kernel
// combines the splits with the usual log-sum-exp rescaling.
//
// bf16 caches: attn_mfma_kernel. Each wavefront of a workgroup is its own
// split and walks 32-key chunks with no workgroup barriers:
//   S = Q K^T    v_mfma_f32_16x16x32_bf16; the 16-row Q tiles stay in
//                registers, K rows are read straight from HBM (one 16-byte
//                chunk of 8 head dims per lane);
//   softmax      online per row; a row of a 16x16 score tile lives in one
//                16-lane DPP row, so its max and sum take four DPP steps;
//   O += P V     P goes through a per-wavefront LDS tile into the A-operand
//                layout, split into bf16 high and low parts (two products)
//                so the probabilities keep ~16 mantissa bits; V is cached
//                head-dim major, so the B operand (8 consecutive keys of one
//                dim) is one 16-byte load.
// Lane layout of the 16x16x32 product (lane l): A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] for e < 8; D[4(l/16)+e][l%16] for e < 4.
//
// fp32 caches (the fp32 workload): attn_valu_kernel, LDS-staged 64-key tiles,
// one key per lane for the scores, one head-dim column per thread for P V.
#include "attention.hpp"
#include "common.hpp"

#ifndef DFL_ATTN_CPW
#define DFL_ATTN_CPW 1  // 32-key chunks per wavefront (bf16 caches)
#endif

namespace dfl {

constexpr int kTile = 64;   // keys per tile, fp32 kernel
constexpr int kChunk = 32;  // keys per chunk, MFMA kernel
constexpr int kMaxParts = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// reductions over the 16 lanes of a DPP row: xor 1, xor 2 (quad permutes),
// then rotations by 4 and 8 within the row
#define DFL_DPP(v, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false))
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, DFL_DPP(v, 0xB1));   // quad_perm [1,0,3,2]
    v = fmaxf(v, DFL_DPP(v, 0x4E));   // quad_perm [2,3,0,1]
    v = fmaxf(v, DFL_DPP(v, 0x124));  // row_ror:4
    v = fmaxf(v, DFL_DPP(v, 0x128));  // row_ror:8
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += DFL_DPP(v, 0xB1);
    v += DFL_DPP(v, 0x4E);
    v += DFL_DPP(v, 0x124);
    v += DFL_DPP(v, 0x128);
    return v;
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    uint4 o;
    o.x = pack_bf16x2(f[0], f[1]);
    o.y = pack_bf16x2(f[2], f[3]);
    o.z = pack_bf16x2(f[4], f[5]);
    o.w = pack_bf16x2(f[6], f[7]);
    return o;
}

// ---------------------------------------------------------------------------
// MFMA kernel (bf16 caches)

template <int HD, int NRT>
__global__ __launch_bounds__(kBlock) void attn_mfma_kernel(const AttnParams p) {
    constexpr int KS = HD / 32;  // k-steps of S = Q K^T
    constexpr int DT = HD / 16;  // head-dim tiles of O
    constexpr int PLD = kChunk + 8;  // padded P row (bf16 elements)
    __shared__ __align__(16) uint16_t plds[4][2][NRT][16][PLD];  // P as bf16 high and low parts

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x % p.nsplit;
    const int bg = blockIdx.x / p.nsplit;
    const int g = bg % p.hkv, b = bg / p.hkv;
    const int qpg = p.hq / p.hkv;
    const int R = qpg * p.gamma;
    const int lenb = min(max(p.len[b], 0), p.cap);
    const int part = s * 4 + wave;  // this wavefront's split
    const int nch = (lenb + kChunk - 1) / kChunk;
    const int cpp = (nch + p.nparts - 1) / p.nparts;
    const int c_begin = part * cpp;
    const int c_end = min(nch, c_begin + cpp);
    const bool do_block = (part == 0);  // the gamma block keys go to split 0

    const int64_t qkv_ld = p.qkv_ld;
    const float* qrow0 = p.qkv + (int64_t)b * p.gamma * qkv_ld;
    const int kcol = p.hq * HD + g * HD;
    const int vcol = p.hq * HD + p.hkv * HD + g * HD;
    const uint16_t* kc = static_cast<const uint16_t*>(p.kcache) + ((int64_t)b * p.hkv + g) * p.cap * HD;
    const uint16_t* vc = static_cast<const uint16_t*>(p.vcache) + ((int64_t)b * p.hkv + g) * HD * (int64_t)p.cap;

    // Q tiles as A operands: row = rt*16 + col, dims ks*32 + 8*grp + e
    uint4 qa[NRT][KS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = rt * 16 + col;
        const float* src = nullptr;
        if (r < R) {
            const int h = g * qpg + r / p.gamma, i = r % p.gamma;
            src = qrow0 + (int64_t)i * qkv_ld + h * HD;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = src ? src[ks * 32 + 8 * grp + e] : 0.f;
            qa[rt][ks] = pack8(f);
        }
    }

    f32x4 o[NRT][DT];
    float m[NRT][4], l[NRT][4];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) { m[rt][e] = -INFINITY; l[rt][e] = 0.f; }
    }

    // one chunk of up to 32 keys: keys [c0, c0 + nvalid) of the context, or of the block
    auto chunk = [&](const bool block, const int c0, const int nvalid) {
        f32x4 sacc[NRT][2];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) sacc[rt][0] = sacc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int j = nt * 16 + col;  // key within the chunk
            uint4 kb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (j < nvalid) {
                    if (block) {
                        const float* src = qrow0 + (int64_t)j * qkv_ld + kcol + ks * 32 + 8 * grp;
                        float f[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] = src[e];
                        kb[ks] = pack8(f);
                    } else {
                        kb[ks] = *reinterpret_cast<const uint4*>(kc + (int64_t)(c0 + j) * HD + ks * 32 + 8 * grp);
                    }
                } else {
                    kb[ks] = make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sacc[rt][nt] = mfma16(qa[rt][ks], kb[ks], sacc[rt][nt]);
        }
        // online softmax; lane holds rows 4*grp+e, keys col and 16+col
        const bool v0ok = col < nvalid, v1ok = 16 + col < nvalid;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s0 = v0ok ? sacc[rt][0][e] * p.scale : -INFINITY;
                const float s1 = v1ok ? sacc[rt][1][e] * p.scale : -INFINITY;
                const float mx = row16_max(fmaxf(s0, s1));
                const float mn = fmaxf(m[rt][e], mx);
                float p0 = 0.f, p1 = 0.f, al = 1.f;
                if (mn != -INFINITY) {
                    p0 = v0ok ? expf(s0 - mn) : 0.f;
                    p1 = v1ok ? expf(s1 - mn) : 0.f;
                    al = expf(m[rt][e] - mn);
                }
                l[rt][e] = l[rt][e] * al + row16_sum(p0 + p1);
                m[rt][e] = mn;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[rt][dt][e] *= al;
                // P = hi + lo with both parts bf16: the product keeps ~16 mantissa bits of P
                const uint32_t h0 = f32_to_bf16_bits(p0), h1 = f32_to_bf16_bits(p1);
                plds[wave][0][rt][4 * grp + e][col] = (uint16_t)h0;
                plds[wave][0][rt][4 * grp + e][16 + col] = (uint16_t)h1;
                plds[wave][1][rt][4 * grp + e][col] = (uint16_t)f32_to_bf16_bits(p0 - bf16_bits_to_f32(h0));
                plds[wave][1][rt][4 * grp + e][16 + col] = (uint16_t)f32_to_bf16_bits(p1 - bf16_bits_to_f32(h1));
            }
        }
        // P as A operands (row col, keys 8*grp .. +8); LDS ops of one wavefront are ordered
        uint4 pa[NRT], pl[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            pa[rt] = *reinterpret_cast<const uint4*>(&plds[wave][0][rt][col][8 * grp]);
            pl[rt] = *reinterpret_cast<const uint4*>(&plds[wave][1][rt][col][8 * grp]);
        }
        // V as B operands: keys 8*grp + e, dim dt*16 + col
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int dim = dt * 16 + col;
            uint4 vb;
            if (block) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 8 * grp + e;
                    f[e] = j < nvalid ? qrow0[(int64_t)j * qkv_ld + vcol + dim] : 0.f;
                }
                vb = pack8(f);
            } else {
                vb = *reinterpret_cast<const uint4*>(vc + (int64_t)dim * p.cap + c0 + 8 * grp);
                // keys past the context are zeroed (P is zero there; the cache may hold anything)
                const int nk = nvalid - 8 * grp;
                if (nk < 8) {
                    uint32_t w[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (2 * q >= nk) w[q] = 0u;
                        else if (2 * q + 1 >= nk) w[q] &= 0xFFFFu;
                    }
                    vb = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) o[rt][dt] = mfma16(pl[rt], vb, mfma16(pa[rt], vb, o[rt][dt]));
        }
    };

    for (int c = c_begin; c < c_end; ++c) chunk(false, c * kChunk, min(kChunk, lenb - c * kChunk));
    if (do_block) chunk(true, 0, p.gamma);

    // partials of this split: [B][hq][nparts][gamma][HD + 2]
    const int W = HD + 2;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rt * 16 + 4 * grp + e;
            if (r >= R) continue;
            const int h = g * qpg + r / p.gamma, i = r % p.gamma;
            float* dst = p.part + ((((int64_t)b * p.hq + h) * p.nparts + part) * p.gamma + i) * W;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) dst[dt * 16 + col] = o[rt][dt][e];
            if (col == 0) {
                dst[HD] = m[rt][e];
                dst[HD + 1] = l[rt][e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// VALU kernel (fp32 caches)

template <int HD, int RMAX>
__global__ __launch_bounds__(kBlock) void attn_valu_kernel(const AttnParams p) {
    constexpr int NPH = kBlock / HD;    // P.V phases (threads per head-dim column)
    constexpr int RPT = (RMAX + NPH - 1) / NPH;
    constexpr int RPWV = (RMAX + 3) / 4;  // softmax rows per wavefront
    __shared__ __align__(16) float qs[RMAX * HD];
    __shared__ __align__(16) float ks[kTile * (HD + 4)];
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
    const float* kc = static_cast<const float*>(p.kcache) + ((int64_t)b * p.hkv + g) * p.cap * HD;
    const float* vc = static_cast<const float*>(p.vcache) + ((int64_t)b * p.hkv + g) * HD * (int64_t)p.cap;

    for (int e = tid; e < R * HD; e += kBlock) {
        const int r = e / HD, dd = e - r * HD;
        const int h = g * qpg + r / p.gamma, i = r % p.gamma;
        qs[r * HD + dd] = qrow0[(int64_t)i * qkv_ld + h * HD + dd];
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
        for (int e = tid; e < kTile * HD; e += kBlock) {
            const int key = e / HD, dd = e - key * HD;
            const int kk = t0 + key;
            float kv = 0.f, vv = 0.f;
            if (kk < lenb) {
                kv = kc[(int64_t)kk * HD + dd];
                vv = vc[(int64_t)dd * p.cap + kk];
            } else if (kk < T) {
                const float* rowp = qrow0 + (int64_t)(kk - lenb) * qkv_ld;
                kv = rowp[kcol + dd];
                vv = rowp[vcol + dd];
            }
            ks[key * (HD + 4) + dd] = kv;
            vs[key * HD + dd] = vv;
        }
        __syncthreads();
        {
            const int kk = t0 + lane;
            const bool valid = kk < end;
#pragma unroll
            for (int j = 0; j < RPWV; ++j) {
                const int r = wave + 4 * j;
                if (r >= R) break;
                float acc = 0.f;
                for (int d = 0; d < HD; ++d) acc = fmaf(qs[r * HD + d], ks[lane * (HD + 4) + d], acc);
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
        __syncthreads();
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int r = ph + NPH * j;
            if (r < R) o[j] *= alpha[r];
        }
        const int nk = min(kTile, end - t0);
        for (int key = 0; key < nk; ++key) {
            const float v = vs[key * HD + dcol];
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int r = ph + NPH * j;
                if (r < R) o[j] = fmaf(ps[r * kTile + key], v, o[j]);
            }
        }
    }

    const int W = HD + 2;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = ph + NPH * j;
        if (r < R) {
            const int h = g * qpg + r / p.gamma, i = r % p.gamma;
            p.part[((((int64_t)b * p.hq + h) * p.nparts + s) * p.gamma + i) * W + dcol] = o[j];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < RPWV; ++j) {
            const int r = wave + 4 * j;
            if (r < R) {
                const int h = g * qpg + r / p.gamma, i = r % p.gamma;
                const int64_t base = ((((int64_t)b * p.hq + h) * p.nparts + s) * p.gamma + i) * W;
                p.part[base + HD] = mrow[j];
                p.part[base + HD + 1] = lrow[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One workgroup per (b, head, block row): combine the partials. The weights
// exp(m_s - M) are formed once in LDS; each thread group adds a fixed subset
// of the partials and the groups are combined in a fixed order.
template <int HD>
__global__ __launch_bounds__(kBlock) void attn_merge_kernel(const AttnParams p) {
    constexpr int G = kBlock / HD;
    __shared__ float wts[kMaxParts];
    __shared__ float red[4];
    __shared__ float part[G][HD];
    const int row = blockIdx.x;  // (b*hq + h)*gamma + i
    const int i = row % p.gamma;
    const int bh = row / p.gamma;
    const int h = bh % p.hq, b = bh / p.hq;
    const int W = HD + 2;
    const float* base = p.part + ((int64_t)bh * p.nparts * p.gamma + i) * W;
    const int64_t sstride = (int64_t)p.gamma * W;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float ms = -INFINITY, ls = 0.f;
    if (t < p.nparts) {
        ms = base[t * sstride + HD];
        ls = base[t * sstride + HD + 1];
    }
    float M = wave_max(ms);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float w = (ms == -INFINITY) ? 0.f : expf(ms - M);
    wts[t] = w;
    float L = wave_sum(w * ls);
    __syncthreads();
    if (lane == 0) red[wave] = L;
    __syncthreads();
    L = red[0] + red[1] + red[2] + red[3];
    const int gi = t / HD, dcol = t % HD;
    float acc = 0.f;
#pragma unroll 8
    for (int sidx = gi; sidx < p.nparts; sidx += G) acc += wts[sidx] * base[sidx * sstride + dcol];
    part[gi][dcol] = acc;
    __syncthreads();
    if (gi == 0) {
        float y = 0.f;
#pragma unroll
        for (int q = 0; q < G; ++q) y += part[q][dcol];
        y /= L;
        const int64_t o = ((int64_t)b * p.gamma + i) * p.out_ld + h * HD + dcol;
        if (p.round_out)
            reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16_bits(y);
        else
            p.out[o] = y;
    }
}

// ---------------------------------------------------------------------------

void attention_splits(int cap, int gamma, int kv_f32, int* nsplit, int* nparts) {
    if (kv_f32) {
        int ns = (cap + gamma + kTile - 1) / kTile;
        ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
        *nsplit = ns;
        *nparts = ns;
    } else {
        const int chunks = (cap + kChunk - 1) / kChunk;
        const int parts = (chunks + DFL_ATTN_CPW - 1) / DFL_ATTN_CPW;
        int ns = (parts + 3) / 4;
        ns = ns < 1 ? 1 : (ns > kMaxParts / 4 ? kMaxParts / 4 : ns);
        *nsplit = ns;
        *nparts = 4 * ns;
    }
}

int attention_max_rows(int kv_f32) { return kv_f32 ? 40 : 48; }

template <int HD>
static hipError_t launch_hd(const AttnParams& p, hipStream_t s) {
    const int R = (p.hq / p.hkv) * p.gamma;
    dim3 grid((unsigned)((int64_t)p.B * p.hkv * p.nsplit));
    (void)hipGetLastError();  // report only this launch's status
    if (p.kv_f32) {
        if (R <= 8)
            hipLaunchKernelGGL((attn_valu_kernel<HD, 8>), grid, dim3(kBlock), 0, s, p);
        else if (R <= 40)
            hipLaunchKernelGGL((attn_valu_kernel<HD, 40>), grid, dim3(kBlock), 0, s, p);
        else
            return hipErrorInvalidValue;
    } else {
        if (R <= 16)
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 1>), grid, dim3(kBlock), 0, s, p);
        else if (R <= 32)
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 2>), grid, dim3(kBlock), 0, s, p);
        else if (R <= 48)
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 3>), grid, dim3(kBlock), 0, s, p);
        else
            return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_merge_kernel<HD>), dim3((unsigned)(p.B * p.hq * p.gamma)), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
    if (p.nparts > kMaxParts || p.gamma > kChunk) return hipErrorInvalidValue;
    if (!p.kv_f32 && (p.cap % kChunk)) return hipErrorInvalidValue;
    if (p.hd == 128) return launch_hd<128>(p, s);
    if (p.hd == 64) return launch_hd<64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace dfl
