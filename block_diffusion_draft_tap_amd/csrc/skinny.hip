// Matrix-core projections of the drafter's block rows when a batch of
// sequences gives 16 or more of them (B sequences x gamma block tokens, the
// Q/K/V, output, FFN and LM-head products of each round). At that row count a
// projection is a small dense contraction; the per-8-row GEMV passes would
// stream each weight matrix from HBM once per 8 rows, here it is streamed once.
//
// A workgroup of kSW wavefronts owns kSCols consecutive weight rows (output
// columns) and walks K in chunks of 128. Each wavefront streams its own
// 16 * kSNB weight rows straight from memory into registers, two chunks ahead
// of the one it multiplies, already in the B-operand layout of
// v_mfma_f32_16x16x32_bf16 (lane l: weight row l % 16, k offset 8 (l / 16);
// one load instruction reads 16 rows x 64 contiguous bytes). The activation
// chunk (all M rows x 128) is shared by the wavefronts through LDS, double
// buffered with one barrier per chunk; every workgroup of a launch reads the
// same activation rows, so they mostly come from L2. Activations are loaded
// two chunks ahead too, each chunk's before its weights: loads complete in
// issue order, so the wait for chunk c + 1's activations (before their LDS
// store) leaves the weights of c + 1 and c + 2 in flight. Lane l holds
//   A[l % 16][8 (l / 16) + e],  B[8 (l / 16) + e][l % 16]   (e < 8)
//   D[4 (l / 16) + e][l % 16]                               (e < 4)
// of each 16 x 16 product, and a wavefront keeps the M x 16 kSNB accumulators
// of its weight rows.
//
// The same kernel serves the round's context rows (B sequences x the committed
// block rows): the tap concatenation times W_c (A read from the m tap buffers)
// and the K/V rows of every layer at once (grid.z = layer).
//
// Epilogues act on the accumulators in place: fp32 or bf16 store (with the
// head-dim-major redirect of the block values), residual add, the gated FFN
// activation (a wavefront's fragments pair 16 gate rows with the matching 16 up
// rows, so both products of an output sit in the same lane), the per-row
// (max, lowest index) of the LM head, and the K/V cache scatter. Launches with
// too few column tiles to fill the GPU split K: fp32 partial sums go to a
// buffer, and a second kernel adds them in split order and applies the
// epilogue (or the caller consumes them).
#include <cstdio>

#include "common.hpp"
#include "skinny.hpp"
#include "trace.hpp"

namespace dfl {

// wavefronts per workgroup, 16-row weight fragments per wavefront, and the
// workgroup count that split-K aims for (compile-time tunables)
#ifndef DFL_SK_WAVES
#define DFL_SK_WAVES 4
#endif
#ifndef DFL_SK_NB
#define DFL_SK_NB 2
#endif
#ifndef DFL_SK_WGS
#define DFL_SK_WGS 256
#endif
// chunks of activations loaded ahead of the one multiplied (1 or 2; with 2, the wait
// for chunk c + 1's activations before their LDS store leaves the weights of c + 1 and
// c + 2 in flight, loads completing in issue order), and the wavefronts per SIMD the
// kernel is compiled for. Two wavefronts per SIMD (two workgroups per CU, one's LDS and
// barrier work overlapping the other's weight stream) fit the register budget only with
// one chunk of activations ahead: with two the kernel spills, and so does the 8-fragment
// (113 to 128 rows) kernel, which keeps one wavefront per SIMD.
#ifndef DFL_SK_ADEPTH
#define DFL_SK_ADEPTH 1
#endif
#ifndef DFL_SK_OCC
#define DFL_SK_OCC 2
#endif

namespace {

constexpr int kSW = DFL_SK_WAVES, kSNB = DFL_SK_NB, kST = 64 * kSW;
constexpr int kSCols = 16 * kSNB * kSW;  // weight rows per workgroup tile
constexpr int kSKC = kSkinnyK;           // K per chunk
constexpr int kSLd = kSKC + 16;          // padded LDS row (bf16): 72 words, 8 past a multiple of 32 (conflict-free fragment reads)
constexpr int kSSteps = kSKC / 32;       // MFMA k-steps per chunk
static_assert(kSNB % 2 == 0, "the gated epilogue pairs gate and up fragments");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// cache slot of global row r for SK_KV: sequence b and position pos (-1: not stored)
__device__ __forceinline__ void kv_slot(const SkinnyParams& p, int r, int& b, int& pos) {
    b = 0;
    while (b + 1 < p.B && p.row_offsets[b + 1] <= r) ++b;
    const int rows_b = p.row_offsets[b + 1] - p.row_offsets[b];
    const int i = r - p.row_offsets[b];
    const int cnt = p.counts ? min(p.counts[b], rows_b) : rows_b;
    pos = p.len[b] + i;
    if (i < 0 || i >= cnt || pos >= p.cap) pos = -1;
}

__device__ __forceinline__ void kv_store(const SkinnyParams& p, int z, int b, int pos, int n, float y) {
    const int kvw = p.hkv * p.hd;
    const int which = n / kvw;
    const int head = (n - which * kvw) / p.hd;
    const int dim = n - which * kvw - head * p.hd;
    const int64_t hb = (int64_t)z * p.layer_stride + ((int64_t)b * p.hkv + head) * p.cap * p.hd;
    uint16_t* base = which ? p.vcache : p.kcache;
    base[hb + (which ? (int64_t)dim * p.cap + pos : (int64_t)pos * p.hd + dim)] = (uint16_t)f32_to_bf16_bits(y);
}

// the SK_STORE / SK_RESID epilogue of one output
template <int EPI>
__device__ __forceinline__ void store_one(const SkinnyParams& p, int m, int n, float y) {
    if constexpr (EPI == SK_STORE) {
        if (p.out_bf16) {
            const uint16_t b = (uint16_t)f32_to_bf16_bits(y);
            if (p.vt && n >= p.vt_col) {
                const int row = p.row_base + m, bb = row / p.gamma, key = row - bb * p.gamma;
                const int c = n - p.vt_col, head = c / p.hd, dim = c - head * p.hd;
                p.vt[(((int64_t)bb * p.hkv + head) * p.hd + dim) * 32 + key] = b;
            } else {
                static_cast<uint16_t*>(p.out)[(int64_t)m * p.out_ld + n] = b;
            }
        } else {
            static_cast<float*>(p.out)[(int64_t)m * p.out_ld + n] = y;
        }
    } else {
        float* o = static_cast<float*>(p.out) + (int64_t)m * p.out_ld + n;
        *o += y;
    }
}

template <int MT, int EPI>
__global__ __launch_bounds__(kST, MT >= 8 ? 1 : DFL_SK_OCC) void skinny_kernel(const SkinnyParams p) {
    constexpr int RED = EPI == SK_ARGMAX ? MT * 16 : 1;
    constexpr int META = EPI == SK_KV ? MT * 16 : 1;
    __shared__ __align__(16) uint16_t As[2][MT * 16][kSLd];
    __shared__ float red_v[kSW][RED];
    __shared__ int red_i[kSW][RED];
    __shared__ int meta_b[META], meta_pos[META];
    const uint64_t t_start = trace_start(p.stamps);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x, split = blockIdx.y, z = blockIdx.z;
    const int kbeg = split * p.kslice;
    const int nc = (min(p.K, kbeg + p.kslice) - kbeg) / kSKC;
    // this layer's weights and activations (pointer choices made with compares, so the
    // pointer arrays stay in kernel-argument registers)
    const uint16_t* W = p.w[0];
#pragma unroll
    for (int q = 1; q < kMaxLayers; ++q)
        if (z == q) W = p.w[q];
    const uint16_t* A = p.a + (int64_t)z * p.a_layer_stride;

    if constexpr (EPI == SK_KV) {
        // cache slot of every row (read after the main loop's barriers)
        for (int m = threadIdx.x; m < MT * 16; m += kST) {
            int b = 0, pos = -1;
            if (m < p.M) kv_slot(p, p.row_base + m, b, pos);
            meta_b[m] = b;
            meta_pos[m] = pos;
        }
    }

    // weight rows of this wavefront: fragment f, lane row col (rows past the end
    // read the last row; their outputs are never stored)
    const uint16_t* wp[kSNB];
#pragma unroll
    for (int f = 0; f < kSNB; ++f) {
        int row;
        if constexpr (EPI == SK_GATED) {
            const int j = tile * (kSCols / 2) + wave * 8 * kSNB + (f / 2) * 16 + col;
            row = (f & 1) * p.F + min(j, p.F - 1);
        } else {
            row = min(tile * kSCols + wave * 16 * kSNB + f * 16 + col, p.N - 1);
        }
        wp[f] = W + (p.w_row0 + row) * (int64_t)p.K + kbeg + 8 * grp;
    }

    f32x4 acc[MT][kSNB];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int f = 0; f < kSNB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // three register sets of weights: chunk c lives in set c % 3. Loads past the last
    // chunk re-read it (never multiplied): unconditional loads let the compiler count the
    // loads in flight, so waiting for an older load never drains the younger ones
    u32x4 w0[kSNB][kSSteps], w1[kSNB][kSSteps], w2[kSNB][kSSteps];
    auto load_w = [&](u32x4 (&wr)[kSNB][kSSteps], int c) {
        const int cc = min(c, nc - 1);
#pragma unroll
        for (int s = 0; s < kSSteps; ++s)
#pragma unroll
            for (int f = 0; f < kSNB; ++f)
                wr[f][s] = *reinterpret_cast<const u32x4*>(wp[f] + cc * kSKC + s * 32);
    };
    // the activation chunk: MT*16 rows x 16 pieces of 16 bytes, spread over the threads
    constexpr int PIECES = MT * 16 * (kSKC / 8);
    constexpr int APT = (PIECES + kST - 1) / kST;
    u32x4 ast[APT], ast2[APT];
    // (past the last chunk it reloads the last one, which is never stored: unconditional
    // loads keep the staging registers out of scratch memory)
    auto load_a_into = [&](u32x4 (&dst)[APT], int c) {
        const int k0 = kbeg + min(c, nc - 1) * kSKC;
        const uint16_t* src;
        if (p.seg_k > 0) {  // tap segments: a chunk never straddles two
            const int j = k0 / p.seg_k;
            src = p.a_seg[0];
#pragma unroll
            for (int q = 1; q < kMaxTaps; ++q)
                if (j == q) src = p.a_seg[q];
            src += k0 - j * p.seg_k;
        } else {
            src = A + k0;
        }
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = min((int)threadIdx.x + kST * i, PIECES - 1);
            const int row = min(q >> 4, p.M - 1);  // rows past M: any valid row, never stored
            dst[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)row * p.a_ld + 8 * (q & 15));
        }
    };
    auto store_a_from = [&](const u32x4 (&srcr)[APT], int buf) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int q = threadIdx.x + kST * i;
            if (PIECES % kST == 0 || q < PIECES) *reinterpret_cast<u32x4*>(&As[buf][q >> 4][8 * (q & 15)]) = srcr[i];
        }
    };
    auto load_a = [&](int c) { load_a_into(ast, c); };
    auto store_a = [&](int buf) { store_a_from(ast, buf); };
    auto mma = [&](int buf, const u32x4 (&wr)[kSNB][kSSteps]) {
#pragma unroll
        for (int s = 0; s < kSSteps; ++s) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(&As[buf][i * 16 + col][s * 32 + 8 * grp]);
#pragma unroll
                for (int f = 0; f < kSNB; ++f) acc[i][f] = mfma_bf16(af, wr[f][s], acc[i][f]);
            }
        }
    };

    // chunk c multiplies LDS buffer c % 2; the activations of c + 1 are loaded before the
    // weights of c + 2, so the wait for them before their LDS store leaves the weights in
    // flight. Whole triples of chunks run without branches (a store into the idle buffer
    // past the last chunk is never read); the last one or two chunks follow.
#if DFL_SK_ADEPTH == 2
    // activations two chunks ahead as well: A(k) sits in staging set k % 2 from its load
    // (during chunk k - 2) until its LDS store (end of chunk k - 1); six chunks per trip
    auto stage = [&](int cc, u32x4 (&wc)[kSNB][kSSteps], u32x4 (&wn)[kSNB][kSSteps], u32x4 (&al)[APT],
                     const u32x4 (&as)[APT]) {
        load_a_into(al, cc + 2);
        load_w(wn, cc + 2);
        mma(cc & 1, wc);
        store_a_from(as, (cc + 1) & 1);
        __syncthreads();
    };
    load_w(w0, 0);
    load_w(w1, 1);
    load_a_into(ast, 0);
    load_a_into(ast2, 1);
    store_a_from(ast, 0);
    __syncthreads();
    int c = 0;
    for (; c + 6 <= nc; c += 6) {
        stage(c, w0, w2, ast, ast2);
        stage(c + 1, w1, w0, ast2, ast);
        stage(c + 2, w2, w1, ast, ast2);
        stage(c + 3, w0, w2, ast2, ast);
        stage(c + 4, w1, w0, ast, ast2);
        stage(c + 5, w2, w1, ast2, ast);
    }
    if (c < nc) stage(c, w0, w2, ast, ast2);
    if (c + 1 < nc) stage(c + 1, w1, w0, ast2, ast);
    if (c + 2 < nc) stage(c + 2, w2, w1, ast, ast2);
    if (c + 3 < nc) stage(c + 3, w0, w2, ast2, ast);
    if (c + 4 < nc) stage(c + 4, w1, w0, ast, ast2);
#else
    load_w(w0, 0);
    load_w(w1, 1);
    load_a(0);
    store_a(0);
    __syncthreads();
    int c = 0;
    for (; c + 3 <= nc; c += 3) {
        load_a(c + 1);
        load_w(w2, c + 2);
        mma(c & 1, w0);
        store_a((c + 1) & 1);
        __syncthreads();
        load_a(c + 2);
        load_w(w0, c + 3);
        mma((c + 1) & 1, w1);
        store_a(c & 1);
        __syncthreads();
        load_a(c + 3);
        load_w(w1, c + 4);
        mma(c & 1, w2);
        store_a((c + 1) & 1);
        __syncthreads();
    }
    if (c < nc) {
        load_a(c + 1);
        mma(c & 1, w0);
        store_a((c + 1) & 1);
        __syncthreads();
        if (c + 1 < nc) mma((c + 1) & 1, w1);
    }
#endif


    // ---- epilogue: lane holds rows i*16 + 4*grp + e, columns of fragment f at col
    if constexpr (EPI == SK_GATED) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = i * 16 + 4 * grp + e;
                if (m >= p.M) continue;
#pragma unroll
                for (int q = 0; q < kSNB / 2; ++q) {
                    const int j = tile * (kSCols / 2) + wave * 8 * kSNB + q * 16 + col;
                    if (j >= p.F) continue;
                    const float g = acc[i][2 * q][e], u = acc[i][2 * q + 1][e];
                    const float y = (p.act == 0 ? gelu_tanh(g) : silu(g)) * u;
                    static_cast<uint16_t*>(p.out)[(int64_t)m * p.out_ld + j] = (uint16_t)f32_to_bf16_bits(y);
                }
            }
    } else if constexpr (EPI == SK_ARGMAX) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = -INFINITY;
                int idx = 0x7fffffff;
                const int mrow = i * 16 + 4 * grp + e;
#pragma unroll
                for (int f = 0; f < kSNB; ++f) {
                    const int n = tile * kSCols + wave * 16 * kSNB + f * 16 + col;
                    if (n < p.N) {
                        const float y = acc[i][f][e];
                        argmax_pick(v, idx, (p.base && mrow < p.M) ? y + p.base[(int64_t)mrow * p.base_ld + n] : y, n);
                    }
                }
                // the 16 lanes of a group hold the same row
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) {
                    const float v2 = __shfl_xor(v, o, kWave);
                    const int i2 = __shfl_xor(idx, o, kWave);
                    argmax_pick(v, idx, v2, i2);
                }
                if (col == 0) {
                    red_v[wave][i * 16 + 4 * grp + e] = v;
                    red_i[wave][i * 16 + 4 * grp + e] = idx;
                }
            }
        __syncthreads();
        const int m = threadIdx.x;
        if (m < p.M) {
            float v = red_v[0][m];
            int idx = red_i[0][m];
#pragma unroll
            for (int w = 1; w < kSW; ++w) argmax_pick(v, idx, red_v[w][m], red_i[w][m]);
            p.part_val[(int64_t)m * p.nblocks + tile] = v;
            p.part_idx[(int64_t)m * p.nblocks + tile] = idx;
        }
    } else {
        float* part = (EPI == SK_PARTIAL) ? p.part + ((int64_t)z * p.nsplit + split) * p.M * p.N : nullptr;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = i * 16 + 4 * grp + e;
                if (m >= p.M) continue;
                int kb = 0, kpos = -1;
                if constexpr (EPI == SK_KV) {
                    kb = meta_b[m];
                    kpos = meta_pos[m];
                    if (kpos < 0) continue;
                }
#pragma unroll
                for (int f = 0; f < kSNB; ++f) {
                    const int n = tile * kSCols + wave * 16 * kSNB + f * 16 + col;
                    if (n >= p.N) continue;
                    if constexpr (EPI == SK_PARTIAL)
                        part[(int64_t)m * p.N + n] = acc[i][f][e];
                    else if constexpr (EPI == SK_KV)
                        kv_store(p, z, kb, kpos, n, acc[i][f][e]);
                    else
                        store_one<EPI>(p, m, n, acc[i][f][e]);
                }
            }
    }
    trace_end(p.stamps, t_start);
}

// the sum of the split-K partials in split order, then the epilogue; 4 outputs a
// thread, grid.y = layer. SK_GATED (N = F): the partials hold 2F rows per activation
// row, gate rows [0, F) then up rows [F, 2F)
template <int EPI>
__global__ __launch_bounds__(kBlock) void skinny_reduce_kernel(const SkinnyParams p) {
    const int64_t mn = (int64_t)p.M * p.N;
    const int64_t e = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
    if (e >= mn) return;
    const int z = blockIdx.y;
    const int m = (int)(e / p.N), n = (int)(e - (int64_t)m * p.N);
    if constexpr (EPI == SK_GATED) {
        // partials hold the 2F gate and up rows; this thread's 4 outputs j = n .. n+3 (N = F)
        const int64_t mn2 = 2 * mn;
        const float* gp = p.part + (int64_t)m * 2 * p.N + n;
        float4 g = *reinterpret_cast<const float4*>(gp), u = *reinterpret_cast<const float4*>(gp + p.N);
        for (int sp = 1; sp < p.nsplit; ++sp) {
            const float4 tg = *reinterpret_cast<const float4*>(gp + sp * mn2);
            const float4 tu = *reinterpret_cast<const float4*>(gp + sp * mn2 + p.N);
            g.x += tg.x; g.y += tg.y; g.z += tg.z; g.w += tg.w;
            u.x += tu.x; u.y += tu.y; u.z += tu.z; u.w += tu.w;
        }
        const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
        uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t)m * p.out_ld + n;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = (uint16_t)f32_to_bf16_bits((p.act == 0 ? gelu_tanh(gv[q]) : silu(gv[q])) * uv[q]);
        return;
    }
    const float* src = p.part + (int64_t)z * p.nsplit * mn + e;
    float4 s = *reinterpret_cast<const float4*>(src);
    for (int sp = 1; sp < p.nsplit; ++sp) {
        const float4 t = *reinterpret_cast<const float4*>(src + sp * mn);
        s.x += t.x;
        s.y += t.y;
        s.z += t.z;
        s.w += t.w;
    }
    if constexpr (EPI == SK_KV) {
        int b, pos;
        kv_slot(p, p.row_base + m, b, pos);
        if (pos < 0) return;
        kv_store(p, z, b, pos, n, s.x);
        kv_store(p, z, b, pos, n + 1, s.y);
        kv_store(p, z, b, pos, n + 2, s.z);
        kv_store(p, z, b, pos, n + 3, s.w);
    } else {
        store_one<EPI>(p, m, n, s.x);
        store_one<EPI>(p, m, n + 1, s.y);
        store_one<EPI>(p, m, n + 2, s.z);
        store_one<EPI>(p, m, n + 3, s.w);
    }
}

// one wavefront per row: the row and its sum of squares in registers, then the
// scaled row rounded to bf16; grid.y = layer (gain), or every layer in turn from
// the same registers when all_layers is set
__global__ __launch_bounds__(kBlock) void norm_rows_kernel(const NormRowsParams p) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= p.rows) return;
    constexpr int UM = kNormMaxK / 512;
    const float* src = p.x + (int64_t)row * p.x_ld;
    float v[UM][8];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < UM; ++u) {
        const int k = lane * 8 + u * 512;
        if (k < p.K) {
            const float4 a = *reinterpret_cast<const float4*>(src + k);
            const float4 b = *reinterpret_cast<const float4*>(src + k + 4);
            v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
            v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[u][e] * v[u][e];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)p.K + p.eps);
    const int z0 = p.all_layers ? 0 : (int)blockIdx.y, z1 = p.all_layers ? p.layers : z0 + 1;
    for (int z = z0; z < z1; ++z) {
        const void* gain = p.gain[0];
#pragma unroll
        for (int q = 1; q < kMaxLayers; ++q)
            if (z == q) gain = p.gain[q];
        uint16_t* o = p.dst + (int64_t)z * p.dst_layer_stride + (int64_t)row * p.dst_ld;
#pragma unroll
        for (int u = 0; u < UM; ++u) {
            const int k = lane * 8 + u * 512;
            if (k < p.K) {
                float g[8];
                load_gain8(gain, p.gain_f32, k, g);
                uint4 q;
                q.x = pack_bf16x2(v[u][0] * r * g[0], v[u][1] * r * g[1]);
                q.y = pack_bf16x2(v[u][2] * r * g[2], v[u][3] * r * g[3]);
                q.z = pack_bf16x2(v[u][4] * r * g[4], v[u][5] * r * g[5]);
                q.w = pack_bf16x2(v[u][6] * r * g[6], v[u][7] * r * g[7]);
                *reinterpret_cast<uint4*>(o + k) = q;
            }
        }
    }
}

// one workgroup per row: the split partials summed in order into the residual row,
// its sum of squares reduced over the workgroup, then the normalised row as bf16
constexpr int kRnThreads = 1024;  // a row of up to 8192 values: two float4 per thread, all loads in flight at once
__global__ __launch_bounds__(kRnThreads) void resid_norm_kernel(const float* part, int nsplit, int M, int N, float* h,
                                                                int64_t h_ld, const void* gain, int gain_f32, float eps,
                                                                uint16_t* dst, int64_t dst_ld) {
    constexpr int kBlock = kRnThreads;
    constexpr int U = kNormMaxK / (4 * kBlock);
    __shared__ float red[kBlock / kWave];
    const int m = blockIdx.x, tid = threadIdx.x;
    const int64_t mn = (int64_t)M * N;
    float* hr = h + (int64_t)m * h_ld;
    float4 v[U];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = (tid + u * kBlock) * 4;
        if (k < N) {
            const float* src = part + (int64_t)m * N + k;
            float4 a = *reinterpret_cast<const float4*>(src);
#pragma unroll 8
            for (int sp = 1; sp < nsplit; ++sp) {
                const float4 t = *reinterpret_cast<const float4*>(src + sp * mn);
                a.x += t.x;
                a.y += t.y;
                a.z += t.z;
                a.w += t.w;
            }
            const float4 o = *reinterpret_cast<const float4*>(hr + k);
            v[u] = make_float4(o.x + a.x, o.y + a.y, o.z + a.z, o.w + a.w);
            *reinterpret_cast<float4*>(hr + k) = v[u];
            ss += v[u].x * v[u].x + v[u].y * v[u].y + v[u].z * v[u].z + v[u].w * v[u].w;
        }
    }
    ss = wave_sum(ss);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) tot += red[w];
    const float r = 1.0f / sqrtf(tot / (float)N + eps);
    uint16_t* o = dst + (int64_t)m * dst_ld;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = (tid + u * kBlock) * 4;
        if (k < N) {
            float g[4];
            if (gain_f32) {
                const float4 gv = *reinterpret_cast<const float4*>(static_cast<const float*>(gain) + k);
                g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
            } else {
                const uint2 gv = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(gain) + k);
                g[0] = bf16_lo(gv.x); g[1] = bf16_hi(gv.x); g[2] = bf16_lo(gv.y); g[3] = bf16_hi(gv.y);
            }
            uint2 q;
            q.x = pack_bf16x2(v[u].x * r * g[0], v[u].y * r * g[1]);
            q.y = pack_bf16x2(v[u].z * r * g[2], v[u].w * r * g[3]);
            *reinterpret_cast<uint2*>(o + k) = q;
        }
    }
}

// instrumentation: the stamp slice of one matrix-core launch (algorithmic bytes =
// weights + activation rows + outputs, per layer)
template <int MT, int EPI>
uint64_t* skinny_trace(const SkinnyParams& p, int tiles) {
    const double nout = EPI == SK_GATED ? p.N / 2 : (EPI == SK_ARGMAX ? 0 : p.N);
    const double bytes = p.layers * ((double)p.N * p.K * 2.0 + (double)p.M * p.K * 2.0 + (double)p.M * nout * 4.0);
    char name[48];
    snprintf(name, sizeof name, "skinny_kernel<%d, %d>", MT, EPI);
    return trace_launch(EPI == SK_ARGMAX ? TRACE_LM_HEAD : TRACE_PROJECTIONS, name,
                        (int64_t)tiles * p.nsplit * p.layers, bytes, 0.0);
}

template <int MT, int EPI>
hipError_t launch_mt(const SkinnyParams& p, hipStream_t s) {
    const int tiles = skinny_tiles(EPI, p.N);
    (void)hipGetLastError();  // report only these launches' status
    if constexpr (EPI == SK_STORE || EPI == SK_RESID || EPI == SK_KV) {
        if (p.nsplit > 1) {
            SkinnyParams q = p;
            q.stamps = skinny_trace<MT, SK_PARTIAL>(p, tiles);
            hipLaunchKernelGGL((skinny_kernel<MT, SK_PARTIAL>), dim3(tiles, p.nsplit, p.layers), dim3(kST), 0, s, q);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t blocks = ((int64_t)p.M * p.N / 4 + kBlock - 1) / kBlock;
            hipLaunchKernelGGL((skinny_reduce_kernel<EPI>), dim3((unsigned)blocks, p.layers), dim3(kBlock), 0, s, p);
            return hipGetLastError();
        }
    }
    SkinnyParams q = p;
    q.stamps = skinny_trace<MT, EPI>(p, tiles);
    hipLaunchKernelGGL((skinny_kernel<MT, EPI>), dim3(tiles, p.nsplit, p.layers), dim3(kST), 0, s, q);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const SkinnyParams& p, hipStream_t s) {
    switch ((p.M + 15) / 16) {
        case 1: return launch_mt<1, EPI>(p, s);
        case 2: return launch_mt<2, EPI>(p, s);
        case 3: return launch_mt<3, EPI>(p, s);
        case 4: return launch_mt<4, EPI>(p, s);
        case 5: return launch_mt<5, EPI>(p, s);
        case 6: return launch_mt<6, EPI>(p, s);
        case 7: return launch_mt<7, EPI>(p, s);
        case 8: return launch_mt<8, EPI>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int skinny_tiles(int epi, int N) {
    if (epi == SK_GATED) return (N / 2 + kSCols / 2 - 1) / (kSCols / 2);
    return (N + kSCols - 1) / kSCols;
}

void skinny_split(int epi, int N, int K, int layers, int* nsplit, int* kslice) {
    const int chunks = K / kSKC;
    int s = 1;
    if (epi == SK_STORE || epi == SK_RESID || epi == SK_KV || epi == SK_PARTIAL) {
        s = DFL_SK_WGS / (skinny_tiles(epi, N) * (layers > 0 ? layers : 1));
        s = s < 1 ? 1 : (s > chunks ? chunks : s);
    }
    const int per = chunks > 0 ? (chunks + s - 1) / s : 1;
    *kslice = per * kSKC;
    *nsplit = chunks > 0 ? (chunks + per - 1) / per : 1;
}

hipError_t launch_skinny(int epi, const SkinnyParams& p, hipStream_t s) {
    if (p.M < 1 || p.M > kSkinnyRows || p.N <= 0 || p.K <= 0 || (p.K % kSKC)) return hipErrorInvalidValue;
    if (p.layers < 1 || p.layers > kMaxLayers || (p.layers > 1 && epi != SK_KV && epi != SK_PARTIAL))
        return hipErrorInvalidValue;
    if (p.kslice <= 0 || (p.kslice % kSKC) || p.nsplit < 1 || (int64_t)p.nsplit * p.kslice < p.K ||
        (int64_t)(p.nsplit - 1) * p.kslice >= p.K)
        return hipErrorInvalidValue;
    const bool partials = p.nsplit > 1 || epi == SK_PARTIAL;
    if (partials && (!p.part || (p.N % 4) || epi == SK_GATED || epi == SK_ARGMAX)) return hipErrorInvalidValue;
    if (p.seg_k < 0 || (p.seg_k > 0 && ((p.seg_k % kSKC) || p.K > kMaxTaps * p.seg_k))) return hipErrorInvalidValue;
    if (epi == SK_GATED && (p.F <= 0 || p.N != 2 * p.F)) return hipErrorInvalidValue;
    if (epi == SK_ARGMAX && p.nblocks != skinny_tiles(SK_ARGMAX, p.N)) return hipErrorInvalidValue;
    if (epi == SK_STORE && p.vt && (p.gamma <= 0 || p.gamma > 32 || p.hd <= 0 || p.hkv <= 0))
        return hipErrorInvalidValue;
    if (epi == SK_KV && (p.N != 2 * p.hkv * p.hd || p.B < 1 || p.cap <= 0 || !p.kcache || !p.vcache || !p.len ||
                         !p.row_offsets))
        return hipErrorInvalidValue;
    switch (epi) {
        case SK_STORE: return launch_epi<SK_STORE>(p, s);
        case SK_RESID: return launch_epi<SK_RESID>(p, s);
        case SK_GATED: return launch_epi<SK_GATED>(p, s);
        case SK_ARGMAX: return launch_epi<SK_ARGMAX>(p, s);
        case SK_KV: return launch_epi<SK_KV>(p, s);
        case SK_PARTIAL: return launch_epi<SK_PARTIAL>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(int epi, const SkinnyParams& p, hipStream_t s) {
    if (p.M < 1 || p.N <= 0 || (p.N % 4) || p.nsplit < 1 || !p.part) return hipErrorInvalidValue;
    if (epi == SK_KV ? (!p.kcache || !p.vcache || p.layers < 1 || p.layers > kMaxLayers) : !p.out)
        return hipErrorInvalidValue;
    const int64_t blocks = ((int64_t)p.M * p.N / 4 + kBlock - 1) / kBlock;
    (void)hipGetLastError();  // report only this launch's status
    if (epi == SK_RESID)
        hipLaunchKernelGGL((skinny_reduce_kernel<SK_RESID>), dim3((unsigned)blocks, 1), dim3(kBlock), 0, s, p);
    else if (epi == SK_GATED)
        hipLaunchKernelGGL((skinny_reduce_kernel<SK_GATED>), dim3((unsigned)blocks, 1), dim3(kBlock), 0, s, p);
    else if (epi == SK_STORE)
        hipLaunchKernelGGL((skinny_reduce_kernel<SK_STORE>), dim3((unsigned)blocks, 1), dim3(kBlock), 0, s, p);
    else if (epi == SK_KV)
        hipLaunchKernelGGL((skinny_reduce_kernel<SK_KV>), dim3((unsigned)blocks, (unsigned)p.layers), dim3(kBlock), 0,
                           s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_resid_norm(const float* part, int nsplit, int M, int N, float* h, int64_t h_ld, const void* gain,
                             int gain_f32, float eps, uint16_t* dst, int64_t dst_ld, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (N <= 0 || (N % 4) || N > kNormMaxK || nsplit < 1 || (h_ld % 4) || (dst_ld % 4)) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(resid_norm_kernel, dim3((unsigned)M), dim3(kRnThreads), 0, s, part, nsplit, M, N, h, h_ld, gain,
                       gain_f32, eps, dst, dst_ld);
    return hipGetLastError();
}

hipError_t launch_norm_rows(const NormRowsParams& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    if (p.K <= 0 || (p.K % 8) || p.K > kNormMaxK || (p.x_ld % 4) || (p.dst_ld % 8) || (p.dst_layer_stride % 8) ||
        p.layers < 1 || p.layers > kMaxLayers)
        return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(norm_rows_kernel, dim3((unsigned)((p.rows + 3) / 4), p.all_layers ? 1 : p.layers),
                       dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace dfl
