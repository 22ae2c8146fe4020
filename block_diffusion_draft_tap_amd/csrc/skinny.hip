// Matrix-core projections of the drafter's block rows when a batch of
// sequences gives 16 or more of them (B sequences x gamma block tokens, the
// Q/K/V, output, FFN and LM-head products of each round). At that row count a
// projection is a small dense contraction; the per-8-row GEMV passes would
// stream each weight matrix from HBM once per 8 rows, here it is streamed once.
//
// A workgroup of kSW wavefronts owns kSCols consecutive weight rows (output
// columns) and walks K in chunks of 128. Each wavefront streams its own
// 16 * kSNB weight rows into registers one chunk ahead of the one it
// multiplies, reading whole rows: 16 lanes take 256 contiguous bytes of one
// row (16-row, 64-byte pieces per load, the B-operand layout itself, stream
// about a fifth slower from HBM). Before the products, each 16-row fragment
// passes through the wavefront's own LDS tile into the B-operand layout of
// v_mfma_f32_16x16x32_bf16 (lane l: weight row l % 16, k offset 8 (l / 16)).
// The activation chunk (all M rows x 128) is shared by the wavefronts through
// LDS, double buffered with one barrier per chunk; every workgroup of a launch
// reads the same activation rows, so they mostly come from L2. A chunk's
// activations are loaded before its weights: loads complete in issue order,
// so the wait for them (before their LDS store) leaves the weights in flight
// across the barrier. LDS rows hold 16 pieces of 16 bytes, piece p of row r
// at slot p ^ (r % 16), so fragment reads (16 rows, one piece each) and row
// stores both touch every bank once. Lane l holds
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
// wavefronts per SIMD the kernel is compiled for: two (two workgroups per CU, one's LDS and
// barrier work overlapping the other's weight stream); the 8-fragment (113 to 128 rows)
// kernel keeps one
#ifndef DFL_SK_OCC
#define DFL_SK_OCC 2
#endif


namespace {

constexpr int kSW = DFL_SK_WAVES, kSNB = DFL_SK_NB, kST = 64 * kSW;
constexpr int kSCols = 16 * kSNB * kSW;  // weight rows per workgroup tile
constexpr int kSKC = kSkinnyK;           // K per chunk
constexpr int kSSteps = kSKC / 32;       // MFMA k-steps per chunk
static_assert(kSSteps == 4 && kSKC == 128, "a weight row's chunk is 16 lanes x 16 bytes; 16 rows take 4 loads");
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
    base[hb + (which ? v_cache_off(pos, dim, p.hd, p.cap, false) : (int64_t)pos * p.hd + dim)] =
        (uint16_t)f32_to_bf16_bits(y);
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

// ---- epilogue: lane holds rows i*16 + 4*grp + e, columns of fragment f at col. red_v /
// red_i: [kSW][RED] LDS scratch of the argmax; meta_b / meta_pos: the K/V cache slots of
// the rows (set before the main loop's barriers)
template <int MT, int EPI>
__device__ __forceinline__ void skinny_epilogue(const SkinnyParams& p, f32x4 (&acc)[MT][kSNB], const int tile,
                                                const int split, const int z, const int wave, const int col,
                                                const int grp, float* red_v, int* red_i, const int* meta_b,
                                                const int* meta_pos) {
    constexpr int RED = EPI == SK_ARGMAX ? MT * 16 : 1;
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
                    red_v[wave * RED + i * 16 + 4 * grp + e] = v;
                    red_i[wave * RED + i * 16 + 4 * grp + e] = idx;
                }
            }
        __syncthreads();
        const int m = threadIdx.x;
        if (m < p.M) {
            float v = red_v[m];
            int idx = red_i[m];
#pragma unroll
            for (int w = 1; w < kSW; ++w) argmax_pick(v, idx, red_v[w * RED + m], red_i[w * RED + m]);
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
}

template <int MT, int EPI>
__global__ __launch_bounds__(kST, MT >= 8 ? 1 : DFL_SK_OCC) void skinny_kernel(const SkinnyParams p) {
    constexpr int RED = EPI == SK_ARGMAX ? MT * 16 : 1;
    constexpr int META = EPI == SK_KV ? MT * 16 : 1;
    // LDS tiles, rows of 16 pieces of 16 bytes with piece p of row r at slot p ^ (r % 16): the
    // 16 lanes of a fragment read (rows col, one piece each) and of a row write (one row,
    // all pieces) both touch every bank once
    __shared__ __align__(16) uint16_t As[2][MT * 16][kSKC];  // activation chunk, double buffered
    __shared__ __align__(16) uint16_t Ws[kSW][16][kSKC];     // a wavefront's weight fragment in transit
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

    // weight rows of this wavefront: fragment f, row r of the fragment (rows past the end
    // read the last row; their outputs are never stored). Loads read whole rows: load s of
    // a fragment gives lane (col, grp) 16 bytes at k offset 8 col of row r = 4 s + grp (16
    // lanes read 256 contiguous bytes of a row), and the fragment then goes through the
    // wavefront's LDS tile into the B-operand layout (lane: row col, k offset 8 grp + 32 s)
    int jrow[kSNB];
#pragma unroll
    for (int f = 0; f < kSNB; ++f)
        jrow[f] = EPI == SK_GATED ? tile * (kSCols / 2) + wave * 8 * kSNB + (f / 2) * 16 + grp
                                  : tile * kSCols + wave * 16 * kSNB + f * 16 + grp;
    const uint16_t* wbase = W + p.w_row0 * (int64_t)p.K + kbeg + 8 * col;
    auto wrow = [&](int f, int s) {
        if constexpr (EPI == SK_GATED) return (f & 1) * p.F + min(jrow[f] + 4 * s, p.F - 1);
        return min(jrow[f] + 4 * s, p.N - 1);
    };

    f32x4 acc[MT][kSNB];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int f = 0; f < kSNB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // two register sets of weights: chunk c lives in set c % 2 from its load (during chunk
    // c - 1) until its stores into the wavefront's LDS tile. Loads past the last chunk re-read
    // it (never multiplied): unconditional loads let the compiler count the loads in flight,
    // so waiting for an older load never drains the younger ones
    u32x4 w0[kSNB][kSSteps], w1[kSNB][kSSteps];
    auto load_w = [&](u32x4 (&wr)[kSNB][kSSteps], int c) {
        const int cc = min(c, nc - 1);
#pragma unroll
        for (int f = 0; f < kSNB; ++f)
#pragma unroll
            for (int s = 0; s < kSSteps; ++s)
                wr[f][s] = stream_load(reinterpret_cast<const u32x4*>(wbase + (int64_t)wrow(f, s) * p.K + cc * kSKC));
    };
    // the activation chunk: MT*16 rows x 16 pieces of 16 bytes, spread over the threads
    constexpr int PIECES = MT * 16 * (kSKC / 8);
    constexpr int APT = (PIECES + kST - 1) / kST;
    u32x4 ast[APT];
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
            if (PIECES % kST == 0 || q < PIECES)
                *reinterpret_cast<u32x4*>(&As[buf][q >> 4][8 * ((q ^ (q >> 4)) & 15)]) = srcr[i];
        }
    };
    auto load_a = [&](int c) { load_a_into(ast, c); };
    auto store_a = [&](int buf) { store_a_from(ast, buf); };
    auto mma = [&](int buf, const u32x4 (&wr)[kSNB][kSSteps]) {
        // the fragments into B operands, one at a time through the wavefront's LDS tile (the
        // wavefront's LDS accesses complete in order, so the second fragment's stores follow
        // the first one's loads)
        u32x4 wb[kSNB][kSSteps];
#pragma unroll
        for (int f = 0; f < kSNB; ++f) {
#pragma unroll
            for (int s = 0; s < kSSteps; ++s) {
                const int r = 4 * s + grp;
                *reinterpret_cast<u32x4*>(&Ws[wave][r][8 * (col ^ r)]) = wr[f][s];
            }
#pragma unroll
            for (int s = 0; s < kSSteps; ++s)
                wb[f][s] = *reinterpret_cast<const u32x4*>(&Ws[wave][col][8 * ((4 * s + grp) ^ col)]);
        }
#pragma unroll
        for (int s = 0; s < kSSteps; ++s) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const u32x4 af = *reinterpret_cast<const u32x4*>(&As[buf][i * 16 + col][8 * ((4 * s + grp) ^ col)]);
#pragma unroll
                for (int f = 0; f < kSNB; ++f) acc[i][f] = mfma_bf16(af, wb[f][s], acc[i][f]);
            }
        }
    };

    // chunk c multiplies LDS buffer c % 2. Chunk c + 1's activations are loaded before its
    // weights, so the wait for them before their LDS store (after chunk c's products) leaves
    // the weights in flight across the barrier. Whole pairs of chunks run without branches (a
    // store into the idle buffer past the last chunk is never read); an odd last one follows.
    load_w(w0, 0);
    load_a(0);
    store_a(0);
    __syncthreads();
    int c = 0;
    for (; c + 2 <= nc; c += 2) {
        load_a(c + 1);
        load_w(w1, c + 1);
        mma(0, w0);
        store_a(1);
        __syncthreads();
        load_a(c + 2);
        load_w(w0, c + 2);
        mma(1, w1);
        store_a(0);
        __syncthreads();
    }
    if (c < nc) mma(0, w0);

    skinny_epilogue<MT, EPI>(p, acc, tile, split, z, wave, col, grp, &red_v[0][0], &red_i[0][0], meta_b, meta_pos);
    trace_end(p.stamps, t_start);
}

// Direct-to-LDS variant, for many activation rows: there the products and LDS reads per
// weight byte are several times those of a few rows, a workgroup's activation tiles take
// most of a CU's LDS, and weights kept in flight in registers are what the register budget
// leaves over. Here weights and activations go from memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's LDS base + 16 l),
// with no staging registers, and each wavefront keeps its weight rows kDmaStages chunks deep
// in its own LDS stages (two chunks ahead of the one it multiplies). The loads choose their
// sources so that the LDS tiles come out in the slot layout above (piece p of row r at slot
// p ^ (r % 16)); a row's 16 lanes still read its 256 contiguous bytes.
//
// Chunk c's activations are loaded after the barrier that ends chunk c - 1's reads of their
// buffer, and before chunk c + 1's weights; the wait at the top of chunk c (this wavefront's
// chunk c weights and activations landed: only chunk c + 1's weights may still be in
// flight) then a barrier (every wavefront's activation pieces landed) open the products.
template <int MT>
constexpr int dma_stages() {
    return 2 * MT * 16 * kSKC * 2 + kSW * 3 * kSNB * 16 * kSKC * 2 + 4096 <= 163840 ? 3 : 2;
}

// 16 bytes a lane from src into LDS at lds_base + 16 * lane (lds_base the same in every lane).
// Written out as the instruction itself: the compiler, seeing the intrinsic's LDS store,
// would wait for every load in flight before each LDS read and barrier, which is the
// pipeline this kernel exists for; the waits are explicit here. M0 is taken at issue.
// (M0 is reserved to the compiler, which warns on the clobber; it keeps no value there in
// these kernels: M0 appears only in these instructions)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const uint16_t* src, const uint16_t* lds_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// the same with the non-temporal hint of streamed data (the weights)
__device__ __forceinline__ void lds_dma16_nt(const uint16_t* src, const uint16_t* lds_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)lds_base);
#if DFL_STREAM_NT
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds) : "memory", "m0");
#else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

// chunk c may start: this wavefront's loads other than the last `keep` (0 or 8) landed, its
// LDS reads done, then the workgroup barrier (the compiler sees a memory barrier)
__device__ __forceinline__ void dma_sync(const bool keep8) {
    if (keep8)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The 64-wide pipeline (DFL_SK_DMA_K64, for row tiles where the 128-wide one fits only two
// weight stages: 128 rows): K chunks of 64, four activation buffers and five weight stages,
// so a chunk's activations load three chunks ahead and its weights four (1.5 and 2 chunks
// of 128; measured at 128 rows 51.0 -> 47.7 us per context launch, at 112 rows, where the
// 128-wide pipeline keeps three weight stages, 25.6 -> 26.8 us per projection). Rows
// of 64 hold 8 pieces of 16 bytes, piece p of row r at slot p ^ ((r >> 1) & 7): a fragment
// read (16 rows, one piece each) touches every bank once. A chunk's activation pieces are
// padded to whole instructions (the padding lanes write slots past the tile, from clamped
// sources), so every wavefront issues the same loads.
#ifndef DFL_SK_DMA_K64
#define DFL_SK_DMA_K64 1
#endif
constexpr int kDK = 64, kDA64 = 4, kDW64 = 5;
template <int MT>
constexpr int k64_nai() {  // activation loads per thread per chunk
    return (MT * 16 * (kDK / 8) + kST - 1) / kST;
}

// chunk c may start (64-wide pipeline): this wavefront's loads other than the last keep
// landed, its LDS reads done, then the workgroup barrier; keep is one of four values known
// at compile time (three, two, one or no later chunks issued)
template <int K3, int K2, int K1>
__device__ __forceinline__ void dma_sync64(const int later) {
    if (later >= 3)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(K3) : "memory");
    else if (later == 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(K2) : "memory");
    else if (later == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(K1) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int MT, int EPI>
__global__ __launch_bounds__(kST, 1) void skinny_dma_kernel(const SkinnyParams p) {
    constexpr int RED = EPI == SK_ARGMAX ? MT * 16 : 1;
    constexpr int META = EPI == SK_KV ? MT * 16 : 1;
    constexpr int D = dma_stages<MT>();
    constexpr bool K64 = DFL_SK_DMA_K64 && D < 3;
    constexpr int NAI = k64_nai<MT>();
    // 128-wide pipeline: activation chunk double buffered, each wavefront's weight stages
    __shared__ __align__(16) uint16_t As[K64 ? 1 : 2][K64 ? 1 : MT * 16][K64 ? 8 : kSKC];
    __shared__ __align__(16) uint16_t Wst[K64 ? 1 : kSW][K64 ? 1 : D][kSNB][16][K64 ? 8 : kSKC];
    // 64-wide pipeline: activation buffers (NAI * kST pieces each) and weight stages
    __shared__ __align__(16) uint16_t As64[K64 ? kDA64 : 1][K64 ? NAI * kST * 8 : 8];
    __shared__ __align__(16) uint16_t Wst64[K64 ? kSW : 1][K64 ? kDW64 : 1][kSNB][16][K64 ? kDK : 8];
    __shared__ float red_v[kSW][RED];
    __shared__ int red_i[kSW][RED];
    __shared__ int meta_b[META], meta_pos[META];
    const uint64_t t_start = trace_start(p.stamps);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int z = blockIdx.z;
    const uint16_t* W = p.w[0];
#pragma unroll
    for (int q = 1; q < kMaxLayers; ++q)
        if (z == q) W = p.w[q];
    const uint16_t* A = p.a + (int64_t)z * p.a_layer_stride;

    if constexpr (EPI == SK_KV) {
        for (int m = threadIdx.x; m < MT * 16; m += kST) {
            int b = 0, pos = -1;
            if (m < p.M) kv_slot(p, p.row_base + m, b, pos);
            meta_b[m] = b;
            meta_pos[m] = pos;
        }
    }

    f32x4 acc[MT][kSNB];
    // 64-wide pipeline: the products of column tile `tile` over K [kbeg, kbeg + 64 nc)
    auto item64 = [&](const int tile, const int kbeg, const int nc) __attribute__((always_inline)) {
        // weight loads: instruction t of fragment f gives lane l row r = 8 t + (l >> 3) of the
        // fragment and LDS slot l & 7, which holds piece (l & 7) ^ ((r >> 1) & 7)
        const int lr = lane >> 3, lq = lane & 7;
        int jrow[kSNB];
#pragma unroll
        for (int f = 0; f < kSNB; ++f)
            jrow[f] = EPI == SK_GATED ? tile * (kSCols / 2) + wave * 8 * kSNB + (f / 2) * 16 + lr
                                      : tile * kSCols + wave * 16 * kSNB + f * 16 + lr;
        const uint16_t* wbase = W + p.w_row0 * (int64_t)p.K + kbeg;
        auto wrow = [&](int f, int t) {
            if constexpr (EPI == SK_GATED) return (f & 1) * p.F + min(jrow[f] + 8 * t, p.F - 1);
            return min(jrow[f] + 8 * t, p.N - 1);
        };
        auto load_w = [&](int c) {
            const int st = c % kDW64;
#pragma unroll
            for (int f = 0; f < kSNB; ++f)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int r = 8 * t + lr;
                    lds_dma16_nt(wbase + (int64_t)wrow(f, t) * p.K + c * kDK + 8 * (lq ^ ((r >> 1) & 7)),
                              &Wst64[wave][st][f][8 * t][0]);
                }
        };
        // activations: piece q = kST i + threadIdx.x of the chunk is row q / 8, slot q % 8
        auto load_a = [&](int c) {
            const int k0 = kbeg + c * kDK;
            const uint16_t* src;
            if (p.seg_k > 0) {  // tap segments (multiples of 128): a chunk never straddles two
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
            for (int i = 0; i < NAI; ++i) {
                const int q = min(kST * i + (int)threadIdx.x, MT * 16 * 8 - 1);
                const int row = q >> 3;
                const int piece = (q & 7) ^ ((row >> 1) & 7);
                lds_dma16(src + (int64_t)min(row, p.M - 1) * p.a_ld + 8 * piece,
                          &As64[c % kDA64][0] + (kST * i + 64 * wave) * 8);
            }
        };

#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int f = 0; f < kSNB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

        // chunk j's weights go out with chunk j - 1's activations (activations three chunks
        // ahead, weights four): at the top of chunk c only chunks c + 1 .. c + 3's loads after
        // chunk c's activations may be in flight
        constexpr int nW = 2 * kSNB;
        load_w(0);
#pragma unroll
        for (int j = 0; j < kDA64 - 1; ++j) {
            if (j < nc) load_a(j);
            if (j + 1 < nc) load_w(j + 1);
        }
        const int sw = (col >> 1) & 7;  // slot swizzle of the fragment rows this lane reads
        for (int c = 0; c < nc; ++c) {
            dma_sync64<3 * nW + 2 * NAI, 2 * nW + 2 * NAI, nW + NAI>(min(nc - 1 - c, 3));
            if (c + kDA64 - 1 < nc) load_a(c + kDA64 - 1);  // into the buffer chunk c - 1 read
            if (c + kDW64 - 1 < nc) load_w(c + kDW64 - 1);  // into the stage chunk c - 1 used
            const int st = c % kDW64, buf = c % kDA64;
#pragma unroll
            for (int s = 0; s < kDK / 32; ++s) {
                const int slot = (4 * s + grp) ^ sw;
                u32x4 wb[kSNB];
#pragma unroll
                for (int f = 0; f < kSNB; ++f)
                    wb[f] = *reinterpret_cast<const u32x4*>(&Wst64[wave][st][f][col][8 * slot]);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const u32x4 af = *reinterpret_cast<const u32x4*>(&As64[buf][(i * 16 + col) * kDK + 8 * slot]);
#pragma unroll
                    for (int f = 0; f < kSNB; ++f) acc[i][f] = mfma_bf16(af, wb[f], acc[i][f]);
                }
            }
        }
    };

    // the products of one work item: column tile `tile` over chunks [kbeg, kbeg + 128 nc)
    auto item = [&](const int tile, const int kbeg, const int nc) __attribute__((always_inline)) {
        if constexpr (K64) {
            item64(tile, kbeg, 2 * nc);
            return;
        }
        // weight rows: load s of fragment f gives lane (col, grp) row r = 4 s + grp of the
        // fragment, piece col ^ r (LDS slot col of that row)
        int jrow[kSNB];
#pragma unroll
        for (int f = 0; f < kSNB; ++f)
            jrow[f] = EPI == SK_GATED ? tile * (kSCols / 2) + wave * 8 * kSNB + (f / 2) * 16 + grp
                                      : tile * kSCols + wave * 16 * kSNB + f * 16 + grp;
        const uint16_t* wbase = W + p.w_row0 * (int64_t)p.K + kbeg;
        auto wrow = [&](int f, int s) {
            if constexpr (EPI == SK_GATED) return (f & 1) * p.F + min(jrow[f] + 4 * s, p.F - 1);
            return min(jrow[f] + 4 * s, p.N - 1);
        };
        auto load_w = [&](int c) {
            const int st = c % D;
#pragma unroll
            for (int f = 0; f < kSNB; ++f)
#pragma unroll
                for (int s = 0; s < kSSteps; ++s) {
                    const int r = 4 * s + grp;
                    lds_dma16_nt(wbase + (int64_t)wrow(f, s) * p.K + c * kSKC + 8 * (col ^ r), &Wst[wave][st][f][4 * s][0]);
                }
        };
        // activations: LDS piece q = kST i + threadIdx.x of the tile is row q / 16, slot q % 16
        auto load_a = [&](int c) {
            const int k0 = kbeg + c * kSKC;
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
            for (int i = 0; i < MT; ++i) {
                const int q = kST * i + (int)threadIdx.x;
                const int row = q >> 4;
                const int piece = (q & 15) ^ (row & 15);
                lds_dma16(src + (int64_t)min(row, p.M - 1) * p.a_ld + 8 * piece,
                          &As[c & 1][0][0] + (kST * i + 64 * wave) * 8);
            }
        };

#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int f = 0; f < kSNB; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

        load_a(0);
        load_w(0);
        if (D == 3 && nc > 1) load_w(1);
        for (int c = 0; c < nc; ++c) {
            // this wavefront's loads after chunk c's activations: chunk c + 1's weights (D = 3)
            dma_sync(D == 3 && c + 1 < nc);
            if (c + 1 < nc) load_a(c + 1);          // into the buffer chunk c - 1 read
            if (c + D - 1 < nc) load_w(c + D - 1);  // into the stage chunk c - 1 used
            const int st = c % D, buf = c & 1;
#pragma unroll
            for (int s = 0; s < kSSteps; ++s) {
                u32x4 wb[kSNB];
#pragma unroll
                for (int f = 0; f < kSNB; ++f)
                    wb[f] = *reinterpret_cast<const u32x4*>(&Wst[wave][st][f][col][8 * ((4 * s + grp) ^ col)]);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const u32x4 af =
                        *reinterpret_cast<const u32x4*>(&As[buf][i * 16 + col][8 * ((4 * s + grp) ^ col)]);
#pragma unroll
                    for (int f = 0; f < kSNB; ++f) acc[i][f] = mfma_bf16(af, wb[f], acc[i][f]);
                }
            }
        }
    };

    if constexpr (EPI == SK_GATED) {
        if (p.bal_main > 0) {
            // balanced launch: whole tiles blockIdx.x, + gridDim.x, ... below bal_main, then at
            // most one K range of a tail tile, whose partial sums of the gate and up rows go to
            // bal_part [split][M][2 Ft] (gate columns [0, Ft), up [Ft, 2 Ft), Ft the tail's
            // gate rows) for the gated reduce. Before each item after the first, every
            // wavefront's reads of the LDS tiles end (the next item's loads refill them).
            bool first = true;
            for (int t = blockIdx.x; t < p.bal_main; t += gridDim.x) {
                if (!first) dma_sync(false);
                first = false;
                item(t, 0, p.K / kSKC);
                skinny_epilogue<MT, EPI>(p, acc, t, 0, z, wave, col, grp, &red_v[0][0], &red_i[0][0], meta_b,
                                         meta_pos);
            }
            const int q = blockIdx.x;
            if (q < p.bal_items) {
                if (!first) dma_sync(false);
                const int t = p.bal_main + q / p.bal_splits, sp = q % p.bal_splits;
                const int kb = sp * p.bal_kslice;
                item(t, kb, (min(p.K, kb + p.bal_kslice) - kb) / kSKC);
                const int j0 = p.bal_main * (kSCols / 2), Ft = p.F - j0;
                float* part = p.bal_part + (int64_t)sp * p.M * 2 * Ft;
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = i * 16 + 4 * grp + e;
                        if (m >= p.M) continue;
#pragma unroll
                        for (int f = 0; f < kSNB; ++f) {
                            const int j = t * (kSCols / 2) + wave * 8 * kSNB + (f / 2) * 16 + col;
                            if (j < p.F) part[(int64_t)m * 2 * Ft + (f & 1) * Ft + (j - j0)] = acc[i][f][e];
                        }
                    }
            }
            trace_end(p.stamps, t_start);
            return;
        }
    }
    const int tile = blockIdx.x, split = blockIdx.y;
    const int kbeg = split * p.kslice;
    item(tile, kbeg, (min(p.K, kbeg + p.kslice) - kbeg) / kSKC);
    skinny_epilogue<MT, EPI>(p, acc, tile, split, z, wave, col, grp, &red_v[0][0], &red_i[0][0], meta_b, meta_pos);
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

// the block rows of B sequences (row r = b gamma + j) with the first layer's RMSNorm:
// j = 0: v = sum_s part[s][b] (split order) + block_pos[0], the anchor's token projection
// from its split partials; j > 0: v = mask_emb[j - 1] + block_pos[j]. h[r] = v (fp32),
// dst[r] = bf16(v (mean v^2 + eps)^-1/2 gain). One workgroup per row, as resid_norm_kernel
__global__ __launch_bounds__(kRnThreads) void block_norm_kernel(const float* part, int nsplit, int B, int gamma, int N,
                                                                float* h, const uint16_t* block_pos,
                                                                const uint16_t* mask_emb, const void* gain,
                                                                int gain_f32, float eps, uint16_t* dst) {
    constexpr int kBlock = kRnThreads;
    constexpr int U = kNormMaxK / (4 * kBlock);
    __shared__ float red[kBlock / kWave];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int b = r / gamma, j = r - b * gamma;
    const int64_t bn = (int64_t)B * N;
    float* hr = h + (int64_t)r * N;
    float4 v[U];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = (tid + u * kBlock) * 4;
        if (k < N) {
            const uint2 bp = *reinterpret_cast<const uint2*>(block_pos + (int64_t)j * N + k);
            float4 a;
            if (j == 0) {
                const float* src = part + (int64_t)b * N + k;
                a = *reinterpret_cast<const float4*>(src);
#pragma unroll 8
                for (int sp = 1; sp < nsplit; ++sp) {
                    const float4 t = *reinterpret_cast<const float4*>(src + sp * bn);
                    a.x += t.x;
                    a.y += t.y;
                    a.z += t.z;
                    a.w += t.w;
                }
            } else {
                const uint2 me = *reinterpret_cast<const uint2*>(mask_emb + (int64_t)(j - 1) * N + k);
                a = make_float4(bf16_lo(me.x), bf16_hi(me.x), bf16_lo(me.y), bf16_hi(me.y));
            }
            v[u] = make_float4(a.x + bf16_lo(bp.x), a.y + bf16_hi(bp.x), a.z + bf16_lo(bp.y), a.w + bf16_hi(bp.y));
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
    const float rs = 1.0f / sqrtf(tot / (float)N + eps);
    uint16_t* o = dst + (int64_t)r * N;
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
            q.x = pack_bf16x2(v[u].x * rs * g[0], v[u].y * rs * g[1]);
            q.y = pack_bf16x2(v[u].z * rs * g[2], v[u].w * rs * g[3]);
            *reinterpret_cast<uint2*>(o + k) = q;
        }
    }
}

// instrumentation: the stamp slice of one matrix-core launch (algorithmic bytes =
// weights + activation rows + outputs, per layer)
// The direct-to-LDS kernel serves launches of at least DFL_SK_DMA_MIN_MT row tiles whose
// workgroups number at most DFL_SK_DMA_MAX_WGS (about one per CU of the 256-CU part, where
// its deeper weight stream pays); with more workgroups, two register-path workgroups per CU
// keep more in flight than its one (measured: the 2374-tile LM head of 112 rows, 361 us
// direct against 335 us per round with the non-temporal weight loads on both, 444 against
// 377 before them, and the 544-workgroup gate/up product are faster on the register path;
// the 224-240 workgroup Q/K/V, O, down and K/V launches 14-16% faster direct).
#ifndef DFL_SK_DMA_MIN_MT
#define DFL_SK_DMA_MIN_MT 5
#endif
#ifndef DFL_SK_DMA_MAX_WGS
#define DFL_SK_DMA_MAX_WGS 384
#endif

template <int MT>
bool use_dma(const SkinnyParams& p, int tiles) {
    return MT >= DFL_SK_DMA_MIN_MT && (int64_t)tiles * p.nsplit * p.layers <= DFL_SK_DMA_MAX_WGS;
}

template <int MT, int EPI>
uint64_t* skinny_trace(const SkinnyParams& p, int tiles) {
    const double nout = EPI == SK_GATED ? p.N / 2 : (EPI == SK_ARGMAX ? 0 : p.N);
    const double bytes = p.layers * ((double)p.N * p.K * 2.0 + (double)p.M * p.K * 2.0 + (double)p.M * nout * 4.0);
    char name[48];
    snprintf(name, sizeof name, use_dma<MT>(p, tiles) ? "skinny_dma_kernel<%d, %d>" : "skinny_kernel<%d, %d>", MT,
             EPI);
    return trace_launch(EPI == SK_ARGMAX ? TRACE_LM_HEAD : TRACE_PROJECTIONS, name,
                        (int64_t)tiles * p.nsplit * p.layers, bytes, 0.0);
}

template <int MT, int EPI>
void launch_kernel(const SkinnyParams& q, const int tiles, hipStream_t s) {
    const dim3 grid(tiles, q.nsplit, q.layers);
    if constexpr (MT >= DFL_SK_DMA_MIN_MT) {
        if (use_dma<MT>(q, tiles)) {
            hipLaunchKernelGGL((skinny_dma_kernel<MT, EPI>), grid, dim3(kST), 0, s, q);
            return;
        }
    }
    hipLaunchKernelGGL((skinny_kernel<MT, EPI>), grid, dim3(kST), 0, s, q);
}

template <int MT, int EPI>
hipError_t launch_mt(const SkinnyParams& p, hipStream_t s) {
    const int tiles = skinny_tiles(EPI, p.N);
    (void)hipGetLastError();  // report only these launches' status
    if constexpr (EPI == SK_STORE || EPI == SK_RESID || EPI == SK_KV) {
        if (p.nsplit > 1) {
            SkinnyParams q = p;
            q.stamps = skinny_trace<MT, SK_PARTIAL>(p, tiles);
            launch_kernel<MT, SK_PARTIAL>(q, tiles, s);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int64_t blocks = ((int64_t)p.M * p.N / 4 + kBlock - 1) / kBlock;
            hipLaunchKernelGGL((skinny_reduce_kernel<EPI>), dim3((unsigned)blocks, p.layers), dim3(kBlock), 0, s, p);
            return hipGetLastError();
        }
    }
    SkinnyParams q = p;
    q.stamps = skinny_trace<MT, EPI>(p, tiles);
    launch_kernel<MT, EPI>(q, tiles, s);
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

// The gated product balanced over the CUs on the direct-to-LDS kernel (one workgroup per
// CU): with T column tiles and G CUs, each workgroup takes T / G whole tiles and the rest
// (T mod G tiles) is split into K ranges of nearly equal length, at most one per workgroup,
// whose partial sums the gated reduce adds in range order. A plain launch of T > G tiles at
// one workgroup per CU would take a second full round of the chip for the last T mod G.
constexpr int kMaxCus = 512;  // bound of the tail partials' size (devices up to this many CUs)

int device_cus() {
    static int cus[16] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n < kMaxCus ? n : kMaxCus;
    }
    return cus[dev];
}

struct GatedPlan {
    int main, rem, splits, kslice, items;
};

bool gated_plan(int M, int N2, int K, GatedPlan* g) {
    const int MT = (M + 15) / 16;
    if (MT < DFL_SK_DMA_MIN_MT || MT > 8 || (N2 % 8) || (K % kSKC)) return false;
    const int F = N2 / 2, T = skinny_tiles(SK_GATED, N2), G = device_cus(), nc = K / kSKC;
    if (T <= G || (F % 4)) return false;
    g->main = (T / G) * G;
    g->rem = T - g->main;
    g->splits = 0;
    g->kslice = K;
    g->items = 0;
    if (g->rem > 0) {
        int kch = (nc * g->rem + G - 1) / G;
        while (g->rem * ((nc + kch - 1) / kch) > G) ++kch;
        g->splits = (nc + kch - 1) / kch;
        g->kslice = kch * kSKC;
        g->items = g->rem * g->splits;
    }
    return true;
}

template <int MT>
hipError_t launch_gated_balanced(SkinnyParams q, const GatedPlan& g, hipStream_t s) {
    q.bal_main = g.main;
    q.bal_items = g.items;
    q.bal_splits = g.splits > 0 ? g.splits : 1;
    q.bal_kslice = g.kslice;
    q.bal_part = q.part;
    q.nsplit = 1;
    q.kslice = q.K;
    const int G = device_cus();
    const dim3 grid((unsigned)G, 1, 1);
    char name[48];
    snprintf(name, sizeof name, "skinny_dma_kernel<%d, %d>", MT, SK_GATED);
    const double bytes = (double)q.N * q.K * 2.0 + (double)q.M * q.K * 2.0 + (double)q.M * (q.N / 2) * 2.0;
    q.stamps = trace_launch(TRACE_PROJECTIONS, name, G, bytes, 0.0);
    (void)hipGetLastError();
    hipLaunchKernelGGL((skinny_dma_kernel<MT, SK_GATED>), grid, dim3(kST), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.items == 0) return e;
    // the tail's gate and up partial sums, added in range order, then the activation
    const int j0 = g.main * (kSCols / 2), Ft = q.F - j0;
    SkinnyParams r = q;
    r.N = Ft;
    r.part = q.bal_part;
    r.nsplit = g.splits;
    r.out = static_cast<uint16_t*>(q.out) + j0;
    r.layers = 1;
    const int64_t blocks = ((int64_t)r.M * r.N / 4 + kBlock - 1) / kBlock;
    hipLaunchKernelGGL((skinny_reduce_kernel<SK_GATED>), dim3((unsigned)blocks, 1), dim3(kBlock), 0, s, r);
    return hipGetLastError();
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

size_t skinny_gated_balanced_floats(int M) { return (size_t)M * 2 * (kSCols / 2) * kMaxCus; }

bool skinny_gated_balanced(int M, int N, int K) {
    GatedPlan g;
    return gated_plan(M, N, K, &g);
}

hipError_t launch_skinny_gated_balanced(const SkinnyParams& p, hipStream_t s) {
    GatedPlan g;
    if (p.layers != 1 || p.F * 2 != p.N || !p.part || !p.out || !gated_plan(p.M, p.N, p.K, &g))
        return hipErrorInvalidValue;
    switch ((p.M + 15) / 16) {
        case 5: return launch_gated_balanced<5>(p, g, s);
        case 6: return launch_gated_balanced<6>(p, g, s);
        case 7: return launch_gated_balanced<7>(p, g, s);
        case 8: return launch_gated_balanced<8>(p, g, s);
    }
    return hipErrorInvalidValue;
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

hipError_t launch_block_norm(const float* part, int nsplit, int B, int gamma, int N, float* h,
                             const uint16_t* block_pos, const uint16_t* mask_emb, const void* gain, int gain_f32,
                             float eps, uint16_t* dst, hipStream_t s) {
    if (B <= 0 || gamma <= 0) return hipSuccess;
    if (N <= 0 || (N % 4) || N > kNormMaxK || nsplit < 1) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(block_norm_kernel, dim3((unsigned)(B * gamma)), dim3(kRnThreads), 0, s, part, nsplit, B, gamma,
                       N, h, block_pos, mask_emb, gain, gain_f32, eps, dst);
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
