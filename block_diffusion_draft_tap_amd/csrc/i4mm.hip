// int4-g64 weights on matrix cores for up to 16 activation rows: the per-round
// projections and the LM head of the int4 drafters (the Wide4 and DFlash2
// workloads: 4 and 7 block rows), where the dot-product GEMVs are bound by the
// code unpack and their activation reads, not by HBM.
//
// Products run on v_mfma_f32_16x16x32_bf16 with the activation rows as the A
// operand (rows past M are zero) and 16 weight rows as the B operand. Over a
// weight group (64 columns, one bf16 scale s and bias b):
//   sum_k (s q_k + b) x_k = s sum_k (128 + q_k) x_k + (b - 128 s) sum_k x_k
// The codes become bf16 (128 + q) with two integer operations per pair (the
// exponent of 128 or'ed above the 4-bit code), so the B operand costs no float
// arithmetic; each group's MFMA partial is then scaled and the bias term added
// with its activation sum (summed once per workgroup while the rows are staged).
//
// With M <= 4 or 8 activation rows, an MFMA's 16 rows hold 4 or 2 slots of the
// rows: slot h's rows see only the k columns taken from one quantisation group
// (zero A elsewhere; slot h takes groups 16 h / kG + t over the sets t), so one
// MFMA output holds the partials of kG groups and each lane scales one group
// per set, not every group (the
// scaling was most of the kernel's VALU work at few rows). Lane (c, g) of a
// wavefront (c = lane % 16, g = lane / 16) supplies k-chunk g of every MFMA: 8
// consecutive columns of one group, so the codes of weight row c there are one
// 32-bit word, and the lane's words of a group set are consecutive. The slots'
// sums meet in one lane by cross-lane adds at the end. A workgroup (four
// wavefronts, 64 weight rows) takes a K range of up to 8 blocks of 128 columns:
// it reads its rows' codes as contiguous 512-byte runs into LDS (loaded fragment
// by fragment, the codes would come as 16 rows x 32 bytes per instruction, a
// pattern DRAM serves at about half the rate), stages that range of the
// activation rows once in LDS, already in the codes' pair order, with each row's
// per-group sum, and loads its output columns' scales and biases; then the
// products run from LDS.
//
// Results are fp32 partial sums per K range; an ordered reduce applies the
// epilogue (the skinny reduce kernels, or the split argmax below).
#include <cstdio>

#include "common.hpp"
#include "i4mm.hpp"
#include "trace.hpp"

namespace dfl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// (x & mask) | one in one instruction (the compiler splits it into an and and an or)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t one) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask), "v"(one));
    return r;
}

// a word of 8 codes (low nibble first) as bf16 pairs (128 + q_i, 128 + q_(i+4)), i = 0..3;
// mask = 0x000F000F and one = 0x43004300 (bf16 128.0 in both halves), held in registers
__device__ __forceinline__ u32x4 codes_bf16(uint32_t c, uint32_t mask, uint32_t one) {
    u32x4 r;
    r[0] = and_or(c, mask, one);
    r[1] = and_or(c >> 4, mask, one);
    r[2] = and_or(c >> 8, mask, one);
    r[3] = and_or(c >> 12, mask, one);
    return r;
}

// 8 consecutive bf16 activations (x0, x1), (x2, x3), (x4, x5), (x6, x7) in the pair
// order of the codes: (x0, x4), (x1, x5), (x2, x6), (x3, x7)
__device__ __forceinline__ u32x4 pair_order(const u32x4& x) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(x[2], x[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(x[2], x[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(x[3], x[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(x[3], x[1], 0x07060302u);
    return r;
}

constexpr int kAld = kI4MaxBlocks * kI4Block + 8;  // LDS activation row (bf16), padded by 16 bytes
constexpr int kMaxGroups = kI4MaxBlocks * kI4Block / 64;
constexpr int kCodeLd = kI4MaxBlocks * kI4Block / 8 + 4;  // LDS code row (32-bit words), padded by 16 bytes
constexpr int kCodeChunks = 64 * kI4MaxBlocks * kI4Block / 32 / kBlock;  // 16-byte code chunks per thread

// MT: activation rows staged (4, 8 or 16; rows past M are zero, MFMA rows past MT too).
// FULL: every K range is 8 blocks and K/64 a multiple of 16, so a lane's 16 scales (and
// biases) of its range are two 16-byte loads.
template <int MT, bool FULL>
__global__ __launch_bounds__(kBlock) void i4mm_kernel(const I4Params p) {
    // An MFMA's 16 rows are kG = 16 / MT slots of MT activation rows; slot h takes 32 / kG
    // of its 32 k columns from quantisation group kSets h + t (group set t), so one MFMA
    // output holds kG groups' partials and every lane scales one group per set.
    constexpr int kG = 16 / MT;                // 4, 2, 1
    constexpr int kCPG = 4 / kG;               // 8-column k-chunks per slot
    constexpr int kSteps = 8 / kCPG;           // k-steps per group
    constexpr int kSets = kMaxGroups / kG;     // group sets of a 1024-column range
    static_assert(kG * MT == 16 && kSets * kG == kMaxGroups, "slot layout");
    __shared__ __align__(16) uint16_t as[(MT + 1) * kAld];      // rows in the codes' pair order; row MT zero
    __shared__ __align__(16) uint32_t cs[64 * kCodeLd];         // the workgroup's 64 weight rows' codes
    __shared__ __align__(16) float xs[kMaxGroups][kI4Rows];     // sum of each row's group (rows past MT: 0)
    const uint64_t t_start = trace_start(p.stamps);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    // the K ranges of one group of 64 weight rows are consecutive workgroups, so they run
    // together and share the rows' scale and bias lines in L2
    const int s = blockIdx.x % p.nsplit;
    const int layer = blockIdx.y;
    const int kb = s * p.kslice;
    const int nblk = min(p.kslice, p.K - kb) / kI4Block;  // 1 .. kI4MaxBlocks
    const int kw = nblk * kI4Block;
    const int tile = (blockIdx.x / p.nsplit) * 4 + wave;   // 16 weight rows of this wavefront
    const int n = min(tile * 16 + col, p.N - 1);           // this lane's weight row and output column

    // the range's activation rows and a zero row: issued first (loads return in order)
    constexpr int kRowChunks = kI4MaxBlocks * kI4Block / 8;
    constexpr int kChunks = ((MT + 1) * kRowChunks + kBlock - 1) / kBlock;  // 16-byte chunks per thread
    const int cpr = FULL ? kRowChunks : kw / 8;                             // chunks per row
    // the range lies in one column segment (seg_k a multiple of kslice)
    const uint16_t* abase = p.seg_k > 0 ? p.a_seg[kb / p.seg_k] + kb % p.seg_k
                                        : p.a + layer * p.a_layer_stride + kb;
    u32x4 av[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int idx = min(tid + i * kBlock, (MT + 1) * cpr - 1);
        const int m = idx / cpr, c = idx - m * cpr;
        av[i] = *reinterpret_cast<const u32x4*>(abase + (int64_t)min(m, p.M - 1) * p.a_ld + 8 * c);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the weight loads

    // the workgroup's codes: its 64 weight rows' K range, read as contiguous runs of each row
    // (32 threads cover a row's 512 bytes) and staged in LDS; rows past N repeat row N - 1
    const int K8 = p.K / 8, K64 = p.K / 64;
    const int row0 = (blockIdx.x / p.nsplit) * 64;
    const int ccr = FULL ? kI4MaxBlocks * kI4Block / 32 : kw / 32;  // 16-byte code chunks per row
    u32x4 cv[kCodeChunks];
#pragma unroll
    for (int i = 0; i < kCodeChunks; ++i) {
        const int idx = min(tid + i * kBlock, 64 * ccr - 1);
        const int r = idx / ccr, c = idx - r * ccr;
        const int64_t grow = p.w_row0 + min(row0 + r, p.N - 1);
        cv[i] = stream_load(reinterpret_cast<const u32x4*>(p.codes[layer] + grow * K8 + kb / 8 + 4 * c));
    }
    // this lane's output column's scales and biases, for the groups of its output slot: the
    // kSets consecutive groups kSets slot + t (one or two 16-byte loads or one 8-byte load;
    // for a shorter range, loads clamped to it: its products and sums are zero past it)
    const int slot = grp / kCPG;
    const int ng = kw / 64;
    const int64_t wrow = p.w_row0 + n;
    const uint16_t* srow = p.scales[layer] + wrow * K64 + kb / 64;
    const uint16_t* brow = p.biases[layer] + wrow * K64 + kb / 64;
    const int g0 = kSets * slot;
    uint32_t sc[kSets / 2], bi[kSets / 2];  // bf16 pairs: groups g0 + 2i (low), g0 + 2i + 1 (high)
    if constexpr (FULL) {
        if constexpr (kSets == 4) {
            const uint2 sv = *reinterpret_cast<const uint2*>(srow + g0);
            const uint2 bv = *reinterpret_cast<const uint2*>(brow + g0);
            sc[0] = sv.x; sc[1] = sv.y;
            bi[0] = bv.x; bi[1] = bv.y;
        } else {
#pragma unroll
            for (int h = 0; h < kSets / 8; ++h) {
                const u32x4 sv = *reinterpret_cast<const u32x4*>(srow + g0 + 8 * h);
                const u32x4 bv = *reinterpret_cast<const u32x4*>(brow + g0 + 8 * h);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sc[4 * h + q] = sv[q];
                    bi[4 * h + q] = bv[q];
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kSets / 2; ++i) {
            const int ga = min(g0 + 2 * i, ng - 1), gb = min(g0 + 2 * i + 1, ng - 1);
            sc[i] = (uint32_t)srow[ga] | ((uint32_t)srow[gb] << 16);
            bi[i] = (uint32_t)brow[ga] | ((uint32_t)brow[gb] << 16);
        }
    }

    // stage the rows in pair order (unconditional stores: threads past the range repeat the
    // last chunk with its value, so no load is moved into a branch and waited for there)
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int idx = min(tid + i * kBlock, (MT + 1) * cpr - 1);
        const int m = idx / cpr, c = idx - m * cpr;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&as[m * kAld + 8 * c]) = (m < p.M && m < MT) ? pair_order(av[i]) : z;
    }
#pragma unroll
    for (int i = 0; i < kCodeChunks; ++i) {
        const int idx = min(tid + i * kBlock, 64 * ccr - 1);
        const int r = idx / ccr, c = idx - r * ccr;
        *reinterpret_cast<u32x4*>(&cs[r * kCodeLd + 4 * c]) = cv[i];
    }
    __syncthreads();
    // each row's group sums (any order of the group's 64 values: a sum)
    {
        const int m = tid / kMaxGroups, g = tid - m * kMaxGroups;
        float t = 0.f;
        if (m < MT && g < ng) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(&as[m * kAld + 64 * g + 8 * q]);
#pragma unroll
                for (int e = 0; e < 4; ++e) t = dot2_bf16(v[e], 0x3F803F80u, t);  // + both halves
            }
        }
        if (m < kI4Rows) xs[g][m] = t;  // 256 threads: every (group, row) slot written
    }
    __syncthreads();

    // Lane (col, grp) supplies k-chunk grp of every MFMA: chunk c = grp % kCPG of slot
    // `slot`, i.e. the columns 8 (c kSteps + j) .. + 8 of group g0 + t at k-step j of set t.
    // Its A fragment is activation row col % MT when col lies in that slot's rows, else the
    // zero row; its B fragment is weight row col's codes there, kSteps consecutive words.
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int chunk = grp % kCPG;
    const bool areal = col / MT == slot;
    const uint16_t* arow = &as[(areal ? col % MT : MT) * kAld + 64 * g0 + 8 * kSteps * chunk];
    const uint16_t* azero = &as[MT * kAld];
    const uint32_t* crow = &cs[(wave * 16 + col) * kCodeLd + 8 * g0 + kSteps * chunk];
    const uint32_t mk = p.nib_mask, one = p.bf16_128;
    f32x4 acc = zero;
#pragma unroll
    for (int t = 0; t < kSets; ++t) {
        if (FULL || t < ng) {
            // past the range (slots whose group t lies beyond it) the A fragments are the zero row
            const uint16_t* ap = (FULL || g0 + t < ng) ? arow + 64 * t : azero;
            uint32_t cw[kSteps];
            if constexpr (kSteps == 8) {
                const u32x4 c0 = *reinterpret_cast<const u32x4*>(crow + 8 * t);
                const u32x4 c1 = *reinterpret_cast<const u32x4*>(crow + 8 * t + 4);
#pragma unroll
                for (int q = 0; q < 4; ++q) { cw[q] = c0[q]; cw[4 + q] = c1[q]; }
            } else if constexpr (kSteps == 4) {
                const u32x4 c0 = *reinterpret_cast<const u32x4*>(crow + 8 * t);
#pragma unroll
                for (int q = 0; q < 4; ++q) cw[q] = c0[q];
            } else {
                const uint2 c0 = *reinterpret_cast<const uint2*>(crow + 8 * t);
                cw[0] = c0.x;
                cw[1] = c0.y;
            }
            // the slots' group partials: sum_k (128 + q) x over this lane's output group
            f32x4 pg = zero;
#pragma unroll
            for (int j = 0; j < kSteps; ++j)
                pg = mma(*reinterpret_cast<const u32x4*>(ap + 8 * j), codes_bf16(cw[j], mk, one), pg);
            // rows (4 grp) % MT + e of group g0 + t (its activation sums: zero past the range)
            const f32x4 xg = *reinterpret_cast<const f32x4*>(&xs[g0 + t][(4 * grp) % MT]);
            const float sg = (t & 1) ? bf16_hi(sc[t / 2]) : bf16_lo(sc[t / 2]);
            const float bg = ((t & 1) ? bf16_hi(bi[t / 2]) : bf16_lo(bi[t / 2])) - 128.0f * sg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] = fmaf(sg, pg[e], acc[e]);
                acc[e] = fmaf(bg, xg[e], acc[e]);
            }
        }
    }
    // the slots of one row block: lanes 16 apart (kG = 4) and 32 apart (kG >= 2)
    if constexpr (kG >= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], 32, kWave);
    }
    if constexpr (kG == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], 16, kWave);
    }

    // slot 0's lanes hold output column tile * 16 + col of activation rows 4 grp + e
    const int nout = tile * 16 + col;
    if (nout < p.N && slot == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * grp + e;
            if (m < p.M) p.part[(((int64_t)layer * p.nsplit + s) * p.M + m) * p.N + nout] = acc[e];
        }
    }
    trace_end(p.stamps, t_start);
}

__global__ __launch_bounds__(kBlock) void i4_split_argmax_kernel(const float* part, int nsplit, int M, int N,
                                                                 float* pv, int32_t* pi, int nblocks) {
    __shared__ float sv[kBlock / 64];
    __shared__ int si[kBlock / 64];
    const int c = blockIdx.x, m = blockIdx.y;
    const int n0 = c * kI4ArgChunk, n1 = min(N, n0 + kI4ArgChunk);
    float v = -INFINITY;
    int idx = 0x7fffffff;
    for (int n = n0 + threadIdx.x; n < n1; n += kBlock) {
        float t = 0.f;
        for (int s = 0; s < nsplit; ++s) t += part[((int64_t)s * M + m) * N + n];
        argmax_pick(v, idx, t, n);
    }
    wave_argmax(v, idx);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { sv[wave] = v; si[wave] = idx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kBlock / 64; ++w) argmax_pick(v, idx, sv[w], si[w]);
        pv[(int64_t)m * nblocks + c] = v;
        pi[(int64_t)m * nblocks + c] = idx;
    }
}

}  // namespace

bool i4mm_ok(int K, int M) { return K > 0 && K % kI4Block == 0 && M >= 1 && M <= kI4Rows; }

void i4mm_split(int K, int* nsplit, int* kslice) {
    const int maxk = kI4MaxBlocks * kI4Block;
    int ns = (K + maxk - 1) / maxk;
    int ks = ((K + ns - 1) / ns + kI4Block - 1) / kI4Block * kI4Block;
    ns = (K + ks - 1) / ks;
    *nsplit = ns;
    *kslice = ks;
}

hipError_t launch_i4mm(I4Params p, hipStream_t s) {
    if (!i4mm_ok(p.K, p.M) || p.N <= 0 || !p.part || p.layers < 1 || p.layers > kI4MaxLayers || p.w_row0 < 0)
        return hipErrorInvalidValue;
    for (int z = 0; z < p.layers; ++z)
        if (!p.codes[z] || !p.scales[z] || !p.biases[z]) return hipErrorInvalidValue;
    if (p.kslice <= 0 || p.kslice % kI4Block || p.kslice > kI4MaxBlocks * kI4Block || p.a_ld % 8)
        return hipErrorInvalidValue;
    if (p.seg_k > 0) {
        if (p.seg_k % p.kslice || p.a_ld < p.seg_k || (p.K + p.seg_k - 1) / p.seg_k > kI4MaxSegs) return hipErrorInvalidValue;
        for (int j = 0; j < (p.K + p.seg_k - 1) / p.seg_k; ++j)
            if (!p.a_seg[j]) return hipErrorInvalidValue;
    } else if (!p.a || p.a_ld < p.K) {
        return hipErrorInvalidValue;
    }
    if (p.nsplit != (p.K + p.kslice - 1) / p.kslice) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((p.N + 63) / 64) * p.nsplit), (unsigned)p.layers);
    p.nib_mask = 0x000F000Fu;
    p.bf16_128 = 0x43004300u;
    // instrumentation: algorithmic bytes = int4 weights (codes, scales, biases) + activations + partials
    const double bytes = p.layers * ((double)p.N * p.K * (0.5 + 4.0 / 64) + (double)p.M * p.K * 2.0 +
                                     (double)p.nsplit * p.M * p.N * 4.0);
    const int mt = p.M <= 4 ? 4 : (p.M <= 8 ? 8 : 16);
    char name[32];
    snprintf(name, sizeof name, "i4mm_kernel<%d>", mt);
    p.stamps = trace_launch(TRACE_PROJECTIONS, name, (int64_t)grid.x * grid.y, bytes, 0.0);
    (void)hipGetLastError();  // report only this launch's status
    const bool full = p.kslice == kI4MaxBlocks * kI4Block && p.K % p.kslice == 0;
#define DFL_I4_LAUNCH(MT)                                                                \
    if (full)                                                                            \
        hipLaunchKernelGGL((i4mm_kernel<MT, true>), grid, dim3(kBlock), 0, s, p);        \
    else                                                                                 \
        hipLaunchKernelGGL((i4mm_kernel<MT, false>), grid, dim3(kBlock), 0, s, p);
    if (mt == 4) {
        DFL_I4_LAUNCH(4)
    } else if (mt == 8) {
        DFL_I4_LAUNCH(8)
    } else {
        DFL_I4_LAUNCH(16)
    }
#undef DFL_I4_LAUNCH
    return hipGetLastError();
}

int i4_argmax_blocks(int N) { return (N + kI4ArgChunk - 1) / kI4ArgChunk; }

hipError_t launch_i4_split_argmax(const float* part, int nsplit, int M, int N, float* pv, int32_t* pi, int nblocks,
                                  hipStream_t s) {
    if (M <= 0 || N <= 0 || nsplit < 1 || nblocks != i4_argmax_blocks(N)) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(i4_split_argmax_kernel, dim3((unsigned)nblocks, (unsigned)M), dim3(kBlock), 0, s, part, nsplit, M,
                       N, pv, pi, nblocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// int4-g64 rows expanded into bf16 high and low parts (the prefill's matrix-core GEMM reads
// them as one [N, 2K] bf16 matrix against [A | A]); one thread per code word (8 values)
__global__ __launch_bounds__(256) void i4_expand_kernel(const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ biases, int K, int64_t row0,
                                                        int N, uint16_t* __restrict__ out) {
    const int K8 = K / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)N * K8) return;
    const int64_t n = t / K8;
    const int w = (int)(t - n * K8);
    const int64_t row = row0 + n;
    const uint32_t c = codes[row * K8 + w];
    const int g = w / 8;  // 64-column group: 8 words
    const float sc = bf16_lo((uint32_t)scales[row * (K / 64) + g]);
    const float bi = bf16_lo((uint32_t)biases[row * (K / 64) + g]);
    float hv[8], lv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = fmaf(sc, (float)((c >> (4 * e)) & 15u), bi);
        const uint32_t h = f32_to_bf16_bits(v);
        hv[e] = bf16_lo(h);
        lv[e] = v - hv[e];
    }
    u32x4 hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        hi[q] = pack_bf16x2(hv[2 * q], hv[2 * q + 1]);
        lo[q] = pack_bf16x2(lv[2 * q], lv[2 * q + 1]);
    }
    uint16_t* o = out + n * 2 * (int64_t)K + 8 * (int64_t)w;
    *reinterpret_cast<u32x4*>(o) = hi;
    *reinterpret_cast<u32x4*>(o + K) = lo;
}

hipError_t launch_i4_expand(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int K, int64_t row0,
                            int N, uint16_t* out, hipStream_t s) {
    if (!codes || !scales || !biases || !out || K <= 0 || (K % 64) || N <= 0) return hipErrorInvalidValue;
    const int64_t words = (int64_t)N * (K / 8);
    (void)hipGetLastError();
    hipLaunchKernelGGL(i4_expand_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, codes, scales, biases,
                       K, row0, N, out);
    return hipGetLastError();
}

}  // namespace dfl
