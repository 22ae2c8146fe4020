// Matrix-core GEMM for the context prefill (Eq 2 over a whole prompt and the
// per-layer context K/V of Eq 3): at hundreds of rows and more these
// projections are dense contractions, far past the HBM/MFMA ridge point.
//
// Tiles: a workgroup of GWM x GWN wavefronts owns a BM x BN output tile and
// walks K in steps of 64. Each step's A and B tiles (rows x 64 bf16) go through
// registers into one of two LDS buffers (rows padded to 80 elements: no bank
// conflicts for the 16-byte fragment reads and tile writes, where a pad of 8
// measured conflicts on 37% of the LDS cycles) while the other buffer feeds the
// matrix cores; one barrier per step. The global loads run one step ahead
// (normalised A) or two (tap A, two register sets). Wavefront (wm, wn) computes its
// (BM/GWM) x (BN/GWN) block of the tile as 16 x 16 products of
// v_mfma_f32_16x16x32_bf16, lane l holding
//   A[l % 16][8 (l / 16) + e],  B[8 (l / 16) + e][l % 16]   (e < 8)
//   D[4 (l / 16) + e][l % 16]                               (e < 4),
// where B[k][n] is weight row n, so both operands are read as 16-byte rows.
//
// A operands: bf16 segments (the concatenation of the tapped hidden states,
// one pointer per tap; or each layer's pre-normalised context rows, one set per
// grid.z) or fp32 rows scaled by a per-row RMS factor and a per-column gain and
// rounded to bf16 while they are staged. Epilogues: fp32 store, or the K/V
// cache scatter of the context append.
#include "common.hpp"
#include "gemm.hpp"

namespace dfl {

// Tile shape (compile-time tunables): a BM x BN output tile per workgroup of
// GWM x GWN wavefronts, each owning a (BM/GWM) x (BN/GWN) block of 16 x 16
// products; K steps of 64.
#ifndef DFL_GEMM_BM
#define DFL_GEMM_BM 256
#endif
#ifndef DFL_GEMM_BN
#define DFL_GEMM_BN 256
#endif
#ifndef DFL_GEMM_WM
#define DFL_GEMM_WM 4
#endif
#ifndef DFL_GEMM_WN
#define DFL_GEMM_WN 2
#endif
// K steps whose global loads are in flight ahead of the step being multiplied (1 or 2),
// for tap A operands and for normalised fp32 A operands (whose staging takes twice the
// registers: two sets spill)
#ifndef DFL_GEMM_DEPTH_TAPS
#define DFL_GEMM_DEPTH_TAPS 2
#endif
#ifndef DFL_GEMM_DEPTH_NORM
#define DFL_GEMM_DEPTH_NORM 1
#endif
// LDS row padding (bf16 elements)
#ifndef DFL_GEMM_PAD
#define DFL_GEMM_PAD 16
#endif
// consecutive output tiles of one XCD walk GROUP_M row tiles for each column tile
#ifndef DFL_GEMM_GROUP_M
#define DFL_GEMM_GROUP_M 4
#endif

constexpr int kBM = DFL_GEMM_BM, kBN = DFL_GEMM_BN, kBK = 64;
constexpr int kGWM = DFL_GEMM_WM, kGWN = DFL_GEMM_WN, kThreads = 64 * kGWM * kGWN;
constexpr int kMT = kBM / kGWM / 16, kNT = kBN / kGWN / 16;  // 16 x 16 products per wavefront
constexpr int kLd = kBK + DFL_GEMM_PAD;  // padded LDS row (bf16 elements)
constexpr int kAC = kBM * 8 / kThreads, kBC = kBN * 8 / kThreads;  // 16-byte chunks per thread
static_assert(kAC * kThreads == kBM * 8 && kBC * kThreads == kBN * 8, "tile must split evenly");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// staged global data of one BM x 64 A tile: kAC chunks of 8 elements per thread
template <int AMODE>
struct AStage;
template <>
struct AStage<GEMM_A_TAPS> { u32x4 v[kAC]; };
template <>
struct AStage<GEMM_A_NORM> { float4 lo[kAC], hi[kAC]; float r[kAC]; };

// tap segment holding columns [k0, k0 + 64): a uniform choice (segments are
// multiples of 64), made with compares so the pointer array stays in registers;
// a launch over layers (grid.z) reads each layer's own rows, a_layer_stride apart
__device__ __forceinline__ const uint16_t* tap_base(const GemmParams& p, int k0) {
    const int j = k0 / p.seg_k;
    const uint16_t* a = p.a[0];
#pragma unroll
    for (int q = 1; q < kMaxTaps; ++q)
        if (j == q) a = p.a[q];
    return a + (int64_t)blockIdx.z * p.a_layer_stride + (k0 - j * p.seg_k);
}

template <int AMODE>
__device__ __forceinline__ void load_a(const GemmParams& p, int m0, int k0, AStage<AMODE>& st) {
    const int t = threadIdx.x;
    if (p.a_period > 0) k0 %= p.a_period;
    const uint16_t* abase = nullptr;
    if constexpr (AMODE == GEMM_A_TAPS) abase = tap_base(p, k0);
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
        const int c = t + kThreads * i;
        const int row = min(m0 + (c >> 3), p.M - 1);  // rows past M: any valid row, never stored
        if constexpr (AMODE == GEMM_A_TAPS) {
            st.v[i] = *reinterpret_cast<const u32x4*>(abase + (int64_t)row * p.a_ld + 8 * (c & 7));
        } else {
            const float* src = p.x + (int64_t)row * p.a_ld + k0 + 8 * (c & 7);
            st.lo[i] = *reinterpret_cast<const float4*>(src);
            st.hi[i] = *reinterpret_cast<const float4*>(src + 4);
            st.r[i] = p.rinv[row];
        }
    }
}

template <int AMODE>
__device__ __forceinline__ void store_a(const GemmParams& p, int k0, const void* gain, const AStage<AMODE>& st,
                                        uint16_t (*As)[kLd]) {
    const int t = threadIdx.x;
    if (p.a_period > 0) k0 %= p.a_period;
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
        const int c = t + kThreads * i;
        const int r = c >> 3, kc = 8 * (c & 7);
        u32x4 v;
        if constexpr (AMODE == GEMM_A_TAPS) {
            v = st.v[i];
        } else {
            float g[8];
            load_gain8(gain, p.gain_f32, k0 + kc, g);
            const float x[8] = {st.lo[i].x, st.lo[i].y, st.lo[i].z, st.lo[i].w,
                                st.hi[i].x, st.hi[i].y, st.hi[i].z, st.hi[i].w};
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = x[e] * st.r[i] * g[e];
            v.x = pack_bf16x2(y[0], y[1]);
            v.y = pack_bf16x2(y[2], y[3]);
            v.z = pack_bf16x2(y[4], y[5]);
            v.w = pack_bf16x2(y[6], y[7]);
        }
        *reinterpret_cast<u32x4*>(&As[r][kc]) = v;
    }
}

__device__ __forceinline__ void load_b(const GemmParams& p, const uint16_t* B, int n0, int k0, u32x4 (&st)[kBC]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kBC; ++i) {
        const int c = t + kThreads * i;
        const int64_t row = p.b_row0 + min(n0 + (c >> 3), p.N - 1);
        st[i] = *reinterpret_cast<const u32x4*>(B + row * p.K + k0 + 8 * (c & 7));
    }
}

__device__ __forceinline__ void store_b(const u32x4 (&st)[kBC], uint16_t (*Bs)[kLd]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kBC; ++i) {
        const int c = t + kThreads * i;
        *reinterpret_cast<u32x4*>(&Bs[c >> 3][8 * (c & 7)]) = st[i];
    }
}

// Output tile of a workgroup. Workgroups are dispatched round-robin over the 8
// XCDs; tile ids are renumbered so each XCD takes a contiguous range, and
// within it consecutive tiles walk GROUP_M row tiles per column tile: the
// workgroups resident on one XCD share their B rows and a few A row blocks in
// that XCD's L2.
__device__ __forceinline__ void tile_of(int wg, int mt, int nt, int& tm, int& tn) {
    const int total = mt * nt;
    const int full = total / 8 * 8;  // renumbered part (a permutation of [0, full)); the tail keeps its ids
    const int id = wg < full ? (wg % 8) * (full / 8) + wg / 8 : wg;
    const int group = DFL_GEMM_GROUP_M * nt;
    const int g = id / group, first_m = g * DFL_GEMM_GROUP_M;
    const int gm = min(mt - first_m, DFL_GEMM_GROUP_M);
    const int r = id - g * group;
    tm = first_m + r % gm;
    tn = r / gm;
}

template <int AMODE, int EPI>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmParams p) {
    __shared__ __align__(16) uint16_t As[2][kBM][kLd];
    __shared__ __align__(16) uint16_t Bs[2][kBN][kLd];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / kGWN, wn = wave % kGWN;
    const int col = lane & 15, grp = lane >> 4;
    const int mtiles = (p.M + kBM - 1) / kBM, ntiles = (p.N + kBN - 1) / kBN;
    int tm, tn;
    tile_of(blockIdx.x, mtiles, ntiles, tm, tn);
    const int n0 = tn * kBN, m0 = tm * kBM, layer = blockIdx.z;
    const int KT = p.K / kBK;
    // per-layer pointers, chosen with compares (kept in registers)
    const uint16_t* Bw = p.b[0];
    const void* gain = p.gain[0];
#pragma unroll
    for (int q = 1; q < kMaxLayers; ++q)
        if (layer == q) {
            Bw = p.b[q];
            gain = p.gain[q];
        }

    f32x4 acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one K step: the products of LDS buffer `cur`, with the global loads of a
    // later step in flight in register set `rs`
    auto mma_step = [&](const int cur) {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            u32x4 af[kMT], bfr[kNT];
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(&As[cur][wm * (kBM / kGWM) + i * 16 + col][ks * 32 + 8 * grp]);
#pragma unroll
            for (int j = 0; j < kNT; ++j)
                bfr[j] = *reinterpret_cast<const u32x4*>(&Bs[cur][wn * (kBN / kGWN) + j * 16 + col][ks * 32 + 8 * grp]);
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
        }
    };

    constexpr int kDepth = AMODE == GEMM_A_TAPS ? DFL_GEMM_DEPTH_TAPS : DFL_GEMM_DEPTH_NORM;
    if constexpr (kDepth == 1) {
        AStage<AMODE> sa;
        u32x4 sb[kBC];
        load_a<AMODE>(p, m0, 0, sa);
        load_b(p, Bw, n0, 0, sb);
        store_a<AMODE>(p, 0, gain, sa, As[0]);
        store_b(sb, Bs[0]);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            // the next step's tiles (the last step reloads its own, into the idle buffer)
            const int kn = min(kt + 1, KT - 1) * kBK;
            load_a<AMODE>(p, m0, kn, sa);
            load_b(p, Bw, n0, kn, sb);
            // keep the loads ahead of the products (left alone, the scheduler sinks them
            // below most of the step's products and the step then waits for them)
            __builtin_amdgcn_sched_barrier(0);
            mma_step(cur);
            store_a<AMODE>(p, kn, gain, sa, As[cur ^ 1]);
            store_b(sb, Bs[cur ^ 1]);
            __syncthreads();
        }
    } else {
        // two register sets: step t's tiles live in set t % 2 from their load (two
        // steps ahead) until they are written to LDS buffer t % 2 one step ahead
        AStage<AMODE> sa0, sa1;
        u32x4 sb0[kBC], sb1[kBC];
        const int k1 = min(1, KT - 1) * kBK;
        load_a<AMODE>(p, m0, 0, sa0);
        load_b(p, Bw, n0, 0, sb0);
        load_a<AMODE>(p, m0, k1, sa1);
        load_b(p, Bw, n0, k1, sb1);
        store_a<AMODE>(p, 0, gain, sa0, As[0]);
        store_b(sb0, Bs[0]);
        __syncthreads();
        for (int kt = 0; kt < KT; kt += 2) {
            {   // even step kt: LDS 0; set 0 fetches step kt + 2; set 1 (step kt + 1) goes to LDS 1
                const int k2 = min(kt + 2, KT - 1) * kBK, k1n = min(kt + 1, KT - 1) * kBK;
                load_a<AMODE>(p, m0, k2, sa0);
                load_b(p, Bw, n0, k2, sb0);
                mma_step(0);
                store_a<AMODE>(p, k1n, gain, sa1, As[1]);
                store_b(sb1, Bs[1]);
                __syncthreads();
            }
            if (kt + 1 < KT) {  // odd step kt + 1: LDS 1; set 1 fetches step kt + 3; set 0 goes to LDS 0
                const int k3 = min(kt + 3, KT - 1) * kBK, k2n = min(kt + 2, KT - 1) * kBK;
                load_a<AMODE>(p, m0, k3, sa1);
                load_b(p, Bw, n0, k3, sb1);
                mma_step(1);
                store_a<AMODE>(p, k2n, gain, sa0, As[0]);
                store_b(sb0, Bs[0]);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: lane holds rows 4*grp + e of each 16 x 16 product, column col
    const int kvw = p.hkv * p.hd;
    // sequence b of the lane's current row, its rows [seq_lo, seq_hi), appended-row count
    // and cache length: rows grow along (i, e), so b only advances and these reload only
    // when a row passes seq_hi
    int b = 0, seq_lo = 0, seq_hi = -1, cnt = 0, len_b = 0;  // rows are >= 0: the first row loads
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = m0 + wm * (kBM / kGWM) + i * 16 + 4 * grp + e;
            if (row >= p.M) continue;
            if constexpr (EPI == GEMM_EPI_F32) {
                float* dst = p.c + (int64_t)row * p.c_ld;
#pragma unroll
                for (int j = 0; j < kNT; ++j) {
                    const int n = n0 + wn * (kBN / kGWN) + j * 16 + col;
                    if (n < p.N) dst[n] = acc[i][j][e];
                }
            } else {
                if (row >= seq_hi) {
                    while (b + 1 < p.B && p.row_offsets[b + 1] <= row) ++b;
                    seq_lo = p.row_offsets[b];
                    seq_hi = p.row_offsets[b + 1];
                    const int rows_b = seq_hi - seq_lo;
                    cnt = p.counts ? min(p.counts[b], rows_b) : rows_b;
                    len_b = p.len[b];
                }
                const int ri = row - seq_lo;
                const int pos = len_b + ri;
                if (ri < 0 || ri >= cnt || pos >= p.cap) continue;
#pragma unroll
                for (int j = 0; j < kNT; ++j) {
                    const int n = n0 + wn * (kBN / kGWN) + j * 16 + col;
                    if (n >= p.N) continue;
                    const int which = n / kvw;
                    const int head = (n - which * kvw) / p.hd;
                    const int dim = n - which * kvw - head * p.hd;
                    const int64_t hb = (int64_t)layer * p.layer_stride + ((int64_t)b * p.hkv + head) * p.cap * p.hd;
                    uint16_t* base = static_cast<uint16_t*>(which ? p.vcache : p.kcache);
                    const int64_t off = hb + (which ? v_cache_off(pos, dim, p.hd, p.cap, false) : (int64_t)pos * p.hd + dim);
                    base[off] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
                }
            }
        }
    }
}

// one wavefront per row
__global__ __launch_bounds__(kBlock) void row_rinv_kernel(const float* x, int64_t ld, int rows, int K, float eps,
                                                          float* rinv) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float* src = x + (int64_t)row * ld;
    float s = 0.f;
#pragma unroll 4
    for (int k = lane * 4; k < K; k += 256) {
        const float4 a = *reinterpret_cast<const float4*>(src + k);
        s += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
    s = wave_sum(s);
    if (lane == 0) rinv[row] = 1.0f / sqrtf(s / (float)K + eps);
}

template <int AMODE, int EPI>
static hipError_t launch_t(const GemmParams& p, int layers, hipStream_t s) {
    const int64_t tiles = (int64_t)((p.N + kBN - 1) / kBN) * ((p.M + kBM - 1) / kBM);
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)tiles, 1, (unsigned)layers);
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL((gemm_kernel<AMODE, EPI>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm(int amode, int epi, const GemmParams& p, int layers, hipStream_t s) {
    if (p.M <= 0 || p.N <= 0 || p.K <= 0 || (p.K % kBK) || layers < 1 || layers > kMaxLayers)
        return hipErrorInvalidValue;
    const int a_cols = p.a_period > 0 ? p.a_period : p.K;  // A's own columns
    if (p.a_period < 0 || (p.a_period > 0 && (p.a_period % kBK || p.K % p.a_period))) return hipErrorInvalidValue;
    if (amode == GEMM_A_TAPS && (p.seg_k <= 0 || (p.seg_k % kBK) || a_cols > kMaxTaps * p.seg_k))
        return hipErrorInvalidValue;
    if (amode == GEMM_A_TAPS && epi == GEMM_EPI_F32) return launch_t<GEMM_A_TAPS, GEMM_EPI_F32>(p, layers, s);
    if (amode == GEMM_A_TAPS && epi == GEMM_EPI_KV) return launch_t<GEMM_A_TAPS, GEMM_EPI_KV>(p, layers, s);
    if (amode == GEMM_A_NORM && epi == GEMM_EPI_KV) return launch_t<GEMM_A_NORM, GEMM_EPI_KV>(p, layers, s);
    return hipErrorInvalidValue;
}

hipError_t launch_row_rinv(const float* x, int64_t ld, int rows, int K, float eps, float* rinv, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (K % 4) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(row_rinv_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(kBlock), 0, s, x, ld, rows, K, eps,
                       rinv);
    return hipGetLastError();
}

}  // namespace dfl
