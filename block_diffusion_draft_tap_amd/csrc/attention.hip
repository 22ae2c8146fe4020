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
//   S^T = K Q^T  v_mfma_f32_16x16x32_bf16 with K rows as the A operand (one
//                16-byte chunk of 8 head dims per lane, straight from HBM) and
//                the 16-row Q tiles, held in registers, as the B operand;
//   softmax      online per query row; the 32 keys of a row sit in the four
//                lanes col, col+16, col+32, col+48 (8 each), so its max and
//                sum take two row swaps; the reference max moves lazily;
//   O^T += V^T P^T  P stays in the row's lanes as the B operand, split into
//                bf16 high and low parts (two products) so the probabilities
//                keep ~16 mantissa bits; V is cached in 32-key chunks of all
//                head dims ([cap/32][hd][32]), so the A operand (8 consecutive
//                keys of one dim) is one 16-byte load and a unit's values are
//                one contiguous 8 KB run (1 KB per load instruction).
// attn_rows_kernel (33..48 query rows, few units) gives each 16-row tile its own
// wavefront and forms S = Q K^T, passing P through LDS.
// Lane layout of the 16x16x32 product (lane l): A[l%16][8(l/16)+e],
// B[8(l/16)+e][l%16] for e < 8; D[4(l/16)+e][l%16] for e < 4.
//
// fp32 caches (the fp32 workload): attn_valu_kernel, LDS-staged 64-key tiles,
// one key per lane for the scores, one head-dim column per thread for P V.
#include <cstdio>

#include "attention.hpp"
#include "common.hpp"
#include "trace.hpp"


namespace dfl {

constexpr int kTile = 64;   // keys per tile, fp32 kernel
constexpr int kChunk = 32;  // keys per chunk, MFMA kernel
static_assert(kChunk == kAttnMaxGamma, "the block's keys form one chunk");
constexpr int kMaxParts = 256;
constexpr int kMaxSplit = 64;  // workgroups per (sequence, kv head), MFMA kernel
constexpr int kMaxRows = 48;   // query rows per kv head, MFMA kernel

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
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
// MFMA kernel (bf16 caches; Q, K_b and V_b arrive as bf16)
//
// Scores are formed transposed, S^T = K Q^T (K rows the A operand, Q rows the B
// operand), and the output as O^T = V^T P^T: the probabilities of a query row then
// stay in the lanes of that row, from the score accumulator straight into the B
// operand of the value product, with no trip through LDS. Key tile nt of a unit
// loads key 8*(c/4) + 4*nt + c%4 into A row c, so lane (col, grp) of the score tiles
// holds keys 8*grp .. 8*grp + 7 of query row col -- the keys that lane's B operand
// carries in the value product, whose A operand (V^T, 8 consecutive keys of one
// head dim per lane) is one 16-byte load of the chunked V cache.

// max and sum over the four lanes col, col + 16, col + 32, col + 48: gfx950's row
// swaps exchange rows 0/1 and 2/3, then the two halves; every lane ends with the
// same value (the two operands of each step are the same pair in either order)
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32_e32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float rows4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One unit's online softmax for one 16-row query tile held transposed: sc[nt][e] is the
// score of key 8*grp + 4*nt + e for query row col (raw Q.K). Keys outside [lo, nvalid)
// take no weight when `ragged`. m is the row's reference max (log2 units) and l its sum
// of exp2(score - m). The reference moves only when some row of the tile passes it by
// more than kLazy: until then the probabilities may reach 2^kLazy (fp32 and the two-part
// bf16 P hold that) and o and l need no rescaling, which on most units saves the pass
// over o (held in accumulation registers, so each rescale is a read, a multiply and a
// write per element). When it moves, every row of the tile takes its own max (rows
// below their reference keep it: exp2(0) = 1 exactly) and o is rescaled when `rescale`
// (o is still zero on a wavefront's first unit). Returns P = hi + lo as two bf16 B
// operands (keys 8*grp .. +7 in order), so the product keeps ~16 mantissa bits of P.
constexpr float kLazy = 8.0f;

template <int DT>
__device__ __forceinline__ void softmax_tile(const f32x4 (&sc)[2], const bool ragged, const int grp, const int lo,
                                             const int nvalid, const float sl2, const bool rescale, float& m,
                                             float& l, f32x4 (&o)[DT], u32x4& ph, u32x4& pl) {
    float sv[8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * nt + e] = sc[nt][e];
    if (ragged) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = 8 * grp + j;
            if (key < lo || key >= nvalid) sv[j] = -INFINITY;
        }
    }
    // finite: a unit holds a valid key
    const float mt =
        sl2 * rows4_max(vmax(vmax3(sv[0], sv[1], sv[2]), vmax3(vmax3(sv[3], sv[4], sv[5]), sv[6], sv[7])));
    if (__builtin_amdgcn_ballot_w64(mt > m + kLazy)) {
        const float mn = fmaxf(m, mt);
        const float al = __builtin_amdgcn_exp2f(m - mn);
        l *= al;
        m = mn;
        if (rescale) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= al;
        }
    }
    float pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pv[j] = __builtin_amdgcn_exp2f(fmaf(sv[j], sl2, -m));
    l += rows4_sum(((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7])));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t h = pack_bf16x2(pv[2 * q], pv[2 * q + 1]);
        ph[q] = h;
        pl[q] = pack_bf16x2(pv[2 * q] - bf16_lo(h), pv[2 * q + 1] - bf16_hi(h));
    }
}

// keys past nvalid are zeroed in a V operand (lane keys 8*grp .. +7; P is zero there, the
// cache may hold anything)
template <int DT>
__device__ __forceinline__ void mask_v(u32x4 (&vb)[DT], const int nvalid, const int grp) {
    const int nk = nvalid - 8 * grp;  // valid keys among this lane's 8
    u32x4 mk;
#pragma unroll
    for (int q = 0; q < 4; ++q) mk[q] = (2 * q + 1 < nk) ? 0xFFFFFFFFu : ((2 * q < nk) ? 0x0000FFFFu : 0u);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vb[dt] &= mk;
}

// Workgroups start in block order, and a sequence's work grows with its length, so the
// sequences are taken longest first (ties by index): the last workgroups to start are the
// shortest, which evens out when the compute units run dry. Sequence of rank `pos` in
// that order; the rank is formed from the lengths on the device (every workgroup alike).
#ifndef DFL_ATTN_LPT
#define DFL_ATTN_LPT 1
#endif
constexpr int kLptMaxSeqs = 256;
__device__ __forceinline__ int lpt_sequence(const AttnParams& p, const int pos) {
    if (!DFL_ATTN_LPT || p.B <= 1 || p.B > kLptMaxSeqs) return pos;
    __shared__ int chosen;
    auto len = [&](int j) {
        const int L = min(max(p.len[j], 0), p.cap);
        return p.window > 0 ? min(L, p.window) : L;
    };
    for (int t = threadIdx.x; t < p.B; t += blockDim.x) {
        const int lt = len(t);
        int rank = 0;
        for (int j = 0; j < p.B; ++j) {
            const int lj = len(j);
            rank += (lj > lt) || (lj == lt && j < t);
        }
        if (rank == pos) chosen = t;
    }
    __syncthreads();
    return chosen;
}

// K/V cache loads (streamed: each byte read once a launch)
__device__ __forceinline__ u32x4 kv_load(const uint16_t* p) { return stream_load(reinterpret_cast<const u32x4*>(p)); }

template <int HD, int NRT>
__global__ __launch_bounds__(kBlock) void attn_mfma_kernel(const AttnParams p) {
    const uint64_t t_start = trace_start(p.stamps);
    constexpr int KS = HD / 32;  // k-steps of S^T = K Q^T
    constexpr int DT = HD / 16;  // head-dim tiles of O^T
    constexpr int OLD = HD + 4;  // padded o row (floats)
    __shared__ __align__(16) float ob[4][NRT * 16][OLD];  // o of the four wavefronts, row major
    __shared__ float wm[4][NRT * 16], wl[4][NRT * 16], wf[4][NRT * 16];
    __shared__ float rowm[NRT * 16], rowl[NRT * 16];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x % p.nsplit;
    const int bg = blockIdx.x / p.nsplit;
    const int g = bg % p.hkv;
    const int b = lpt_sequence(p, bg / p.hkv);
    const int qpg = p.hq / p.hkv;
    const int R = qpg * p.gamma;
    const int lenb = min(max(p.len[b], 0), p.cap);
    // work units: the 32-key chunks from the one holding the first attended key (key 0,
    // or the window's first), then the block's gamma keys; wavefronts take equal runs of
    // consecutive units
    const int kbeg = p.window > 0 ? max(0, lenb - p.window) : 0;
    const int cb = kbeg & ~(kChunk - 1);
    const int nch = (lenb - cb + kChunk - 1) / kChunk;
    const int nunits = nch + 1;
    const int upw = (nunits + 4 * p.nsplit - 1) / (4 * p.nsplit);
    const int u_begin = min(nunits, (s * 4 + wave) * upw);
    const int u_end = min(nunits, u_begin + upw);

    const int64_t qkv_ld = p.qkv_ld;
    const uint16_t* qrow0 = static_cast<const uint16_t*>(p.qkv) + (int64_t)b * p.gamma * qkv_ld;
    const int kcol = p.hq * HD + g * HD;
    const uint16_t* kc = static_cast<const uint16_t*>(p.kcache) + ((int64_t)b * p.hkv + g) * p.cap * HD;
    const uint16_t* vc = static_cast<const uint16_t*>(p.vcache) + ((int64_t)b * p.hkv + g) * HD * (int64_t)p.cap;
    const float sl2 = p.scale * 1.4426950408889634f;  // scores in log2 units
    const uint16_t* vblk = p.vblk + ((int64_t)b * p.hkv + g) * HD * kChunk;

    // K: A row col of key tile nt is key kq + 4*nt (dims ks*32 + 8*grp ..); V: keys
    // 8*grp .. +8 of dims dt*16 + col. Keys past nvalid come from in-bounds rows (cache
    // rows below cap, clamped block rows): their scores are masked and their values zeroed
    // before use. The next unit's K goes out as soon as this unit's scores are issued and
    // its V once the value products are, so they land during the softmax and products
    // instead of after them, with no second register set.
    const int kq = 8 * (col >> 2) + (col & 3);
    auto load_k = [&](const int u, u32x4 (&kb)[2][KS]) {
        const uint16_t *k0, *k1;
        if (u != nch) {
            k0 = kc + (int64_t)(cb + u * kChunk + kq) * HD + 8 * grp;
            k1 = k0 + 4 * HD;
        } else {
            k0 = qrow0 + (int64_t)min(kq, p.gamma - 1) * qkv_ld + kcol + 8 * grp;
            k1 = qrow0 + (int64_t)min(kq + 4, p.gamma - 1) * qkv_ld + kcol + 8 * grp;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kb[0][ks] = kv_load(k0 + ks * 32);
            kb[1][ks] = kv_load(k1 + ks * 32);
        }
    };
    auto load_v = [&](const int u, u32x4 (&vb)[DT]) {
        const uint16_t* vp;
        if (u != nch)
            vp = vc + ((int64_t)(cb / kChunk + u) * HD + col) * kChunk + 8 * grp;
        else
            vp = vblk + col * kChunk + 8 * grp;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vb[dt] = kv_load(vp + dt * 16 * kChunk);
    };
    u32x4 kA[2][KS], vA[DT];
    // the first unit's loads go out together with Q's
    if (u_begin < u_end) {
        load_k(u_begin, kA);
        load_v(u_begin, vA);
    }

    // Q tiles as B operands: query row rt*16 + col, dims ks*32 + 8*grp ..; rows past R
    // repeat row R-1 and are never stored
    u32x4 qa[NRT][KS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = min(rt * 16 + col, R - 1);
        const uint16_t* src = qrow0 + (int64_t)(r % p.gamma) * qkv_ld + (g * qpg + r / p.gamma) * HD + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[rt][ks] = *reinterpret_cast<const u32x4*>(src + ks * 32);
    }

    // o[rt][dt]: lane holds dims dt*16 + 4*grp + e of query row rt*16 + col; m, l of that row
    f32x4 o[NRT][DT];
    float m[NRT], l[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[rt] = -INFINITY;
        l[rt] = 0.f;
    }

    // one unit from register set (kb, vb); the set's K then V are reloaded with unit `next`
    // (if `reload`) as soon as the products that read them are issued
    auto unit = [&](const int u, u32x4 (&kb)[2][KS], u32x4 (&vb)[DT], const int next, const bool reload) {
        const int nvalid = (u == nch) ? p.gamma : min(kChunk, lenb - cb - u * kChunk);
        // keys of the first chunk before the window's first key take no weight (they are
        // held context rows: their values are finite and meet zero probabilities)
        const int lo = (u == 0 && u != nch) ? kbeg - cb : 0;

        f32x4 sacc[NRT][2];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                sacc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sacc[rt][nt] = mfma16(kb[nt][ks], qa[rt][ks], sacc[rt][nt]);
            }
        if (reload) load_k(next, kb);
        const bool ragged = lo > 0 || nvalid < kChunk;
        const bool rescale = (u != u_begin);  // o is still zero on a wavefront's first unit
        u32x4 ph[NRT], pl[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
            softmax_tile<DT>(sacc[rt], ragged, grp, lo, nvalid, sl2, rescale, m[rt], l[rt], o[rt], ph[rt], pl[rt]);
        if (nvalid < kChunk) mask_v<DT>(vb, nvalid, grp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) o[rt][dt] = mfma16(vb[dt], pl[rt], mfma16(vb[dt], ph[rt], o[rt][dt]));
        if (reload) load_v(next, vb);
    };
    for (int u = u_begin; u < u_end; ++u) unit(u, kA, vA, u + 1, u + 1 < u_end);

    // merge the four wavefronts in LDS: each writes its o rows; the per-row weights
    // exp2(m_w - M) and sums L are formed once; then each thread adds the four
    // contributions (wavefront order 0..3) of four consecutive dims of a row and stores them
    if (grp == 0) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            wm[wave][rt * 16 + col] = m[rt];
            wl[wave][rt * 16 + col] = l[rt];
        }
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(&ob[wave][rt * 16 + col][dt * 16 + 4 * grp]) = o[rt][dt];
    __syncthreads();
    for (int r = threadIdx.x; r < NRT * 16; r += kBlock) {
        const float M = fmaxf(fmaxf(wm[0][r], wm[1][r]), fmaxf(wm[2][r], wm[3][r]));
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = (wm[w][r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wm[w][r] - M);
            wf[w][r] = f;
            L += f * wl[w][r];
        }
        rowm[r] = M;
        rowl[r] = L;
    }
    __syncthreads();
    constexpr int QPR = HD / 4;  // four-dim pieces per row
    for (int idx = threadIdx.x; idx < R * QPR; idx += kBlock) {
        const int r = idx / QPR, d4 = (idx - r * QPR) * 4;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) v += wf[w][r] * *reinterpret_cast<const f32x4*>(&ob[w][r][d4]);
        const int h = g * qpg + r / p.gamma, i = r % p.gamma;
        float* dst = p.part + ((((int64_t)b * p.hq + h) * p.nparts + s) * p.gamma + i) * (HD + 2);
        *reinterpret_cast<f32x2*>(dst + d4) = f32x2{v[0], v[1]};
        *reinterpret_cast<f32x2*>(dst + d4 + 2) = f32x2{v[2], v[3]};
        if (d4 == 0) {
            dst[HD] = rowm[r] * 0.6931471805599453f;  // natural-log units
            dst[HD + 1] = rowl[r];
        }
    }
    trace_end(p.stamps, t_start);
}

// ---------------------------------------------------------------------------
// Shared-stage MFMA kernel (bf16 caches, head dim 128, 17..48 query rows per kv head,
// launches bound by the K/V stream). One wavefront per 16-row query tile, as in the
// row-split kernel below, but the workgroup's wavefronts share each 32-key unit through
// LDS: the unit's K rows and V columns go from memory straight into one of kAttnStages
// LDS stages (global_load_lds_dwordx4, lane l's 16 bytes at the instruction's LDS base +
// 16 l; the wavefronts split the 16 loads of a unit), kAttnStages - 1 units ahead of the
// one being multiplied, so each byte is fetched once and no registers hold loads in
// flight. Scores are transposed as in attn_mfma_kernel (P stays in registers); K and V
// operands are read from the stage. Stage tiles are swizzled in 16-byte pieces: K row r
// (a key) holds its piece p at slot p ^ f(r), f(r) = (r & 3) | ((r >> 1) & 12), V row d (a
// head dim, 4 pieces of 8 keys) holds piece q at slot q ^ ((d >> 2) & 3), so the 16 lanes
// of an operand read touch every bank once; each lane of a load picks the source piece its
// slot holds (a row's lanes still read its contiguous bytes).
#ifndef DFL_ATTN_STAGES
#define DFL_ATTN_STAGES 4
#endif
constexpr int kAttnStages = DFL_ATTN_STAGES;
static_assert(kAttnStages >= 2 && kAttnStages <= 5, "stage count");
constexpr int kStageK = kChunk * 128;  // bf16 elements of a unit's K tile (head dim 128)

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes a lane from src into LDS at lds_base + 16 * lane (lds_base uniform). Written as
// the instruction itself: through the intrinsic the compiler waits for every load in flight
// before each later LDS read and barrier; the waits here are explicit. M0 is read at issue
// and appears only in these instructions.
__device__ __forceinline__ void attn_dma16(const uint16_t* src, const uint16_t* lds_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)lds_base);
#if DFL_STREAM_NT
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds) : "memory", "m0");
#else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

template <int NRT>
__global__ __launch_bounds__(64 * NRT) void attn_lds_kernel(const AttnParams p) {
    constexpr int HD = 128, KS = HD / 32, DT = HD / 16;
    constexpr int D = kAttnStages;
    constexpr int NLOAD = 2 * HD / 16;                 // 1 KB loads per unit (K, then V)
    constexpr int PER = (NLOAD + NRT - 1) / NRT;      // loads per wavefront per unit (at most)
    constexpr int LOW = NLOAD / NRT;                  // (at least)
    __shared__ __align__(16) uint16_t stage[D][2][kStageK];  // [stage][K rows | V rows]
    const uint64_t t_start = trace_start(p.stamps);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;  // wave = this wavefront's row tile
    const int col = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x % p.nsplit;
    const int bg = blockIdx.x / p.nsplit;
    const int g = bg % p.hkv;
    const int b = lpt_sequence(p, bg / p.hkv);
    const int qpg = p.hq / p.hkv;
    const int R = qpg * p.gamma;
    const int lenb = min(max(p.len[b], 0), p.cap);
    const int kbeg = p.window > 0 ? max(0, lenb - p.window) : 0;
    const int cb = kbeg & ~(kChunk - 1);
    const int nch = (lenb - cb + kChunk - 1) / kChunk;
    const int nunits = nch + 1;
    const int upw = (nunits + p.nsplit - 1) / p.nsplit;
    const int u_begin = min(nunits, s * upw);
    const int u_end = min(nunits, u_begin + upw);

    const int64_t qkv_ld = p.qkv_ld;
    const uint16_t* qrow0 = static_cast<const uint16_t*>(p.qkv) + (int64_t)b * p.gamma * qkv_ld;
    const int kcol = p.hq * HD + g * HD;
    const uint16_t* kc = static_cast<const uint16_t*>(p.kcache) + ((int64_t)b * p.hkv + g) * p.cap * HD;
    const uint16_t* vc = static_cast<const uint16_t*>(p.vcache) + ((int64_t)b * p.hkv + g) * HD * (int64_t)p.cap;
    const uint16_t* vblk = p.vblk + ((int64_t)b * p.hkv + g) * HD * kChunk;
    const float sl2 = p.scale * 1.4426950408889634f;

    // load j of unit u (this wavefront issues j = wave, wave + NRT, ...): j < HD/16 is K rows
    // 4j .. 4j+3, else V rows (head dims) 16(j - HD/16) .. +15
    auto issue = [&](const int u, const int j) {
        uint16_t* dst = &stage[u % D][0][0];
        const uint16_t* src;
        if (j < HD / 16) {
            const int r = 4 * j + (lane >> 4), slot = lane & 15;
            const int piece = slot ^ ((r & 3) | ((r >> 1) & 12));
            src = (u != nch) ? kc + (int64_t)(cb + u * kChunk + r) * HD
                             : qrow0 + (int64_t)min(r, p.gamma - 1) * qkv_ld + kcol;
            src += 8 * piece;
            dst += j * 512;
        } else {
            const int jj = j - HD / 16;
            const int d = 16 * jj + (lane >> 2), slot = lane & 3;
            const int piece = slot ^ ((d >> 2) & 3);
            src = (u != nch) ? vc + ((int64_t)(cb / kChunk + u) * HD + d) * kChunk : vblk + d * kChunk;
            src += 8 * piece;
            dst += kStageK + jj * 512;
        }
        attn_dma16(src, dst);
    };
    auto issue_unit = [&](const int u) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int j = wave + NRT * q;
            if (j < NLOAD) issue(u, j);
        }
    };

    // this wavefront's Q tile (rows past R repeat row R-1, never stored)
    u32x4 qa[KS];
    {
        const int r = min(wave * 16 + col, R - 1);
        const uint16_t* src = qrow0 + (int64_t)(r % p.gamma) * qkv_ld + (g * qpg + r / p.gamma) * HD + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const u32x4*>(src + ks * 32);
        // consumed here, before the stage loads go out: the compiler does not count those, and
        // its wait for Q at the first product would otherwise wait for them too
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qa[ks]));
    }
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (int u = u_begin; u < u_begin + D - 1 && u < u_end; ++u) issue_unit(u);
    const int kq = 8 * (col >> 2) + (col & 3);
    for (int u = u_begin; u < u_end; ++u) {
        // unit u's loads landed (this wavefront's): later units' loads may stay in flight;
        // the count is the fewest any wavefront issued, so a wavefront with more waits a
        // little early. Then every wavefront's pieces, and every read of the stage reused next.
        const int later = min(u_end - 1 - u, D - 2);
        if (later >= 3)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * LOW) : "memory");
        else if (later == 2)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOW) : "memory");
        else if (later == 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOW) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (u + D - 1 < u_end) issue_unit(u + D - 1);

        const uint16_t* Kt = &stage[u % D][0][0];
        const uint16_t* Vt = &stage[u % D][1][0];
        const int nvalid = (u == nch) ? p.gamma : min(kChunk, lenb - cb - u * kChunk);
        const int lo = (u == 0 && u != nch) ? kbeg - cb : 0;
        f32x4 sc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int r = kq + 4 * nt;
            const int f = (r & 3) | ((r >> 1) & 12);
            sc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 ka = *reinterpret_cast<const u32x4*>(Kt + r * HD + 8 * ((4 * ks + grp) ^ f));
                sc[nt] = mfma16(ka, qa[ks], sc[nt]);
            }
        }
        u32x4 ph, pl;
        softmax_tile<DT>(sc, lo > 0 || nvalid < kChunk, grp, lo, nvalid, sl2, u != u_begin, m, l, o, ph, pl);
        u32x4 vb[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = 16 * dt + col;
            vb[dt] = *reinterpret_cast<const u32x4*>(Vt + d * kChunk + 8 * (grp ^ ((d >> 2) & 3)));
        }
        if (nvalid < kChunk) mask_v<DT>(vb, nvalid, grp);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = mfma16(vb[dt], pl, mfma16(vb[dt], ph, o[dt]));
    }

    // this wavefront's rows: lane holds dims dt*16 + 4*grp + e of row wave*16 + col
    const int r = wave * 16 + col;
    if (r < R) {
        const int h = g * qpg + r / p.gamma, i = r % p.gamma;
        float* dst = p.part + ((((int64_t)b * p.hq + h) * p.nparts + s) * p.gamma + i) * (HD + 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            *reinterpret_cast<f32x2*>(dst + 16 * dt + 4 * grp) = f32x2{o[dt][0], o[dt][1]};
            *reinterpret_cast<f32x2*>(dst + 16 * dt + 4 * grp + 2) = f32x2{o[dt][2], o[dt][3]};
        }
        if (grp == 0) {
            dst[HD] = m * 0.6931471805599453f;  // natural-log units (-inf without units)
            dst[HD + 1] = l;
        }
    }
    trace_end(p.stamps, t_start);
}

// ---------------------------------------------------------------------------
// Row-split MFMA kernel (bf16 caches, 33..48 query rows per kv head): one
// wavefront per 16-row tile, every wavefront walking all of the workgroup's
// units. Each wavefront holds one tile's Q, O and softmax state (about half
// the registers of one wavefront holding all tiles), so two wavefronts fit on
// a SIMD and the next unit's K and V go into a second register set while the
// current unit is multiplied. The wavefronts read the same K and V (served by
// L2 and L1 after the first) and write their own rows' partial results: no
// in-workgroup merge.

template <int HD, int NRT>
__global__ __launch_bounds__(64 * NRT, 2) void attn_rows_kernel(const AttnParams p) {
    const uint64_t t_start = trace_start(p.stamps);
    constexpr int KS = HD / 32, DT = HD / 16;
    constexpr int PLD = kChunk + 8;
    __shared__ __align__(16) uint16_t plds[NRT][2][16][PLD];  // P tiles (high, low) per wavefront

    const int lane = threadIdx.x & 63, rt = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x % p.nsplit;
    const int bg = blockIdx.x / p.nsplit;
    const int g = bg % p.hkv, b = bg / p.hkv;
    const int qpg = p.hq / p.hkv;
    const int R = qpg * p.gamma;
    const int lenb = min(max(p.len[b], 0), p.cap);
    // units: the 32-key chunks from the one holding the first attended key, then the
    // block's gamma keys; the workgroup takes an equal run of consecutive units
    const int kbeg = p.window > 0 ? max(0, lenb - p.window) : 0;
    const int cb = kbeg & ~(kChunk - 1);
    const int nch = (lenb - cb + kChunk - 1) / kChunk;
    const int nunits = nch + 1;
    const int upw = (nunits + p.nsplit - 1) / p.nsplit;
    const int u_begin = min(nunits, s * upw);
    const int u_end = min(nunits, u_begin + upw);

    const int64_t qkv_ld = p.qkv_ld;
    const uint16_t* qrow0 = static_cast<const uint16_t*>(p.qkv) + (int64_t)b * p.gamma * qkv_ld;
    const int kcol = p.hq * HD + g * HD;
    const uint16_t* kc = static_cast<const uint16_t*>(p.kcache) + ((int64_t)b * p.hkv + g) * p.cap * HD;
    const uint16_t* vc = static_cast<const uint16_t*>(p.vcache) + ((int64_t)b * p.hkv + g) * HD * (int64_t)p.cap;
    const uint16_t* vblk = p.vblk + ((int64_t)b * p.hkv + g) * HD * kChunk;
    const float sl2 = p.scale * 1.4426950408889634f;  // scores in log2 units

    // K rows c0 + nt*16 + col (dims ks*32 + 8*grp ..) and V keys c0 + 8*grp .. +8 of dims
    // dt*16 + col (rows past the valid keys: in-bounds rows, masked / zeroed before use)
    u32x4 kA[2][KS], vA[DT], kB[2][KS], vB[DT];
    auto load_unit = [&](const int u, u32x4 (&kb)[2][KS], u32x4 (&vb)[DT]) {
        const uint16_t *k0, *k1, *vp;
        int64_t vstride;
        if (u != nch) {
            k0 = kc + (int64_t)(cb + u * kChunk + col) * HD + 8 * grp;
            k1 = k0 + 16 * HD;
            vp = vc + ((int64_t)(cb / kChunk + u) * HD + col) * kChunk + 8 * grp;
            vstride = 16 * kChunk;
        } else {
            k0 = qrow0 + (int64_t)min(col, p.gamma - 1) * qkv_ld + kcol + 8 * grp;
            k1 = qrow0 + (int64_t)min(16 + col, p.gamma - 1) * qkv_ld + kcol + 8 * grp;
            vp = vblk + col * kChunk + 8 * grp;
            vstride = 16 * kChunk;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kb[0][ks] = kv_load(k0 + ks * 32);
            kb[1][ks] = kv_load(k1 + ks * 32);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vb[dt] = kv_load(vp + dt * vstride);
    };
    const bool any = u_begin < u_end;
    if (any) load_unit(u_begin, kA, vA);

    // this wavefront's Q tile: rows rt*16 + col (rows past R repeat row R-1, never stored)
    u32x4 qa[KS];
    {
        const int r = min(rt * 16 + col, R - 1);
        const uint16_t* src = qrow0 + (int64_t)(r % p.gamma) * qkv_ld + (g * qpg + r / p.gamma) * HD + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const u32x4*>(src + ks * 32);
    }

    f32x4 o[DT];
    float m[4], l[4];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) { m[e] = -INFINITY; l[e] = 0.f; }

    auto unit = [&](const int u, u32x4 (&kb)[2][KS], u32x4 (&vb)[DT]) {
        const int nvalid = (u == nch) ? p.gamma : min(kChunk, lenb - cb - u * kChunk);
        const int lo = (u == 0 && u != nch) ? kbeg - cb : 0;  // keys before the window's first
        f32x4 sacc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[nt] = mfma16(qa[ks], kb[nt][ks], sacc[nt]);
        }
        const bool v0ok = col >= lo && col < nvalid, v1ok = 16 + col >= lo && 16 + col < nvalid;
        const bool rescale = (u != u_begin);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float s0 = v0ok ? sacc[0][e] * sl2 : -INFINITY;
            const float s1 = v1ok ? sacc[1][e] * sl2 : -INFINITY;
            const float mn = fmaxf(m[e], row16_max(fmaxf(s0, s1)));  // finite: a unit holds a valid key
            const float p0 = __builtin_amdgcn_exp2f(s0 - mn);
            const float p1 = __builtin_amdgcn_exp2f(s1 - mn);
            const float al = __builtin_amdgcn_exp2f(m[e] - mn);
            l[e] = l[e] * al + row16_sum(p0 + p1);
            m[e] = mn;
            if (rescale) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt][e] *= al;
            }
            const uint32_t hp = pack_bf16x2(p0, p1);
            const uint32_t lp = pack_bf16x2(p0 - bf16_lo(hp), p1 - bf16_hi(hp));
            plds[rt][0][4 * grp + e][col] = (uint16_t)hp;
            plds[rt][0][4 * grp + e][16 + col] = (uint16_t)(hp >> 16);
            plds[rt][1][4 * grp + e][col] = (uint16_t)lp;
            plds[rt][1][4 * grp + e][16 + col] = (uint16_t)(lp >> 16);
        }
        const u32x4 pa = *reinterpret_cast<const u32x4*>(&plds[rt][0][col][8 * grp]);
        const u32x4 pl = *reinterpret_cast<const u32x4*>(&plds[rt][1][col][8 * grp]);
        if (nvalid < kChunk) {
            const int nk = nvalid - 8 * grp;
            u32x4 mk;
#pragma unroll
            for (int q = 0; q < 4; ++q) mk[q] = (2 * q + 1 < nk) ? 0xFFFFFFFFu : ((2 * q < nk) ? 0x0000FFFFu : 0u);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vb[dt] &= mk;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = mfma16(pl, vb[dt], mfma16(pa, vb[dt], o[dt]));
    };

    // two units per trip (set A: even offsets from u_begin, set B: odd); the loads of the
    // last trip re-read the last unit, never multiplied
    for (int u = u_begin; u < u_end; u += 2) {
        load_unit(min(u + 1, u_end - 1), kB, vB);
        unit(u, kA, vA);
        if (u + 1 >= u_end) break;
        load_unit(min(u + 2, u_end - 1), kA, vA);
        unit(u + 1, kB, vB);
    }

    // this wavefront's rows: o (lane holds dims dt*16 + col of rows 4*grp + e), m, l
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = rt * 16 + 4 * grp + e;
        if (r >= R) continue;
        const int h = g * qpg + r / p.gamma, i = r % p.gamma;
        float* dst = p.part + ((((int64_t)b * p.hq + h) * p.nparts + s) * p.gamma + i) * (HD + 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) dst[dt * 16 + col] = o[dt][e];
        if (col == 0) {
            dst[HD] = m[e] * 0.6931471805599453f;  // natural-log units (-inf without units)
            dst[HD + 1] = l[e];
        }
    }
    trace_end(p.stamps, t_start);
}

// ---------------------------------------------------------------------------
// VALU kernel (fp32 caches)

template <int HD, int RMAX>
__global__ __launch_bounds__(kBlock) void attn_valu_kernel(const AttnParams p) {
    const uint64_t t_start = trace_start(p.stamps);
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
    // keys: the attended context rows kbeg .. lenb-1 (all, or the window's), then the block's
    const int kbeg = p.window > 0 ? max(0, lenb - p.window) : 0;
    const int nctx = lenb - kbeg;
    const int T = nctx + p.gamma;
    int C = (T + p.nsplit - 1) / p.nsplit;
    C = ((C + kTile - 1) / kTile) * kTile;
    const int start = s * C;
    const int end = min(T, start + C);

    const int64_t qkv_ld = p.qkv_ld;
    const float* qrow0 = static_cast<const float*>(p.qkv) + (int64_t)b * p.gamma * qkv_ld;
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
            if (kk < nctx) {
                kv = kc[(int64_t)(kbeg + kk) * HD + dd];
                vv = vc[(int64_t)dd * p.cap + kbeg + kk];
            } else if (kk < T) {
                const float* rowp = qrow0 + (int64_t)(kk - nctx) * qkv_ld;
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
    trace_end(p.stamps, t_start);
}

// ---------------------------------------------------------------------------
// One wavefront per (b, head, block row), four rows per workgroup, no barriers:
// combine the nparts partials (o, m, l) of the row. The (m, l) of the first 64
// partials (one per lane) and the values of the first MR go out in one batch, so
// up to MR partials cost one round trip (MR = 8, 32 or 64, the smallest that holds
// the partials: a wider batch issues loads of clamped indexes whose values go
// unused). M = max m_s, weights w_s = exp(m_s - M) (lane s, read back uniformly),
// L = sum w_s l_s, and each lane
// sums its HD/64 head-dim columns over the partials in order s = 0, 1, ...
template <int HD, int MR>
__global__ __launch_bounds__(kBlock) void attn_merge_kernel(const AttnParams p) {
    constexpr int DPL = HD / 64;  // head-dim columns per lane
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*hq + h)*gamma + i
    if (row >= p.B * p.hq * p.gamma) return;
    const int i = row % p.gamma;
    const int bh = row / p.gamma;
    const int h = bh % p.hq, b = bh / p.hq;
    const int W = HD + 2;
    const int np = p.nparts;
    const float* base = p.part + ((int64_t)bh * np * p.gamma + i) * W;
    const int64_t sstride = (int64_t)p.gamma * W;
    float ms = -INFINITY, ls = 0.f;
    if (lane < np) {
        ms = base[lane * sstride + HD];
        ls = base[lane * sstride + HD + 1];
    }
    float v[MR][DPL];  // partials past np: clamped, in bounds, unused
#pragma unroll
    for (int j = 0; j < MR; ++j)
#pragma unroll
        for (int q = 0; q < DPL; ++q) v[j][q] = base[(int64_t)min(j, np - 1) * sstride + lane + 64 * q];
    float mx = ms;
    for (int sidx = 64 + lane; sidx < np; sidx += 64) mx = fmaxf(mx, base[sidx * sstride + HD]);
    const float M = wave_max(mx);
    float w = (lane < np && ms != -INFINITY) ? expf(ms - M) : 0.f;
    float lsum = w * ls;
    float acc[DPL];
#pragma unroll
    for (int q = 0; q < DPL; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < MR; ++j) {
        if (j < np) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
#pragma unroll
            for (int q = 0; q < DPL; ++q) acc[q] += wj * v[j][q];
        }
    }
    for (int c0 = 0; c0 < np; c0 += 64) {
        if (c0 > 0) {  // the weights of partials c0 .. c0 + 63
            const int sidx = c0 + lane;
            w = 0.f;
            if (sidx < np) {
                const float m2 = base[sidx * sstride + HD];
                w = (m2 == -INFINITY) ? 0.f : expf(m2 - M);
                lsum += w * base[sidx * sstride + HD + 1];
            }
        }
        const int j0 = c0 == 0 ? MR : 0, cnt = min(64, np - c0);
#pragma unroll 8
        for (int j = j0; j < cnt; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
            const float* src = base + (int64_t)(c0 + j) * sstride;
#pragma unroll
            for (int q = 0; q < DPL; ++q) acc[q] += wj * src[lane + 64 * q];
        }
    }
    const float L = wave_sum(lsum);
#pragma unroll
    for (int q = 0; q < DPL; ++q) {
        const float y = acc[q] / L;
        const int64_t o = ((int64_t)b * p.gamma + i) * p.out_ld + h * HD + lane + 64 * q;
        if (p.round_out)
            reinterpret_cast<uint16_t*>(p.out)[o] = (uint16_t)f32_to_bf16_bits(y);
        else
            p.out[o] = y;
    }
}

// ---------------------------------------------------------------------------

// attention workgroups a launch aims for over all (sequence, kv head) pairs (with the K/V
// stream non-temporal, 512 beats 768 at Batched: fewer partials and longer runs of units)
#ifndef DFL_ATTN_WGS
#define DFL_ATTN_WGS 512
#endif

// workgroups the row-split kernel aims for (three wavefronts each)
#ifndef DFL_ATTN_ROWS_WGS
#define DFL_ATTN_ROWS_WGS 2048
#endif
// the row-split kernel serves launches of up to this many 32-key units in all (pairs x
// units): there attention is latency-bound. Beyond it (many long sequences) the K/V
// stream is the bound, and the kernel's three reads of each unit cost more than its
// registers save.
#ifndef DFL_ATTN_ROWS_MAX_UNITS
#define DFL_ATTN_ROWS_MAX_UNITS 8192
#endif

static bool use_rows_kernel(int rows, int kv_f32, int pairs, int cap) {
    const int64_t units = (int64_t)(cap + kChunk - 1) / kChunk + 1;
    return !kv_f32 && rows > 32 && rows <= kMaxRows && (int64_t)pairs * units <= DFL_ATTN_ROWS_MAX_UNITS;
}

// the shared-stage kernel: bf16 caches, head dim 128, two 16-row tiles (Wide4's 20 rows: 77 ->
// 52 us per round against the all-tiles kernel), where the row-split kernel does not apply.
// With three tiles (Batched's 35 rows) the all-tiles kernel measured faster (785 against
// 843 us per round).
#ifndef DFL_ATTN_LDS_MIN_ROWS
#define DFL_ATTN_LDS_MIN_ROWS 17
#endif
#ifndef DFL_ATTN_LDS_MAX_ROWS
#define DFL_ATTN_LDS_MAX_ROWS 32
#endif
#ifndef DFL_ATTN_LDS_WGS
#define DFL_ATTN_LDS_WGS 1024
#endif
static bool use_lds_kernel(int rows, int kv_f32, int pairs, int cap, int hd) {
    return !kv_f32 && hd == 128 && rows >= DFL_ATTN_LDS_MIN_ROWS && rows <= DFL_ATTN_LDS_MAX_ROWS &&
           !use_rows_kernel(rows, kv_f32, pairs, cap);
}

void attention_splits(int cap, int gamma, int kv_f32, int pairs, int rows, int hd, int* nsplit, int* nparts) {
    const int units = (cap + kChunk - 1) / kChunk + 1;
    const int np = pairs > 0 ? pairs : 1;
    if (use_lds_kernel(rows, kv_f32, pairs, cap, hd)) {
        // one workgroup walks its run of units with all its wavefronts
        int ns = (DFL_ATTN_LDS_WGS + np - 1) / np;
        ns = ns > units ? units : ns;
        ns = ns < 1 ? 1 : (ns > kMaxSplit ? kMaxSplit : ns);
        *nsplit = ns;
        *nparts = ns;
        return;
    }
    if (use_rows_kernel(rows, kv_f32, pairs, cap)) {
        // a workgroup walks its units with three wavefronts; enough workgroups to fill the GPU
        int ns = (DFL_ATTN_ROWS_WGS + np - 1) / np;
        ns = ns > units ? units : ns;
        ns = ns < 1 ? 1 : (ns > kMaxSplit ? kMaxSplit : ns);
        *nsplit = ns;
        *nparts = ns;
        return;
    }
    if (kv_f32) {
        int ns = (cap + gamma + kTile - 1) / kTile;
        ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
        *nsplit = ns;
        *nparts = ns;
    } else {
        // one unit per wavefront (cap/32 chunks plus the block) while the launch stays
        // below DFL_ATTN_WGS workgroups; with many (sequence, kv head) pairs, fewer splits
        // of more units each (fewer partial results, and the GPU is full either way)
        int ns = (units + 3) / 4;
        const int want = (DFL_ATTN_WGS + np - 1) / np;
        if (ns > want) ns = want;
        ns = ns < 1 ? 1 : (ns > kMaxSplit ? kMaxSplit : ns);
        *nsplit = ns;
        *nparts = ns;
    }
}

int attention_max_rows(int kv_f32) { return kv_f32 ? 40 : kMaxRows; }

template <int HD>
static hipError_t launch_hd(const AttnParams& p, hipStream_t s) {
    const int R = (p.hq / p.hkv) * p.gamma;
    dim3 grid((unsigned)((int64_t)p.B * p.hkv * p.nsplit));
    // instrumentation: the launch reads Q, the block's keys and values and every held
    // context row's keys and values (counted by the caller from the lengths), and writes O
    const double esz = p.kv_f32 ? 4.0 : 2.0;
    const double rows = (double)p.B * p.gamma;
    const double bytes = rows * p.hq * HD * esz * 2.0 + rows * p.hkv * HD * 2.0 * esz;
    const double ctx_row_bytes = (double)p.hkv * HD * 2.0 * esz;
    char name[40];
    AttnParams q = p;
    (void)hipGetLastError();  // report only this launch's status
    if (p.kv_f32) {
        if (R <= 8) {
            snprintf(name, sizeof name, "attn_valu_kernel<%d, 8>", HD);
            q.stamps = trace_launch(TRACE_ATTENTION, name, grid.x, bytes, ctx_row_bytes);
            hipLaunchKernelGGL((attn_valu_kernel<HD, 8>), grid, dim3(kBlock), 0, s, q);
        } else if (R <= 40) {
            snprintf(name, sizeof name, "attn_valu_kernel<%d, 40>", HD);
            q.stamps = trace_launch(TRACE_ATTENTION, name, grid.x, bytes, ctx_row_bytes);
            hipLaunchKernelGGL((attn_valu_kernel<HD, 40>), grid, dim3(kBlock), 0, s, q);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        const int nrt = R <= 16 ? 1 : (R <= 32 ? 2 : 3);
        const int span = attn_span(p.cap, p.window);
        const bool rows_kernel = R > 32 && use_rows_kernel(R, 0, p.B * p.hkv, span);
        const bool lds_kernel = use_lds_kernel(R, 0, p.B * p.hkv, span, HD);
        if (R > kMaxRows) return hipErrorInvalidValue;
        snprintf(name, sizeof name,
                 lds_kernel ? "attn_lds_kernel<%d, %d>"
                            : (rows_kernel ? "attn_rows_kernel<%d, %d>" : "attn_mfma_kernel<%d, %d>"),
                 HD, nrt);
        q.stamps = trace_launch(TRACE_ATTENTION, name, grid.x, bytes, ctx_row_bytes);
        if constexpr (HD == 128) {
            if (lds_kernel) {
                if (nrt == 2)
                    hipLaunchKernelGGL((attn_lds_kernel<2>), grid, dim3(128), 0, s, q);
                else
                    hipLaunchKernelGGL((attn_lds_kernel<3>), grid, dim3(192), 0, s, q);
                hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                goto merge;
            }
        }
        if (nrt == 1)
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 1>), grid, dim3(kBlock), 0, s, q);
        else if (nrt == 2)
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 2>), grid, dim3(kBlock), 0, s, q);
        else if (rows_kernel)
            hipLaunchKernelGGL((attn_rows_kernel<HD, 3>), grid, dim3(64 * 3), 0, s, q);
        else
            hipLaunchKernelGGL((attn_mfma_kernel<HD, 3>), grid, dim3(kBlock), 0, s, q);
    }
    {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
merge:
    const dim3 mgrid((unsigned)((p.B * p.hq * p.gamma + 3) / 4));
    if (p.nparts <= 8)
        hipLaunchKernelGGL((attn_merge_kernel<HD, 8>), mgrid, dim3(kBlock), 0, s, p);
    else if (p.nparts <= 32)
        hipLaunchKernelGGL((attn_merge_kernel<HD, 32>), mgrid, dim3(kBlock), 0, s, p);
    else
        hipLaunchKernelGGL((attn_merge_kernel<HD, 64>), mgrid, dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

int attn_span(int cap, int window) { return window > 0 && window + kChunk < cap ? window + kChunk : cap; }

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
    if (p.nparts > kMaxParts || p.gamma > kChunk || p.window < 0) return hipErrorInvalidValue;
    if (!p.kv_f32 && p.nsplit > kMaxSplit) return hipErrorInvalidValue;
    if (!p.kv_f32 && (p.cap % kChunk)) return hipErrorInvalidValue;
    if (p.hd == 128) return launch_hd<128>(p, s);
    if (p.hd == 64) return launch_hd<64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace dfl
