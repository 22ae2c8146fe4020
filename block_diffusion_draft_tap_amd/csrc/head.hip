// Small kernels of the drafter round:
//   argmax_merge_kernel   per-workgroup (max, index) partials -> greedy ids
//   verify_partial_kernel per (verify row, vocab slice) argmax of target logits
//   verify_final_kernel   prefix compare: accepted, committed, ids, next anchor (from the
//                         split partials of given logits, or from the target's greedy ids)
//   dspark_step_kernel    one step of the DSpark greedy loop (previous token, Markov operand,
//                         confidence, pruning length)
//   rownorm_kernel        RMSNorm of fp32 rows (sum of split partials) with a gain (Eq 2)
//   rownorm1_kernel       the same on 16-byte chunks (rows of a multiple of 4 values)
//   gather_rows_kernel    bf16 table rows by id (the anchors' embeddings)
//   block_fill_kernel     block rows around a stored anchor product (Eq 3 block init)
//   advance_len_kernel    len[b] += appended rows (retained context grows)
//   f32_to_bf16_kernel    fp32 -> bf16 copy for optional outputs
// Every reduction runs in a fixed order and resolves equal maxima to the
// lowest index, so results are deterministic run to run.
#include "common.hpp"
#include "head.hpp"

namespace dfl {

__device__ __forceinline__ void block_argmax(float& v, int& i, float* sv, int* si) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wave_argmax(v, i);
    if (lane == 0) { sv[wave] = v; si[wave] = i; }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = (blockDim.x + 63) / 64;
        for (int w = 1; w < nw; ++w) argmax_pick(v, i, sv[w], si[w]);
    }
}

__global__ __launch_bounds__(kBlock) void argmax_merge_kernel(const float* part_val, const int32_t* part_idx,
                                                              int nblocks, int32_t* ids, float* max_logit) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int m = blockIdx.x;
    float v = -INFINITY;
    int i = 0x7fffffff;
    // (max, lowest index) is order-independent: the loop is unrolled so a thread's loads go out together
#pragma unroll 4
    for (int j = threadIdx.x; j < nblocks; j += blockDim.x)
        argmax_pick(v, i, part_val[(int64_t)m * nblocks + j], part_idx[(int64_t)m * nblocks + j]);
    block_argmax(v, i, sv, si);
    if (threadIdx.x == 0) {
        ids[m] = i;
        if (max_logit) max_logit[m] = v;
    }
}

__global__ __launch_bounds__(kBlock) void verify_partial_kernel(const float* logits, int V, int nsplit,
                                                                float* part_val, int32_t* part_idx) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int row = blockIdx.x / nsplit, s = blockIdx.x % nsplit;
    const int chunk = (((V + nsplit - 1) / nsplit) + 3) & ~3;
    const int v0 = s * chunk, v1 = min(V, v0 + chunk);
    const float* src = logits + (int64_t)row * V;
    float v = -INFINITY;
    int i = 0x7fffffff;
    if ((V & 3) == 0) {
#pragma unroll 4
        for (int j = v0 + 4 * threadIdx.x; j < v1; j += 4 * blockDim.x) {
            const float4 a = stream_load(reinterpret_cast<const float4*>(src + j));
            argmax_pick(v, i, a.x, j);
            argmax_pick(v, i, a.y, j + 1);
            argmax_pick(v, i, a.z, j + 2);
            argmax_pick(v, i, a.w, j + 3);
        }
    } else {
        for (int j = v0 + threadIdx.x; j < v1; j += blockDim.x) argmax_pick(v, i, src[j], j);
    }
    block_argmax(v, i, sv, si);
    if (threadIdx.x == 0) {
        part_val[blockIdx.x] = v;
        part_idx[blockIdx.x] = i;
    }
}

// one 64-lane wavefront per sequence; lane j handles verify row j (gamma + 1 <= 64). With
// lengths (a pruned block proposes its first lengths[b] drafts) the prefix stops there too.
// tids: the target's greedy tokens [B][gamma+1] when they are already known (the verify
// from the target's hidden states), else merged here from the split partials
__global__ __launch_bounds__(64) void verify_final_kernel(const float* part_val, const int32_t* part_idx, int nsplit,
                                                          const int32_t* draft, int gamma, const int32_t* lengths,
                                                          int32_t* accepted, int32_t* committed, int32_t* ids,
                                                          int32_t* next_anchor, const int32_t* tids) {
    const int b = blockIdx.x, j = threadIdx.x;
    const int W = gamma + 1;
    int t = -1;
    if (j < W && tids) {
        t = tids[(int64_t)b * W + j];
    } else if (j < W) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        const int64_t base = ((int64_t)b * W + j) * nsplit;
        for (int s = 0; s < nsplit; ++s) argmax_pick(v, i, part_val[base + s], part_idx[base + s]);
        t = i;
    }
    const int lim = lengths ? min(max(lengths[b], 0), gamma) : gamma;
    const bool mismatch = (j < gamma) && (j >= lim || draft[(int64_t)b * gamma + j] != t);
    const unsigned long long mask = __ballot(mismatch);
    const int a = mask ? (__ffsll((long long)mask) - 1) : gamma;
    if (j < W) ids[(int64_t)b * W + j] = (j <= a) ? t : -1;
    if (j == a && next_anchor) next_anchor[b] = t;
    if (j == 0) {
        accepted[b] = a;
        committed[b] = a + 1;
    }
}

// One step of the DSpark greedy loop for sequence b = blockIdx.x (page 3, forwardRows with
// #markov and #confidence): the previous token (the anchor at step 0, else the argmax of the
// previous step's (max, index) partials, lowest index on ties) becomes draft step - 1; the
// Markov operand row e1 = w1[previous] is written for this step's projection; this step's
// confidence sigmoid([block row; e1] . conf_w + conf_b) and the Alg 1 length update (a row
// still at full length is cut to `step` when the confidence falls below the step's
// threshold; step 0 always stays). step == gamma only merges the last step's partials.
__global__ __launch_bounds__(kBlock) void dspark_step_kernel(const DsparkStepParams p) {
    __shared__ float sv[4];
    __shared__ int si[4];
    __shared__ int prev_s;
    __shared__ float red[4];
    const int b = blockIdx.x, tid = threadIdx.x;
    if (p.step == 0) {
        if (tid == 0) prev_s = p.anchors[b];
    } else {
        float v = -INFINITY;
        int i = 0x7fffffff;
        const int64_t base = (int64_t)b * p.nblocks;
        for (int j = tid; j < p.nblocks; j += blockDim.x) argmax_pick(v, i, p.part_val[base + j], p.part_idx[base + j]);
        block_argmax(v, i, sv, si);
        if (tid == 0) {
            prev_s = i;
            p.ids[(int64_t)b * p.gamma + p.step - 1] = i;
        }
    }
    __syncthreads();
    if (p.step == p.gamma) return;
    const int prev = min(max(prev_s, 0), p.V - 1);
    const int64_t row = (int64_t)b * p.gamma + p.step;
    float acc = 0.f;
    for (int c = tid; c < p.r; c += blockDim.x) {
        float e;
        if (p.f32) {
            e = static_cast<const float*>(p.w1)[(int64_t)prev * p.r + c];
            static_cast<float*>(p.e1)[(int64_t)b * p.r + c] = e;
        } else {
            const uint16_t bits = static_cast<const uint16_t*>(p.w1)[(int64_t)prev * p.r + c];
            e = bf16_bits_to_f32(bits);
            static_cast<uint16_t*>(p.e1)[(int64_t)b * p.r + c] = bits;
        }
        acc += e * load_gain(p.conf_w, p.f32, p.d + c);
    }
    for (int c = tid; c < p.d; c += blockDim.x) {
        const float h = p.f32 ? static_cast<const float*>(p.hout)[row * p.d + c]
                              : bf16_bits_to_f32(static_cast<const uint16_t*>(p.hout)[row * p.d + c]);
        acc += h * load_gain(p.conf_w, p.f32, c);
    }
    acc = wave_sum(acc);
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        float z = load_gain(p.conf_b, p.f32, 0);
        for (int w = 0; w < (int)(blockDim.x + 63) / 64; ++w) z += red[w];
        const float c = 1.0f / (1.0f + expf(-z));
        if (p.conf) p.conf[row] = c;
        if (p.step == 0) {
            p.lengths[b] = p.gamma;
        } else {
            const float thr = p.thresholds ? p.thresholds[p.step] : p.min_conf;
            if (p.lengths[b] == p.gamma && c < thr) p.lengths[b] = p.step;
        }
    }
}

hipError_t launch_dspark_step(const DsparkStepParams& p, hipStream_t s) {
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(dspark_step_kernel, dim3(p.B), dim3(kBlock), 0, s, p);
    return hipGetLastError();
}

// dst[r] = RMSNorm(sum_z src[z][r]; gain): the split-K partials are added in
// a fixed order (z = 0, 1, ...); dst may alias src when there is one split.
// A thread holds KP elements of its row (rows of up to KP*256 elements) and
// takes the splits in batches of kZB: every load of a batch is issued before
// the first add (indexes past the row or the split count are clamped to valid
// addresses and their values unused), so a row costs ceil(nsplit / kZB) round
// trips.
constexpr int kZB = 4;

template <int KP>
__global__ __launch_bounds__(kBlock) void rownorm_kernel(const float* src, int nsplit, int64_t split_stride,
                                                         float* dst, int d, const void* gain, int gain_f32,
                                                         float eps) {
    __shared__ float sv[4];
    const int64_t roff = (int64_t)blockIdx.x * d;
    const int tid = threadIdx.x;
    float vals[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) vals[j] = 0.f;
    for (int z0 = 0; z0 < nsplit; z0 += kZB) {
        float t[kZB][KP];
#pragma unroll
        for (int zb = 0; zb < kZB; ++zb) {
            const int64_t zo = (int64_t)min(z0 + zb, nsplit - 1) * split_stride + roff;
#pragma unroll
            for (int j = 0; j < KP; ++j) t[zb][j] = src[zo + min(tid + j * kBlock, d - 1)];
        }
#pragma unroll
        for (int zb = 0; zb < kZB; ++zb)
            if (z0 + zb < nsplit) {
#pragma unroll
                for (int j = 0; j < KP; ++j) vals[j] += t[zb][j];
            }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
        if (tid + j * kBlock >= d) vals[j] = 0.f;
        s += vals[j] * vals[j];
    }
    s = wave_sum(s);
    if ((tid & 63) == 0) sv[tid >> 6] = s;
    __syncthreads();
    const float tot = sv[0] + sv[1] + sv[2] + sv[3];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int j = 0; j < KP; ++j) {
        const int k = tid + j * kBlock;
        if (k < d) dst[roff + k] = vals[j] * r * load_gain(gain, gain_f32, k);
    }
}

// rows of 16-byte-aligned chunks: each chunk of the row is the sum of the split partials
// in split order (one partial: the row itself), read into registers (the splits in
// batches of kZB, every load of a batch issued before the first add), the sum of squares
// reduced across the workgroup while the gains load, then scaled and written (in place
// when src == dst and nsplit == 1: every thread writes only the chunks it read)
template <int KP4>
__global__ __launch_bounds__(kBlock) void rownorm1_kernel(const float* src, int nsplit, int64_t split_stride,
                                                          float* dst, int d, const void* gain, int gain_f32,
                                                          float eps) {
    __shared__ float sv[4];
    const int64_t roff = (int64_t)blockIdx.x * d;
    const int tid = threadIdx.x, n4 = d / 4;
    f32x4 v[KP4];
#pragma unroll
    for (int j = 0; j < KP4; ++j)
        v[j] = *reinterpret_cast<const f32x4*>(src + roff + 4 * min(tid + j * kBlock, n4 - 1));
    for (int z0 = 1; z0 < nsplit; z0 += kZB) {
        f32x4 t[kZB][KP4];
#pragma unroll
        for (int zb = 0; zb < kZB; ++zb) {
            const int64_t zo = (int64_t)min(z0 + zb, nsplit - 1) * split_stride + roff;
#pragma unroll
            for (int j = 0; j < KP4; ++j)
                t[zb][j] = *reinterpret_cast<const f32x4*>(src + zo + 4 * min(tid + j * kBlock, n4 - 1));
        }
#pragma unroll
        for (int zb = 0; zb < kZB; ++zb)
            if (z0 + zb < nsplit) {
#pragma unroll
                for (int j = 0; j < KP4; ++j) {
                    v[j].x += t[zb][j].x;
                    v[j].y += t[zb][j].y;
                    v[j].z += t[zb][j].z;
                    v[j].w += t[zb][j].w;
                }
            }
    }
    float s = 0.f;
    f32x4 g[KP4];
#pragma unroll
    for (int j = 0; j < KP4; ++j) {
        const int k = 4 * min(tid + j * kBlock, n4 - 1);
        g[j].x = load_gain(gain, gain_f32, k);
        g[j].y = load_gain(gain, gain_f32, k + 1);
        g[j].z = load_gain(gain, gain_f32, k + 2);
        g[j].w = load_gain(gain, gain_f32, k + 3);
        if (tid + j * kBlock < n4) s += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
    }
    s = wave_sum(s);
    if ((tid & 63) == 0) sv[tid >> 6] = s;
    __syncthreads();
    const float tot = sv[0] + sv[1] + sv[2] + sv[3];
    const float r = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
    for (int j = 0; j < KP4; ++j) {
        const int q = tid + j * kBlock;
        if (q < n4) {
            f32x4 o;
            o.x = v[j].x * r * g[j].x;
            o.y = v[j].y * r * g[j].y;
            o.z = v[j].z * r * g[j].z;
            o.w = v[j].w * r * g[j].w;
            *reinterpret_cast<f32x4*>(dst + roff + 4 * q) = o;
        }
    }
}

// dst[r] = table[clamp(ids[r])] for rows of K bf16 values (K a multiple of 8); one
// workgroup per row, 16-byte copies
__global__ __launch_bounds__(kBlock) void gather_rows_kernel(const uint16_t* table, int table_rows, const int32_t* ids,
                                                            int K, uint16_t* dst) {
    const int r = blockIdx.x;
    const int id = min(max(ids[r], 0), table_rows - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(table + (int64_t)id * K);
    u32x4* out = reinterpret_cast<u32x4*>(dst + (int64_t)r * K);
    for (int i = threadIdx.x; i < K / 8; i += kBlock) out[i] = src[i];
}

// the block rows of sequence b around its stored anchor product h[b][0][:] = E_in[anchor] W_tok^T:
// h[b][0][n] += block_pos[0][n]; h[b][k][n] = mask_emb[k-1][n] + block_pos[k][n] for 0 < k < gamma
__global__ __launch_bounds__(kBlock) void block_fill_kernel(float* h, int gamma, int d, const void* block_pos,
                                                           const void* mask_emb, int gain_f32) {
    const int b = blockIdx.y, k = blockIdx.z;
    const int n = blockIdx.x * kBlock + threadIdx.x;
    if (n >= d) return;
    float* row = h + ((int64_t)b * gamma + k) * d;
    if (k == 0)
        row[n] += load_gain(block_pos, gain_f32, n);
    else
        row[n] = load_gain(mask_emb, gain_f32, (k - 1) * d + n) + load_gain(block_pos, gain_f32, k * d + n);
}

// one reading of the device wall clock (the tick counter of the launch stamps)
__global__ void wall_clock_kernel(uint64_t* out) {
    if (threadIdx.x == 0) out[0] = (uint64_t)wall_clock64();
}

__global__ void advance_len_kernel(int32_t* len, const int32_t* row_offsets, const int32_t* counts, int B, int cap,
                                   int32_t* save) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int rows = row_offsets[b + 1] - row_offsets[b];
        const int add = counts ? min(counts[b], rows) : rows;
        const int old = len[b];
        if (save) save[b] = old;
        len[b] = min(cap, old + max(add, 0));
    }
}

__global__ void f32_to_bf16_kernel(const float* src, uint16_t* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = (uint16_t)f32_to_bf16_bits(src[i]);
}

__global__ void copy_f32_kernel(const float* src, float* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------

hipError_t launch_argmax_merge(const float* pv, const int32_t* pi, int nblocks, int M, int32_t* ids, float* maxl,
                               hipStream_t s) {
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(argmax_merge_kernel, dim3(M), dim3(kBlock), 0, s, pv, pi, nblocks, ids, maxl);
    return hipGetLastError();
}

int verify_splits(int V) {
    int ns = (V + 4095) / 4096;
    return ns < 1 ? 1 : (ns > 64 ? 64 : ns);
}

hipError_t launch_verify(const float* logits, const int32_t* draft, int B, int gamma, int V, int32_t* accepted,
                         int32_t* committed, int32_t* ids, int32_t* next_anchor, float* pv, int32_t* pi,
                         hipStream_t s, const int32_t* lengths) {
    const int ns = verify_splits(V);
    const int rows = B * (gamma + 1);
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(verify_partial_kernel, dim3(rows * ns), dim3(kBlock), 0, s, logits, V, ns, pv, pi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(verify_final_kernel, dim3(B), dim3(64), 0, s, pv, pi, ns, draft, gamma, lengths, accepted,
                       committed, ids, next_anchor, (const int32_t*)nullptr);
    return hipGetLastError();
}

hipError_t launch_verify_ids(const int32_t* tids, const int32_t* draft, int B, int gamma, int32_t* accepted,
                             int32_t* committed, int32_t* ids, int32_t* next_anchor, const int32_t* lengths,
                             hipStream_t s) {
    if (gamma + 1 > 64) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(verify_final_kernel, dim3(B), dim3(64), 0, s, (const float*)nullptr, (const int32_t*)nullptr, 0,
                       draft, gamma, lengths, accepted, committed, ids, next_anchor, tids);
    return hipGetLastError();
}

hipError_t launch_rownorm(const float* src, int nsplit, int64_t split_stride, float* dst, int rows, int d,
                          const void* gain, int gain_f32, float eps, hipStream_t s) {
    (void)hipGetLastError();  // report only this launch's status
    // in place only without partials (rows are read whole before they are written)
    const bool vec = d % 4 == 0 && (nsplit == 1 || (split_stride % 4 == 0 && src != dst)) &&
                     ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    if (vec && d <= 4 * kBlock) {
        hipLaunchKernelGGL(rownorm1_kernel<1>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
        return hipGetLastError();
    }
    if (vec && d <= 8 * kBlock) {
        hipLaunchKernelGGL(rownorm1_kernel<2>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
        return hipGetLastError();
    }
    if (vec && d <= 32 * kBlock) {
        hipLaunchKernelGGL(rownorm1_kernel<8>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
        return hipGetLastError();
    }
    if (d <= 4 * kBlock)
        hipLaunchKernelGGL(rownorm_kernel<4>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
    else if (d <= 8 * kBlock)
        hipLaunchKernelGGL(rownorm_kernel<8>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
    else if (d <= 32 * kBlock)
        hipLaunchKernelGGL(rownorm_kernel<32>, dim3(rows), dim3(kBlock), 0, s, src, nsplit, split_stride, dst, d, gain,
                           gain_f32, eps);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* table, int table_rows, const int32_t* ids, int rows, int K,
                              uint16_t* dst, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if ((K % 8) || table_rows <= 0) return hipErrorInvalidValue;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)rows), dim3(kBlock), 0, s, table, table_rows, ids, K, dst);
    return hipGetLastError();
}

hipError_t launch_block_fill(float* h, int B, int gamma, int d, const void* block_pos, const void* mask_emb,
                             int gain_f32, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(block_fill_kernel, dim3((unsigned)((d + kBlock - 1) / kBlock), (unsigned)B, (unsigned)gamma),
                       dim3(kBlock), 0, s, h, gamma, d, block_pos, mask_emb, gain_f32);
    return hipGetLastError();
}

hipError_t launch_wall_clock(uint64_t* out, hipStream_t s) {
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(wall_clock_kernel, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

hipError_t launch_advance_len(int32_t* len, const int32_t* row_offsets, const int32_t* counts, int B, int cap,
                              hipStream_t s, int32_t* save) {
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(advance_len_kernel, dim3(1), dim3(64), 0, s, len, row_offsets, counts, B, cap, save);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
    const int64_t blocks = (n + 255) / 256;
    (void)hipGetLastError();  // report only this launch's status
    hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace dfl
