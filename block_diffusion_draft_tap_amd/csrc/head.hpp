// Argmax merge, greedy verification and small helper kernels (see head.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

hipError_t launch_argmax_merge(const float* pv, const int32_t* pi, int nblocks, int M, int32_t* ids, float* maxl,
                               hipStream_t s);
int verify_splits(int V);
hipError_t launch_verify(const float* logits, const int32_t* draft, int B, int gamma, int V, int32_t* accepted,
                         int32_t* committed, int32_t* ids, int32_t* next_anchor, float* pv, int32_t* pi,
                         hipStream_t s, const int32_t* lengths = nullptr);
// the same prefix rule from the target's greedy ids tids [B][gamma+1]
hipError_t launch_verify_ids(const int32_t* tids, const int32_t* draft, int B, int gamma, int32_t* accepted,
                             int32_t* committed, int32_t* ids, int32_t* next_anchor, const int32_t* lengths,
                             hipStream_t s);

// One step of the DSpark greedy loop per sequence (see head.hip)
struct DsparkStepParams {
    int step, gamma, B, V, r, d, nblocks, f32;  // f32: head weights and block rows in fp32
    const int32_t* anchors;                     // [B]
    const float* part_val;                      // previous step's argmax partials [B][nblocks]
    const int32_t* part_idx;
    const void* w1;                             // [V, r]
    const void* hout;                           // block rows [B * gamma, d]
    const void* conf_w;                         // [d + r]
    const void* conf_b;                         // [1]
    const float* thresholds;                    // [gamma] or null (then min_conf)
    float min_conf;
    void* e1;                                   // out: Markov operand rows [B, r]
    int32_t* ids;                               // out: drafts [B, gamma]
    float* conf;                                // out: [B, gamma] or null
    int32_t* lengths;                           // out: [B]
};
hipError_t launch_dspark_step(const DsparkStepParams& p, hipStream_t s);
hipError_t launch_rownorm(const float* src, int nsplit, int64_t split_stride, float* dst, int rows, int d,
                          const void* gain, int gain_f32, float eps, hipStream_t s);
// dst[r][:] = table[clamp(ids[r])][:] (bf16 rows of K, K a multiple of 8)
hipError_t launch_gather_rows(const uint16_t* table, int table_rows, const int32_t* ids, int rows, int K,
                              uint16_t* dst, hipStream_t s);
// block rows around stored anchor products: h[b][0] += block_pos[0]; h[b][k] = mask_emb[k-1] + block_pos[k]
hipError_t launch_block_fill(float* h, int B, int gamma, int d, const void* block_pos, const void* mask_emb,
                             int gain_f32, hipStream_t s);
// len[b] += the appended rows of b (capped at cap); with save, the lengths before go to save[b]
// out[0] = the device wall clock (one workgroup)
hipError_t launch_wall_clock(uint64_t* out, hipStream_t s);
hipError_t launch_advance_len(int32_t* len, const int32_t* row_offsets, const int32_t* counts, int B, int cap,
                              hipStream_t s, int32_t* save = nullptr);
hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

}  // namespace dfl
