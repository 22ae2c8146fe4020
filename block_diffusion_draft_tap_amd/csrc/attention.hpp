// Split-K non-causal block attention (see attention.hip).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dfl {

// The block's keys (gamma of them) form one 32-key unit of the attention kernels,
// and the block values travel in one [hd][32] tile per (sequence, kv head).
constexpr int kAttnMaxGamma = 32;

struct AttnParams {
    const void* qkv;       // [B*gamma][qkv_ld]: Q cols [0, hq hd), K_b cols, then V_b cols
                           // (fp32 with fp32 caches; bf16 with bf16 caches, V_b then in vblk)
    const uint16_t* vblk;  // bf16 caches: block values head-dim major [B][hkv][hd][32], keys < gamma
    int64_t qkv_ld;
    const void* kcache;    // this layer's keys   [B][hkv][cap][hd]
    const void* vcache;    // this layer's values [B][hkv][cap/32][hd][32] (bf16; fp32: [B][hkv][hd][cap])
    const int32_t* len;    // [B] context rows per sequence
    int B, hq, hkv, hd, gamma, cap, nsplit, kv_f32;
    int window;            // attend to the last `window` context keys of each sequence; 0 = all
    int nparts;            // partial results per (b, head): nsplit workgroups x parts each
    float scale;
    float* part;           // [B][hq][nparts][gamma][hd+2]  (o, running max, running sum)
    float* out;            // O [B*gamma][out_ld], head h at columns h*hd
    int64_t out_ld;
    int round_out;         // 1: O is rounded and stored as bf16 (out reinterpreted as uint16)
    uint64_t* stamps;      // set by the launcher when the launch is traced: (start, end) wall clock per workgroup
};

// Workgroups per (sequence, kv head) and partial results per (sequence, head)
// for a cache of `cap` rows, `pairs` (sequence, kv head) pairs and `rows` query
// rows per kv head at head dim `hd` (one partial per workgroup); the workspace holds
// B*hq*nparts*gamma*(hd+2) floats.
void attention_splits(int cap, int gamma, int kv_f32, int pairs, int rows, int hd, int* nsplit, int* nparts);
// context keys a sequence can attend in a cache of `cap` rows under a window (0: cap): the
// window plus the part of its first 32-key chunk before it; pass it as attention_splits' cap
int attn_span(int cap, int window);
hipError_t launch_attention(const AttnParams& p, hipStream_t s);
int attention_max_rows(int kv_f32);

}  // namespace dfl
