// Greedy verification without a caller workspace, for callers that cannot
// allocate (code under graph capture, serving loops that forbid allocation).
//
// The verify kernels' partial results (per verify row and vocabulary split, a
// (max, index) pair) live in a file-scope device array instead of a workspace
// argument. Each device holds its own copy of the array from module load to the
// end of the process; its address on a device is looked up once, on the first
// call with that device current, and kept per device. Calls that overlap on one
// device share the array and race; calls ordered on one stream do not. Nothing in
// it has to start at zero: every pair is written before it is read.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/dflash.h"
#include "head.hpp"

namespace dfl {
int api_gate();               // DFLASH_OK, or DFLASH_DECLINED (kill switch, not gfx950)
void api_count_invocation();  // dflash_invocations() bookkeeping
}  // namespace dfl

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // 1 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// the device address of this device's copy of `scratch` (looked up once per device)
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_verify_noalloc_max_bytes(void) { return kScratchBytes; }

int dflash_verify_greedy_noalloc(const float* target_logits, const int32_t* draft_ids, int32_t B, int32_t gamma,
                                 int32_t V, int32_t* accepted, int32_t* committed, int32_t* ids, int32_t* next_anchor,
                                 void* stream) {
    if (!target_logits || !draft_ids || !accepted || !committed || !ids) return DFLASH_EINVAL;
    if (B <= 0 || gamma <= 0 || V <= 0) return DFLASH_EINVAL;
    if (gamma + 1 > 64) return DFLASH_DECLINED;
    if (reinterpret_cast<uintptr_t>(target_logits) & 15) return DFLASH_DECLINED;
    const size_t need = dflash_verify_workspace_bytes(B, gamma, V);
    if (need == 0 || need > kScratchBytes) return DFLASH_ENOSPC;
    const int g = dfl::api_gate();
    if (g != DFLASH_OK) return g;
    void* base = nullptr;
    const int rc = scratch_on_current_device(&base);
    if (rc != DFLASH_OK) return rc;
    char* c = static_cast<char*>(base);
    float* pv = reinterpret_cast<float*>(c);
    int32_t* pi = reinterpret_cast<int32_t*>(c + need / 2);
    if (dfl::launch_verify(target_logits, draft_ids, B, gamma, V, accepted, committed, ids, next_anchor, pv, pi,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
        return DFLASH_EHIP;
    dfl::api_count_invocation();
    return DFLASH_OK;
}

}  // extern "C"
