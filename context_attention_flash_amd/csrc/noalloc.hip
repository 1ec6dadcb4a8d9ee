// ring_attn_bwd_noalloc: the backward of the rank share with its workspace in
// a static device array, for callers that cannot allocate device memory.
//
// The array below is reserved on every GPU the library runs on, at module
// load, and kept until the process ends.  Host code never passes its name to a
// kernel or a copy (in host code the name is only a stand-in): the address of
// each device's copy is taken once per device with hipGetSymbolAddress and
// used from then on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "abi_internal.h"
#include "ring_attn.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 128;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (looked up once per device).
int scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RA_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RA_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RA_OK;
}

}  // namespace

extern "C" {

int64_t ring_attn_noalloc_scratch_bytes(void) { return (int64_t)kScratchBytes; }

int ring_attn_bwd_noalloc(const ring_attn_desc* desc, const void* dout, const void* q,
                          const void* k, const void* v, const void* out, const float* lse,
                          const int32_t* cu_seqlens, float* dq, float* dk, float* dv,
                          void* stream) {
    const int64_t need = ra::bwd_need_bytes(desc);
    if (need < 0) return (int)need;
    if (need > (int64_t)kScratchBytes) return RA_E_SCRATCH;
    void* ws = nullptr;
    const int rc = scratch_of_current_device(&ws);
    if (rc != RA_OK) return rc;
    // the backward writes every part of its workspace before reading it, so
    // the scratch left by an earlier call needs no clearing
    return ra::bwd_impl(desc, dout, q, k, v, out, lse, cu_seqlens, dq, dk, dv, ws, kScratchBytes,
                        stream, /*build_plan=*/false);
}

}  // extern "C"
