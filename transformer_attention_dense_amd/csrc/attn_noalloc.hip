// attn_fwd_ex_noalloc: attn_fwd_ex without any allocation, for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). Declared in include/attn_dense.h.
//
// The split-KV partial results go to `scratch`, a file-scope device array of
// kScratchBytes that every GPU the library runs on holds until the process ends. In
// host code the array's name is only a host-side stand-in: its device address is
// looked up once per device with hipGetSymbolAddress (each GPU has its own copy at its
// own address) and only that address is handed to the kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn_dense.h"
#include "attn_launch.h"

namespace {

constexpr long long kScratchBytes = 64LL << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (null on failure).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int attn_fwd_ex_noalloc(const void* q, const void* k0, const void* v0, int n0, const void* k1,
                        const void* v1, int n1, void* out, int B, int Nq, int H, int D,
                        int num_splits, int waves, void* stream) {
    if ((long long)n0 + n1 < 1 || n0 < 0 || n1 < 0) return ATTN_ERR_SHAPE;
    int splits = 0;
    long long need = 0;
    const int rc = attn_plan(B, Nq, n0 + n1, H, D, num_splits, waves, &splits, nullptr,
                             nullptr, &need);
    if (rc != ATTN_OK) return rc;
    if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;
    attn::FixedWorkspace fixed = {nullptr, kScratchBytes};
    if (need > 0) {
        fixed.ptr = scratch_address();
        if (!fixed.ptr) return ATTN_ERR_HIP;
    }
    return attn::run_fwd(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D, num_splits, waves,
                         stream, &fixed);
}

}  // extern "C"
