// rns_gemm_noalloc: rns_gemm with its workspace in a fixed device array of
// this library, for callers that cannot allocate device memory.
//
// The array `scratch` below is a file-scope __device__ object: every GPU the
// library runs on holds its own copy, at its own address, from the time the
// code object is loaded there until the process ends.  In host code the name
// `scratch` is only a host-side stand-in, never a device address; the device
// address of the current GPU's copy is taken once per device with
// hipGetSymbolAddress and kept, and only that address is passed on.
//
// The entry point allocates nothing: no hipMalloc, hipFree or allocating
// library call.  The kernels it launches are exactly rns_gemm's, which write
// every byte of the workspace they later read (operand planes with their
// padding, the status words, the product planes, the split-tile residues), so
// the array needs no clearing between calls.  Calls on one GPU share that
// GPU's array: two calls whose work overlaps on one GPU (two streams, or two
// host threads) race on it and must be ordered by the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rns_internal.h"

namespace rns {
namespace {

constexpr size_t kScratchBytes = RNS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on
// that device, then cached).
int scratch_on_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RNS_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return RNS_E_ARG;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RNS_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RNS_OK;
}

}  // namespace
}  // namespace rns

extern "C" int rns_gemm_noalloc(const rns_plan_t *plan, int64_t M, int64_t N, int64_t K,
                                const int64_t *A, int32_t a_limbs, const int64_t *B, int32_t b_limbs,
                                int64_t *C, int32_t c_limbs, hipStream_t stream) {
    size_t need = 0;
    int rc = rns_workspace_size(plan, M, N, K, 0, &need);   // validates the plan and the sizes
    if (rc) return rc;
    if (need > rns::kScratchBytes) return RNS_E_SCRATCH;
    void *ws = nullptr;
    rc = rns::scratch_on_current_device(&ws);
    if (rc) return rc;
    return rns_gemm(plan, M, N, K, A, a_limbs, B, b_limbs, C, c_limbs, ws, rns::kScratchBytes, stream);
}
