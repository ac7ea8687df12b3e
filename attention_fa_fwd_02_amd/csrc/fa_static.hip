// fa_fwd_split_static: the key-split forward pass with its partial results in
// a library-held device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is a file-scope device variable: the code object
// loader gives every device that loads the library its own copy, at its own
// address, which stays allocated until the process ends.  In host code the
// name `scratch` is only a host-side stand-in for that symbol; its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels.
//
// The kernels are those of fa_fwd_split (the split kernel, then the merge).
// Nothing has to start at zero: every split writes its lse for every row it
// covers (-inf when the split holds none of the row's keys) and the merge
// never reads the O partial of such a split, so no clearing pass is needed.
// All calls on one device share its array: calls that overlap on one device
// (different streams, or other threads) race on it.
#include "fa_internal.h"

#include <mutex>

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's copy of `scratch` (looked up on the
// first call on that device).
fa_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = (g_scratch_err[dev] == hipSuccess) ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
        return FA_ERR_HIP;
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

} // namespace

extern "C" fa_status fa_fwd_split_static(const void *q, const void *k, const void *v, void *o, float *lse,
                                         int64_t B, int64_t H, int64_t N, int64_t D, float scale, int causal,
                                         fa_dtype dtype, int64_t n_splits, fa_stream_t stream) {
    fa_status st = fa_check_args(q, k, v, o, lse, B, H, N, D, scale, causal, (int)dtype, nullptr);
    if (st != FA_OK)
        return st;
    if (n_splits < 1)
        return FA_ERR_INVALID_ARG;
    if (n_splits > FA_MAX_SPLITS)
        return FA_ERR_UNSUPPORTED;
    const uint64_t need = fa_fwd_split_workspace_bytes(B, H, N, D, n_splits);
    if (need == 0 || need > (uint64_t)FA_STATIC_SCRATCH_BYTES)
        return FA_ERR_UNSUPPORTED;
    if ((st = fa::split_grid_ok(B, H, N, D, n_splits)) != FA_OK)
        return st;
    if ((st = fa::check_device_arch()) != FA_OK)
        return st;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != FA_OK)
        return st;
    return fa::split_enqueue(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, n_splits, ws, stream);
}
