// C ABI of libfa: argument validation on the host, device-architecture
// check, and dispatch to the gfx950 kernels.  See include/fa.h for the
// contract (argument meaning, layout, ownership, error behaviour).
#include "../../include/fa.h"
#include "fa_internal.h"

#include <cmath>
#include <cstring>
#include <mutex>

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
char g_arch[kMaxDevices][256];
hipError_t g_arch_err[kMaxDevices];

size_t elem_size(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

} // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char *fa_status_string(int status) {
    switch (status) {
    case FA_OK:
        return "ok";
    case FA_ERR_INVALID_ARG:
        return "invalid argument (null pointer, non-positive size, non-finite scale, bad causal or "
               "dtype, misaligned pointer, or outputs overlapping inputs)";
    case FA_ERR_UNSUPPORTED:
        return "unsupported (head dim not 64/128, problem too large for one launch, or device is "
               "not gfx950)";
    case FA_ERR_HIP:
        return "HIP runtime error (device query or kernel launch failed)";
    default:
        return "unknown status";
    }
}

fa_status fa_check_args(const void *q, const void *k, const void *v, const void *o,
                        const float *lse, int64_t B, int64_t H, int64_t N, int64_t D,
                        float scale, int causal, int dtype, const char *arch) {
    if (!q || !k || !v || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale))
        return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1)
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
        return FA_ERR_INVALID_ARG;
    if ((uintptr_t)lse & 3u)
        return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128)
        return FA_ERR_UNSUPPORTED;
    // size limits: rows per launch and bytes per tensor
    if (N >= (int64_t(1) << 30) || B >= (int64_t(1) << 36) || H >= (int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (BH >= (int64_t(1) << 36) || BH * N >= (int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    const int64_t n_qblk = (N + fa::kQueryBlock - 1) / fa::kQueryBlock;
    // the dispatch grid is counted in work-items (32-bit): 512 per workgroup
    if (BH * n_qblk >= (int64_t(1) << 23))
        return FA_ERR_UNSUPPORTED;
    const uint64_t tbytes = (uint64_t)(BH * N * D) * elem_size(dtype);
    const uint64_t lbytes = (uint64_t)(BH * N) * 4u;
    if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
        overlaps(o, tbytes, v, tbytes) || overlaps(o, tbytes, lse, lbytes) ||
        overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, k, tbytes) ||
        overlaps(lse, lbytes, v, tbytes))
        return FA_ERR_INVALID_ARG;
    if (arch && std::strncmp(arch, "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                 int64_t H, int64_t N, int64_t D, float scale, int causal, fa_dtype dtype,
                 fa_stream_t stream) {
    fa_status st = fa_check_args(q, k, v, o, lse, B, H, N, D, scale, causal, (int)dtype, nullptr);
    if (st != FA_OK)
        return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA_ERR_HIP;
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_err[dev] = hipGetDeviceProperties(&prop, dev);
        if (g_arch_err[dev] == hipSuccess) {
            std::strncpy(g_arch[dev], prop.gcnArchName, sizeof(g_arch[dev]) - 1);
            g_arch[dev][sizeof(g_arch[dev]) - 1] = '\0';
        }
    });
    if (g_arch_err[dev] != hipSuccess)
        return FA_ERR_HIP;
    if (std::strncmp(g_arch[dev], "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;

    fa::FwdArgs args;
    args.q = q;
    args.k = k;
    args.v = v;
    args.o = o;
    args.lse = lse;
    args.N = (int32_t)N;
    args.n_qblk = (int32_t)((N + fa::kQueryBlock - 1) / fa::kQueryBlock);
    const float log2e = 1.44269504088896340736f;
    // c > 0 always: for |scale| * log2(e) below 1e-30 every weight exp2(c*s - m) is
    // exactly 1.0f, the same as for scale = 0, and masked scores (-inf) give
    // exp2(-inf) = 0 instead of the NaN that -inf * 0 would produce
    args.c = std::fmax(std::fabs(scale) * log2e, 1e-30f);
    args.qneg = std::signbit(scale) ? (dtype == FA_DTYPE_F32 ? 0x80000000u : 0x80008000u) : 0u;
    const hipError_t err = fa::launch_fwd((int)dtype, (int)D, causal != 0, B * H, args,
                                          reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

} // extern "C"
