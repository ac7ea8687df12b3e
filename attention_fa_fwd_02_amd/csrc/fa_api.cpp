// C ABI of libfa: argument validation on the host, device-architecture
// check, and dispatch to the gfx950 kernels.  See include/fa.h for the
// contract (argument meaning, layout, ownership, error behaviour).
#include "../../include/fa.h"
#include "fa_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
char g_arch[kMaxDevices][256];
int g_cus[kMaxDevices];
hipError_t g_arch_err[kMaxDevices];

size_t elem_size(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

// Head dims of the forward kernels: 64 and 128 for fp32; every multiple of 32
// from 32 to 256 for bf16 / fp16 (the backward takes the same sets).
bool fwd_head_dim_ok(int64_t D, int dtype) {
    if (D == 64 || D == 128)
        return true;
    return dtype != FA_DTYPE_F32 && D >= 32 && D <= 256 && D % 32 == 0;
}

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// Current device must be gfx950 (cached per device after the first query,
// with its compute-unit count, stored in *n_cus when asked for).
fa_status check_device(int *n_cus = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return FA_ERR_HIP;
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_err[dev] = hipGetDeviceProperties(&prop, dev);
        if (g_arch_err[dev] == hipSuccess) {
            std::strncpy(g_arch[dev], prop.gcnArchName, sizeof(g_arch[dev]) - 1);
            g_arch[dev][sizeof(g_arch[dev]) - 1] = '\0';
            g_cus[dev] = prop.multiProcessorCount;
        }
    });
    if (g_arch_err[dev] != hipSuccess)
        return FA_ERR_HIP;
    if (std::strncmp(g_arch[dev], "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;
    if (n_cus)
        *n_cus = g_cus[dev];
    return FA_OK;
}

fa::FwdArgs make_args(const void *q, const void *k, const void *v, void *o, float *lse, int64_t N,
                      int64_t D, float scale, fa_dtype dtype) {
    fa::FwdArgs args{};
    args.q = q;
    args.k = k;
    args.v = v;
    args.o = o;
    args.lse = lse;
    args.N = (int32_t)N;
    args.n_qblk = (int32_t)((N + fa::query_block(D) - 1) / fa::query_block(D));
    const float log2e = 1.44269504088896340736f;
    // c > 0 always: for |scale| * log2(e) below 1e-30 every weight exp2(c*s - m) is
    // exactly 1.0f, the same as for scale = 0, and masked scores (-inf) give
    // exp2(-inf) = 0 instead of the NaN that -inf * 0 would produce
    args.c = std::fmax(std::fabs(scale) * log2e, 1e-30f);
    args.qneg = std::signbit(scale) ? (dtype == FA_DTYPE_F32 ? 0x80000000u : 0x80008000u) : 0u;
    return args;
}

// Keys per split: whole 128-key tiles, ceil(tiles / n_splits) of them.
constexpr int64_t kSplitTile = 128;
int64_t split_keys(int64_t N, int64_t n_splits) {
    const int64_t tiles = (N + kSplitTile - 1) / kSplitTile;
    return kSplitTile * ((tiles + n_splits - 1) / n_splits);
}

bool mul_ok(uint64_t a, uint64_t b, uint64_t *out) {
    if (a != 0 && b > UINT64_MAX / a)
        return false;
    *out = a * b;
    return true;
}

// a * b < lim for a, b >= 1 and lim >= 1, without forming the product.
bool prod_below(int64_t a, int64_t b, int64_t lim) { return a <= (lim - 1) / b; }

} // namespace

namespace fa {

fa_status check_device_arch() { return check_device(); }

fa_status split_grid_ok(int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_splits) {
    const int64_t n_qblk = (N + query_block(D) - 1) / query_block(D);
    if (B * H * n_qblk * n_splits >= (int64_t(1) << 23))
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status split_enqueue(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                        int64_t N, int64_t D, float scale, int causal, fa_dtype dtype, int64_t n_splits,
                        void *workspace, fa_stream_t stream) {
    FwdArgs args = make_args(q, k, v, o, lse, N, D, scale, dtype);
    const int64_t rows = B * H * N;
    args.part_o = (float *)workspace;
    args.part_lse = (float *)((char *)workspace + (uint64_t)n_splits * (uint64_t)rows * (uint64_t)D * 4u);
    args.part_rows = rows;
    args.split_keys = (int32_t)split_keys(N, n_splits);
    args.n_splits = (int32_t)n_splits;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t err = launch_fwd((int)dtype, (int)D, causal != 0, kSplit, B * H * n_splits, args, hs);
    if (err == hipSuccess)
        err = launch_merge((int)dtype, args.part_o, args.part_lse, (int)n_splits, rows, (int)D, o, lse, hs);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

} // namespace fa

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
        return "unsupported (head dim not a multiple of 32 in 32..256 (64/128 for fp32), "
               "problem too large for one launch, too many "
               "key splits or merge parts, merge head dim not a multiple of 8 in 8..512, or "
               "device is not gfx950)";
    case FA_ERR_HIP:
        return "HIP runtime error (device query or kernel launch failed)";
    default:
        return "unknown status";
    }
}

const char *fa_fwd_kernel_name(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                               int64_t n_cus) {
    // any distinct, aligned addresses: only the sizes and flags are checked
    const uintptr_t base = uintptr_t(1) << 60, step = uintptr_t(1) << 56;
    const void *q = (const void *)base, *k = (const void *)(base + step), *v = (const void *)(base + 2 * step);
    void *o = (void *)(base + 3 * step);
    float *lse = (float *)(base + 4 * step);
    if (n_cus < 1 || fa_check_args(q, k, v, o, lse, B, H, N, D, 0.f, causal, dtype, nullptr) != FA_OK)
        return "";
    return fa::fwd_kernel_name(dtype, (int)D, causal != 0, fa::kDense,
                               fa::choose_key_groups(B * H, N, D, dtype, n_cus));
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
    if (!fwd_head_dim_ok(D, dtype))
        return FA_ERR_UNSUPPORTED;
    // size limits: rows per launch and bytes per tensor
    // B, H < 2^31 keep B * H (< 2^62) exact; the products are then compared
    // against their limits without being formed
    if (N >= (int64_t(1) << 30) || B >= (int64_t(1) << 31) || H >= (int64_t(1) << 31))
        return FA_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (BH >= (int64_t(1) << 36) || !prod_below(BH, N, int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    const int64_t n_qblk = (N + fa::query_block(D) - 1) / fa::query_block(D);
    // the dispatch grid is counted in work-items (32-bit): up to 512 per workgroup
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
    int n_cus = 0;
    if ((st = check_device(&n_cus)) != FA_OK)
        return st;
    fa::FwdArgs args = make_args(q, k, v, o, lse, N, D, scale, dtype);
    const int kg = fa::choose_key_groups(B * H, N, D, (int)dtype, n_cus);
    const int64_t qblk = fa::query_block(D) / kg;
    args.n_qblk = (int32_t)((N + qblk - 1) / qblk);
    const hipError_t err = fa::launch_fwd((int)dtype, (int)D, causal != 0, fa::kDense, B * H, args,
                                          reinterpret_cast<hipStream_t>(stream), kg);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

uint64_t fa_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_splits) {
    if (B < 1 || H < 1 || N < 1 || D < 1 || n_splits < 1)
        return 0;
    uint64_t x = 0;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &x) || !mul_ok(x, (uint64_t)N, &x) ||
        !mul_ok(x, (uint64_t)D + 1u, &x) || !mul_ok(x, (uint64_t)n_splits, &x) || !mul_ok(x, 4u, &x))
        return 0;
    return x;
}

int64_t fa_fwd_split_choose(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int64_t n_cus) {
    if (B < 1 || H < 1 || N < 1 || D < 1 || n_cus < 1 || (causal != 0 && causal != 1))
        return 0;
    const uint64_t n_qblk = ((uint64_t)N + fa::query_block(D) - 1) / fa::query_block(D);
    uint64_t wgs = 0;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &wgs) || !mul_ok(wgs, n_qblk, &wgs) || wgs >= (uint64_t)n_cus)
        return 1; // the grid already has a workgroup for every compute unit
    int64_t s = (int64_t)(((uint64_t)n_cus + wgs - 1) / wgs);
    // each split keeps >= 8 key tiles: a split's partial costs 8 bytes per row
    // and feature (fp32 written, then read by the merge) against 4 flops per
    // row, feature and key, so 1024 keys per split keep that round trip small
    // next to the split's MFMA work
    const int64_t tiles = (N + kSplitTile - 1) / kSplitTile;
    s = std::min(s, tiles / 8);
    s = std::min<int64_t>(s, FA_MAX_SPLITS);
    return std::max<int64_t>(s, 1);
}

fa_status fa_fwd_split(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                       int64_t H, int64_t N, int64_t D, float scale, int causal, fa_dtype dtype,
                       int64_t n_splits, void *workspace, uint64_t workspace_bytes,
                       fa_stream_t stream) {
    fa_status st = fa_check_args(q, k, v, o, lse, B, H, N, D, scale, causal, (int)dtype, nullptr);
    if (st != FA_OK)
        return st;
    if (n_splits < 1 || !workspace || ((uintptr_t)workspace & 15u))
        return FA_ERR_INVALID_ARG;
    if (n_splits > FA_MAX_SPLITS)
        return FA_ERR_UNSUPPORTED;
    const uint64_t need = fa_fwd_split_workspace_bytes(B, H, N, D, n_splits);
    if (need == 0 || workspace_bytes < need)
        return FA_ERR_INVALID_ARG;
    const int64_t BH = B * H;
    const uint64_t tbytes = (uint64_t)(BH * N * D) * elem_size(dtype);
    const uint64_t lbytes = (uint64_t)(BH * N) * 4u;
    if (overlaps(workspace, need, q, tbytes) || overlaps(workspace, need, k, tbytes) ||
        overlaps(workspace, need, v, tbytes) || overlaps(workspace, need, o, tbytes) ||
        overlaps(workspace, need, lse, lbytes))
        return FA_ERR_INVALID_ARG;
    if ((st = fa::split_grid_ok(B, H, N, D, n_splits)) != FA_OK)
        return st;
    if ((st = check_device()) != FA_OK)
        return st;
    return fa::split_enqueue(q, k, v, o, lse, B, H, N, D, scale, causal, dtype, n_splits, workspace, stream);
}

fa_status fa_check_varlen_args(const void *q, const void *k, const void *v, const void *o,
                               const float *lse, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_k, int64_t n_seqs, int64_t H, int64_t total_q,
                               int64_t total_k, int64_t max_seqlen_q, int64_t D, float scale, int causal,
                               int dtype, const char *arch) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k)
        return FA_ERR_INVALID_ARG;
    if (n_seqs < 1 || H < 1 || total_q < 1 || total_k < 1 || D < 1)
        return FA_ERR_INVALID_ARG;
    if (max_seqlen_q < 1 || max_seqlen_q > total_q)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || (causal != 0 && causal != 1))
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u)
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u)
        return FA_ERR_INVALID_ARG;
    if (!fwd_head_dim_ok(D, dtype))
        return FA_ERR_UNSUPPORTED;
    if (total_q >= (int64_t(1) << 30) || total_k >= (int64_t(1) << 30) || n_seqs >= (int64_t(1) << 30) ||
        H >= (int64_t(1) << 20))
        return FA_ERR_UNSUPPORTED;
    if (H * total_q >= (int64_t(1) << 36) || H * total_k >= (int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    const int64_t n_qblk = (max_seqlen_q + fa::query_block(D) - 1) / fa::query_block(D);
    if (n_seqs * H * n_qblk >= (int64_t(1) << 23))
        return FA_ERR_UNSUPPORTED;
    const uint64_t qbytes = (uint64_t)(H * total_q * D) * elem_size(dtype);
    const uint64_t kbytes = (uint64_t)(H * total_k * D) * elem_size(dtype);
    const uint64_t lbytes = (uint64_t)(H * total_q) * 4u;
    const uint64_t cbytes = (uint64_t)(n_seqs + 1) * 4u;
    const void *ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
    const uint64_t in_bytes[5] = {qbytes, kbytes, kbytes, cbytes, cbytes};
    for (int i = 0; i < 5; ++i)
        if (overlaps(o, qbytes, ins[i], in_bytes[i]) || overlaps(lse, lbytes, ins[i], in_bytes[i]))
            return FA_ERR_INVALID_ARG;
    if (overlaps(o, qbytes, lse, lbytes))
        return FA_ERR_INVALID_ARG;
    if (arch && std::strncmp(arch, "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int64_t n_seqs,
                        int64_t H, int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t D,
                        float scale, int causal, fa_dtype dtype, fa_stream_t stream) {
    fa_status st = fa_check_varlen_args(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, H, total_q,
                                        total_k, max_seqlen_q, D, scale, causal, (int)dtype, nullptr);
    if (st != FA_OK)
        return st;
    if ((st = check_device()) != FA_OK)
        return st;
    fa::FwdArgs args = make_args(q, k, v, o, lse, 0, D, scale, dtype);
    args.n_qblk = (int32_t)((max_seqlen_q + fa::query_block(D) - 1) / fa::query_block(D));
    args.cu_q = cu_seqlens_q;
    args.cu_k = cu_seqlens_k;
    args.n_heads = (int32_t)H;
    args.total_q = (int32_t)total_q;
    args.total_k = (int32_t)total_k;
    const hipError_t err = fa::launch_fwd((int)dtype, (int)D, causal != 0, fa::kVarlen, n_seqs * H, args,
                                          reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

uint64_t fa_fwd_fp8_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return 0;
    const uint64_t npad = ((uint64_t)N + 127u) / 128u * 128u;
    uint64_t x = 0;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &x) || !mul_ok(x, (uint64_t)D, &x) || !mul_ok(x, npad, &x))
        return 0;
    return x;
}

fa_status fa_check_fp8_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                            int64_t B, int64_t H, int64_t N, int64_t D, float scale, float q_descale,
                            float k_descale, float v_descale, int causal, const void *workspace,
                            uint64_t workspace_bytes, const char *arch) {
    if (!q || !k || !v || !o || !lse || !workspace)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !std::isfinite(q_descale) || !std::isfinite(k_descale) ||
        !std::isfinite(v_descale) || !std::isfinite(scale * q_descale * k_descale) ||
        (causal != 0 && causal != 1))
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)workspace) & 15u)
        return FA_ERR_INVALID_ARG;
    if ((uintptr_t)lse & 3u)
        return FA_ERR_INVALID_ARG;
    if (D < 32 || D > 256 || D % 32 != 0)
        return FA_ERR_UNSUPPORTED;
    // V^T rows are addressed with 32-bit offsets: D * Npad < 2^32
    if (N >= (int64_t(1) << 24) || B >= (int64_t(1) << 31) || H >= (int64_t(1) << 31))
        return FA_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (BH >= (int64_t(1) << 36) || !prod_below(BH, N, int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    if (BH * ((N + 255) / 256) >= (int64_t(1) << 23) || BH >= (int64_t(1) << 16))
        return FA_ERR_UNSUPPORTED;
    const uint64_t need = fa_fwd_fp8_workspace_bytes(B, H, N, D);
    if (workspace_bytes < need)
        return FA_ERR_INVALID_ARG;
    const uint64_t ib = (uint64_t)(BH * N * D);  // E4M3 inputs
    const uint64_t ob = ib * 2u;                 // bf16 output
    const uint64_t lb = (uint64_t)(BH * N) * 4u;
    const void *ins[3] = {q, k, v};
    for (int i = 0; i < 3; ++i)
        if (overlaps(o, ob, ins[i], ib) || overlaps(lse, lb, ins[i], ib) || overlaps(workspace, need, ins[i], ib))
            return FA_ERR_INVALID_ARG;
    if (overlaps(o, ob, lse, lb) || overlaps(o, ob, workspace, need) || overlaps(lse, lb, workspace, need))
        return FA_ERR_INVALID_ARG;
    if (arch && std::strncmp(arch, "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                     int64_t N, int64_t D, float scale, float q_descale, float k_descale, float v_descale,
                     int causal, void *workspace, uint64_t workspace_bytes, fa_stream_t stream) {
    fa_status st = fa_check_fp8_args(q, k, v, o, lse, B, H, N, D, scale, q_descale, k_descale, v_descale, causal,
                                     workspace, workspace_bytes, nullptr);
    if (st != FA_OK)
        return st;
    if ((st = check_device()) != FA_OK)
        return st;
    fa::Fp8Args args{};
    args.q = q;
    args.k = k;
    args.v = v;
    args.vt = workspace;
    args.o = o;
    args.lse = lse;
    args.N = (int32_t)N;
    args.Npad = (int32_t)((N + 127) / 128 * 128);
    args.n_qblk = (int32_t)((N + 255) / 256);
    const float s = scale * q_descale * k_descale;
    args.c = std::fmax(std::fabs(s) * 1.44269504088896340736f, 1e-30f);
    args.v_descale = v_descale;
    args.qneg = std::signbit(s) ? 0x80808080u : 0u;
    const hipError_t err = fa::launch_fp8((int)D, causal != 0, B * H, args, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

uint64_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return 0;
    uint64_t x = 0;
    if (!mul_ok((uint64_t)B, (uint64_t)H, &x) || !mul_ok(x, (uint64_t)N, &x) || !mul_ok(x, 4u, &x))
        return 0;
    return x;
}

fa_status fa_check_bwd_args(const void *q, const void *k, const void *v, const void *o, const void *dout,
                            const float *lse, const void *dq, const void *dk, const void *dv, int64_t B,
                            int64_t H, int64_t N, int64_t D, float scale, int causal, int dtype,
                            const void *workspace, uint64_t workspace_bytes, const char *arch) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || D < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || (causal != 0 && causal != 1))
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
        return FA_ERR_INVALID_ARG;
    if ((uintptr_t)lse & 3u)
        return FA_ERR_INVALID_ARG;
    if (!fwd_head_dim_ok(D, dtype))
        return FA_ERR_UNSUPPORTED;
    // B, H < 2^31 keep B * H (< 2^62) exact; the products are then compared
    // against their limits without being formed
    if (N >= (int64_t(1) << 30) || B >= (int64_t(1) << 31) || H >= (int64_t(1) << 31))
        return FA_ERR_UNSUPPORTED;
    const int64_t BH = B * H;
    if (BH >= (int64_t(1) << 36) || !prod_below(BH, N, int64_t(1) << 36))
        return FA_ERR_UNSUPPORTED;
    if (BH * ((N + 127) / 128) >= (int64_t(1) << 23))
        return FA_ERR_UNSUPPORTED;
    const uint64_t need = fa_bwd_workspace_bytes(B, H, N, D);
    if (workspace_bytes < need)
        return FA_ERR_INVALID_ARG;
    const uint64_t tbytes = (uint64_t)(BH * N * D) * elem_size(dtype);
    const uint64_t lbytes = (uint64_t)(BH * N) * 4u;
    const void *ins[6] = {q, k, v, o, dout, lse};
    const uint64_t in_bytes[6] = {tbytes, tbytes, tbytes, tbytes, tbytes, lbytes};
    const void *outs[4] = {dq, dk, dv, workspace};
    const uint64_t out_bytes[4] = {tbytes, tbytes, tbytes, need};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
                return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
                return FA_ERR_INVALID_ARG;
    }
    if (arch && std::strncmp(arch, "gfx950", 6) != 0)
        return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

fa_status fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
                 const float *lse, void *dq, void *dk, void *dv, int64_t B, int64_t H, int64_t N, int64_t D,
                 float scale, int causal, fa_dtype dtype, void *workspace, uint64_t workspace_bytes,
                 fa_stream_t stream) {
    fa_status st = fa_check_bwd_args(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, D, scale, causal, (int)dtype,
                                     workspace, workspace_bytes, nullptr);
    if (st != FA_OK)
        return st;
    if ((st = check_device()) != FA_OK)
        return st;
    fa::BwdArgs args{};
    args.q = q;
    args.k = k;
    args.v = v;
    args.o = o;
    args.dout = dout;
    args.lse = lse;
    args.delta = (float *)workspace;
    args.dq = dq;
    args.dk = dk;
    args.dv = dv;
    args.N = (int32_t)N;
    args.c2 = scale * 1.44269504088896340736f;
    args.scale = scale;
    const hipError_t err = fa::launch_bwd((int)dtype, (int)D, causal != 0, B * H, args,
                                          reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_lse_merge(const float *part_o, const float *part_lse, int64_t n_parts, int64_t rows,
                       int64_t D, void *o, float *lse, fa_dtype dtype, fa_stream_t stream) {
    if (!part_o || !part_lse || !o || !lse)
        return FA_ERR_INVALID_ARG;
    if (n_parts < 1 || rows < 1 || D < 1)
        return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    if ((((uintptr_t)part_o | (uintptr_t)o) & 15u) || (((uintptr_t)part_lse | (uintptr_t)lse) & 3u))
        return FA_ERR_INVALID_ARG;
    if (n_parts > 1024 || D < 8 || D > 512 || (D % 8) != 0)
        return FA_ERR_UNSUPPORTED;
    if (rows >= (int64_t(1) << 40) || n_parts * rows * D >= (int64_t(1) << 40))
        return FA_ERR_UNSUPPORTED;
    const uint64_t pobytes = (uint64_t)(n_parts * rows * D) * 4u;
    const uint64_t plbytes = (uint64_t)(n_parts * rows) * 4u;
    const uint64_t obytes = (uint64_t)(rows * D) * elem_size(dtype);
    const uint64_t lbytes = (uint64_t)rows * 4u;
    if (overlaps(o, obytes, lse, lbytes) || overlaps(o, obytes, part_o, pobytes) ||
        overlaps(o, obytes, part_lse, plbytes) || overlaps(lse, lbytes, part_o, pobytes) ||
        overlaps(lse, lbytes, part_lse, plbytes))
        return FA_ERR_INVALID_ARG;
    fa_status st = check_device();
    if (st != FA_OK)
        return st;
    const hipError_t err = fa::launch_merge((int)dtype, part_o, part_lse, (int)n_parts, rows, (int)D, o,
                                            lse, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

} // extern "C"
