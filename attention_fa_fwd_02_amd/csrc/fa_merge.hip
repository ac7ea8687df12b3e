// Merge of key-split partial results (gfx950).
//
// Part p of a row is the attention output over one key set, already
// normalised (O_p = sum_j w_j v_j / sum_j w_j over the set) together with
// that set's logsumexp lse_p.  For disjoint key sets the result over their
// union follows from the online-softmax merge of a running state with a new
// block (KingOfEgg's FlashAttention v1 post, dandandamowang.xyz, section
// 4.3: new maximum, old terms rescaled by exp(m_old - m_new)), with each
// part's (m, l) pair entering as lse_p = m_p + ln l_p:
//   m = max_p lse_p,  w_p = exp(lse_p - m),  O = sum_p w_p O_p / sum_p w_p,
//   lse = m + ln sum_p w_p.
// A part with lse_p = -inf saw no key: weight 0, and its O_p is not read.
// A row whose parts are all -inf gets O = 0 and lse = -inf.
//
// Memory-bound: every partial element is read once and every output
// element written once.  One lane handles 8 consecutive features of one row
// (two 16-byte loads per part, one 16-byte store for 16-bit outputs), so the
// lanes of a block cover whole consecutive rows of a part per load.
#include "fa_internal.h"

namespace fa {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2m = 0.693147180559945309f;

template <int OUT> // 0: fp32, 1: bf16, 2: fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack2(float x, float y) {
    f32x2 v = {x, y};
    if constexpr (OUT == 1)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// One block handles rows_pb = 256 / (D/8) consecutive rows: thread t merges
// features 8c .. 8c + 7 (c = t % (D/8)) of row t / (D/8); blocks stride over
// the rows.
template <int OUT>
__global__ __launch_bounds__(kMergeThreads) void fa_merge_kernel(const float *__restrict__ part_o,
                                                                 const float *__restrict__ part_lse,
                                                                 int n_parts, int64_t rows, int D,
                                                                 void *__restrict__ o,
                                                                 float *__restrict__ lse) {
    const int d8 = D / 8;
    const int rows_pb = kMergeThreads / d8;
    const int t = threadIdx.x;
    const int lr = t / d8, c = t - lr * d8;
    if (lr >= rows_pb) // the last t % d8 threads of a block have no row
        return;
    for (int64_t row = (int64_t)blockIdx.x * rows_pb + lr; row < rows; row += (int64_t)gridDim.x * rows_pb) {
        float m = -INFINITY;
        for (int p = 0; p < n_parts; ++p)
            m = fmaxf(m, part_lse[p * rows + row]);
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        float out_lse = -INFINITY;
        if (m != -INFINITY) {
            float l = 0.f;
            for (int p = 0; p < n_parts; ++p) {
                const float lp = part_lse[p * rows + row];
                if (lp == -INFINITY)
                    continue;
                const float w = __builtin_amdgcn_exp2f((lp - m) * kLog2e);
                const f32x4 *src = (const f32x4 *)(part_o + (p * rows + row) * D + 8 * c);
                const f32x4 x0 = src[0], x1 = src[1];
                l += w;
                acc0 += w * x0;
                acc1 += w * x1;
            }
            const float inv = 1.0f / l;
            acc0 *= inv;
            acc1 *= inv;
            out_lse = m + __builtin_amdgcn_logf(l) * kLn2m;
        }
        if constexpr (OUT == 0) {
            f32x4 *dst = (f32x4 *)((float *)o + row * D + 8 * c);
            dst[0] = acc0;
            dst[1] = acc1;
        } else {
            const u32x4 w = {pack2<OUT>(acc0[0], acc0[1]), pack2<OUT>(acc0[2], acc0[3]),
                             pack2<OUT>(acc1[0], acc1[1]), pack2<OUT>(acc1[2], acc1[3])};
            *(u32x4 *)((uint16_t *)o + row * D + 8 * c) = w;
        }
        if (c == 0)
            lse[row] = out_lse;
    }
}

} // namespace

hipError_t launch_merge(int dtype, const float *part_o, const float *part_lse, int n_parts,
                        int64_t rows, int D, void *o, float *lse, hipStream_t stream) {
    const int rows_pb = kMergeThreads / (D / 8);
    // enough workgroups to fill the device several times over; the kernel
    // strides over the rest
    const int64_t want = (rows + rows_pb - 1) / rows_pb;
    const unsigned nwg = (unsigned)(want < (int64_t(1) << 16) ? want : (int64_t(1) << 16));
    if (dtype == 0)
        hipLaunchKernelGGL(fa_merge_kernel<0>, dim3(nwg), dim3(kMergeThreads), 0, stream, part_o,
                           part_lse, n_parts, rows, D, o, lse);
    else if (dtype == 1)
        hipLaunchKernelGGL(fa_merge_kernel<1>, dim3(nwg), dim3(kMergeThreads), 0, stream, part_o,
                           part_lse, n_parts, rows, D, o, lse);
    else
        hipLaunchKernelGGL(fa_merge_kernel<2>, dim3(nwg), dim3(kMergeThreads), 0, stream, part_o,
                           part_lse, n_parts, rows, D, o, lse);
    return hipGetLastError();
}

} // namespace fa
