// Device building blocks of the 16-bit forward kernels in fa_fwd.hip (the
// one-barrier and the ping-pong kernel): the Q operand load, the masks of a
// transposed score tile, the online softmax of one tile against the running
// reference, and the O epilogue.  The layouts are those of the
// v_mfma_f32_32x32x16 S^T = K Q^T tiles: lane (r, g) holds query row r of a
// 32-row block, and accumulator entry i of lane half g is key 2i + g of a
// 32-key block.
#pragma once
#include "fa_device.h"

namespace fa {
namespace {

// Q^T operand of the score MFMA: lane (r, g) holds q_qi[16c + 8g .. +7] for
// step c (zero for rows at or past Nq); qneg flips the sign bits when the
// scale is negative.
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qf)[D / 16], const uint16_t *__restrict__ Q, int qi, int Nq, int g,
                                       uint32_t qneg) {
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
        qf[cc] = qi < Nq ? *(const u32x4 *)(Q + (int64_t)qi * D + 16 * cc + 8 * g) : zero4;
        qf[cc] ^= qneg;
    }
}

// Masks of one S^T tile: entry (kb, i) of lane half g is key k0 + 32 kb + 2 i + g.
// mask_keys: keys at or past Nk, and (causal) keys after query qi + coff, get
// score -inf.  mask_below: the same through one per-lane bound, lim = (first
// invisible key) - k0 - g, compared with the compile-time 32 kb + 2 i, which
// keeps the mask free of per-entry registers.
template <int KB, bool CAUSAL>
__device__ __forceinline__ void mask_keys(f32x16 (&s)[KB], int k0, int Nk, int qi, int coff, int g) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 2 * i + g;
            const bool vis = key < Nk && (!CAUSAL || key <= qi + coff);
            s[kb][i] = vis ? s[kb][i] : -INFINITY;
        }
}
template <int KB>
__device__ __forceinline__ void mask_below(f32x16 (&s)[KB], int lim) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s[kb][i] = (32 * kb + 2 * i < lim) ? s[kb][i] : -INFINITY;
}

// Online softmax of one S^T tile against the running reference m_run
// (log2 domain, c = |scale| log2 e): P~ = exp2(s c - m_run), summed into
// l_run in fp32 and rounded into pk for the PV MFMA (pk[kb][j] holds entries
// 2j, 2j + 1 of block kb).  The reference moves only when it is missing (the
// first tile: no optimistic pass then) or some row's share of the tile's sum
// exceeds 2^kTau, i.e. a score beat the reference by more than kTau (log2
// units); P~ <= 2^kTau keeps fp32 far from overflow.  Then O and l are
// rescaled to the row maximum and P~ is redone.
template <typename E, int KB, int OB>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[KB], uint32_t (&pk)[KB][8], f32x16 (&o)[OB],
                                               float &m_run, float &l_run, float c) {
    constexpr float kLimit = 256.0f; // 2^kTau, kTau = 8
    float lt = 0.f;
    auto exps = [&](float m_ref) __attribute__((always_inline)) {
        lt = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, -m_ref));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], c, -m_ref));
                lt += p0 + p1;
                pk[kb][i >> 1] = E::pack(p0, p1);
            }
    };
    bool move = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0;
    if (!move) {
        exps(m_run);
        move = __builtin_amdgcn_ballot_w64(!(lt <= kLimit)) != 0;
    }
    if (move) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                mx = fmaxf(mx, s[kb][i]);
        const float m_new = fmaxf(m_run, pair_max(mx) * c);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < OB; ++b)
            o[b] *= alpha;
        m_run = m_new;
        exps(m_run == -INFINITY ? 0.f : m_run);
    }
    l_run += lt;
}

// Epilogue of one wave: O / l rounded to the element type into the wave's
// private LDS rows ow (pitch 2D + 16 bytes; o[b][i] is feature
// 32b + 8(i/4) + 4g + i%4 of query qi), lse = (m + log2 l) ln 2, then the
// rows are stored as 16-byte chunks covering whole cache lines.  Every wave
// of the workgroup calls it (it holds a workgroup barrier).
template <typename E, int D>
__device__ __forceinline__ void store_o(const f32x16 (&o)[D / 32], float inv, float m_run, float l_tot,
                                        lds_char *ow, uint16_t *__restrict__ O, float *__restrict__ LSE, int q0w,
                                        int Nq, int lane) {
    constexpr int OB = D / 32, KCH = D / 8, OP = 2 * D + 16;
    const int r = lane & 31, g = lane >> 5, qi = q0w + r;
    if (q0w < Nq) {
#pragma unroll
        for (int b = 0; b < OB; ++b)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const u32x2 w = {E::pack(o[b][4 * a4] * inv, o[b][4 * a4 + 1] * inv),
                                 E::pack(o[b][4 * a4 + 2] * inv, o[b][4 * a4 + 3] * inv)};
                *(__attribute__((address_space(3))) u32x2 *)(ow + r * OP + (32 * b + 8 * a4 + 4 * g) * 2) = w;
            }
        if (g == 0 && qi < Nq)
            LSE[qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
    __syncthreads();
    if (q0w < Nq) {
        constexpr int kChunks = 32 * KCH; // 16-byte chunks in the wave's 32 rows
#pragma unroll
        for (int j = 0; j < kChunks / 64; ++j) {
            const int ch = 64 * j + lane;
            const int row = ch / KCH, col = ch % KCH;
            const int q = q0w + row;
            const u32x4 val = *(const __attribute__((address_space(3))) u32x4 *)(ow + row * OP + col * 16);
            if (q < Nq)
                *(u32x4 *)(O + (int64_t)q * D + col * 8) = val;
        }
    }
}

} // namespace
} // namespace fa
