// FP8 (OCP E4M3) attention forward pass for gfx950.
//
// The same tiled online-softmax forward pass as the 16-bit kernels, with
// both contractions on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands,
// fp32 accumulation, unit block scales): S^T = K Q^T over the head dim and
// O^T += V^T P~^T over the keys, with P~ rounded to E4M3.  Per-tensor
// descale factors multiply the stored values: the scores use
// c = |scale * q_descale * k_descale| * log2(e) in the one FMA before exp2,
// and v_descale joins the final 1/l.  FP8 Tensor Core paths are the FA-3
// direction the pages name (lesson 13 "GPU 内核与 FlashAttention",
// hpc.payai.win, answer to Q3).
//
// Operand layouts (32x32x64: a lane holds 32 consecutive k-values, k = 32 g
// + 0..31 for lane half g; verified on the device):
//   S^T: A = K rows, B = Q rows (registers).  The K tile sits in LDS in MFMA
//        row order: LDS row R of a 32-key block holds key 16 ((R/4)%2) +
//        4 (R/8) + R%4, so accumulator entry e of lane half g is key 16 g + e.
//   O^T: A = V^T rows (feature-major), B = P~: for a 64-key step, lane half g
//        holds its 16 keys of each of the two 32-key blocks, i.e. keys
//        16 g + 0..15 and 32 + 16 g + 0..15, which are two 16-byte runs of a
//        V^T row.  V^T comes from fa_fp8_vt_kernel, which transposes V once
//        per call into the caller's workspace (keys padded with zeros to a
//        whole key tile).
//
// Schedule: the ping-pong order of the 16-bit dense kernel.  A wave's tile
// work is split into an MFMA phase (PV of the previous tile, then the
// scores of this one) and a softmax phase; waves 4..7 run one phase behind
// waves 0..3, so the two waves of a SIMD overlap one's MFMAs with the
// other's exponentials.  V^T tiles trail K tiles by one, in two K and two
// V^T stages.
#include "fa_device.h"
#include "fa_internal.h"

#include <type_traits>

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Waves = 8;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8Rows = 32 * kF8Waves; // query rows per workgroup
constexpr int kScaleOne = 127;          // E8M0 block scale 2^0
constexpr int kF8Ahead = 2;             // MFMAs whose LDS operands are read ahead

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, kScaleOne);
}

// Direct global -> LDS load of 16 bytes per lane with a scalar offset added.
__device__ __forceinline__ void load_lds_16s(const void *base, uint32_t bytes, uint32_t voff, uint32_t soff,
                                             lds_char *lds) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// Key of LDS row R of a 32-row K block (MFMA row order, see above).
__device__ __forceinline__ int k_row_key(int R) {
    return 16 * ((R >> 2) & 1) + 4 * (R >> 3) + (R & 3);
}

// ----------------------------------------------------------------------------
// V [BH][N][D] -> V^T [BH][D][Npad], keys N .. Npad-1 zero
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fa_fp8_vt_kernel(const uint8_t *__restrict__ V, uint8_t *__restrict__ Vt,
                                                        int N, int Npad) {
    constexpr int TK = 64;              // keys per block
    constexpr int CH = TK * D / 16;     // 16-byte chunks of the tile (both ways)
    __shared__ uint8_t tile[TK][D + 4];
    const int bh = blockIdx.y;
    const int k0 = blockIdx.x * TK;
    const uint8_t *src = V + (int64_t)bh * N * D;
    uint8_t *dst = Vt + (int64_t)bh * D * Npad;
    for (int ch = threadIdx.x; ch < CH; ch += 256) {
        const int key = ch / (D / 16), c = ch % (D / 16);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k0 + key < N)
            v = *(const u32x4 *)(src + (int64_t)(k0 + key) * D + 16 * c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            *(uint32_t *)&tile[key][16 * c + 4 * w] = v[w];
        }
    }
    __syncthreads();
    for (int ch = threadIdx.x; ch < CH; ch += 256) {
        const int f = ch / (TK / 16), c = ch % (TK / 16); // feature row, 16-key chunk
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t x = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                x |= (uint32_t)tile[16 * c + 4 * w + b][f] << (8 * b);
            v[w] = x;
        }
        *(u32x4 *)(dst + (int64_t)f * Npad + k0 + 16 * c) = v;
    }
}

// ----------------------------------------------------------------------------
// forward kernel
// ----------------------------------------------------------------------------
template <int D>
struct F8Cfg {
    // keys per tile: 128, or 64 at D = 256 (the O accumulators take 128
    // registers there, and two waves per SIMD need the score tile to shrink)
    static constexpr int BC = D > 192 ? 64 : 128;
    static constexpr int KP = D + 16;        // K row pitch (bytes)
    static constexpr int VTP = BC + 16;      // V^T row pitch (bytes)
    static constexpr int NK = BC * KP / 1024;
    // 1 KB blocks of a V^T tile; when D is an odd multiple of 32 the last
    // block is half spare (its slots lie past the last feature row and read
    // zeros)
    static constexpr int NV = (D * VTP + 1023) / 1024;
    static_assert(NK * 1024 == BC * KP, "K tiles are whole 1 KB blocks");
    static constexpr int LPW = (NK + NV + kF8Waves - 1) / kF8Waves; // loads per wave and tile
    static constexpr int OP = 2 * D + 16;    // bf16 O staging pitch
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF8Threads) void fa_fwd_fp8_kernel(Fp8Args a) {
    using Cfg = F8Cfg<D>;
    // DS 64-wide k-steps of the score MFMA; when D is an odd multiple of 32 the
    // last step's upper half (features D .. D + 31, lane half g = 1) has a zero
    // Q operand
    constexpr int BC = Cfg::BC, KB = BC / 32, DS = (D + 63) / 64, OB = D / 32;
    constexpr bool HALF_STEP = D % 64 != 0;
    static_assert(D % 32 == 0, "features in 32-wide MFMA blocks");
    constexpr int KP = Cfg::KP, VTP = Cfg::VTP, OP = Cfg::OP;
    constexpr int NK = Cfg::NK, NV = Cfg::NV, LPW = Cfg::LPW;
    constexpr float kLimit = 256.0f; // P~ <= 2^8: within E4M3's range (448)
    constexpr int KBYTES = NK * 1024;                    // K stage: the K tile
    constexpr int VBYTES = (kF8Waves * LPW - NK) * 1024; // V^T stage: the tile and the spare blocks
    static_assert(NV * 1024 <= VBYTES && KBYTES <= VBYTES, "stage sizes");
    __shared__ __attribute__((aligned(16))) char ks0_raw[KBYTES];
    __shared__ __attribute__((aligned(16))) char ks1_raw[KBYTES];
    __shared__ __attribute__((aligned(16))) char vs0_raw[VBYTES];
    __shared__ __attribute__((aligned(16))) char vs1_raw[VBYTES];
    lds_char *const ks0 = (lds_char *)ks0_raw;
    lds_char *const ks1 = (lds_char *)ks1_raw;
    lds_char *const vs0 = (lds_char *)vs0_raw;
    lds_char *const vs1 = (lds_char *)vs1_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31;
    const int g = lane >> 5;
    const int N = a.N, Npad = a.Npad;

    const Work wk = map_workgroup(blockIdx.x, gridDim.x, a.n_qblk, CAUSAL);
    const uint8_t *__restrict__ Q = (const uint8_t *)a.q + (int64_t)wk.bh * N * D;
    const uint8_t *__restrict__ K = (const uint8_t *)a.k + (int64_t)wk.bh * N * D;
    const uint8_t *__restrict__ Vt = (const uint8_t *)a.vt + (int64_t)wk.bh * D * Npad;
    uint16_t *__restrict__ O = (uint16_t *)a.o + (int64_t)wk.bh * N * D;
    float *__restrict__ LSE = a.lse + (int64_t)wk.bh * N;

    const int q0 = wk.qb * kF8Rows;
    const int q0w = q0 + 32 * wave;
    const int qi = q0w + r;
    const int kv_end = CAUSAL ? min(N, q0 + kF8Rows) : N;
    const int n_tiles = (kv_end + BC - 1) / BC;

    // loader: batch b = the K rows of tile b and the V^T columns of tile
    // b - 1.  Load j of wave w fills 1 KB block w + 8 j: blocks [0, NK) go to
    // the K stage (rows in MFMA row order), the rest to the V^T stage
    // (feature rows of 128 keys, then spare blocks).
    // Loads, as in the 16-bit ping-pong kernel: spread, the four waves of
    // group 0 issue every load of a batch among the MFMAs of their M phase;
    // split burst (D = 256, and causal D = 192, whose spread instances would
    // spill), every wave issues its share at the start of its own softmax
    // phase.  Issued back to back by all eight waves at the start of a
    // phase, the loads stall every issuing wave until the address unit has
    // taken them.
    constexpr bool SPREAD = D <= 128 || (D == 192 && !CAUSAL);
    constexpr int IW = SPREAD ? 4 : kF8Waves, LPI = (NK + NV + IW - 1) / IW;
    static_assert(IW * LPI <= kF8Waves * LPW, "the loads fit the stage");
    const int iwave = SPREAD ? (wave & 3) : wave;
    uint32_t voff[LPI];
#pragma unroll
    for (int j = 0; j < LPI; ++j) {
        const int blk = iwave + IW * j;
        uint32_t off = 0;
        if (blk < NK) {
            const int pos = 1024 * blk + 16 * lane;
            const int R = pos / KP, chunk = (pos % KP) / 16;
            const int key = 32 * (R >> 5) + k_row_key(R & 31);
            off = (uint32_t)(key * D + (chunk < D / 16 ? 16 * chunk : 0));
        } else if (blk < NK + NV) {
            const int pos = 1024 * (blk - NK) + 16 * lane;
            const int f = pos / VTP, chunk = (pos % VTP) / 16;
            off = (uint32_t)f * (uint32_t)Npad + (chunk < BC / 16 ? 16u * chunk : 0u);
        }
        voff[j] = off;
    }
    const uint32_t vt_bytes = __builtin_amdgcn_readfirstlane((uint32_t)D * (uint32_t)Npad);
    auto load_one = [&](int b, lds_char *kd, lds_char *vd, int j) __attribute__((always_inline)) {
        const int kk = b * BC, kv = max(b - 1, 0) * BC;
        const uint32_t k_bytes =
            __builtin_amdgcn_readfirstlane((uint32_t)(b < n_tiles ? min(kv_end - kk, BC) * D : 0));
        // V^T rows hold keys up to Npad (zero-padded); past the last tile nothing is read
        const uint32_t v_bytes = (b >= 1 && b - 1 < n_tiles) ? vt_bytes : 0u;
        const uint8_t *const kb_ = (const uint8_t *)K + (int64_t)kk * D;
        const int blk = iwave + IW * j; // wave-uniform
        // K or V^T block chosen by selects, not branches
        const bool isk = blk < NK;
        load_lds_16s(isk ? (const void *)kb_ : (const void *)Vt, isk ? k_bytes : v_bytes, voff[j],
                     isk ? 0u : (uint32_t)kv, isk ? kd + 1024 * blk : vd + 1024 * (blk - NK));
    };
    auto issue_batch = [&](int b, lds_char *kd, lds_char *vd) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < LPI; ++j)
            load_one(b, kd, vd, j);
    };

    // B operand of S^T: lane (r, g) holds q_qi[64 s + 32 g .. + 31]; a negative
    // scale flips the sign bit of every E4M3 byte
    i32x8 qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
        if (qi < N && 64 * s + 32 * g < D) {
            const u32x4 lo = *(const u32x4 *)(Q + (int64_t)qi * D + 64 * s + 32 * g);
            const u32x4 hi = *(const u32x4 *)(Q + (int64_t)qi * D + 64 * s + 32 * g + 16);
            qf[s] = i32x8{(int)(lo[0] ^ a.qneg), (int)(lo[1] ^ a.qneg), (int)(lo[2] ^ a.qneg), (int)(lo[3] ^ a.qneg),
                          (int)(hi[0] ^ a.qneg), (int)(hi[1] ^ a.qneg), (int)(hi[2] ^ a.qneg), (int)(hi[3] ^ a.qneg)};
        } else {
            qf[s] = i32x8{};
        }
    }

    f32x16 o[OB];
#pragma unroll
    for (int b = 0; b < OB; ++b)
        o[b] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float c = a.c;
    const int k_lane = r * KP + 32 * g;      // LDS row r of a K block, k half g
    const int v_lane = r * VTP + 16 * g;     // V^T row r of a feature block

    f32x16 s[KB];       // S^T of the wave's current tile
    uint32_t pk[KB][4]; // its weights in E4M3: pk[kb][w] holds entries 4w .. 4w+3 of block kb
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            pk[kb][w] = 0u;

    auto active = [&](int t) __attribute__((always_inline)) {
        return (q0w < N) && (!CAUSAL || t * BC <= q0w + 31);
    };
    // S^T = K Q^T over the head dim in 64-wide steps
    struct LB_ {
        int b;
        lds_char *kd, *vd;
    };
    auto scores = [&](const lds_char *kst, LB_ x, int j0, auto nl) __attribute__((always_inline)) {
        constexpr int NL = decltype(nl)::value, NM = DS * KB;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            s[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < DS; ++st)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                // (the zero half of a half step reads its row's first half instead:
                // finite bytes inside the tile, multiplied by the zero Q operand)
                const int kofs = (HALF_STEP && st == DS - 1) ? 64 * st - 32 * g : 64 * st;
                const lds_char *p = kst + k_lane + 32 * kb * KP + kofs;
                const u32x4 lo = *(const __attribute__((address_space(3))) u32x4 *)p;
                const u32x4 hi = *(const __attribute__((address_space(3))) u32x4 *)(p + 16);
                const i32x8 kv = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kb] = mfma8(kv, qf[st], s[kb]);
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    if (i * NM / NL == st * KB + kb)
                        load_one(x.b, x.kd, x.vd, j0 + i);
            }
        // kF8Ahead MFMAs' reads ahead, then two reads per MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kF8Ahead, 0);
#pragma unroll
        for (int n = 0; n < DS * KB - kF8Ahead; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kF8Ahead, 0);
    };
    // O^T += V^T P~^T over 64-key steps (blocks 2 s', 2 s' + 1)
    auto accumulate = [&](const lds_char *vst, LB_ x, int j0, auto nl) __attribute__((always_inline)) {
        constexpr int NL = decltype(nl)::value, NM = OB * KB / 2;
        const lds_char *vs = vst + v_lane;
#pragma unroll
        for (int sp = 0; sp < KB / 2; ++sp)
#pragma unroll
            for (int b = 0; b < OB; ++b) {
                const lds_char *p = vs + 32 * b * VTP + 64 * sp;
                const u32x4 lo = *(const __attribute__((address_space(3))) u32x4 *)p;
                const u32x4 hi = *(const __attribute__((address_space(3))) u32x4 *)(p + 32);
                const i32x8 vv = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                const i32x8 pb = {(int)pk[2 * sp][0], (int)pk[2 * sp][1], (int)pk[2 * sp][2], (int)pk[2 * sp][3],
                                  (int)pk[2 * sp + 1][0], (int)pk[2 * sp + 1][1], (int)pk[2 * sp + 1][2],
                                  (int)pk[2 * sp + 1][3]};
                o[b] = mfma8(vv, pb, o[b]);
#pragma unroll
                for (int i = 0; i < NL; ++i)
                    if (i * NM / NL == sp * OB + b)
                        load_one(x.b, x.kd, x.vd, j0 + i);
            }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kF8Ahead, 0);
#pragma unroll
        for (int n = 0; n < OB * KB / 2 - kF8Ahead; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kF8Ahead, 0);
    };
    auto softmax = [&](int t) __attribute__((always_inline)) {
        const int k0 = t * BC;
        // entry e of block kb, lane half g: key k0 + 32 kb + 16 g + e
        if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0w)) {
            const int lim = (CAUSAL ? min(N, qi + 1) : N) - k0 - 16 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s[kb][e] = (32 * kb + e < lim) ? s[kb][e] : -INFINITY;
        }
        // P~ = exp2(s c - m_ref) <= 2^8, summed in fp32, rounded to E4M3 for PV
        float lt = 0.f;
        auto exps = [&](float m_ref) __attribute__((always_inline)) {
            lt = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float p[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * w + u], c, -m_ref));
                        lt += p[u];
                    }
                    // both halves are written: the register's old value is passed
                    // through only so that no zeroing move is needed
                    int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], (int)pk[kb][w], false);
                    x = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
                    pk[kb][w] = (uint32_t)x;
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
                for (int e = 0; e < 16; ++e)
                    mx = fmaxf(mx, s[kb][e]);
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
    };
    // M(t): O += P~(t-1) V(t-1), then S(t); X(t): softmax of S(t)
    using z_t = std::integral_constant<int, 0>;
    auto M = [&](int t, const lds_char *vprev, const lds_char *kcur) __attribute__((always_inline)) {
        const LB_ none{0, nullptr, nullptr};
        if (t >= 1 && t - 1 < n_tiles && active(t - 1))
            accumulate(vprev, none, 0, z_t{});
        if (t < n_tiles && active(t))
            scores(kcur, none, 0, z_t{});
    };
    constexpr int LA = LPI / 2;
    auto ML = [&](int t, const lds_char *vprev, const lds_char *kcur, lds_char *kn, lds_char *vn)
                  __attribute__((always_inline)) {
        const LB_ x{t + 1, kn, vn};
        if (t >= 1 && t - 1 < n_tiles && active(t - 1)) {
            accumulate(vprev, x, 0, std::integral_constant<int, LA>{});
        } else {
#pragma unroll
            for (int j = 0; j < LA; ++j)
                load_one(t + 1, kn, vn, j);
        }
        if (t < n_tiles && active(t)) {
            scores(kcur, x, LA, std::integral_constant<int, LPI - LA>{});
        } else {
#pragma unroll
            for (int j = LA; j < LPI; ++j)
                load_one(t + 1, kn, vn, j);
        }
    };
    auto X = [&](int t) __attribute__((always_inline)) {
        if (t >= 0 && t < n_tiles && active(t))
            softmax(t);
    };

    // Ping-pong schedule (as in the 16-bit dense kernel): waves 4..7 run one
    // phase behind waves 0..3, so on every SIMD one wave issues MFMAs while
    // the other does its softmax.  Phase 2c: batch c + 1 goes out (spread:
    // among group 0's MFMAs; split burst: group 1's share), group 0 runs M(c),
    // group 1 X(c - 1).  Phase 2c + 1: (split burst: group 0's share goes
    // out) group 0 runs X(c), group 1 M(c); batch c + 1 has landed at its end
    // (the stages it fills are read by neither phase).
    const int grp = wave >> 2;
    if (!SPREAD || grp == 0)
        issue_batch(0, ks0, vs1);
    wait_vmcnt<0>();
    tile_barrier();
    if (grp == 0) {
        auto step = [&](int cc, lds_char *kn, lds_char *vn, const lds_char *vprev, const lds_char *kcur)
                        __attribute__((always_inline)) {
            if constexpr (SPREAD)
                ML(cc, vprev, kcur, kn, vn);
            else
                M(cc, vprev, kcur);
            tile_barrier();
            // (split burst: group 0's share of batch c + 1 goes out at the start
            // of its softmax phase, into stages neither phase reads)
            if (!SPREAD && cc + 1 <= n_tiles)
                issue_batch(cc + 1, kn, vn);
            X(cc);
            wait_vmcnt<0>();
            tile_barrier();
        };
        int cc = 0;
        for (; cc + 1 <= n_tiles; cc += 2) {
            step(cc, ks1, vs0, vs1, ks0);
            step(cc + 1, ks0, vs1, vs0, ks1);
        }
        if (cc <= n_tiles)
            step(cc, ks1, vs0, vs1, ks0);
    } else {
        auto step = [&](int cc, lds_char *kn, lds_char *vn, const lds_char *vprev, const lds_char *kcur)
                        __attribute__((always_inline)) {
            if (!SPREAD && cc + 1 <= n_tiles)
                issue_batch(cc + 1, kn, vn);
            X(cc - 1);
            tile_barrier();
            M(cc, vprev, kcur);
            wait_vmcnt<0>();
            tile_barrier();
        };
        int cc = 0;
        for (; cc + 1 <= n_tiles; cc += 2) {
            step(cc, ks1, vs0, vs1, ks0);
            step(cc + 1, ks0, vs1, vs0, ks1);
        }
        if (cc <= n_tiles)
            step(cc, ks1, vs0, vs1, ks0);
    }

    // epilogue: O = acc * v_descale / l in bf16, staged through LDS; lse
    const float l_tot = pair_sum(l_run);
    const float inv = a.v_descale / l_tot;
    // every tile read is done; waves 2i and 2i + 1 stage their rows in stage
    // array i, or (when two waves' rows do not fit an array) waves i and i + 4
    // use array i in two rounds: waves 0..3 write, read back and store, then
    // waves 4..7 (every wave passes the same barriers)
    constexpr bool TWO_ROUNDS = 2 * 32 * OP > KBYTES;
    constexpr int ROUNDS = TWO_ROUNDS ? 2 : 1;
    static_assert(32 * OP <= KBYTES, "a wave's O rows fit in a stage array");
    const int sa = TWO_ROUNDS ? (wave & 3) : (wave >> 1);
    lds_char *const own = sa == 0 ? ks0 : sa == 1 ? ks1 : sa == 2 ? vs0 : vs1;
    lds_char *ow = own + (TWO_ROUNDS ? 0 : (wave & 1) * 32 * OP);
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) {
        const bool mine = !TWO_ROUNDS || (wave >> 2) == round;
        if (mine && q0w < N) {
#pragma unroll
            for (int b = 0; b < OB; ++b)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const u32x2 w = {Bf16::pack(o[b][4 * a4] * inv, o[b][4 * a4 + 1] * inv),
                                     Bf16::pack(o[b][4 * a4 + 2] * inv, o[b][4 * a4 + 3] * inv)};
                    *(__attribute__((address_space(3))) u32x2 *)(ow + r * OP + (32 * b + 8 * a4 + 4 * g) * 2) = w;
                }
            if (g == 0 && qi < N)
                LSE[qi] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
        }
        __syncthreads();
        if (mine && q0w < N) {
#pragma unroll
            for (int j = 0; j < 32 * (D / 8) / 64; ++j) {
                const int ch = 64 * j + lane;
                const int row = ch / (D / 8), col = ch % (D / 8);
                const int q = q0w + row;
                const u32x4 val = *(const __attribute__((address_space(3))) u32x4 *)(ow + row * OP + col * 16);
                if (q < N)
                    *(u32x4 *)(O + (int64_t)q * D + col * 8) = val;
            }
        }
        if (round + 1 < ROUNDS)
            __syncthreads(); // the next round's rows go where this round's were read
    }
}

template <int D>
hipError_t launch_fp8_t(bool causal, int64_t BH, const Fp8Args &args, hipStream_t stream) {
    const dim3 tgrid((unsigned)(args.Npad / 64), (unsigned)BH);
    hipLaunchKernelGGL((fa_fp8_vt_kernel<D>), tgrid, dim3(256), 0, stream, (const uint8_t *)args.v,
                       (uint8_t *)args.vt, args.N, args.Npad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t nwg = BH * (int64_t)args.n_qblk;
    if (causal)
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, true>), dim3((unsigned)nwg), dim3(kF8Threads), 0, stream, args);
    else
        hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, false>), dim3((unsigned)nwg), dim3(kF8Threads), 0, stream, args);
    return hipGetLastError();
}

} // namespace

hipError_t launch_fp8(int D, bool causal, int64_t BH, const Fp8Args &args, hipStream_t stream) {
    switch (D) {
    case 32:
        return launch_fp8_t<32>(causal, BH, args, stream);
    case 64:
        return launch_fp8_t<64>(causal, BH, args, stream);
    case 96:
        return launch_fp8_t<96>(causal, BH, args, stream);
    case 160:
        return launch_fp8_t<160>(causal, BH, args, stream);
    case 192:
        return launch_fp8_t<192>(causal, BH, args, stream);
    case 224:
        return launch_fp8_t<224>(causal, BH, args, stream);
    case 256:
        return launch_fp8_t<256>(causal, BH, args, stream);
    default:
        return launch_fp8_t<128>(causal, BH, args, stream);
    }
}

} // namespace fa
