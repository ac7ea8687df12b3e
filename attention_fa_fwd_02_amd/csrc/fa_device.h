// Device-side building blocks shared by the forward and backward kernels
// (gfx950): vector types, the LDS barrier and wait helpers, the
// direct-to-LDS buffer load, lane-pair reductions and the 16-bit element
// types with their MFMA and round-to-nearest-even packing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLn2 = 0.693147180559945309f;
// Word 3 of a raw buffer descriptor on gfx9-family parts: 32-bit data format,
// no swizzle, so loads address plain bytes and are range-checked against the
// descriptor's record count (out-of-range loads return zeros).
constexpr int kBufferWord3 = 0x00020000;

// Workgroup barrier without the memory fence __syncthreads() adds: the fence
// waits for every outstanding global load (vmcnt(0)), including direct-to-LDS
// loads issued ahead for later tiles.  Callers wait for the loads that must
// have landed (s_waitcnt vmcnt(n)) before calling; every LDS read of the
// current tile has been consumed by an MFMA before the barrier is reached.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 16, "vmcnt fits the low field");
    __builtin_amdgcn_s_waitcnt(0xF70 | n);
}

// Direct global -> LDS load of 16 bytes per lane through a buffer descriptor
// over [base, base + bytes): lane l's bytes from offset voff land at LDS
// address lds + 16 l (lds is wave-uniform).  Offsets at or past `bytes` read
// zeros and touch no memory.
__device__ __forceinline__ void load_lds_16(const void *base, uint32_t bytes, uint32_t voff, lds_char *lds) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}

// Max / sum over the lane pair (l, l^32) that shares one query row.
__device__ __forceinline__ float pair_max(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)s[0]), __builtin_bit_cast(float, (uint32_t)s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto s = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)s[0]) + __builtin_bit_cast(float, (uint32_t)s[1]);
}

struct Work {
    int bh;
    int qb;
};

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), and within
// an XCD in increasing id.  When the grid is a multiple of 8, XCD x takes the
// contiguous logical range [x * n/8, (x+1) * n/8), so the query blocks of a
// slice share one L2.  Causal query blocks differ in length (block qb has
// qb + 1 blocks' worth of keys): when each XCD's range holds whole slices,
// they are handed out longest first, so the short ones fill in at the end
// instead of a long one starting last.  The XCD's slices are taken four at a
// time (longest first within each group of four), so that fewer slices' K
// and V are read through the XCD's L2 at once.
__device__ __forceinline__ Work map_workgroup(int wg, int nwg, int n_qblk, bool causal) {
    Work w;
    if ((nwg & 7) == 0) {
        const int per = nwg >> 3;
        const int x = wg & 7, j = wg >> 3;
        if (causal && per % n_qblk == 0) {
            const int hx = per / n_qblk;             // slices per XCD
            const int gs = (hx & 3) == 0 ? 4 : hx;   // slices per group
            const int gsz = gs * n_qblk, grp = j / gsz, in = j - grp * gsz;
            w.bh = x * hx + grp * gs + in % gs;
            w.qb = n_qblk - 1 - in / gs;
            return w;
        }
        const int L = x * per + j;
        w.bh = L / n_qblk;
        const int qb = L - w.bh * n_qblk;
        w.qb = causal ? (n_qblk - 1 - qb) : qb;
        return w;
    }
    w.bh = wg / n_qblk;
    const int qb = wg - w.bh * n_qblk;
    w.qb = causal ? (n_qblk - 1 - qb) : qb; // causal: most key tiles first
    return w;
}

// ----------------------------------------------------------------------------
// 16-bit element types
// ----------------------------------------------------------------------------
struct Bf16 {
    __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // round two fp32 to nearest-even 16-bit values, first in the low half
    __device__ static __forceinline__ uint32_t pack(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    // the two 16-bit values of a word, low half first (exact)
    __device__ static __forceinline__ f32x2 unpack(uint32_t w) {
        const f32x2 v = {__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
        return v;
    }
};

struct F16 {
    __device__ static __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack(float x, float y) {
        f32x2 v = {x, y};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    __device__ static __forceinline__ f32x2 unpack(uint32_t w) {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    }
};

} // namespace
} // namespace fa
