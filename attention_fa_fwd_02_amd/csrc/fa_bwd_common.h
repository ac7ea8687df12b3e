// Device pieces shared by the backward kernels (fa_bwd.hip, fa_bwd_f32.hip):
// the base-2 exponent constant, the 4-byte direct-to-LDS load and the
// XCD-aware block mapping.
#pragma once
#include "fa_device.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

// Direct global -> LDS load of 4 bytes per lane through a buffer descriptor
// over [base, base + bytes): lane l's word from offset voff lands at LDS
// address lds + 4 l (lds is wave-uniform); offsets at or past `bytes` read
// zeros.
__device__ __forceinline__ void load_lds_4(const void *base, uint32_t bytes, uint32_t voff, lds_char *lds) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

// Workgroups go round-robin over the 8 XCDs (id % 8); with a grid that is a
// multiple of 8, XCD x takes the contiguous logical range [x n/8, (x+1) n/8),
// so the blocks of one (batch, head) slice share an L2.  `reverse` hands the
// blocks of a slice out last index first.
struct Blk {
    int bh;
    int blk;
};
__device__ __forceinline__ Blk map_bwd(int wg, int nwg, int n_blk, bool reverse) {
    int L = wg;
    if ((nwg & 7) == 0)
        L = (wg & 7) * (nwg >> 3) + (wg >> 3);
    Blk b;
    b.bh = L / n_blk;
    b.blk = L - b.bh * n_blk;
    if (reverse)
        b.blk = n_blk - 1 - b.blk;
    return b;
}

} // namespace
} // namespace fa
