// Internal interface between the C ABI (fa_api.cpp) and the kernels (fa_fwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace fa {

// Kernel arguments, passed by value.
struct FwdArgs {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int32_t N;      // keys = queries per (batch, head) slice
    int32_t n_qblk; // query blocks per slice: ceil(N / query_block(D))
    float c;        // |scale| * log2(e): scores enter exp2 through one FMA
    uint32_t qneg;  // sign-bit mask XORed onto Q words when scale < 0 (0 otherwise)
    // key-split launches only (ignored otherwise): split s of slice bh covers
    // keys [s * split_keys, (s + 1) * split_keys) and writes its normalised
    // fp32 output and lse to part_o[s][bh][n][:] and part_lse[s][bh][n]
    float *part_o;
    float *part_lse;
    int64_t part_rows; // rows per split in part_o / part_lse: B * H * N
    int32_t split_keys; // a multiple of 128 (the key tile of every path)
    int32_t n_splits;
    // packed variable-length launches only (ignored otherwise): q, o are
    // [n_heads][total_q][D], k, v [n_heads][total_k][D], lse [n_heads][total_q];
    // sequence b owns rows cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1
    const int32_t *cu_q;
    const int32_t *cu_k;
    int32_t n_heads;
    int32_t total_q;
    int32_t total_k;
};

// Kernel modes: one (batch, head) slice per grid row; that plus key splits;
// packed variable-length sequences.
enum FwdMode { kDense = 0, kSplit = 1, kVarlen = 2 };

// Query rows per workgroup of the forward kernels for head dim D: 8 waves x
// 32 rows, or 4 waves x 32 rows for D > 192 (the O accumulators and Q
// operands then need the register file of one wave per SIMD).
constexpr int kQueryBlock = 256;
constexpr int query_block(int64_t D) { return D > 192 ? 128 : 256; }

// Key groups of a dense fa_fwd launch (1, 2 or 4): with kg > 1 the kernel
// (16-bit for D <= 128, fp32 for D = 64) splits its 8 waves into 8/kg row
// groups of 32 query rows times kg groups of keys, so a workgroup covers
// query_block(D) / kg rows and the grid has kg times as many workgroups.  Chosen for grids of
// B*H*ceil(N/256) workgroups that leave compute units idle: the kg that
// minimises the number of rounds of workgroups per compute unit times the
// work of one workgroup (ties go to the smaller kg).  Always 1 for D > 128
// and for fp32 at D = 128.
int choose_key_groups(int64_t BH, int64_t N, int64_t D, int dtype, int64_t n_cus);

// Enqueue the forward pass; arguments are already validated.  `rows` is the
// number of grid rows: B*H slices (kDense), B*H*n_splits (kSplit, which
// writes part_o / part_lse instead of o / lse) or n_seqs*n_heads (kVarlen);
// each row has args.n_qblk query blocks.
hipError_t launch_fwd(int dtype, int D, bool causal, FwdMode mode, int64_t rows,
                      const FwdArgs &args, hipStream_t stream, int kg = 1);

// Name of the kernel launch_fwd runs for these arguments (static string; ""
// for a combination it cannot launch).
const char *fwd_kernel_name(int dtype, int D, bool causal, FwdMode mode, int kg = 1);

// FP8 (E4M3) forward arguments, passed by value.
struct Fp8Args {
    const void *q;      // [B*H][N][D] E4M3
    const void *k;
    const void *v;
    void *vt;           // workspace: V^T [B*H][D][Npad] E4M3, keys >= N zero
    void *o;            // [B*H][N][D] bf16
    float *lse;         // [B*H][N]
    int32_t N;
    int32_t Npad;       // N rounded up to the 128-key tile
    int32_t n_qblk;     // ceil(N / 256)
    float c;            // |scale * q_descale * k_descale| * log2(e)
    float v_descale;
    uint32_t qneg;      // 0x80808080 when scale * q_descale * k_descale < 0
};

hipError_t launch_fp8(int D, bool causal, int64_t BH, const Fp8Args &args, hipStream_t stream);

// Backward-pass kernel arguments, passed by value.
struct BwdArgs {
    const void *q;
    const void *k;
    const void *v;
    const void *o;
    const void *dout;
    const float *lse;   // forward logsumexp (natural log), [B*H][N]
    float *delta;       // workspace: Delta_i = dO_i . O_i, [B*H][N]
    void *dq;
    void *dk;
    void *dv;
    int32_t N;
    float c2;           // scale * log2(e) (signed): P = exp2(c2 * q.k - log2(e) * lse)
    float scale;        // dQ = scale * dS K, dK = scale * dS^T Q
};

// Enqueue the three backward kernels (Delta, dQ, dK/dV) for a [B*H] x N x D
// problem; arguments are already validated.
hipError_t launch_bwd(int dtype, int D, bool causal, int64_t BH, const BwdArgs &args,
                      hipStream_t stream);
// The fp32 kernels of the same three steps (D = 64 or 128).
hipError_t launch_bwd_f32(int D, bool causal, int64_t BH, const BwdArgs &args, hipStream_t stream);

// Host-side pieces of the key-split path shared by fa_fwd_split and its
// static-scratch variant (arguments already validated by the caller):
// the current device is gfx950; the split grid fits one launch; enqueue the
// split kernel and the merge with the partials in `workspace`
// (fa_fwd_split_workspace_bytes bytes, 16-byte aligned).
fa_status check_device_arch();
fa_status split_grid_ok(int64_t B, int64_t H, int64_t N, int64_t D, int64_t n_splits);
fa_status split_enqueue(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t H,
                        int64_t N, int64_t D, float scale, int causal, fa_dtype dtype, int64_t n_splits,
                        void *workspace, fa_stream_t stream);

// Merge n_parts partial results per row: part_o [n_parts][rows][D] fp32,
// part_lse [n_parts][rows]; writes o [rows][D] (dtype 0 fp32, 1 bf16, 2 fp16)
// and lse [rows].  D is a multiple of 8, at most 512.
hipError_t launch_merge(int dtype, const float *part_o, const float *part_lse, int n_parts,
                        int64_t rows, int D, void *o, float *lse, hipStream_t stream);

} // namespace fa
