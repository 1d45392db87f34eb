// Internal launch interface between the C ABI (attn_api.hip) and the kernels
// (attn_kernels.hip). Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Arguments of the fused forward kernel. Keys are segment 0 (k0/v0, n0 rows) then
// segment 1 (k1/v1, n1 rows); all tensors [B, rows, H, D] BF16 bits.
struct FwdParams {
    const uint16_t* q;
    const uint16_t* k0;
    const uint16_t* v0;
    const uint16_t* k1;
    const uint16_t* v1;
    uint16_t* out;
    float* part_o;    // split-KV partial outputs [splits][B*Nq*H][D], FP32, normalised
    float* part_lse;  // split-KV log2-sum-exp2 per row [splits][B*Nq*H]
    int B, Nq, H;
    int n0, n1;
    int keys_per_split;  // multiple of the key tile; the last split may be shorter
    int splits;
    int m_blocks;  // query blocks per (batch, head)
    float c;       // D^-0.5 * log2(e)
    // Block-causal visibility (null for full visibility): image ids [Nq] (keys are
    // the queries' own positions) and per-32-row block summaries of them (bc_meta).
    const int* ids;
    const int* meta;
};

// Summary of the image ids of rows [32 b, 32 b + 32) of a block-causal call, four
// ints per block: smallest and largest nonnegative id (INT_MAX / -1 when there is
// none), number of negative (text) ids, and 0.
constexpr int kMetaRows = 32;

struct CombineParams {
    const float* part_o;
    const float* part_lse;
    uint16_t* out;
    long rows;  // B*Nq*H
    int splits;
};

// Arguments of the 3-D neighborhood attention kernel (attn_na3d.hip), D = 64. All
// tensors [B, T, Y, X, H, D] BF16 bits; windows (kt, ky, kx) odd and at most their axes.
struct NaParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    int B, T, Y, X, H;
    int kt, ky, kx;
    // set by na3d_configure: a wave's query tile (32 / qb rows y x qb positions on X)
    int qb;       // 16, 8 or 4
    int kw;       // positions on X of a key block (32, 16 or 8; 32 / kw rows)
    int strips;   // ceil(X / qb): strips of qb positions on the X axis
    int wt;       // frames t of a workgroup (1, 2 or 4), each with 4 / wt tiles of rows y
    int yblocks;  // blocks of rows y of a workgroup: ceil(Y / (4 / wt * 32 / qb))
    int t_inner;  // workgroup order within a head (na_decode): t fastest (1) or slowest (0)
};
void na3d_configure(NaParams& p);
long long na3d_workgroups(const NaParams& p);
hipError_t launch_na3d(const NaParams& p, hipStream_t stream);

// A work space handed to one forward call (instead of the device's shared one).
struct FixedWorkspace {
    void* ptr;
    long long bytes;
};

// The dense / prefix / cross forward behind the C entry points (attn_api.hip): checks
// the arguments, plans the launch and enqueues the kernels. Returns ATTN_OK or an
// ATTN_ERR_* code. With `fixed` null the split-KV work space is the device's shared
// one; otherwise `fixed` must hold the plan's work space (else ATTN_ERR_WORKSPACE).
int run_fwd(const void* q, const void* k0, const void* v0, int n0, const void* k1,
            const void* v1, int n1, void* out, int B, int Nq, int H, int D, int num_splits,
            int waves, void* stream, const FixedWorkspace* fixed);

// Keys per tile of the forward kernels; split ranges are multiples of it.
constexpr int kKeyTile = 64;

// waves 2 or 4: attn_fwd_kernel (attn_kernels.hip); waves 8: the ping-pong kernel
// (attn_pingpong.hip).
hipError_t launch_fwd(int D, int waves, const FwdParams& p, long long workgroups,
                      hipStream_t stream);
hipError_t launch_fwd_pingpong(int D, const FwdParams& p, long long workgroups,
                               hipStream_t stream);
// Block-causal attention: the ping-pong kernel with per-tile visibility (p.ids and
// p.meta set, one key split), after launch_bc_meta has filled p.meta.
hipError_t launch_fwd_block_causal(int D, const FwdParams& p, long long workgroups,
                                   hipStream_t stream);
hipError_t launch_bc_meta(const int* ids, int n, int* meta, hipStream_t stream);
hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream);

}  // namespace attn
