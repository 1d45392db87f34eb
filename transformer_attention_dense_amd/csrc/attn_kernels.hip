// Fused attention forward kernels for MI355X (gfx950, CDNA4).
//
// Computes O = softmax(Q K^T * D^-0.5) V for [B, N, H, D] BF16 tensors, as defined
// by page "Audit SGLang interfaces and refresh validated kernel solutions",
// definitions/dense_attention/noncausal_dense_attention_h32_d{64,128}.json
// (reference: FP32 scores, softmax over keys, FP32 accumulation, BF16 output) and
// definitions/block_causal_attention/prefix_cached_block_causal_h32_d128.json
// (keys and values are prefix rows followed by current rows; every key visible).
//
// One pass over the keys (flash-style online softmax): per workgroup a block of
// queries of one (batch, head) streams BN-key tiles of K and V through LDS.
//
// Data layout per wave (64 lanes, 32 query rows):
//   * S^T = K Q^T is computed with v_mfma_f32_32x32x16_bf16: A = K tile rows
//     (keys x 16 head dims) from LDS, B = Q^T fragments kept in registers for the
//     whole loop. In the 32x32 accumulator, lane (n + 32g) holds query n of the wave
//     and the 16 keys 8*(r/4) + 4g + (r%4), r = 0..15, of each 32-key block. The row
//     maximum over keys is therefore a register reduction plus one exchange with
//     lane n ^ 32 (v_permlane32_swap), and the row sum needs no exchange until the end.
//   * O^T += V^T P^T: the accumulator of S^T, exponentiated and rounded to BF16, is
//     directly the B operand (keys are the contraction index; the key order inside a
//     16-key step is permuted consistently for both operands). The A operand V^T is
//     read from the row-major V tile with ds_read_b64_tr_b16, which hands each lane
//     4 keys of one head dimension.
//   * Softmax runs in the exp2 domain with scale * log2(e) folded into one FMA. The
//     running maximum is only raised when the tile maximum exceeds it by more than
//     2^kRescaleLog2 in the exp2 domain; O and l share that reference, so the final
//     O / l is unchanged in exact arithmetic (probabilities stay <= 2^8 before
//     normalisation, well inside FP32 and BF16 range).
//
// Split-KV: with several key ranges per (query block, head) the kernel writes the
// normalised partial output (FP32) and its log2-sum-exp2; attn_combine merges them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kRescaleLog2 = 8.0f;
constexpr int kWave = 64;

__device__ __forceinline__ float wave_swap_max(float x) {
    // max(x[lane], x[lane ^ 32]) for every lane
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                              false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup -> (query block, batch*head, split). Workgroups are dispatched to the
// 8 XCDs round-robin by linear id; this remap gives each XCD a contiguous range of
// (query block, head) work so the query blocks sharing one head's K/V run on the same
// XCD and hit its L2.
__device__ __forceinline__ void decode_workgroup(int m_blocks, int bh_count, int& mb, int& bh,
                                                 int& split) {
    const int L = blockIdx.x;
    const int T = gridDim.x;
    const int per = T >> 3;
    const int L2 = (L < (per << 3)) ? (L & 7) * per + (L >> 3) : L;
    mb = L2 % m_blocks;
    const int rest = L2 / m_blocks;
    bh = rest % bh_count;
    split = rest / bh_count;
}

template <int D, int NW, int BN>
__global__ __launch_bounds__(NW* kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(FwdParams p) {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "key tile");
    constexpr int NB = BN / 32;           // 32-key blocks per tile
    constexpr int KS = D / 16;            // MFMA k-steps over the head dim
    constexpr int DB = D / 32;            // 32-wide head-dim blocks of O^T
    constexpr int KSTR = D + 8;           // LDS row stride of K (elements)
    constexpr int VSTR = D + 16;          // LDS row stride of V (elements)
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int NT = NW * kWave;
    constexpr int PER_T = BN * CPR / NT;  // chunks per thread per tensor per tile
    static_assert(BN * CPR % NT == 0, "loader");

    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t sV[BN * VSTR];

    int mb, bh, split;
    decode_workgroup(p.m_blocks, p.B * p.H, mb, bh, split);
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    const int H = p.H;
    const int nk = p.n0 + p.n1;
    const int kbeg = split * p.keys_per_split;
    const int kend = min(nk, kbeg + p.keys_per_split);

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int n = lane & 31;
    const int g = lane >> 5;
    const int q0 = mb * (NW * 32) + wave * 32;
    const bool active = q0 < p.Nq;

    // Q^T fragments (B operand), one per 16-dim k-step: lane holds query n, dims
    // 16*ks + 8g .. +7.
    bf16x8 qf[KS];
    {
        const int qi = min(q0 + n, p.Nq - 1);
        const uint16_t* qrow = p.q + ((long)(b * p.Nq + qi) * H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * g);
    }

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m_ref = -INFINITY;  // running reference maximum (raw score units)
    float l_part = 0.f;       // this lane's partial row sum
    const float c = p.c;

    // Global -> register staging of one K/V tile.
    u32x4 kreg[PER_T], vreg[PER_T];
    auto load_tile = [&](int t0) {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int ch = tid + i * NT;
            const int row = ch / CPR;
            const int col = (ch % CPR) * 8;
            const int key = min(t0 + row, kend - 1);
            const uint16_t* ks;
            const uint16_t* vs;
            if (key < p.n0) {
                const long off = ((long)(b * p.n0 + key) * H + h) * D + col;
                ks = p.k0 + off;
                vs = p.v0 + off;
            } else {
                const long off = ((long)(b * p.n1 + (key - p.n0)) * H + h) * D + col;
                ks = p.k1 + off;
                vs = p.v1 + off;
            }
            kreg[i] = *reinterpret_cast<const u32x4*>(ks);
            vreg[i] = *reinterpret_cast<const u32x4*>(vs);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int ch = tid + i * NT;
            const int row = ch / CPR;
            const int col = (ch % CPR) * 8;
            *reinterpret_cast<u32x4*>(&sK[row * KSTR + col]) = kreg[i];
            *reinterpret_cast<u32x4*>(&sV[row * VSTR + col]) = vreg[i];
        }
    };

    // Per-lane LDS offsets (elements).
    const int k_off = n * KSTR + 8 * g;  // + (kb*32)*KSTR + 16*ks
    const int tr_r = (lane & 15) >> 2;
    const int tr_q = lane & 3;
    const int v_off = (4 * g + tr_r) * VSTR + 16 * ((lane >> 4) & 1) + 4 * tr_q;

    const int ntiles = (kend - kbeg + BN - 1) / BN;
    load_tile(kbeg);
    for (int t = 0; t < ntiles; ++t) {
        const int t0 = kbeg + t * BN;
        __syncthreads();
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t0 + BN);
        if (!active) continue;

        // ---- S^T = K Q^T for the tile
        f32x16 s[NB];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8*>(&sK[k_off + kb * 32 * KSTR + 16 * ks]);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
            }
        }

        // ---- mask keys past the end of this range (ragged last tile)
        if (t0 + BN > kend) {
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= kend) s[kb][r] = -INFINITY;
                }
        }

        // ---- online softmax (exp2 domain)
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = wave_swap_max(mx);
        const bool need = (mx - m_ref) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f((m_ref - m_new) * c);
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) o[i] *= alpha;
            m_ref = m_new;
        }
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
        bf16x8 pf[NB][2];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
                l_part += e;
                pf[kb][r >> 3][r & 7] = (__bf16)e;
            }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int rowbase = kb * 32 + 16 * tt;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int off = v_off + rowbase * VSTR + 32 * db;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)((lds_u16*)sV + off));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)((lds_u16*)sV + off + 8 * VSTR));
                    const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    const bf16x8 a = __builtin_bit_cast(bf16x8, a16);
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb][tt], o[db], 0, 0, 0);
                }
            }
    }

    if (!active) return;

    // ---- epilogue
    const float l_tot = wave_swap_sum(l_part);
    const int qi = q0 + n;
    if (p.splits == 1) {
        const float inv = 1.0f / l_tot;
        if (qi < p.Nq) {
            uint16_t* orow = p.out + ((long)(b * p.Nq + qi) * H + h) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * j + e] * inv);
                    *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * j + 4 * g) = v;
                }
        }
    } else {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        if (qi < p.Nq) {
            const long row = (long)(b * p.Nq + qi) * H + h;
            const long rows = (long)p.B * p.Nq * H;
            float* prow = p.part_o + ((long)split * rows + row) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = o[db][4 * j + e] * inv;
                    *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * j + 4 * g) = v;
                }
            if (g == 0) {
                const float mref2 = (m_ref == -INFINITY) ? 0.f : m_ref * c;
                p.part_lse[(long)split * rows + row] =
                    l_tot > 0.f ? mref2 + __log2f(l_tot) : -INFINITY;
            }
        }
    }
}

// Merges split-KV partial results: O = sum_s w_s O_s / sum_s w_s with
// w_s = 2^(lse_s - max_s lse_s). One wave per row, each lane D/64 head dims.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineParams p) {
    constexpr int PER = D / kWave;
    const long row = (long)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= p.rows) return;
    float mx = -INFINITY;
    for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.part_lse[(long)s * p.rows + row]);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    for (int s = 0; s < p.splits; ++s) {
        const float lse = p.part_lse[(long)s * p.rows + row];
        const float w = (lse == -INFINITY) ? 0.f : exp2f(lse - mx);
        wsum += w;
        const float* src = p.part_o + ((long)s * p.rows + row) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * src[e];
    }
    const float inv = 1.0f / wsum;
    uint16_t* dst = p.out + row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const __bf16 v = (__bf16)(acc[e] * inv);
        dst[e] = __builtin_bit_cast(uint16_t, v);
    }
}

}  // namespace

template <int D, int NW>
static hipError_t launch_fwd_t(const FwdParams& p, long long workgroups, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, 64>), dim3((unsigned)workgroups), dim3(NW * kWave),
                       0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fwd(int D, int waves, const FwdParams& p, long long workgroups,
                      hipStream_t stream) {
    if (D == 64 && waves == 4) return launch_fwd_t<64, 4>(p, workgroups, stream);
    if (D == 64 && waves == 2) return launch_fwd_t<64, 2>(p, workgroups, stream);
    if (D == 128 && waves == 4) return launch_fwd_t<128, 4>(p, workgroups, stream);
    if (D == 128 && waves == 2) return launch_fwd_t<128, 2>(p, workgroups, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_combine(int D, const CombineParams& p, hipStream_t stream) {
    const unsigned blocks = (unsigned)((p.rows + 3) / 4);
    if (D == 64)
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(blocks), dim3(256), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace attn
