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

#include <type_traits>
#include <utility>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

using namespace dev;

// Waves per SIMD the kernel is compiled for, at D = 64 three: a call whose key ranges fit
// one tile (NSLOT = 1) needs one score buffer and no ring, and the LDS (K, V, and the
// query rows) still holds six two-wave workgroups per CU; the four-wave ring form fits
// 168 VGPRs (one spilled) and three workgroups per CU (48 KiB of ring each), which took
// 10-13% off grids of thousands of short query blocks (B=64 N=128 H=32: 25.8 -> 23.2 us;
// B=32 N=200: 33.8 -> 29.5) and left grids of one or two workgroups per CU unchanged.
// Otherwise two (registers for two score buffers).
template <int D, int NW, int NSLOT>
constexpr int fwd_waves_per_simd() {
    return (D == 64 && (NSLOT == 1 || NW == 4)) ? 3 : 2;
}

template <int D, int NW, int BN, int NSLOT>
__global__ __launch_bounds__(NW* kWave) __attribute__((amdgpu_waves_per_eu(
    fwd_waves_per_simd<D, NW, NSLOT>(), fwd_waves_per_simd<D, NW, NSLOT>()))) void attn_fwd_kernel(FwdParams p) {
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0 && BN <= 128, "key tile");
    static_assert(NSLOT >= 1 && NSLOT <= 3, "LDS ring depth (1: one tile per workgroup)");
    constexpr int NB = BN / 32;            // 32-key blocks per tile
    constexpr int KS = D / 16;             // MFMA k-steps over the head dim
    constexpr int DB = D / 32;             // 32-wide head-dim blocks of O^T
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int ROWB = 2 * D;            // bytes per LDS row
    constexpr int TILEB = BN * ROWB;       // bytes per K or V tile
    constexpr int NT = NW * kWave;
    constexpr int PER_T = BN * CPR / NT;   // 16-byte loads per thread per tensor per tile
    static_assert(BN * CPR % NT == 0 && NT % CPR == 0, "loader");

    // Three K slots then three V slots, rows of 2*D bytes, chunks swizzled. One-tile
    // calls add each wave's 32 query rows, which also stage its output rows.
    constexpr int QOB = (NSLOT == 1) ? NW * 32 * ROWB : 0;
    __shared__ __attribute__((aligned(1024))) char smem[2 * NSLOT * TILEB + QOB];

    int mb, bh, split;
    decode_workgroup(p.m_blocks, p.B * p.H, mb, bh, split);
    const int H = p.H;
    const int b = bh / H;
    const int h = bh - b * H;
    const int HD = H * D;  // elements between consecutive sequence rows
    const int n0 = p.n0;
    const int nk = n0 + p.n1;
    const int kbeg = split * p.keys_per_split;
    const int kend = min(nk, kbeg + p.keys_per_split);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
    const int lane = tid % kWave;
    const int n = lane & 31;
    const int g = lane >> 5;
    const int q0 = mb * (NW * 32) + wave * 32;
    const bool active = q0 < p.Nq;

    // Per-(batch, head) bases of the two key segments (element offsets of row 0).
    const uint16_t* kseg0 = uniform_ptr(p.k0 + ((long)b * n0 * HD + (long)h * D));
    const uint16_t* vseg0 = uniform_ptr(p.v0 + ((long)b * n0 * HD + (long)h * D));
    const uint16_t* kseg1 =
        uniform_ptr(p.k1 ? p.k1 + ((long)b * p.n1 * HD + (long)h * D) : kseg0);
    const uint16_t* vseg1 =
        uniform_ptr(p.v1 ? p.v1 + ((long)b * p.n1 * HD + (long)h * D) : vseg0);

    // Q^T fragments (B operand), one per 16-dim k-step: lane holds query n, dims
    // 16*ks + 8g .. +7. One-tile calls read them from LDS after the copies below.
    bf16x8 qf[KS];
    if constexpr (NSLOT != 1) {
        const int qi = min(q0 + n, p.Nq - 1);
        const uint16_t* qrow = p.q + ((long)(b * p.Nq + qi) * H + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * g);
    }
    // One-tile calls: the wave's rows of Q arrive through LDS as whole rows and the
    // output leaves through the same rows, so a wave's loads and stores cover whole
    // 128- or 256-byte rows instead of 16- to 32-byte pieces of 32 rows, which matters
    // when every workgroup moves only a few KiB.
    char* const qo = smem + 2 * NSLOT * TILEB + wave * 32 * ROWB;
    const long qrow0 = ((long)b * p.Nq * H + (long)q0 * H + h) * D;  // the wave's row 0

    // Loader: load round i of thread tid fills physical chunk P = i*NT + tid of a
    // tile, i.e. row r = P / CPR at chunk position P % CPR, which holds logical chunk
    // (P % CPR) ^ swizzle(r). Rounds advance by RSTEP rows; the swizzle pattern has a
    // period of SWP rows, so the per-lane offsets repeat every SWP / RSTEP rounds.
    constexpr int RSTEP = NT / CPR;
    constexpr int SWP = 16;
    constexpr int NPAT = (RSTEP % SWP == 0) ? 1 : SWP / RSTEP;
    static_assert(RSTEP % SWP == 0 || SWP % RSTEP == 0, "loader pattern");
    int ld_off[NPAT];
#pragma unroll
    for (int i = 0; i < NPAT; ++i) {
        const int P = i * NT + tid;
        const int r = P / CPR;
        const int c = (P % CPR) ^ lds_swizzle<CPR>(r);
        ld_off[i] = r * HD + c * 8;
    }

    // nt_c: non-temporal copies (a tile no other workgroup reads)
    auto issue = [&](const uint16_t* seg0, const uint16_t* seg1, int t0, char* slot, auto nt_c) {
        constexpr bool NTL = decltype(nt_c)::value;
        char* const dst = slot + wave * kWave * 16;
        const bool whole = (t0 + BN <= kend) && (t0 + BN <= n0 || t0 >= n0);
        if (whole) {
            const long rowoff = (t0 < n0) ? (long)t0 * HD : (long)(t0 - n0) * HD;
            const uint16_t* base = ((t0 < n0) ? seg0 : seg1) + rowoff;
#pragma unroll
            for (int i = 0; i < PER_T; ++i)  // uniform base, per-lane offset
                load16_to_lds_sbase<NTL>(base + (long)(i / NPAT) * NPAT * RSTEP * HD,
                                         2u * ld_off[i % NPAT], dst + i * NT * 16);
        } else {
            // ragged or segment-straddling tile: clamp rows into [t0, kend) and pick
            // the segment per row
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int r = (i * NT + tid) / CPR;
                const int key = min(t0 + r, kend - 1);
                const int co = ld_off[i % NPAT] - (r - (i / NPAT) * NPAT * RSTEP) * HD;
                const uint16_t* src =
                    key < n0 ? seg0 + (long)key * HD : seg1 + (long)(key - n0) * HD;
                load16_to_lds<NTL>(src + co, dst + i * NT * 16);
            }
        }
    };
    auto issue_k = [&](int t0, int slot) {
        issue(kseg0, kseg1, t0, smem + slot * TILEB, std::false_type{});
    };
    auto issue_v = [&](int t0, int slot) {
        issue(vseg0, vseg1, t0, smem + (NSLOT + slot) * TILEB, std::false_type{});
    };

    // Per-lane LDS byte offsets of the K operand reads (per k-step) and of the V
    // transpose reads (per head-dim block and 8-key half), relative to a K or V slot;
    // key blocks and 16-key steps add whole rows.
    int koff[KS];
    {
        const int t = lds_swizzle<CPR>(n) ^ g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = n * ROWB + 16 * ((2 * ks) ^ t);
    }
    constexpr int VH = 2;  // the two 8-key halves of a 16-key step use different swizzles
    int voff[DB][VH];
    {
        const int tr_r = (lane & 15) >> 2;
        const int tr_q = lane & 3;
        const int half = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int h2 = 0; h2 < VH; ++h2) {
                const int row = 8 * h2 + 4 * g + tr_r;
                const int c = (4 * db + 2 * half + (tr_q >> 1)) ^ lds_swizzle<CPR>(row);
                voff[db][h2] = row * ROWB + 16 * c + 8 * (tr_q & 1);
            }
    }

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    float m_ref = -INFINITY;  // running reference maximum (raw score units)
    float l_part = 0.f;       // this lane's partial row sum (of BF16-rounded probabilities)
    const float c = p.c;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    constexpr int NQ = KS * NB;         // QK^T MFMAs per tile
    constexpr int NP = 2 * NB * DB;     // PV MFMAs per tile
    constexpr int NF = NQ + NP;         // LDS operand fragments per pipelined tile
    constexpr int NPAIR = NB * 8;       // exp pairs per lane per tile
    // exp pairs per step of the second block, so that every 16-key chunk of P is
    // complete before its first PV MFMA
    constexpr int QUOTA = (NPAIR + (NQ / 2 + NP - DB) - 1) / (NQ / 2 + NP - DB);

    // K operand fragment m of a K tile (k-step m / NB, key block m % NB).
    auto read_k = [&](const char* kt, auto mc) {
        constexpr int m = decltype(mc)::value;
        return *reinterpret_cast<const bf16x8*>(kt + koff[m / NB] + (m % NB) * 32 * ROWB);
    };
    // V^T operand fragment j of a V tile: 16-key chunk j / DB = (kb, tt), head-dim
    // block j % DB; two transpose reads of 4 keys each.
    auto read_v = [&](const char* vt, auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int cc = j / DB, kb = cc / 2, tt = cc % 2, db = j % DB;
        constexpr int rowbase = (kb * 32 + 16 * tt) * ROWB;
        const int o_lo = voff[db][0] + rowbase;
        const int o_hi = (VH == 2 ? voff[db][VH - 1] : voff[db][0] + 8 * ROWB) + rowbase;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + o_lo));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + o_hi));
        const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, a16);
    };
    // P for one pair of keys: exp2(s*c - m*c) rounded to BF16; the row sum adds the
    // rounded values.
    auto exp_pair = [&](const f32x16 (&s)[NB], auto pc, float mc, bf16x8 (&pf)[NB][2]) {
        constexpr int pi = decltype(pc)::value;
        constexpr int cc = pi / 4, kb = cc / 2, tt = cc % 2, r = 8 * tt + 2 * (pi % 4);
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc));
        const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_part, false);
        pf[kb][tt][r & 7] = pk[0];
        pf[kb][tt][(r & 7) + 1] = pk[1];
    };
    auto mask_tail = [&](f32x16 (&s)[NB], int t0) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = t0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (key >= kend) s[kb][r] = -INFINITY;
            }
    };
    // Raises the reference maximum (and rescales O and l) only when some row's
    // tile maximum exceeds it by more than 2^kRescaleLog2 in the exp2 domain.
    auto update_max = [&](float mx) {
        const bool need = (mx - m_ref) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f((m_ref - m_new) * c);
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) o[i] *= alpha;
            m_ref = m_new;
        }
        return (m_ref == -INFINITY) ? 0.f : m_ref * c;
    };
    auto sv = [&](const f32x16 (&s)[NB], int e) -> float { return s[e / 16][e % 16]; };

    // S^T = K Q^T for one K tile, unpipelined (first tile).
    auto qk_full = [&](const char* kt, f32x16 (&s)[NB]) {
        static_for<NQ>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            const bf16x8 a = read_k(kt, mc);
            s[m % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, qf[m / NB], m < NB ? f32x16{} : s[m % NB], 0, 0, 0);
        });
    };

    // One pipelined tile: the MFMAs of S(t+1) = K(t+1) Q^T run while S(t) is reduced
    // and exponentiated; then O += P(t) V(t). LDS fragments are read two MFMAs ahead
    // and each MFMA is paired with a fixed slice of VALU work between scheduling
    // fences.
    auto tile_pipelined = [&](const f32x16 (&sc)[NB], f32x16 (&sn)[NB], const char* kt,
                              const char* vt) {
        bf16x8 fr[3];
        auto read_f = [&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f < NQ)
                fr[f % 3] = read_k(kt, fc);
            else
                fr[f % 3] = read_v(vt, std::integral_constant<int, f - NQ>{});
        };
        read_f(std::integral_constant<int, 0>{});
        read_f(std::integral_constant<int, 1>{});
        float mx = fmaxf(sv(sc, 0), sv(sc, 1));
        // score pairs folded into the maximum per step of block 1
        constexpr int MPS = (NB * 8 - 1 + NQ / 2 - 1) / (NQ / 2);
        __builtin_amdgcn_sched_barrier(0);
        // block 1: S(t+1) for the first half of the k-steps; row maximum of S(t)
        static_for<NQ / 2>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            read_f(std::integral_constant<int, i + 2>{});
            sn[i % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                fr[i % 3], qf[i / NB], i < NB ? f32x16{} : sn[i % NB], 0, 0, 0);
            static_for<MPS>([&](auto qc) {
                constexpr int e = 2 + 2 * (i * MPS + decltype(qc)::value);
                if constexpr (e + 1 < NB * 16) mx = fmaxf(fmaxf(mx, sv(sc, e)), sv(sc, e + 1));
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        const float mc = update_max(wave_swap_max(mx));
        // block 2: rest of S(t+1); exponentials of S(t); O += P(t) V(t)
        bf16x8 pf[NB][2];
        static_for<NQ / 2 + NP>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int f = NQ / 2 + i;
            if constexpr (f + 2 < NF) read_f(std::integral_constant<int, f + 2>{});
            if constexpr (f < NQ) {
                sn[f % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % 3], qf[f / NB],
                                                                     sn[f % NB], 0, 0, 0);
            } else {
                constexpr int j = f - NQ;
                constexpr int cc = j / DB, kb = cc / 2, tt = cc % 2, db = j % DB;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % 3], pf[kb][tt], o[db], 0,
                                                                0, 0);
            }
            static_for<QUOTA>([&](auto qc) {
                constexpr int pi = i * QUOTA + decltype(qc)::value;
                if constexpr (pi < NPAIR) exp_pair(sc, std::integral_constant<int, pi>{}, mc, pf);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // Last tile of the range: no next tile; keys past the end are masked.
    auto tile_last = [&](f32x16 (&sc)[NB], int t0, const char* vt) {
        if (t0 + BN > kend) mask_tail(sc, t0);
        float mx = sv(sc, 0);
#pragma unroll
        for (int e = 1; e < NB * 16; ++e) mx = fmaxf(mx, sv(sc, e));
        const float mc = update_max(wave_swap_max(mx));
        bf16x8 pf[NB][2];
        static_for<NPAIR>([&](auto pc) { exp_pair(sc, pc, mc, pf); });
        static_for<NP>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int cc = j / DB, kb = cc / 2, tt = cc % 2, db = j % DB;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vt, jc), pf[kb][tt], o[db], 0,
                                                            0, 0);
        });
    };

    // Pipeline over the tiles of the range. Tile j of K and of V lives in slot
    // j % NSLOT. Three slots: during tile t the loads of K(t+3) and V(t+2) are issued,
    // and at its end only those may still be in flight (K(t+2) and V(t+1) must have
    // landed). Two slots (half the LDS, so two workgroups fit on a CU with 64-key
    // tiles at D = 128): K(t+2) and V(t+1) are issued and waited for within tile t.
    // One barrier per tile.
    const int ntiles = (kend - kbeg + BN - 1) / BN;
    auto kslot = [&](int j) { return smem + (j % NSLOT) * TILEB; };
    auto vslot = [&](int j) { return smem + (NSLOT + j % NSLOT) * TILEB; };
    if constexpr (NSLOT == 1) {
        // every key range of the call is one tile (the launcher checks it). The copies
        // of what only this workgroup reads are non-temporal: its Q rows when the keys
        // are not split, its K and V tile when a (batch, head) has one query block
        // (B=1024 N=64: 185.7 -> 168.1 us with the non-temporal output stores).
        if (p.splits == 1)
            copy_wave_rows_to_lds<D, true>(p.q + qrow0, HD, p.Nq - q0, qo);
        else
            copy_wave_rows_to_lds<D>(p.q + qrow0, HD, p.Nq - q0, qo);
        if (p.m_blocks == 1) {
            issue(kseg0, kseg1, kbeg, smem, std::true_type{});
            issue(vseg0, vseg1, kbeg, smem + TILEB, std::true_type{});
        } else {
            issue_k(kbeg, 0);
            issue_v(kbeg, 0);
        }
        barrier_vmcnt<0>();
        if (active) {
            read_wave_rows_qf<D>(qo, qf);
            f32x16 s1[NB];
            qk_full(kslot(0), s1);
            tile_last(s1, kbeg, vslot(0));
        }
    } else {
    issue_k(kbeg, 0);
    issue_v(kbeg, 0);
    if (ntiles > 1) {
        issue_k(kbeg + BN, 1);
        if constexpr (NSLOT == 3) issue_v(kbeg + BN, 1);
    }
    if (NSLOT == 3 && ntiles > 2) issue_k(kbeg + 2 * BN, 2);
    barrier_vmcnt<0>();
    f32x16 sA[NB], sB[NB];
    if (active) qk_full(kslot(0), sA);
    // K slot 0 is refilled during the first tile
    if constexpr (NSLOT == 3)
        barrier_vmcnt<2 * PER_T>();
    else
        barrier_vmcnt<0>();

    // One tile of the steady state. J = t mod 6 is a compile-time constant, so the
    // LDS slots (period 3) and the score buffers (period 2) fold into immediates.
    auto step = [&](int t, auto jc) {
        constexpr int J = decltype(jc)::value;
        f32x16(&sc)[NB] = (J % 2 == 0) ? sA : sB;
        f32x16(&sn)[NB] = (J % 2 == 0) ? sB : sA;
        const int t0 = kbeg + t * BN;
        const bool more_k = t + NSLOT < ntiles;
        const bool more_v = t + NSLOT - 1 < ntiles;
        if (more_k) issue_k(t0 + NSLOT * BN, J % NSLOT);
        if (more_v) issue_v(t0 + (NSLOT - 1) * BN, (J + NSLOT - 1) % NSLOT);
        if (active)
            tile_pipelined(sc, sn, kslot(J + 1), vslot(J));
        if (NSLOT == 3 && more_k)
            barrier_vmcnt<2 * PER_T>();
        else if (NSLOT == 3 && more_v)
            barrier_vmcnt<PER_T>();
        else
            barrier_vmcnt<0>();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    int t = 0;
    for (; t + 6 < ntiles; t += 6) {
        step(t, I0{});
        step(t + 1, I1{});
        step(t + 2, I2{});
        step(t + 3, I3{});
        step(t + 4, I4{});
        step(t + 5, I5{});
    }
    // 0..5 more pipelined tiles, then the last tile (t is a multiple of 6 here)
    const int rest = ntiles - 1 - t;
    if (rest > 0) step(t, I0{});
    if (rest > 1) step(t + 1, I1{});
    if (rest > 2) step(t + 2, I2{});
    if (rest > 3) step(t + 3, I3{});
    if (rest > 4) step(t + 4, I4{});
    if (active) {
        const int tl = t + rest;
        tile_last((rest % 2 == 0) ? sA : sB, kbeg + tl * BN, vslot(tl));
    }
    }

    if (!active) return;

    // ---- epilogue
    const float l_tot = wave_swap_sum(l_part);
    const int qi = q0 + n;
    // Whole-row stores through LDS: the one-tile form has its own rows; with a ring, no
    // wave reads a K slot after the last tile barrier, and the K slots hold every wave's
    // 32 rows of 2·D bytes (BF16 outputs, or FP32 partials half a row at a time).
    static_assert(NSLOT == 1 || NSLOT * TILEB >= NW * 32 * ROWB, "staging space");
    char* const stage = (NSLOT == 1) ? qo : smem + wave * 32 * ROWB;
    if (p.splits == 1) {
        store_wave_rows_via_lds<D>(o, 1.0f / l_tot, stage, p.out + qrow0, HD, p.Nq - q0);
    } else {
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const long rows = (long)p.B * p.Nq * H;
        store_wave_rows_f32_via_lds<D>(
            o, inv, stage, p.part_o + ((long)split * rows + (long)(b * p.Nq + q0) * H + h) * D,
            HD, p.Nq - q0);
        if (qi < p.Nq) {
            const long row = (long)(b * p.Nq + qi) * H + h;
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
    // Key tile and LDS ring depth: 64-key tiles in three slots at D = 64; at D = 128
    // with 4 waves, 64-key tiles in two slots (64 KiB, two workgroups per CU); with 2
    // waves, 32-key tiles in three slots (48 KiB, three workgroups per CU).
    // When every key range is one 64-key tile (short sequences), one tile in LDS and no
    // ring, with more workgroups per CU.
    if (p.keys_per_split <= kKeyTile) {
        hipLaunchKernelGGL((attn_fwd_kernel<D, NW, kKeyTile, 1>), dim3((unsigned)workgroups),
                           dim3(NW * kWave), 0, stream, p);
        return hipGetLastError();
    }
    constexpr int BN = (D == 128 && NW == 2) ? 32 : kKeyTile;
    constexpr int NSLOT = (D == 128 && NW == 4) ? 2 : 3;
    hipLaunchKernelGGL((attn_fwd_kernel<D, NW, BN, NSLOT>), dim3((unsigned)workgroups),
                       dim3(NW * kWave), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_fwd(int D, int waves, const FwdParams& p, long long workgroups,
                      hipStream_t stream) {
    if (waves == 8) return launch_fwd_pingpong(D, p, workgroups, stream);
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
