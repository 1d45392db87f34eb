// Ping-pong attention forward kernel for MI355X (gfx950), for grids with many query
// blocks. Same operation and data layout per wave as attn_fwd_kernel in
// attn_kernels.hip (page "Audit SGLang interfaces and refresh validated kernel
// solutions": the noncausal dense and prefix-cached attention definitions, FP32
// accumulation, BF16 output), with a different schedule:
//
//   * A workgroup has 8 waves (256 query rows, 32 per wave) in two groups of 4; wave
//     w and wave w + 4 share a SIMD. Every tile of 64 keys is processed in two
//     phases per wave: G (MFMA: S(t) = K(t) Q^T and O += P(t-1) V(t-1)) and S
//     (VALU: online softmax of S(t) into P(t)). Group 1 runs one phase behind group
//     0, and all waves meet at one barrier per phase, so on every SIMD one wave
//     issues MFMAs while the other works through the softmax.
//   * K and V tiles stream global -> LDS (global_load_lds_dwordx4) into three-slot
//     rings, two tiles ahead; the barrier before a tile's first use waits only for
//     the copies it needs.
//   * Tile phases are unrolled by 3 so the LDS slot of every access is a
//     compile-time offset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

using namespace dev;

// Block-causal visibility (page "Audit SGLang interfaces and refresh validated kernel
// solutions", definitions/block_causal_attention/
// prefix_cached_block_causal_h32_d128_prefix0.json): query i sees key j when j <= i,
// or when image_ids[i] >= 0 and image_ids[j] == image_ids[i].
//
// End (exclusive) of the keys rows [qa, qb] may see: every key up to qb, plus the
// 64-key tiles after qb whose range of nonnegative ids overlaps the rows' range
// (conservative; the per-element mask decides). Lane-parallel over tiles, the result
// is uniform across the wave.
__device__ int bc_key_end(const int* meta, int n, int qa, int qb, int lane) {
    int qmin = 0x7fffffff, qmax = -1;
    for (int blk = qa / kMetaRows; blk <= qb / kMetaRows; ++blk) {
        qmin = min(qmin, meta[4 * blk]);
        qmax = max(qmax, meta[4 * blk + 1]);
    }
    const int end = qb + 1;
    if (qmax < 0) return end;  // only text rows: causal
    const int nblk = (n + kMetaRows - 1) / kMetaRows;
    const int tiles = (n + 63) / 64;
    const int first = qb / 64 + 1;  // first tile that starts after row qb
    for (int base = first + ((tiles - first - 1) / 64) * 64; base >= first; base -= 64) {
        const int tt = base + lane;
        bool hit = false;
        if (tt < tiles) {
            const int b0 = 2 * tt, b1 = min(2 * tt + 1, nblk - 1);
            const int kmin = min(meta[4 * b0], meta[4 * b1]);
            const int kmax = max(meta[4 * b0 + 1], meta[4 * b1 + 1]);
            hit = kmax >= qmin && kmin <= qmax;
        }
        const unsigned long long m = __builtin_amdgcn_ballot_w64(hit);
        if (m) {
            const int top = base + 63 - __builtin_clzll(m);
            return max(end, min(n, 64 * top + 64));
        }
    }
    return end;
}

template <int D, bool BC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_pp_kernel(FwdParams p) {
    static_assert(D == 64 || D == 128, "head dim");
    constexpr int NW = 8;
    constexpr int NT = NW * kWave;
    // keys per tile (a multiple of 32): 128 at D = 64, so a phase holds as many MFMAs as at
    // D = 128 and the barriers per key halve (4-6% faster); the block-causal form keeps 64,
    // the granularity of its key ends
    constexpr int BN = (D == 64 && !BC) ? 128 : 64;
    constexpr int NB = BN / 32;            // 32-key blocks per tile
    constexpr int KS = D / 16;             // MFMA k-steps over the head dim
    constexpr int DB = D / 32;             // 32-wide head-dim blocks of O^T
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int ROWB = 2 * D;            // bytes per LDS row
    constexpr int TILEB = BN * ROWB;       // bytes per K or V tile
    constexpr int PER_T = BN * CPR / NT;   // 16-byte copies per thread per tensor per tile
    constexpr int RSTEP = NT / CPR;        // rows per copy round
    constexpr int NTG = NT / 2;            // threads of one wave group
    constexpr int PER_G = BN * CPR / NTG;  // copies per thread of a group copying a tile
    constexpr int RSTEP_G = NTG / CPR;     // rows per copy round of a group
    constexpr int NSLOT = 3;
    constexpr int NQ = KS * NB;            // QK^T MFMAs per tile
    constexpr int NP = 2 * NB * DB;        // PV MFMAs per tile
    constexpr int NPAIR = NB * 8;          // exp pairs per lane per tile
    static_assert(BN * CPR % NT == 0 && RSTEP % 16 == 0, "loader pattern");
    static_assert(BN * CPR % NTG == 0 && RSTEP_G % 16 == 0, "group loader pattern");

    // K ring, V ring, then each wave's 32 query rows (Q on the way in, O on the way out)
    constexpr int WB = 32 * ROWB;
    __shared__ __attribute__((aligned(1024))) char smem[2 * NSLOT * TILEB + NW * WB];

    int mb, bh, split;
    decode_workgroup(p.m_blocks, p.B * p.H, mb, bh, split, BC);
    const int H = p.H;
    const int b = bh / H;
    const int h = bh - b * H;
    const int HD = H * D;
    const int n0 = p.n0;
    const int nk = n0 + p.n1;
    const int kbeg = split * p.keys_per_split;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    // block-causal: the keys of this workgroup's rows stop at their last visible tile
    // (one key split)
    const int kend =
        BC ? min(nk, bc_key_end(p.meta, p.Nq, mb * (NW * 32), min(mb * (NW * 32) + NW * 32 - 1,
                                                                   p.Nq - 1), lane))
           : min(nk, kbeg + p.keys_per_split);
    const int T = (kend - kbeg + BN - 1) / BN;

    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int grp = wave >> 2;
    const int n = lane & 31;
    const int g = lane >> 5;
    const int q0 = mb * (NW * 32) + wave * 32;
    const bool active = q0 < p.Nq;
    // block-causal: this lane's query image id, and whether the wave's 32 rows all
    // carry one nonnegative id (then a tile of keys with only that id is fully visible)
    int idq = -1, wq_id = -1, wq_max = -1;
    bool wq_uniform = false;
    if constexpr (BC) {
        idq = p.ids[min(q0 + n, p.Nq - 1)];
        if (active) {
            const int* wm = p.meta + 4 * (q0 / kMetaRows);
            wq_uniform = wm[2] == 0 && wm[0] == wm[1];
            wq_id = wm[0];   // smallest nonnegative id of the rows
            wq_max = wm[1];  // largest (-1: text rows only)
        }
    }

    const uint16_t* kseg0 = uniform_ptr(p.k0 + ((long)b * n0 * HD + (long)h * D));
    const uint16_t* vseg0 = uniform_ptr(p.v0 + ((long)b * n0 * HD + (long)h * D));
    const uint16_t* kseg1 =
        uniform_ptr(p.k1 ? p.k1 + ((long)b * p.n1 * HD + (long)h * D) : kseg0);
    const uint16_t* vseg1 =
        uniform_ptr(p.v1 ? p.v1 + ((long)b * p.n1 * HD + (long)h * D) : vseg0);

    // Q^T fragments (B operand): lane holds query n, dims 16*ks + 8g .. +7.
    // They arrive through the wave's LDS rows (below): lane i of round r copies 16-byte
    // chunk 64 r + i of the wave's 32 rows, swizzled like the K/V rows, so each copy
    // instruction covers whole rows rather than 32 bytes of 32 rows. Without a key split no
    // other workgroup reads these rows, so they take the non-temporal path and leave L2 to
    // the K/V tiles that every query tile of the head re-reads.
    bf16x8 qf[KS];
    char* const qo = smem + 2 * NSLOT * TILEB + wave * WB;
    auto issue_q = [&]() {
        static_for<CPR / 2>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int id = i * kWave + lane;
            const int r = id / CPR;
            const int lc = (id % CPR) ^ lds_swizzle<CPR>(r);
            const int qi = min(q0 + r, p.Nq - 1);
            const uint16_t* const src = p.q + ((long)(b * p.Nq + qi) * H + h) * D + lc * 8;
            if (p.splits == 1)
                load16_to_lds<true>(src, qo + i * kWave * 16);
            else
                load16_to_lds(src, qo + i * kWave * 16);
        });
    };

    // Loader: copy round i of thread tid fills physical chunk i*NT + tid of a tile:
    // row r = (i*NT + tid) / CPR, chunk position tid % CPR holding logical chunk
    // (tid % CPR) ^ swizzle(r). Rounds advance by RSTEP rows, a multiple of the
    // swizzle period, so one per-lane offset serves every round.
    const int ld_row0 = tid / CPR;
    const int ld_off = ld_row0 * HD + ((tid % CPR) ^ lds_swizzle<CPR>(ld_row0)) * 8;
    auto issue = [&](const uint16_t* seg0, const uint16_t* seg1, int t0, char* slot) {
        char* const dst = slot + wave * kWave * 16;
        const bool whole = (t0 + BN <= kend) && (t0 + BN <= n0 || t0 >= n0);
        if (whole) {
            const long rowoff = (t0 < n0) ? (long)t0 * HD : (long)(t0 - n0) * HD;
            const uint16_t* base = ((t0 < n0) ? seg0 : seg1) + rowoff;
#pragma unroll
            for (int i = 0; i < PER_T; ++i)  // uniform base, per-lane offset
                load16_to_lds_sbase(base + (long)i * RSTEP * HD, 2u * ld_off, dst + i * NT * 16);
        } else {
            // ragged or segment-straddling tile: clamp rows into [t0, kend) and pick
            // the segment per row
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int r = ld_row0 + i * RSTEP;
                const int key = min(t0 + r, kend - 1);
                const int co = ld_off - ld_row0 * HD;
                const uint16_t* src =
                    key < n0 ? seg0 + (long)key * HD : seg1 + (long)(key - n0) * HD;
                load16_to_lds(src + co, dst + i * NT * 16);
            }
        }
    };
    // Group loader: the same pattern over the 256 threads of this wave's group, so one
    // group copies a whole tile (the group in its softmax phase issues the copies; the
    // other one goes straight to its MFMAs).
    const int tidg = tid & (NTG - 1);
    const int ldg_row0 = tidg / CPR;
    const int ldg_off = ldg_row0 * HD + ((tidg % CPR) ^ lds_swizzle<CPR>(ldg_row0)) * 8;
    auto issue_g = [&](const uint16_t* seg0, const uint16_t* seg1, int t0, char* slot) {
        char* const dst = slot + (wave & 3) * kWave * 16;
        const bool whole = (t0 + BN <= kend) && (t0 + BN <= n0 || t0 >= n0);
        if (whole) {
            const long rowoff = (t0 < n0) ? (long)t0 * HD : (long)(t0 - n0) * HD;
            const uint16_t* base = ((t0 < n0) ? seg0 : seg1) + rowoff;
#pragma unroll
            for (int i = 0; i < PER_G; ++i)  // uniform base, per-lane offset
                load16_to_lds_sbase(base + (long)i * RSTEP_G * HD, 2u * ldg_off,
                                    dst + i * NTG * 16);
        } else {
#pragma unroll
            for (int i = 0; i < PER_G; ++i) {
                const int r = ldg_row0 + i * RSTEP_G;
                const int key = min(t0 + r, kend - 1);
                const int co = ldg_off - ldg_row0 * HD;
                const uint16_t* src =
                    key < n0 ? seg0 + (long)key * HD : seg1 + (long)(key - n0) * HD;
                load16_to_lds(src + co, dst + i * NTG * 16);
            }
        }
    };
    auto kslot = [&](int j) { return smem + j * TILEB; };
    auto vslot = [&](int j) { return smem + (NSLOT + j) * TILEB; };
    auto issue_k = [&](int t0, int slot) { issue(kseg0, kseg1, t0, kslot(slot)); };
    auto issue_v = [&](int t0, int slot) { issue(vseg0, vseg1, t0, vslot(slot)); };
    auto issue_kg = [&](int t0, int slot) { issue_g(kseg0, kseg1, t0, kslot(slot)); };
    auto issue_vg = [&](int t0, int slot) { issue_g(vseg0, vseg1, t0, vslot(slot)); };

    // Per-lane LDS byte offsets: K operand reads per k-step, V transpose reads per
    // head-dim block and 8-key half.
    int koff[KS];
    {
        const int tsw = lds_swizzle<CPR>(n) ^ g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = n * ROWB + 16 * ((2 * ks) ^ tsw);
    }
    int voff[DB][2];
    {
        const int tr_r = (lane & 15) >> 2;
        const int tr_q = lane & 3;
        const int half = (lane >> 4) & 1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int row = 8 * h2 + 4 * g + tr_r;
                const int c = (4 * db + 2 * half + (tr_q >> 1)) ^ lds_swizzle<CPR>(row);
                voff[db][h2] = row * ROWB + 16 * c + 8 * (tr_q & 1);
            }
    }

    f32x16 o[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] = f32x16{};
    f32x16 s[NB];       // scores of the tile between its G and S phases
    bf16x8 pf[NB][2];   // probabilities of the tile between its S and next G phases
    float m_ref = -INFINITY;
    float mc_ref = 0.f;        // m_ref * c (0 while m_ref is -inf)
    bool lazy_ok = false;      // wave-uniform: the next tile may skip its row maximum
    bool eager_rows = false;   // wave-uniform: these rows stay on the row-maximum path
    float l_part = 0.f;
    const float c = p.c;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    auto read_k = [&](const char* kt, auto mc) {
        constexpr int m = decltype(mc)::value;
        return *reinterpret_cast<const bf16x8*>(kt + koff[m / NB] + (m % NB) * 32 * ROWB);
    };
    auto read_v = [&](const char* vt, auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int cc = j / DB, kb = cc / 2, tt = cc % 2, db = j % DB;
        constexpr int rowbase = (kb * 32 + 16 * tt) * ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + voff[db][0] + rowbase));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vt + voff[db][1] + rowbase));
        const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, a16);
    };

    // G phase: MFMAs of S(t) (QK) and O += P(t-1) V(t-1) (PV), interleaved, with LDS
    // operand fragments read PF MFMAs ahead.
    auto g_phase = [&](const char* kt, const char* vt, auto qk_c, auto pv_c) {
        constexpr bool QK = decltype(qk_c)::value;
        constexpr bool PV = decltype(pv_c)::value;
        constexpr int NF = (QK ? NQ : 0) + (PV ? NP : 0);
        // fragment f: with both, even f = QK m = f/2, odd f = PV j = f/2
        auto is_qk = [](int f) { return QK && (!PV || (f % 2 == 0)); };
        auto idx = [](int f) { return (QK && PV) ? f / 2 : f; };
        constexpr int PF = 3;  // fragments read ahead of their MFMA
        bf16x8 fr[PF + 1];
        auto read_f = [&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (is_qk(f))
                fr[f % (PF + 1)] = read_k(kt, std::integral_constant<int, idx(f)>{});
            else
                fr[f % (PF + 1)] = read_v(vt, std::integral_constant<int, idx(f)>{});
        };
        static_for<PF>([&](auto fc) { read_f(fc); });
        static_for<NF>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            if constexpr (f + PF < NF) read_f(std::integral_constant<int, f + PF>{});
            if constexpr (is_qk(f)) {
                constexpr int m = idx(f);
                s[m % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    fr[f % (PF + 1)], qf[m / NB], (m < NB) ? f32x16{} : s[m % NB], 0, 0, 0);
            } else {
                constexpr int j = idx(f);
                constexpr int cc = j / DB, kb = cc / 2, tt = cc % 2, db = j % DB;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % (PF + 1)], pf[kb][tt],
                                                                o[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // S phase: online softmax of S(t) (tile starting at key t0) into P(t).
    // Block-causal mask of the tile at key t0 (keys >= kend hidden as well). Skipped
    // when every key of the tile is visible to every row of the wave: the tile lies
    // at or below the wave's first row, or keys and rows all carry the same image id.
    // Returns false when no key of the tile is visible to any row of the wave (every
    // key after the wave's last row, and no image id shared with the rows): the caller
    // then sets the probabilities to zero without computing them.
    // The classes of the wave's tiles u0 .. u0 + 63 (bit u - u0), one lane per tile from the
    // row-block summaries: every key visible to every row (full), or none to any (hidden).
    unsigned long long bc_full = 0, bc_hidden = 0;
    int bc_u0 = 0;
    auto bc_classify = [&](int u0) {
        const int u = u0 + lane;
        const int t0 = kbeg + u * BN;
        bool full = false, hidden = false;
        if (t0 < kend) {
            const bool whole = t0 + BN <= kend;
            full = whole && t0 + BN - 1 <= q0;
            if (!full) {
                const int nblk = (p.Nq + kMetaRows - 1) / kMetaRows;
                // summaries of the tile's NB row blocks of 32 keys
                int kmin = 0x7fffffff, kmax = -1;
                bool uni = true;
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) {
                    const int* km = p.meta + 4 * min(t0 / kMetaRows + kb, nblk - 1);
                    kmin = min(kmin, km[0]);
                    kmax = max(kmax, km[1]);
                    uni = uni && km[2] == 0 && km[0] == wq_id && km[1] == wq_id;
                }
                hidden = t0 > q0 + 31 && (wq_max < 0 || kmax < wq_id || kmin > wq_max);
                if (!hidden && whole && wq_uniform) full = uni;
            }
        }
        bc_full = __builtin_amdgcn_ballot_w64(full);
        bc_hidden = __builtin_amdgcn_ballot_w64(hidden);
        bc_u0 = u0;
    };
    auto bc_mask = [&](int t0) __attribute__((always_inline)) {
        const int u = (t0 - kbeg) / BN;
        if (u - bc_u0 >= 64) bc_classify(u);
        const unsigned long long bit = 1ull << (u - bc_u0);
        if (bc_hidden & bit) return false;
        if (bc_full & bit) return true;
        const int i = q0 + n;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                // registers 4 q4 .. 4 q4 + 3 hold keys j0 .. j0 + 3
                const int j0 = t0 + kb * 32 + 8 * q4 + 4 * g;
                int idk[4];
                if (j0 + 3 < p.Nq) {
                    const int4 v4 = *reinterpret_cast<const int4*>(p.ids + j0);
                    idk[0] = v4.x;
                    idk[1] = v4.y;
                    idk[2] = v4.z;
                    idk[3] = v4.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) idk[e] = p.ids[min(j0 + e, p.Nq - 1)];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + e;
                    const bool vis = j < kend && (j <= i || (idq >= 0 && idk[e] == idq));
                    if (!vis) s[kb][4 * q4 + e] = -INFINITY;
                }
            }
        return true;
    };

    auto s_phase = [&](int t0) __attribute__((always_inline)) {
        if constexpr (BC) {
            if (!bc_mask(t0)) {  // nothing visible: P = 0, running max and sums unchanged
#pragma unroll
                for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) pf[kb][tt] = bf16x8{};
                return;
            }
        } else if (t0 + BN > kend) {
            // register r of block kb holds key t0 + 32 kb + 8 (r / 4) + 4 g + r % 4; the
            // keys from kend on get -inf by bit selection against one per-lane limit (no
            // per-register offsets or compare masks to keep live)
            const int lim = kend - t0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    const int hide = (lim - off - 1) >> 31;  // all ones when off >= lim
                    s[kb][r] = __int_as_float((__float_as_int(s[kb][r]) & ~hide) |
                                              (int)(0xff800000u & (unsigned)hide));
                }
        }
        if (lazy_ok) {
            // Lazy tile (every tile after the rows' first): probabilities against the
            // running reference m_ref, without the tile's row maximum. The lane's sum of
            // its probabilities bounds each of them; if no sum exceeds kLazySumLimit and
            // all are finite, the tile is done (the reference may lag the true maximum:
            // O and l share it, so O / l is unchanged). Otherwise the tile is redone
            // below against its own maximum, as is every later tile of these rows.
            float l2[2] = {0.f, 0.f};
            static_for<NPAIR>([&](auto pc) {
                constexpr int pi = decltype(pc)::value;
                constexpr int cc = pi / 4, kb = cc / 2, tt = cc % 2, r = 8 * tt + 2 * (pi % 4);
                const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc_ref));
                const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc_ref));
                const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
                l2[pi % 2] = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l2[pi % 2], false);
                pf[kb][tt][r & 7] = pk[0];
                pf[kb][tt][(r & 7) + 1] = pk[1];
            });
            const float ls = l2[0] + l2[1];
            if (__builtin_amdgcn_ballot_w64(!(ls <= kLazySumLimit)) == 0) {
                l_part += ls;
                return;
            }
            lazy_ok = false;  // redo this tile, and every later one of these rows, eagerly
            eager_rows = true;
        }
        // row maximum: four independent chains of EPC consecutive registers, then one
        // exchange with lane ^ 32
        constexpr int EPC = NB * 4;
        auto sv = [&](int e) __attribute__((always_inline)) { return s[e / 16][e % 16]; };
        float m4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) m4[k] = fmaxf(sv(k * EPC), sv(k * EPC + 1));
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int r = 2; r < EPC; r += 2)
                m4[k] = fmaxf(fmaxf(m4[k], sv(k * EPC + r)), sv(k * EPC + r + 1));
        const float mx = wave_swap_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
        const bool need = (mx - m_ref) * c > kRescaleLog2;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = (m_ref == -INFINITY) ? 0.f : exp2f((m_ref - m_new) * c);
            l_part *= alpha;
#pragma unroll
            for (int i = 0; i < DB; ++i) o[i] *= alpha;
            m_ref = m_new;
            mc_ref = (m_ref == -INFINITY) ? 0.f : m_ref * c;
        }
        const float mc = mc_ref;
        float l2[2] = {0.f, 0.f};
        static_for<NPAIR>([&](auto pc) {
            constexpr int pi = decltype(pc)::value;
            constexpr int cc = pi / 4, kb = cc / 2, tt = cc % 2, r = 8 * tt + 2 * (pi % 4);
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc));
            const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
            l2[pi % 2] = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l2[pi % 2], false);
            pf[kb][tt][r & 7] = pk[0];
            pf[kb][tt][(r & 7) + 1] = pk[1];
        });
        l_part += l2[0] + l2[1];
        // After the rows' first tile: the later tiles go lazy when every row has a finite
        // reference of moderate size. Rows whose logits reach beyond 2^kLazyRefLog2 tend
        // to keep growing past kLazySumLimit, so they stay on this path for good.
        if (!eager_rows) {
            eager_rows = __builtin_amdgcn_ballot_w64(
                             !(m_ref > -INFINITY && fabsf(mc_ref) <= kLazyRefLog2)) != 0;
            lazy_ok = !eager_rows;
        }
    };

    using TRUE_ = std::true_type;
    using FALSE_ = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;

    // ---- prologue: the wave's Q rows, K(0), K(1), V(0) resident before phase 0
    issue_q();
    issue_k(kbeg, 0);
    if (T > 1) issue_k(kbeg + BN, 1);
    issue_v(kbeg, 0);
    if constexpr (BC) {
        if (active) bc_classify(0);
    }
    barrier_vmcnt<0>();
    {
        const int tsw = lds_swizzle<CPR>(n) ^ g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(qo + n * ROWB + 16 * ((2 * ks) ^ tsw));
    }

    // Each group runs its own straight-line phase sequence; both execute the same
    // barriers in the same order. Group 0: G(u) then S(u) in tile u; group 1: S(u-1)
    // then G(u).
    auto run = [&](auto grp_c) {
        constexpr int GRP = decltype(grp_c)::value;
        // phase 0 (tile 0): group 1 copies K(2); group 0 computes S(0)
        if (GRP == 1 && T > 2) issue_kg(kbeg + 2 * BN, 2);
        if (GRP == 0 && active) g_phase(kslot(0), vslot(0), TRUE_{}, FALSE_{});
        barrier_vmcnt<63>();
        // phase 1: group 0 copies V(1) and runs the softmax of tile 0, group 1
        // computes S(0)
        if (GRP == 0 && T > 1) issue_vg(kbeg + BN, 1);
        if (active) {
            if (GRP == 0)
                s_phase(kbeg);
            else
                g_phase(kslot(0), vslot(0), TRUE_{}, FALSE_{});
        }
        // steady state: tile u in 1 .. T-1 (phases 2u and 2u+1); J = u mod 3
        auto tile = [&](int u, auto jc) {
            constexpr int J = decltype(jc)::value;
            const int t0 = kbeg + u * BN;
            // This tile reads K(u) and V(u-1). Group 1 copies the K tiles (first phase
            // of a tile), group 0 the V tiles (second phase); each waits for its own:
            // group 1 may keep K(u+1) in flight, group 0 V(u).
            if (GRP == 1) {
                if (u + 1 < T)
                    barrier_vmcnt<PER_G>();
                else
                    barrier_vmcnt<0>();
            } else {
                barrier_vmcnt<PER_G>();
            }
            if (GRP == 1 && u + 2 < T) issue_kg(t0 + 2 * BN, (J + 2) % NSLOT);
            if (active) {
                if (GRP == 0)
                    g_phase(kslot(J), vslot((J + 2) % NSLOT), TRUE_{}, TRUE_{});
                else
                    s_phase(t0 - BN);
            }
            barrier_vmcnt<63>();
            if (GRP == 0 && u + 1 < T) issue_vg(t0 + BN, (J + 1) % NSLOT);
            if (active) {
                if (GRP == 0)
                    s_phase(t0);
                else
                    g_phase(kslot(J), vslot((J + 2) % NSLOT), TRUE_{}, TRUE_{});
            }
        };
        int u = 1;
        for (; u + 2 < T; u += 3) {
            tile(u, I1{});
            tile(u + 1, I2{});
            tile(u + 2, I0{});
        }
        if (u < T) {
            tile(u, I1{});
            ++u;
        }
        if (u < T) {
            tile(u, I2{});
            ++u;
        }
        // tail (tile T): O += P(T-1) V(T-1)
        barrier_vmcnt<0>();
        const char* vlast = vslot((T - 1) % NSLOT);
        if (active) {
            if (GRP == 0)
                g_phase(kslot(0), vlast, FALSE_{}, TRUE_{});
            else
                s_phase(kbeg + (T - 1) * BN);
        }
        barrier_vmcnt<63>();
        if (GRP == 1 && active) g_phase(kslot(0), vlast, FALSE_{}, TRUE_{});
    };
    if (grp == 0)
        run(I0{});
    else
        run(I1{});

    if (!active) return;

    // ---- epilogue
    const float l_tot = wave_swap_sum(l_part);
    const int qi = q0 + n;
    if (p.splits == 1) {
        // The output rows go out through the wave's LDS rows so that each store covers
        // whole rows (16 or 8 lanes per row) rather than 8 bytes of 32 rows; nothing here
        // reads them again, so the stores are non-temporal.
        char* const stage = qo;
        const float inv = 1.0f / l_tot;
        const int sw = lds_swizzle<CPR>(n);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * j + e] * inv);
                // row n, chunk 4 db + j holds dims 32 db + 8 j ..
                *reinterpret_cast<bf16x4*>(stage + n * ROWB + 16 * ((4 * db + j) ^ sw) + 8 * g) = v;
            }
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        __asm__ volatile("" ::: "memory");
        static_for<CPR / 2>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int id = i * kWave + lane;
            const int r = id / CPR;
            const int pc = id % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * ROWB + 16 * pc);
            if (q0 + r < p.Nq)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.out + ((long)(b * p.Nq + q0 + r) * H + h) * D +
                                          (pc ^ lds_swizzle<CPR>(r)) * 8));
        });
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

// Summaries of the image ids, kMetaRows per block: thread i reads id i (coalesced);
// each group of 32 lanes reduces its block with lane exchanges. Rows past n count as
// neither text nor image.
__global__ void attn_bc_meta_kernel(const int* ids, int n, int* meta) {
    static_assert(kMetaRows == 32, "one half-wave per block of ids");
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int id = i < n ? ids[i] : -1;
    int lo = (i < n && id >= 0) ? id : 0x7fffffff;
    int hi = (i < n && id >= 0) ? id : -1;
    int text = (i < n && id < 0) ? 1 : 0;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
        lo = min(lo, __shfl_xor(lo, off, 32));
        hi = max(hi, __shfl_xor(hi, off, 32));
        text += __shfl_xor(text, off, 32);
    }
    if ((i % kMetaRows) == 0 && i < n) {
        int4 m;
        m.x = lo;
        m.y = hi;
        m.z = text;
        m.w = 0;
        reinterpret_cast<int4*>(meta)[i / kMetaRows] = m;
    }
}

}  // namespace

hipError_t launch_fwd_pingpong(int D, const FwdParams& p, long long workgroups,
                               hipStream_t stream) {
    if (D == 64)
        hipLaunchKernelGGL((attn_fwd_pp_kernel<64, false>), dim3((unsigned)workgroups),
                           dim3(512), 0, stream, p);
    else if (D == 128)
        hipLaunchKernelGGL((attn_fwd_pp_kernel<128, false>), dim3((unsigned)workgroups),
                           dim3(512), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fwd_block_causal(int D, const FwdParams& p, long long workgroups,
                                   hipStream_t stream) {
    if (!p.ids || !p.meta || p.splits != 1) return hipErrorInvalidValue;
    if (D == 64)
        hipLaunchKernelGGL((attn_fwd_pp_kernel<64, true>), dim3((unsigned)workgroups),
                           dim3(512), 0, stream, p);
    else if (D == 128)
        hipLaunchKernelGGL((attn_fwd_pp_kernel<128, true>), dim3((unsigned)workgroups),
                           dim3(512), 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_bc_meta(const int* ids, int n, int* meta, hipStream_t stream) {
    hipLaunchKernelGGL(attn_bc_meta_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, ids, n, meta);
    return hipGetLastError();
}

}  // namespace attn
