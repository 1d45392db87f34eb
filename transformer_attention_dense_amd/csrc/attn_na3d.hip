// 3-D neighborhood attention forward kernel for MI355X (gfx950), D = 64 (page "Audit
// SGLang interfaces and refresh validated kernel solutions",
// definitions/neighborhood_attention/neighborhood_attention_3d_*: natten's na3d with
// kernel (kt, ky, kx) and scale 1, Q already scaled, layout [B, T, Y, X, H, D]; the
// neighborhood is NATTEN's: on each axis an odd window centred on the query, moved
// inside the axis at its ends).
//
// A wave owns 32 queries of one (b, t, h): QA rows y x QB positions on X (QB = 16, 8 or
// 4, QA = 32 / QB, picked per window shape); a workgroup holds four waves on 1, 2 or 4
// frames t (4, 2 or 1 tiles of QA rows each), arranged where their windows overlap most. Every
// (t', y') row of a query's window is a run of consecutive positions on X, and the X
// windows of the QB positions lie in the KW positions starting at the window of the first
// one (KW = 32 for QB = 16, 16 for QB = 8, 16 or 8 for QB = 4; kx <= KW - QB + 1), so a key
// block of 32 keys holds KW positions of 32 / KW rows. The workgroup walks the union of its waves' Y windows for
// each t' of the union of their T windows as such blocks, streamed through a four-slot LDS ring
// exactly like the dense kernels stream key tiles; each block is copied once and used by
// every wave whose rows' windows reach its rows:
//
//   * copy the K and V block (global_load_lds_dwordx4, scalar base + per-lane offsets
//     fixed for the workgroup; positions past the end of the X axis are clamped and never
//     visible), three blocks ahead of their use;
//   * S^T = K Q^T with 32x32x16 BF16 MFMAs (S in FP32), accumulated onto a per-lane
//     0/-inf mask of the keys outside its query's X window; where the block is not inside
//     every Y window of the wave, the rows outside a query's window are left out of its
//     maximum and its exponentials of them get a reference of +inf (so they are 0);
//   * online softmax in the exp2 domain (scale 1, so c = log2 e), P rounded to BF16;
//   * O^T += V^T P^T with the V operand read transposed from LDS (ds_read_b64_tr_b16).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_device.h"
#include "attn_launch.h"

namespace attn {
namespace {

using namespace dev;

// start of the window of odd size k around i on an axis of length L (k <= L)
__device__ __forceinline__ int na_start(int i, int k, int L) {
    return max(0, min(i - k / 2, L - k));
}

// Barrier after waiting for the copies of all but the min(left, K) most recently issued
// tiles (two loads per tile: K and V); left is uniform.
template <int K>
__device__ __forceinline__ void barrier_tiles_left(int left) {
    if constexpr (K == 0) {
        barrier_vmcnt<0>();
    } else {
        if (left >= K)
            barrier_vmcnt<2 * K>();
        else
            barrier_tiles_left<K - 1>(left);
    }
}

constexpr int kNaWaves = 4;  // waves per workgroup (frames x row tiles: na3d_configure)

// Workgroup -> (b, block of frames t, block of rows y, strip of QB positions on X, h). Each XCD
// (it runs the workgroups whose linear ids are equal mod 8) gets a contiguous range of
// the order (b, h, ...), so the workgroups of a head, whose windows share K/V rows, run
// on one XCD and meet the rows in its L2. Within a head: t slowest, then the block of
// rows y, strip fastest; or (t_inner) t fastest, then strip, block of rows slowest,
// which the host picks when a head has to be shared by several XCDs and cutting it
// along Y or X duplicates fewer K/V rows than cutting it along T.
// t is the workgroup's block of wt frames (its waves' frames wt t .. wt t + wt - 1).
__device__ __forceinline__ void na_decode(const NaParams& p, int& b, int& t, int& yblk,
                                          int& strip, int& h) {
    long idx = blockIdx.x;
    const long per = (long)gridDim.x >> 3;
    if (idx < (per << 3)) idx = (idx & 7) * per + (idx >> 3);
    const int nt = (p.T + p.wt - 1) / p.wt;
    if (p.t_inner) {
        t = (int)(idx % nt);
        idx /= nt;
        strip = (int)(idx % p.strips);
        idx /= p.strips;
        yblk = (int)(idx % p.yblocks);
        idx /= p.yblocks;
    } else {
        strip = (int)(idx % p.strips);
        idx /= p.strips;
        yblk = (int)(idx % p.yblocks);
        idx /= p.yblocks;
        t = (int)(idx % nt);
        idx /= nt;
    }
    h = (int)(idx % p.H);
    b = (int)(idx / p.H);
}

// Query tile of a wave: QA rows y x QB positions on X (32 queries). A key block is RPB
// rows of KW positions on X (32 keys), the X windows of the QB positions lying in the KW
// positions from the window of the first one (so kx <= KW - QB + 1). Register r of a lane
// holds key 8 (r / 4) + 4 g + r % 4 of the block, so row hr of the block is registers
// 16 / RPB * hr .. 16 / RPB * (hr + 1) - 1.
template <int QB, int KW_>
struct NaTile {
    static constexpr int QA = 32 / QB;
    static constexpr int KW = KW_;
    static constexpr int RPB = 32 / KW;
    static constexpr int max_kx = KW - QB + 1;
};

// Four waves per SIMD (at most 128 VGPRs): the kernel is latency bound, and above 128
// registers the compiler keeps the MFMA accumulators in AGPRs and copies them around.
template <int QB, int KW_>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void attn_na3d_kernel(NaParams p) {
    using Tile = NaTile<QB, KW_>;
    constexpr int QA = Tile::QA, KW = Tile::KW, RPB = Tile::RPB;
    constexpr int D = 64;
    constexpr int KS = D / 16;       // MFMA k-steps over the head dim
    constexpr int DB = D / 32;       // 32-wide head-dim blocks of O^T
    constexpr int CPR = D / 8;       // 16-byte chunks per row
    constexpr int ROWB = 2 * D;      // bytes per LDS row
    constexpr int BN = 32;           // keys per block
    constexpr int TILEB = BN * ROWB; // bytes per K or V block
    constexpr int NT = kNaWaves * kWave;
    static_assert(BN * CPR == NT, "one 16-byte copy per thread per tensor and block");
    constexpr int NSLOT = 4;         // LDS ring slots
    constexpr int AHEAD = NSLOT - 1; // blocks copied ahead of the one in use
    constexpr int NPAIR = 8;         // exp pairs per lane per block

    __shared__ __attribute__((aligned(1024))) char smem[NSLOT * 2 * TILEB];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n = lane & 31;
    const int g = lane >> 5;

    int b, tb, yblk, strip, h;
    na_decode(p, b, tb, yblk, strip, h);

    // The workgroup's four waves: wt frames (wt tb ..) by 4 / wt tiles of QA rows (from row
    // yblk * (4 / wt) * QA); wave w is frame w / (4 / wt), row tile w % (4 / wt)
    const int X = p.X, Y = p.Y;
    const long HD = (long)p.H * D;
    const int ay = kNaWaves / p.wt;                          // row tiles of the workgroup
    const int t = p.wt * tb + wave / ay;                     // the wave's frame
    const int wy0 = (yblk * ay + wave % ay) * QA;            // its first row y
    const bool active = wy0 < Y && t < p.T;
    const int yq = wy0 + n / QB;            // this lane's query row
    const int xq = strip * QB + n % QB;     // and position on X
    const int yqc = min(yq, Y - 1), xqc = min(xq, X - 1);
    const int tqc = min(t, p.T - 1);
    const long pos_q = (((long)b * p.T + tqc) * Y + yqc) * X + xqc;

    // Q^T fragments (B operand): lane holds query n, dims 16*ks + 8g .. +7
    bf16x8 qf[KS];
    {
        const uint16_t* qrow = p.q + pos_q * HD + (long)h * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * g);
    }

    // windows: T per wave (common to its queries), Y and X per query
    const int tw0 = na_start(tqc, p.kt, p.T);
    const int ys_q = na_start(yqc, p.ky, Y);
    const int xs_q = na_start(xqc, p.kx, X);
    const int xa = na_start(strip * QB, p.kx, X);  // first key position of a block
    // rows y' the wave needs (the union of its rows' windows), the rows every one of
    // its queries sees (the intersection), and the rows the workgroup walks
    const int wlast = min(wy0 + QA - 1, Y - 1);
    const int wv0 = na_start(min(wy0, Y - 1), p.ky, Y);
    const int wv1 = na_start(wlast, p.ky, Y) + p.ky;
    const int wc0 = na_start(wlast, p.ky, Y);
    const int wc1 = wv0 + p.ky;
    // the workgroup's union of windows: frames t' [tu0, tu1), rows y' [yu0, yu1)
    const int yfirst = yblk * ay * QA, ylast = yfirst + ay * QA - 1;
    const int yu0 = na_start(min(yfirst, Y - 1), p.ky, Y);
    const int yu1 = na_start(min(ylast, Y - 1), p.ky, Y) + p.ky;
    const int tu0 = na_start(min(p.wt * tb, p.T - 1), p.kt, p.T);
    const int tu1 = na_start(min(p.wt * tb + p.wt - 1, p.T - 1), p.kt, p.T) + p.kt;
    const int nbr = (yu1 - yu0 + RPB - 1) / RPB;  // blocks per t'
    const int nblocks = (tu1 - tu0) * nbr;

    // Loader: thread tid copies physical chunk tid of a block: key j = tid / CPR (row
    // j / KW of the block, position xa + j % KW, clamped to the axis), position tid % CPR
    // holding logical chunk (tid % CPR) ^ swizzle(j). ld_off1 reads the block's first row
    // in place of its second, for a last block whose second row is past the axis.
    unsigned ld_off, ld_off1;
    const int ld_row = (tid / CPR) / KW;  // the lane's row of the block
    {
        const int j = tid / CPR;
        const int xk = min(xa + j % KW, X - 1);
        const int chunk = (tid % CPR) ^ lds_swizzle<CPR>(j);
        ld_off1 = (unsigned)(2 * ((long)xk * HD + chunk * 8));
        ld_off = ld_off1 + (unsigned)(2 * (long)(j / KW) * X * HD);
    }
    const char* kbase = reinterpret_cast<const char*>(uniform_ptr(p.k));
    const char* vbase = reinterpret_cast<const char*>(uniform_ptr(p.v));
    auto kslot = [&](int j) { return smem + j * 2 * TILEB; };
    auto vslot = [&](int j) { return smem + j * 2 * TILEB + TILEB; };
    // Block i covers rows (tu0 + i / nbr, yu0 + RPB * (i % nbr) ...) and goes to slot
    // i % NSLOT. Two cursors walk the blocks in order (the copies AHEAD blocks in front of
    // the computation), so no step divides by nbr or multiplies out a row address.
    const long rowb = (long)X * HD * 2;  // bytes per row y of one frame
    const long bh0 = ((long)b * p.T * Y * X * HD + (long)h * D) * 2;
    const int yend = yu0 + nbr * RPB;
    const long frame_step = (long)(Y - nbr * RPB) * rowb;  // from a frame's last block
    int cp_y = yu0;                                          // next block to copy
    const char* cp_k = kbase + bh0 + ((long)tu0 * Y + yu0) * rowb;
    const char* cp_v = vbase + bh0 + ((long)tu0 * Y + yu0) * rowb;
    // the wave's LDS addresses in each slot, once
    unsigned lds_k[NSLOT], lds_v[NSLOT];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
        lds_k[j] = __builtin_amdgcn_readfirstlane(lds_offset(kslot(j) + wave * kWave * 16));
        lds_v[j] = __builtin_amdgcn_readfirstlane(lds_offset(vslot(j) + wave * kWave * 16));
    }
    auto issue_next = [&](int slot) {
        unsigned off;
        if constexpr (RPB <= 2)
            off = (RPB == 1 || cp_y + 1 < Y) ? ld_off : ld_off1;
        else  // rows past the axis read its last row (never visible)
            off = ld_off1 + (unsigned)min(ld_row, Y - 1 - cp_y) * (unsigned)rowb;
        load16_to_lds_sbase_at(cp_k, off, lds_k[slot]);
        load16_to_lds_sbase_at(cp_v, off, lds_v[slot]);
        cp_y += RPB;
        cp_k += RPB * rowb;
        cp_v += RPB * rowb;
        if (cp_y == yend) {  // the next frame's first block
            cp_y = yu0;
            cp_k += frame_step;
            cp_v += frame_step;
        }
    };

    // Per-lane LDS byte offsets: K operand reads per k-step, V transpose reads per
    // head-dim block and 8-key half (as in the dense kernels).
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
    float m_ref = -INFINITY;
    float l_part = 0.f;  // this lane's partial row sum (of BF16-rounded probabilities)
    const float c = 1.4426950408889634f;  // log2(e): scale 1
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // Score register r of a lane holds key j = 8 (r / 4) + 4 g + r % 4 of the block: row
    // j / KW, position xa + j % KW. The X window of a query covers the same keys of every
    // block: the score accumulators start at -inf for the keys outside it (registers r
    // and r + 8 share a position when KW = 16), so the mask costs no instruction per block.
    f32x16 xm;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int xk = xa + (8 * (r >> 2) + 4 * g + (r & 3)) % KW;
        xm[r] = (xk < xs_q || xk >= xs_q + p.kx) ? -INFINITY : 0.f;
    }

    // One block; ymask when some of its rows lie outside the Y window of some query of
    // the wave (those rows' keys are hidden from that query). ymask is uniform.
    auto compute = [&](const char* kt_lds, const char* vt_lds, int yy, bool ymask) {
        // ---- S^T = K Q^T, onto the X window mask
        f32x16 s = xm;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt_lds + koff[ks]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
        }
        // ---- online softmax: running maximum raised only when a row's block maximum
        // exceeds it by more than 2^kRescaleLog2 in the exp2 domain. Where rows of the
        // block lie outside the query's Y window (ymask), they are left out of the maximum
        // and their exponentials get a reference of +inf (so they are 0), instead of -inf
        // added to each of their scores.
        constexpr int RR = 16 / RPB;  // registers per row of the block
        float mx;
        bool hid[RPB];
        if (ymask) {
            mx = -INFINITY;
#pragma unroll
            for (int hr = 0; hr < RPB; ++hr) {
                hid[hr] = !(yy + hr >= ys_q && yy + hr < ys_q + p.ky);
                float m = s[RR * hr];
#pragma unroll
                for (int r = RR * hr + 1; r < RR * (hr + 1); ++r) m = fmaxf(m, s[r]);
                mx = fmaxf(mx, hid[hr] ? -INFINITY : m);
            }
        } else {
#pragma unroll
            for (int hr = 0; hr < RPB; ++hr) hid[hr] = false;
            mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        }
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
        // a query that has seen no key yet keeps m_ref = -inf; its scores are -inf too
        const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
        float mcr[RPB];
#pragma unroll
        for (int hr = 0; hr < RPB; ++hr) mcr[hr] = hid[hr] ? INFINITY : mc;
        bf16x8 pf[2];
        static_for<NPAIR>([&](auto pc) {
            constexpr int pi = decltype(pc)::value;
            constexpr int tt2 = pi / 4, r = 8 * tt2 + 2 * (pi % 4);
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mcr[r / RR]));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], c, -mcr[(r + 1) / RR]));
            const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
            l_part = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_part, false);
            pf[tt2][r & 7] = pk[0];
            pf[tt2][(r & 7) + 1] = pk[1];
        });
        // ---- O^T += V^T P^T
#pragma unroll
        for (int j = 0; j < 2 * DB; ++j) {
            const int tt2 = j / DB, db = j % DB;
            const int rowbase = 16 * tt2 * ROWB;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vt_lds + voff[db][0] + rowbase));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vt_lds + voff[db][1] + rowbase));
            const i16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a16),
                                                            pf[tt2], o[db], 0, 0, 0);
        }
    };

    // ---- pipeline: block i is copied AHEAD blocks ahead into slot i % NSLOT; the
    // barrier before block i waits for its copies and lets the later ones stay in flight
    const int npre = min(AHEAD, nblocks);
    for (int i = 0; i < npre; ++i) issue_next(i % NSLOT);
    // Q is resident before the loop (with the first blocks): a wait the compiler sees, so
    // it puts none for the Q registers inside the loop, where the hardware count would
    // also take in the block copies just issued and expose their latency on every step.
    __builtin_amdgcn_s_waitcnt((0) | (0 << 14) | (7 << 4) | (15 << 8));  // vmcnt(0)
    // Which of the steps c0 .. c0 + 63 the wave computes (its windows reach the block's
    // frame and rows) and which need the Y mask, one lane per step (bit i - c0).
    unsigned long long st_act = 0, st_ym = 0;
    int st_c0 = 0;
    auto classify_steps = [&](int c0) {
        const int i = c0 + lane;
        bool act = false, ym = false;
        if (active && i < nblocks) {
            const int ti = tu0 + i / nbr, yi = yu0 + RPB * (i % nbr);
            act = yi < wv1 && yi + RPB > wv0 && ti >= tw0 && ti < tw0 + p.kt;
            ym = yi < wc0 || yi + RPB > wc1;
        }
        st_act = __builtin_amdgcn_ballot_w64(act);
        st_ym = __builtin_amdgcn_ballot_w64(ym);
        st_c0 = c0;
    };
    // The loop is unrolled over the ring's slots, so each block's slot is a constant and
    // the LDS reads take it in their immediate offsets.
    int yy = yu0;  // first row of the block computed
    for (int i0 = 0; i0 < nblocks; i0 += NSLOT) {
        if ((i0 & 63) == 0) classify_steps(i0);  // NSLOT divides 64
        static_for<NSLOT>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            const int i = i0 + J;
            if (i < nblocks) {
                barrier_tiles_left<AHEAD - 1>(nblocks - 1 - i);
                if (i + AHEAD < nblocks) issue_next((J + AHEAD) % NSLOT);  // block i-1's slot
                const unsigned long long bit = 1ull << (i - st_c0);
                if (st_act & bit) compute(kslot(J), vslot(J), yy, (st_ym & bit) != 0);
                yy += RPB;
                if (yy == yend) yy = yu0;
            }
        });
    }

    // ---- epilogue
    if (!active) return;
    const float l_tot = wave_swap_sum(l_part);
    // Through LDS, whole 128-byte rows per store: after the last block's barrier only
    // that block's slot is read, so two of the other slots (8 KiB each) hold the four
    // waves' rows. Row r of the wave is query (wy0 + r / QB, strip * QB + r % QB).
    char* const rows = smem + ((nblocks + wave / 2) % NSLOT) * 2 * TILEB + (wave % 2) * (32 * ROWB);
    const long frame = ((long)b * p.T + t) * Y;
    store_wave_rows_via_lds_to<D>(o, 1.0f / l_tot, rows, [&](int r) -> uint16_t* {
        const int yr = wy0 + r / QB, xr = strip * QB + r % QB;
        if (yr >= Y || xr >= X) return nullptr;
        return p.out + ((frame + yr) * X + xr) * HD + (long)h * D;
    });
}

}  // namespace

// Picks the wave tile and key block whose blocks cover a query's window with the fewest
// blocks per t' (QA + ky - 1 rows in blocks of 32 / KW rows), among those whose blocks hold
// the X windows; ties go to the option listed first. Blocks of four rows of 8 positions
// suit narrow windows (kx <= 5: 3x5x5 walks 18 blocks per workgroup instead of 24).
void na3d_configure(NaParams& p) {
    struct Opt { int qb, qa, kw, max_kx; };
    const Opt opts[] = {{16, NaTile<16, 32>::QA, 32, NaTile<16, 32>::max_kx},
                        {8, NaTile<8, 16>::QA, 16, NaTile<8, 16>::max_kx},
                        {4, NaTile<4, 16>::QA, 16, NaTile<4, 16>::max_kx},
                        {4, NaTile<4, 8>::QA, 8, NaTile<4, 8>::max_kx}};
    long best = -1;
    p.qb = 0;
    p.kw = 0;
    p.strips = p.yblocks = 0;  // no tile holds the window: nothing to launch
    p.wt = 1;
    int qa = 0, rpb = 0;
    for (const Opt& o : opts) {
        if (p.kx > o.max_kx) continue;
        // four-row blocks: a lane's byte offset to its row (at most three rows) in 32 bits
        if (o.kw == 8 && 8LL * p.X * p.H * 64 >= (1LL << 32)) continue;
        const int orpb = 32 / o.kw;
        const long cost = (long)((o.qa + p.ky - 1 + orpb - 1) / orpb) * 32;
        if (best < 0 || cost < best) {
            best = cost;
            p.qb = o.qb;
            p.kw = o.kw;
            qa = o.qa;
            rpb = 32 / o.kw;
        }
    }
    if (p.qb) {
        // Arrange the workgroup's four waves as wt frames by 4 / wt row tiles where they
        // share the most of their windows: the workgroup walks the union of its waves' T
        // windows (kt + wt - 1 frames) over the union of their Y windows (4 / wt tiles of
        // qa rows, widened by ky - 1), and a wave computes only the blocks in its own
        // windows, so fewer block steps waste fewer barriers. Ties go to more frames.
        auto blocks_of = [&](int rows) { return (std::min(p.Y, rows + p.ky - 1) + rpb - 1) / rpb; };
        long best_steps = -1;
        for (int wt = 1; wt <= kNaWaves; wt *= 2) {
            const long steps = (long)std::min(p.T, p.kt + wt - 1) * blocks_of(kNaWaves / wt * qa);
            if (best_steps < 0 || steps <= best_steps) {
                best_steps = steps;
                p.wt = wt;
            }
        }
        p.strips = (p.X + p.qb - 1) / p.qb;
        const int rows = kNaWaves / p.wt * qa;
        p.yblocks = (p.Y + rows - 1) / rows;
    }
    // Heads shared by n XCDs are cut along the slowest axis of the order: T (t slowest),
    // else the blocks of rows y, or the strips when there is one block of rows. Each part
    // fetches the K/V rows of its range plus the window's halo; take the cheaper cut.
    p.t_inner = 0;
    const long heads = (long)p.B * p.H;
    if (heads < 8 && p.qb) {
        const int n = (int)((8 + heads - 1) / heads);
        auto dup = [n](int len, int win) {  // K/V rows read per row of the axis
            const double part = (double)len / n;
            return n * std::min((double)len, part + win - 1) / len;
        };
        const int nt = (p.T + p.wt - 1) / p.wt;  // units along T
        const double cut_t = nt >= n ? dup(p.T, p.kt) : 1e30;
        const double cut_yx = p.yblocks >= n ? dup(p.Y, p.ky)
                              : (p.yblocks == 1 && p.strips >= n ? dup(p.X, p.kx) : 1e30);
        p.t_inner = cut_yx < cut_t ? 1 : 0;
    }
}

long long na3d_workgroups(const NaParams& p) {
    const long long nt = (p.T + p.wt - 1) / p.wt;
    return (long long)p.B * nt * p.yblocks * p.strips * p.H;
}

hipError_t launch_na3d(const NaParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)na3d_workgroups(p)), block(kNaWaves * kWave);
    switch (p.qb * 100 + p.kw) {
        case 1632: hipLaunchKernelGGL((attn_na3d_kernel<16, 32>), grid, block, 0, stream, p); break;
        case 816: hipLaunchKernelGGL((attn_na3d_kernel<8, 16>), grid, block, 0, stream, p); break;
        case 416: hipLaunchKernelGGL((attn_na3d_kernel<4, 16>), grid, block, 0, stream, p); break;
        case 408: hipLaunchKernelGGL((attn_na3d_kernel<4, 8>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
