// Device-side building blocks shared by the attention forward kernels (gfx950).
// Internal to the library; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kRescaleLog2 = 8.0f;
// Largest sum of one lane's probabilities of a tile that is accepted without computing
// the tile's row maximum (lazy softmax): every probability is then at most 2^64, and a
// row's output accumulates at most (keys) * 2^64 * |V|, far inside FP32 range; BF16
// probabilities keep their relative precision at any magnitude.
constexpr float kLazySumLimit = 18446744073709551616.0f;  // 2^64
// Largest |running reference| (scaled logits, log2 units) of rows that go lazy.
constexpr float kLazyRefLog2 = 40.0f;
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

// Workgroups one XCD holds at once for the 8-wave kernels: one per CU, 32 CUs per XCD.
constexpr int kXcdSlots = 32;

// Workgroup -> (query block, batch*head, split). Workgroups are dispatched to the
// 8 XCDs round-robin by linear id; this remap gives each XCD a contiguous range of
// (query block, head) work so the query blocks sharing one head's K/V run on the same
// XCD and hit its L2.
//
// heavy_last_blocks (causal-like masks, where later query blocks see more keys): the
// XCD's share of heads is cut into groups of heads whose blocks together fill the XCD's
// workgroup slots (slots_per_xcd); within a group, query blocks are handed out from the
// last to the first, cycling over the group's heads, so the longest workgroups start
// first. The first group's blocks all start together and read each K/V tile of a head
// at nearly the same time; a later group's light blocks start while its heavy blocks
// still run, so they find the first K/V tiles in the XCD's L2 more often than when the
// heavy blocks of every head in the share go first.
__device__ __forceinline__ void decode_workgroup(int m_blocks, int bh_count, int& mb, int& bh,
                                                 int& split, bool heavy_last_blocks = false,
                                                 int slots_per_xcd = kXcdSlots) {
    const int L = blockIdx.x;
    const int T = gridDim.x;
    const int per = T >> 3;
    int L2 = (L < (per << 3)) ? (L & 7) * per + (L >> 3) : L;
    if (heavy_last_blocks && L < (per << 3) && per % m_blocks == 0) {
        const int hx = per / m_blocks;  // heads in this XCD's share
        const int g = max(1, min(hx, slots_per_xcd / m_blocks));  // heads per group
        const int r = L2 % per;
        const int h0 = (r / (g * m_blocks)) * g;  // first head of r's group
        const int gn = min(g, hx - h0);           // heads in r's group
        const int q = r - h0 * m_blocks;          // position inside the group
        L2 = (L2 - r) + (h0 + q % gn) * m_blocks + (m_blocks - 1 - q / gn);
    } else if (heavy_last_blocks) {
        L2 = (L2 / m_blocks) * m_blocks + (m_blocks - 1 - L2 % m_blocks);
    }
    mb = L2 % m_blocks;
    const int rest = L2 / m_blocks;
    bh = rest % bh_count;
    split = rest / bh_count;
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1 (compile-time indices).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS byte address of a generic pointer into LDS: its low 32 bits (the flat aperture
// of the LDS is 4 GiB aligned). The same as the address-space cast, without the cast's
// test for a null pointer, which the compiler cannot drop for these pointers.
__device__ __forceinline__ unsigned lds_offset(const void* p) {
    return (unsigned)(uintptr_t)p;
}

// 16-byte global -> LDS copy (global_load_lds_dwordx4). Lane i of the wave writes
// LDS bytes [dst + 16*i, dst + 16*i + 16); dst must be the same for the whole wave.
// NT marks the load non-temporal: for bytes no other workgroup reads, so the caches do
// not keep them at the expense of data that is shared.
template <bool NT = false>
__device__ __forceinline__ void load16_to_lds(const uint16_t* src, char* dst) {
    // Issued as inline assembly on purpose: the compiler cannot tell which LDS bytes an
    // LDS-DMA copy writes, so for the builtin it waits for every copy in flight before
    // each later LDS read it cannot disambiguate (the transposed V reads), which would
    // expose the memory latency of the prefetched tiles on every tile. The kernels order
    // copies and reads themselves (barrier_vmcnt); hidden copies can only make the
    // compiler's own vmcnt waits for other loads stricter, never looser.
    // M0 holds the wave's LDS base; lane i writes bytes [16 i, 16 i + 16) above it.
    const unsigned lds = __builtin_amdgcn_readfirstlane(lds_offset(dst));
    // M0 is clobbered on purpose: nothing else in these kernels keeps a value in it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (NT)
        __asm__ volatile(
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off nt"
            :
            : "v"(src), "s"(lds)
            : "memory", "m0");
    else
        __asm__ volatile(
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, off"
            :
            : "v"(src), "s"(lds)
            : "memory", "m0");
#pragma clang diagnostic pop
}

// A 64-bit value that is the same for the whole wave, moved to scalar registers. The
// halves go through readfirstlane, which returns int: each is converted to unsigned
// before widening, so the low half is zero-extended, never sign-extended.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t a) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}

// The same copy with a wave-uniform base address and a per-lane 32-bit byte offset:
// the load adds them itself (scalar-base form), so issuing it takes no vector
// instructions. base must be the same for the whole wave.
// lds: the wave's LDS byte address (uniform), as lds_offset() gives it.
template <bool NT = false>
__device__ __forceinline__ void load16_to_lds_sbase_at(const void* base, unsigned voff,
                                                       unsigned lds) {
    const uint64_t sb = uniform_u64((uint64_t)(uintptr_t)base);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    if constexpr (NT)
        __asm__ volatile(
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1 nt"
            :
            : "v"(voff), "s"(sb), "s"(lds)
            : "memory", "m0");
    else
        __asm__ volatile(
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %0, %1"
            :
            : "v"(voff), "s"(sb), "s"(lds)
            : "memory", "m0");
#pragma clang diagnostic pop
}

template <bool NT = false>
__device__ __forceinline__ void load16_to_lds_sbase(const void* base, unsigned voff, char* dst) {
    load16_to_lds_sbase_at<NT>(base, voff, __builtin_amdgcn_readfirstlane(lds_offset(dst)));
}

// A pointer that is the same for the whole wave, kept in scalar registers.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
    return reinterpret_cast<T*>((uintptr_t)uniform_u64((uint64_t)(uintptr_t)ptr));
}

// XOR swizzle of the 16-byte chunks of LDS row r (CPR chunks per row, period 16
// rows). Chunk c of row r is stored at chunk position c ^ lds_swizzle(r). Chosen so
// that (a) the 16 lanes of a K operand read (16 consecutive rows, one logical chunk)
// hit 64 different banks, and (b) the 32 lanes of a V transpose read (4 consecutive
// rows, 4 consecutive chunks) hit 64 different banks: the pattern keeps aligned
// groups of 4 chunks together and moves whole groups between those rows.
//   D = 128 (16 chunks, one row = all 64 banks): ((r & 3) << 2) | ((r >> 2) & 3)
//   D = 64 (8 chunks, rows of one parity share a bank half): x = (r >> 1) & 7,
//   ((x & 1) << 2) | ((x >> 1) & 3)
template <int CPR>
__device__ __forceinline__ int lds_swizzle(int r) {
    if constexpr (CPR == 16) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        const int x = (r >> 1) & 7;
        return ((x & 1) << 2) | ((x >> 1) & 3);
    }
}

// Workgroup barrier that first waits until at most N of this wave's global->LDS
// copies are outstanding and all of its LDS reads have returned. Unlike
// __syncthreads(), later copies may stay in flight across the barrier. The empty asm
// statements keep the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void barrier_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// One wave's 32 rows of D BF16 values through LDS, as whole rows. Row r of the wave
// is at base + r * stride (elements); rows at or past nvalid are clamped to the last
// valid one on the way in and skipped on the way out. In LDS the rows are 2*D bytes
// with 16-byte chunks swizzled like the K/V tiles, so a lane's 16-byte chunk of a row
// is read and written without bank conflicts. Lane i of round k moves chunk 64 k + i.
//
// Copy in: global -> LDS (global_load_lds_dwordx4, D/16 copies per lane); the caller
// waits for them (vmcnt) before reading the rows.
template <int D, bool NT = false>
__device__ __forceinline__ void copy_wave_rows_to_lds(const uint16_t* base, long stride,
                                                      int nvalid, char* rows) {
    constexpr int CPR = D / 8;
    const int lane = threadIdx.x % kWave;
    static_for<CPR / 2>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int id = i * kWave + lane;
        const int r = id / CPR;
        const int lc = (id % CPR) ^ lds_swizzle<CPR>(r);
        load16_to_lds<NT>(base + (long)min(r, nvalid - 1) * stride + lc * 8, rows + i * kWave * 16);
    });
}

// The Q^T fragments of the rows: lane (n, g) holds row n, elements 16 ks + 8 g .. +7.
template <int D>
__device__ __forceinline__ void read_wave_rows_qf(const char* rows, bf16x8 (&qf)[D / 16]) {
    constexpr int CPR = D / 8;
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31, g = lane >> 5;
    const int tsw = lds_swizzle<CPR>(n) ^ g;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = *reinterpret_cast<const bf16x8*>(rows + n * 2 * D + 16 * ((2 * ks) ^ tsw));
}

// Store out: the wave's O^T accumulators (o[db][4 j + e] holds row n, element
// 32 db + 8 j + 4 g + e, for lane (n, g)) times inv, rounded to BF16, go to its LDS rows
// and from there to global memory, each store instruction covering whole rows. Row r
// goes to row_ptr(r), or nowhere when that is null.
template <int D, typename RowPtr>
__device__ __forceinline__ void store_wave_rows_via_lds_to(const f32x16 (&o)[D / 32],
                                                           float inv, char* rows,
                                                           RowPtr row_ptr) {
    constexpr int CPR = D / 8;
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31, g = lane >> 5;
    const int sw = lds_swizzle<CPR>(n);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * j + e] * inv);
            *reinterpret_cast<bf16x4*>(rows + n * 2 * D + 16 * ((4 * db + j) ^ sw) + 8 * g) = v;
        }
    // the rows are read back by other lanes of the wave: LDS writes complete first
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    static_for<CPR / 2>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int id = i * kWave + lane;
        const int r = id / CPR;
        const int pc = id % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(rows + r * 2 * D + 16 * pc);
        uint16_t* dst = row_ptr(r);
        if (dst) *reinterpret_cast<u32x4*>(dst + (pc ^ lds_swizzle<CPR>(r)) * 8) = v;
    });
}

// The same for rows `stride` elements apart from base, of which the first nvalid exist;
// the stores are non-temporal (the output is not read again by the kernel).
template <int D>
__device__ __forceinline__ void store_wave_rows_via_lds(const f32x16 (&o)[D / 32], float inv,
                                                        char* rows, uint16_t* base,
                                                        long stride, int nvalid) {
    constexpr int CPR = D / 8;
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31, g = lane >> 5;
    const int sw = lds_swizzle<CPR>(n);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[db][4 * j + e] * inv);
            *reinterpret_cast<bf16x4*>(rows + n * 2 * D + 16 * ((4 * db + j) ^ sw) + 8 * g) = v;
        }
    // the rows are read back by other lanes of the wave: LDS writes complete first
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    static_for<CPR / 2>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int id = i * kWave + lane;
        const int r = id / CPR;
        const int pc = id % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(rows + r * 2 * D + 16 * pc);
        if (r < nvalid)
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base + (long)r * stride + (pc ^ lds_swizzle<CPR>(r)) * 8));
    });
}

// FP32 rows (split-KV partial outputs, D floats per row) through the same 32 × 2·D-byte
// LDS rows, in two passes of D/2 floats: in pass p lane (n, g) writes, for each of its
// head-dim blocks db of that half and each j, the four floats of elements
// 32 db + 8 j + 4 g .. as one 16-byte chunk; then whole half-rows go out.
template <int D>
__device__ __forceinline__ void store_wave_rows_f32_via_lds(const f32x16 (&o)[D / 32],
                                                            float inv, char* rows, float* base,
                                                            long stride, int nvalid) {
    constexpr int CPR = D / 8;  // 16-byte chunks in half a row of D floats
    constexpr int DBH = D / 64;  // head-dim blocks per half
    const int lane = threadIdx.x % kWave;
    const int n = lane & 31, g = lane >> 5;
    const int sw = lds_swizzle<CPR>(n);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int d = 0; d < DBH; ++d)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = o[half * DBH + d][4 * j + e] * inv;
                *reinterpret_cast<f32x4*>(rows + n * 2 * D + 16 * ((8 * d + 2 * j + g) ^ sw)) = v;
            }
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        __asm__ volatile("" ::: "memory");
        static_for<CPR / 2>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int id = i * kWave + lane;
            const int r = id / CPR;
            const int pc = id % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(rows + r * 2 * D + 16 * pc);
            if (r < nvalid)
                *reinterpret_cast<u32x4*>(base + (long)r * stride + half * (D / 2) +
                                          (pc ^ lds_swizzle<CPR>(r)) * 4) = v;
        });
        // the next pass rewrites the rows: these reads complete first
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        __asm__ volatile("" ::: "memory");
    }
}

}  // namespace dev
}  // namespace attn
