// C ABI of the dense attention library: argument validation, launch planning,
// split-KV work-space ownership and kernel dispatch. Declared in include/attn_dense.h.
//
// Every check runs before the first HIP call, so invalid arguments are reported
// without touching the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <vector>

#include "attn_dense.h"
#include "attn_launch.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr long long kIndexLimit = (1LL << 31) - 1;

// Split-KV (and block-causal id summary) work space of one device. The library's own
// buffer only grows; a superseded buffer is never freed, because launches already
// enqueued on any stream and HIP graphs captured earlier may still use it (it is
// released with the process). A caller-supplied buffer (attn_set_workspace) takes
// precedence and is never grown.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    std::vector<void*> retired;
    void* user = nullptr;
    size_t user_bytes = 0;
};

std::mutex g_ws_mutex;
Workspace g_ws[kMaxDevices];
constexpr size_t kWsGranule = 2u << 20;  // growth is rounded up to 2 MiB

struct Plan {
    int splits;
    int waves;
    int m_blocks;
    int keys_per_split;
    long long workgroups;
    long long workspace_bytes;
};

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlaps(const void* a, long long abytes, const void* b, long long bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Sizes and launch shape. Returns ATTN_OK or an error code.
int make_plan(int B, int Nq, int Nk, int H, int D, int num_splits, int waves, Plan* out) {
    if (B < 1 || Nq < 1 || Nk < 1 || H < 1) return ATTN_ERR_SHAPE;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    if (num_splits < 0 || (waves != 0 && waves != 2 && waves != 4 && waves != 8))
        return ATTN_ERR_UNSUPPORTED;
    // Offsets inside one batch of a tensor are formed in 32 bits before widening.
    if ((long long)Nq * H * D > kIndexLimit || (long long)Nk * H * D > kIndexLimit)
        return ATTN_ERR_OVERFLOW;
    if ((long long)B * H > kIndexLimit || (long long)B * Nq > kIndexLimit ||
        (long long)B * Nk > kIndexLimit)
        return ATTN_ERR_OVERFLOW;

    const int tile = attn::kKeyTile;
    const int key_tiles = (Nk + tile - 1) / tile;
    int w = waves;
    if (w == 0) {
        // The 8-wave ping-pong kernel (256 query rows per workgroup, one workgroup per
        // CU) when it alone fills the 256 CUs: at D = 128, and at D = 64 too (2-5% faster
        // than two 4-wave workgroups per CU on B=1..2, N=2048..16384, H=16..32; equal on
        // B=4 N=1024). Otherwise 4 waves; 2 waves for query ranges of at most 64 rows, and
        // for grids of fewer than 256 4-wave workgroups over fewer than 32 key tiles
        // (twice as many workgroups: B=1 N=256 H=32 D=64 measured 6.8 us against 7.4;
        // Nq=512 Nk=512 H=32 D=128 14.6 against 22.4). Over longer keys 4 waves with
        // their splits win: Nq=256 Nk=4096 H=32 D=128 30.5 us against 39.1, Nq=1024
        // Nk=4096 H=16 48.1 against 64.0.
        const long long pp_blocks = (long long)((Nq + 255) / 256) * B * H;
        const long long blocks4 = (long long)((Nq + 127) / 128) * B * H;
        if (Nq >= 256 && pp_blocks >= 256)
            w = 8;
        else
            w = (Nq <= 64 || (blocks4 < 256 && key_tiles < 32)) ? 2 : 4;
    }
    const int bm = 32 * w;
    const long long m_blocks = (Nq + bm - 1) / bm;
    const long long base = m_blocks * B * H;

    int s = num_splits;
    if (s == 0) {
        // Split the keys only when the grid underfills the GPU, keeping at least four key
        // tiles per split: first up to one workgroup per CU (256 CUs); then, for the 2-
        // and 4-wave kernels, which hold two or three workgroups per CU, up to two per CU
        // while every split keeps 16 (2 waves) or 32 (4 waves) tiles, where the shorter
        // key loops outweigh the merge of the partial results. Measured on MI355X: B=1
        // N=1024 H=32 D=128 (4 waves) 21.8 us unsplit against 35.1 us in two splits;
        // Nq=64 Nk=4096 H=32 D=128 (2 waves) best with 8 splits (23.0 us; 27.4 with 16);
        // Nq=256 Nk=4096 H=32 D=128 best with 4 (39.2 us; 50.3 with 2).
        s = 1;
        while (base * s * 2 <= 256 && key_tiles / (s * 2) >= 4) s *= 2;
        if (w != 8) {
            const int keep = (w == 4) ? 32 : 16;
            while (base * s * 2 <= 512 && key_tiles / (s * 2) >= keep) s *= 2;
        }
    }
    if (s > key_tiles) s = key_tiles;
    if (s < 1) s = 1;
    const int tiles_per_split = (key_tiles + s - 1) / s;
    s = (key_tiles + tiles_per_split - 1) / tiles_per_split;  // no empty split

    const long long wg = base * s;
    if (wg > kIndexLimit) return ATTN_ERR_OVERFLOW;
    out->splits = s;
    out->waves = w;
    out->m_blocks = (int)m_blocks;
    out->keys_per_split = tiles_per_split * tile;
    out->workgroups = wg;
    const long long rows = (long long)B * Nq * H;
    out->workspace_bytes = (s > 1) ? (long long)s * rows * (D + 1) * 4 + 256 : 0;
    return ATTN_OK;
}

int current_device(int* dev) {
    if (hipGetDevice(dev) != hipSuccess) {
        (void)hipGetLastError();
        return ATTN_ERR_HIP;
    }
    if (*dev < 0 || *dev >= kMaxDevices) return ATTN_ERR_WORKSPACE;
    return ATTN_OK;
}

// Returns in *ptr_out a work space of at least `bytes` on the current device: the
// caller's buffer when one is set (ATTN_ERR_WORKSPACE if it is too small), else the
// library's, grown if needed. The pointer stays valid until the process ends (or, for
// a caller's buffer, as long as the caller keeps it).
int reserve(long long bytes, void** ptr_out) {
    if (bytes <= 0) {
        if (ptr_out) *ptr_out = nullptr;
        return ATTN_OK;
    }
    int dev = 0;
    const int drc = current_device(&dev);
    if (drc != ATTN_OK) return drc;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[dev];
    if (ws.user) {
        if (ws.user_bytes < (size_t)bytes) return ATTN_ERR_WORKSPACE;
        if (ptr_out) *ptr_out = ws.user;
        return ATTN_OK;
    }
    if (ws.bytes < (size_t)bytes) {
        // Fault injection for tests: behave as if the allocation failed.
        if (getenv("ATTN_TEST_FAIL_ALLOC")) return ATTN_ERR_WORKSPACE;
        size_t want = (size_t)bytes > 2 * ws.bytes ? (size_t)bytes : 2 * ws.bytes;
        want = (want + kWsGranule - 1) / kWsGranule * kWsGranule;
        void* p = nullptr;
        if (hipMalloc(&p, want) != hipSuccess || !p) {
            (void)hipGetLastError();
            p = nullptr;
            want = (size_t)bytes;  // the doubling may be what did not fit
            if (hipMalloc(&p, want) != hipSuccess || !p) {
                (void)hipGetLastError();
                return ATTN_ERR_WORKSPACE;
            }
        }
        if (ws.ptr) ws.retired.push_back(ws.ptr);
        ws.ptr = p;
        ws.bytes = want;
    }
    if (ptr_out) *ptr_out = ws.ptr;
    return ATTN_OK;
}

}  // namespace

namespace attn {

// The dense / prefix / cross forward behind every entry point. `fixed` (may be null)
// is a work space handed in for this call only; without it the device's work space
// (reserve) is used when the plan splits the keys.
__attribute__((visibility("hidden"))) int run_fwd(const void* q, const void* k0, const void* v0,
                                                  int n0, const void* k1, const void* v1, int n1,
                                                  void* out, int B, int Nq, int H, int D,
                                                  int num_splits, int waves, void* stream,
                                                  const FixedWorkspace* fixed) {
    if (!q || !out) return ATTN_ERR_NULL;
    if (n0 < 0 || n1 < 0) return ATTN_ERR_SHAPE;
    if (n0 > 0 && (!k0 || !v0)) return ATTN_ERR_NULL;
    if (n1 > 0 && (!k1 || !v1)) return ATTN_ERR_NULL;
    if ((long long)n0 + n1 > kIndexLimit) return ATTN_ERR_OVERFLOW;
    const int nk = n0 + n1;
    Plan plan;
    const int rc = make_plan(B, Nq, nk, H, D, num_splits, waves, &plan);
    if (rc != ATTN_OK) return rc;
    if (misaligned(q) || misaligned(out) || (n0 && (misaligned(k0) || misaligned(v0))) ||
        (n1 && (misaligned(k1) || misaligned(v1))))
        return ATTN_ERR_ALIGN;
    const long long qbytes = 2LL * B * Nq * H * D;
    const long long s0 = 2LL * B * n0 * H * D;
    const long long s1 = 2LL * B * n1 * H * D;
    if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k0, s0) ||
        overlaps(out, qbytes, v0, s0) || overlaps(out, qbytes, k1, s1) ||
        overlaps(out, qbytes, v1, s1))
        return ATTN_ERR_ALIAS;

    // ---- device work from here on
    void* ws = nullptr;
    if (plan.splits > 1) {
        if (fixed) {
            if (!fixed->ptr || fixed->bytes < plan.workspace_bytes) return ATTN_ERR_WORKSPACE;
            ws = fixed->ptr;
        } else {
            const int wrc = reserve(plan.workspace_bytes, &ws);
            if (wrc != ATTN_OK) return wrc;
        }
        // a caller's work space must not overlap the tensors of the call
        const long long wb = plan.workspace_bytes;
        if (overlaps(ws, wb, out, qbytes) || overlaps(ws, wb, q, qbytes) ||
            overlaps(ws, wb, k0, s0) || overlaps(ws, wb, v0, s0) || overlaps(ws, wb, k1, s1) ||
            overlaps(ws, wb, v1, s1))
            return ATTN_ERR_ALIAS;
    }
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    attn::FwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k0 = static_cast<const uint16_t*>(n0 ? k0 : k1);
    p.v0 = static_cast<const uint16_t*>(n0 ? v0 : v1);
    p.k1 = static_cast<const uint16_t*>(n0 ? k1 : nullptr);
    p.v1 = static_cast<const uint16_t*>(n0 ? v1 : nullptr);
    p.n0 = n0 ? n0 : n1;
    p.n1 = n0 ? n1 : 0;
    p.out = static_cast<uint16_t*>(out);
    const long long rows = (long long)B * Nq * H;
    p.part_o = nullptr;
    p.part_lse = nullptr;
    if (plan.splits > 1) {
        p.part_lse = static_cast<float*>(ws);
        const long long lse_bytes = ((long long)plan.splits * rows * 4 + 255) & ~255LL;
        p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + lse_bytes);
    }
    p.B = B;
    p.Nq = Nq;
    p.H = H;
    p.keys_per_split = plan.keys_per_split;
    p.splits = plan.splits;
    p.m_blocks = plan.m_blocks;
    p.c = (float)(pow((double)D, -0.5) * 1.4426950408889634);  // D^-0.5 * log2(e)
    p.ids = nullptr;
    p.meta = nullptr;

    if (attn::launch_fwd(D, plan.waves, p, plan.workgroups, st) != hipSuccess)
        return ATTN_ERR_HIP;
    if (plan.splits > 1) {
        attn::CombineParams cp;
        cp.part_o = p.part_o;
        cp.part_lse = p.part_lse;
        cp.out = p.out;
        cp.rows = rows;
        cp.splits = plan.splits;
        if (attn::launch_combine(D, cp, st) != hipSuccess) return ATTN_ERR_HIP;
    }
    return ATTN_OK;
}

}  // namespace attn

namespace {

using attn::run_fwd;

// Block-causal attention without prefix: keys are the queries' own positions.
int run_block_causal(const void* q, const void* k, const void* v, const int* ids, void* out,
                     int B, int N, int H, int D, void* stream) {
    if (!q || !k || !v || !ids || !out) return ATTN_ERR_NULL;
    Plan plan;
    const int rc = make_plan(B, N, N, H, D, 1, 8, &plan);  // one key split, ping-pong
    if (rc != ATTN_OK) return rc;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(ids) || misaligned(out))
        return ATTN_ERR_ALIGN;
    const long long bytes = 2LL * B * N * H * D;
    const long long idbytes = 4LL * N;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
        overlaps(out, bytes, v, bytes) || overlaps(out, bytes, ids, idbytes))
        return ATTN_ERR_ALIAS;

    // ---- device work from here on: per-row-block id summaries in the work space
    const long long nblk = (N + attn::kMetaRows - 1) / attn::kMetaRows;
    void* ws = nullptr;
    const int wrc = reserve(nblk * 16, &ws);
    if (wrc != ATTN_OK) return wrc;
    if (overlaps(ws, nblk * 16, out, bytes) || overlaps(ws, nblk * 16, q, bytes) ||
        overlaps(ws, nblk * 16, k, bytes) || overlaps(ws, nblk * 16, v, bytes) ||
        overlaps(ws, nblk * 16, ids, idbytes))
        return ATTN_ERR_ALIAS;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    attn::FwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k0 = static_cast<const uint16_t*>(k);
    p.v0 = static_cast<const uint16_t*>(v);
    p.k1 = nullptr;
    p.v1 = nullptr;
    p.n0 = N;
    p.n1 = 0;
    p.out = static_cast<uint16_t*>(out);
    p.part_o = nullptr;
    p.part_lse = nullptr;
    p.B = B;
    p.Nq = N;
    p.H = H;
    p.keys_per_split = plan.keys_per_split;
    p.splits = 1;
    p.m_blocks = plan.m_blocks;
    p.c = (float)(pow((double)D, -0.5) * 1.4426950408889634);
    p.ids = ids;
    p.meta = static_cast<int*>(ws);
    if (attn::launch_bc_meta(ids, N, static_cast<int*>(ws), st) != hipSuccess)
        return ATTN_ERR_HIP;
    if (attn::launch_fwd_block_causal(D, p, plan.workgroups, st) != hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

// 3-D neighborhood attention (attn_na3d.hip).
// Checks the sizes and window of a 3-D neighborhood call and fills p's sizes and launch
// shape (not its pointers).
int na3d_shape(int B, int T, int Y, int X, int H, int D, int kt, int ky, int kx,
               attn::NaParams& p) {
    if (B < 1 || T < 1 || Y < 1 || X < 1 || H < 1) return ATTN_ERR_SHAPE;
    if (kt < 1 || ky < 1 || kx < 1 || kt % 2 == 0 || ky % 2 == 0 || kx % 2 == 0 || kt > T ||
        ky > Y || kx > X)
        return ATTN_ERR_SHAPE;
    if (D != 64 || kx > 17) return ATTN_ERR_UNSUPPORTED;
    p.B = B;
    p.T = T;
    p.Y = Y;
    p.X = X;
    p.H = H;
    p.kt = kt;
    p.ky = ky;
    p.kx = kx;
    attn::na3d_configure(p);
    const long long elems = (long long)B * T * Y * X * H * D;
    // byte offsets within two consecutive (b, t, y) rows of X positions fit in 32 bits
    if (elems >= (1LL << 40) || 2LL * X * H * D >= (1LL << 31) ||
        attn::na3d_workgroups(p) >= (1LL << 31))
        return ATTN_ERR_OVERFLOW;
    return ATTN_OK;
}

int run_na3d(const void* q, const void* k, const void* v, void* out, int B, int T, int Y, int X,
             int H, int D, int kt, int ky, int kx, void* stream) {
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    attn::NaParams p;
    const int rc = na3d_shape(B, T, Y, X, H, D, kt, ky, kx, p);
    if (rc != ATTN_OK) return rc;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out)) return ATTN_ERR_ALIGN;
    const long long bytes = 2LL * B * T * Y * X * H * D;
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
        overlaps(out, bytes, v, bytes))
        return ATTN_ERR_ALIAS;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.out = static_cast<uint16_t*>(out);
    if (attn::launch_na3d(p, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_block_causal(const void* q, const void* k, const void* v, const int* image_ids,
                      void* out, int B, int N, int H, int D, void* stream) {
    return run_block_causal(q, k, v, image_ids, out, B, N, H, D, stream);
}

int attn_na3d(const void* q, const void* k, const void* v, void* out, int B, int T, int Y, int X,
              int H, int D, int kt, int ky, int kx, void* stream) {
    return run_na3d(q, k, v, out, B, T, Y, X, H, D, kt, ky, kx, stream);
}

int attn_dense(const void* q, const void* k, const void* v, void* out, int B, int N, int H,
               int D, void* stream) {
    if (N < 1) return ATTN_ERR_SHAPE;
    return run_fwd(q, k, v, N, nullptr, nullptr, 0, out, B, N, H, D, 0, 0, stream, nullptr);
}

int attn_prefix(const void* q, const void* kp, const void* vp, const void* kc, const void* vc,
                void* out, int B, int Nq, int Np, int H, int D, void* stream) {
    if (Np < 0 || Nq < 1) return ATTN_ERR_SHAPE;
    if (!kc || !vc) return ATTN_ERR_NULL;
    return run_fwd(q, kp, vp, Np, kc, vc, Nq, out, B, Nq, H, D, 0, 0, stream, nullptr);
}

int attn_cross(const void* q, const void* k, const void* v, void* out, int B, int Nq, int Nk,
               int H, int D, void* stream) {
    if (Nk < 1) return ATTN_ERR_SHAPE;
    return run_fwd(q, k, v, Nk, nullptr, nullptr, 0, out, B, Nq, H, D, 0, 0, stream, nullptr);
}

int attn_fwd_ex(const void* q, const void* k0, const void* v0, int n0, const void* k1,
                const void* v1, int n1, void* out, int B, int Nq, int H, int D, int num_splits,
                int waves, void* stream) {
    if ((long long)n0 + n1 < 1) return ATTN_ERR_SHAPE;
    return run_fwd(q, k0, v0, n0, k1, v1, n1, out, B, Nq, H, D, num_splits, waves, stream,
                   nullptr);
}

int attn_plan(int B, int Nq, int Nk, int H, int D, int num_splits, int waves, int* splits,
              int* waves_out, long long* workgroups, long long* workspace_bytes) {
    Plan plan;
    const int rc = make_plan(B, Nq, Nk, H, D, num_splits, waves, &plan);
    if (rc != ATTN_OK) return rc;
    if (splits) *splits = plan.splits;
    if (waves_out) *waves_out = plan.waves;
    if (workgroups) *workgroups = plan.workgroups;
    if (workspace_bytes) *workspace_bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int attn_na3d_plan(int B, int T, int Y, int X, int H, int D, int kt, int ky, int kx,
                   int* query_cols, long long* workgroups) {
    attn::NaParams p;
    const int rc = na3d_shape(B, T, Y, X, H, D, kt, ky, kx, p);
    if (rc != ATTN_OK) return rc;
    if (query_cols) *query_cols = p.qb;
    if (workgroups) *workgroups = attn::na3d_workgroups(p);
    return ATTN_OK;
}

int attn_reserve_workspace(long long bytes) { return reserve(bytes, nullptr); }

int attn_set_workspace(void* ptr, long long bytes) {
    if (ptr && bytes < 0) return ATTN_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return ATTN_ERR_ALIGN;
    int dev = 0;
    const int drc = current_device(&dev);
    if (drc != ATTN_OK) return drc;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    g_ws[dev].user = ptr;
    g_ws[dev].user_bytes = ptr ? (size_t)bytes : 0;
    return ATTN_OK;
}

const char* attn_strerror(int code) {
    switch (code) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "a batch, sequence or head count is out of range";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or launch option";
        case ATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case ATTN_ERR_ALIAS: return "the output or the caller's work space overlaps an input";
        case ATTN_ERR_OVERFLOW: return "a size exceeds the kernels' index range";
        case ATTN_ERR_WORKSPACE:
            return "the work space could not be allocated or the caller's is too small";
        case ATTN_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        default: return "unknown error code";
    }
}

int attn_abi_version(void) { return 1; }

}  // extern "C"
