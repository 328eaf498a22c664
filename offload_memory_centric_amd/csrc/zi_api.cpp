// zi_api.cpp -- the C ABI: contexts, the tile ring (stager), passes, timing.
//
// The stager follows the pages' description of memory-centric tiling (ZeRO-
// Infinity transformer-math page, section "Memory-centric tiling: operators
// bigger than the device"; pwwt.cn article, section "关键技术一：Memory-centric
// tiling", worked example: load W_i, compute Y_i, release W_i and its
// gradient, load W_{i+1}, ...) with the copy of later tiles overlapping the
// products of the current one (pwwt.cn article, section "关键技术三：Overlap-
// Centric Design": CPU-to-GPU copies run ahead of compute; in the backward
// the gradient write-back to host overlaps the next tiles' products).
//
// Ring: d weight slots over the caller's workspace.  Global tile number g
// (counted across calls on one context) uses slot g mod d.  Per slot:
//   w_ready[s]  recorded on the copy-in stream after the tile landed,
//   w_free[s]   recorded after the last reader of the slot (compute stream,
//               or the write-back stream when dW_i is formed in the slot).
// The copy of tile g waits on w_free of its slot, whose latest record is
// tile g - d's release; the products of tile g wait on w_ready.  Because the
// numbering continues across calls, the first copies of a call overlap the
// last products of the previous call.  Gradient slots (dw_slots of them) work
// the same way with dw_ready (compute) and dw_free (write-back stream).
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <unistd.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/zi.h"
#include "zi_host.h"
#include "zi_internal.h"

namespace zi {

static thread_local char g_err[512];

zi_status fail(zi_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

void clear_error() { g_err[0] = 0; }

enum Kind { K_FWD = 0, K_FWD_GELU, K_DX, K_DW, K_FWD_RECOMPUTE, K_GELU_BWD, K_COUNT };
static const char *kKindNames[K_COUNT] = {"gemm_fwd", "gemm_fwd_gelu", "gemm_dx",
                                          "gemm_dw",  "gemm_fwd_recompute", "gelu_bwd"};

struct KernelRec {
    int kind;
    double flops;
    hipEvent_t a, b;
    int op;                    // kernel identity: GemmOp (or -1: GeLU backward) and launch shape
    int64_t rows, cols, red;
};
struct CopyRec {
    int d2h;
    double bytes;
    hipEvent_t a, b;
};

}  // namespace zi

using namespace zi;

struct zi_ctx {
    int device = 0;
    hipStream_t comp = nullptr, h2d = nullptr, d2h = nullptr;
    // optional second product stream: a forward pass alternates its tiles'
    // products between comp and comp2 (forked from and joined back into comp)
    hipStream_t comp2 = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    int cus = 256;  // compute units of the device
    char *ws = nullptr;
    uint64_t ws_bytes = 0;
    // workspace past the ring for the split GeLU forward, one set per product
    // stream (comp, comp2); null if too small
    float *split_part[2] = {nullptr, nullptr};
    uint32_t *split_cnt[2] = {nullptr, nullptr};
    int d = 1, dw_slots = 0;
    uint64_t slot_bytes = 0, dw_slot_bytes = 0;
    std::vector<hipEvent_t> w_ready, w_free, dw_ready, dw_free;
    std::vector<char> w_free_rec, dw_free_rec;
    int64_t seq = 0, dw_seq = 0;
    zi_status sticky = ZI_OK;
    std::string sticky_msg;
    bool timing = false;
    uint32_t debug = 0;     // ZI_DEBUG_* flags
    uint32_t delay_us = 0;  // host-side delay before every tile copy
    std::vector<hipEvent_t> pool;
    size_t pool_used = 0;
    std::vector<KernelRec> krec;
    std::vector<CopyRec> crec;
    std::vector<std::pair<const zi_plan *, zi_adam *>> adams;  // optimizers attached per plan
    std::vector<std::pair<const zi_plan *, zi_file_source *>> sources;  // file sources per plan

    zi_adam *adam_of(const zi_plan *p) const {
        for (const auto &e : adams)
            if (e.first == p) return e.second;
        return nullptr;
    }
    zi_file_source *source_of(const zi_plan *p) const {
        for (const auto &e : sources)
            if (e.first == p) return e.second;
        return nullptr;
    }

    char *wslot(int s) const { return ws + (uint64_t)s * slot_bytes; }
    char *dwslot(int s) const { return ws + (uint64_t)d * slot_bytes + (uint64_t)s * dw_slot_bytes; }
};

namespace {

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

zi_status hip_fail(zi_ctx *c, hipError_t e, const char *what) {
    // the runtime also keeps the error as the thread's last one; take it, so
    // that the caller's next, unrelated error check does not report it again
    (void)hipGetLastError();
    char buf[400];
    snprintf(buf, sizeof(buf), "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
    if (c && c->sticky == ZI_OK) {
        c->sticky = ZI_ERR_HIP;
        c->sticky_msg = buf;
    }
    return fail(ZI_ERR_HIP, "%s", buf);
}

#define HIPCHK(c, call)                                     \
    do {                                                    \
        hipError_t e_ = (call);                             \
        if (e_ != hipSuccess) return hip_fail((c), e_, #call); \
    } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Host function of the copy-delay debug aid: holds its stream for `arg` us.
void sleep_us(void *arg) { usleep((useconds_t)(uintptr_t)arg); }

bool pinned_range(const void *p, uint64_t bytes) {
    if (!p || !bytes) return false;
    const char *q[2] = {static_cast<const char *>(p), static_cast<const char *>(p) + bytes - 1};
    for (const char *x : q) {
        hipPointerAttribute_t a;
        hipError_t e = hipPointerGetAttributes(&a, x);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        if (a.type != hipMemoryTypeHost) return false;
    }
    return true;
}

zi_status ev_timed(zi_ctx *c, hipEvent_t *out) {
    if (c->pool_used == c->pool.size()) {
        hipEvent_t e;
        HIPCHK(c, hipEventCreate(&e));
        c->pool.push_back(e);
    }
    *out = c->pool[c->pool_used++];
    return ZI_OK;
}

zi_status check_ctx(zi_ctx *c) {
    if (!c) return fail(ZI_ERR_ARG, "context is NULL");
    if (c->sticky != ZI_OK) return fail(c->sticky, "context has a sticky error: %s", c->sticky_msg.c_str());
    int dev = -1;
    HIPCHK(nullptr, hipGetDevice(&dev));
    if (dev != c->device)
        return fail(ZI_ERR_STATE, "current device %d is not the context's device %d", dev, c->device);
    return ZI_OK;
}

zi_status check_pass(zi_ctx *c, const zi_plan *p, bool backward) {
    zi_status st = check_ctx(c);
    if (st != ZI_OK) return st;
    if (!p) return fail(ZI_ERR_ARG, "plan is NULL");
    const zi_problem &pr = p->prob;
    const zi_plan_info &in = p->info;
    if (pr.d != c->d) return fail(ZI_ERR_STATE, "plan depth d=%d differs from the context's %d", pr.d, c->d);
    if (in.tile_bytes > c->slot_bytes)
        return fail(ZI_ERR_STATE, "plan tile of %llu B does not fit the context's %llu B slots",
                    (unsigned long long)in.tile_bytes, (unsigned long long)c->slot_bytes);
    const uint64_t wbytes = (uint64_t)pr.M * (uint64_t)pr.K * 2u;
    if (!c->source_of(p)) {  // with a file source the tiles come from its staging buffers
        if (!pr.W_host) return fail(ZI_ERR_ARG, "plan has no W_host");
        if (!pinned_range(pr.W_host, wbytes))
            return fail(ZI_ERR_NOT_PINNED, "W_host is not page-locked host memory over its %llu bytes",
                        (unsigned long long)wbytes);
    }
    if (backward) {
        if (!pr.dW_host) return fail(ZI_ERR_ARG, "a backward needs a plan with dW_host");
        const uint64_t dwbytes = (uint64_t)pr.M * (uint64_t)pr.K * ((pr.flags & ZI_FLAG_F32_OUT) ? 4u : 2u);
        if (!pinned_range(pr.dW_host, dwbytes))
            return fail(ZI_ERR_NOT_PINNED, "dW_host is not page-locked host memory over its %llu bytes",
                        (unsigned long long)dwbytes);
        const uint64_t room = c->dw_slots > 0 ? c->dw_slot_bytes : c->slot_bytes;
        if (in.dw_tile_bytes > room)
            return fail(ZI_ERR_STATE, "gradient tile of %llu B does not fit the context's %llu B slot",
                        (unsigned long long)in.dw_tile_bytes, (unsigned long long)room);
    }
    return ZI_OK;
}

zi_status check_dev_ptr(const void *p, const char *name) {
    if (!p) return fail(ZI_ERR_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(ZI_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return ZI_OK;
}

// Copy global tile g (tile index `tile` of plan p) into its slot.
zi_status stage(zi_ctx *c, const zi_plan *p, int64_t g, int64_t tile) {
    // the tile's pending optimizer update must have rewritten W_host first
    if (zi_adam *a = c->adam_of(p)) adam_wait_tile(a, tile);
    const int s = (int)(g % c->d);
    if (c->w_free_rec[s]) HIPCHK(c, hipStreamWaitEvent(c->h2d, c->w_free[s], 0));
    if (c->debug & ZI_DEBUG_POISON)  // a reader still using the slot would now see NaNs
        HIPCHK(c, hipMemsetAsync(c->wslot(s), 0xFF, c->slot_bytes, c->h2d));
    if (c->delay_us) HIPCHK(c, hipLaunchHostFunc(c->h2d, sleep_us, reinterpret_cast<void *>((uintptr_t)c->delay_us)));
    const uint64_t bytes = p->info.tile_bytes;
    const char *src = static_cast<const char *>(p->prob.W_host) + (uint64_t)tile * bytes;
    zi_file_source *fs = c->source_of(p);
    int fslot = -1;
    if (fs) {  // the tile comes from the file source's staging buffer, once read
        const void *staged = nullptr;
        const zi_status st = source_acquire(fs, tile, &staged, &fslot);
        if (st != ZI_OK) {  // passes already enqueued in part: the context stays failed
            if (c->sticky == ZI_OK) {
                c->sticky = st;
                c->sticky_msg = zi_last_error();
            }
            return st;
        }
        src = static_cast<const char *>(staged);
    }
    hipEvent_t ea = nullptr, eb = nullptr;
    if (c->timing) {
        zi_status st = ev_timed(c, &ea);
        if (st != ZI_OK) {
            if (fs) source_abandon(fs, fslot);
            return st;
        }
        HIPCHK(c, hipEventRecord(ea, c->h2d));
    }
    {
        hipError_t e = hipMemcpyAsync(c->wslot(s), src, bytes, hipMemcpyHostToDevice, c->h2d);
        if (e == hipSuccess && fs) e = hipEventRecord(source_copy_event(fs, fslot), c->h2d);
        if (e != hipSuccess) {
            if (fs) source_abandon(fs, fslot);
            return hip_fail(c, e, "hipMemcpyAsync(tile to device)");
        }
        if (fs) source_release(fs, fslot);
    }
    if (c->timing) {
        zi_status st = ev_timed(c, &eb);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(eb, c->h2d));
        c->crec.push_back(CopyRec{0, (double)bytes, ea, eb});
    }
    HIPCHK(c, hipEventRecord(c->w_ready[s], c->h2d));
    return ZI_OK;
}

zi_status write_back(zi_ctx *c, const zi_plan *p, int64_t tile, const void *src, hipEvent_t ready,
                     hipEvent_t done) {
    HIPCHK(c, hipStreamWaitEvent(c->d2h, ready, 0));
    const uint64_t bytes = p->info.dw_tile_bytes;
    char *dst = static_cast<char *>(p->prob.dW_host) + (uint64_t)tile * bytes;
    hipEvent_t ea = nullptr, eb = nullptr;
    if (c->timing) {
        zi_status st = ev_timed(c, &ea);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(ea, c->d2h));
    }
    HIPCHK(c, hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, c->d2h));
    if (c->timing) {
        zi_status st = ev_timed(c, &eb);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(eb, c->d2h));
        c->crec.push_back(CopyRec{1, (double)bytes, ea, eb});
    }
    HIPCHK(c, hipEventRecord(done, c->d2h));
    return ZI_OK;
}

zi_status gemm(zi_ctx *c, int kind, GemmOp op, int dtype, const GemmArgs &a, double flops,
               hipStream_t stream = nullptr) {
    if (!stream) stream = c->comp;
    hipEvent_t ea = nullptr, eb = nullptr;
    if (c->timing) {
        zi_status st = ev_timed(c, &ea);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(ea, stream));
    }
    hipError_t e = launch_gemm(op, dtype, a, stream);
    if (e != hipSuccess) return hip_fail(c, e, kKindNames[kind]);
    if (c->timing) {
        zi_status st = ev_timed(c, &eb);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(eb, stream));
        c->krec.push_back(KernelRec{kind, flops, ea, eb, (int)op, a.rows, a.cols, a.red});
    }
    return ZI_OK;
}

zi_status run_fwd(zi_ctx *c, const zi_plan *p, const void *X, void *Y, void *H) {
    const zi_problem &pr = p->prob;
    const zi_plan_info &in = p->info;
    const bool f32 = (pr.flags & ZI_FLAG_F32_OUT) != 0;
    const int64_t N = pr.N, n = in.n;
    const int d = c->d;
    const int64_t base = c->seq;
    const double tile_flops = 2.0 * (double)pr.T * (double)pr.K * (double)n;
    zi_status st;
    // The tiles' products are independent (disjoint output columns), so with a
    // second product stream they alternate between the two: the next tile's
    // workgroups take the compute units that the last wave of the previous
    // tile's leaves idle.  comp2 first waits for everything before this pass
    // on comp, and comp waits for comp2 at its end.
    // Only tiles whose product takes a few waves of workgroups gain: with many
    // waves the partial last one is a small share (measured: 3.5 waves per
    // tile, -5 %; 12.5 waves, no change).
    const int64_t wgs = gemm_workgroups(H ? GemmOp::FwdGelu : GemmOp::Fwd, pr.T, n);
    const bool two = c->comp2 && N > 1 && wgs < 8 * (int64_t)c->cus;
    if (two) {
        HIPCHK(c, hipEventRecord(c->fork, c->comp));
        HIPCHK(c, hipStreamWaitEvent(c->comp2, c->fork, 0));
    }
    for (int64_t j = 0; j < std::min<int64_t>(d, N); ++j)
        if ((st = stage(c, p, base + j, j)) != ZI_OK) return st;
    for (int64_t i = 0; i < N; ++i) {
        const int s = (int)((base + i) % d);
        hipStream_t ks = (two && (i & 1)) ? c->comp2 : c->comp;
        HIPCHK(c, hipStreamWaitEvent(ks, c->w_ready[s], 0));
        GemmArgs a{};
        a.Q = c->wslot(s);
        a.ldq = pr.K;
        a.P = X;
        a.ldp = pr.K;
        a.C = static_cast<char *>(Y) + i * n * (f32 ? 4 : 2);
        a.ldc = pr.M;
        a.C2 = H ? static_cast<char *>(H) + i * n * 2 : nullptr;
        a.rows = pr.T;
        a.cols = n;
        a.red = pr.K;
        a.out_f32 = f32 ? 1 : 0;
        if (H) {  // each product stream has its own split workspace: one launch at a time uses it
            const int k = ks == c->comp ? 0 : 1;
            a.split_part = c->split_part[k];
            a.split_cnt = c->split_cnt[k];
            a.split_cap = c->cus;
        }
        st = gemm(c, H ? K_FWD_GELU : K_FWD, H ? GemmOp::FwdGelu : GemmOp::Fwd, pr.dtype, a, tile_flops, ks);
        if (st != ZI_OK) return st;
        HIPCHK(c, hipEventRecord(c->w_free[s], ks));
        c->w_free_rec[s] = 1;
        if (i + d < N && (st = stage(c, p, base + i + d, i + d)) != ZI_OK) return st;
    }
    if (two) {
        HIPCHK(c, hipEventRecord(c->join, c->comp2));
        HIPCHK(c, hipStreamWaitEvent(c->comp, c->join, 0));
    }
    c->seq += N;
    return ZI_OK;
}

zi_status run_bwd(zi_ctx *c, const zi_plan *p, const void *X, const void *dY, float *dX, void *Yr) {
    const zi_problem &pr = p->prob;
    const zi_plan_info &in = p->info;
    const bool f32 = (pr.flags & ZI_FLAG_F32_OUT) != 0;
    const int64_t N = pr.N, n = in.n;
    const int d = c->d;
    const int64_t base = c->seq, dbase = c->dw_seq;
    const double tile_flops = 2.0 * (double)pr.T * (double)pr.K * (double)n;
    // With separate gradient slots and at least two weight slots, the dX
    // product of tiles 2j and 2j + 1 is one launch over both (a reduction of
    // 2n), which halves the fp32 read-add-store passes over dX.  Tile 2j stays
    // in its slot until that launch has read it; the dW product of tile 2j + 1
    // runs after it and covers the copy of the next tile into the freed slot.
    static_assert(kPairStep == kGemmStep, "pairs split the reduction at a GEMM step");
    const bool pairs = pairs_apply((int)N, d, c->dw_slots, n);
    // The recomputed forward of such a pair is one launch too (output columns
    // of both tiles), run once tile 2j + 1 has landed, where that takes fewer
    // rounds of workgroups over the compute units than two launches: at
    // T = 32768 a 1600-column tile is 855 workgroups of 320 x 192 (4 rounds
    // of 256, the last a third full) and the pair 1710 (7 rounds).  The
    // launch's macro-tile must not straddle the two tiles' columns.
    bool re_pairs = false;
    if (pairs && Yr) {
        int tr = 0, tc = 0;
        gemm_tile(GemmOp::Fwd, pr.T, 2 * n, &tr, &tc);
        const int64_t cus = c->cus > 0 ? c->cus : 1;
        const int64_t w1 = gemm_workgroups(GemmOp::Fwd, pr.T, n), w2 = gemm_workgroups(GemmOp::Fwd, pr.T, 2 * n);
        re_pairs = n % tc == 0 && (w2 + cus - 1) / cus < 2 * ((w1 + cus - 1) / cus);
    }
    zi_status st;
    // The products of a backward pass stay on one stream: running the
    // recomputed forward beside the previous tile's dW on the second stream
    // was measured slower (452 -> 478 ms for the block's down-projection).
    int64_t staged = std::min<int64_t>(d, N);
    for (int64_t j = 0; j < staged; ++j)
        if ((st = stage(c, p, base + j, j)) != ZI_OK) return st;
    int64_t released = -1;  // every tile <= released has had its weight slot freed
    for (int64_t i = 0; i < N; ++i) {
        const int s = (int)((base + i) % d);
        HIPCHK(c, hipStreamWaitEvent(c->comp, c->w_ready[s], 0));
        const uint16_t *dYi = static_cast<const uint16_t *>(dY) + i * n;
        const bool first_of_pair = pairs && (i % 2 == 0) && i + 1 < N;
        const bool second_of_pair = pairs && (i % 2 == 1);
        if (Yr && !(re_pairs && first_of_pair)) {  // recomputed forward slice(s) from the staged tile(s)
            const bool both = re_pairs && second_of_pair;
            const int64_t i0 = both ? i - 1 : i;
            GemmArgs a{};
            a.Q = c->wslot(both ? (int)((base + i0) % d) : s);
            a.ldq = pr.K;
            if (both) {
                a.Q2 = c->wslot(s);
                a.qsplit = n;
            }
            a.P = X;
            a.ldp = pr.K;
            a.C = static_cast<char *>(Yr) + i0 * n * (f32 ? 4 : 2);
            a.ldc = pr.M;
            a.rows = pr.T;
            a.cols = (i - i0 + 1) * n;
            a.red = pr.K;
            a.out_f32 = f32 ? 1 : 0;
            if ((st = gemm(c, K_FWD_RECOMPUTE, GemmOp::Fwd, pr.dtype, a, tile_flops * (double)(i - i0 + 1))) !=
                ZI_OK)
                return st;
        }
        if (!first_of_pair) {  // dX (+)= dY_i W_i^T (or over tiles i-1, i): W^t[r][k] read across its rows
            const int64_t i0 = second_of_pair ? i - 1 : i;
            GemmArgs a{};
            a.Q = c->wslot(second_of_pair ? (int)((base + i0) % d) : s);
            a.ldq = pr.K;
            if (second_of_pair) {
                a.Q2 = c->wslot(s);
                a.qsplit = n;
            }
            a.P = static_cast<const uint16_t *>(dY) + i0 * n;
            a.ldp = pr.M;
            a.C = dX;
            a.ldc = pr.K;
            a.rows = pr.T;
            a.cols = pr.K;
            a.red = (i - i0 + 1) * n;
            a.accumulate = i0 > 0 ? 1 : 0;
            // one persistent workgroup per compute unit
            a.wg_cap = (c->debug & ZI_DEBUG_DX_PER_TILE) ? 0 : std::max(8, c->cus / 8 * 8);
            if ((st = gemm(c, K_DX, GemmOp::Dx, pr.dtype, a, tile_flops * (double)(i - i0 + 1))) != ZI_OK)
                return st;
        }
        char *dst;
        hipEvent_t ready, done;
        int ds = -1;
        if (c->dw_slots > 0) {
            if (!first_of_pair) {
                for (int64_t t = (second_of_pair ? i - 1 : i); t <= i; ++t) {
                    const int ts = (int)((base + t) % d);
                    HIPCHK(c, hipEventRecord(c->w_free[ts], c->comp));
                    c->w_free_rec[ts] = 1;
                }
                released = i;
            }
            ds = (int)((dbase + i) % c->dw_slots);
            if (c->dw_free_rec[ds]) HIPCHK(c, hipStreamWaitEvent(c->comp, c->dw_free[ds], 0));
            dst = c->dwslot(ds);
            ready = c->dw_ready[ds];
            done = c->dw_free[ds];
        } else {
            dst = c->wslot(s);  // the weight tile is consumed; its slot takes dW_i
            ready = c->dw_ready[s];
            done = c->w_free[s];
        }
        if (c->debug & ZI_DEBUG_POISON)  // a write-back still reading the slot would copy NaNs
            HIPCHK(c, hipMemsetAsync(dst, 0xFF, in.dw_tile_bytes, c->comp));
        {  // dW_i^t[m][k] = sum_t dY[t][i n + m] X[t][k]
            GemmArgs a{};
            a.Q = X;
            a.ldq = pr.K;
            a.P = dYi;
            a.ldp = pr.M;
            a.C = dst;
            a.ldc = pr.K;
            a.rows = n;
            a.cols = pr.K;
            a.red = pr.T;
            a.out_f32 = f32 ? 1 : 0;
            if ((st = gemm(c, K_DW, GemmOp::Dw, pr.dtype, a, tile_flops)) != ZI_OK) return st;
        }
        HIPCHK(c, hipEventRecord(ready, c->comp));
        if ((st = write_back(c, p, i, dst, ready, done)) != ZI_OK) return st;
        if (zi_adam *a = c->adam_of(p)) {  // update tile i on the host once dW_i has landed
            hipEvent_t landed = nullptr;
            HIPCHK(c, hipEventCreateWithFlags(&landed, hipEventDisableTiming | hipEventBlockingSync));
            const hipError_t e = hipEventRecord(landed, c->d2h);
            if (e != hipSuccess) {
                (void)hipEventDestroy(landed);
                return hip_fail(c, e, "hipEventRecord(gradient landed)");
            }
            adam_enqueue(a, i, landed);
        }
        if (ds >= 0) {
            c->dw_free_rec[ds] = 1;
        } else {
            c->w_free_rec[s] = 1;
            released = i;
        }
        // stage every tile whose slot has now been released
        for (; staged < N && staged - d <= released; ++staged)
            if ((st = stage(c, p, base + staged, staged)) != ZI_OK) return st;
    }
    c->seq += N;
    c->dw_seq += N;
    return ZI_OK;
}

}  // namespace

extern "C" {

const char *zi_last_error(void) { return g_err; }

int32_t zi_version(void) { return 100; }

zi_status zi_host_alloc(uint64_t bytes, void **out) {
    clear_error();
    if (!out || !bytes) return fail(ZI_ERR_ARG, "zi_host_alloc needs bytes > 0 and an out pointer");
    *out = nullptr;
    HIPCHK(nullptr, hipHostMalloc(out, bytes, hipHostMallocDefault));
    return ZI_OK;
}

zi_status zi_stream_create(void **out) {
    clear_error();
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    *out = nullptr;
    hipStream_t s = nullptr;
    HIPCHK(nullptr, hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
    *out = s;
    return ZI_OK;
}

zi_status zi_copy_stream_create(int32_t n_cus, void **out) {
    clear_error();
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (n_cus < 1) return fail(ZI_ERR_ARG, "n_cus = %d must be at least 1", n_cus);
    int dev = 0, cus = 0, xccs = 1;
    HIPCHK(nullptr, hipGetDevice(&dev));
    HIPCHK(nullptr, hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    HIPCHK(nullptr, hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev));
    if (xccs < 1) xccs = 1;
    if (n_cus > cus || n_cus % xccs)
        return fail(ZI_ERR_ARG, "n_cus = %d must be a multiple of the %d XCCs, at most %d", n_cus, xccs,
                    cus);
    std::vector<uint32_t> mask((size_t)(cus + 31) / 32, 0u);
    for (int i = 0; i < n_cus; ++i) mask[(size_t)i / 32] |= 1u << (i % 32);
    hipStream_t s = nullptr;
    HIPCHK(nullptr, hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data()));
    *out = s;
    return ZI_OK;
}

zi_status zi_stream_destroy(void *stream) {
    clear_error();
    if (!stream) return ZI_OK;
    HIPCHK(nullptr, hipStreamDestroy(static_cast<hipStream_t>(stream)));
    return ZI_OK;
}

zi_status zi_host_free(void *ptr) {
    clear_error();
    if (!ptr) return ZI_OK;
    HIPCHK(nullptr, hipHostFree(ptr));
    return ZI_OK;
}

// The forward GeLU epilogue reads per-device tables of H over every 16-bit A;
// the first context created on a device builds them (once, on its compute
// stream, and waits for them).
static zi_status ensure_gelu_tables(int device, hipStream_t stream) {
    static std::mutex mu;
    static std::vector<char> built;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)built.size() <= device) built.resize(device + 1, 0);
    if (built[device]) return ZI_OK;
    hipError_t e = build_gelu_tables(stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(nullptr, e, "building the GeLU tables");
    built[device] = 1;
    return ZI_OK;
}

zi_status zi_ctx_create(const zi_plan *plan, void *workspace_dev, uint64_t workspace_bytes,
                        void *compute_stream, void *h2d_stream, void *d2h_stream, zi_ctx **out) {
    clear_error();
    if (!plan || !out) return fail(ZI_ERR_ARG, "plan and out are required");
    *out = nullptr;
    if (!workspace_dev) return fail(ZI_ERR_ARG, "workspace is NULL");
    if ((uintptr_t)workspace_dev & 255u) return fail(ZI_ERR_ALIGN, "workspace is not 256-byte aligned");
    const zi_plan_info &in = plan->info;
    if (workspace_bytes < in.ring_bytes)
        return fail(ZI_ERR_BUDGET, "workspace of %llu B is smaller than the ring's %llu B",
                    (unsigned long long)workspace_bytes, (unsigned long long)in.ring_bytes);
    zi_ctx *c = new (std::nothrow) zi_ctx;
    if (!c) return fail(ZI_ERR_ARG, "out of host memory");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        delete c;
        return fail(ZI_ERR_HIP, "hipGetDevice failed");
    }
    c->device = dev;
    if (hipDeviceGetAttribute(&c->cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c->cus < 1)
        c->cus = 256;
    if (ensure_gelu_tables(dev, static_cast<hipStream_t>(compute_stream)) != ZI_OK) {
        delete c;
        return ZI_ERR_HIP;
    }
    c->comp = static_cast<hipStream_t>(compute_stream);
    c->h2d = static_cast<hipStream_t>(h2d_stream);
    c->d2h = static_cast<hipStream_t>(d2h_stream);
    c->ws = static_cast<char *>(workspace_dev);
    c->ws_bytes = workspace_bytes;
    c->d = in.d;
    c->dw_slots = in.dw_slots;
    c->slot_bytes = round_up(in.tile_bytes, 256);
    c->dw_slot_bytes = in.dw_slots ? round_up(in.dw_tile_bytes, 256) : 0;
    const int nd = std::max(c->d, std::max(c->dw_slots, 1));
    auto mk = [&](std::vector<hipEvent_t> &v, int count) -> bool {
        v.assign(count, nullptr);
        for (int i = 0; i < count; ++i)
            if (hipEventCreateWithFlags(&v[i], hipEventDisableTiming) != hipSuccess) return false;
        return true;
    };
    if (!mk(c->w_ready, c->d) || !mk(c->w_free, c->d) || !mk(c->dw_ready, nd) ||
        !mk(c->dw_free, std::max(c->dw_slots, 1))) {
        zi_ctx_destroy(c);
        return fail(ZI_ERR_HIP, "hipEventCreateWithFlags failed");
    }
    c->w_free_rec.assign(c->d, 0);
    c->dw_free_rec.assign(std::max(c->dw_slots, 1), 0);
    const uint64_t split_at = round_up(in.ring_bytes, 256);
    if (workspace_bytes >= split_at + 2 * kSplitBytes) {
        // the counters start at zero; each launch leaves them at zero
        for (int k = 0; k < 2; ++k) {
            char *at = c->ws + split_at + (uint64_t)k * kSplitBytes;
            c->split_part[k] = reinterpret_cast<float *>(at);
            c->split_cnt[k] = reinterpret_cast<uint32_t *>(at + kSplitPartBytes);
            if (hipMemsetAsync(c->split_cnt[k], 0, kSplitBytes - kSplitPartBytes, c->comp) != hipSuccess) {
                zi_ctx_destroy(c);
                return fail(ZI_ERR_HIP, "clearing the split counters failed");
            }
        }
        if (hipStreamSynchronize(c->comp) != hipSuccess) {
            zi_ctx_destroy(c);
            return fail(ZI_ERR_HIP, "clearing the split counters failed");
        }
    }
    *out = c;
    return ZI_OK;
}

uint64_t zi_gelu_split_bytes(void) { return 2 * kSplitBytes; }

zi_status zi_ctx_destroy(zi_ctx *c) {
    clear_error();
    if (!c) return ZI_OK;
    if (c->comp || c->h2d || c->d2h) {
        if (c->comp2) (void)hipStreamSynchronize(c->comp2);
        (void)hipStreamSynchronize(c->comp);
        (void)hipStreamSynchronize(c->h2d);
        (void)hipStreamSynchronize(c->d2h);
    }
    for (auto *v : {&c->w_ready, &c->w_free, &c->dw_ready, &c->dw_free, &c->pool})
        for (hipEvent_t e : *v)
            if (e) (void)hipEventDestroy(e);
    if (c->fork) (void)hipEventDestroy(c->fork);
    if (c->join) (void)hipEventDestroy(c->join);
    delete c;
    return ZI_OK;
}

zi_status zi_tiled_linear_fwd(zi_ctx *ctx, const zi_plan *plan, const void *X_dev, void *Y_dev) {
    clear_error();
    zi_status st = check_pass(ctx, plan, false);
    if (st != ZI_OK) return st;
    if ((st = check_dev_ptr(X_dev, "X")) != ZI_OK || (st = check_dev_ptr(Y_dev, "Y")) != ZI_OK) return st;
    return run_fwd(ctx, plan, X_dev, Y_dev, nullptr);
}

zi_status zi_tiled_linear_fwd_gelu(zi_ctx *ctx, const zi_plan *plan, const void *X_dev, void *A_dev,
                                   void *H_dev) {
    clear_error();
    zi_status st = check_pass(ctx, plan, false);
    if (st != ZI_OK) return st;
    if ((st = check_dev_ptr(X_dev, "X")) != ZI_OK || (st = check_dev_ptr(A_dev, "A")) != ZI_OK ||
        (st = check_dev_ptr(H_dev, "H")) != ZI_OK)
        return st;
    return run_fwd(ctx, plan, X_dev, A_dev, H_dev);
}

zi_status zi_tiled_linear_bwd(zi_ctx *ctx, const zi_plan *plan, const void *X_dev, const void *dY_dev,
                              float *dX_dev) {
    clear_error();
    zi_status st = check_pass(ctx, plan, true);
    if (st != ZI_OK) return st;
    if ((st = check_dev_ptr(X_dev, "X")) != ZI_OK || (st = check_dev_ptr(dY_dev, "dY")) != ZI_OK ||
        (st = check_dev_ptr(dX_dev, "dX")) != ZI_OK)
        return st;
    return run_bwd(ctx, plan, X_dev, dY_dev, dX_dev, nullptr);
}

zi_status zi_tiled_linear_bwd_recompute(zi_ctx *ctx, const zi_plan *plan, const void *X_dev,
                                        const void *dY_dev, float *dX_dev, void *Yr_dev) {
    clear_error();
    zi_status st = check_pass(ctx, plan, true);
    if (st != ZI_OK) return st;
    if ((st = check_dev_ptr(X_dev, "X")) != ZI_OK || (st = check_dev_ptr(dY_dev, "dY")) != ZI_OK ||
        (st = check_dev_ptr(dX_dev, "dX")) != ZI_OK || (st = check_dev_ptr(Yr_dev, "Yr")) != ZI_OK)
        return st;
    return run_bwd(ctx, plan, X_dev, dY_dev, dX_dev, Yr_dev);
}

zi_status zi_ctx_attach_source(zi_ctx *ctx, const zi_plan *plan, zi_file_source *src) {
    clear_error();
    if (!ctx || !plan) return fail(ZI_ERR_ARG, "context and plan are required");
    if (src && source_plan(src) != plan) return fail(ZI_ERR_STATE, "the source was made for another plan");
    if (src && ctx->adam_of(plan))
        return fail(ZI_ERR_STATE, "an optimizer is attached to this plan; it updates W_host, not the file");
    for (auto it = ctx->sources.begin(); it != ctx->sources.end(); ++it) {
        if (it->first != plan) continue;
        if (src)
            it->second = src;
        else
            ctx->sources.erase(it);
        return ZI_OK;
    }
    if (src) ctx->sources.emplace_back(plan, src);
    return ZI_OK;
}

zi_status zi_ctx_attach_adam(zi_ctx *ctx, const zi_plan *plan, zi_adam *adam) {
    clear_error();
    if (!ctx || !plan) return fail(ZI_ERR_ARG, "context and plan are required");
    if (adam && adam_plan(adam) != plan) return fail(ZI_ERR_STATE, "the optimizer was made for another plan");
    if (adam && ctx->source_of(plan))
        return fail(ZI_ERR_STATE, "a file source is attached to this plan; the optimizer would update W_host");
    for (auto it = ctx->adams.begin(); it != ctx->adams.end(); ++it) {
        if (it->first != plan) continue;
        if (adam)
            it->second = adam;
        else
            ctx->adams.erase(it);
        return ZI_OK;
    }
    if (adam) ctx->adams.emplace_back(plan, adam);
    return ZI_OK;
}

static zi_status gelu_bwd(zi_ctx *ctx, int32_t dtype, const float *dH_dev, const void *A_dev, void *dA_dev,
                          int64_t count, bool out_f32) {
    clear_error();
    zi_status st = check_ctx(ctx);
    if (st != ZI_OK) return st;
    if (dtype != ZI_F16 && dtype != ZI_BF16) return fail(ZI_ERR_ARG, "bad dtype %d", dtype);
    if (count < 0) return fail(ZI_ERR_ARG, "count < 0");
    if ((st = check_dev_ptr(dH_dev, "dH")) != ZI_OK || (st = check_dev_ptr(A_dev, "A")) != ZI_OK ||
        (st = check_dev_ptr(dA_dev, "dA")) != ZI_OK)
        return st;
    hipEvent_t ea = nullptr, eb = nullptr;
    if (ctx->timing) {
        if ((st = ev_timed(ctx, &ea)) != ZI_OK) return st;
        HIPCHK(ctx, hipEventRecord(ea, ctx->comp));
    }
    hipError_t e = launch_gelu_bwd(dtype, dH_dev, A_dev, dA_dev, count, out_f32, ctx->comp);
    if (e != hipSuccess) return hip_fail(ctx, e, "gelu_bwd");
    if (ctx->timing) {
        if ((st = ev_timed(ctx, &eb)) != ZI_OK) return st;
        HIPCHK(ctx, hipEventRecord(eb, ctx->comp));
        ctx->krec.push_back(KernelRec{K_GELU_BWD, (double)count, ea, eb, -1, count, 1, 1});
    }
    return ZI_OK;
}

zi_status zi_gelu_bwd(zi_ctx *ctx, int32_t dtype, const float *dH_dev, const void *A_dev, void *dA_dev,
                      int64_t count) {
    return gelu_bwd(ctx, dtype, dH_dev, A_dev, dA_dev, count, false);
}

zi_status zi_gelu_bwd_f32(zi_ctx *ctx, int32_t dtype, const float *dH_dev, const void *A_dev, float *dA_dev,
                          int64_t count) {
    return gelu_bwd(ctx, dtype, dH_dev, A_dev, dA_dev, count, true);
}

zi_status zi_sync(zi_ctx *ctx) {
    clear_error();
    if (!ctx) return fail(ZI_ERR_ARG, "context is NULL");
    if (ctx->comp2) {
        const hipError_t e0 = hipStreamSynchronize(ctx->comp2);
        if (e0 != hipSuccess) return hip_fail(ctx, e0, "hipStreamSynchronize(second compute)");
    }
    hipError_t e1 = hipStreamSynchronize(ctx->comp);
    hipError_t e2 = hipStreamSynchronize(ctx->h2d);
    hipError_t e3 = hipStreamSynchronize(ctx->d2h);
    if (e1 != hipSuccess) return hip_fail(ctx, e1, "hipStreamSynchronize(compute)");
    if (e2 != hipSuccess) return hip_fail(ctx, e2, "hipStreamSynchronize(h2d)");
    if (e3 != hipSuccess) return hip_fail(ctx, e3, "hipStreamSynchronize(d2h)");
    for (const auto &e : ctx->adams) {
        const zi_status st = adam_wait_all(e.second);
        if (st != ZI_OK) return st;
    }
    if (ctx->sticky != ZI_OK) return fail(ctx->sticky, "%s", ctx->sticky_msg.c_str());
    return ZI_OK;
}

zi_status zi_ctx_set_second_stream(zi_ctx *ctx, void *stream) {
    clear_error();
    zi_status st = check_ctx(ctx);
    if (st != ZI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (s && (s == ctx->comp || s == ctx->h2d || s == ctx->d2h))
        return fail(ZI_ERR_ARG, "the second product stream must be a stream of its own");
    if (s && !ctx->fork) {
        HIPCHK(ctx, hipEventCreateWithFlags(&ctx->fork, hipEventDisableTiming));
        HIPCHK(ctx, hipEventCreateWithFlags(&ctx->join, hipEventDisableTiming));
    }
    // work already on the old second stream must be done before it is let go
    if (ctx->comp2) HIPCHK(ctx, hipStreamSynchronize(ctx->comp2));
    ctx->comp2 = s;
    return ZI_OK;
}

zi_status zi_ctx_set_debug(zi_ctx *ctx, uint32_t flags, uint32_t copy_delay_us) {
    clear_error();
    if (!ctx) return fail(ZI_ERR_ARG, "context is NULL");
    if (flags & ~(ZI_DEBUG_POISON | ZI_DEBUG_DX_PER_TILE)) return fail(ZI_ERR_ARG, "unknown debug flags 0x%x", flags);
    if (copy_delay_us > 10000000u) return fail(ZI_ERR_ARG, "copy delay above 10 s");
    ctx->debug = flags;
    ctx->delay_us = copy_delay_us;
    return ZI_OK;
}

zi_status zi_ctx_set_timing(zi_ctx *ctx, int32_t enable) {
    clear_error();
    if (!ctx) return fail(ZI_ERR_ARG, "context is NULL");
    ctx->timing = enable != 0;
    return ZI_OK;
}

zi_status zi_ctx_reset_stats(zi_ctx *ctx) {
    zi_status st = zi_sync(ctx);
    if (st != ZI_OK) return st;
    ctx->krec.clear();
    ctx->crec.clear();
    ctx->pool_used = 0;
    return ZI_OK;
}

zi_status zi_ctx_stats(zi_ctx *ctx, zi_stats *out) {
    zi_status st = zi_sync(ctx);
    if (st != ZI_OK) return st;
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    memset(out, 0, sizeof(*out));
    out->kind_count = K_COUNT;
    for (int k = 0; k < K_COUNT; ++k) snprintf(out->kind_name[k], sizeof(out->kind_name[k]), "%s", kKindNames[k]);
    hipEvent_t ref = nullptr;
    if (!ctx->krec.empty()) ref = ctx->krec.front().a;
    if (!ctx->crec.empty() && !ref) ref = ctx->crec.front().a;
    double lo = 0, hi = 0;
    bool any = false;
    auto span = [&](hipEvent_t a, hipEvent_t b) -> zi_status {
        float t0 = 0, t1 = 0;
        HIPCHK(ctx, hipEventElapsedTime(&t0, ref, a));
        HIPCHK(ctx, hipEventElapsedTime(&t1, ref, b));
        if (!any || t0 < lo) lo = t0;
        if (!any || t1 > hi) hi = t1;
        any = true;
        return ZI_OK;
    };
    std::vector<std::pair<double, double>> busy;  // kernel intervals, ms after the first event
    std::vector<double> dur;                        // per launch, in krec order
    for (const KernelRec &r : ctx->krec) {
        float ms = 0, t0 = 0;
        HIPCHK(ctx, hipEventElapsedTime(&ms, r.a, r.b));
        HIPCHK(ctx, hipEventElapsedTime(&t0, ref, r.a));
        out->launches[r.kind] += 1;
        out->kernel_ms[r.kind] += ms;
        out->flops[r.kind] += r.flops;
        busy.emplace_back(t0, (double)t0 + ms);
        dur.push_back(ms);
        if ((st = span(r.a, r.b)) != ZI_OK) return st;
    }
    // Per kernel (product and launch shape): totals, and the launches that ran
    // alone.  A launch ran alone when no other launch's interval reaches into
    // it; intervals that only touch (within 2 us, the events' resolution on one
    // stream) do not count as overlapping.
    {
        const size_t n = busy.size();
        std::vector<size_t> order(n);
        for (size_t i = 0; i < n; ++i) order[i] = i;
        std::sort(order.begin(), order.end(), [&](size_t x, size_t y) { return busy[x] < busy[y]; });
        std::vector<char> solo(n, 1);
        constexpr double eps = 2e-3;
        double reach = -1e300;  // latest end among the launches started so far
        size_t reach_of = n;
        for (size_t j = 0; j < n; ++j) {
            const size_t i = order[j];
            if (busy[i].first < reach - eps) {
                solo[i] = 0;
                if (reach_of < n) solo[reach_of] = 0;
            }
            if (busy[i].second > reach) {
                reach = busy[i].second;
                reach_of = i;
            }
        }
        for (size_t i = 0; i < n; ++i) {
            const KernelRec &r = ctx->krec[i];
            int e = 0;
            while (e < out->kernel_count &&
                   !(out->kernel[e].rows == r.rows && out->kernel[e].cols == r.cols && out->kernel[e].red == r.red &&
                     strcmp(out->kernel[e].name, kKindNames[r.op == -1 ? K_GELU_BWD : r.op]) == 0))
                ++e;
            if (e == out->kernel_count) {
                if (e == ZI_STATS_KERNELS) continue;
                ++out->kernel_count;
                zi_kernel_stats &k = out->kernel[e];
                // the name of the product, whichever pass launched it
                snprintf(k.name, sizeof(k.name), "%s", kKindNames[r.op == -1 ? K_GELU_BWD : r.op]);
                k.rows = r.rows;
                k.cols = r.cols;
                k.red = r.red;
            }
            zi_kernel_stats &k = out->kernel[e];
            k.launches += 1;
            k.ms += dur[i];
            k.flops += r.flops;
            if (solo[i]) {
                k.solo_launches += 1;
                k.solo_ms += dur[i];
            }
        }
    }
    // time the compute units had work: the union of the kernel intervals
    // (kernels on the two product streams may overlap)
    std::sort(busy.begin(), busy.end());
    double cur_lo = 0, cur_hi = -1;
    for (const auto &b : busy) {
        if (b.first > cur_hi) {
            if (cur_hi > cur_lo) out->compute_busy_ms += cur_hi - cur_lo;
            cur_lo = b.first;
            cur_hi = b.second;
        } else if (b.second > cur_hi) {
            cur_hi = b.second;
        }
    }
    if (cur_hi > cur_lo) out->compute_busy_ms += cur_hi - cur_lo;
    for (const CopyRec &r : ctx->crec) {
        float ms = 0;
        HIPCHK(ctx, hipEventElapsedTime(&ms, r.a, r.b));
        if (r.d2h) {
            out->d2h_copies += 1;
            out->d2h_ms += ms;
            out->d2h_bytes += r.bytes;
        } else {
            out->h2d_copies += 1;
            out->h2d_ms += ms;
            out->h2d_bytes += r.bytes;
        }
        if ((st = span(r.a, r.b)) != ZI_OK) return st;
    }
    out->span_ms = any ? hi - lo : 0.0;
    return ZI_OK;
}

zi_status zi_ctx_timed_records(zi_ctx *ctx, zi_timed_rec *out, int32_t cap, int32_t *count) {
    clear_error();
    if (!ctx || !count) return fail(ZI_ERR_ARG, "ctx and count are required");
    if (cap < 0 || (cap > 0 && !out)) return fail(ZI_ERR_ARG, "out must hold cap = %d records", cap);
    zi_status st = zi_sync(ctx);
    if (st != ZI_OK) return st;
    const size_t total = ctx->krec.size() + ctx->crec.size();
    *count = total > (size_t)INT32_MAX ? INT32_MAX : (int32_t)total;
    hipEvent_t ref = nullptr;
    if (!ctx->krec.empty()) ref = ctx->krec.front().a;
    if (!ctx->crec.empty() && !ref) ref = ctx->crec.front().a;
    int32_t n = 0;
    auto put = [&](int32_t what, int32_t kind, int64_t rows, int64_t cols, int64_t red, hipEvent_t a,
                   hipEvent_t b) -> zi_status {
        if (n >= cap) return ZI_OK;
        float t0 = 0, t1 = 0;
        HIPCHK(ctx, hipEventElapsedTime(&t0, ref, a));
        HIPCHK(ctx, hipEventElapsedTime(&t1, ref, b));
        out[n++] = zi_timed_rec{what, kind, rows, cols, red, (double)t0, (double)t1};
        return ZI_OK;
    };
    for (const KernelRec &r : ctx->krec)
        if ((st = put(0, r.kind, r.rows, r.cols, r.red, r.a, r.b)) != ZI_OK) return st;
    for (const CopyRec &r : ctx->crec)
        if ((st = put(r.d2h ? 2 : 1, -1, (int64_t)r.bytes, 0, 0, r.a, r.b)) != ZI_OK) return st;
    return ZI_OK;
}

}  // extern "C"
