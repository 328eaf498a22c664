// zi_noalloc.hip -- the tiled forward for callers that cannot allocate.
//
// zi_tiled_linear_fwd_noalloc runs the products of zi_tiled_linear_fwd (the
// same GEMM kernel, the same tile order) with the tile buffer in `scratch`, a
// file-scope device array that the library owns, instead of a context's
// workspace, and with every copy and product on the one stream the caller
// passes.  It makes no allocation of any kind: no device or host memory, no
// events, no context.
//
// `scratch` holds one weight tile at a time: tile i is copied into it, its
// product is launched, and the copy of tile i + 1 (on the same stream) waits
// for that product.  So the copies do not overlap the products here; the
// ring and its overlap are the context's business.
//
// Per device, the array's device address is looked up once, with that device
// current, and kept; host code uses only that address (the array's name
// denotes a host-side stand-in in host code).  Every call on a device shares
// its array, which keeps the last tile that was copied into it: calls that
// overlap on one device (on two streams, or from two threads) race and give
// wrong results.  Nothing in the array needs to start at zero: each product
// reads only the tile copied in just before it on the same stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/zi.h"
#include "zi_host.h"
#include "zi_internal.h"

namespace {

static __device__ __align__(256) char scratch[ZI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device (null: not looked up yet)

zi_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return zi::fail(ZI_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return zi::fail(ZI_ERR_STATE, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return zi::fail(ZI_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                            hipGetErrorString(e));
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ZI_OK;
}

bool pinned(const void *p, uint64_t bytes) {
    const char *q[2] = {static_cast<const char *>(p), static_cast<const char *>(p) + bytes - 1};
    for (const char *x : q) {
        hipPointerAttribute_t a;
        if (hipPointerGetAttributes(&a, x) != hipSuccess) {
            (void)hipGetLastError();
            return false;
        }
        if (a.type != hipMemoryTypeHost) return false;
    }
    return true;
}

}  // namespace

extern "C" zi_status zi_tiled_linear_fwd_noalloc(const zi_plan *plan, const void *X_dev, void *Y_dev,
                                                  void *stream) {
    zi::clear_error();
    if (!plan) return zi::fail(ZI_ERR_ARG, "plan is NULL");
    if (!X_dev || !Y_dev) return zi::fail(ZI_ERR_ARG, "X and Y are required");
    if (((uintptr_t)X_dev & 15u) || ((uintptr_t)Y_dev & 15u))
        return zi::fail(ZI_ERR_ALIGN, "X and Y must be 16-byte aligned");
    const zi_problem &pr = plan->prob;
    const zi_plan_info &in = plan->info;
    if (in.tile_bytes > (uint64_t)ZI_NOALLOC_SCRATCH_BYTES)
        return zi::fail(ZI_ERR_BUDGET,
                        "a weight tile of %llu B exceeds the %llu B static tile buffer of the no-allocation "
                        "forward; split W into more tiles",
                        (unsigned long long)in.tile_bytes, (unsigned long long)ZI_NOALLOC_SCRATCH_BYTES);
    if (!pr.W_host) return zi::fail(ZI_ERR_ARG, "plan has no W_host");
    if (!pinned(pr.W_host, (uint64_t)pr.M * (uint64_t)pr.K * 2u))
        return zi::fail(ZI_ERR_NOT_PINNED, "W_host is not page-locked host memory");
    void *buf = nullptr;
    zi_status st = scratch_of_current_device(&buf);
    if (st != ZI_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f32 = (pr.flags & ZI_FLAG_F32_OUT) != 0;
    const int64_t n = in.n;
    for (int64_t i = 0; i < pr.N; ++i) {
        const char *src = static_cast<const char *>(pr.W_host) + (uint64_t)i * in.tile_bytes;
        hipError_t e = hipMemcpyAsync(buf, src, in.tile_bytes, hipMemcpyHostToDevice, s);
        if (e == hipSuccess) {
            zi::GemmArgs a{};
            a.Q = buf;
            a.ldq = pr.K;
            a.P = X_dev;
            a.ldp = pr.K;
            a.C = static_cast<char *>(Y_dev) + i * n * (f32 ? 4 : 2);
            a.ldc = pr.M;
            a.rows = pr.T;
            a.cols = n;
            a.red = pr.K;
            a.out_f32 = f32 ? 1 : 0;
            e = zi::launch_gemm(zi::GemmOp::Fwd, pr.dtype, a, s);
        }
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return zi::fail(ZI_ERR_HIP, "tile %lld of the no-allocation forward: %s", (long long)i,
                            hipGetErrorString(e));
        }
    }
    return ZI_OK;
}
