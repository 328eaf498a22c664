// zi_adam.cpp -- Adam on the host, beside the tiled path.
//
// The Adam update is elementwise (about 12 FLOPs against 24 bytes), so no
// tier can hide it behind GPU work and it runs on the CPU next to the memory
// it touches (ZeRO-Infinity transformer-math page, section "Applying the
// test: which state can live where").  Its state is an fp32 master weight and
// two fp32 moments, 12 bytes per parameter (GPU ZeRO-sharding page, section
// "The architecture: every piece explained"), and the updated 16-bit
// parameters are the next step's resting copy (same page, "End-to-end flow").
// The update is Adam as Kingma and Ba publish it: bias-corrected moments, no
// weight decay; the per-element order of the fp32 operations is fixed (see
// zi.h) and is the same in the vector and the scalar code, which therefore
// agree bit for bit.
//
// With a context attached, each tile is updated as soon as its dW has been
// written back: one coordinator thread per process takes the tiles of every
// optimizer in the order they were queued, waits for each tile's copy event,
// then splits the tile over a persistent pool of worker threads.
#include <hip/hip_runtime_api.h>
#include <immintrin.h>
#include <math.h>
#include <sched.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "zi_host.h"

// Keep every multiply and add separately rounded, as the order above states.
#pragma clang fp contract(off)

namespace zi {
namespace {

struct AdamK {
    float b1, omb1, b2, omb2, step_size, c2, eps;
};

AdamK adam_consts(const zi_adam_hparams &hp, int64_t step) {
    const double b1t = pow((double)hp.beta1, (double)step);
    const double b2t = pow((double)hp.beta2, (double)step);
    AdamK k;
    k.b1 = hp.beta1;
    k.omb1 = (float)(1.0 - (double)hp.beta1);
    k.b2 = hp.beta2;
    k.omb2 = (float)(1.0 - (double)hp.beta2);
    k.step_size = (float)((double)hp.lr / (1.0 - b1t));
    k.c2 = (float)(1.0 / (1.0 - b2t));
    k.eps = hp.eps;
    return k;
}

// ---- 16-bit formats (exact decode, round-to-nearest-even encode) ----

inline float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}
inline uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

inline float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t e = (h >> 10) & 0x1f, mant = h & 0x3ffu;
    if (e == 0) {  // zero or subnormal: mant * 2^-24, exact in fp32
        const float v = (float)mant * 5.9604644775390625e-08f;
        return bits_f32(f32_bits(v) | sign);
    }
    if (e == 31) return bits_f32(sign | 0x7f800000u | (mant << 13));
    return bits_f32(sign | ((e + 112) << 23) | (mant << 13));
}

inline uint16_t f32_to_f16(float f) {
    uint32_t x = f32_bits(f);
    const uint32_t sign = (x >> 16) & 0x8000u;
    x &= 0x7fffffffu;
    if (x >= 0x7f800000u) return (uint16_t)(sign | (x > 0x7f800000u ? 0x7e00u : 0x7c00u));
    if (x >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // >= 65520 rounds to infinity
    if (x < 0x38800000u) {  // below 2^-14: a multiple of 2^-24, rounded to nearest even
        const float a = bits_f32(x) * 16777216.0f;  // exact: a power-of-two scale
        return (uint16_t)(sign | (uint32_t)nearbyintf(a));
    }
    uint32_t h = ((((x >> 23) - 112) << 10) | ((x >> 13) & 0x3ffu));
    const uint32_t rem = x & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
}

inline float bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

inline uint16_t f32_to_bf16(float f) {
    const uint32_t x = f32_bits(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);  // quiet NaN
    return (uint16_t)((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
}

struct Span {
    AdamK k;
    int dtype;     // ZI_F16 / ZI_BF16: format of w (and of grad unless grad_f32)
    int grad_f32;
    const void *grad;
    float *master, *m, *v;
    void *w;
};

inline void adam_one(const AdamK &k, float g, float &master, float &m, float &v) {
    m = k.b1 * m + k.omb1 * g;
    v = k.b2 * v + k.omb2 * (g * g);
    const float den = sqrtf(v * k.c2) + k.eps;
    master = master - (k.step_size * m) / den;
}

void span_scalar(const Span &s, int64_t b, int64_t e) {
    for (int64_t i = b; i < e; ++i) {
        float g;
        if (s.grad_f32)
            g = static_cast<const float *>(s.grad)[i];
        else if (s.dtype == ZI_F16)
            g = f16_to_f32(static_cast<const uint16_t *>(s.grad)[i]);
        else
            g = bf16_to_f32(static_cast<const uint16_t *>(s.grad)[i]);
        adam_one(s.k, g, s.master[i], s.m[i], s.v[i]);
        static_cast<uint16_t *>(s.w)[i] =
            s.dtype == ZI_F16 ? f32_to_f16(s.master[i]) : f32_to_bf16(s.master[i]);
    }
}

// Eight elements per iteration with AVX2 and F16C; the same operations in the
// same order as adam_one, each IEEE-rounded, so the results equal the scalar
// code's.  bf16 outputs are rounded by the scalar helper.
__attribute__((target("avx2,f16c"))) void span_avx2(const Span &s, int64_t b, int64_t e) {
    const __m256 B1 = _mm256_set1_ps(s.k.b1), OMB1 = _mm256_set1_ps(s.k.omb1);
    const __m256 B2 = _mm256_set1_ps(s.k.b2), OMB2 = _mm256_set1_ps(s.k.omb2);
    const __m256 SS = _mm256_set1_ps(s.k.step_size), C2 = _mm256_set1_ps(s.k.c2);
    const __m256 EPS = _mm256_set1_ps(s.k.eps);
    int64_t i = b;
    for (; i + 8 <= e; i += 8) {
        __m256 g;
        if (s.grad_f32) {
            g = _mm256_loadu_ps(static_cast<const float *>(s.grad) + i);
        } else if (s.dtype == ZI_F16) {
            g = _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i *>(
                static_cast<const uint16_t *>(s.grad) + i)));
        } else {
            const __m128i h = _mm_loadu_si128(reinterpret_cast<const __m128i *>(
                static_cast<const uint16_t *>(s.grad) + i));
            g = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
        }
        __m256 m = _mm256_loadu_ps(s.m + i), v = _mm256_loadu_ps(s.v + i);
        __m256 w = _mm256_loadu_ps(s.master + i);
        m = _mm256_add_ps(_mm256_mul_ps(B1, m), _mm256_mul_ps(OMB1, g));
        v = _mm256_add_ps(_mm256_mul_ps(B2, v), _mm256_mul_ps(OMB2, _mm256_mul_ps(g, g)));
        const __m256 den = _mm256_add_ps(_mm256_sqrt_ps(_mm256_mul_ps(v, C2)), EPS);
        w = _mm256_sub_ps(w, _mm256_div_ps(_mm256_mul_ps(SS, m), den));
        _mm256_storeu_ps(s.m + i, m);
        _mm256_storeu_ps(s.v + i, v);
        _mm256_storeu_ps(s.master + i, w);
        uint16_t *wo = static_cast<uint16_t *>(s.w) + i;
        if (s.dtype == ZI_F16) {
            _mm_storeu_si128(reinterpret_cast<__m128i *>(wo), _mm256_cvtps_ph(w, _MM_FROUND_TO_NEAREST_INT));
        } else {
            for (int j = 0; j < 8; ++j) wo[j] = f32_to_bf16(s.master[i + j]);
        }
    }
    span_scalar(s, i, e);
}

bool vector_ok() {
    static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
    return ok;
}

void run_span(const Span &s, int64_t b, int64_t e) {
    if (vector_ok())
        span_avx2(s, b, e);
    else
        span_scalar(s, b, e);
}

int default_threads() {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        const int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    const unsigned h = std::thread::hardware_concurrency();
    return h ? (int)h : 1;
}

// Split [0, count) into `threads` contiguous chunks of whole 64-element
// blocks and run them concurrently (the calling thread takes the first).
void parallel_update(const Span &s, int64_t count, int threads) {
    const int64_t blocks = (count + 63) / 64;
    const int t = (int)std::max<int64_t>(1, std::min<int64_t>(threads, blocks));
    if (t == 1) {
        run_span(s, 0, count);
        return;
    }
    std::vector<std::thread> pool;
    pool.reserve(t - 1);
    auto range = [&](int j, int64_t &b, int64_t &e) {
        b = std::min<int64_t>(count, blocks * j / t * 64);
        e = std::min<int64_t>(count, blocks * (j + 1) / t * 64);
    };
    for (int j = 1; j < t; ++j) {
        int64_t b, e;
        range(j, b, e);
        pool.emplace_back([&s, b, e] { run_span(s, b, e); });
    }
    int64_t b, e;
    range(0, b, e);
    run_span(s, b, e);
    for (auto &th : pool) th.join();
}

zi_status check_hparams(const zi_adam_hparams *hp) {
    if (!hp) return fail(ZI_ERR_ARG, "hyperparameters are NULL");
    if (!(hp->lr >= 0.0f) || !std::isfinite(hp->lr)) return fail(ZI_ERR_ARG, "lr must be finite and >= 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f)) return fail(ZI_ERR_ARG, "beta1 must be in [0, 1)");
    if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) return fail(ZI_ERR_ARG, "beta2 must be in [0, 1)");
    if (!(hp->eps >= 0.0f) || !std::isfinite(hp->eps)) return fail(ZI_ERR_ARG, "eps must be finite and >= 0");
    return ZI_OK;
}

}  // namespace
}  // namespace zi

using namespace zi;

struct zi_adam {
    const zi_plan *plan = nullptr;
    zi_adam_hparams hp{};
    float *master = nullptr, *m = nullptr, *v = nullptr;
    int threads = 1;
    int device = 0;
    int dtype = ZI_F16;
    int grad_f32 = 0;
    int64_t N = 0, tile_elems = 0;
    // Guarded by the engine's mutex.
    std::vector<int64_t> queued, done;  // per tile: updates queued / completed (= its step count)
    int64_t pending = 0;                // updates queued and not yet completed
    zi_status err = ZI_OK;
    std::string err_msg;
    int64_t tiles_done = 0;
    double busy_s = 0, bytes = 0;
};

namespace zi {
namespace {

// Persistent fork-join pool: run() splits one span over the caller and up to
// `workers` pool threads, in contiguous chunks of whole 64-element blocks.
// Used by one thread at a time (the engine's coordinator).
class Pool {
  public:
    void ensure(int workers) {
        while ((int)threads_.size() < workers) {
            const int j = (int)threads_.size() + 1;
            uint64_t now;
            {
                std::lock_guard<std::mutex> lock(mu_);
                now = gen_;  // a new worker waits for the next span, not the last one
            }
            threads_.emplace_back([this, j, now] { work(j, now); });
        }
    }

    void run(const Span &s, int64_t count, int parts) {
        const int64_t blocks = (count + 63) / 64;
        parts = (int)std::max<int64_t>(1, std::min<int64_t>({(int64_t)parts, blocks,
                                                             (int64_t)threads_.size() + 1}));
        if (parts == 1) {
            run_span(s, 0, count);
            return;
        }
        {
            std::lock_guard<std::mutex> lock(mu_);
            span_ = &s;
            count_ = count;
            blocks_ = blocks;
            parts_ = parts;
            pending_ = parts - 1;
            ++gen_;
        }
        go_.notify_all();
        int64_t b, e;
        range(0, b, e);
        run_span(s, b, e);
        std::unique_lock<std::mutex> lock(mu_);
        fin_.wait(lock, [&] { return pending_ == 0; });
    }

    void shutdown() {
        {
            std::lock_guard<std::mutex> lock(mu_);
            quit_ = true;
        }
        go_.notify_all();
        for (auto &t : threads_) t.join();
        threads_.clear();
        std::lock_guard<std::mutex> lock(mu_);
        quit_ = false;
    }

  private:
    void range(int j, int64_t &b, int64_t &e) const {
        b = std::min<int64_t>(count_, blocks_ * j / parts_ * 64);
        e = std::min<int64_t>(count_, blocks_ * (j + 1) / parts_ * 64);
    }

    void work(int j, uint64_t seen) {
        for (;;) {
            int64_t b = 0, e = 0;
            const Span *s = nullptr;
            {
                std::unique_lock<std::mutex> lock(mu_);
                go_.wait(lock, [&] { return quit_ || gen_ != seen; });
                if (quit_) return;
                seen = gen_;
                if (j >= parts_) continue;  // not needed for this span
                s = span_;
                range(j, b, e);
            }
            run_span(*s, b, e);
            {
                std::lock_guard<std::mutex> lock(mu_);
                --pending_;
            }
            fin_.notify_one();
        }
    }

    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable go_, fin_;
    uint64_t gen_ = 0;
    bool quit_ = false;
    const Span *span_ = nullptr;
    int64_t count_ = 0, blocks_ = 0;
    int parts_ = 1, pending_ = 0;
};

// One engine per process.  Its coordinator thread takes the queued tile
// updates of every optimizer in the order they were queued (the order the
// gradients were written back, which is also the order the next passes need
// the tiles in), waits for each tile's gradient to land, and splits the
// update over the pool, so the host's cores work on one tile at a time.
struct Engine {
    struct Task {
        zi_adam *a;
        int64_t tile;
        hipEvent_t landed;
    };
    std::mutex life;  // serialises starting and stopping the coordinator
    std::mutex mu;    // guards the queue and every optimizer's counters
    std::condition_variable cv;
    std::deque<Task> queue;
    std::thread coordinator;
    int users = 0;
    bool stop = false;
    Pool pool;

    void run() {
        int cur_dev = -1;
        for (;;) {
            Task t;
            {
                std::unique_lock<std::mutex> lock(mu);
                cv.wait(lock, [&] { return stop || !queue.empty(); });
                if (queue.empty()) break;
                t = queue.front();
                queue.pop_front();
            }
            zi_adam *a = t.a;
            if (a->device != cur_dev && hipSetDevice(a->device) == hipSuccess) cur_dev = a->device;
            const hipError_t e = hipEventSynchronize(t.landed);
            (void)hipEventDestroy(t.landed);
            const auto t0 = std::chrono::steady_clock::now();
            const int64_t step = a->done[t.tile] + 1;  // only this thread writes done[]
            if (e == hipSuccess) {
                const int64_t off = t.tile * a->tile_elems;
                Span s;
                s.k = adam_consts(a->hp, step);
                s.dtype = a->dtype;
                s.grad_f32 = a->grad_f32;
                s.grad = static_cast<const char *>(a->plan->prob.dW_host) + off * (a->grad_f32 ? 4 : 2);
                s.master = a->master + off;
                s.m = a->m + off;
                s.v = a->v + off;
                s.w = static_cast<char *>(const_cast<void *>(a->plan->prob.W_host)) + off * 2;
                pool.ensure(a->threads - 1);
                pool.run(s, a->tile_elems, a->threads);
            }
            const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
            {
                std::lock_guard<std::mutex> lock(mu);
                if (e != hipSuccess && a->err == ZI_OK) {
                    a->err = ZI_ERR_HIP;
                    a->err_msg = std::string("waiting for a gradient tile: ") + hipGetErrorString(e);
                }
                a->done[t.tile] = step;  // also on failure, so that no waiter hangs
                --a->pending;
                if (e == hipSuccess) {
                    ++a->tiles_done;
                    a->busy_s += secs;
                    a->bytes += (double)a->tile_elems * (a->grad_f32 ? 30.0 : 28.0);
                }
            }
            cv.notify_all();
        }
        pool.shutdown();
    }

    // Register an optimizer; the first one starts the coordinator.
    bool join_user() {
        std::lock_guard<std::mutex> l(life);
        {
            std::lock_guard<std::mutex> lock(mu);
            if (users++ > 0) return true;
            stop = false;
        }
        try {
            coordinator = std::thread([this] { run(); });
        } catch (...) {
            std::lock_guard<std::mutex> lock(mu);
            --users;
            return false;
        }
        return true;
    }

    // Unregister an optimizer whose updates are all done; the last one stops
    // the coordinator and the pool.
    void leave_user() {
        std::lock_guard<std::mutex> l(life);
        bool last;
        {
            std::lock_guard<std::mutex> lock(mu);
            last = --users == 0;
            if (last) stop = true;
        }
        if (!last) return;
        cv.notify_all();
        coordinator.join();
    }
};

// Never destroyed: the coordinator is joined when the last optimizer goes,
// and an optimizer never released leaves a thread blocked on the queue,
// which process exit ends.
Engine &engine() {
    static Engine *e = new Engine;
    return *e;
}

}  // namespace

// Hooks for the context (zi_api.cpp).
const zi_plan *adam_plan(const zi_adam *a) { return a->plan; }

void adam_enqueue(zi_adam *a, int64_t tile, void *landed_event) {
    Engine &g = engine();
    {
        std::lock_guard<std::mutex> lock(g.mu);
        ++a->queued[tile];
        ++a->pending;
        g.queue.push_back(Engine::Task{a, tile, static_cast<hipEvent_t>(landed_event)});
    }
    g.cv.notify_all();
}

void adam_wait_tile(zi_adam *a, int64_t tile) {
    Engine &g = engine();
    std::unique_lock<std::mutex> lock(g.mu);
    g.cv.wait(lock, [&] { return a->done[tile] >= a->queued[tile]; });
}

zi_status adam_wait_all(zi_adam *a) {
    Engine &g = engine();
    std::unique_lock<std::mutex> lock(g.mu);
    g.cv.wait(lock, [&] { return a->pending == 0; });
    if (a->err != ZI_OK) return fail(a->err, "%s", a->err_msg.c_str());
    return ZI_OK;
}

}  // namespace zi

extern "C" {

zi_status zi_adam_update(const zi_adam_hparams *hp, int32_t dtype, int32_t grad_f32, int64_t step,
                         int64_t count, const void *grad, float *master, float *m, float *v, void *w,
                         int32_t threads) {
    clear_error();
    zi_status st = check_hparams(hp);
    if (st != ZI_OK) return st;
    if (dtype != ZI_F16 && dtype != ZI_BF16) return fail(ZI_ERR_ARG, "bad dtype %d", dtype);
    if (grad_f32 != 0 && grad_f32 != 1) return fail(ZI_ERR_ARG, "grad_f32 must be 0 or 1");
    if (step < 1) return fail(ZI_ERR_ARG, "step counts from 1 (got %lld)", (long long)step);
    if (count < 0) return fail(ZI_ERR_ARG, "count < 0");
    if (count == 0) return ZI_OK;
    if (!grad || !master || !m || !v || !w) return fail(ZI_ERR_ARG, "NULL array");
    Span s;
    s.k = adam_consts(*hp, step);
    s.dtype = dtype;
    s.grad_f32 = grad_f32;
    s.grad = grad;
    s.master = master;
    s.m = m;
    s.v = v;
    s.w = w;
    parallel_update(s, count, threads > 0 ? threads : default_threads());
    return ZI_OK;
}

zi_status zi_adam_create(const zi_plan *plan, const zi_adam_hparams *hp, float *master, float *m, float *v,
                         int32_t threads, zi_adam **out) {
    clear_error();
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!plan) return fail(ZI_ERR_ARG, "plan is NULL");
    zi_status st = check_hparams(hp);
    if (st != ZI_OK) return st;
    if (!master || !m || !v) return fail(ZI_ERR_ARG, "master, m and v are required");
    if (!plan->prob.W_host || !plan->prob.dW_host)
        return fail(ZI_ERR_STATE, "the plan needs W_host and dW_host for an optimizer");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(ZI_ERR_HIP, "hipGetDevice failed");
    zi_adam *a = new (std::nothrow) zi_adam;
    if (!a) return fail(ZI_ERR_ARG, "out of host memory");
    a->plan = plan;
    a->hp = *hp;
    a->master = master;
    a->m = m;
    a->v = v;
    a->threads = threads > 0 ? threads : default_threads();
    a->device = dev;
    a->dtype = plan->prob.dtype;
    a->grad_f32 = (plan->prob.flags & ZI_FLAG_F32_OUT) ? 1 : 0;
    a->N = plan->prob.N;
    a->tile_elems = plan->info.n * plan->prob.K;
    a->queued.assign(a->N, 0);
    a->done.assign(a->N, 0);
    if (!engine().join_user()) {
        delete a;
        return fail(ZI_ERR_ARG, "could not start the optimizer thread");
    }
    *out = a;
    return ZI_OK;
}

zi_status zi_adam_destroy(zi_adam *a) {
    clear_error();
    if (!a) return ZI_OK;
    zi_status st = adam_wait_all(a);
    engine().leave_user();
    delete a;
    return st;
}

zi_status zi_adam_wait(zi_adam *a) {
    clear_error();
    if (!a) return fail(ZI_ERR_ARG, "optimizer is NULL");
    return adam_wait_all(a);
}

zi_status zi_adam_stats_get(zi_adam *a, zi_adam_stats *out) {
    clear_error();
    if (!a || !out) return fail(ZI_ERR_ARG, "optimizer and out are required");
    std::lock_guard<std::mutex> lock(engine().mu);
    out->tiles_done = a->tiles_done;
    out->busy_s = a->busy_s;
    out->bytes = a->bytes;
    return ZI_OK;
}

}  // extern "C"
