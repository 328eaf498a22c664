// Stress test of the host optimizer's engine, on the CPU: zi_adam.cpp is
// compiled with host stand-ins for the HIP calls it makes (every gradient
// copy event is already complete).  Two optimizers take tile updates in the
// order the backward passes queue them, for several steps, and are destroyed
// and made again between rounds (the engine's coordinator and worker pool
// stop with the last optimizer and start with the next one).  Every weight,
// master and moment must equal what one zi_adam_update per tile and step
// gives on the same gradients.
#include "../../offload_memory_centric_amd/csrc/zi_adam.cpp"
#include <stdarg.h>
#include <random>
extern "C" {
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "stub"; }
}
namespace zi {
zi_status fail(zi_status st, const char *fmt, ...) { va_list a; va_start(a, fmt); vfprintf(stderr, fmt, a); va_end(a); fprintf(stderr, "\n"); return st; }
void clear_error() {}
}

struct Weight {
    zi_plan plan{};
    std::vector<uint16_t> w, g;
    std::vector<float> master, m, v;
    std::vector<uint16_t> w_ref;
    std::vector<float> master_ref, m_ref, v_ref;
};

static void init(Weight &x, int K, int n, int N, uint32_t seed) {
    x.plan.prob.K = K; x.plan.prob.M = (int64_t)n * N; x.plan.prob.N = N; x.plan.prob.T = 8;
    x.plan.prob.d = 2; x.plan.prob.dtype = ZI_BF16;
    x.plan.info.n = n;
    const size_t count = (size_t)K * n * N;
    std::mt19937 r(seed);
    std::normal_distribution<float> nd(0.f, 0.02f);
    x.master.resize(count); x.m.assign(count, 0.f); x.v.assign(count, 0.f);
    x.w.resize(count); x.g.resize(count);
    for (size_t i = 0; i < count; ++i) x.master[i] = nd(r);
    x.master_ref = x.master; x.m_ref = x.m; x.v_ref = x.v;
    x.w_ref.resize(count);
    x.plan.prob.W_host = x.w.data();
    x.plan.prob.dW_host = x.g.data();
}

static void fill_grad(Weight &x, int64_t tile, int step, uint32_t salt) {
    const size_t te = (size_t)x.plan.prob.K * x.plan.info.n;
    std::mt19937 r(salt * 7919u + (uint32_t)step * 131u + (uint32_t)tile);
    std::normal_distribution<float> nd(0.f, 1e-2f);
    for (size_t i = 0; i < te; ++i) {
        const float f = nd(r);
        uint32_t b; memcpy(&b, &f, 4);
        x.g[tile * te + i] = (uint16_t)(b >> 16);  // truncation is fine: any bf16 gradient will do
    }
}

int main() {
    const zi_adam_hparams hp{1e-3f, 0.9f, 0.999f, 1e-8f};
    int bad = 0;
    std::mt19937 rng(3);
    for (int round = 0; round < 4; ++round) {
        Weight a, b;
        init(a, 64, 96, 5, 10 + round);
        init(b, 128, 64, 3, 20 + round);
        zi_adam *oa = nullptr, *ob = nullptr;
        if (zi_adam_create(&a.plan, &hp, a.master.data(), a.m.data(), a.v.data(), 1 + round, &oa) != ZI_OK) return 3;
        if (zi_adam_create(&b.plan, &hp, b.master.data(), b.m.data(), b.v.data(), 3, &ob) != ZI_OK) return 3;
        const int steps = 6;
        for (int s = 1; s <= steps; ++s) {
            // backward of b, then of a: each tile's gradient lands, its update is queued;
            // a gradient buffer is rewritten only after the tile's previous update (as stage() waits)
            for (Weight *x : {&b, &a}) {
                zi_adam *o = x == &a ? oa : ob;
                const uint32_t salt = x == &a ? 1u : 2u;
                for (int64_t t = 0; t < x->plan.prob.N; ++t) {
                    adam_wait_tile(o, t);
                    fill_grad(*x, t, s, salt);
                    const size_t te = (size_t)x->plan.prob.K * x->plan.info.n, off = t * te;
                    zi_adam_update(&hp, ZI_BF16, 0, s, (int64_t)te, &x->g[off], &x->master_ref[off], &x->m_ref[off],
                                   &x->v_ref[off], &x->w_ref[off], 1);
                    adam_enqueue(o, t, nullptr);
                    if (rng() % 7 == 0) std::this_thread::yield();
                }
            }
        }
        if (adam_wait_all(oa) != ZI_OK || adam_wait_all(ob) != ZI_OK) ++bad;
        for (Weight *x : {&a, &b}) {
            if (memcmp(x->w.data(), x->w_ref.data(), x->w.size() * 2) ||
                memcmp(x->master.data(), x->master_ref.data(), x->master.size() * 4) ||
                memcmp(x->m.data(), x->m_ref.data(), x->m.size() * 4) || memcmp(x->v.data(), x->v_ref.data(), x->v.size() * 4))
                ++bad;
        }
        zi_adam_stats st;
        zi_adam_stats_get(oa, &st);
        if (st.tiles_done != steps * a.plan.prob.N) ++bad;
        zi_adam_destroy(oa);
        zi_adam_destroy(ob);
    }
    printf("bad %d\n", bad);
    return bad != 0;
}
