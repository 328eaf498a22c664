// Stress test of the file tier's read-ahead and cache, on the CPU:
// zi_source.cpp is compiled with host stand-ins for the HIP calls it makes
// (aligned malloc for page-locked memory, events that are always complete).
// A consumer stages tiles as the passes do, in order and out of order,
// restarting the read-ahead and abandoning requests at random, and checks
// every staged buffer against the file's bytes; with as many buffers as
// tiles, every tile must be read exactly once.  Usage: tier_stress DIR
#include "../../offload_memory_centric_amd/csrc/zi_source.cpp"
#include <unistd.h>

#include <chrono>
#include <random>
#include <thread>
#include <stdarg.h>
extern "C" {
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipHostMalloc(void **p, size_t n, unsigned int) { return posix_memalign(p, 4096, n) ? hipErrorOutOfMemory : hipSuccess; }
hipError_t hipHostFree(void *p) { free(p); return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned) { *e = (hipEvent_t)malloc(8); return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) { free(e); return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
const char *hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetLastError() { return hipSuccess; }
}
namespace zi {
zi_status fail(zi_status st, const char *fmt, ...) { va_list a; va_start(a, fmt); vfprintf(stderr, fmt, a); va_end(a); fprintf(stderr, "\n"); return st; }
void clear_error() {}
}
static std::vector<uint8_t> make_file(const char *path, size_t n, int seed) {
    std::vector<uint8_t> d(n);
    std::mt19937 r(seed);
    for (auto &x : d) x = (uint8_t)r();
    FILE *f = fopen(path, "wb"); fwrite(d.data(), 1, n, f); fclose(f);
    return d;
}
int main(int argc, char **argv) {
    if (argc < 2) return 2;
    const int K = 256, n = 512, N = 4;  // tile = 256 KiB
    zi_plan plan{};
    plan.prob.K = K; plan.prob.M = n * N; plan.prob.N = N; plan.prob.T = 8; plan.prob.d = 2; plan.prob.dtype = ZI_F16;
    plan.info.n = n; plan.info.tile_bytes = (uint64_t)K * n * 2;
    const size_t tb = plan.info.tile_bytes;
    std::vector<std::vector<uint8_t>> data;
    std::string names[3];
    const char *paths[3];
    for (int i = 0; i < 3; ++i) {
        names[i] = std::string(argv[1]) + "/w" + std::to_string(i) + ".bin";
        paths[i] = names[i].c_str();
        data.push_back(make_file(paths[i], tb * N, i + 1));
    }
    int bad = 0, served = 0;
    std::mt19937 rng(7);
    auto serve = [&](zi_file_source *s, int which, int64_t tile, bool maybe_abandon) {
        const void *host = nullptr; int slot = -1;
        if (source_acquire(s, tile, &host, &slot) != ZI_OK) { ++bad; return; }
        if (memcmp(host, data[which].data() + tile * tb, tb) != 0) ++bad;
        ++served;
        if (maybe_abandon && rng() % 50 == 0) { source_abandon(s, slot); return; }
        source_release(s, slot);
    };
    // 1. a standalone source, passes in order
    {
        zi_file_source *s = nullptr;
        zi_file_source_create(&plan, paths[0], 0, 3, 3, &s);
        for (int pass = 0; pass < 40; ++pass)
            for (int t = 0; t < N; ++t) serve(s, 0, t, true);
        zi_source_stats st; zi_file_source_stats_get(s, &st);
        printf("standalone: restarts %lld tiles_read %lld\n", (long long)st.restarts, (long long)st.tiles_read);
        zi_file_source_destroy(s);
    }
    // 1b. as many buffers as tiles: every tile is read once, then served from memory
    {
        zi_file_source *s = nullptr;
        zi_file_source_create(&plan, paths[1], 0, N, 2, &s);
        for (int pass = 0; pass < 30; ++pass)
            for (int t = 0; t < N; ++t) serve(s, 1, t, false);
        zi_source_stats st; zi_file_source_stats_get(s, &st);
        printf("cached: tiles_read %lld\n", (long long)st.tiles_read);
        if (st.tiles_read != N) ++bad;
        zi_file_source_destroy(s);
    }
    // 2. a shared tier over three sources: a recorded step, then replays with perturbations
    {
        zi_tier *tier = nullptr; zi_tier_create(4, 3, &tier);
        zi_file_source *s[3];
        for (int i = 0; i < 3; ++i) { zi_file_source_create(&plan, paths[i], 0, 2, 2, &s[i]); zi_tier_add(tier, s[i]); }
        auto step = [&](int kind) {
            if (kind == 1) { for (int t = 0; t < N; ++t) serve(s[1], 1, t, true); return; }  // unknown order
            if (kind == 2) { for (int t = 0; t < N; ++t) serve(s[0], 0, t, true); return; }  // truncated
            for (int t = 0; t < N; ++t) serve(s[0], 0, t, true);
            for (int t = 0; t < N; ++t) serve(s[1], 1, t, true);
            for (int t = 0; t < N; ++t) serve(s[0], 0, t, true);
            for (int t = 0; t < 2; ++t) serve(s[2], 2, t, true);
        };
        step(0);
        zi_tier_step(tier);
        for (int k = 0; k < 80; ++k) {
            const unsigned r = rng() % 20;
            step(r == 0 ? 1 : r == 1 ? 2 : 0);
            if (rng() % 10) zi_tier_step(tier);
        }
        zi_tier_stats ts; zi_tier_stats_get(tier, &ts);
        printf("tier: trace %lld steps %lld read %lld restarts %lld demand %lld\n", (long long)ts.trace_len,
               (long long)ts.steps, (long long)ts.tiles_read, (long long)ts.restarts, (long long)ts.demand_reads);
        zi_tier_destroy(tier);
        for (int i = 0; i < 3; ++i) zi_file_source_destroy(s[i]);
    }
    // 3. few buffers and requests off the trace: an on-demand read must not be
    //    evicted by the read-ahead before its request takes it
    {
        zi_tier *tier = nullptr; zi_tier_create(2, 2, &tier);
        zi_file_source *s[3];
        for (int i = 0; i < 3; ++i) { zi_file_source_create(&plan, paths[i], 0, 2, 2, &s[i]); zi_tier_add(tier, s[i]); }
        for (int t = 0; t < N; ++t) serve(s[0], 0, t, false);
        for (int t = 0; t < N; ++t) serve(s[1], 1, t, false);
        zi_tier_step(tier);
        for (int k = 0; k < 300; ++k) {
            const int t = (int)(rng() % N);
            if (rng() % 3 == 0) serve(s[2], 2, t, false);  // never in the trace
            serve(s[k % 2], k % 2, (k / 2) % N, false);
        }
        zi_tier_stats ts; zi_tier_stats_get(tier, &ts);
        printf("off-trace: demand %lld restarts %lld\n", (long long)ts.demand_reads, (long long)ts.restarts);
        zi_tier_destroy(tier);
        for (int i = 0; i < 3; ++i) zi_file_source_destroy(s[i]);
    }
    // 4. the cache against the offline optimum: a block-like step (source 0's
    //    tiles three times, source 1's twice) under C buffers reads no fewer
    //    tiles per step than Belady's eviction with C slots (no policy can),
    //    and with a buffer per distinct tile nothing after the first step
    for (int C : {2, 3, 5, 8}) {
        zi_tier *tier = nullptr; zi_tier_create(C, 2, &tier);
        zi_file_source *s[2];
        for (int i = 0; i < 2; ++i) { zi_file_source_create(&plan, paths[i], 0, 2, 2, &s[i]); zi_tier_add(tier, s[i]); }
        std::vector<std::pair<int, int>> step;
        for (int pass : {0, 1, 0, 1, 0})
            for (int t = 0; t < N; ++t) step.push_back({pass, t});
        auto run_step = [&] { for (auto &r : step) serve(s[r.first], r.first, r.second, false); };
        run_step();
        zi_tier_step(tier);
        const int steps = 6;
        zi_tier_stats a; zi_tier_stats_get(tier, &a);
        for (int k = 0; k < steps; ++k) { run_step(); zi_tier_step(tier); }
        zi_tier_stats b; zi_tier_stats_get(tier, &b);
        // Belady with C slots over the same steps (steady state: after a first step)
        std::vector<std::pair<int, int>> seq;
        for (int k = 0; k < steps + 2; ++k) seq.insert(seq.end(), step.begin(), step.end());
        std::vector<std::pair<int, int>> cache;
        long misses = 0;
        for (size_t i = 0; i < seq.size(); ++i) {
            bool hit = false;
            for (auto &c : cache) hit = hit || c == seq[i];
            if (hit) continue;
            if (i >= step.size() && i < step.size() * (steps + 1)) ++misses;
            if ((int)cache.size() == C) {
                size_t far = 0, vi = 0;
                for (size_t c = 0; c < cache.size(); ++c) {
                    size_t j = i + 1;
                    while (j < seq.size() && !(seq[j] == cache[c])) ++j;
                    if (j >= far) { far = j; vi = c; }
                }
                cache.erase(cache.begin() + vi);
            }
            cache.push_back(seq[i]);
        }
        const long got = (long)(b.tiles_read - a.tiles_read);
        printf("cache C=%d: reads %ld over %d steps, Belady %ld\n", C, got, steps, misses);
        if (got < misses || got > (long)(steps * step.size() + C)) ++bad;
        if (C >= 2 * N && got != 0) ++bad;
        zi_tier_destroy(tier);
        for (int i = 0; i < 2; ++i) zi_file_source_destroy(s[i]);
    }
    // 5. an off-trace request after the read-ahead has taken every buffer for
    //    upcoming trace positions: the reader must give one of them back for
    //    the read on demand (a hang here is caught by the alarm)
    for (int round = 0; round < 3; ++round) {
        alarm(60);
        zi_tier *tier = nullptr; zi_tier_create(2, 2, &tier);
        zi_file_source *s[2];
        for (int i = 0; i < 2; ++i) { zi_file_source_create(&plan, paths[i], 0, 2, 2, &s[i]); zi_tier_add(tier, s[i]); }
        for (int t = 0; t < N; ++t) serve(s[0], 0, t, false);
        zi_tier_step(tier);
        serve(s[0], 0, 0, false);
        std::this_thread::sleep_for(std::chrono::milliseconds(200));  // both buffers now hold trace tiles 1, 2
        serve(s[1], 1, round % N, false);                             // never in the trace
        for (int t = 1; t < N; ++t) serve(s[0], 0, t, false);         // the trace goes on
        serve(s[0], 0, 0, false);
        zi_tier_stats ts; zi_tier_stats_get(tier, &ts);
        printf("read-ahead given back: demand %lld restarts %lld\n", (long long)ts.demand_reads, (long long)ts.restarts);
        if (ts.demand_reads < 1) ++bad;
        zi_tier_destroy(tier);
        for (int i = 0; i < 2; ++i) zi_file_source_destroy(s[i]);
        alarm(0);
    }
    for (auto p : paths) remove(p);
    printf("served %d bad %d\n", served, bad);
    return bad != 0;
}
