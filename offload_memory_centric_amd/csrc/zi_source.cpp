// zi_source.cpp -- the NVMe tier in front of the host tier: weight tiles read
// from a file on local storage into pinned staging buffers, from which the
// ring's host-to-device copies take them.
//
// The pages place parameters on NVMe and bring each one up the hierarchy
// (NVMe -> CPU memory -> GPU) shortly before it is needed, with the NVMe
// reads running ahead of the CPU -> GPU copies so that both tiers overlap the
// products (pwwt.cn ZeRO-Infinity article, section "关键技术三：Overlap-Centric
// Design": the reads of later parameters, the copies of nearer ones and the
// compute of the current one run at the same time; transformer-math page,
// section "Applying the test: which state can live where", for the bandwidth
// bar the NVMe tier must clear).  Here a reader thread per source reads tiles
// in the order the passes will want them (every pass walks its tiles in
// ascending order, so after tile i comes i + 1, and after the last tile the
// first one of the next pass), into a ring of S pinned staging buffers, each
// read split over several threads issuing positioned reads.  A staging buffer
// is reused once the host-to-device copy that reads it has completed.  When a
// pass asks for a tile other than the one read ahead, the read-ahead restarts
// at that tile.
#include <errno.h>
#include <stdlib.h>
#include <fcntl.h>
#include <hip/hip_runtime_api.h>
#include <string.h>
#include <sys/stat.h>
#include <unistd.h>

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

namespace zi {
namespace {

constexpr uint64_t kDirectAlign = 4096;  // O_DIRECT offset, size and buffer alignment
constexpr uint64_t kChunk = 16ull << 20;  // bytes per positioned read

// Read [off, off + bytes) of fd into dst on `threads` threads, in kChunk
// pieces dealt round-robin (piece p to thread p mod threads), so the threads
// read neighbouring parts of the file at any moment.  With `bounce` (one
// aligned kChunk buffer per thread), each thread reads into its buffer and
// copies the piece to dst: O_DIRECT reads cannot target page-locked memory
// from hipHostMalloc (the kernel cannot pin those pages again and fails the
// read with EFAULT).  The bounce buffers are kept and touched in advance:
// allocating them per read made every read fault them in again, which halved
// the read rate.  Returns 0 or an errno (EIO for a short file).
int parallel_pread(int fd, char *dst, uint64_t off, uint64_t bytes, int threads, char *const *bounce) {
    const uint64_t pieces = (bytes + kChunk - 1) / kChunk;
    const int t = (int)std::max<uint64_t>(1, std::min<uint64_t>((uint64_t)threads, pieces));
    std::vector<int> errs(t, 0);
    auto work = [&](int j) {
        for (uint64_t p = (uint64_t)j; p < pieces && !errs[j]; p += (uint64_t)t) {
            const uint64_t at = p * kChunk;
            const size_t want = (size_t)std::min<uint64_t>(kChunk, bytes - at);
            char *to = bounce ? bounce[j] : dst + at;
            size_t have = 0;
            while (have < want) {  // a direct read returns whole pieces; a buffered one may not
                const ssize_t got = pread(fd, to + have, want - have, (off_t)(off + at + have));
                if (got < 0) {
                    if (errno == EINTR) continue;
                    errs[j] = errno;
                    break;
                }
                if (got == 0) {
                    errs[j] = EIO;  // the file ends before the tile does
                    break;
                }
                have += (size_t)got;
            }
            if (!errs[j] && bounce) memcpy(dst + at, to, want);
        }
    };
    std::vector<std::thread> pool;
    pool.reserve(t - 1);
    for (int j = 1; j < t; ++j) pool.emplace_back(work, j);
    work(0);
    for (auto &th : pool) th.join();
    for (int e : errs)
        if (e) return e;
    return 0;
}

// `count` aligned kChunk buffers, touched so that their pages exist.
std::vector<char *> bounce_buffers(int count) {
    std::vector<char *> out;
    for (int j = 0; j < count; ++j) {
        void *p = nullptr;
        if (posix_memalign(&p, kDirectAlign, kChunk) != 0) break;
        memset(p, 0, kChunk);
        out.push_back(static_cast<char *>(p));
    }
    return out;
}

void free_buffers(std::vector<char *> &v) {
    for (char *p : v) free(p);
    v.clear();
}

}  // namespace
}  // namespace zi

using namespace zi;

struct zi_file_source {
    const zi_plan *plan = nullptr;
    int fd = -1;
    bool direct = false;
    uint64_t offset = 0, tile_bytes = 0;
    int64_t N = 0;
    int S = 2, threads = 4;
    zi_tier *tier = nullptr;  // the tier that reads this source's tiles
    bool own_tier = false;    // a private tier made on first use, its trace the tiles in order
    // statistics, under the tier's mutex
    int64_t tiles_read = 0;
    double read_s = 0, bytes = 0, wait_s = 0;
};

// A tier of file sources: S pinned tile buffers and one reader thread that
// reads the sources' tiles ahead of the passes, in the order of a trace.  A
// shared tier records the order of the requests during the first step (the
// requests are then served on demand) and replays it in every later step; a
// standalone source gets a private tier whose trace is its tiles in order.
//
// The buffers are also a cache of the file in host memory: a tile still held
// by a buffer is served again without a read.  When the reader needs a buffer
// for a read, it takes one that no pending request is waiting for, preferring
// one that holds nothing, else the one whose tile the trace needs again
// latest (with the order of future requests known, that choice keeps the
// fewest reads of any eviction order, as Belady showed for page replacement).
struct zi_tier {
    enum State { FREE, READING, READY };
    struct Item {
        zi_file_source *src = nullptr;
        int64_t tile = -1;
        bool operator==(const Item &o) const { return src == o.src && tile == o.tile; }
    };
    struct Buf {
        Item item;            // the tile the buffer holds or is reading
        State state = FREE;   // FREE: holds nothing valid
        int err = 0;          // errno of a failed read
        bool held = false;    // handed to a request whose copy is not enqueued yet
        bool reserved = false;// read on demand for a request that has not taken it yet
        uint64_t copies = 0;  // copies out of it enqueued ('copied' recorded after each)
        uint64_t synced = 0;  // copies known to be done
        hipEvent_t copied = nullptr;
    };

    int S = 2, threads = 4;
    bool shared = false;
    std::vector<zi_file_source *> srcs;
    std::vector<char *> buf;     // pinned tile buffers, made on first use
    std::vector<char *> bounce;  // per-thread buffers for direct reads
    std::vector<Buf> bufs;
    std::vector<Item> trace, rec;
    bool recording = false;      // a shared tier records until its first step mark
    int64_t pos = 0;             // trace position the next request is expected at
    int64_t rpos = 0;            // first trace position without a buffer yet
    std::deque<int> assigned;    // buffer of each trace position in [pos, rpos)
    bool demand = false;         // a request off the trace, read before the trace's next
    Item demand_item;
    int device = -1;
    bool started = false, stop = false;
    std::mutex mu;
    std::condition_variable cv;
    std::thread reader;
    int64_t tiles_read = 0, hits = 0, restarts = 0, demand_reads = 0, steps = 0;
    double read_s = 0, bytes = 0, wait_s = 0;

    bool read_ahead() const { return !recording && !trace.empty(); }
    const Item &at(int64_t q) const { return trace[(size_t)(q % (int64_t)trace.size())]; }

    int holding(const Item &it) const {  // buffer holding or reading `it`, or -1
        for (int b = 0; b < S; ++b)
            if (bufs[b].state != FREE && bufs[b].item == it) return b;
        return -1;
    }

    bool pending(int b) const {
        for (int x : assigned)
            if (x == b) return true;
        return false;
    }

    // Trace distance from rpos to the next request for `it` (L + 1: none).
    int64_t next_use(const Item &it) const {
        const int64_t L = (int64_t)trace.size();
        if (!read_ahead()) return L + 1;
        for (int64_t j = 0; j < L; ++j)
            if (at(rpos + j) == it) return j;
        return L + 1;
    }

    // An off-trace request has found every buffer kept for upcoming trace
    // positions: give back read-ahead buffers from the farthest position
    // down, until one may be overwritten.  A buffer given back keeps its tile
    // (the cache may still serve it when the read-ahead comes back there).
    // Returns whether anything was given back.
    bool trim_read_ahead() {
        bool any = false;
        while (!assigned.empty() && victim() < 0) {
            if (bufs[assigned.back()].state == READING) break;
            assigned.pop_back();
            --rpos;
            any = true;
        }
        return any;
    }

    // A buffer the reader may overwrite, or -1.
    int victim() const {
        int best = -1;
        int64_t far = -1;
        for (int b = 0; b < S; ++b) {
            const Buf &x = bufs[b];
            if (x.state == READING || x.held || x.reserved || pending(b)) continue;
            if (x.state == FREE) return b;
            const int64_t d = next_use(x.item);
            if (d > far) {
                far = d;
                best = b;
            }
        }
        return best;
    }

    void run() {
        if (device >= 0) (void)hipSetDevice(device);
        std::unique_lock<std::mutex> lock(mu);
        for (;;) {
            if (stop) return;
            // what to read next: an off-trace request first, then the trace
            Item want;
            bool have = false, for_trace = false;
            if (demand) {
                if (holding(demand_item) >= 0) {
                    demand = false;  // served from a buffer meanwhile
                } else {
                    want = demand_item;
                    have = true;
                }
            }
            if (!have && read_ahead() && rpos - pos < S) {
                const Item &it = at(rpos);
                const int b = holding(it);
                if (b >= 0) {  // already held: no read
                    assigned.push_back(b);
                    ++rpos;
                    ++hits;
                    cv.notify_all();
                    continue;
                }
                want = it;
                have = true;
                for_trace = true;
            }
            if (!have) {
                cv.wait(lock);
                continue;
            }
            const int k = victim();
            if (k < 0) {
                // only the consumer frees a held buffer; buffers kept for the
                // trace are given back to a request the trace does not hold,
                // which would otherwise wait for them forever
                if (!for_trace && trim_read_ahead()) continue;
                cv.wait(lock);
                continue;
            }
            if (bufs[k].synced < bufs[k].copies) {
                // the buffer is free once the copies that read it are done (the
                // event was recorded after the last one before its count rose)
                const uint64_t upto = bufs[k].copies;
                hipEvent_t ev = bufs[k].copied;
                lock.unlock();
                (void)hipEventSynchronize(ev);
                lock.lock();
                bufs[k].synced = std::max(bufs[k].synced, upto);
                continue;  // the plan may have changed meanwhile
            }
            bufs[k].item = want;
            bufs[k].state = READING;
            bufs[k].err = 0;
            if (for_trace) {
                assigned.push_back(k);
                ++rpos;
            } else {  // kept for the waiting request until it takes the buffer
                demand = false;
                bufs[k].reserved = true;
                ++demand_reads;
            }
            lock.unlock();
            const auto t0 = std::chrono::steady_clock::now();
            zi_file_source *src = want.src;
            const int err = parallel_pread(src->fd, buf[k], src->offset + (uint64_t)want.tile * src->tile_bytes,
                                           src->tile_bytes, threads, src->direct ? bounce.data() : nullptr);
            const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
            lock.lock();
            bufs[k].state = READY;
            bufs[k].err = err;
            if (!err) {
                ++tiles_read;
                read_s += secs;
                bytes += (double)src->tile_bytes;
                ++src->tiles_read;
                src->read_s += secs;
                src->bytes += (double)src->tile_bytes;
            }
            cv.notify_all();
        }
    }
};

namespace zi {

const zi_plan *source_plan(const zi_file_source *s) { return s->plan; }

// First use, on the context's device: pinned staging buffers (the largest
// tile of the tier's sources each), their events, the read buffers and the
// reader thread.
static zi_status tier_start(zi_tier *t) {
    if (t->started) return ZI_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(ZI_ERR_HIP, "hipGetDevice failed");
    uint64_t bytes = 0;
    bool direct = false;
    for (zi_file_source *s : t->srcs) {
        bytes = std::max(bytes, s->tile_bytes);
        direct = direct || s->direct;
    }
    std::vector<char *> bufs(t->S, nullptr);
    std::vector<hipEvent_t> evs(t->S, nullptr);
    std::vector<char *> bb;
    auto undo = [&] {
        for (hipEvent_t e : evs)
            if (e) (void)hipEventDestroy(e);
        for (char *p : bufs)
            if (p) (void)hipHostFree(p);
        free_buffers(bb);
    };
    for (int k = 0; k < t->S; ++k) {
        void *p = nullptr;
        hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
        if (e != hipSuccess) {
            (void)hipGetLastError();  // not the caller's next error
            undo();
            return fail(ZI_ERR_HIP, "hipHostMalloc of a %llu B staging buffer: %s", (unsigned long long)bytes,
                        hipGetErrorString(e));
        }
        bufs[k] = static_cast<char *>(p);
        e = hipEventCreateWithFlags(&evs[k], hipEventDisableTiming | hipEventBlockingSync);
        if (e != hipSuccess) {
            evs[k] = nullptr;
            undo();
            return fail(ZI_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
    }
    if (direct) {
        bb = bounce_buffers(t->threads);
        if ((int)bb.size() != t->threads) {
            undo();
            return fail(ZI_ERR_ARG, "out of host memory for the read buffers");
        }
    }
    t->device = dev;
    t->buf = bufs;
    t->bounce = bb;
    for (int k = 0; k < t->S; ++k) t->bufs[k].copied = evs[k];
    try {
        t->reader = std::thread([t] { t->run(); });
    } catch (...) {
        for (auto &sl : t->bufs) sl.copied = nullptr;
        t->buf.clear();
        t->bounce.clear();
        undo();
        return fail(ZI_ERR_STATE, "could not start the reader thread");
    }
    t->started = true;
    return ZI_OK;
}

// Stop the reader, wait for every copy out of the staging buffers, free them.
static void tier_stop(zi_tier *t) {
    if (!t->started) return;
    {
        std::lock_guard<std::mutex> lock(t->mu);
        t->stop = true;
    }
    t->cv.notify_all();
    t->reader.join();
    for (auto &sl : t->bufs)
        if (sl.copied) {
            (void)hipEventSynchronize(sl.copied);
            (void)hipEventDestroy(sl.copied);
            sl.copied = nullptr;
        }
    for (char *p : t->buf)
        if (p) (void)hipHostFree(p);
    t->buf.clear();
    free_buffers(t->bounce);
    t->started = false;
}

zi_status source_acquire(zi_file_source *s, int64_t tile, const void **host, int *slot) {
    if (tile < 0 || tile >= s->N) return fail(ZI_ERR_ARG, "tile %lld out of range", (long long)tile);
    if (!s->tier) {  // a standalone source: a private tier that reads its tiles in order
        zi_tier *t = new (std::nothrow) zi_tier;
        if (!t) return fail(ZI_ERR_ARG, "out of host memory");
        t->S = s->S;
        t->threads = s->threads;
        t->srcs.push_back(s);
        t->bufs.assign(t->S, zi_tier::Buf{});
        for (int64_t i = 0; i < s->N; ++i) t->trace.push_back(zi_tier::Item{s, i});
        s->tier = t;
        s->own_tier = true;
    }
    zi_tier *t = s->tier;
    zi_status st = tier_start(t);
    if (st != ZI_OK) return st;
    const auto t0 = std::chrono::steady_clock::now();
    const zi_tier::Item want{s, tile};
    std::unique_lock<std::mutex> lock(t->mu);
    if (t->recording && t->rec.size() < (1u << 20)) t->rec.push_back(want);
    bool on_trace = t->read_ahead() && t->at(t->pos) == want;
    if (!on_trace && t->read_ahead()) {
        // restart the read-ahead at the request's next place in the trace
        const int64_t L = (int64_t)t->trace.size();
        for (int64_t j = 1; j < L && !on_trace; ++j)
            if (t->at(t->pos + j) == want) {
                ++t->restarts;
                t->assigned.clear();
                t->pos = t->rpos = t->pos + j;
                on_trace = true;
            }
        t->cv.notify_all();
    }
    int b;
    if (on_trace) {
        t->cv.wait(lock, [&] { return !t->assigned.empty() && t->bufs[t->assigned.front()].state == zi_tier::READY; });
        b = t->assigned.front();
        t->assigned.pop_front();
        ++t->pos;
    } else {
        // off the trace (or while recording): a buffer that holds it, else a read on demand
        b = t->holding(want);
        if (b >= 0 && t->bufs[b].state == zi_tier::READY) {
            ++t->hits;
        } else if (b < 0) {
            t->demand = true;
            t->demand_item = want;
            t->cv.notify_all();
        }
        t->cv.wait(lock, [&] {
            const int h = t->holding(want);
            return h >= 0 && t->bufs[h].state == zi_tier::READY;
        });
        b = t->holding(want);
    }
    t->cv.notify_all();  // the reader may run further ahead now
    const double waited = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    t->wait_s += waited;
    s->wait_s += waited;
    if (t->bufs[b].err) {
        const int err = t->bufs[b].err;
        t->bufs[b].state = zi_tier::FREE;
        t->bufs[b].item = zi_tier::Item{};
        t->bufs[b].reserved = false;
        // later positions may have been given the same buffer: plan them again
        t->assigned.clear();
        t->rpos = t->pos;
        t->cv.notify_all();
        return fail(ZI_ERR_IO, "reading tile %lld: %s", (long long)tile, strerror(err));
    }
    t->bufs[b].held = true;
    for (auto &x : t->bufs)  // an on-demand read of this tile is no longer waited for
        if (x.item == want) x.reserved = false;
    *host = t->buf[b];
    *slot = b;
    return ZI_OK;
}

hipEvent_t source_copy_event(zi_file_source *s, int slot) { return s->tier->bufs[slot].copied; }

void source_release(zi_file_source *s, int slot) {
    zi_tier *t = s->tier;
    {
        std::lock_guard<std::mutex> lock(t->mu);
        t->bufs[slot].held = false;
        ++t->bufs[slot].copies;
    }
    t->cv.notify_all();
}

// A request that fails after source_acquire (the copy could not be enqueued)
// gives the buffer back; its tile stays cached.
void source_abandon(zi_file_source *s, int slot) {
    zi_tier *t = s->tier;
    {
        std::lock_guard<std::mutex> lock(t->mu);
        t->bufs[slot].held = false;
    }
    t->cv.notify_all();
}

// The tier's buffer policy run without threads or files on a trace of item
// ids: before each request the reader fills its window (up to W positions
// ahead, W <= S; a held tile assigned without a read, else a read into the
// buffer the policy picks), then the request takes its position's buffer.
// Returns the reads attributed to each step (by the position read).
static std::vector<int64_t> tier_simulate(const std::vector<int64_t> &trace, int S, int W, int steps) {
    const int64_t L = (int64_t)trace.size();
    std::vector<int64_t> reads(steps, 0);
    std::vector<int64_t> item(S, -1);
    std::deque<int> pend;
    int64_t pos = 0, rpos = 0;
    auto at = [&](int64_t q) { return trace[(size_t)(q % L)]; };
    auto next_use = [&](int64_t it) -> int64_t {
        for (int64_t j = 0; j < L; ++j)
            if (at(rpos + j) == it) return j;
        return L + 1;
    };
    for (int64_t r = 0; r < (int64_t)steps * L; ++r) {
        while (rpos - pos < W && rpos < (int64_t)steps * L) {
            const int64_t it = at(rpos);
            int b = -1;
            for (int k = 0; k < S && b < 0; ++k)
                if (item[k] == it) b = k;
            if (b < 0) {
                int64_t far = -1;
                for (int k = 0; k < S; ++k) {
                    bool p = false;
                    for (int x : pend) p = p || x == k;
                    if (p) continue;
                    if (item[k] < 0) {
                        b = k;
                        break;
                    }
                    const int64_t d = next_use(item[k]);
                    if (d > far) {
                        far = d;
                        b = k;
                    }
                }
                if (b < 0) break;  // every buffer waits for a pending request
                item[b] = it;
                ++reads[(size_t)(rpos / L)];
            }
            pend.push_back(b);
            ++rpos;
        }
        pend.pop_front();  // request r (= pos) takes its buffer
        ++pos;
    }
    return reads;
}

}  // namespace zi

extern "C" {

zi_status zi_tier_simulate_reads(const int64_t *trace, int64_t len, int32_t buffers, int32_t window, int32_t steps,
                                 int64_t *reads_per_step) {
    clear_error();
    if (!trace || !reads_per_step || len < 1) return fail(ZI_ERR_ARG, "a trace of at least one request is required");
    if (buffers < 2) return fail(ZI_ERR_ARG, "at least two buffers (got %d)", buffers);
    if (window < 1 || window > buffers) return fail(ZI_ERR_ARG, "window must be in 1..buffers (got %d)", window);
    if (steps < 1) return fail(ZI_ERR_ARG, "steps must be >= 1");
    const std::vector<int64_t> t(trace, trace + len);
    const std::vector<int64_t> r = tier_simulate(t, buffers, window, steps);
    for (int k = 0; k < steps; ++k) reads_per_step[k] = r[(size_t)k];
    return ZI_OK;
}

zi_status zi_tier_trace_get(zi_tier *t, int64_t *ids, int64_t cap, int64_t *len) {
    clear_error();
    if (!t || !len) return fail(ZI_ERR_ARG, "tier and len are required");
    std::lock_guard<std::mutex> lock(t->mu);
    if (t->recording) return fail(ZI_ERR_STATE, "the trace is still being recorded (no zi_tier_step yet)");
    *len = (int64_t)t->trace.size();
    for (int64_t k = 0; k < *len && k < cap && ids; ++k) {
        const zi_tier::Item &it = t->trace[(size_t)k];
        int64_t s = 0;
        while (s < (int64_t)t->srcs.size() && t->srcs[(size_t)s] != it.src) ++s;
        ids[k] = (s << 32) | it.tile;
    }
    return ZI_OK;
}

zi_status zi_file_source_create(const zi_plan *plan, const char *path, uint64_t offset, int32_t staging,
                                int32_t threads, zi_file_source **out) {
    clear_error();
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!plan || !path) return fail(ZI_ERR_ARG, "plan and path are required");
    if (staging < 2) return fail(ZI_ERR_ARG, "at least two staging buffers (got %d)", staging);
    if (threads < 1) return fail(ZI_ERR_ARG, "threads must be >= 1 (got %d)", threads);
    const uint64_t tile = plan->info.tile_bytes;
    const uint64_t need = offset + tile * (uint64_t)plan->prob.N;
    const bool can_direct = offset % kDirectAlign == 0 && tile % kDirectAlign == 0;
    int fd = -1;
    bool direct = false;
    if (can_direct) {
        fd = open(path, O_RDONLY | O_DIRECT | O_CLOEXEC);
        direct = fd >= 0;
    }
    if (fd < 0) fd = open(path, O_RDONLY | O_CLOEXEC);  // file systems without O_DIRECT
    if (fd < 0) return fail(ZI_ERR_IO, "open %s: %s", path, strerror(errno));
    struct stat sb;
    if (fstat(fd, &sb) != 0 || (uint64_t)sb.st_size < need) {
        close(fd);
        return fail(ZI_ERR_IO, "%s holds %lld bytes; the weight needs %llu from offset %llu", path,
                    (long long)sb.st_size, (unsigned long long)need, (unsigned long long)offset);
    }
    zi_file_source *s = new (std::nothrow) zi_file_source;
    if (!s) {
        close(fd);
        return fail(ZI_ERR_ARG, "out of host memory");
    }
    s->plan = plan;
    s->fd = fd;
    s->direct = direct;
    s->offset = offset;
    s->tile_bytes = tile;
    s->N = plan->prob.N;
    s->S = staging;
    s->threads = threads;
    *out = s;
    return ZI_OK;
}

zi_status zi_file_source_destroy(zi_file_source *s) {
    clear_error();
    if (!s) return ZI_OK;
    if (s->tier && !s->own_tier) return fail(ZI_ERR_STATE, "the source belongs to a tier: destroy the tier first");
    if (s->own_tier) {
        tier_stop(s->tier);
        delete s->tier;
    }
    close(s->fd);
    delete s;
    return ZI_OK;
}

zi_status zi_file_source_read(zi_file_source *s, int64_t tile, void *dst) {
    clear_error();
    if (!s || !dst) return fail(ZI_ERR_ARG, "source and dst are required");
    if (tile < 0 || tile >= s->N) return fail(ZI_ERR_ARG, "tile %lld out of range", (long long)tile);
    if (s->direct && (uintptr_t)dst % kDirectAlign)
        return fail(ZI_ERR_ALIGN, "dst must be %llu-byte aligned for direct reads",
                    (unsigned long long)kDirectAlign);
    const uint64_t at = s->offset + (uint64_t)tile * s->tile_bytes;
    int err = parallel_pread(s->fd, static_cast<char *>(dst), at, s->tile_bytes, s->threads, nullptr);
    if (err == EFAULT && s->direct) {  // page-locked destination: read through bounce buffers
        std::vector<char *> tmp = bounce_buffers(s->threads);
        err = (int)tmp.size() == s->threads
                  ? parallel_pread(s->fd, static_cast<char *>(dst), at, s->tile_bytes, s->threads, tmp.data())
                  : ENOMEM;
        free_buffers(tmp);
    }
    if (err) return fail(ZI_ERR_IO, "reading tile %lld: %s", (long long)tile, strerror(err));
    return ZI_OK;
}

zi_status zi_file_source_stats_get(zi_file_source *s, zi_source_stats *out) {
    clear_error();
    if (!s || !out) return fail(ZI_ERR_ARG, "source and out are required");
    out->direct = s->direct ? 1 : 0;
    if (!s->tier) {
        out->tiles_read = out->restarts = 0;
        out->read_s = out->bytes = out->wait_s = 0.0;
        return ZI_OK;
    }
    std::lock_guard<std::mutex> lock(s->tier->mu);
    out->tiles_read = s->tiles_read;
    out->restarts = s->tier->restarts + s->tier->demand_reads;
    out->read_s = s->read_s;
    out->bytes = s->bytes;
    out->wait_s = s->wait_s;
    return ZI_OK;
}

zi_status zi_tier_create(int32_t staging, int32_t threads, zi_tier **out) {
    clear_error();
    if (!out) return fail(ZI_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (staging < 2) return fail(ZI_ERR_ARG, "at least two staging buffers (got %d)", staging);
    if (threads < 1) return fail(ZI_ERR_ARG, "threads must be >= 1 (got %d)", threads);
    zi_tier *t = new (std::nothrow) zi_tier;
    if (!t) return fail(ZI_ERR_ARG, "out of host memory");
    t->S = staging;
    t->threads = threads;
    t->shared = true;
    t->recording = true;
    t->bufs.assign(staging, zi_tier::Buf{});
    *out = t;
    return ZI_OK;
}

zi_status zi_tier_add(zi_tier *t, zi_file_source *s) {
    clear_error();
    if (!t || !s) return fail(ZI_ERR_ARG, "tier and source are required");
    if (s->tier) return fail(ZI_ERR_STATE, "the source is already read by a tier (or has been used on its own)");
    std::lock_guard<std::mutex> lock(t->mu);
    if (t->started) return fail(ZI_ERR_STATE, "the tier is in use: add every source before the first pass");
    t->srcs.push_back(s);
    s->tier = t;
    return ZI_OK;
}

zi_status zi_tier_step(zi_tier *t) {
    clear_error();
    if (!t) return fail(ZI_ERR_ARG, "tier is NULL");
    {
        std::lock_guard<std::mutex> lock(t->mu);
        ++t->steps;
        if (t->recording) {
            t->trace = t->rec;
            t->rec.clear();
            t->recording = false;
            t->pos = t->rpos = 0;
            t->assigned.clear();
        } else if (!t->trace.empty()) {
            const int64_t L = (int64_t)t->trace.size();
            if (t->pos % L == 0) return ZI_OK;  // in step with the trace
            ++t->restarts;  // the step ended elsewhere: start the next one at the trace's start
            t->pos = t->rpos = (t->pos + L - 1) / L * L;
            t->assigned.clear();
        }
    }
    t->cv.notify_all();
    return ZI_OK;
}

zi_status zi_tier_destroy(zi_tier *t) {
    clear_error();
    if (!t) return ZI_OK;
    tier_stop(t);
    for (zi_file_source *s : t->srcs) s->tier = nullptr;
    delete t;
    return ZI_OK;
}

zi_status zi_tier_stats_get(zi_tier *t, zi_tier_stats *out) {
    clear_error();
    if (!t || !out) return fail(ZI_ERR_ARG, "tier and out are required");
    std::lock_guard<std::mutex> lock(t->mu);
    out->trace_len = (int64_t)(t->recording ? t->rec.size() : t->trace.size());
    out->steps = t->steps;
    out->tiles_read = t->tiles_read;
    out->restarts = t->restarts;
    out->demand_reads = t->demand_reads;
    out->hits = t->hits;
    out->read_s = t->read_s;
    out->bytes = t->bytes;
    out->wait_s = t->wait_s;
    return ZI_OK;
}

}  // extern "C"
