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
    enum State { FREE, READING, READY, IN_COPY };
    struct Slot {
        int64_t tile = -1;
        State state = FREE;
        int err = 0;        // errno of a failed read
        hipEvent_t copied = nullptr;
    };

    const zi_plan *plan = nullptr;
    int fd = -1;
    bool direct = false;
    uint64_t offset = 0, tile_bytes = 0;
    int64_t N = 0;
    int S = 2, threads = 4;
    int device = -1;

    std::vector<char *> buf;     // pinned staging buffers (hipHostMalloc), made on first use
    std::vector<char *> bounce;  // the reader's per-thread buffers for direct reads
    std::vector<Slot> slots;
    std::mutex mu;
    std::condition_variable cv;
    std::thread reader;
    bool started = false, stop = false;
    int64_t next_tile = 0;  // the reader's next tile
    int next_slot = 0;      // the slot the reader fills next
    int cons_slot = 0;      // the slot the next request is served from
    uint64_t gen = 0;       // bumped when the read-ahead restarts
    // statistics
    int64_t tiles_read = 0, restarts = 0;
    double read_s = 0, bytes = 0, wait_s = 0;

    void run() {
        if (device >= 0) (void)hipSetDevice(device);
        std::unique_lock<std::mutex> lock(mu);
        for (;;) {
            const int k = next_slot;
            cv.wait(lock, [&] { return stop || slots[k].state == FREE || slots[k].state == IN_COPY; });
            if (stop) return;
            if (slots[k].state == IN_COPY) {
                // the staging buffer is free once the copy that reads it is done
                hipEvent_t ev = slots[k].copied;
                lock.unlock();
                (void)hipEventSynchronize(ev);
                lock.lock();
                if (slots[k].state == IN_COPY) slots[k].state = FREE;
                continue;
            }
            const int64_t t = next_tile;
            const uint64_t g = gen;
            slots[k].tile = t;
            slots[k].state = READING;
            slots[k].err = 0;
            next_tile = (t + 1) % N;
            next_slot = (k + 1) % S;
            lock.unlock();
            const auto t0 = std::chrono::steady_clock::now();
            const int err = parallel_pread(fd, buf[k], offset + (uint64_t)t * tile_bytes, tile_bytes, threads,
                                           direct ? bounce.data() : nullptr);
            const double secs = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
            lock.lock();
            if (gen != g) {
                slots[k].state = FREE;  // the read-ahead restarted meanwhile: discard
                slots[k].tile = -1;
            } else {
                slots[k].state = READY;
                slots[k].err = err;
                if (!err) {
                    ++tiles_read;
                    read_s += secs;
                    bytes += (double)tile_bytes;
                }
            }
            cv.notify_all();
        }
    }
};

namespace zi {

const zi_plan *source_plan(const zi_file_source *s) { return s->plan; }

// First use, on the context's device: pinned staging buffers, their events and
// the reader thread.
static zi_status source_start(zi_file_source *s) {
    if (s->started) return ZI_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(ZI_ERR_HIP, "hipGetDevice failed");
    std::vector<char *> bufs(s->S, nullptr);
    std::vector<hipEvent_t> evs(s->S, nullptr);
    auto undo = [&] {
        for (hipEvent_t e : evs)
            if (e) (void)hipEventDestroy(e);
        for (char *p : bufs)
            if (p) (void)hipHostFree(p);
    };
    for (int k = 0; k < s->S; ++k) {
        void *p = nullptr;
        hipError_t e = hipHostMalloc(&p, s->tile_bytes, hipHostMallocDefault);
        if (e != hipSuccess) {
            undo();
            return fail(ZI_ERR_HIP, "hipHostMalloc of a %llu B staging buffer: %s",
                        (unsigned long long)s->tile_bytes, hipGetErrorString(e));
        }
        bufs[k] = static_cast<char *>(p);
        e = hipEventCreateWithFlags(&evs[k], hipEventDisableTiming | hipEventBlockingSync);
        if (e != hipSuccess) {
            evs[k] = nullptr;
            undo();
            return fail(ZI_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
    }
    if (s->direct) {
        s->bounce = bounce_buffers(s->threads);
        if ((int)s->bounce.size() != s->threads) {
            free_buffers(s->bounce);
            undo();
            return fail(ZI_ERR_ARG, "out of host memory for the read buffers");
        }
    }
    s->device = dev;
    s->buf = bufs;
    for (int k = 0; k < s->S; ++k) s->slots[k].copied = evs[k];
    try {
        s->reader = std::thread([s] { s->run(); });
    } catch (...) {
        for (auto &sl : s->slots) sl.copied = nullptr;
        s->buf.clear();
        free_buffers(s->bounce);
        undo();
        return fail(ZI_ERR_STATE, "could not start the reader thread");
    }
    s->started = true;
    return ZI_OK;
}

zi_status source_acquire(zi_file_source *s, int64_t tile, const void **host, int *slot) {
    zi_status st = source_start(s);
    if (st != ZI_OK) return st;
    if (tile < 0 || tile >= s->N) return fail(ZI_ERR_ARG, "tile %lld out of range", (long long)tile);
    const auto t0 = std::chrono::steady_clock::now();
    std::unique_lock<std::mutex> lock(s->mu);
    const int k = s->cons_slot;
    const bool ahead = (s->slots[k].state == zi_file_source::READING || s->slots[k].state == zi_file_source::READY) &&
                       s->slots[k].tile == tile;
    const bool coming = s->slots[k].state != zi_file_source::READING && s->slots[k].state != zi_file_source::READY &&
                        s->next_slot == k && s->next_tile == tile;
    if (!ahead && !coming) {
        // restart the read-ahead at `tile`, from the slot the request takes
        ++s->gen;
        ++s->restarts;
        for (int j = 0; j < s->S; ++j)
            if (s->slots[j].state == zi_file_source::READY) {
                s->slots[j].state = zi_file_source::FREE;
                s->slots[j].tile = -1;
            }
        s->next_tile = tile;
        s->next_slot = k;
        s->cv.notify_all();
    }
    s->cv.wait(lock, [&] {
        return s->slots[k].state == zi_file_source::READY && s->slots[k].tile == tile;
    });
    s->wait_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    if (s->slots[k].err) {
        const int err = s->slots[k].err;
        s->slots[k].state = zi_file_source::FREE;
        s->slots[k].tile = -1;
        s->cv.notify_all();
        return fail(ZI_ERR_IO, "reading tile %lld: %s", (long long)tile, strerror(err));
    }
    *host = s->buf[k];
    *slot = k;
    return ZI_OK;
}

hipEvent_t source_copy_event(zi_file_source *s, int slot) { return s->slots[slot].copied; }

void source_release(zi_file_source *s, int slot) {
    {
        std::lock_guard<std::mutex> lock(s->mu);
        s->slots[slot].state = zi_file_source::IN_COPY;
        s->cons_slot = (slot + 1) % s->S;
    }
    s->cv.notify_all();
}

// A request that fails after source_acquire (the copy could not be enqueued)
// gives the buffer back unread by any copy.
void source_abandon(zi_file_source *s, int slot) {
    {
        std::lock_guard<std::mutex> lock(s->mu);
        s->slots[slot].state = zi_file_source::FREE;
        s->slots[slot].tile = -1;
        ++s->gen;
        s->next_slot = slot;
        s->cons_slot = slot;
    }
    s->cv.notify_all();
}

}  // namespace zi

extern "C" {

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
    s->slots.assign(staging, zi_file_source::Slot{});
    *out = s;
    return ZI_OK;
}

zi_status zi_file_source_destroy(zi_file_source *s) {
    clear_error();
    if (!s) return ZI_OK;
    if (s->started) {
        {
            std::lock_guard<std::mutex> lock(s->mu);
            s->stop = true;
        }
        s->cv.notify_all();
        s->reader.join();
        // no copy may still read a staging buffer when it is freed
        for (auto &sl : s->slots)
            if (sl.copied) {
                (void)hipEventSynchronize(sl.copied);
                (void)hipEventDestroy(sl.copied);
            }
        for (char *p : s->buf)
            if (p) (void)hipHostFree(p);
        free_buffers(s->bounce);
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
    std::lock_guard<std::mutex> lock(s->mu);
    out->tiles_read = s->tiles_read;
    out->restarts = s->restarts;
    out->read_s = s->read_s;
    out->bytes = s->bytes;
    out->wait_s = s->wait_s;
    out->direct = s->direct ? 1 : 0;
    return ZI_OK;
}

}  // extern "C"
