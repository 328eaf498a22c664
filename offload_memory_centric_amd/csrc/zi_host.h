// zi_host.h -- host-side internals shared by zi_plan.cpp and zi_api.cpp.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/zi.h"

struct zi_plan {
    zi_problem prob;
    zi_plan_info info;
};

namespace zi {

// Record an error for zi_last_error() and return its status.
zi_status fail(zi_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// with_grad: the plan will run backward passes (gradient slots are sized);
// zi_plan_tiles passes dW_host != NULL.
zi_status plan_validate_and_fill(const zi_problem *p, zi_plan_info *info, bool with_grad);

// One pass over the ring, times in seconds per tile.
struct PassModel {
    int N = 1, d = 1, dw_slots = 0;
    bool backward = false;
    // backward: the dX products of tiles 2j and 2j + 1 run as one launch once
    // both are resident (the stager does so with gradient slots, d >= 2,
    // N >= 2 and n a multiple of the GEMM's reduction step)
    bool pairs = false;
    // with pairs: the recomputed forward products of tiles 2j and 2j + 1 also
    // run together, once tile 2j + 1 is resident (the stager does so where one
    // launch takes fewer rounds of workgroups than two)
    bool re_pairs = false;
    double t_h2d = 0, t_d2h = 0;
    double t_fwd = 0, t_recompute = 0, t_dx = 0, t_dw = 0;
};
struct Prediction {
    double t_pass = 0, t_compute = 0, t_link = 0, stall = 0;
};
Prediction simulate_pass(const PassModel &m);
// Whether the backward pairs the dX products of tiles 2j and 2j + 1 (one
// launch with a reduction of 2n): with gradient slots, d >= 2, N >= 2 and n a
// multiple of the GEMM's reduction step, so that the second tile's rows start
// on a step boundary.  The stager (zi_api.cpp) and the timing model both use it.
constexpr int64_t kPairStep = 64;
bool pairs_apply(int N, int d, int dw_slots, int64_t n);
// Time of one step (the passes in order) in a run of back-to-back steps on
// one ring: the third step's end minus the second's.  All passes share the
// first one's d and gradient slots.
double simulate_steady_step(const PassModel *passes, int count);

// The host optimizer (zi_adam.cpp), as the context drives it.
const zi_plan *adam_plan(const zi_adam *a);
// Queue the update of `tile`; it starts once `landed_event` (a hipEvent_t
// recorded after the tile's gradient copy) has completed, and owns the event.
void adam_enqueue(zi_adam *a, int64_t tile, void *landed_event);
// Block until every queued update of `tile` is done.
void adam_wait_tile(zi_adam *a, int64_t tile);
// Block until the queue is empty; the first failure, if any.
zi_status adam_wait_all(zi_adam *a);

// The file source (zi_source.cpp), as the context drives it.
const zi_plan *source_plan(const zi_file_source *s);
// Block until `tile` is in a staging buffer; its host address and slot.
zi_status source_acquire(zi_file_source *s, int64_t tile, const void **host, int *slot);
// The event the caller records on the copy stream after the copy out of `slot`.
hipEvent_t source_copy_event(zi_file_source *s, int slot);
// The copy out of `slot` is enqueued and its event recorded.
void source_release(zi_file_source *s, int slot);
// No copy out of `slot` was enqueued after all.
void source_abandon(zi_file_source *s, int slot);

}  // namespace zi
