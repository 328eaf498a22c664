/*
 * zi.h -- memory-centric tiling of a large linear operator on one AMD MI355X.
 *
 * The method (ZeRO-Infinity transformer-math page, section "Memory-centric
 * tiling: operators bigger than the device"; pwwt.cn ZeRO-Infinity article,
 * section "关键技术一：Memory-centric tiling for working memory"): a linear
 * operator Y = X W whose weight W[K x M] does not fit the device is split
 * along its output dimension into N tiles W_1..W_N of n = M/N columns.  The
 * tiles stay in pinned host memory and are brought into device memory one at
 * a time; each produces its slice Y_i = X W_i of the output with no
 * communication between tiles, and its buffer is released before the next
 * tile needs it.  Here the tiles flow through a d-slot ring of device buffers
 * fed by host-to-device copies on a dedicated copy stream, so that the copy of
 * tile i+d overlaps the products of tile i (the prefetch of the same page's
 * section "Prefetch depth: how far ahead the pipeline must run").  The
 * backward pass stages every tile again (the FLOPs-per-byte section counts the
 * parameters climbing twice per step), forms dX += dY_i W_i^T and
 * dW_i = X^T dY_i, and writes each dW_i back to pinned host memory on a second
 * copy stream.
 *
 * Data layout (all row-major, element = 16-bit input format unless stated):
 *   X   [T x K]   device, activations                       (caller owned)
 *   W^t [M x K]   pinned host, "out-major": row m of W^t is column m of W,
 *                 so tile i is the contiguous rows [i*n, (i+1)*n) of W^t,
 *                 at byte offset i*K*n*2                     (caller owned)
 *   Y   [T x M]   device, output of the forward             (caller owned)
 *   dY  [T x M]   device, upstream gradient                 (caller owned)
 *   dX  [T x K]   device, fp32, accumulated over the tiles  (caller owned)
 *   dW^t[M x K]   pinned host, same layout as W^t           (caller owned)
 *
 * Conventions shared by every call:
 *   - Every call returns a zi_status and never throws.  On an error nothing
 *     has been enqueued; zi_last_error() returns a text for the calling
 *     thread's most recent error.
 *   - Forward/backward calls only enqueue work on the context's streams and
 *     return at once.  Inputs must stay valid, and outputs (device or host)
 *     must not be read, until zi_sync() on that context returns ZI_OK.
 *   - An asynchronous HIP failure makes the context's error sticky
 *     (ZI_ERR_HIP): zi_sync() and every later call on it return it.
 *   - Streams are hipStream_t values passed as void*; they must be streams of
 *     the current device with default priority.  The library creates only
 *     hipEvents; it never allocates device memory inside a call, so the ring
 *     lives in the caller's workspace and the device budget holds by
 *     construction.
 *   - One host thread at a time per context.
 */
#ifndef ZI_H
#define ZI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZI_OK = 0,
    ZI_ERR_ARG = 1,        /* NULL where a pointer is required, bad enum, bad size */
    ZI_ERR_SHAPE = 2,      /* N does not divide M, K or n not a multiple of 8, ... */
    ZI_ERR_BUDGET = 3,     /* ring does not fit the device budget or the workspace */
    ZI_ERR_NOT_PINNED = 4, /* host weight or gradient buffer is not page-locked */
    ZI_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned */
    ZI_ERR_HIP = 6,        /* a HIP runtime call failed (sticky on the context) */
    ZI_ERR_STATE = 7,      /* plan and context disagree, or the context is unusable */
    ZI_ERR_IO = 8          /* a file could not be opened or read */
} zi_status;

typedef enum { ZI_F16 = 1, ZI_BF16 = 2 } zi_dtype;

/* zi_problem.flags */
#define ZI_FLAG_F32_OUT 0x1u /* Y and dW^t are written in fp32 instead of the input
                                format (same kernels, fp32 epilogue): the form in
                                which rounding-free results can be compared.  The
                                caller sizes Y and dW_host for 4-byte elements. */

/* The problem, as the pages state it: X, W, the number of tiles, the prefetch
 * depth and the device memory the tiles may occupy. */
typedef struct {
    int64_t T;            /* tokens: rows of X, Y, dY, dX                      (>= 1) */
    int64_t K;            /* in_features: columns of X; multiple of 8          (>= 8) */
    int64_t M;            /* out_features: columns of Y; N must divide it       (>= 8) */
    int32_t N;            /* number of weight tiles along M; n = M/N multiple of 8 */
    int32_t d;            /* ring depth: device slots for weight tiles          (>= 1) */
    int32_t dtype;        /* zi_dtype of X, W, dY, Y and dW */
    uint32_t flags;       /* ZI_FLAG_* */
    uint64_t device_budget_bytes; /* device bytes the tile buffers may use; 0 = no cap */
    const void *W_host;   /* pinned W^t [M x K]; may be NULL for a planning-only call */
    void *dW_host;        /* pinned dW^t [M x K]; NULL if no backward will be run */
} zi_problem;

/* What a plan decided and what one pass costs (closed forms of the method). */
typedef struct {
    int64_t n;                 /* tile width M / N */
    uint64_t tile_bytes;       /* K * n * 2: one weight tile, one host-to-device copy */
    uint64_t dw_tile_bytes;    /* K * n * 2 (or * 4 with ZI_FLAG_F32_OUT) */
    int32_t d;                 /* weight-tile slots in the ring */
    int32_t dw_slots;          /* separate gradient slots; 0 = dW_i written into W_i's slot */
    uint64_t ring_bytes;       /* device bytes the ring uses = workspace the context needs */
    double flops_fwd;          /* 2 T K M */
    double flops_bwd;          /* 4 T K M */
    double h2d_bytes_pass;     /* K * M * 2: every tile staged once per pass */
    double d2h_bytes_bwd;      /* dW write-back bytes of one backward */
    double ait_fwd;            /* flops_fwd / h2d bytes  (= T)  */
    double ait_bwd;            /* flops_bwd / h2d bytes  (= 2T) */
    double working_bytes_one;  /* layer bytes / N: one tile resident */
    double working_bytes_two;  /* twice that: one tile computing, one in flight */
    int32_t fwd_tile[2];       /* output rows (of T) x columns (of n) one workgroup of the
                                  forward product covers: 256 x 256, or 192 x 320 when
                                  that covers the tile width with clearly less padding */
    int32_t dw_tile[2];        /* the same for the gradient product dW_i^t [n x K]:
                                  256 x 256, or 320 x 192 */
} zi_plan_info;

typedef struct zi_plan zi_plan; /* library-owned, immutable after creation */
typedef struct zi_ctx zi_ctx;   /* library-owned: ring over caller workspace, events */

/* Plan the tiling of one linear operator.
 * The split is the method's core step (pwwt.cn article, section
 * "关键技术一：Memory-centric tiling", core idea and its worked example of a
 * 64K x 256K layer in N = 16 tiles: W is cut along its output dimension into N
 * tiles W_1..W_N of M/N columns, each small enough to sit in device memory on
 * its own); the working-memory figures follow the transformer-math page,
 * section "Memory-centric tiling: operators bigger than the device" (the layer's
 * bytes divided by the tile count for one resident tile, twice that with one
 * tile in flight beside it).
 * Validates the shapes (N | M, K % 8 == 0, n % 8 == 0, T >= 1), the dtype,
 * and the budget: the forward needs d weight slots; the backward additionally
 * needs somewhere to form dW_i -- up to two separate gradient slots if the
 * budget allows, otherwise dW_i is formed in W_i's own slot after the dX
 * product has consumed it.  ZI_ERR_BUDGET if even d weight slots do not fit.
 * W_host/dW_host are not dereferenced here (checked when a pass is enqueued).
 * out may be NULL (planning only); info may be NULL. */
zi_status zi_plan_tiles(const zi_problem *problem, zi_plan **out, zi_plan_info *info);
zi_status zi_plan_destroy(zi_plan *plan);

/* Smallest integer depth d >= t_fetch / t_layer, at least 1 (transformer-math
 * page, section "Prefetch depth": d >= t_fetch / t_layer, buffers d * layer). */
int32_t zi_prefetch_depth(double t_fetch_s, double t_layer_s);

/* Predicted timing of one pass from the ring's event recurrence: tile i's copy
 * starts when the link is free and its slot has been released by tile i-d;
 * its products start when the compute stream is free and the copy has landed
 * (pwwt.cn article, section "关键技术三：Overlap-Centric Design": the pipeline
 * runs at the pace of its slowest stage).  backward: 0 = forward pass,
 * 1 = backward pass, 2 = backward with the forward product recomputed per
 * tile, 3 = the same with the recomputed products of a dX pair (tiles 2j and
 * 2j + 1, see zi_tiled_linear_bwd_recompute) run together once tile 2j + 1
 * has landed, the order the context takes where one launch over both tiles
 * needs fewer rounds of workgroups than two (the model, priced by FLOP rates,
 * cannot tell that itself).  Rates: flop_rate in FLOP/s (products), link
 * rates in bytes/s. */
typedef struct {
    double t_pass_s;        /* first copy issued -> last product (and write-back) done */
    double t_compute_s;     /* sum of product times */
    double t_link_s;        /* sum of host-to-device copy times */
    double stall_frac;      /* 1 - t_compute / t_pass: compute-stream idle share */
    int32_t d_pages;        /* ceil(t_fetch(tile) / t_compute(tile)) */
} zi_prediction;
zi_status zi_plan_predict(const zi_plan *plan, int32_t backward, double flop_rate,
                          double h2d_bytes_per_s, double d2h_bytes_per_s, zi_prediction *out);

/* Rates measured at a few tile widths, for one T, K and dtype: at width n[j]
 * the forward, dX and dW products of one tile run at fwd[j], dx[j] and dw[j]
 * FLOP/s (dx or dw NULL: fwd's rates), and one tile's host-to-device and
 * device-to-host copies at h2d[j] and d2h[j] bytes/s (NULL: the link rates
 * passed to zi_plan_choose).  The widths are the candidates zi_plan_choose
 * considers; no rate is inferred between them. */
typedef struct {
    int32_t count;
    const int64_t *n;
    const double *fwd;
    const double *dx;
    const double *dw;
    const double *h2d;
    const double *d2h;
} zi_rate_curve;

/* One candidate tiling and its predicted step. */
typedef struct {
    int32_t N, d;          /* tile count and weight slots */
    int64_t n;             /* tile width M / N */
    int32_t dw_slots;      /* as zi_plan_info */
    uint64_t ring_bytes;   /* device bytes of the ring (<= the budget) */
    double t_fwd_s;        /* one forward pass on its own (as zi_plan_predict) */
    double t_bwd_s;        /* one backward pass on its own (0 with backward = 0) */
    double t_step_s;       /* a step (forward, then backward) among back-to-back
                              steps on one ring, whose copies run ahead into the
                              next pass: the third step's end minus the second's */
} zi_choice;

/* Choose the tile count N and the ring depth d of `problem` (its N and d are
 * ignored) under its device budget.  The page's trade-off (transformer-math
 * page, section "Memory-centric tiling: operators bigger than the device"):
 * more tiles shrink the resident bytes, layer bytes / N per slot, but make
 * each product smaller and slower; fewer tiles also lengthen the first copy,
 * which nothing hides.  Candidates: every width n[j] of `curve` with
 * M % n[j] == 0 and n[j] % 8 == 0, with d = 1 .. max_d, whose ring fits the
 * budget (the rules of zi_plan_tiles; with backward > 0 as for a plan with
 * dW_host, so gradient slots are sized in).  Each is priced with the ring's
 * event recurrence (as zi_plan_predict) using that width's measured rates,
 * over back-to-back steps of one forward pass plus, for backward = 1, 2 or 3,
 * one backward pass (2: with the forward product recomputed per tile; 3: as
 * zi_plan_predict's 3), the
 * ring's state carried from pass to pass.  The choice has the least t_step_s;
 * candidates within a relative 1e-9 of it count as equal, and then the
 * smaller ring, the smaller d and the smaller N win, in that order.
 * table: optional array of table_cap rows that receives every candidate in
 * the order considered (widths in curve order, d ascending); *table_len (if
 * not NULL) is set to the number of candidates, which may exceed table_cap.
 * ZI_ERR_ARG on a NULL problem, curve or out, non-positive or non-finite
 * rates, a width < 1, max_d < 1, or backward outside 0..3; ZI_ERR_SHAPE if
 * the problem's own shapes are invalid; ZI_ERR_BUDGET if no candidate fits. */
zi_status zi_plan_choose(const zi_problem *problem, const zi_rate_curve *curve, double h2d_bytes_per_s,
                         double d2h_bytes_per_s, int32_t backward, int32_t max_d, zi_choice *out,
                         zi_choice *table, int32_t table_cap, int32_t *table_len);

/* A context: the tile ring over caller-owned device workspace and three
 * caller-owned streams (products, host-to-device, device-to-host).  The ring
 * geometry (slot sizes, d, gradient slots) is taken from `plan`; any plan with
 * the same d whose tiles fit the slots may then run on this context, and
 * consecutive calls share the ring, so the copies of the next call's first
 * tiles overlap the previous call's last products.
 * workspace_dev: 256-byte aligned device memory of at least info.ring_bytes.
 * With at least zi_gelu_split_bytes() more past info.ring_bytes rounded up to
 * 256, the context also lets the GeLU forward (zi_tiled_linear_fwd_gelu) split
 * the reduction of a launch's last round of tiles when that round would keep
 * at most half of the compute units busy: each of its tiles is then taken by
 * two workgroups, one half of K each, and the second to finish adds the
 * other's fp32 sums and writes A and H.  The sums then group differently from
 * an unsplit launch (exact on integer-valued inputs, within the fp32 sum's
 * error otherwise); the forward's results do not depend on which half
 * finishes first, so a recomputation gives the same bits.
 * The context keeps no reference to the plan.  The first context created on
 * a device also builds that device's GeLU tables (H over every 16-bit A, read
 * by the forward GeLU epilogue) on compute_stream and waits for them;
 * ZI_ERR_HIP if that fails. */
/* Extra workspace bytes that let a context split the GeLU forward's last
 * round of tiles (see zi_ctx_create): for each of the context's two product
 * streams (the compute stream and the second one of zi_ctx_set_second_stream),
 * 128 tiles of two 256 x 256 fp32 half-sums (64 MiB) and their arrival
 * counters (512 B), which the context clears when it is created and every
 * launch leaves cleared.  A stream runs one launch at a time, so no two
 * launches use one set at once, and the results do not depend on whether
 * the second stream is used. */
uint64_t zi_gelu_split_bytes(void);

zi_status zi_ctx_create(const zi_plan *plan, void *workspace_dev, uint64_t workspace_bytes,
                        void *compute_stream, void *h2d_stream, void *d2h_stream,
                        zi_ctx **out);
/* Waits for outstanding work, then frees the context's events. */
zi_status zi_ctx_destroy(zi_ctx *ctx);

/* Forward: Y[:, i*n:(i+1)*n] = RNE(X W_i) for i = 0..N-1, tiles in ascending
 * order, fp32 accumulation, one rounding into the input format (or fp32 with
 * ZI_FLAG_F32_OUT).  X [T x K] and Y [T x M] (ldc = M) are device pointers,
 * 16-byte aligned.
 * This is the forward of the pages' tiled operator: each tile is brought into
 * device memory, multiplies X into its own output slice, and is released before
 * the next one needs its buffer (pwwt.cn article, section "关键技术一：Memory-
 * centric tiling", worked example: load W_i, compute Y_i, free W_i, go on with
 * W_{i+1}); the column slices need no communication between tiles and their
 * concatenation is Y (transformer-math page, section "Memory-centric tiling:
 * operators bigger than the device").  The copy of tile i + d runs under the
 * products of tile i (the same page, section "Prefetch depth: how far ahead the
 * pipeline must run").  ZI_ERR_ARG / ZI_ERR_ALIGN on NULL or misaligned
 * pointers, ZI_ERR_STATE when the plan does not fit the context,
 * ZI_ERR_NOT_PINNED when W_host is not page-locked; nothing is enqueued then. */
zi_status zi_tiled_linear_fwd(zi_ctx *ctx, const zi_plan *plan, const void *X_dev, void *Y_dev);

/* Forward with the GeLU of the feed-forward block fused into the epilogue
 * (the 1T model's FFN, transformer-math page, section "Memory-centric
 * tiling"): A = RNE(X W) and H = RNE(GeLU(A)), GeLU in the exact erf form
 * evaluated in fp64 on the stored (rounded) A and rounded once into the input
 * format, so H is the correctly rounded GeLU of A (the epilogue reads it from
 * a per-device table over every 16-bit A).  A and H are [T x M] device
 * buffers in the input format.  With ZI_FLAG_F32_OUT, A is written in fp32
 * instead (the fp32 accumulator itself: A_dev then holds 4-byte elements)
 * while H is still GeLU of A rounded to the input format, exactly as without
 * the flag. */
zi_status zi_tiled_linear_fwd_gelu(zi_ctx *ctx, const zi_plan *plan, const void *X_dev,
                                   void *A_dev, void *H_dev);

/* Backward: for each tile i in ascending order,
 *   dX (+)= dY[:, i*n:(i+1)*n] W_i^T   (fp32; the first tile overwrites dX),
 *   dW_i  = X^T dY[:, i*n:(i+1)*n]     (fp32 accumulation, one rounding into the
 *                                        input format, or fp32 with ZI_FLAG_F32_OUT),
 * and dW_i is copied to dW_host rows [i*n, (i+1)*n) on the write-back stream.
 * dX_dev: fp32 [T x K].  Requires a plan with dW_host.  dW_host must not be
 * read before zi_sync().
 * The backward stages every tile a second time (transformer-math page, section
 * "The FLOPs-per-byte test every tier must pass": the parameters climb to the
 * device once for the forward and once more for the backward), and each
 * tile's gradient leaves for host memory while the next tiles' products run
 * (pwwt.cn article, section "关键技术三：Overlap-Centric Design": the gradient
 * copies to the CPU overlap the backward's compute).  dX is summed over the
 * tiles in fp32, in ascending tile order.  Errors as zi_tiled_linear_fwd,
 * plus ZI_ERR_ARG without dW_host and ZI_ERR_NOT_PINNED when it is not
 * page-locked. */
zi_status zi_tiled_linear_bwd(zi_ctx *ctx, const zi_plan *plan, const void *X_dev,
                              const void *dY_dev, float *dX_dev);

/* Backward with the forward product recomputed from the same staged tile
 * (activation checkpointing: forward, recomputed forward and backward,
 * transformer-math page, section "The FLOPs-per-byte test every tier must
 * pass"): per tile, Yr[:, i*n:(i+1)*n] = RNE(X W_i) first, then the two
 * backward products as in zi_tiled_linear_bwd.  Where the backward runs the
 * dX products of tiles 2j and 2j + 1 as one launch (gradient slots, d >= 2,
 * n a multiple of 64) and one launch over both tiles' columns takes fewer
 * rounds of workgroups than two, the recomputed products of the pair are
 * that one launch, run once tile 2j + 1 has landed.  Yr is bit-identical to
 * the forward's Y either way.  Yr_dev: [T x M] device. */
zi_status zi_tiled_linear_bwd_recompute(zi_ctx *ctx, const zi_plan *plan, const void *X_dev,
                                        const void *dY_dev, float *dX_dev, void *Yr_dev);

/* dA = RNE(dH * GeLU'(A)) elementwise on the compute stream, GeLU'(a) =
 * Phi(a) + a phi(a) evaluated in fp32 on the stored A, once per 16-bit code
 * and device into a table that the kernel reads (the chain rule through the
 * block's GeLU; transformer-math page, section "Memory-centric tiling": the
 * 1T model's FFN).  dH: fp32 device, A and dA: device, input format
 * `dtype`; `count` elements each, 16-byte aligned pointers. */
zi_status zi_gelu_bwd(zi_ctx *ctx, int32_t dtype, const float *dH_dev, const void *A_dev,
                      void *dA_dev, int64_t count);

/* The same product left in fp32: dA_dev[i] = dH[i] * GeLU'(A[i]), the value
 * that zi_gelu_bwd rounds once into the input format (the form in which the
 * result can be compared without that rounding).  dA_dev: fp32 device. */
zi_status zi_gelu_bwd_f32(zi_ctx *ctx, int32_t dtype, const float *dH_dev, const void *A_dev,
                          float *dA_dev, int64_t count);

/* The forward of zi_tiled_linear_fwd for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same products, same kernel, same tile order, same results as
 * zi_tiled_linear_fwd (bit for bit), but with no context: each weight tile is
 * copied into a static device buffer that the library owns (one per device,
 * ZI_NOALLOC_SCRATCH_BYTES, held until the process ends) and multiplied
 * there, every copy and product on `stream` (a hipStream_t of the current
 * device, default priority, passed as void*; NULL: the null stream).  The call
 * allocates nothing: no device or host memory, no events; its first call on a
 * device looks up that device's buffer address once.
 * The copies do not overlap the products (one stream, one buffer); the ring of
 * a context is the overlapped form.  The caller passes X [T x K] and Y [T x M]
 * (16-byte aligned device pointers) and a plan whose W_host is pinned; the
 * plan's d, budget and dW_host are not used.  Returns at once; Y is complete
 * when `stream` is.  Calls that overlap on one device (two streams, two host
 * threads) share that device's buffer and race: serialise them.
 * ZI_ERR_BUDGET when one tile exceeds ZI_NOALLOC_SCRATCH_BYTES (split W into
 * more tiles), ZI_ERR_ARG / ZI_ERR_ALIGN on NULL or misaligned pointers,
 * ZI_ERR_NOT_PINNED when W_host is not page-locked: all before anything is
 * enqueued.  ZI_ERR_HIP when a copy or launch cannot be enqueued (earlier
 * tiles may then be enqueued already). */
#define ZI_NOALLOC_SCRATCH_BYTES (64ull << 20)
zi_status zi_tiled_linear_fwd_noalloc(const zi_plan *plan, const void *X_dev, void *Y_dev, void *stream);

/* Wait for everything enqueued on the context's three streams (and the
 * second product stream, if set) and for the host optimizers attached to it;
 * return the first error, which stays with the context (sticky).  The passes
 * only enqueue work so that the copies of later tiles run ahead of the
 * products (transformer-math page, section "Prefetch depth: how far ahead the
 * pipeline must run"; pwwt.cn article, section "关键技术三：Overlap-Centric
 * Design"); this is the one point at which the host waits for them.  After
 * ZI_OK every output of the enqueued passes, device and host, may be read.
 * How far ahead a caller enqueues is its own choice, but keep it to about one
 * training step: with many steps of passes enqueued at once the HIP runtime
 * was seen, after a while, to carry the tile copies out as copy kernels that
 * take compute units from the products (steps 15-40 % longer), and with two
 * or more whole steps in flight to stall write-backs; enqueueing a step once
 * the previous one has reached its middle kept the feed-forward block's steps
 * steady.  For a single operator whose step is one forward and one backward,
 * enqueueing the next step once the forward had run slowed the write-backs of
 * the step in flight, while a few steps enqueued at once did not. */
zi_status zi_sync(zi_ctx *ctx);

/* Per-context timing (off by default).  When on, every kernel launch and
 * every copy is bracketed by timing events; zi_ctx_stats() (after zi_sync)
 * reports the totals since the last reset. */
#define ZI_STATS_KERNELS 16
/* One kernel: a product (or the GeLU backward) at one launch shape.  Launches
 * of different roles that run the same kernel on the same shape (a forward
 * product and its recomputation, for instance) share an entry. */
typedef struct {
    char name[24];               /* "gemm_fwd", "gemm_fwd_gelu", "gemm_dx", "gemm_dw", "gelu_bwd" */
    int64_t rows, cols, red;     /* output rows and columns and reduction length of one launch
                                    (gelu_bwd: rows = elements, cols = red = 1) */
    int64_t launches;
    double ms;                   /* sum of event-measured durations of all launches */
    double flops;                /* algorithmic FLOPs of those launches (gelu_bwd: elements) */
    int64_t solo_launches;       /* launches no other kernel of the context overlapped */
    double solo_ms;              /* their summed durations: the kernel's time on its own */
} zi_kernel_stats;
typedef struct {
    int32_t kind_count;          /* number of valid entries below */
    char kind_name[8][24];       /* "gemm_fwd", "gemm_fwd_gelu", "gemm_dx", "gemm_dw", ... */
    int64_t launches[8];
    double kernel_ms[8];         /* sum of event-measured durations */
    double flops[8];             /* algorithmic FLOPs of those launches */
    int64_t h2d_copies, d2h_copies;
    double h2d_ms, d2h_ms;       /* sums of event-measured copy durations */
    double h2d_bytes, d2h_bytes;
    double span_ms;              /* first timed event -> last timed event */
    double compute_busy_ms;      /* time some kernel ran: the union of their intervals */
    int32_t kernel_count;        /* valid entries of kernel[] (launch shapes beyond the
                                    table's size are counted in the per-kind totals only) */
    zi_kernel_stats kernel[ZI_STATS_KERNELS];
} zi_stats;
zi_status zi_ctx_set_timing(zi_ctx *ctx, int32_t enable);

/* A second product stream (caller-owned, default priority, distinct from the
 * context's three; NULL: none).  A forward pass whose tile products take
 * fewer than 8 waves of workgroups (one 256 x 256 output block per compute
 * unit and wave) then launches the products of its odd tiles on it and of
 * its even tiles on the first: the tiles' outputs are disjoint, and the next
 * tile's workgroups fill the compute units that the last, partial wave of the
 * previous tile's leaves idle.  Backward passes keep
 * all their products on the first stream.  The second stream waits for
 * everything enqueued before
 * the pass, and the first stream waits for the second at the pass's end, so
 * the context's ordering toward later calls is unchanged.  With timing on,
 * kernel durations of overlapping products include the time they share the
 * device; compute_busy_ms counts the union of the kernels' intervals. */
zi_status zi_ctx_set_second_stream(zi_ctx *ctx, void *stream);

/* Debug aids for testing the ring's ordering and its stall accounting.
 * ZI_DEBUG_POISON: every weight slot is filled with 0xFF bytes (a NaN in
 * fp16, bf16 and fp32) on the copy stream just before a new tile is copied
 * into it, and every gradient slot on the product stream just before a new
 * dW is formed in it; a product that still read a released slot, or a
 * write-back that still read a gradient slot, would then see NaNs.
 * copy_delay_us: a host function on the copy stream sleeps that long before
 * every tile copy (at most 10 s), which slows the host link as far as the
 * ring can tell.  Both cost time; they are for tests.  ZI_ERR_ARG on unknown
 * flags or a longer delay. */
#define ZI_DEBUG_POISON 0x1u
/* ZI_DEBUG_DX_PER_TILE: dX products run one workgroup per 256 x 256 output
 * block, instead of one persistent workgroup per compute unit that takes
 * its blocks in turn and moves the next block's first copies and its C
 * under the stores of the last (the results are identical; the switch is
 * there to compare the two forms). */
#define ZI_DEBUG_DX_PER_TILE 0x2u
zi_status zi_ctx_set_debug(zi_ctx *ctx, uint32_t flags, uint32_t copy_delay_us);
zi_status zi_ctx_reset_stats(zi_ctx *ctx);
zi_status zi_ctx_stats(zi_ctx *ctx, zi_stats *out);

/* One timed launch or copy: what it was, and when it ran, in ms after the
 * first timed event of the context (since the last reset). */
typedef struct {
    int32_t what;                /* 0: kernel, 1: host-to-device copy, 2: device-to-host copy */
    int32_t kind;                /* kernels: index into zi_stats.kind_name; copies: -1 */
    int64_t rows, cols, red;     /* kernels: as zi_kernel_stats; copies: rows = bytes, cols = red = 0 */
    double start_ms, end_ms;
} zi_timed_rec;
/* The launches and copies timed since the last reset (zi_ctx_set_timing),
 * kernels in launch order, then copies in enqueue order, for attributing a
 * step's time to its products and copies step by step (the per-step view that
 * zi_ctx_stats' totals do not give).  Waits for the context's work like
 * zi_ctx_stats.  Writes at most cap records to out (out may be NULL with
 * cap = 0) and the total in *count.  ZI_ERR_ARG on a NULL ctx or count, a
 * negative cap, or a NULL out with cap > 0. */
zi_status zi_ctx_timed_records(zi_ctx *ctx, zi_timed_rec *out, int32_t cap, int32_t *count);

/* A new non-blocking stream of default priority, owned by the caller (release
 * with zi_stream_destroy).  The HIP runtime multiplexes streams onto a few
 * hardware queues; when the product stream and a copy stream share a queue, a
 * wait enqueued on the copy stream also holds back the products queued behind
 * it, and the ring loses its overlap.  Streams created one after another land
 * on distinct queues, so a context's streams are best created together,
 * rather than taken from a pool that other code has already drawn from. */
zi_status zi_stream_create(void **out);

/* A stream for the device-to-host copies whose work is confined to `n_cus`
 * compute units: the mask enables the lowest n_cus CU indices, which the HIP
 * runtime spreads round-robin over the XCCs, and it needs some in each, so
 * n_cus must be a positive multiple of the XCC count (8 on MI355X), at most
 * the CU count; ZI_ERR_ARG otherwise.
 * The HIP runtime may carry out a device-to-host hipMemcpyAsync as a copy
 * kernel on the stream's queue instead of a DMA engine; such a kernel's
 * workgroups occupy compute units for as long as the copy waits on the host
 * link, and a product kernel whose workgroup needs a whole compute unit
 * cannot start there meanwhile.  Confining the copy stream to a few compute
 * units bounds that loss.  Default priority.  The stream is owned by the
 * caller: release it with zi_stream_destroy after its last use. */
zi_status zi_copy_stream_create(int32_t n_cus, void **out);
zi_status zi_stream_destroy(void *stream);

/* ---- Adam on the host: the optimizer step beside the path -----------------
 *
 * The Adam update is elementwise, about 12 FLOPs against 24 bytes, so no tier
 * hides it behind GPU work and it runs on the CPU, next to the memory it
 * touches (transformer-math page, section "Applying the test: which state can
 * live where").  Its state is 12 bytes per parameter: an fp32 master weight
 * and two fp32 moments (GPU ZeRO-sharding page, section "The architecture:
 * every piece explained", and its offload paragraph: optimizer state and
 * update on the CPU); the updated 16-bit parameters become the next step's
 * resting copy (same page, section "End-to-end flow").
 *
 * One step of Adam (Kingma and Ba: bias-corrected moments, no weight decay),
 * per element, in fp32 and in this order:
 *   m      = beta1 * m + (1 - beta1) * g
 *   v      = beta2 * v + (1 - beta2) * (g * g)
 *   master = master - ((lr / (1 - beta1^step)) * m) / (sqrt(v * (1 / (1 - beta2^step))) + eps)
 *   w      = RNE of master in the 16-bit format
 * (the two bias factors are computed in double and rounded to fp32 once). */
typedef struct {
    float lr;     /* step size, finite and >= 0 */
    float beta1;  /* in [0, 1) */
    float beta2;  /* in [0, 1) */
    float eps;    /* >= 0 */
} zi_adam_hparams;

/* One Adam step over `count` elements, on `threads` host threads (<= 0: as
 * many as the process may run on).  grad: `count` gradients in the 16-bit
 * format `dtype` (grad_f32 = 0) or in fp32 (grad_f32 = 1); master, m, v: fp32
 * state, updated in place; w: `count` outputs in `dtype`.  Host memory of any
 * kind; no GPU is involved.  ZI_ERR_ARG on a NULL pointer (count > 0),
 * count < 0, step < 1, a bad dtype or hyperparameters out of range; nothing
 * is written then. */
zi_status zi_adam_update(const zi_adam_hparams *hp, int32_t dtype, int32_t grad_f32, int64_t step,
                         int64_t count, const void *grad, float *master, float *m, float *v, void *w,
                         int32_t threads);

/* An optimizer for one plan's weight.  master, m, v: caller-owned host arrays
 * of M * K fp32 each, in the layout of W^t (master holds the weights the
 * 16-bit W_host was rounded from, m and v the moments, zero before the first
 * step); the plan must have W_host and dW_host.  Every tile keeps its own
 * step count, starting at 1.
 * Attached to a context (zi_ctx_attach_adam), the optimizer updates tile i as
 * soon as dW_i has landed in dW_host -- on its own host threads, while the
 * GPU goes on with the next tiles -- and writes the new 16-bit tile into the
 * plan's W_host.  Any later copy of tile i to the device waits, on the
 * calling host thread, until that update is done; zi_sync() on the context
 * also waits for the updates queued so far.  Updates run in the order their
 * gradients were written back.  A failed update (a HIP error while waiting
 * for its gradient) is reported by zi_adam_wait() and zi_sync(). */
typedef struct zi_adam zi_adam;
zi_status zi_adam_create(const zi_plan *plan, const zi_adam_hparams *hp, float *master, float *m, float *v,
                         int32_t threads, zi_adam **out);
/* Waits for the queued updates, then releases the optimizer.  Detach it from
 * every context first (destroy the context, or attach NULL for its plan). */
zi_status zi_adam_destroy(zi_adam *adam);
/* Attach `adam` (or NULL: detach) to `plan` on `ctx`.  ZI_ERR_STATE if adam
 * was made for another plan. */
zi_status zi_ctx_attach_adam(zi_ctx *ctx, const zi_plan *plan, zi_adam *adam);
/* Wait until every queued update is done; the first error, if any. */
zi_status zi_adam_wait(zi_adam *adam);
/* Totals since creation: tiles updated, seconds the update threads were busy,
 * and host bytes the updates moved (28 per parameter with 16-bit gradients). */
typedef struct {
    int64_t tiles_done;
    double busy_s;
    double bytes;
} zi_adam_stats;
zi_status zi_adam_stats_get(zi_adam *adam, zi_adam_stats *out);

/* The NVMe tier: a weight read from a file on local storage instead of
 * W_host (pwwt.cn ZeRO-Infinity article, section "关键技术三：Overlap-Centric
 * Design": reads of later parameters from NVMe overlap the copies of nearer
 * ones to the GPU and the compute of the current one).  The file holds W^t
 * [M x K] of the plan's dtype from byte `offset` on, tile i at
 * offset + i * tile_bytes.  A reader thread reads tiles ahead of the passes
 * that use them into `staging` (>= 2) pinned buffers of one tile each, made
 * on first use on the current device, each read split over `threads`
 * positioned reads; with offset and tile_bytes multiples of 4096 the file is
 * read with O_DIRECT where the file system allows it.  The read-ahead
 * expects the tiles in ascending order, the first tile following the last
 * (every pass walks its tiles so); a pass that asks for another tile restarts
 * it there.  Attached to a context (zi_ctx_attach_source), every copy of the
 * plan's tiles to the device reads from the staging buffers: the calling host
 * thread waits, inside the pass call, until the tile's read is done (W_host
 * may then be NULL).  A source serves one context at a time.
 * ZI_ERR_IO if the file cannot be opened or is shorter than
 * offset + M * K * 2 bytes; ZI_ERR_ARG on NULL arguments, staging < 2 or
 * threads < 1.  Creating a source touches no GPU. */
typedef struct zi_file_source zi_file_source;
zi_status zi_file_source_create(const zi_plan *plan, const char *path, uint64_t offset, int32_t staging,
                                int32_t threads, zi_file_source **out);
/* Stops the reader, waits for every copy out of the staging buffers, frees
 * them and closes the file.  Detach the source from its context first.
 * ZI_ERR_STATE for a source under a tier that still exists. */
zi_status zi_file_source_destroy(zi_file_source *src);
/* Attach `src` (or NULL: detach) to `plan` on `ctx`.  ZI_ERR_STATE if the
 * source was made for another plan, or if an optimizer is attached to the
 * plan (it would update W_host, which the passes would no longer read). */
zi_status zi_ctx_attach_source(zi_ctx *ctx, const zi_plan *plan, zi_file_source *src);
/* Read tile `tile` into host memory `dst` (tile_bytes; 4096-byte aligned for a
 * source that reads with O_DIRECT, else ZI_ERR_ALIGN), synchronously, with the
 * source's threads.  No GPU is involved.  ZI_ERR_IO on a failed read. */
zi_status zi_file_source_read(zi_file_source *src, int64_t tile, void *dst);
/* Totals since creation: tiles read for the passes, restarts of the
 * read-ahead (with on-demand reads, counted for the tier the source is in),
 * seconds spent reading, bytes read, seconds the passes waited for a read,
 * and whether the file is read with O_DIRECT. */
typedef struct {
    int64_t tiles_read;
    int64_t restarts;
    double read_s;
    double bytes;
    double wait_s;
    int32_t direct;
} zi_source_stats;
zi_status zi_file_source_stats_get(zi_file_source *src, zi_source_stats *out);

/* A tier of file sources read by one reader in the order the passes use
 * them (pwwt.cn ZeRO-Infinity article, section "关键技术三：Overlap-Centric
 * Design": the prefetcher follows the order in which the operators ran in
 * the first iteration).  The tier owns `staging` (>= 2) pinned buffers of
 * the largest tile of its sources and splits every read over `threads`
 * positioned reads.  During the first step the tier records the order of
 * the tile requests of all its sources and serves each on demand; the first
 * zi_tier_step() call ends the recording, and from then on the reader reads
 * ahead along that trace, across weights and across the end of a step into
 * the next.  A request the trace does not predict restarts the read-ahead at
 * its next place in the trace, or is read on demand.  A standalone source
 * reads ahead with a tier of its own whose trace is its tiles in order.
 * The buffers also cache the files in host memory: a tile a buffer still
 * holds is served without a read.  A read takes a buffer no pending request
 * waits for, preferring an empty one, else the one whose tile the trace needs
 * again latest (the eviction that keeps the fewest reads when the order of
 * future requests is known; Belady, 1966).  With as many buffers as a source
 * has tiles, its weight is read once and then served from host memory. */
typedef struct zi_tier zi_tier;
zi_status zi_tier_create(int32_t staging, int32_t threads, zi_tier **out);
/* Put `src` under the tier; before the source or the tier is first used.
 * ZI_ERR_STATE if the source already has a tier or the tier has started. */
zi_status zi_tier_add(zi_tier *tier, zi_file_source *src);
/* Mark the end of a step (after its passes are enqueued).  The first call
 * fixes the trace; later calls check that the step ended where the trace
 * does and otherwise restart the read-ahead at the trace's start. */
zi_status zi_tier_step(zi_tier *tier);
/* Stops the reader, waits for every copy out of the staging buffers and
 * frees them; the sources are then standalone again.  Detach the sources
 * from their context first; destroy the tier before its sources. */
zi_status zi_tier_destroy(zi_tier *tier);
typedef struct {
    int64_t trace_len;     /* requests per step (so far, while recording) */
    int64_t steps;         /* zi_tier_step calls */
    int64_t tiles_read;
    int64_t restarts;      /* read-ahead restarted at another trace position */
    int64_t demand_reads;  /* requests read on demand (all of the first step's) */
    int64_t hits;          /* requests served by a buffer that still held the tile */
    double read_s, bytes, wait_s;
} zi_tier_stats;
zi_status zi_tier_stats_get(zi_tier *tier, zi_tier_stats *out);
/* The recorded trace, one id per request: (index of the source in the order
 * it was added) << 32 | tile.  *len receives the trace's length; up to cap
 * ids are written (ids may be NULL to ask for the length).  ZI_ERR_STATE
 * while the first step is still being recorded. */
zi_status zi_tier_trace_get(zi_tier *tier, int64_t *ids, int64_t cap, int64_t *len);
/* The tier's buffer policy applied to a trace of item ids without files or
 * threads, for choosing a buffer count: before each request the read-ahead
 * fills its window (up to `window` requests ahead, 1 <= window <= buffers; a
 * tile a buffer holds is assigned without a read, else it is read into the
 * buffer the policy picks), then the request takes its buffer.
 * reads_per_step[k] receives the reads of step k (steps entries; step 0
 * starts empty).  The tier's reads run at most `buffers` requests ahead; a
 * reader held back by the disk runs only one or two ahead and keeps the other
 * buffers as cache, and window = 1 gives the offline optimum of buffers - 1
 * slots or better.  No GPU is involved.  ZI_ERR_ARG on an empty trace,
 * buffers < 2, a window outside 1..buffers or steps < 1. */
zi_status zi_tier_simulate_reads(const int64_t *trace, int64_t len, int32_t buffers, int32_t window, int32_t steps,
                                 int64_t *reads_per_step);

/* Page-locked host memory (hipHostMalloc) for W^t / dW^t; 4096-byte aligned. */
zi_status zi_host_alloc(uint64_t bytes, void **out);
zi_status zi_host_free(void *ptr);

/* Text of the calling thread's most recent error ("" if none). */
const char *zi_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t zi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZI_H */
