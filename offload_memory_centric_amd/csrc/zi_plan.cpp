// zi_plan.cpp -- planning of a tiled linear operator and the ring's timing model.
//
// Host-only code: nothing here touches the GPU, so all of it runs (and is
// tested) without one.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/zi.h"
#include "zi_host.h"
#include "zi_internal.h"

namespace zi {

static uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

zi_status plan_validate_and_fill(const zi_problem *p, zi_plan_info *info, bool with_grad) {
    if (!p) return fail(ZI_ERR_ARG, "problem is NULL");
    if (p->dtype != ZI_F16 && p->dtype != ZI_BF16)
        return fail(ZI_ERR_ARG, "dtype must be ZI_F16 (1) or ZI_BF16 (2), got %d", p->dtype);
    if (p->flags & ~ZI_FLAG_F32_OUT) return fail(ZI_ERR_ARG, "unknown flags 0x%x", p->flags);
    if (p->T < 1 || p->K < 1 || p->M < 1)
        return fail(ZI_ERR_SHAPE, "T, K, M must be >= 1 (got %lld, %lld, %lld)", (long long)p->T,
                    (long long)p->K, (long long)p->M);
    if (p->N < 1) return fail(ZI_ERR_SHAPE, "N must be >= 1 (got %d)", p->N);
    if (p->d < 1) return fail(ZI_ERR_ARG, "prefetch depth d must be >= 1 (got %d)", p->d);
    if (p->M % p->N)
        return fail(ZI_ERR_SHAPE, "N = %d does not divide M = %lld", p->N, (long long)p->M);
    if (p->K % 8) return fail(ZI_ERR_SHAPE, "K = %lld is not a multiple of 8", (long long)p->K);
    const int64_t n = p->M / p->N;
    if (n % 8) return fail(ZI_ERR_SHAPE, "tile width n = M/N = %lld is not a multiple of 8", (long long)n);
    // The kernels address a 256-row panel of any operand with 32-bit offsets
    // below 1 GiB (256 rows x ld x 2 B), and count tiles in int.
    if (p->T > (int64_t)1 << 30 || p->K > (int64_t)1 << 21 || p->M > (int64_t)1 << 21)
        return fail(ZI_ERR_SHAPE, "extent too large (T <= 2^30, K and M <= 2^21)");

    const bool f32 = (p->flags & ZI_FLAG_F32_OUT) != 0;
    const uint64_t tile = (uint64_t)p->K * (uint64_t)n * 2u;
    const uint64_t dw_tile = (uint64_t)p->K * (uint64_t)n * (f32 ? 4u : 2u);
    const uint64_t slot = round_up(tile, 256);
    const uint64_t dw_slot = round_up(dw_tile, 256);
    const uint64_t budget = p->device_budget_bytes;

    const uint64_t w_ring = (uint64_t)p->d * slot;
    if (budget && w_ring > budget)
        return fail(ZI_ERR_BUDGET, "%d weight slots of %llu B need %llu B > budget %llu B", p->d,
                    (unsigned long long)slot, (unsigned long long)w_ring, (unsigned long long)budget);
    // Gradient slots: two for full-duplex write-back when the budget allows,
    // else one, else form dW_i inside W_i's slot (only if it fits there).
    int dw_slots = 2;
    if (budget) {
        const uint64_t left = budget - w_ring;
        dw_slots = (int)std::min<uint64_t>(2, left / dw_slot);
    }
    if (dw_slots == 0 && dw_tile > slot) {
        if (with_grad)
            return fail(ZI_ERR_BUDGET,
                        "no room for a gradient slot and an fp32 gradient tile does not fit a weight slot");
    }
    // A forward-only plan needs no gradient slot at all.
    if (!with_grad) dw_slots = 0;

    zi_plan_info o;
    memset(&o, 0, sizeof(o));
    o.n = n;
    o.tile_bytes = tile;
    o.dw_tile_bytes = dw_tile;
    o.d = p->d;
    o.dw_slots = dw_slots;
    o.ring_bytes = w_ring + (uint64_t)dw_slots * dw_slot;
    const double T = (double)p->T, K = (double)p->K, M = (double)p->M;
    o.flops_fwd = 2.0 * T * K * M;
    o.flops_bwd = 4.0 * T * K * M;
    o.h2d_bytes_pass = K * M * 2.0;
    o.d2h_bytes_bwd = K * M * (f32 ? 4.0 : 2.0);
    o.ait_fwd = o.flops_fwd / o.h2d_bytes_pass;
    o.ait_bwd = o.flops_bwd / o.h2d_bytes_pass;
    o.working_bytes_one = o.h2d_bytes_pass / (double)p->N;
    o.working_bytes_two = 2.0 * o.working_bytes_one;
    gemm_tile(GemmOp::Fwd, p->T, n, &o.fwd_tile[0], &o.fwd_tile[1]);
    gemm_tile(GemmOp::Dw, n, p->K, &o.dw_tile[0], &o.dw_tile[1]);
    *info = o;
    return ZI_OK;
}

// ---- timing model -----------------------------------------------------------------

// Event recurrence of passes over the ring, mirroring the enqueue order of
// the stager: copy j waits for the link and for the release of its slot by
// the tile staged d copies earlier (in this pass or the previous one); the
// products of tile j wait for the compute stream and the copy; dW_j waits for
// its gradient slot's previous write-back.  The state carries from one pass to
// the next as the context's ring does.
struct RingState {
    std::vector<double> wfree, dwfree;
    int64_t seq = 0, dw_seq = 0;
    double link = 0.0, comp = 0.0, back = 0.0;
    RingState(int d, int dw_slots) : wfree(d, 0.0), dwfree(dw_slots > 0 ? dw_slots : 1, 0.0) {}
};

static void run_pass(RingState &st, const PassModel &m, double *busy, double *linkbusy) {
    const int N = m.N, d = m.d;
    for (int i = 0; i < N; ++i) {
        const int s = (int)((st.seq + i) % d);
        const double cs = std::max(st.link, st.wfree[s]);
        const double ready = cs + m.t_h2d;
        st.link = ready;
        *linkbusy += m.t_h2d;
        const double start = std::max(st.comp, ready);
        if (!m.backward) {
            st.comp = start + m.t_fwd;
            *busy += m.t_fwd;
            st.wfree[s] = st.comp;
            continue;
        }
        // recompute (optional) and dX read the weight slot
        if (m.pairs) {
            // tile 2j: recompute and dW only, its slot stays taken; tile 2j+1:
            // recompute, then dX over both, which releases both slots.  With
            // re_pairs tile 2j has only its dW, and tile 2j+1 recomputes both.
            const bool first = i % 2 == 0 && i + 1 < N;
            const bool second = i % 2 == 1;
            const double t_re = !m.re_pairs ? m.t_recompute : first ? 0.0 : second ? 2.0 * m.t_recompute : m.t_recompute;
            const double t_w = t_re + (first ? 0.0 : second ? 2.0 * m.t_dx : m.t_dx);
            const double after_w = start + t_w;
            *busy += t_w + m.t_dw;
            if (!first) {
                st.wfree[s] = after_w;
                if (second) st.wfree[(int)((st.seq + i - 1) % d)] = after_w;
            }
            const int ds = (int)((st.dw_seq + i) % m.dw_slots);
            const double dw_start = std::max(after_w, st.dwfree[ds]);
            st.comp = dw_start + m.t_dw;
            const double wb = std::max(st.back, st.comp) + m.t_d2h;
            st.back = wb;
            st.dwfree[ds] = wb;
            continue;
        }
        const double t_w = m.t_recompute + m.t_dx;
        const double after_w = start + t_w;
        *busy += t_w + m.t_dw;
        if (m.dw_slots > 0) {
            st.wfree[s] = after_w;
            const int ds = (int)((st.dw_seq + i) % m.dw_slots);
            const double dw_start = std::max(after_w, st.dwfree[ds]);
            st.comp = dw_start + m.t_dw;
            const double wb = std::max(st.back, st.comp) + m.t_d2h;
            st.back = wb;
            st.dwfree[ds] = wb;
        } else {
            st.comp = after_w + m.t_dw;
            const double wb = std::max(st.back, st.comp) + m.t_d2h;
            st.back = wb;
            st.wfree[s] = wb;  // dW_i lives in W_i's slot until written back
        }
    }
    st.seq += N;
    if (m.backward) st.dw_seq += N;
}

bool pairs_apply(int N, int d, int dw_slots, int64_t n) {
    return dw_slots > 0 && d >= 2 && N >= 2 && n % kPairStep == 0;
}

Prediction simulate_pass(const PassModel &m) {
    Prediction r;
    RingState st(m.d, m.dw_slots);
    double busy = 0.0, linkbusy = 0.0;
    run_pass(st, m, &busy, &linkbusy);
    r.t_pass = std::max(st.comp, st.back);
    r.t_compute = busy;
    r.t_link = linkbusy;
    r.stall = r.t_pass > 0 ? 1.0 - busy / r.t_pass : 0.0;
    return r;
}

double simulate_steady_step(const PassModel *passes, int count) {
    RingState st(passes[0].d, passes[0].dw_slots);
    double busy = 0.0, linkbusy = 0.0, prev = 0.0, cur = 0.0;
    for (int rep = 0; rep < 3; ++rep) {
        for (int k = 0; k < count; ++k) run_pass(st, passes[k], &busy, &linkbusy);
        prev = cur;
        cur = std::max(st.comp, st.back);
    }
    return cur - prev;
}

}  // namespace zi

using namespace zi;

extern "C" int32_t zi_prefetch_depth(double t_fetch_s, double t_layer_s) {
    if (!(t_layer_s > 0.0) || !(t_fetch_s >= 0.0)) return 1;
    const double r = t_fetch_s / t_layer_s;
    const double c = ceil(r);
    if (c < 1.0) return 1;
    if (c > 1e9) return 1000000000;
    return (int32_t)c;
}

extern "C" zi_status zi_plan_tiles(const zi_problem *problem, zi_plan **out, zi_plan_info *info) {
    clear_error();
    zi_plan_info tmp;
    zi_status st = plan_validate_and_fill(problem, &tmp, problem && problem->dW_host);
    if (st != ZI_OK) return st;
    if (info) *info = tmp;
    if (out) {
        zi_plan *p = new (std::nothrow) zi_plan;
        if (!p) return fail(ZI_ERR_ARG, "out of host memory");
        p->prob = *problem;
        p->info = tmp;
        *out = p;
    }
    return ZI_OK;
}

extern "C" zi_status zi_plan_destroy(zi_plan *plan) {
    clear_error();
    delete plan;
    return ZI_OK;
}

extern "C" zi_status zi_plan_predict(const zi_plan *plan, int32_t backward, double flop_rate,
                                     double h2d_bps, double d2h_bps, zi_prediction *out) {
    clear_error();
    if (!plan || !out) return fail(ZI_ERR_ARG, "plan and out are required");
    if (!(flop_rate > 0) || !(h2d_bps > 0) || (backward && !(d2h_bps > 0)))
        return fail(ZI_ERR_ARG, "rates must be positive");
    if (backward < 0 || backward > 3) return fail(ZI_ERR_ARG, "backward must be 0, 1, 2 or 3");
    if (backward && !plan->prob.dW_host)
        return fail(ZI_ERR_STATE, "a backward needs a plan with dW_host");
    const zi_problem &p = plan->prob;
    const zi_plan_info &i = plan->info;
    PassModel m;
    m.N = p.N;
    m.d = p.d;
    m.backward = backward != 0;
    m.dw_slots = i.dw_slots;
    const double tile_flops = 2.0 * (double)p.T * (double)p.K * (double)i.n;
    m.t_h2d = (double)i.tile_bytes / h2d_bps;
    m.t_fwd = tile_flops / flop_rate;
    m.t_dx = tile_flops / flop_rate;
    m.t_dw = tile_flops / flop_rate;
    m.t_recompute = backward >= 2 ? tile_flops / flop_rate : 0.0;
    m.t_d2h = backward ? (double)i.dw_tile_bytes / d2h_bps : 0.0;
    m.pairs = backward && pairs_apply(m.N, m.d, m.dw_slots, i.n);
    m.re_pairs = backward == 3 && m.pairs;
    Prediction r = simulate_pass(m);
    out->t_pass_s = r.t_pass;
    out->t_compute_s = r.t_compute;
    out->t_link_s = r.t_link;
    out->stall_frac = r.stall;
    const double t_tile = backward ? (m.t_recompute + m.t_dx + m.t_dw) : m.t_fwd;
    out->d_pages = zi_prefetch_depth(m.t_h2d, t_tile);
    return ZI_OK;
}

extern "C" zi_status zi_plan_choose(const zi_problem *problem, const zi_rate_curve *curve, double h2d_bps,
                                    double d2h_bps, int32_t backward, int32_t max_d, zi_choice *out,
                                    zi_choice *table, int32_t table_cap, int32_t *table_len) {
    clear_error();
    if (table_len) *table_len = 0;
    if (!problem || !curve || !out) return fail(ZI_ERR_ARG, "problem, curve and out are required");
    if (backward < 0 || backward > 3) return fail(ZI_ERR_ARG, "backward must be 0, 1, 2 or 3");
    if (max_d < 1) return fail(ZI_ERR_ARG, "max_d must be >= 1 (got %d)", max_d);
    if (curve->count < 1 || !curve->n || !curve->fwd) return fail(ZI_ERR_ARG, "the curve has no samples");
    if (table_cap > 0 && !table) return fail(ZI_ERR_ARG, "table is NULL with table_cap > 0");
    auto rate_ok = [](double r) { return r > 0.0 && std::isfinite(r); };
    if (!(h2d_bps > 0.0) || !std::isfinite(h2d_bps) || (backward && (!(d2h_bps > 0.0) || !std::isfinite(d2h_bps))))
        return fail(ZI_ERR_ARG, "link rates must be positive and finite");
    for (int j = 0; j < curve->count; ++j) {
        if (curve->n[j] < 1) return fail(ZI_ERR_ARG, "curve width %d is %lld", j, (long long)curve->n[j]);
        if (!rate_ok(curve->fwd[j]) || (curve->dx && !rate_ok(curve->dx[j])) ||
            (curve->dw && !rate_ok(curve->dw[j])) || (curve->h2d && !rate_ok(curve->h2d[j])) ||
            (backward && curve->d2h && !rate_ok(curve->d2h[j])))
            return fail(ZI_ERR_ARG, "curve rates at width %lld must be positive and finite",
                        (long long)curve->n[j]);
    }
    const zi_problem &p = *problem;
    const double T = (double)p.T, K = (double)p.K;
    bool any_width = false, have = false;
    zi_choice best{};
    int32_t len = 0;
    for (int j = 0; j < curve->count; ++j) {
        const int64_t n = curve->n[j];
        if (p.M % n != 0 || n % 8 != 0) continue;
        if (p.M / n > (int64_t)INT32_MAX) continue;
        for (int32_t d = 1; d <= max_d; ++d) {
            zi_problem q = p;
            q.N = (int32_t)(p.M / n);
            q.d = d;
            zi_plan_info info;
            const zi_status st = plan_validate_and_fill(&q, &info, backward != 0);
            if (st == ZI_ERR_BUDGET) {
                any_width = true;
                clear_error();
                continue;
            }
            if (st != ZI_OK) return st;  // shapes, dtype or flags of the problem itself
            any_width = true;
            const double tile_flops = 2.0 * T * K * (double)n;
            const double r_fwd = curve->fwd[j];
            const double r_dx = curve->dx ? curve->dx[j] : r_fwd;
            const double r_dw = curve->dw ? curve->dw[j] : r_fwd;
            const double b_h2d = curve->h2d ? curve->h2d[j] : h2d_bps;
            const double b_d2h = curve->d2h ? curve->d2h[j] : d2h_bps;
            PassModel pm[2];
            pm[0].N = q.N;
            pm[0].d = d;
            pm[0].dw_slots = info.dw_slots;
            pm[0].t_h2d = (double)info.tile_bytes / b_h2d;
            pm[0].t_fwd = tile_flops / r_fwd;
            zi_choice c{};
            c.N = q.N;
            c.d = d;
            c.n = n;
            c.dw_slots = info.dw_slots;
            c.ring_bytes = info.ring_bytes;
            c.t_fwd_s = simulate_pass(pm[0]).t_pass;
            if (backward) {
                pm[1] = pm[0];
                pm[1].backward = true;
                pm[1].t_fwd = 0.0;
                pm[1].t_dx = tile_flops / r_dx;
                pm[1].t_dw = tile_flops / r_dw;
                pm[1].t_recompute = backward >= 2 ? tile_flops / r_fwd : 0.0;
                pm[1].t_d2h = (double)info.dw_tile_bytes / b_d2h;
                pm[1].pairs = pairs_apply(q.N, d, info.dw_slots, n);
                pm[1].re_pairs = backward == 3 && pm[1].pairs;
                c.t_bwd_s = simulate_pass(pm[1]).t_pass;
            }
            c.t_step_s = simulate_steady_step(pm, backward ? 2 : 1);
            if (table && len < table_cap) table[len] = c;
            ++len;
            bool better = !have;
            if (have) {
                const double tol = 1e-9 * best.t_step_s;
                if (c.t_step_s < best.t_step_s - tol) {
                    better = true;
                } else if (c.t_step_s <= best.t_step_s + tol) {
                    better = c.ring_bytes != best.ring_bytes ? c.ring_bytes < best.ring_bytes
                             : c.d != best.d                 ? c.d < best.d
                                                             : c.N < best.N;
                }
            }
            if (better) {
                best = c;
                have = true;
            }
        }
    }
    if (table_len) *table_len = len;
    if (!any_width)
        return fail(ZI_ERR_SHAPE, "no width of the curve divides M = %lld into tiles of a multiple of 8",
                    (long long)p.M);
    if (!have) return fail(ZI_ERR_BUDGET, "no candidate tiling fits the budget of %llu B",
                           (unsigned long long)p.device_budget_bytes);
    *out = best;
    return ZI_OK;
}
