// C ABI of the ring-attention rank-share library: validation, the per-shape
// plan cache (schedule + tile lists in device memory) and the per-step kernel
// launches.  See include/ring_attn.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <list>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <functional>
#include <numeric>
#include <queue>
#include <string>
#include <tuple>
#include <vector>

#include "abi_internal.h"
#include "kernel_args.h"
#include "planner.h"
#include "ring_attn.h"

namespace ra {
namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// Plans: the active steps of a rank in ring order, with the per-row visible
// key intervals and the forward / backward tile lists, uploaded once.
// ---------------------------------------------------------------------------

struct DevStep {
    int32_t s = 0, j = 0;
    int64_t pairs = 0;
    const int32_t* rng = nullptr;
    const int32_t* f_off = nullptr;
    const int32_t* f_mid = nullptr;
    const int32_t* f_ent = nullptr;
    const int32_t* f_order = nullptr;
    const int32_t* b_off = nullptr;
    const int32_t* b_mid = nullptr;
    const int32_t* b_ent = nullptr;
    const int32_t* b_order = nullptr;
    const int32_t* q_off = nullptr;   // dQ lists: 256-row query tiles over 64-key tiles
    const int32_t* q_mid = nullptr;
    const int32_t* q_ent = nullptr;
    const int32_t* q_order = nullptr;
    int32_t b_ne = 0;                 // entries of the b lists (dS tiles per batch, q head)
    const int32_t* d_off = nullptr;   // K4c lists: 256-row query tiles over 128-key tiles
    const int32_t* d_ent = nullptr;
    const int32_t* d_order = nullptr;
};

struct Plan {
    int device = 0;
    size_t bytes = 0;   // device bytes held
    int64_t S_pad = 0;
    int32_t nqt = 0;    // forward query tiles
    int32_t nkt_b = 0;  // backward key tiles
    int32_t nqt_dq = 0; // dQ query tiles
    int32_t max_ne = 0; // largest b_ne over the steps
    // One-launch forward over every active step (bf16): per 256-row query
    // tile, the 64-key tiles of all steps (unmasked ones first), entries
    // key tile | step << RING_STEP_SHIFT | partial << 31; the per-row
    // intervals of every step back to back; the KV block of every step.
    bool ring_ok = false;
    const int32_t* ring_off = nullptr;
    const int32_t* ring_mid = nullptr;
    const int32_t* ring_ent = nullptr;
    const int32_t* ring_order = nullptr;
    const int32_t* rng_all = nullptr;
    const int32_t* blk = nullptr;
    // persistent schedules of the one-launch forward (nullptr: one work item
    // per block): whole lists, and (when a list is split) with parts
    const int32_t* pers_off = nullptr;
    const int32_t* pers_items = nullptr;
    int32_t pers_blocks = 0;
    const int32_t* split_off = nullptr;
    const int32_t* split_items = nullptr;
    const int32_t* split_merge = nullptr;
    int32_t split_lists = 0;      // lists that are split (part-merge work-groups)
    int32_t split_slots = 0;      // part slots (parts of all split lists)
    int64_t split_bytes = 0;      // part buffer the split schedule needs (0: none)
    void* dbuf = nullptr;
    std::vector<DevStep> steps;
    ~Plan() {
        if (dbuf) {
            int cur = 0;
            if (hipGetDevice(&cur) == hipSuccess && cur != device) hipSetDevice(device);
            // kernels enqueued earlier on any stream may still read the plan
            (void)hipDeviceSynchronize();
            (void)hipFree(dbuf);
            if (cur != device) hipSetDevice(cur);
        }
    }
};

// Plan cache: least recently used first out, at most g_plan_limit plans.  A
// call holds its plan through a shared_ptr, so an eviction (or
// ring_attn_clear_cache) by another thread frees the plan only after that
// call has enqueued its kernels; the destructor then waits for the device.
// Evicted plans are retired and freed in batches of g_plan_limit (or by
// ring_attn_clear_cache), so that a caller with new document boundaries on
// every step waits for the device once per batch, not on every new plan.
std::mutex g_plan_mu;
std::list<std::pair<std::string, std::shared_ptr<Plan>>> g_plans;   // most recent first
std::map<std::string, decltype(g_plans)::iterator> g_plan_index;
int32_t g_plan_limit = 32;
std::vector<std::shared_ptr<Plan>> g_retired;

void evict_plans_locked(std::vector<std::shared_ptr<Plan>>& dropped) {
    while ((int64_t)g_plans.size() > g_plan_limit) {
        g_retired.push_back(std::move(g_plans.back().second));
        g_plan_index.erase(g_plans.back().first);
        g_plans.pop_back();
    }
    if ((int64_t)g_retired.size() >= g_plan_limit) {
        for (auto& r : g_retired) dropped.push_back(std::move(r));
        g_retired.clear();
    }
}

// Pinned host staging for plan uploads, grown as needed and reused (plans
// are built under g_plan_mu, one at a time), and a library stream per device
// that carries the copy: the host waits for the copy alone, not for work
// queued on the caller's stream.
struct Uploader {
    void* stage = nullptr;
    size_t cap = 0;
    std::map<int, hipStream_t> streams;
} g_up;

int upload_plan(int device, void* dst, const void* src, size_t bytes) {
    if (bytes > g_up.cap) {
        if (g_up.stage) (void)hipHostFree(g_up.stage);
        g_up.stage = nullptr;
        g_up.cap = 0;
        size_t want = std::max<size_t>(bytes, (size_t)1 << 20);
        if (hipHostMalloc(&g_up.stage, want, hipHostMallocDefault) != hipSuccess) {
            g_up.stage = nullptr;
            return RA_E_HIP;
        }
        g_up.cap = want;
    }
    hipStream_t& st = g_up.streams[device];
    if (st == nullptr && hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) {
        st = nullptr;
        return RA_E_HIP;
    }
    std::memcpy(g_up.stage, src, bytes);
    if (hipMemcpyAsync(dst, g_up.stage, bytes, hipMemcpyHostToDevice, st) != hipSuccess) return RA_E_HIP;
    return hipStreamSynchronize(st) == hipSuccess ? RA_OK : RA_E_HIP;
}

// Host image of a plan before upload: a list of int32 arrays.
struct HostArrays {
    std::vector<std::vector<int32_t>> arrays;
    size_t add(std::vector<int32_t>&& a) {
        arrays.push_back(std::move(a));
        return arrays.size() - 1;
    }
};

// Tile lists: list l holds entries off[l] .. off[l+1]-1, the FULL tiles first
// (in tile order) and from mid[l] on the PARTIAL ones, so that a kernel can run
// its unmasked and its masked loop without a per-tile branch.
void build_lists(const std::vector<int8_t>& kinds, int64_t nrows, int64_t ncols, bool by_row,
                 std::vector<int32_t>& off, std::vector<int32_t>& mid, std::vector<int32_t>& ent,
                 std::vector<int32_t>& order) {
    // by_row: lists per row tile (forward, per query tile over key tiles);
    // else lists per column tile (backward, per key tile over query tiles).
    const int64_t nlists = by_row ? nrows : ncols, nitems = by_row ? ncols : nrows;
    off.assign(nlists + 1, 0);
    mid.assign(nlists, 0);
    ent.clear();
    for (int64_t l = 0; l < nlists; ++l) {
        for (int pass = 0; pass < 2; ++pass) {
            const int8_t want = pass == 0 ? TILE_FULL : TILE_PARTIAL;
            if (pass == 1) mid[l] = (int32_t)ent.size();
            for (int64_t it = 0; it < nitems; ++it) {
                const int8_t k = by_row ? kinds[l * ncols + it] : kinds[it * ncols + l];
                if (k != want) continue;
                ent.push_back((int32_t)it | (k == TILE_PARTIAL ? (int32_t)0x80000000u : 0));
            }
        }
        off[l + 1] = (int32_t)ent.size();
    }
    order.resize(nlists);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        return off[x + 1] - off[x] > off[y + 1] - off[y];
    });
}

// Lists of the dQ-from-dS kernel, derived from the backward lists (per key
// tile over 64-row query tiles, entry index = dS tile): for each 256-row query
// tile, the 128-key tiles it meets in increasing order, each with the dS tile
// entry of the four 64-row quarters (-1 where a quarter sees none of the keys).
void build_ds_lists(const std::vector<int32_t>& boff, const std::vector<int32_t>& bent,
                    int64_t nkt, int64_t nqt256, std::vector<int32_t>& off,
                    std::vector<int32_t>& ent, std::vector<int32_t>& order) {
    std::vector<std::vector<std::array<int32_t, 5>>> per(nqt256);
    for (int64_t kt = 0; kt < nkt; ++kt)
        for (int32_t e = boff[kt]; e < boff[kt + 1]; ++e) {
            const int32_t qs = bent[e] & 0x7fffffff;
            auto& L = per[qs >> 2];
            if (L.empty() || L.back()[0] != kt) L.push_back({(int32_t)kt, -1, -1, -1, -1});
            L.back()[1 + (qs & 3)] = e;
        }
    off.assign(nqt256 + 1, 0);
    ent.clear();
    for (int64_t q = 0; q < nqt256; ++q) {
        for (const auto& x : per[q]) ent.insert(ent.end(), x.begin(), x.end());
        off[q + 1] = (int32_t)(ent.size() / 5);
    }
    order.resize(nqt256);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        return off[x + 1] - off[x] > off[y + 1] - off[y];
    });
}

// Blocks of the persistent forward on `device`: its CU count rounded down to
// a multiple of 8 (the XCDs); 0 when the count cannot be read.
int64_t persistent_blocks(int device) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return 0;
    return cus / 8 * 8;
}

// Bytes of the part buffer of a split schedule with `slots` part slots:
// partial outputs [slots][256 rows][d] fp32, then lse [slots][256 rows].
int64_t part_bytes(int64_t slots, int64_t d) {
    return round_up(slots * DQ_BQ * d * 4, 256) + round_up(slots * DQ_BQ * 4, 256);
}

// Whether the bf16 forward runs as one launch over every ring step: the
// entries hold the key tile in 20 bits and the step in 11.
bool ring_capable(const Geometry& g) {
    return g.dtype == RA_BF16 && g.nb <= RING_MAX_STEPS &&
           (g.Skv + DQ_BK - 1) / DQ_BK <= RING_MAX_KEY_TILES;
}

int build_plan(const Geometry& g, int device, std::unique_ptr<Plan>& out) {
    auto plan = std::make_unique<Plan>();
    plan->device = device;
    plan->S_pad = round_up(g.S, S_ALIGN);
    plan->nqt = (int32_t)((g.S + FWD_BQ - 1) / FWD_BQ);
    plan->nkt_b = (int32_t)((g.Skv + BWD_BK - 1) / BWD_BK);
    plan->nqt_dq = (int32_t)((g.S + DQ_BQ - 1) / DQ_BQ);
    const int64_t nkt_f = (g.Skv + FWD_BK - 1) / FWD_BK;
    const int64_t nqt_b = (g.S + BWD_BQ - 1) / BWD_BQ;

    HostArrays H;
    struct Idx { size_t rng, foff, fmid, fent, ford, boff, bmid, bent, bord, qoff, qmid, qent, qord,
                 doff, dent, dord; };
    std::vector<Idx> idx;
    std::vector<StepRanges> all(g.nb);
    // per active step: the forward lists of 256-row query tiles over 64-key
    // tiles (kept for the one-launch lists) and the per-row intervals
    std::vector<std::vector<int32_t>> q_off_h, q_mid_h, q_ent_h;
    std::vector<int32_t> rng_all_h, blk_h;
    int64_t total_pairs = 0;
    std::vector<int64_t> pq;
    rank_positions(g, g.r, pq);
    for (int32_t s = 0; s < g.nb; ++s) {
        step_ranges(g, s, all[s], &pq);
        total_pairs += all[s].pairs;
    }
    std::vector<int8_t> kinds;
    for (int32_t s = 0; s < g.nb; ++s) {
        const StepRanges& sr = all[s];
        // A step with no visible pair is skipped; under a causal basic layout
        // these are exactly the steps with s > rank.  Step 0 is kept when
        // nothing is visible at all so that the output is still written.
        if (sr.pairs == 0 && !(s == 0 && total_pairs == 0)) continue;
        DevStep ds;
        ds.s = s;
        ds.j = sr.j;
        ds.pairs = sr.pairs;
        std::vector<int32_t> rng(2 * plan->S_pad, 0);
        for (int64_t i = 0; i < g.S; ++i) {
            rng[2 * i] = sr.a[i];
            rng[2 * i + 1] = sr.b[i];
        }
        Idx ix;
        rng_all_h.insert(rng_all_h.end(), rng.begin(), rng.end());
        blk_h.push_back(sr.j);
        ix.rng = H.add(std::move(rng));
        std::vector<int32_t> off, mid, ent, order;
        // the 128-row forward lists serve the fp32 kernel only (the bf16
        // forward uses the 256-row lists below)
        if (g.dtype == RA_BF16) {
            off.clear();
            mid.clear();
            ent.clear();
            order.clear();
        } else {
            classify(sr, g.S, g.Skv, FWD_BQ, FWD_BK, kinds);
            build_lists(kinds, plan->nqt, nkt_f, true, off, mid, ent, order);
        }
        ix.foff = H.add(std::move(off));
        ix.fmid = H.add(std::move(mid));
        ix.fent = H.add(std::move(ent));
        ix.ford = H.add(std::move(order));
        classify(sr, g.S, g.Skv, BWD_BQ, BWD_BK, kinds);
        build_lists(kinds, nqt_b, plan->nkt_b, false, off, mid, ent, order);
        {
            std::vector<int32_t> doff, dent, dord;
            build_ds_lists(off, ent, plan->nkt_b, plan->nqt_dq, doff, dent, dord);
            ix.doff = H.add(std::move(doff));
            ix.dent = H.add(std::move(dent));
            ix.dord = H.add(std::move(dord));
        }
        ds.b_ne = (int32_t)ent.size();
        plan->max_ne = std::max(plan->max_ne, ds.b_ne);
        ix.boff = H.add(std::move(off));
        ix.bmid = H.add(std::move(mid));
        ix.bent = H.add(std::move(ent));
        ix.bord = H.add(std::move(order));
        classify(sr, g.S, g.Skv, DQ_BQ, DQ_BK, kinds);
        build_lists(kinds, plan->nqt_dq, (g.Skv + DQ_BK - 1) / DQ_BK, true, off, mid, ent, order);
        q_off_h.push_back(off);
        q_mid_h.push_back(mid);
        q_ent_h.push_back(ent);
        ix.qoff = H.add(std::move(off));
        ix.qmid = H.add(std::move(mid));
        ix.qent = H.add(std::move(ent));
        ix.qord = H.add(std::move(order));
        plan->steps.push_back(ds);
        idx.push_back(ix);
    }
    // The one-launch forward lists: for each query tile, the unmasked entries
    // of every step, then the masked ones.  The steps go in one order for
    // every query tile, the steps with the most visible pairs first (ties in
    // ring order), key tiles ascending within a step: the work-groups of a
    // head (which share an XCD's L2) then start on the same K/V tiles and
    // stay in step through the blocks every query tile sees whole, instead of
    // being offset by the query-tile-dependent part of the diagonal step.
    // The order changes only the rounding of the running sums.
    size_t i_roff = 0, i_rmid = 0, i_rent = 0, i_rord = 0, i_rng_all = 0, i_blk = 0, i_poff = 0,
           i_pitems = 0, i_soff = 0, i_sitems = 0, i_smerge = 0;
    const int64_t n_active = (int64_t)plan->steps.size();
    plan->ring_ok = ring_capable(g) && n_active <= RING_MAX_STEPS;
    if (plan->ring_ok) {
        const int64_t nq = plan->nqt_dq;
        std::vector<int32_t> roff(nq + 1, 0), rmid(nq, 0), rent, rord(nq);
        std::vector<int64_t> step_order(n_active);
        std::iota(step_order.begin(), step_order.end(), 0);
        std::stable_sort(step_order.begin(), step_order.end(), [&](int64_t x, int64_t y) {
            return plan->steps[x].pairs > plan->steps[y].pairs;
        });
        for (int64_t q = 0; q < nq; ++q) {
            for (int pass = 0; pass < 2; ++pass) {
                if (pass == 1) rmid[q] = (int32_t)rent.size();
                for (const int64_t st : step_order) {
                    const auto& off = q_off_h[st];
                    const int32_t a = pass == 0 ? off[q] : q_mid_h[st][q];
                    const int32_t b = pass == 0 ? q_mid_h[st][q] : off[q + 1];
                    for (int32_t e = a; e < b; ++e) {
                        const int32_t kt = q_ent_h[st][e] & 0x7fffffff;
                        rent.push_back(kt | (int32_t)(st << RING_STEP_SHIFT) |
                                       (pass == 1 ? (int32_t)0x80000000u : 0));
                    }
                }
            }
            roff[q + 1] = (int32_t)rent.size();
        }
        std::iota(rord.begin(), rord.end(), 0);
        std::stable_sort(rord.begin(), rord.end(), [&](int32_t x, int32_t y) {
            return roff[x + 1] - roff[x] > roff[y + 1] - roff[y];
        });
        PersSchedule plain, cut;
        persistent_schedule(persistent_blocks(device), (int64_t)g.B * g.Hq, roff, rmid, rord, false, plain);
        if (!plain.off.empty()) {
            plan->pers_blocks = (int32_t)plain.off.size() - 1;
            i_poff = H.add(std::move(plain.off));
            i_pitems = H.add(std::move(plain.items));
            persistent_schedule(persistent_blocks(device), (int64_t)g.B * g.Hq, roff, rmid, rord, true, cut);
            // split only where the cut shortens the busiest block by more than
            // the part merge costs (about 12 us, some 70 cost units)
            if (cut.slots > 0 && cut.makespan + 70 < plain.makespan * 99 / 100) {
                plan->split_lists = (int32_t)cut.merge.size() / 3;
                plan->split_slots = cut.slots;
                plan->split_bytes = part_bytes(cut.slots, g.d);
                i_soff = H.add(std::move(cut.off));
                i_sitems = H.add(std::move(cut.items));
                i_smerge = H.add(std::move(cut.merge));
            }
        }
        i_roff = H.add(std::move(roff));
        i_rmid = H.add(std::move(rmid));
        i_rent = H.add(std::move(rent));
        i_rord = H.add(std::move(rord));
        i_rng_all = H.add(std::move(rng_all_h));
        i_blk = H.add(std::move(blk_h));
    }
    // One device allocation holding every array, each 256-byte aligned.
    std::vector<size_t> offs(H.arrays.size());
    size_t total = 0;
    for (size_t i = 0; i < H.arrays.size(); ++i) {
        offs[i] = total;
        total += round_up((int64_t)std::max<size_t>(1, H.arrays[i].size()) * 4, 256);
    }
    plan->bytes = total;
    std::vector<unsigned char> img(total, 0);
    for (size_t i = 0; i < H.arrays.size(); ++i)
        if (!H.arrays[i].empty())
            std::memcpy(img.data() + offs[i], H.arrays[i].data(), H.arrays[i].size() * 4);
    if (hipMalloc(&plan->dbuf, total) != hipSuccess) {
        plan->dbuf = nullptr;
        return RA_E_HIP;
    }
    if (const int rc = upload_plan(device, plan->dbuf, img.data(), total); rc != RA_OK) return rc;
    auto P = [&](size_t i) { return (const int32_t*)((unsigned char*)plan->dbuf + offs[i]); };
    for (size_t k = 0; k < plan->steps.size(); ++k) {
        DevStep& d = plan->steps[k];
        d.rng = P(idx[k].rng);
        d.f_off = P(idx[k].foff);
        d.f_mid = P(idx[k].fmid);
        d.f_ent = P(idx[k].fent);
        d.f_order = P(idx[k].ford);
        d.b_off = P(idx[k].boff);
        d.b_mid = P(idx[k].bmid);
        d.b_ent = P(idx[k].bent);
        d.b_order = P(idx[k].bord);
        d.q_off = P(idx[k].qoff);
        d.q_mid = P(idx[k].qmid);
        d.q_ent = P(idx[k].qent);
        d.q_order = P(idx[k].qord);
        d.d_off = P(idx[k].doff);
        d.d_ent = P(idx[k].dent);
        d.d_order = P(idx[k].dord);
    }
    if (plan->ring_ok) {
        plan->ring_off = P(i_roff);
        plan->ring_mid = P(i_rmid);
        plan->ring_ent = P(i_rent);
        plan->ring_order = P(i_rord);
        plan->rng_all = P(i_rng_all);
        plan->blk = P(i_blk);
        if (plan->pers_blocks > 0) {
            plan->pers_off = P(i_poff);
            plan->pers_items = P(i_pitems);
        }
        if (plan->split_lists > 0) {
            plan->split_off = P(i_soff);
            plan->split_items = P(i_sitems);
            plan->split_merge = P(i_smerge);
        }
    }
    out = std::move(plan);
    return RA_OK;
}

// The cached plan of this geometry on the current device; with build = false
// a missing plan is RA_E_NO_PLAN instead of being built (no device allocation).
// A plan is not built while `stream` is being captured into a graph (the
// build allocates and copies): RA_E_NO_PLAN then too.
int get_plan(const Geometry& g, std::shared_ptr<const Plan>* out, bool build, hipStream_t stream) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return RA_E_HIP;
    const std::string key = std::to_string(device) + "#" + plan_key(g);
    std::vector<std::shared_ptr<Plan>> dropped;   // freed after the lock is released
    {
        std::lock_guard<std::mutex> lock(g_plan_mu);
        auto it = g_plan_index.find(key);
        if (it != g_plan_index.end()) {
            g_plans.splice(g_plans.begin(), g_plans, it->second);   // now most recent
            *out = g_plans.front().second;
            return RA_OK;
        }
        if (!build) return RA_E_NO_PLAN;
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return RA_E_HIP;
        if (cap != hipStreamCaptureStatusNone) return RA_E_NO_PLAN;
        std::unique_ptr<Plan> p;
        const int rc = build_plan(g, device, p);
        if (rc != RA_OK) return rc;
        g_plans.emplace_front(key, std::shared_ptr<Plan>(std::move(p)));
        g_plan_index[key] = g_plans.begin();
        *out = g_plans.front().second;
        evict_plans_locked(dropped);
    }
    return RA_OK;
}

// ---------------------------------------------------------------------------
// Optional per-kernel event timing
// ---------------------------------------------------------------------------

enum KernelClass {
    KC_FWD = 0, KC_MERGE, KC_FINALIZE, KC_BWD_PRE, KC_BWD, KC_BWD_DQ, KC_BWD_DQ_DS, KC_BWD_POST,
    KC_FWD_PART_MERGE, KC_COUNT
};
const char* kClassNames[KC_COUNT] = {"fwd_step", "lse_merge", "finalize", "bwd_pre",  "bwd_step",
                                     "bwd_dq",   "bwd_dq_ds", "bwd_post", "fwd_part_merge"};

struct Timing {
    std::mutex mu;
    bool on = false;
    std::vector<std::tuple<int, hipEvent_t, hipEvent_t>> pending;
    std::vector<hipEvent_t> pool;
    int64_t launches[KC_COUNT] = {};
    double ms[KC_COUNT] = {};
} g_timing;

// Set while a call that may not allocate is running on this thread: the
// timing then uses pooled events only.
thread_local bool t_no_alloc = false;

hipEvent_t take_event() {
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    if (t_no_alloc) return nullptr;   // the launch then runs untimed
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
hipError_t timed(int cls, hipStream_t s, F&& launch) {
    bool on;
    {
        std::lock_guard<std::mutex> lock(g_timing.mu);
        on = g_timing.on;
    }
    if (!on) return launch();
    hipEvent_t a, b;
    {
        std::lock_guard<std::mutex> lock(g_timing.mu);
        a = take_event();
        b = take_event();
    }
    if (!a || !b) return launch();
    hipEventRecord(a, s);
    const hipError_t err = launch();
    hipEventRecord(b, s);
    std::lock_guard<std::mutex> lock(g_timing.mu);
    g_timing.pending.emplace_back(cls, a, b);
    return err;
}

int collect_timing() {
    std::lock_guard<std::mutex> lock(g_timing.mu);
    for (auto& [cls, a, b] : g_timing.pending) {
        if (hipEventSynchronize(b) != hipSuccess) return RA_E_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return RA_E_HIP;
        g_timing.launches[cls] += 1;
        g_timing.ms[cls] += ms;
        g_timing.pool.push_back(a);
        g_timing.pool.push_back(b);
    }
    g_timing.pending.clear();
    return RA_OK;
}

// ---------------------------------------------------------------------------

int64_t elem_bytes(const Geometry& g) { return g.dtype == RA_BF16 ? 2 : 4; }

int64_t fwd_workspace(const Geometry& g) {
    const int64_t S_pad = round_up(g.S, S_ALIGN);
    // the one-launch forward keeps the running result in registers
    if (g.merge_mode == RA_MERGE_FUSED && ring_capable(g)) return 0;
    if (g.merge_mode != RA_MERGE_SEPARATE) return round_up((int64_t)g.B * g.Hq * S_pad * g.d * 4, 256);
    const int64_t o = round_up((int64_t)g.B * g.S * g.Hq * g.d * 4, 256);
    return 2 * o + round_up((int64_t)g.B * g.Hq * g.S * 4, 256);
}

// Backward workspace: the per-row arrays lse2 and -Delta, [B, Hq, S_pad] fp32
// each, then the dQ accumulator [B, Hq, S_pad, d] fp32.
int64_t bwd_row_bytes(const Geometry& g) {
    return round_up((int64_t)g.B * g.Hq * round_up(g.S, S_ALIGN) * 4, 256);
}
int64_t bwd_workspace(const Geometry& g) {
    const int64_t S_pad = round_up(g.S, S_ALIGN);
    return 2 * bwd_row_bytes(g) + round_up((int64_t)g.B * g.Hq * S_pad * g.d * 4, 256);
}

// The dS tile store (optional part of the backward workspace, after the
// parts above): one tile of DS_TILE_ELEMS bf16 per (batch, q head, entry of a
// step's backward lists), sized for the step with the most entries.
int64_t ds_store_bytes(const Geometry& g, int64_t max_ne) {
    return round_up((int64_t)g.B * g.Hq * max_ne * DS_TILE_ELEMS * 2, 256);
}

// Largest entry count of the backward lists over the active steps, computed
// on the host exactly as the plan does (memoised per geometry).
int64_t host_max_ne(const Geometry& g) {
    static std::mutex mu;
    static std::map<std::string, int64_t> memo;
    const std::string key = plan_key(g);
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = memo.find(key);
        if (it != memo.end()) return it->second;
    }
    int64_t best = 0;
    StepRanges sr;
    std::vector<int8_t> kinds;
    std::vector<int64_t> pq;
    rank_positions(g, g.r, pq);
    for (int32_t s = 0; s < g.nb; ++s) {
        step_ranges(g, s, sr, &pq);
        if (sr.pairs == 0) continue;
        classify(sr, g.S, g.Skv, BWD_BQ, BWD_BK, kinds);
        const int64_t ne = std::count_if(kinds.begin(), kinds.end(),
                                         [](int8_t k) { return k != TILE_EMPTY; });
        best = std::max(best, ne);
    }
    std::lock_guard<std::mutex> lock(mu);
    if (memo.size() >= 256) memo.clear();   // bounded: one entry per geometry seen
    memo[key] = best;
    return best;
}

int check_support(const Geometry& g, bool bwd) {
    if (g.d != 64 && g.d != 128) return RA_E_UNSUPPORTED;
    // kernels address one batch entry of a block, and of q, with 32-bit offsets
    if ((int64_t)g.Skv * g.Hkv * g.d >= (1LL << 31) || (int64_t)g.S * g.Hq * g.d >= (1LL << 31))
        return RA_E_SHAPE;
    if (bwd && g.dtype != RA_BF16) return RA_E_UNSUPPORTED;
    return RA_OK;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? RA_OK : RA_E_HIP; }

}  // namespace
}  // namespace ra

using namespace ra;

extern "C" {

int ring_attn_version(void) { return 1; }

const char* ring_attn_strerror(int code) {
    switch (code) {
        case RA_OK: return "success";
        case RA_E_NULL: return "a required pointer is NULL";
        case RA_E_SHAPE: return "batch, heads, head_dim or seqlen out of range";
        case RA_E_WORLD: return "world < 1 or rank outside [0, world)";
        case RA_E_DIVISIBILITY: return "seqlen not divisible by world (2*world for zigzag)";
        case RA_E_CU_SEQLENS:
            return "cu_seqlens must start at 0, be non-decreasing and end at seqlen; "
                   "document lengths must be multiples of world (varlen ring, varlen "
                   "stripe) or of 2*world (varlen zigzag)";
        case RA_E_HEADS: return "heads_q is not a multiple of heads_kv";
        case RA_E_UNSUPPORTED: return "no kernel for this head_dim / dtype combination";
        case RA_E_WORKSPACE: return "workspace is NULL or smaller than required";
        case RA_E_LAYOUT: return "unknown layout, or batch != 1 with a varlen layout";
        case RA_E_HIP: return "the HIP runtime reported an error";
        case RA_E_ARG: return "an argument is out of range (or a NaN / infinite softmax scale)";
        case RA_E_NO_PLAN:
            return "no cached plan for this shape: an ordinary call outside graph capture builds it "
                   "(the no-allocation entry point and captured calls only use plans that exist)";
        case RA_E_SCRATCH:
            return "the call needs more scratch than the no-allocation entry point's static array";
        default: return "unknown error code";
    }
}

int64_t ring_attn_workspace_bytes(const ring_attn_desc* desc, int is_bwd) {
    Geometry g;
    const int rc = validate(desc, nullptr, &g, false);
    if (rc != RA_OK) return rc;
    return is_bwd ? bwd_workspace(g) : fwd_workspace(g);
}

int64_t ring_attn_bwd_ds_bytes(const ring_attn_desc* desc, const int32_t* cu) {
    try {
        Geometry g;
        const int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        return ds_store_bytes(g, host_max_ne(g));
    } catch (...) {
        return RA_E_ARG;
    }
}

int64_t ring_attn_fwd_split_bytes(const ring_attn_desc* desc) {
    if (!desc) return RA_E_NULL;
    if (desc->head_dim != 64 && desc->head_dim != 128) return RA_E_UNSUPPORTED;
    if (desc->dtype != RA_BF16 || desc->merge_mode != RA_MERGE_FUSED) return 0;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return RA_E_HIP;
    const int64_t nblk = persistent_blocks(device);
    return nblk > 0 ? part_bytes(nblk, desc->head_dim) : 0;   // no persistent schedule: no parts
}

int ring_attn_positions(const ring_attn_desc* desc, const int32_t* cu, int32_t rank,
                        int64_t* pos_out) {
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if (!pos_out) return RA_E_NULL;
        if (rank < 0 || rank >= g.D) return RA_E_WORLD;
        std::vector<int64_t> p;
        rank_positions(g, rank, p);
        std::memcpy(pos_out, p.data(), p.size() * sizeof(int64_t));
        return RA_OK;
    } catch (...) {
        return RA_E_ARG;
    }
}

int ring_attn_kv_positions(const ring_attn_desc* desc, const int32_t* cu, int32_t block,
                           int64_t* pos_out) {
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if (!pos_out) return RA_E_NULL;
        if (block < 0 || block >= g.nb) return RA_E_ARG;
        std::vector<int64_t> p;
        block_positions(g, block, p);
        std::memcpy(pos_out, p.data(), p.size() * sizeof(int64_t));
        return RA_OK;
    } catch (...) {
        return RA_E_ARG;
    }
}

int ring_attn_schedule(const ring_attn_desc* desc, const int32_t* cu, int32_t* block_out,
                       int64_t* pairs_out, int32_t* n_steps) {
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if (!block_out || !pairs_out || !n_steps) return RA_E_NULL;
        StepRanges sr;
        std::vector<int64_t> pq;
        rank_positions(g, g.r, pq);
        for (int32_t s = 0; s < g.nb; ++s) {
            step_ranges(g, s, sr, &pq);
            block_out[s] = sr.j;
            pairs_out[s] = sr.pairs;
        }
        *n_steps = g.nb;
        return RA_OK;
    } catch (...) {
        return RA_E_ARG;
    }
}

int ring_attn_tile_kinds(const ring_attn_desc* desc, const int32_t* cu, int32_t step,
                         int32_t tile_q, int32_t tile_k, int8_t* kinds_out) {
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if (!kinds_out) return RA_E_NULL;
        if (step < 0 || step >= g.nb || tile_q < 1 || tile_k < 1) return RA_E_ARG;
        StepRanges sr;
        step_ranges(g, step, sr);
        std::vector<int8_t> k;
        classify(sr, g.S, g.Skv, tile_q, tile_k, k);
        std::memcpy(kinds_out, k.data(), k.size());
        return RA_OK;
    } catch (...) {
        return RA_E_ARG;
    }
}

int ring_attn_lse_merge(float* out, float* lse, const float* out_j, const float* lse_j,
                        int32_t batch, int64_t seqlen, int32_t heads, int32_t head_dim,
                        void* stream) {
    if (!out || !lse || !out_j || !lse_j) return RA_E_NULL;
    if (batch < 0 || seqlen < 0 || heads < 0 || head_dim < 4 || head_dim % 4) return RA_E_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    return hip_rc(timed(KC_MERGE, s, [&] {
        return launch_lse_merge(out, lse, out_j, lse_j, batch, seqlen, heads, head_dim, s);
    }));
}

int ring_attn_fwd(const ring_attn_desc* desc, const void* q, const void* k, const void* v,
                  const int32_t* cu, void* out, float* lse, void* workspace,
                  size_t workspace_bytes, void* stream) {
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if ((rc = check_support(g, false)) != RA_OK) return rc;
        if (!q || !k || !v || !out || !lse) return RA_E_NULL;
        const int64_t need = fwd_workspace(g);
        if (need > 0 && (!workspace || (int64_t)workspace_bytes < need)) return RA_E_WORKSPACE;
        std::shared_ptr<const Plan> plan;
        if ((rc = get_plan(g, &plan, true, (hipStream_t)stream)) != RA_OK) return rc;
        hipStream_t s = (hipStream_t)stream;

        const int64_t eb = elem_bytes(g);
        const int64_t block_elems = (int64_t)g.B * g.Skv * g.Hkv * g.d;
        FwdArgs a{};
        a.q = q;
        a.lse = lse;
        a.out = out;
        a.B = g.B; a.S = (int32_t)g.S; a.Skv = (int32_t)g.Skv; a.Hq = g.Hq; a.Hkv = g.Hkv;
        // the bf16 kernel walks 256-row query tiles, the fp32 one 128-row tiles
        const bool bf16 = g.dtype == RA_BF16;
        a.nqt = bf16 ? plan->nqt_dq : plan->nqt;
        a.S_pad = (int32_t)plan->S_pad;
        a.total_work = g.B * g.Hq * a.nqt;
        a.scale_log2 = g.scale * 1.4426950408889634f;
        auto set_lists = [&](const DevStep& st) {
            a.rng = st.rng;
            a.t_off = bf16 ? st.q_off : st.f_off;
            a.t_mid = bf16 ? st.q_mid : st.f_mid;
            a.t_ent = bf16 ? st.q_ent : st.f_ent;
            a.t_order = bf16 ? st.q_order : st.f_order;
        };
        auto launch_step = [&](const FwdArgs& args) {
            return timed(KC_FWD, s, [&] {
                return g.dtype == RA_BF16 ? launch_fwd_bf16(args, g.d, s)
                                          : launch_fwd_f32(args, g.d, s);
            });
        };
        const size_t n = plan->steps.size();
        if (g.merge_mode == RA_MERGE_FUSED && plan->ring_ok) {
            // one launch over every active step, the merge carried in registers
            a.ring = 1;
            a.k = k;
            a.v = v;
            a.block_elems = block_elems;
            a.rng = plan->rng_all;
            a.rng_stride = (int32_t)(2 * plan->S_pad);
            a.blk = plan->blk;
            a.t_off = plan->ring_off;
            a.t_mid = plan->ring_mid;
            a.t_ent = plan->ring_ent;
            a.t_order = plan->ring_order;
            a.pers_off = plan->pers_off;
            a.pers_items = plan->pers_items;
            a.pers_blocks = plan->pers_blocks;
            a.mode = FWD_SOLO;
            // the split schedule when the workspace holds its part buffer
            const bool split = plan->split_lists > 0 && workspace != nullptr &&
                               (int64_t)workspace_bytes >= plan->split_bytes;
            if (!split) return hip_rc(launch_step(a));
            a.pers_off = plan->split_off;
            a.pers_items = plan->split_items;
            a.part_o = (float*)workspace;
            a.part_l = (float*)((unsigned char*)workspace +
                                round_up((int64_t)plan->split_slots * DQ_BQ * g.d * 4, 256));
            if ((rc = hip_rc(launch_step(a))) != RA_OK) return rc;
            PartMergeArgs m{};
            m.items = plan->split_merge;
            m.t_order = plan->ring_order;
            m.part_o = a.part_o;
            m.part_l = a.part_l;
            m.out = out;
            m.lse = lse;
            m.n_items = plan->split_lists;
            m.nqt = a.nqt;
            m.S = a.S;
            m.Hq = a.Hq;
            m.d = g.d;
            return hip_rc(timed(KC_FWD_PART_MERGE, s, [&] { return launch_fwd_part_merge(m, s); }));
        }
        if (g.merge_mode != RA_MERGE_SEPARATE) {   // one launch per step, merge in the epilogue
            a.o_run = (float*)workspace;
            for (size_t i = 0; i < n; ++i) {
                const DevStep& st = plan->steps[i];
                a.k = (const unsigned char*)k + st.j * block_elems * eb;
                a.v = (const unsigned char*)v + st.j * block_elems * eb;
                set_lists(st);
                a.mode = n == 1 ? FWD_SOLO : (i == 0 ? FWD_FIRST : (i + 1 == n ? FWD_LAST : FWD_MERGE));
                if ((rc = hip_rc(launch_step(a))) != RA_OK) return rc;
            }
        } else {
            const int64_t o_bytes = round_up((int64_t)g.B * g.S * g.Hq * g.d * 4, 256);
            float* o_run = (float*)workspace;
            float* o_j = (float*)((unsigned char*)workspace + o_bytes);
            float* l_j = (float*)((unsigned char*)workspace + 2 * o_bytes);
            for (size_t i = 0; i < n; ++i) {
                const DevStep& st = plan->steps[i];
                a.k = (const unsigned char*)k + st.j * block_elems * eb;
                a.v = (const unsigned char*)v + st.j * block_elems * eb;
                set_lists(st);
                a.mode = FWD_PARTIAL;
                a.o_part = i == 0 ? o_run : o_j;
                a.lse_part = i == 0 ? lse : l_j;
                if ((rc = hip_rc(launch_step(a))) != RA_OK) return rc;
                if (i > 0) {
                    rc = hip_rc(timed(KC_MERGE, s, [&] {
                        return launch_lse_merge(o_run, lse, o_j, l_j, g.B, g.S, g.Hq, g.d, s);
                    }));
                    if (rc != RA_OK) return rc;
                }
            }
            const int64_t nel = (int64_t)g.B * g.S * g.Hq * g.d;
            rc = hip_rc(timed(KC_FINALIZE, s, [&] {
                return launch_finalize(o_run, out, g.dtype == RA_BF16, nel, s);
            }));
            if (rc != RA_OK) return rc;
        }
        return RA_OK;
    } catch (...) {
        return RA_E_HIP;
    }
}

}  // extern "C"

namespace ra {

int bwd_impl(const ring_attn_desc* desc, const void* dout, const void* q, const void* k,
             const void* v, const void* out, const float* lse, const int32_t* cu, float* dq,
             float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream,
             bool build_plan) {
    struct NoAllocScope {   // no event creation in a call that may not allocate
        bool prev;
        explicit NoAllocScope(bool on) : prev(t_no_alloc) { t_no_alloc = on || prev; }
        ~NoAllocScope() { t_no_alloc = prev; }
    } scope(!build_plan);
    try {
        Geometry g;
        int rc = validate(desc, cu, &g, true);
        if (rc != RA_OK) return rc;
        if ((rc = check_support(g, true)) != RA_OK) return rc;
        if (!dout || !q || !k || !v || !out || !lse || !dq || !dk || !dv) return RA_E_NULL;
        const int64_t need = bwd_workspace(g);
        if (!workspace || (int64_t)workspace_bytes < need) return RA_E_WORKSPACE;
        std::shared_ptr<const Plan> plan;
        if ((rc = get_plan(g, &plan, build_plan, (hipStream_t)stream)) != RA_OK) return rc;
        hipStream_t s = (hipStream_t)stream;
        float* lse2 = (float*)workspace;
        float* ndelta = (float*)((unsigned char*)workspace + bwd_row_bytes(g));
        float* dq_acc = (float*)((unsigned char*)workspace + 2 * bwd_row_bytes(g));
        // with room for the dS tile store, K4a keeps dS and K4c builds dQ from
        // it; otherwise K4b recomputes S and dP
        // The dS tile store takes what the workspace holds beyond `need`, in
        // units of one kv head's share (its q heads' tiles): with room for
        // hc >= 1 kv heads, the kv heads are processed hc at a time through
        // K4a + K4c; with none, K4a runs without the store and K4b recomputes.
        const int group = g.Hq / g.Hkv;
        const int64_t per_kvh = (int64_t)g.B * group * plan->max_ne * DS_TILE_ELEMS * 2;
        const int64_t avail = (int64_t)workspace_bytes - need;
        const int hc = per_kvh > 0 ? (int)std::min<int64_t>(g.Hkv, avail / per_kvh) : 0;
        uint16_t* ds_buf = hc > 0 ? (uint16_t*)((unsigned char*)workspace + need) : nullptr;

        BwdPreArgs pa{};
        pa.dout = dout; pa.out = out; pa.lse = lse; pa.lse2 = lse2; pa.ndelta = ndelta;
        pa.B = g.B; pa.S = (int32_t)g.S; pa.Hq = g.Hq; pa.S_pad = (int32_t)plan->S_pad; pa.d = g.d;
        rc = hip_rc(timed(KC_BWD_PRE, s, [&] { return launch_bwd_pre(pa, 1, s); }));
        if (rc != RA_OK) return rc;

        const int64_t block_elems = (int64_t)g.B * g.Skv * g.Hkv * g.d;
        BwdArgs a{};
        a.q = (const uint16_t*)q; a.dout = (const uint16_t*)dout; a.lse2 = lse2; a.ndelta = ndelta;
        a.B = g.B; a.S = (int32_t)g.S; a.Skv = (int32_t)g.Skv; a.Hq = g.Hq; a.Hkv = g.Hkv;
        a.nkt = plan->nkt_b;
        a.S_pad = (int32_t)plan->S_pad;
        a.hk0 = 0;
        a.nhk = g.Hkv;
        a.total_work = g.B * g.Hkv * plan->nkt_b;
        a.scale = g.scale;
        a.scale_log2 = g.scale * 1.4426950408889634f;
        a.ds = ds_buf;
        DqDsArgs da{};
        da.ds = ds_buf; da.dq_acc = dq_acc;
        da.B = g.B; da.S = (int32_t)g.S; da.Skv = (int32_t)g.Skv; da.Hq = g.Hq; da.Hkv = g.Hkv;
        da.nqt = plan->nqt_dq;
        da.S_pad = (int32_t)plan->S_pad;
        da.total_work = g.B * g.Hq * plan->nqt_dq;
        da.scale = g.scale;
        DqArgs qa{};
        qa.q = (const uint16_t*)q; qa.dout = (const uint16_t*)dout; qa.lse2 = lse2;
        qa.ndelta = ndelta; qa.dq_acc = dq_acc;
        qa.B = g.B; qa.S = (int32_t)g.S; qa.Skv = (int32_t)g.Skv; qa.Hq = g.Hq; qa.Hkv = g.Hkv;
        qa.nqt = plan->nqt_dq;
        qa.S_pad = (int32_t)plan->S_pad;
        qa.total_work = g.B * g.Hq * plan->nqt_dq;
        qa.scale = g.scale;
        qa.scale_log2 = a.scale_log2;
        bool first = true;
        for (const DevStep& st : plan->steps) {
            a.k = (const uint16_t*)k + st.j * block_elems;
            a.v = (const uint16_t*)v + st.j * block_elems;
            a.dk = dk + st.j * block_elems;
            a.dv = dv + st.j * block_elems;
            a.rng = st.rng; a.t_off = st.b_off; a.t_mid = st.b_mid; a.t_ent = st.b_ent; a.t_order = st.b_order;
            a.ds_ne = st.b_ne;
            // the dQ kernels write the accumulator on the first step (also when
            // a step has no visible pair, in which case they write zeros)
            const int32_t first_flag = first ? 1 : 0;
            if (ds_buf) {
                if (st.pairs == 0 && !first) continue;
                da.k = a.k;
                da.t_off = st.d_off; da.t_ent = st.d_ent; da.t_order = st.d_order;
                da.ds_ne = st.b_ne;
                da.first = first_flag;
                for (int c0 = 0; c0 < g.Hkv; c0 += hc) {
                    const int nhk = std::min(hc, g.Hkv - c0);
                    a.hk0 = c0;
                    a.nhk = nhk;
                    a.total_work = g.B * nhk * plan->nkt_b;
                    if (st.pairs > 0) {
                        rc = hip_rc(timed(KC_BWD, s, [&] { return launch_bwd_dkdv_bf16(a, g.d, s); }));
                        if (rc != RA_OK) return rc;
                    }
                    da.h0 = c0 * group;
                    da.nh = nhk * group;
                    da.total_work = g.B * da.nh * plan->nqt_dq;
                    rc = hip_rc(timed(KC_BWD_DQ_DS, s, [&] { return launch_bwd_dq_ds_bf16(da, g.d, s); }));
                    if (rc != RA_OK) return rc;
                }
                first = false;
                continue;
            }
            if (st.pairs > 0) {
                rc = hip_rc(timed(KC_BWD, s, [&] { return launch_bwd_dkdv_bf16(a, g.d, s); }));
                if (rc != RA_OK) return rc;
            }
            qa.k = a.k; qa.v = a.v;
            qa.rng = st.rng; qa.t_off = st.q_off; qa.t_mid = st.q_mid; qa.t_ent = st.q_ent; qa.t_order = st.q_order;
            qa.first = first_flag;
            if (st.pairs > 0 || first) {
                rc = hip_rc(timed(KC_BWD_DQ, s, [&] { return launch_bwd_dq_bf16(qa, g.d, s); }));
                if (rc != RA_OK) return rc;
                first = false;
            }
        }
        rc = hip_rc(timed(KC_BWD_POST, s, [&] {
            return launch_dq_finalize(dq_acc, dq, g.B, (int32_t)g.S, g.Hq, (int32_t)plan->S_pad, g.d, s);
        }));
        return rc;
    } catch (...) {
        return RA_E_HIP;
    }
}

int64_t bwd_need_bytes(const ring_attn_desc* desc) {
    Geometry g;
    const int rc = validate(desc, nullptr, &g, false);
    if (rc != RA_OK) return rc;
    return bwd_workspace(g);
}

}  // namespace ra

extern "C" {

int ring_attn_bwd(const ring_attn_desc* desc, const void* dout, const void* q, const void* k,
                  const void* v, const void* out, const float* lse, const int32_t* cu,
                  float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return bwd_impl(desc, dout, q, k, v, out, lse, cu, dq, dk, dv, workspace, workspace_bytes,
                    stream, true);
}

int ring_attn_timing_enable(int enable) {
    if (!enable) {
        const int rc = collect_timing();
        std::lock_guard<std::mutex> lock(g_timing.mu);
        g_timing.on = false;
        for (int i = 0; i < KC_COUNT; ++i) {
            g_timing.launches[i] = 0;
            g_timing.ms[i] = 0.0;
        }
        return rc;
    }
    std::lock_guard<std::mutex> lock(g_timing.mu);
    g_timing.on = true;
    return RA_OK;
}

int ring_attn_timing_read(const char* name, int64_t* launches, double* total_ms) {
    if (!name || !launches || !total_ms) return RA_E_NULL;
    const int rc = collect_timing();
    if (rc != RA_OK) return rc;
    std::lock_guard<std::mutex> lock(g_timing.mu);
    for (int i = 0; i < KC_COUNT; ++i)
        if (std::strcmp(name, kClassNames[i]) == 0) {
            *launches = g_timing.launches[i];
            *total_ms = g_timing.ms[i];
            return RA_OK;
        }
    return RA_E_ARG;
}

int ring_attn_clear_cache(void) {
    decltype(g_plans) dropped;
    std::vector<std::shared_ptr<Plan>> retired;
    {
        std::lock_guard<std::mutex> lock(g_plan_mu);
        dropped.swap(g_plans);
        retired.swap(g_retired);
        g_plan_index.clear();
    }
    return RA_OK;   // plans still held by a call in flight are freed when it returns
}

int ring_attn_plan_cache_limit(int32_t max_plans) {
    if (max_plans < 1) return RA_E_ARG;
    std::vector<std::shared_ptr<Plan>> dropped;
    std::lock_guard<std::mutex> lock(g_plan_mu);
    const int32_t prev = g_plan_limit;
    g_plan_limit = max_plans;
    evict_plans_locked(dropped);
    return prev;
}

int ring_attn_plan_cache_info(int64_t* n_plans, int64_t* device_bytes) {
    if (!n_plans || !device_bytes) return RA_E_NULL;
    std::lock_guard<std::mutex> lock(g_plan_mu);
    *n_plans = (int64_t)g_plans.size();
    int64_t b = 0;
    for (const auto& e : g_plans) b += (int64_t)e.second->bytes;
    *device_bytes = b;
    return RA_OK;
}

}  // extern "C"
