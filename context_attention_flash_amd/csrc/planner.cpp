// Host planner for the ring-attention rank share.  See planner.h.
//
// Layout definitions follow the variants named on the skillfed
// "ring-flash-attn" fact sheet ("What it is and what it does") and the sharding
// of the ai360xpert "Ring Attention" page ("Sequence sharding and the ring
// topology"); the ring order and the causal rule follow the instagit/nanotron
// page ("Forward Pass Implementation").
#include "planner.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <functional>
#include <queue>
#include <sstream>

namespace ra {

int validate(const ring_attn_desc* desc, const int32_t* cu, Geometry* g, bool check_cu) {
    if (!desc || !g) return RA_E_NULL;
    const ring_attn_desc& d = *desc;
    if (d.batch < 1 || d.heads_q < 1 || d.heads_kv < 1 || d.head_dim < 1 || d.seqlen < 1)
        return RA_E_SHAPE;
    // Local key indices and positions travel as int32 inside the kernels.
    if (d.seqlen > (int64_t)(INT_MAX / 2)) return RA_E_SHAPE;
    if (d.heads_q % d.heads_kv != 0) return RA_E_HEADS;
    if (d.world < 1 || d.rank < 0 || d.rank >= d.world) return RA_E_WORLD;
    if (d.layout < RA_BASIC || d.layout > RA_VARLEN_STRIPE) return RA_E_LAYOUT;
    if (d.causal != 0 && d.causal != 1) return RA_E_ARG;
    if (d.dtype != RA_F32 && d.dtype != RA_BF16) return RA_E_UNSUPPORTED;
    if (d.merge_mode != RA_MERGE_FUSED && d.merge_mode != RA_MERGE_SEPARATE &&
        d.merge_mode != RA_MERGE_STEPWISE)
        return RA_E_ARG;
    {   // a NaN or infinite scale is an error (tested on the bit pattern, which
        // no floating-point compiler option can fold away)
        uint32_t bits;
        std::memcpy(&bits, &d.softmax_scale, sizeof bits);
        if ((bits & 0x7f800000u) == 0x7f800000u) return RA_E_ARG;
    }
    if (d.window_left < -1 || d.window_right < -1) return RA_E_ARG;
    const bool varlen = d.layout == RA_VARLEN_RING || d.layout == RA_LLAMA3 ||
                        d.layout == RA_VARLEN_ZIGZAG || d.layout == RA_VARLEN_STRIPE;
    if (varlen && d.batch != 1) return RA_E_LAYOUT;
    const bool zz = d.layout == RA_ZIGZAG || d.layout == RA_VARLEN_ZIGZAG;
    const int64_t div = zz ? 2LL * d.world : (int64_t)d.world;
    if (d.seqlen % div != 0) return RA_E_DIVISIBILITY;

    Geometry G;
    G.B = d.batch; G.Hq = d.heads_q; G.Hkv = d.heads_kv; G.d = d.head_dim;
    G.N = d.seqlen; G.D = d.world; G.r = d.rank; G.causal = d.causal != 0;
    G.layout = d.layout; G.dtype = d.dtype; G.merge_mode = d.merge_mode;
    G.scale = d.softmax_scale > 0.f ? d.softmax_scale : (float)(1.0 / std::sqrt((double)d.head_dim));
    G.S = d.seqlen / d.world;
    G.Skv = d.layout == RA_LLAMA3 ? d.seqlen : G.S;
    G.nb = d.layout == RA_LLAMA3 ? 1 : d.world;
    G.varlen = varlen;
    G.win_left = d.window_left;
    G.win_right = d.window_right;
    if (varlen && check_cu) {
        if (!cu) return RA_E_NULL;
        if (d.n_seqs < 1) return RA_E_CU_SEQLENS;
        if (cu[0] != 0 || (int64_t)cu[d.n_seqs] != d.seqlen) return RA_E_CU_SEQLENS;
        G.cu.resize(d.n_seqs + 1);
        for (int i = 0; i <= d.n_seqs; ++i) {
            if (i > 0 && cu[i] < cu[i - 1]) return RA_E_CU_SEQLENS;
            G.cu[i] = cu[i];
        }
        // every document must split evenly into the layout's parts
        if (d.layout != RA_LLAMA3)
            for (int i = 0; i < d.n_seqs; ++i)
                if ((G.cu[i + 1] - G.cu[i]) % div != 0) return RA_E_CU_SEQLENS;
    }
    *g = std::move(G);
    return RA_OK;
}

void rank_positions(const Geometry& g, int32_t rank, std::vector<int64_t>& out) {
    out.resize(g.S);
    switch (g.layout) {
        case RA_BASIC:
        case RA_LLAMA3:
            for (int64_t i = 0; i < g.S; ++i) out[i] = rank * g.S + i;
            break;
        case RA_ZIGZAG: {
            const int64_t c = g.N / (2 * g.D);
            for (int64_t i = 0; i < c; ++i) {
                out[i] = rank * c + i;
                out[c + i] = (int64_t)(2 * g.D - 1 - rank) * c + i;
            }
            break;
        }
        case RA_STRIPE:
            for (int64_t i = 0; i < g.S; ++i) out[i] = i * g.D + rank;
            break;
        case RA_VARLEN_RING: {
            int64_t o = 0;
            for (size_t k = 0; k + 1 < g.cu.size(); ++k) {
                const int64_t part = (g.cu[k + 1] - g.cu[k]) / g.D;
                for (int64_t i = 0; i < part; ++i) out[o++] = g.cu[k] + rank * part + i;
            }
            break;
        }
        case RA_VARLEN_ZIGZAG: {
            int64_t o = 0;
            for (size_t k = 0; k + 1 < g.cu.size(); ++k) {
                const int64_t c = (g.cu[k + 1] - g.cu[k]) / (2 * g.D);
                for (int64_t i = 0; i < c; ++i) out[o++] = g.cu[k] + rank * c + i;
                for (int64_t i = 0; i < c; ++i) out[o++] = g.cu[k] + (2 * g.D - 1 - rank) * c + i;
            }
            break;
        }
        case RA_VARLEN_STRIPE: {
            int64_t o = 0;
            for (size_t k = 0; k + 1 < g.cu.size(); ++k)
                for (int64_t t = g.cu[k] + rank; t < g.cu[k + 1]; t += g.D) out[o++] = t;
            break;
        }
    }
}

void block_positions(const Geometry& g, int32_t block, std::vector<int64_t>& out) {
    if (g.layout == RA_LLAMA3) {
        out.resize(g.N);
        for (int64_t i = 0; i < g.N; ++i) out[i] = i;
        return;
    }
    rank_positions(g, block, out);
}

void step_ranges(const Geometry& g, int32_t s, StepRanges& out, const std::vector<int64_t>* pq_in) {
    out.s = s;
    out.j = g.layout == RA_LLAMA3 ? 0 : (int32_t)(((g.r - s) % g.D + g.D) % g.D);
    std::vector<int64_t> pq_own, pk;
    if (pq_in == nullptr) rank_positions(g, g.r, pq_own);
    const std::vector<int64_t>& pq = pq_in != nullptr ? *pq_in : pq_own;
    block_positions(g, out.j, pk);
    out.a.resize(g.S);
    out.b.resize(g.S);
    out.pairs = 0;
    // The visible global positions of row t form the interval [lo, hi]: its
    // document (varlen), up to t (causal), inside the window.  Both ends only
    // grow with t, and every layout's rows and blocks hold ascending
    // positions, so the interval's first and last key index are found by two
    // cursors that only move forward (binary search otherwise).
    const bool sweep = std::is_sorted(pq.begin(), pq.end()) && std::is_sorted(pk.begin(), pk.end());
    const int64_t nk = (int64_t)pk.size();
    int64_t ia = 0, ib = 0;   // first key with position >= lo, first with position > hi
    size_t doc = 0;           // varlen: document of the current row (sweep)
    for (int64_t i = 0; i < g.S; ++i) {
        const int64_t t = pq[i];
        int64_t lo = 0, hi = g.N - 1;  // visible global positions [lo, hi]
        if (g.varlen) {
            if (sweep) {
                while (doc + 2 < g.cu.size() && g.cu[doc + 1] <= t) ++doc;
                lo = g.cu[doc];
                hi = g.cu[doc + 1] - 1;
            } else {
                const auto it = std::upper_bound(g.cu.begin(), g.cu.end(), t);
                lo = *(it - 1);
                hi = *it - 1;
            }
        }
        if (g.causal) hi = std::min(hi, t);
        if (g.win_left >= 0) lo = std::max(lo, t - g.win_left);
        if (g.win_right >= 0) hi = std::min(hi, t + g.win_right);
        int64_t a, b;
        if (sweep) {
            while (ia < nk && pk[ia] < lo) ++ia;
            while (ib < nk && pk[ib] <= hi) ++ib;
            a = ia;
            b = ib;
        } else {
            a = std::lower_bound(pk.begin(), pk.end(), lo) - pk.begin();
            b = std::upper_bound(pk.begin(), pk.end(), hi) - pk.begin();
        }
        out.a[i] = (int32_t)a;
        out.b[i] = (int32_t)std::max(a, b);
        out.pairs += std::max<int64_t>(0, b - a);
    }
}

void classify(const StepRanges& sr, int64_t S, int64_t Skv, int32_t bq, int32_t bk,
              std::vector<int8_t>& kinds) {
    const int64_t nqt = (S + bq - 1) / bq, nkt = (Skv + bk - 1) / bk;
    kinds.assign(nqt * nkt, TILE_EMPTY);
    std::vector<int32_t> diff(nkt + 1);
    for (int64_t qt = 0; qt < nqt; ++qt) {
        const int64_t r0 = qt * bq, r1 = std::min<int64_t>(S, r0 + bq);
        int64_t amax = 0, bmin = INT64_MAX;
        std::fill(diff.begin(), diff.end(), 0);
        for (int64_t i = r0; i < r1; ++i) {
            const int64_t a = sr.a[i], b = sr.b[i];
            amax = std::max(amax, a);
            bmin = std::min(bmin, b);
            if (a < b) {
                diff[a / bk] += 1;
                diff[(b - 1) / bk + 1] -= 1;
            }
        }
        int32_t run = 0;
        for (int64_t kt = 0; kt < nkt; ++kt) {
            run += diff[kt];
            const int64_t k0 = kt * bk, k1 = k0 + bk;
            int8_t kind = TILE_EMPTY;
            if (amax <= k0 && k1 <= bmin && k1 <= Skv) kind = TILE_FULL;
            else if (run > 0) kind = TILE_PARTIAL;
            kinds[qt * nkt + kt] = kind;
        }
    }
}

void persistent_schedule(int64_t nblk, int64_t n_bh, const std::vector<int32_t>& off,
                         const std::vector<int32_t>& mid, const std::vector<int32_t>& order,
                         bool split, PersSchedule& out) {
    out = PersSchedule{};
    constexpr int64_t kXcd = 8, kMaxParts = 8, kTile = 10, kMasked = 14, kItem = 120;
    const int64_t nq = (int64_t)order.size();
    const int64_t W = n_bh * nq;
    if (nblk < kXcd || W <= nblk) return;
    const int64_t per_xcd = nblk / kXcd;
    auto nfull = [&](int64_t w) { const int32_t q = order[w % nq]; return (int64_t)(mid[q] - off[q]); };
    auto nall = [&](int64_t w) { const int32_t q = order[w % nq]; return (int64_t)(off[q + 1] - off[q]); };
    auto cost_of = [&](int64_t w, int64_t a, int64_t b) {   // entries [a, b) of w's list
        const int64_t f = nfull(w);
        const int64_t full = std::max<int64_t>(0, std::min(b, f) - a);
        return kTile * full + kMasked * (b - a - full) + kItem;
    };
    // the threshold of each XCD: a third of its mean block load, raised until
    // the parts fit the part slots
    std::vector<int64_t> thresh(kXcd, INT64_MAX);
    auto parts_of = [&](int64_t w, int64_t T) {
        const int64_t c = cost_of(w, 0, nall(w));
        if (c <= T || nall(w) < 2) return (int64_t)1;
        return std::min({(c + T - 1) / T, kMaxParts, nall(w)});
    };
    if (split) {
        int64_t used = 0;
        for (int64_t x = 0; x < kXcd; ++x) {
            const int64_t w0 = x * W / kXcd, w1 = (x + 1) * W / kXcd;
            int64_t total = 0;
            for (int64_t w = w0; w < w1; ++w) total += cost_of(w, 0, nall(w));
            thresh[x] = std::max<int64_t>(1, total / per_xcd / 3);
        }
        for (;;) {
            used = 0;
            for (int64_t x = 0; x < kXcd; ++x)
                for (int64_t w = x * W / kXcd; w < (x + 1) * W / kXcd; ++w) {
                    const int64_t k = parts_of(w, thresh[x]);
                    if (k > 1) used += k;
                }
            if (used <= nblk) break;
            for (auto& t : thresh) t = t + t / 4 + 1;
        }
    }
    struct Piece { int64_t cost; int32_t w, a, b, slot; };
    std::vector<std::vector<int32_t>> lists(nblk);
    std::vector<Piece> pieces;
    for (int64_t x = 0; x < kXcd; ++x) {
        const int64_t w0 = x * W / kXcd, w1 = (x + 1) * W / kXcd;
        pieces.clear();
        for (int64_t w = w0; w < w1; ++w) {
            const int64_t n = nall(w);
            const int64_t k = split ? parts_of(w, thresh[x]) : 1;
            if (k == 1) {
                pieces.push_back({cost_of(w, 0, n), (int32_t)w, 0, (int32_t)n, -1});
                continue;
            }
            // cut the entries where the running cost passes j/k of the list's
            const int64_t f = nfull(w);
            const int64_t tiles = kTile * std::min(f, n) + kMasked * (n - std::min(f, n));
            out.merge.insert(out.merge.end(), {(int32_t)w, out.slots, (int32_t)k});
            int64_t a = 0, acc = 0, e = 0;
            for (int64_t j = 1; j <= k; ++j) {
                int64_t b = n;
                if (j < k) {
                    const int64_t goal = tiles * j / k;
                    while (e < n && acc < goal) acc += e++ < f ? kTile : kMasked;
                    b = std::max(e, a + 1);
                    b = std::min(b, n - (k - j));   // every later part keeps one entry
                    e = b;
                    acc = kTile * std::min(b, f) + kMasked * (b - std::min(b, f));
                }
                pieces.push_back({cost_of(w, a, b), (int32_t)w, (int32_t)a, (int32_t)b, out.slots++});
                a = b;
            }
        }
        // heaviest first, each to the least loaded block (ties to the lower
        // block index).  (Taking the pieces in their own order instead, as the
        // hardware would dispatch them, balanced basic_s8192 as well but
        // doubled the forward's L2 misses; the time did not change.)
        std::stable_sort(pieces.begin(), pieces.end(),
                         [](const Piece& p, const Piece& q) { return p.cost > q.cost; });
        using Slot = std::pair<int64_t, int64_t>;   // (load, local block index)
        std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
        for (int64_t l = 0; l < per_xcd; ++l) heap.emplace(0, l);
        for (const Piece& pc : pieces) {
            auto [load, l] = heap.top();
            heap.pop();
            auto& L = lists[l * kXcd + x];
            L.insert(L.end(), {pc.w, pc.a, pc.b, pc.slot});
            heap.emplace(load + pc.cost, l);
            out.makespan = std::max(out.makespan, load + pc.cost);
        }
    }
    out.off.assign(nblk + 1, 0);
    for (int64_t i = 0; i < nblk; ++i) {
        out.off[i + 1] = out.off[i] + (int32_t)(lists[i].size() / 4);
        out.items.insert(out.items.end(), lists[i].begin(), lists[i].end());
    }
}

std::string plan_key(const Geometry& g) {
    // The schedule and tile lists depend on the token geometry; which lists a
    // plan holds also depends on the input type; the forward's persistent
    // schedule on the number of (batch, q head) pairs, its part buffer on the
    // head dimension.
    std::ostringstream o;
    o << g.N << ',' << g.D << ',' << g.r << ',' << g.causal << ',' << g.layout << ','
      << g.win_left << ',' << g.win_right << ',' << g.dtype << ',' << g.B << ',' << g.Hq << ','
      << g.d;
    if (g.varlen) {
        o << '|';
        for (int64_t c : g.cu) o << c << ',';
    }
    return o.str();
}

}  // namespace ra
