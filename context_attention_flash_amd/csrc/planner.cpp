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
