"""Host-side C and C++ checks (no GPU):

* include/ring_attn.h is valid C99; a C program links libringattn.so and gets
  the same positions, schedule and workspace sizes as the Python binding;
* the planner, built alone with g++ under AddressSanitizer and
  UndefinedBehaviorSanitizer, runs every layout, world size, rank, causal
  flag, window and document split through validation, position maps, step
  intervals and tile classification, and checks their invariants.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import context_attention_flash_amd as ca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "context_attention_flash_amd", "csrc")
PKG = os.path.join(ROOT, "context_attention_flash_amd")

C_PROG = r"""
#include <stdio.h>
#include <stdlib.h>
#include "ring_attn.h"

int main(void) {
    ring_attn_desc d = {0};
    int64_t pos[64];
    int32_t blk[4];
    int64_t pairs[4];
    int32_t n = 0, i;
    d.batch = 1; d.heads_q = 4; d.heads_kv = 2; d.head_dim = 128; d.seqlen = 256;
    d.world = 4; d.rank = 1; d.causal = 1; d.layout = RA_ZIGZAG; d.dtype = RA_BF16;
    d.softmax_scale = 0.f; d.n_seqs = 0; d.merge_mode = RA_MERGE_FUSED;
    d.window_left = -1; d.window_right = -1;
    if (ring_attn_version() != 1) return 1;
    if (ring_attn_positions(&d, NULL, 1, pos) != RA_OK) return 2;
    for (i = 0; i < 64; ++i) printf("%lld ", (long long)pos[i]);
    printf("\n");
    if (ring_attn_schedule(&d, NULL, blk, pairs, &n) != RA_OK || n != 4) return 3;
    for (i = 0; i < n; ++i) printf("%d:%lld ", blk[i], (long long)pairs[i]);
    printf("\n%lld %lld %lld\n", (long long)ring_attn_workspace_bytes(&d, 0),
           (long long)ring_attn_workspace_bytes(&d, 1), (long long)ring_attn_bwd_ds_bytes(&d, NULL));
    d.world = 0;
    if (ring_attn_workspace_bytes(&d, 0) != RA_E_WORLD) return 4;
    printf("%s\n", ring_attn_strerror(RA_E_WORLD));
    return 0;
}
"""

PLANNER_DRIVER = r"""
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "planner.h"

using namespace ra;

static int fail(const char* what) { std::fprintf(stderr, "FAIL %s\n", what); return 1; }

int main() {
    std::mt19937 rng(7);
    long checked = 0;
    for (int layout = RA_BASIC; layout <= RA_VARLEN_STRIPE; ++layout)
      for (int D : {1, 2, 3, 4, 8})
        for (int causal = 0; causal < 2; ++causal)
          for (int wsel = 0; wsel < 3; ++wsel) {
            const bool zz = layout == RA_ZIGZAG || layout == RA_VARLEN_ZIGZAG;
            const bool packed = layout == RA_VARLEN_RING || layout == RA_LLAMA3 ||
                                layout == RA_VARLEN_ZIGZAG || layout == RA_VARLEN_STRIPE;
            const int mult = zz ? 2 * D : D;
            const int N = mult * (3 + (int)(rng() % 40));
            std::vector<int32_t> cu{0};
            if (packed) {
                const int unit = layout == RA_LLAMA3 ? 1 : mult;
                while (cu.back() < N) {
                    const int len = unit * (1 + (int)(rng() % (N / unit)));
                    cu.push_back(std::min(N, cu.back() + len));
                }
            }
            ring_attn_desc d{};
            d.batch = 1; d.heads_q = 2; d.heads_kv = 1; d.head_dim = 64; d.seqlen = N;
            d.world = D; d.causal = causal; d.layout = layout; d.dtype = RA_BF16;
            d.n_seqs = packed ? (int32_t)cu.size() - 1 : 0; d.merge_mode = RA_MERGE_FUSED;
            d.window_left = wsel == 1 ? 5 : -1;
            d.window_right = wsel == 2 ? 3 : -1;
            std::vector<int64_t> all;
            for (int r = 0; r < D; ++r) {
                d.rank = r;
                Geometry g;
                if (validate(&d, packed ? cu.data() : nullptr, &g, true) != RA_OK) return fail("validate");
                std::vector<int64_t> pq, pk;
                rank_positions(g, r, pq);
                if ((int64_t)pq.size() != g.S) return fail("rows");
                for (size_t i = 1; i < pq.size(); ++i)
                    if (pq[i] <= pq[i - 1]) return fail("increasing");
                for (int32_t s = 0; s < g.nb; ++s) {
                    StepRanges sr;
                    step_ranges(g, s, sr);
                    block_positions(g, sr.j, pk);
                    int64_t sum = 0;
                    auto doc = [&](int64_t t) {
                        if (!packed) return 0;
                        return (int)(std::upper_bound(cu.begin(), cu.end(), (int32_t)t) - cu.begin());
                    };
                    auto visible = [&](int64_t t, int64_t u) {
                        if (causal && u > t) return false;
                        if (doc(u) != doc(t)) return false;
                        if (d.window_left >= 0 && u < t - d.window_left) return false;
                        if (d.window_right >= 0 && u > t + d.window_right) return false;
                        return true;
                    };
                    for (int64_t i = 0; i < g.S; ++i) {
                        if (sr.a[i] < 0 || sr.a[i] > sr.b[i] || sr.b[i] > g.Skv) return fail("interval");
                        // every key inside the interval is visible, the ones next to it are not
                        for (int32_t k = sr.a[i]; k < sr.b[i]; ++k)
                            if (!visible(pq[i], pk[k])) return fail("invisible key inside");
                        if (sr.a[i] < sr.b[i]) {
                            if (sr.a[i] > 0 && visible(pq[i], pk[sr.a[i] - 1])) return fail("left edge");
                            if (sr.b[i] < g.Skv && visible(pq[i], pk[sr.b[i]])) return fail("right edge");
                        }
                        sum += sr.b[i] - sr.a[i];
                    }
                    if (sum != sr.pairs) return fail("pairs");
                    for (int bq : {1, 16, 64}) for (int bk : {8, 64, 128}) {
                        std::vector<int8_t> kinds;
                        classify(sr, g.S, g.Skv, bq, bk, kinds);
                        const int64_t nqt = (g.S + bq - 1) / bq, nkt = (g.Skv + bk - 1) / bk;
                        if ((int64_t)kinds.size() != nqt * nkt) return fail("kinds size");
                        for (int64_t qt = 0; qt < nqt; ++qt)
                            for (int64_t kt = 0; kt < nkt; ++kt) {
                                int64_t vis = 0, tot = 0;
                                for (int64_t i = qt * bq; i < std::min<int64_t>(g.S, (qt + 1) * bq); ++i)
                                    for (int64_t k = kt * bk; k < (kt + 1) * bk; ++k) {
                                        ++tot;
                                        vis += k < g.Skv && k >= sr.a[i] && k < sr.b[i];
                                    }
                                const int8_t want = vis == 0 ? TILE_EMPTY
                                                             : (vis == tot ? TILE_FULL : TILE_PARTIAL);
                                if (kinds[qt * nkt + kt] != want) return fail("kind");
                            }
                    }
                    ++checked;
                }
                all.insert(all.end(), pq.begin(), pq.end());
            }
            if (layout != RA_LLAMA3) {
                std::sort(all.begin(), all.end());
                for (int64_t t = 0; t < N; ++t)
                    if (all[t] != t) return fail("bijection");
            }
          }
    std::printf("checked %ld steps\n", checked);
    return 0;
}
"""


SCHEDULE_DRIVER = r"""
#include <algorithm>
#include <array>
#include <cstdio>
#include <map>
#include <numeric>
#include <random>
#include <vector>
#include "planner.h"

using namespace ra;

static int fail(const char* what, long c) { std::fprintf(stderr, "FAIL %s (case %ld)\n", what, c); return 1; }

int main() {
    std::mt19937 rng(11);
    long cases = 0, splits = 0;
    for (long c = 0; c < 3000; ++c) {
        const int64_t nblk = std::vector<int64_t>{0, 8, 16, 64, 248, 256}[rng() % 6];
        const int64_t n_bh = 1 + rng() % 48;
        const int64_t nq = 1 + rng() % 40;
        // list lengths: mostly alike, some empty, some very long (a long
        // document of a packed stream)
        std::vector<int32_t> off{0}, mid;
        for (int64_t q = 0; q < nq; ++q) {
            int32_t n = (int32_t)(rng() % 12);
            if (rng() % 8 == 0) n = 0;
            if (rng() % 10 == 0) n = 40 + (int32_t)(rng() % 400);
            mid.push_back(off.back() + (int32_t)(rng() % (n + 1)));
            off.push_back(off.back() + n);
        }
        std::vector<int32_t> order(nq);
        std::iota(order.begin(), order.end(), 0);
        if (rng() % 2)
            std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
                return off[x + 1] - off[x] > off[y + 1] - off[y];
            });
        else
            std::shuffle(order.begin(), order.end(), rng);
        const int64_t W = n_bh * nq;
        auto nall = [&](int64_t w) { const int32_t q = order[w % nq]; return (int64_t)(off[q + 1] - off[q]); };
        auto nfull = [&](int64_t w) { const int32_t q = order[w % nq]; return (int64_t)(mid[q] - off[q]); };
        auto cost = [&](int64_t w, int64_t a, int64_t b) {   // 10 per unmasked, 14 per masked tile, 120 per item
            const int64_t f = std::max<int64_t>(0, std::min(b, nfull(w)) - a);
            return 10 * f + 14 * (b - a - f) + 120;
        };
        for (int split = 0; split < 2; ++split) {
            PersSchedule s;
            persistent_schedule(nblk, n_bh, off, mid, order, split != 0, s);
            ++cases;
            if (nblk < 8 || W <= nblk) {
                if (!s.off.empty() || !s.items.empty() || !s.merge.empty() || s.slots) return fail("no schedule", c);
                continue;
            }
            if ((int64_t)s.off.size() != nblk + 1 || s.off[0] != 0) return fail("off", c);
            for (int64_t i = 0; i < nblk; ++i)
                if (s.off[i + 1] < s.off[i]) return fail("off order", c);
            if ((int64_t)s.items.size() != 4 * (int64_t)s.off[nblk]) return fail("items size", c);
            if (s.slots > nblk) return fail("slots bound", c);
            if (!split && (s.slots || !s.merge.empty())) return fail("cut without split", c);
            std::map<int64_t, std::vector<std::array<int32_t, 3>>> pieces;   // w -> (a, b, slot)
            std::vector<int> slot_use(s.slots, 0);
            std::vector<int64_t> load(nblk, 0);
            const int64_t per_xcd = nblk / 8;
            for (int64_t i = 0; i < nblk; ++i)
                for (int32_t it = s.off[i]; it < s.off[i + 1]; ++it) {
                    const int32_t w = s.items[4 * it], a = s.items[4 * it + 1], b = s.items[4 * it + 2],
                                  slot = s.items[4 * it + 3];
                    const int64_t x = i % 8;   // blocks are dealt to the XCDs in turn
                    if (w < x * W / 8 || w >= (x + 1) * W / 8) return fail("xcd range", c);
                    if (a < 0 || b < a || b > nall(w)) return fail("entry range", c);
                    if (slot < -1 || slot >= s.slots) return fail("slot range", c);
                    if (slot >= 0) {
                        if (b == a) return fail("empty part", c);
                        ++slot_use[slot];
                    }
                    pieces[w].push_back({a, b, slot});
                    load[i] += cost(w, a, b);
                }
            for (int u : slot_use)
                if (u != 1) return fail("slot used once", c);
            // every work item exactly once: whole, or cut into contiguous parts
            // whose slots run consecutively as its merge entry says
            std::map<int64_t, std::array<int32_t, 2>> merge;
            for (size_t m = 0; m + 3 <= s.merge.size(); m += 3) {
                if (merge.count(s.merge[m])) return fail("merge twice", c);
                merge[s.merge[m]] = {s.merge[m + 1], s.merge[m + 2]};
            }
            if (s.merge.size() % 3) return fail("merge size", c);
            if ((int64_t)pieces.size() != W) return fail("every work item", c);
            for (auto& [w, ps] : pieces) {
                std::sort(ps.begin(), ps.end());
                if (ps.size() == 1 && ps[0][2] == -1) {
                    if (ps[0][0] != 0 || ps[0][1] != nall(w)) return fail("whole item", c);
                    if (merge.count(w)) return fail("merge of a whole item", c);
                    continue;
                }
                const auto mi = merge.find(w);
                if (mi == merge.end()) return fail("parts without merge", c);
                const int32_t s0 = mi->second[0], k = mi->second[1];
                if (k < 2 || k > 8 || (int64_t)ps.size() != k || k > nall(w)) return fail("part count", c);
                int32_t at = 0;
                for (int32_t j = 0; j < k; ++j) {
                    if (ps[j][0] != at || ps[j][2] != s0 + j) return fail("parts contiguous", c);
                    at = ps[j][1];
                }
                if (at != nall(w)) return fail("parts cover", c);
                ++splits;
            }
            if ((int64_t)merge.size() * 3 != (int64_t)s.merge.size()) return fail("merge entries", c);
            // the reported makespan, and the list-scheduling bound per XCD:
            // heaviest-first to the least loaded block ends within one piece
            // of the mean load
            const int64_t ms = *std::max_element(load.begin(), load.end());
            if (ms != s.makespan) return fail("makespan", c);
            for (int64_t x = 0; x < 8; ++x) {
                int64_t total = 0, biggest = 0, most = 0;
                for (int64_t l = 0; l < per_xcd; ++l) {
                    const int64_t i = l * 8 + x;
                    total += load[i];
                    most = std::max(most, load[i]);
                    for (int32_t it = s.off[i]; it < s.off[i + 1]; ++it)
                        biggest = std::max(biggest, cost(s.items[4 * it], s.items[4 * it + 1], s.items[4 * it + 2]));
                }
                if (most > (total + per_xcd - 1) / per_xcd + biggest) return fail("list bound", c);
            }
        }
    }
    std::printf("checked %ld schedules, %ld split lists\n", cases, splits);
    return splits > 0 ? 0 : fail("no case split a list", -1);
}
"""


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def test_header_is_c99_and_the_library_links(tmp_path):
    _need("gcc")
    src = tmp_path / "abi.c"
    src.write_text(C_PROG)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{INC}",
                    str(src), f"-L{PKG}", "-lringattn", f"-Wl,-rpath,{PKG}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    lines = r.stdout.strip().split("\n")
    desc = ca.make_desc(1, 4, 2, 128, 256, 4, 1, True, ca.ZIGZAG)
    assert [int(x) for x in lines[0].split()] == list(ca.ring_attn_positions(desc))
    sched = [tuple(int(v) for v in x.split(":")) for x in lines[1].split()]
    assert sched == [(j, p) for _, j, p in ca.ring_attn_schedule(desc)]
    ws = [int(x) for x in lines[2].split()]
    assert ws == [ca.ring_attn_workspace_bytes(desc, False), ca.ring_attn_workspace_bytes(desc, True),
                  ca.ring_attn_bwd_ds_bytes(desc)]
    assert lines[3] == ca.ring_attn_strerror(-3)


def test_planner_under_address_and_undefined_sanitizers(tmp_path):
    _need("g++")
    drv = tmp_path / "drv.cpp"
    drv.write_text(PLANNER_DRIVER)
    exe = tmp_path / "drv"
    # host-only build with g++ (no HIP code is involved)
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{INC}", f"-I{CSRC}",
                    os.path.join(CSRC, "planner.cpp"), str(drv), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "checked" in r.stdout


def test_persistent_schedule_under_address_and_undefined_sanitizers(tmp_path):
    """The forward's persistent schedule (host logic, built alone with g++
    under ASan/UBSan) over random list structures, with and without cuts:
    every work item runs exactly once, whole or as contiguous parts whose part
    slots are used once each and named by its merge entry; each block takes
    only its XCD's contiguous range of items; the reported makespan is the
    largest block load, within one piece of the XCD's mean load."""
    _need("g++")
    drv = tmp_path / "sched.cpp"
    drv.write_text(SCHEDULE_DRIVER)
    exe = tmp_path / "sched"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{INC}", f"-I{CSRC}",
                    os.path.join(CSRC, "planner.cpp"), str(drv), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stderr[-2000:]
    assert "checked" in r.stdout
