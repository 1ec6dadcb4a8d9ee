// Host planner: layout -> position maps -> ring schedule -> tile classification.
//
// Pure host C++ (no HIP); compiled into the library and also on its own by the
// host sanitizer test.  Every quantity here is integer and deterministic.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "ring_attn.h"

namespace ra {

struct Geometry {
    int32_t B = 0, Hq = 0, Hkv = 0, d = 0;
    int64_t N = 0;
    int32_t D = 1, r = 0;
    bool causal = false;
    int32_t layout = RA_BASIC;
    int32_t dtype = RA_BF16;
    float scale = 0.f;          // resolved softmax scale (> 0)
    int32_t merge_mode = RA_MERGE_FUSED;
    int64_t S = 0;              // local query rows
    int64_t Skv = 0;            // rows per KV block
    int32_t nb = 1;             // number of KV blocks (ring steps)
    bool varlen = false;
    std::vector<int64_t> cu;    // cu_seqlens (varlen layouts only)
    int64_t win_left = -1;      // sliding window sides, -1 = unbounded
    int64_t win_right = -1;
};

// Validates the descriptor (and cu_seqlens when the layout is varlen).
// Returns RA_OK and fills *g, or a negative RA_E_* code.
int validate(const ring_attn_desc* desc, const int32_t* cu_seqlens, Geometry* g,
             bool check_cu);

// Global positions of the local rows of `rank` (size S), increasing.
void rank_positions(const Geometry& g, int32_t rank, std::vector<int64_t>& out);
// Global positions of the rows of KV block `block` (size Skv), increasing.
void block_positions(const Geometry& g, int32_t block, std::vector<int64_t>& out);

// One ring step of rank g.r: the block it holds and, for every local query
// row i, the half-open interval [a[i], b[i]) of local key indices of that
// block that row i may see.  Because positions inside a block increase, the
// visible keys of a row (same document, not in its future) are contiguous.
struct StepRanges {
    int32_t s = 0, j = 0;
    int64_t pairs = 0;          // sum over rows of (b - a)
    std::vector<int32_t> a, b;
};

// pq: the rank's row positions (rank_positions(g, g.r)) when the caller has
// them already, else computed here.
void step_ranges(const Geometry& g, int32_t s, StepRanges& out,
                 const std::vector<int64_t>* pq = nullptr);

enum TileKind : int8_t { TILE_EMPTY = 0, TILE_PARTIAL = 1, TILE_FULL = 2 };

// kinds[qt * nkt + kt] for query tiles of bq rows and key tiles of bk keys.
// FULL: every (row < S, key) pair of the tile visible; EMPTY: none; else PARTIAL.
// A key tile that runs past Skv is never FULL.
void classify(const StepRanges& sr, int64_t S, int64_t Skv, int32_t bq, int32_t bk,
              std::vector<int8_t>& kinds);

// Persistent schedule of the one-launch forward over `nblk` blocks, one per
// CU (a multiple of 8, the XCD count; with fewer than 8 no schedule is made).
// The kernel holds one work-group per CU (8 waves of 256 registers), so a
// launch of one block per CU keeps every CU busy until its own list ends: no CU waits for the
// dispatcher between two work items, and no CU idles at the end while others
// finish long items.  Work item w = (b, q head) * nq + t runs the list of
// query tile order[t].  Each XCD (blocks are dealt to the 8 XCDs in turn)
// keeps the contiguous range of work items it gets without a schedule, so the
// items of a head still share that XCD's L2; inside the XCD, items go
// heaviest first to the least loaded of its blocks.  The cost of a list, in
// tenths of an unmasked key tile: 10 per unmasked tile, 14 per masked one,
// 120 for a work item's prologue and epilogue (measured: 3024 and 4411 cycles
// per tile, 13.2k per item).
//
// With `split`, a list that costs more than a third of its XCD's mean block
// load is cut into parts of about equal cost (at most 8, at most one per
// entry); each part runs as an item of its own and writes its normalised
// partial to a part slot, and the part-merge kernel folds the parts.  Whole
// items alone cannot balance the blocks when an item is a large fraction of a
// block's load (few items per CU of very different lengths).  The parts never
// outnumber the blocks (the threshold is raised until they fit), which bounds
// the part buffer.
struct PersSchedule {
    std::vector<int32_t> off;     // [blocks + 1]
    std::vector<int32_t> items;   // 4 per item: work, first entry, end entry, part slot (-1)
    std::vector<int32_t> merge;   // 3 per split list: work, first slot, parts
    int32_t slots = 0;
    int64_t makespan = 0;         // largest block load (cost units)
};

// Work items (b, q head) * nq + t for n_bh (batch, q head) pairs and the query
// tile lists of the plan: list q holds entries off[q] .. off[q+1]-1, its
// unmasked tiles before mid[q]; work item t of a pair runs list order[t].
// Leaves `out` empty when there are no more work items than blocks.
void persistent_schedule(int64_t nblk, int64_t n_bh, const std::vector<int32_t>& off,
                         const std::vector<int32_t>& mid, const std::vector<int32_t>& order,
                         bool split, PersSchedule& out);

// Canonical text key of a geometry (for the plan cache).
std::string plan_key(const Geometry& g);

}  // namespace ra
