// Kernel argument blocks and launchers shared between the host ABI and the
// HIP translation units.  Host-visible, no device code.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace ra {

// Per-step epilogue of the forward kernel.
enum FwdMode : int32_t {
    FWD_FIRST = 0,    // write the step's partial as the running result
    FWD_MERGE = 1,    // merge the partial into the running result
    FWD_LAST = 2,     // merge, then write out (input dtype) and lse
    FWD_SOLO = 3,     // single active step: write out and lse directly
    FWD_PARTIAL = 4,  // write the normalised partial, fp32 [B,S,Hq,d], and its lse
};

constexpr int FWD_BQ = 128;   // query rows per fp32 forward work-group (one per thread)
constexpr int FWD_BK = 64;    // keys per forward tile (both forward kernels)
constexpr int BWD_BQ = 64;    // query rows per backward tile
constexpr int BWD_BK = 128;   // keys per backward work-group (4 waves x 32)
constexpr int DQ_BQ = 256;    // query rows per dQ work-group (4 waves x 64) and per
                              // bf16 forward work-group (8 waves x 32)
constexpr int DQ_BK = 64;     // keys per dQ tile
constexpr int S_ALIGN = 256;  // the padded row count S_pad is a multiple of this
// Entries of the one-launch forward: bits 0-19 key tile, 20-30 plan step, 31 partial.
constexpr int RING_STEP_SHIFT = 20;
constexpr int RING_MAX_STEPS = 1 << 11;
constexpr int RING_MAX_KEY_TILES = 1 << 20;

struct FwdArgs {
    const void* q;          // [B, S, Hq, d]
    const void* k;          // block j: [B, Skv, Hkv, d]
    const void* v;
    const int32_t* rng;     // [S_pad][2] visible local key interval [a, b) per query row
    const int32_t* t_off;   // [nqt + 1] tile-list offsets per query tile
    const int32_t* t_mid;   // [nqt] first PARTIAL entry of each list (FULL ones before it)
    const int32_t* t_ent;   // key tile index | (partial << 31)
    const int32_t* t_order; // [nqt] query tiles, heaviest first
    // One launch over every ring step (bf16 kernel, FWD_SOLO): entries are
    // key tile | plan step << RING_STEP_SHIFT | partial << 31, the per-row
    // intervals of plan step p start at rng + p * rng_stride, and blk[p] is the
    // KV block of plan step p (k and v then point at block 0).
    const int32_t* blk;
    int64_t block_elems;    // elements of one KV block [B, Skv, Hkv, d]
    int32_t rng_stride;     // ints between the interval arrays of two plan steps
    int32_t ring;           // 1: the entries span the ring steps as above
    float* o_run;           // running fp32 output (layout private to the kernel family)
    float* lse;             // [B, Hq, S] running / final lse
    void* out;              // [B, S, Hq, d] final output (input dtype)
    float* o_part;          // FWD_PARTIAL: [B, S, Hq, d] fp32
    float* lse_part;        // FWD_PARTIAL: [B, Hq, S]
    int32_t B, S, Skv, Hq, Hkv, nqt, S_pad;
    int32_t mode;
    int32_t total_work;     // B * Hq * nqt
    float scale_log2;       // softmax scale * log2(e)
    // Persistent schedule (ring launch only; NULL: one work item per block):
    // block i walks items pers_off[i] .. pers_off[i + 1] - 1 of pers_items,
    // 4 ints each: work index, first and end entry of the work's list
    // (relative to its start), part slot (-1: the whole list); the launch has
    // pers_blocks blocks.  A part writes its normalised partial output and lse
    // to part_o [slot][256 rows][d] and part_l [slot][256 rows].
    const int32_t* pers_off;
    const int32_t* pers_items;
    int32_t pers_blocks;
    float* part_o;
    float* part_l;
};

// Merge of the parts of split forward lists (fwd_part_merge_kernel): item i
// is items[3i..3i+2] = work index, first part slot, number of parts.
struct PartMergeArgs {
    const int32_t* items;
    const int32_t* t_order;   // [nqt] query tile of each list position
    const float* part_o;
    const float* part_l;
    void* out;                // [B, S, Hq, d] bf16
    float* lse;               // [B, Hq, S]
    int32_t n_items, nqt, S, Hq, d;
};

struct BwdArgs {
    const uint16_t* q;      // [B, S, Hq, d] bf16
    const uint16_t* k;      // block j: [B, Skv, Hkv, d]
    const uint16_t* v;
    const uint16_t* dout;   // [B, S, Hq, d]
    const float* lse2;      // [B, Hq, S_pad] lse * log2(e); +inf for rows that see nothing
    const float* ndelta;    // [B, Hq, S_pad] -rowsum(dout * out); 0 on padding rows
    const int32_t* rng;     // [S_pad][2]
    const int32_t* t_off;   // [nkt + 1] query-tile lists per key tile
    const int32_t* t_mid;   // [nkt] first PARTIAL entry of each list
    const int32_t* t_ent;   // query tile index | (partial << 31)
    const int32_t* t_order; // [nkt] key tiles, heaviest first
    float* dk;              // block j: [B, Skv, Hkv, d] fp32, +=
    float* dv;
    uint16_t* ds;           // NULL, or the dS tile store of the step (see DqDsArgs)
    int32_t ds_ne;          // entries of the step's lists (tiles per (batch, q head))
    int32_t hk0, nhk;       // the launch covers kv heads [hk0, hk0 + nhk)
    int32_t B, S, Skv, Hq, Hkv, nkt, S_pad;
    int32_t total_work;     // B * nhk * nkt
    float scale;            // softmax scale
    float scale_log2;       // softmax scale * log2(e)
};

// dS tile store: one 16 KB tile of bf16 dS = P (dP - Delta) per (batch, q head,
// entry of the dK/dV kernel's lists), i.e. 64 query rows x 128 keys, at tile
// index (b * nh + h - h0) * ds_ne + entry for the q heads [h0, h0 + nh) of the
// launch (the q heads of its kv heads).  Inside a tile the values sit in the
// register order of the dK/dV kernel: u32x4 number (w * 4 + kk) * 64 + lane
// holds, for key 32w + lane%32, the query rows 16kk + 4(lane/32) + {0..3} and
// 16kk + 8 + 4(lane/32) + {0..3} (8 bf16, in that order).
constexpr int DS_TILE_ELEMS = BWD_BQ * BWD_BK;

// K4c: dQ of one ring step from the stored dS tiles (no recomputation).
struct DqDsArgs {
    const uint16_t* k;      // block j: [B, Skv, Hkv, d]
    const uint16_t* ds;     // dS tile store of the step
    const int32_t* t_off;   // [nqt + 1] lists per 256-row query tile
    const int32_t* t_ent;   // 5 ints per entry: 128-key tile, then the dS tile entry
                            // of each 64-row quarter of the query tile (-1: none)
    const int32_t* t_order; // [nqt] query tiles, heaviest first
    float* dq_acc;          // as in DqArgs
    int32_t B, S, Skv, Hq, Hkv, nqt, S_pad;
    int32_t ds_ne;
    int32_t h0, nh;         // the launch covers q heads [h0, h0 + nh)
    int32_t total_work;     // B * nh * nqt
    int32_t first;
    float scale;
};

// K4b: dQ of one ring step.  Uses the forward's per-query-tile lists.
struct DqArgs {
    const uint16_t* q;      // [B, S, Hq, d] bf16
    const uint16_t* k;      // block j: [B, Skv, Hkv, d]
    const uint16_t* v;
    const uint16_t* dout;   // [B, S, Hq, d]
    const float* lse2;      // [B, Hq, S_pad] as in BwdArgs
    const float* ndelta;    // [B, Hq, S_pad]
    const int32_t* rng;     // [S_pad][2]
    const int32_t* t_off;   // [nqt + 1] key-tile lists per 256-row query tile
    const int32_t* t_mid;   // [nqt] first PARTIAL entry of each list
    const int32_t* t_ent;   // key tile index | (partial << 31)
    const int32_t* t_order; // [nqt] query tiles, heaviest first
    float* dq_acc;          // fp32 accumulator in the forward's running-output layout
    int32_t B, S, Skv, Hq, Hkv, nqt, S_pad;
    int32_t total_work;     // B * Hq * nqt (nqt: 256-row query tiles)
    int32_t first;          // first active step: write instead of add
    float scale;
    float scale_log2;
};

// Per-row values of the backward, over the padded rows [B, Hq, S_pad].
struct BwdPreArgs {
    const void* dout;       // [B, S, Hq, d] input dtype
    const void* out;
    const float* lse;       // [B, Hq, S]
    float* lse2;            // [B, Hq, S_pad]
    float* ndelta;          // [B, Hq, S_pad]
    int32_t B, S, Hq, S_pad, d;
};

// Launchers (defined in the .hip files).  Return hipSuccess or the launch error.
hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_fwd_part_merge(const PartMergeArgs& a, hipStream_t s);
hipError_t launch_lse_merge(float* out, float* lse, const float* out_j, const float* lse_j,
                            int32_t B, int64_t S, int32_t H, int32_t d, hipStream_t s);
hipError_t launch_finalize(const float* o, void* out, int is_bf16, int64_t n, hipStream_t s);
hipError_t launch_bwd_pre(const BwdPreArgs& a, int is_bf16, hipStream_t s);
hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dq_bf16(const DqArgs& a, int head_dim, hipStream_t s);
hipError_t launch_bwd_dq_ds_bf16(const DqDsArgs& a, int head_dim, hipStream_t s);
hipError_t launch_dq_finalize(const float* dq_acc, float* dq, int32_t B, int32_t S, int32_t Hq,
                              int32_t S_pad, int32_t d, hipStream_t s);

}  // namespace ra
