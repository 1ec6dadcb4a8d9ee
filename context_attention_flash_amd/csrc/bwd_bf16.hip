// K4: one ring step of the attention backward, bf16 operands, fp32
// accumulation (instagit/nanotron page, "Backward Pass and Gradient
// Accumulation": per step, the flash backward of (dout, q, k_j, v_j, out, lse)
// adds into dq, dk_j and dv_j).  Two kernels share the step:
//
// K4a bwd_dkdv: one work-group = one (batch, kv head, 128-key tile of block
// j); wave w owns keys 32w..32w+31, whose K and V rows stay in registers.  It
// walks every 64-row query tile of every query head of the GQA group that sees
// its keys and computes
//   S = Q K^T and dP = dO V^T        (C layout: lane = key, 16 query rows)
//   P = exp(scale*S - lse), dS = P (dP - Delta)
//   dV^T += dO^T P,  dK^T += Q^T dS  (fp32 accumulators in AGPRs)
// Query tiles stream through two LDS stages (natural rows); dO^T and Q^T
// come from the gfx950 transpose read ds_read_b64_tr_b16 (within each 16-lane
// group, result lane i, element k is the 16-bit value at (address of lane 4k +
// i/4) + 2*(i%4)).
// P and dS feed the MFMAs straight from the accumulator registers, whose query
// order inside each 16-row group is {0-3, 8-11 | 4-7, 12-15} (lanes 0-31 |
// 32-63); the transpose reads pick their rows in that same order.  dK/dV are
// added to the caller's buffers once at the end (one owner per key tile).
//
// K4b bwd_dq: one work-group = one (batch, q head, 256-row query tile); wave w
// owns 64 query rows as two 32-row blocks, lane = query column, Q and dO in
// registers, 64-key tiles of K and V streamed through LDS.  It recomputes
// S^T = K Q^T and dP^T = V dO^T and accumulates dQ^T += K^T dS^T (K^T from
// transpose reads); every LDS operand feeds the MFMAs of both query blocks.
// Each (head, query tile) has one owner per launch, so dQ needs no atomics:
// fp32 atomics on the L2 run about ten times slower than plain stores, and
// the dQ of a key-tile decomposition would be bound by them.
//
// K4c bwd_dq_ds (used when the workspace holds the dS tile store): K4a also
// writes every dS tile it computes (bf16, 16 KB per 64-row x 128-key tile, in
// its register order, four 1 KB stores per wave and tile), and K4c computes
// dQ^T += K^T dS^T from those tiles: one work-group per (batch, q head,
// 256-row query tile), wave w owning the 64-row quarter w, 32-key stages of
// K and of the four quarters' dS streamed through LDS, the dS^T operands taken
// by transpose reads.  This replaces the recomputation of S and dP (4 of
// K4b's 6 flops per pair) by a read of 2 bytes per tile element, written once
// by K4a.
#include <type_traits>

#include "kernel_args.h"
#include "kernel_common.h"

namespace ra {

template <int DH>
struct BwdCfg {
    static constexpr int NT = 256;
    static constexpr int BQ = BWD_BQ, BK = BWD_BK;
    static constexpr int NKS = DH / 16;
    static constexpr int NDT = DH / 32;
    static constexpr int ROWB = DH * 2;             // natural row (bytes)
    static constexpr int KCH = DH / 8;              // 16-byte chunks per natural row
    static constexpr int Q_BYTES = BQ * ROWB;
    // one stage: Q, dO (natural rows), then the row values of the tile:
    // lse2[64], -Delta[64] (fp32) and the key interval [a, b) of each row
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = Q_BYTES;
    static constexpr int OFF_L = 2 * Q_BYTES;
    static constexpr int OFF_ND = OFF_L + 1024;
    static constexpr int OFF_RNG = OFF_ND + 1024;
    static constexpr int STAGE = OFF_RNG + 2048;
    static_assert(BQ * 16 == 1024, "row values: one 16-byte chunk per lane of a wave");
};

template <int NCH>
__device__ __forceinline__ int row_off(int r, int c) { return swz_off<NCH>(r, c); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2_t lds_tr16(const unsigned char* p) {
    const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, r);
}

// MFMA operand (8 bf16 per lane) from a K-major LDS block: rows r1 + j/4 and
// r2 + j/4 (j = lane % 16) give elements 0-3 and 4-7; columns start at c0
// (element index, multiple of 16) + 16 * ((lane / 16) % 2).
template <int NCH>
__device__ __forceinline__ u32x4_t tr_operand(const unsigned char* base, int r1, int r2, int c0,
                                              int lane) {
    const int j = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);   // element index
    const int c = col >> 3, byte = (col & 7) * 2;
    const u32x2_t a = lds_tr16(base + row_off<NCH>(r1 + (j >> 2), c) + byte);
    const u32x2_t b = lds_tr16(base + row_off<NCH>(r2 + (j >> 2), c) + byte);
    return (u32x4_t){a[0], a[1], b[0], b[1]};
}

// One 64-row query tile (head h, tile qt) straight from global memory into a
// stage.  Q and dO come through buffer loads into LDS (buffer_load_dwordx4 ...
// lds: the 16 bytes of lane l land at the wave-uniform LDS base + 16*l).  The
// buffer of a batch entry spans its S rows, so the rows of a last partial tile
// past S read as zeros; the per-lane part of every offset is fixed (voff, the
// XOR swizzle applied through the source chunk as in the dQ kernel) and the
// tile moves only the scalar offset.  Wave 0 also brings the 1 KB of row
// values: lanes 0-15 lse2, 16-31 -Delta, 32-63 the intervals.
template <int DH>
struct DkdvLoader {
    using C = BwdCfg<DH>;
    BufTileLoader<DH, C::BQ> lq, lo;
    // row values: lse2 and -Delta of batch entry b ([Hq][S_pad] each), the
    // intervals ([S_pad][2]); waves 0, 1 and 2 each load 1 KiB of one of them
    // (wave 3 loads lse2 again into a spare slot), so that every wave issues
    // the same instructions and no lane mask splits the loop body
    __amdgpu_buffer_rsrc_t rv;
    int rv_h, rv_q;   // byte offset of the tile: head * rv_h + query tile * rv_q

    __device__ __forceinline__ void init(const BwdArgs& p, int b, int wave, int lane) {
        const int64_t batch = (int64_t)b * p.S * p.Hq * DH;
        lq.init(p.q + batch, p.S, p.Hq, 0, wave, lane);
        lo.init(p.dout + batch, p.S, p.Hq, 0, wave, lane);
        const int rows = p.Hq * p.S_pad * 4;
        const float* base = wave == 1 ? p.ndelta : p.lse2;
        rv_h = wave != 2 ? p.S_pad * 4 : 0;
        rv_q = wave != 2 ? C::BQ * 4 : C::BQ * 8;
        rv = wave == 2 ? __builtin_amdgcn_make_buffer_rsrc((void*)p.rng, (short)0, p.S_pad * 8, 0x00020000)
                       : __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)b * p.Hq * p.S_pad),
                                                           (short)0, rows, 0x00020000);
    }

    __device__ __forceinline__ void load(unsigned char* stage, const BwdArgs& p, int h, int qt,
                                         int wave, int lane) const {
        lq.load(stage + C::OFF_Q, qt, wave, h);
        lo.load(stage + C::OFF_DO, qt, wave, h);
        const int soff = h * rv_h + qt * rv_q;
        auto* dst = (__attribute__((address_space(3))) void*)(stage + C::OFF_L + wave * 1024);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, lane * 16, soff, 0, 0);
    }
};

// Vector instructions the scheduler places after each MFMA (and its two LDS
// reads) in the regions that compute P and dS.
constexpr int K4A_VALU_PER_MFMA = 4;
template <int DH, bool STORE_DS>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_bf16_kernel(BwdArgs p) {
    using C = BwdCfg<DH>;
    // Two stages as separate objects: every access below names its stage
    // statically, which lets the compiler see that the transpose reads of one
    // stage never overlap the direct-to-LDS loads into the other (it would
    // otherwise wait for those loads before every transpose read).
    __shared__ __attribute__((aligned(16))) unsigned char stA[C::STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char stB[C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5,
              l32 = lane & 31;
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nkt, bh = work / p.nkt;
    const int hk = p.hk0 + bh % p.nhk, b = bh / p.nhk;
    const cint_ptr ents = as_const(p.t_ent);
    const int kt = as_const(p.t_order)[t];
    const int e0 = as_const(p.t_off)[kt], e1 = as_const(p.t_off)[kt + 1];
    const int group = p.Hq / p.Hkv;
    // the list holds the FULL tiles first, the PARTIAL ones from entry m on;
    // iterations [0, nF) walk the full tiles of every head of the group, the
    // rest the partial ones
    const int m = as_const(p.t_mid)[kt];
    const int nF = (m - e0) * group;
    const int n_iter = (e1 - e0) * group;

    const int kv_stride = p.Hkv * DH;
    const int key = kt * C::BK + wave * 32 + l32;   // this lane's key (C-layout column)
    const int keyc = min(key, p.Skv - 1);

    // This lane's K and V row are the B operands of S and dP for every tile.
    u32x4_t kreg[C::NKS], vreg[C::NKS];
    {
        const uint16_t* kr = p.k + ((int64_t)b * p.Skv + keyc) * kv_stride + hk * DH;
        const uint16_t* vr = p.v + ((int64_t)b * p.Skv + keyc) * kv_stride + hk * DH;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            kreg[ks] = *(const u32x4_t*)(kr + 16 * ks + 8 * g);
            vreg[ks] = *(const u32x4_t*)(vr + 16 * ks + 8 * g);
        }
    }

    f32x16_t dk_acc[C::NDT], dv_acc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        dk_acc[dt] = (f32x16_t){};
        dv_acc[dt] = (f32x16_t){};
    }
    const float c2 = p.scale_log2;

    // Per-lane LDS offsets.  Every swizzle below depends only on the low four
    // bits of the row, so moving by 16 or 32 rows is a constant offset.
    //   nat[ks]    : natural read of row l32, chunk 2ks+g (S and dP operands)
    //   trq[r][dt] : transpose read of rows {4g, 8+4g} + j/4, head-dim block dt
    const int j = lane & 15, gsel = (lane >> 4) & 1;
    int nat[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) nat[ks] = row_off<C::KCH>(l32, 2 * ks + g);
    int trq[2][C::NDT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int col = 32 * dt + 16 * gsel + 4 * (j & 3);
            trq[r][dt] = row_off<C::KCH>(8 * r + 4 * g + (j >> 2), col >> 3) + (col & 7) * 2;
        }

    // Iteration it -> (query head, list entry).  The entry of the next tile
    // is fetched one iteration ahead so that its scalar load is off the path.
    DkdvLoader<DH> ld;
    ld.init(p, b, wave, lane);
    // Iteration cursor: the full tiles of every q head of the group, then the
    // partial ones; (hd, jt) = (q head within the group, position in the
    // class's list), base and n = that class's first entry and length.  It
    // advances by additions only (no division per iteration).
    struct Cursor {
        int hd, jt, base, n;
    };
    auto advance = [&](Cursor c) {
        if (++c.jt == c.n) {
            c.jt = 0;
            if (++c.hd == group && c.base == e0 && m != e0) {   // full tiles done
                c.hd = 0;
                c.base = m;
                c.n = e1 - m;
            }
        }
        return c;
    };
    auto index_of = [&](const Cursor& c) { return c.base + c.jt; };
    auto head_of = [&](const Cursor& c) { return hk * group + c.hd; };
    auto load = [&](const Cursor& c, int ent, unsigned char* st) {
        ld.load(st, p, head_of(c), ent & 0x7fffffff, wave, lane);
    };

    // S = Q K^T and dP - Delta = dO V^T - Delta for the 32-row half mt of the
    // tile in stage `st`, in two parts: the LDS reads (the A operands and -Delta
    // of the half's rows, element r being query row 32*mt + 8*(r/4) + 4*g +
    // r%4), issued one scheduling region ahead, and the MFMAs; the dP
    // accumulators start from -Delta.
    struct SOps {
        u32x4_t qa[C::NKS], oa[C::NKS];
        f32x16_t nd;
        f32x4_t L[4];        // lse2 of the half's rows, used by p_half
        int4 ab[4][2];       // their key intervals (masked tiles only)
    };
    auto s_read = [&](const unsigned char* st, int mt, SOps& o, auto partial_tag) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        // -Delta first: the first dP MFMA needs all of it
        const float* nd = (const float*)(st + C::OFF_ND);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const f32x4_t x = *(const f32x4_t*)(nd + 32 * mt + 8 * rg + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) o.nd[4 * rg + i] = x[i];
        }
        const float* L2 = (const float*)(st + C::OFF_L);
        const int32_t* R = (const int32_t*)(st + C::OFF_RNG);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const int r0 = 32 * mt + 8 * rg + 4 * g;
            o.L[rg] = *(const f32x4_t*)(L2 + r0);
            if (PARTIAL) {
                o.ab[rg][0] = *(const int4*)(R + 2 * r0);
                o.ab[rg][1] = *(const int4*)(R + 2 * r0 + 4);
            }
        }
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            o.qa[ks] = *(const u32x4_t*)(st + C::OFF_Q + nat[ks] + mt * 32 * C::ROWB);
            o.oa[ks] = *(const u32x4_t*)(st + C::OFF_DO + nat[ks] + mt * 32 * C::ROWB);
        }
    };
    auto s_mfma = [&](const SOps& o, f32x16_t& sacc, f32x16_t& pacc) {
        sacc = (f32x16_t){};
        pacc = o.nd;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            sacc = mfma_32x32x16(o.qa[ks], kreg[ks], sacc);
            pacc = mfma_32x32x16(o.oa[ks], vreg[ks], pacc);
        }
    };

    // P = exp2(S * scale * log2(e) - lse2) and dS = P (dP - Delta) of half mt,
    // packed to bf16 as the B operands of dV^T and dK^T for the query blocks
    // kk = 2*mt and 2*mt + 1.
    auto p_half = [&](const SOps& o, int mt, auto partial_tag, const f32x16_t& sacc,
                      const f32x16_t& pacc, u32x4_t (&pb)[2], u32x4_t (&db)[2], uint16_t* ds_tile) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            const f32x4_t L = o.L[rg];
            float pr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(fmaf(sacc[4 * rg + i], c2, -L[i]));
            if (PARTIAL) {  // keys outside a row's interval [a, b) are invisible
                const int4 ab0 = o.ab[rg][0];
                const int4 ab1 = o.ab[rg][1];
                const int av[4] = {ab0.x, ab0.z, ab1.x, ab1.z};
                const int bv[4] = {ab0.y, ab0.w, ab1.y, ab1.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[i] = ((key >= av[i]) & (key < bv[i])) ? pr[i] : 0.f;
            }
            float ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ds[i] = pr[i] * pacc[4 * rg + i];
            const int kk = rg >> 1, w = (rg & 1) * 2;
            pb[kk][w] = pack_bf16x2(pr[0], pr[1]);
            pb[kk][w + 1] = pack_bf16x2(pr[2], pr[3]);
            db[kk][w] = pack_bf16x2(ds[0], ds[1]);
            db[kk][w + 1] = pack_bf16x2(ds[2], ds[3]);
        }
        if constexpr (STORE_DS) {   // the dS tile store, in this register order
            // non-temporal: the tile is read once, by the dQ kernel, after
            // the whole launch; streaming it out keeps the caches for Q and dO
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                (void*)ds_tile, (short)0, DS_TILE_ELEMS * 2, 0x00020000);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                __builtin_amdgcn_raw_buffer_store_b128(db[kk], r, (wave * 256 + lane) * 16,
                                                       (2 * mt + kk) * 1024, 2);
        }
    };

    // dV^T += dO^T P and dK^T += Q^T dS over the query rows of half mt; the K
    // dimension of query block kk = 2*mt + k2 takes rows 16kk + 4g + 0..3 and
    // 16kk + 8 + 4g + 0..3.
    // The transposed operands of half mt of the tile in stage st, all head-dim
    // blocks (the dV/dK MFMAs of that half then need no LDS read).
    auto read_half = [&](const unsigned char* st, int mt, u32x4_t (&oa)[C::NDT][2],
                         u32x4_t (&qa)[C::NDT][2]) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int o16 = (2 * mt + k2) * 16 * C::ROWB;
                const u32x2_t o1 = lds_tr16(st + C::OFF_DO + trq[0][dt] + o16);
                const u32x2_t o2 = lds_tr16(st + C::OFF_DO + trq[1][dt] + o16);
                const u32x2_t q1 = lds_tr16(st + C::OFF_Q + trq[0][dt] + o16);
                const u32x2_t q2 = lds_tr16(st + C::OFF_Q + trq[1][dt] + o16);
                oa[dt][k2] = (u32x4_t){o1[0], o1[1], o2[0], o2[1]};
                qa[dt][k2] = (u32x4_t){q1[0], q1[1], q2[0], q2[1]};
            }
    };
    auto mfma_half = [&](const u32x4_t (&oa)[C::NDT][2], const u32x4_t (&qa)[C::NDT][2],
                         const u32x4_t (&pb)[2], const u32x4_t (&db)[2]) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                dv_acc[dt] = mfma_32x32x16(oa[dt][k2], pb[k2], dv_acc[dt]);
                dk_acc[dt] = mfma_32x32x16(qa[dt][k2], db[k2], dk_acc[dt]);
            }
    };

    // dV/dK of the second half of a tile run in the next iteration, after its
    // barrier: their operands (read below, at the end of the tile) and P/dS
    // wait in registers, and the MFMAs execute while the wave issues the next
    // tile's loads.  Every LDS read of a stage is complete before that
    // barrier, so two stages still suffice.  Zero-initialised, the first
    // iteration's carried MFMAs add nothing.
    u32x4_t c_oa[C::NDT][2], c_qa[C::NDT][2], c_pb[2], c_db[2];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) c_oa[dt][k2] = c_qa[dt][k2] = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) c_pb[k2] = c_db[k2] = (u32x4_t){0u, 0u, 0u, 0u};

    // One query tile, pipelined in halves: S/dP of half 1 run on the matrix
    // cores while P/dS of half 0 run on the vector ALUs, then dV/dK of half 0
    // while P/dS of half 1; the operands of half 1's dV/dK are read last.
    // Scheduling fences split the tile into regions; the LDS reads of each
    // region's MFMAs (and the row values its vector work needs) are issued in
    // the region before, so that the MFMAs do not wait for them, and the
    // fences bound the registers in flight.  Inside a region, group barriers
    // interleave the MFMAs with the LDS reads and the vector work: with one
    // wave per SIMD nothing else fills the matrix pipe while the wave issues
    // a run of other instructions.
    auto tile = [&](const unsigned char* st, auto partial_tag, uint16_t* ds_tile, const SOps& o0) {
        f32x16_t s0, p0, s1, p1;
        u32x4_t pb0[2], db0[2];
        SOps o1;
        u32x4_t oa[C::NDT][2], qa[C::NDT][2];
        s_mfma(o0, s0, p0);
        s_read(st, 1, o1, partial_tag);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        s_mfma(o1, s1, p1);
        p_half(o0, 0, partial_tag, s0, p0, pb0, db0, ds_tile);
        read_half(st, 0, oa, qa);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            __builtin_amdgcn_sched_group_barrier(0x002, K4A_VALU_PER_MFMA, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_half(oa, qa, pb0, db0);
        p_half(o1, 1, partial_tag, s1, p1, c_pb, c_db, ds_tile);
        read_half(st, 1, c_oa, c_qa);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
            __builtin_amdgcn_sched_group_barrier(0x002, K4A_VALU_PER_MFMA, 3);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Iteration it: the barrier that makes tile it visible and frees the
    // other stage; then, in one region, the loads of tile it+1 into that
    // stage, the LDS reads of half 0 of tile it and the carried dV/dK MFMAs
    // of tile it-1, interleaved so that the MFMAs run while the wave issues
    // the loads (each direct-to-LDS load holds the wave for about as long as
    // an MFMA executes).  The last iteration loads a tile again (the loads
    // are unconditional, so that no branch splits the region).  Even
    // iterations use stage A, odd ones stage B.
    // cursors of tiles it, it+1 and it+2
    Cursor cu0 = m != e0 ? Cursor{0, 0, e0, m - e0} : Cursor{0, 0, m, e1 - m};
    Cursor cu1 = advance(cu0), cu2 = advance(cu1);
    int ent_nx = n_iter > 1 ? ents[index_of(cu1)] : 0;   // entry of tile it+1
    auto step = [&](int it, unsigned char* cur, unsigned char* nxt, auto partial_tag) {
        // this wave's loads of tile it have landed; with the dS store, the
        // four dS stores of tile it-1, issued after those loads, may still be
        // in flight (vmcnt <= 4: vector memory operations complete in order)
        __builtin_amdgcn_s_waitcnt(STORE_DS ? 0x0004 : 0);
        __syncthreads();
        {
            const bool more = it + 1 < n_iter;
            const Cursor cl = more ? cu1 : cu0;
            load(cl, ent_nx, nxt);
        }
        SOps o0;
        s_read(cur, 0, o0, partial_tag);
        mfma_half(c_oa, c_qa, c_pb, c_db);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+a"(dk_acc[dt]), "+a"(dv_acc[dt]));
        uint16_t* ds_tile = nullptr;   // this tile's place in the dS tile store
        if constexpr (STORE_DS)
            ds_tile = p.ds + ((int64_t)(b * p.nhk + hk - p.hk0) * group + cu0.hd) * p.ds_ne * DS_TILE_ELEMS +
                      (int64_t)index_of(cu0) * DS_TILE_ELEMS;
        tile(cur, partial_tag, ds_tile, o0);
        // the scalar load goes out after the tile's LDS reads: while it is in
        // flight every LDS wait must be a full one (scalar loads return out of
        // order)
        if (it + 2 < n_iter) ent_nx = ents[index_of(cu2)];
        cu0 = cu1;
        cu1 = cu2;
        cu2 = advance(cu2);
    };
    // The unmasked loop covers an even number of iterations; a last full tile
    // left over goes through the masked loop, where the mask keeps every key.
    const int nF2 = nF & ~1;
    if (n_iter > 0) load(cu0, ents[index_of(cu0)], stA);
    if constexpr (STORE_DS) __builtin_amdgcn_s_waitcnt(0);   // the first wait counts on none in flight
    int it = 0;
    for (; it < nF2; it += 2) {
        step(it, stA, stB, std::false_type{});
        step(it + 1, stB, stA, std::false_type{});
    }
    for (; it < n_iter; it += 2) {
        step(it, stA, stB, std::true_type{});
        if (it + 1 < n_iter) step(it + 1, stB, stA, std::true_type{});
    }
    mfma_half(c_oa, c_qa, c_pb, c_db);   // the last tile's second half
    // the last iteration's load (of a tile nobody reads) lands before the
    // work-group can end and release its LDS
    __builtin_amdgcn_s_waitcnt(0);

    // dK_j += scale * dK^T acc, dV_j += dV^T acc (this lane's key, DH head-dim
    // values of each).  Every load is issued before the first store: a store
    // to dK may alias a later load of dV as far as the compiler knows, so
    // interleaved load-add-store would wait for a memory round trip per pair.
    if (key < p.Skv) {
        float* dkr = p.dk + ((int64_t)b * p.Skv + key) * kv_stride + hk * DH;
        float* dvr = p.dv + ((int64_t)b * p.Skv + key) * kv_stride + hk * DH;
        f32x4_t xk[C::NDT][4], xv[C::NDT][4];
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = 32 * dt + 8 * rg + 4 * g;
                xk[dt][rg] = *(const f32x4_t*)(dkr + d0);
                xv[dt][rg] = *(const f32x4_t*)(dvr + d0);
            }
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = 32 * dt + 8 * rg + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xk[dt][rg][i] += p.scale * dk_acc[dt][4 * rg + i];
                    xv[dt][rg][i] += dv_acc[dt][4 * rg + i];
                }
                *(f32x4_t*)(dkr + d0) = xk[dt][rg];
                *(f32x4_t*)(dvr + d0) = xv[dt][rg];
            }
    }
}

// Explicit instantiations: with several specialisations of one kernel
// template launched from one function, the host pass emitted the launch stub
// of the first one only (the build checks the library for missing stubs).
template __global__ void bwd_dkdv_bf16_kernel<128, true>(BwdArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, false>(BwdArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, true>(BwdArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, false>(BwdArgs);

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    const bool st = a.ds != nullptr;
    if (head_dim == 128 && st)
        hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64 && st)
        hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K4b: dQ of one ring step (query-stationary, no atomics)
// ---------------------------------------------------------------------------

template <int DH>
struct DqCfg {
    static constexpr int NT = 256;
    static constexpr int BQ = DQ_BQ, BK = DQ_BK;     // 4 waves x 64 queries, 64 keys
    static constexpr int NKS = DH / 16;
    static constexpr int NDT = DH / 32;
    static constexpr int ROWB = DH * 2;
    static constexpr int KCH = DH / 8;
    static constexpr int K_BYTES = BK * ROWB;
    static constexpr int STAGE = 2 * K_BYTES;        // K and V tiles, natural rows
};

template <int DH>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dq_bf16_kernel(DqArgs p) {
    using C = DqCfg<DH>;
    // two stages as separate objects, named statically below (see the dK/dV
    // kernel: the transpose reads then need not wait for the loads in flight)
    __shared__ __attribute__((aligned(16))) unsigned char stA[C::STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char stB[C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nqt, bh = work / p.nqt;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int qt = as_const(p.t_order)[t];
    const int hk = (h * p.Hkv) / p.Hq;
    const cint_ptr ents = as_const(p.t_ent);
    const int e0 = as_const(p.t_off)[qt], e1 = as_const(p.t_off)[qt + 1];
    const int m = as_const(p.t_mid)[qt];   // FULL tiles in [e0, m), PARTIAL in [m, e1)

    // Wave w owns query rows qt*256 + 64w + 32qb + l32 for qb = 0, 1: every K
    // or V operand read from LDS feeds the MFMAs of both query blocks.
    const int q_stride = p.Hq * DH;
    u32x4_t qreg[2][C::NKS], oreg[2][C::NKS];
    float L2[2], nD[2];
    int ra[2], rb[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int iq = qt * C::BQ + wave * 64 + qb * 32 + l32;   // < S_pad
        const int iqc = min(iq, p.S - 1);
        const uint16_t* qrow = p.q + ((int64_t)b * p.S + iqc) * q_stride + h * DH;
        const uint16_t* orow = p.dout + ((int64_t)b * p.S + iqc) * q_stride + h * DH;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            qreg[qb][ks] = *(const u32x4_t*)(qrow + 16 * ks + 8 * g);
            oreg[qb][ks] = *(const u32x4_t*)(orow + 16 * ks + 8 * g);
        }
        L2[qb] = p.lse2[((int64_t)b * p.Hq + h) * p.S_pad + iq];   // +inf on padding rows
        nD[qb] = p.ndelta[((int64_t)b * p.Hq + h) * p.S_pad + iq];
        ra[qb] = p.rng[2 * iq];
        rb[qb] = p.rng[2 * iq + 1];
    }

    KvLoader<DH, C::BK> ld;   // K and V tiles of 64 keys
    ld.init(p.k, p.v, b, p.Skv, p.Hkv, hk, wave, lane);

    // per-lane LDS offsets (see the dK/dV kernel): natural reads of key row
    // l32 (+32 per key half), chunk 2ks+g; transpose reads of key rows
    // {4g, 8+4g} + j/4 (+16 per key step), head-dim block dt
    const int j = lane & 15, gsel = (lane >> 4) & 1;
    int nat[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) nat[ks] = row_off<C::KCH>(l32, 2 * ks + g);
    int trk[2][C::NDT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int col = 32 * dt + 16 * gsel + 4 * (j & 3);
            trk[r][dt] = row_off<C::KCH>(8 * r + 4 * g + (j >> 2), col >> 3) + (col & 7) * 2;
        }

    f32x16_t acc[2][C::NDT];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) acc[qb][dt] = (f32x16_t){};
    const float c2 = p.scale_log2;

    // Key half kh (keys 32kh .. 32kh+31 of the tile) of stage `st`:
    // S^T = K Q^T and dP^T = V dO^T for both query blocks (element r of a
    // block is key 32kh + 8*(r/4) + 4*g + r%4), the A operands read one
    // scheduling region ahead.
    struct SOps {
        u32x4_t ka[C::NKS], va[C::NKS];
    };
    auto s_read = [&](const unsigned char* st, int kh, SOps& o) {
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            o.ka[ks] = *(const u32x4_t*)(st + nat[ks] + kh * 32 * C::ROWB);
            o.va[ks] = *(const u32x4_t*)(st + C::K_BYTES + nat[ks] + kh * 32 * C::ROWB);
        }
    };
    auto s_mfma = [&](const SOps& o, f32x16_t (&sacc)[2], f32x16_t (&pacc)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            sacc[qb] = (f32x16_t){};
            pacc[qb] = (f32x16_t){};
        }
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                sacc[qb] = mfma_32x32x16(o.ka[ks], qreg[qb][ks], sacc[qb]);
                pacc[qb] = mfma_32x32x16(o.va[ks], oreg[qb][ks], pacc[qb]);
            }
    };
    // P = exp(scale*S - lse), dS = P (dP - Delta), packed to bf16 as the B
    // operands of dQ^T for the two 16-key steps of the half
    auto p_half = [&](int kt, int kh, auto partial_tag, const f32x16_t (&sacc)[2],
                      const f32x16_t (&pacc)[2], u32x4_t (&db)[2][2]) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float pv[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    float pr = fast_exp2(fmaf(sacc[qb][r + u], c2, -L2[qb]));
                    if (PARTIAL) {  // keys outside [ra, rb) are invisible
                        const int key = kt * C::BK + 32 * kh + 8 * ((r + u) >> 2) + 4 * g + ((r + u) & 3);
                        pr = ((key >= ra[qb]) & (key < rb[qb])) ? pr : 0.f;
                    }
                    pv[u] = pr * (pacc[qb][r + u] + nD[qb]);
                }
                db[qb][r >> 3][(r & 7) >> 1] = pack_bf16x2(pv[0], pv[1]);
            }
    };
    // K^T operands of half kh: the K dimension (keys) of step kk takes rows
    // 32kh + 16kk + 4g + 0..3 and 32kh + 16kk + 8 + 4g + 0..3, as dS is held
    auto t_read = [&](const unsigned char* st, int kh, u32x4_t (&kt4)[2][C::NDT]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                const int o = (2 * kh + kk) * 16 * C::ROWB;
                const u32x2_t a1 = lds_tr16(st + trk[0][dt] + o);
                const u32x2_t a2 = lds_tr16(st + trk[1][dt] + o);
                kt4[kk][dt] = (u32x4_t){a1[0], a1[1], a2[0], a2[1]};
            }
    };
    auto q_mfma = [&](const u32x4_t (&kt4)[2][C::NDT], const u32x4_t (&db)[2][2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    acc[qb][dt] = mfma_32x32x16(kt4[kk][dt], db[qb][kk], acc[qb][dt]);
    };

    // dQ of the second key half runs at the start of the next iteration,
    // before its barrier (as in the dK/dV kernel); zero operands at first.
    u32x4_t c_kt[2][C::NDT], c_db[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) c_kt[kk][dt] = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) c_db[qb][kk] = (u32x4_t){0u, 0u, 0u, 0u};
    }

    // One key tile in four scheduling regions: S/dP of half 0; S/dP of half
    // 1 with P/dS of half 0; dQ of half 0 with P/dS of half 1 (and the K^T
    // reads of half 1, for the carried dQ).  Each region's LDS reads are
    // issued in the region before.
    auto tile = [&](const unsigned char* st, int kt, auto partial_tag) {
        f32x16_t s0[2], p0[2], s1[2], p1[2];
        u32x4_t db0[2][2];
        SOps o0, o1;
        u32x4_t kt0[2][C::NDT];
        s_read(st, 0, o0);
        __builtin_amdgcn_sched_barrier(0);
        s_mfma(o0, s0, p0);
        s_read(st, 1, o1);
        __builtin_amdgcn_sched_barrier(0);
        s_mfma(o1, s1, p1);
        p_half(kt, 0, partial_tag, s0, p0, db0);
        t_read(st, 0, kt0);
        __builtin_amdgcn_sched_barrier(0);
        q_mfma(kt0, db0);
        p_half(kt, 1, partial_tag, s1, p1, c_db);
        t_read(st, 1, c_kt);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Two LDS stages, even list positions in stage A: the barrier at the top
    // of position i makes tile i visible and frees the other stage, which
    // then receives tile i+1.  The entry of tile i+1 is fetched a position
    // ahead.  Full tiles run unmasked in pairs; a last odd full tile joins the
    // masked loop (its mask keeps every key).
    const int n = e1 - e0;
    const int nF2 = (m - e0) & ~1;
    int ent_nx = n > 1 ? ents[e0 + 1] : 0;
    auto step = [&](int i, const unsigned char* cur, unsigned char* nxt, auto partial_tag) {
        q_mfma(c_kt, c_db);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+a"(acc[qb][dt]));
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile i have landed
        __syncthreads();
        if (i + 1 < n) ld.load(nxt, nxt + C::K_BYTES, ent_nx & 0x7fffffff, wave);
        const int kt = ents[e0 + i] & 0x7fffffff;
        tile(cur, kt, partial_tag);
        if (i + 2 < n) ent_nx = ents[e0 + i + 2];
    };
    if (n > 0) ld.load(stA, stA + C::K_BYTES, ents[e0] & 0x7fffffff, wave);
    int i = 0;
    for (; i < nF2; i += 2) {
        step(i, stA, stB, std::false_type{});
        step(i + 1, stB, stA, std::false_type{});
    }
    for (; i < n; i += 2) {
        step(i, stA, stB, std::true_type{});
        if (i + 1 < n) step(i + 1, stB, stA, std::true_type{});
    }
    q_mfma(c_kt, c_db);   // the last tile's second half

    // dq_acc (+)= scale * acc in the accumulator layout: element (dt, r) of
    // query block qb is head-dim index 32*dt + 8*(r/4) + 4*g + r%4 of query
    // row qt*256 + 64*wave + 32*qb + l32.
    // (one branch on `first` for the whole update, and all loads of a 32-row
    // block issued before its stores: per element, the branch split the
    // update into one load-wait-store round trip each)
    const bool add = !p.first;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        f32x4_t* dst = (f32x4_t*)p.dq_acc +
                       (((int64_t)b * p.Hq + h) * (p.S_pad / 32) + (qt * 8 + wave * 2 + qb)) * (8 * DH) + lane;
        f32x4_t old[C::NDT][4];
        if (add) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) old[dt][rg] = dst[(dt * 4 + rg) * 64];
        }
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4_t o = {acc[qb][dt][4 * rg] * p.scale, acc[qb][dt][4 * rg + 1] * p.scale,
                             acc[qb][dt][4 * rg + 2] * p.scale, acc[qb][dt][4 * rg + 3] * p.scale};
                if (add) o += old[dt][rg];
                dst[(dt * 4 + rg) * 64] = o;
            }
    }
}

hipError_t launch_bwd_dq_bf16(const DqArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL(bwd_dq_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL(bwd_dq_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K4c: dQ of one ring step from the dS tiles stored by K4a (no recompute)
// ---------------------------------------------------------------------------

template <int DH>
struct DsCfg {
    static constexpr int KH = 32;                       // keys per stage (a quarter of a dS tile)
    static constexpr int NDT = DH / 32;
    static constexpr int ROWB = DH * 2;
    static constexpr int KCH = DH / 8;
    static constexpr int DS_BYTES = BWD_BQ * KH * 2;    // one quarter's dS over KH keys: 4 KB
    static constexpr int NDS = DS_BYTES / 1024;         // 1 KB loads per wave
    static constexpr int SPT = BWD_BK / KH;             // stages per dS tile
    static constexpr int OFF_K = 4 * DS_BYTES;
    static constexpr int STAGE = OFF_K + KH * ROWB;     // + the K rows of those keys
};

// LDS place of 16-byte chunk f of a quarter's dS over one 32-key group
// (f = kk*64 + lane in the stored register order): bits 2 and 3 of f are
// flipped by bits 6 and 5, which makes the transpose reads below touch every
// bank once per half-wave.  The map is its own inverse.
__device__ __forceinline__ int ds_pos(int f) {
    return f ^ ((((f >> 6) & 1) << 2) | (((f >> 5) & 1) << 3));
}

// One wave's quarter of a dS tile over KH keys (NDS KB, starting at byte
// `soff` of the 16 KB tile) into LDS, each chunk f at ds_pos(f).  dS is read
// once, so the loads are non-temporal; a quarter without a tile (present ==
// false) reads zeros through an empty buffer range.
template <int NDS>
struct DsQuarterLoader {
    int dvo[NDS];
    __device__ __forceinline__ void init(int lane) {
#pragma unroll
        for (int i = 0; i < NDS; ++i) dvo[i] = 16 * ds_pos(64 * i + lane);
    }
    __device__ __forceinline__ void load(unsigned char* lds, const uint16_t* tile, bool present,
                                         int soff) const {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)tile, (short)0, present ? DS_TILE_ELEMS * 2 : 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < NDS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(lds + 1024 * i), 16, dvo[i], soff, 0, 2);
    }
};

template <int DH>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_bf16_kernel(DqDsArgs p) {
    using C = DsCfg<DH>;
    __shared__ __attribute__((aligned(16))) unsigned char stA[C::STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char stB[C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nqt, bh = work / p.nqt;
    const int h = p.h0 + bh % p.nh, b = bh / p.nh;
    const int qt = as_const(p.t_order)[t];
    const int hk = (h * p.Hkv) / p.Hq;
    const cint_ptr ents = as_const(p.t_ent);
    const int e0 = as_const(p.t_off)[qt], e1 = as_const(p.t_off)[qt + 1];
    const int n_iter = C::SPT * (e1 - e0);   // SPT stages per 128-key tile

    // K rows of the stage (KH keys of head hk) and this wave's quarter of dS
    BufTileLoader<DH, C::KH> lk;
    lk.init(p.k + (int64_t)b * p.Skv * p.Hkv * DH, p.Skv, p.Hkv, hk, wave, lane);
    DsQuarterLoader<C::NDS> lds_ds;
    lds_ds.init(lane);
    const uint16_t* ds_head = p.ds + (int64_t)(b * p.nh + h - p.h0) * p.ds_ne * DS_TILE_ELEMS;
    // iteration it: key tile kt = entry (it/SPT), keys KH*(it%SPT).. of it
    auto load = [&](int it, int kt, int e, unsigned char* st) {
        lk.load(st + C::OFF_K, C::SPT * kt + it % C::SPT, wave);
        lds_ds.load(st + wave * C::DS_BYTES, e >= 0 ? ds_head + (int64_t)e * DS_TILE_ELEMS : p.ds,
                    e >= 0, (it % C::SPT) * C::DS_BYTES);
    };

    // Transpose-read offsets.  dS^T operand (B) of query block qb, key step
    // ks: lane L takes query 32qb + L%32 and keys 16ks + 8(L/32) + 0..7; the
    // reading lane s of each 16-lane group G points at query rows
    // 32qb + 16(G%2) + 4(s%4) .. +3 of key 16ks + 8(G/2) + 4r + s/4.
    const int G = lane >> 4, sl = lane & 15, c = sl & 3, kq = sl >> 2;
    int dsr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int f = (G & 1) * 64 + 32 * (c & 1) + 8 * (G >> 1) + 4 * r + kq;
        dsr[r] = wave * C::DS_BYTES + 16 * ds_pos(f) + 8 * (c >> 1);
    }
    // K^T operand (A) of head-dim block dt, key step ks: rows (keys)
    // 16ks + 8(L/32) + 4r + j/4, columns 32dt + 16((L/16)%2) + 4(j%4)
    const int j = lane & 15, gsel = (lane >> 4) & 1, hsel = lane >> 5;
    int trk[2][C::NDT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int col = 32 * dt + 16 * gsel + 4 * (j & 3);
            trk[r][dt] = C::OFF_K + row_off<C::KCH>(8 * hsel + 4 * r + (j >> 2), col >> 3) + (col & 7) * 2;
        }

    f32x16_t acc[2][C::NDT];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) acc[qb][dt] = (f32x16_t){};

    // Operands of key step ks (16 keys) of stage st.
    static_assert(C::KH == 32, "two key steps per stage");
    struct Ops {
        u32x4_t ka[C::NDT], da[2];
    };
    auto read_ks = [&](const unsigned char* st, int ks, Ops& o) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const u32x2_t a1 = lds_tr16(st + trk[0][dt] + ks * 16 * C::ROWB);
            const u32x2_t a2 = lds_tr16(st + trk[1][dt] + ks * 16 * C::ROWB);
            o.ka[dt] = (u32x4_t){a1[0], a1[1], a2[0], a2[1]};
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int off = 2048 * qb + 256 * ks;
            const u32x2_t d1 = lds_tr16(st + dsr[0] + off);
            const u32x2_t d2 = lds_tr16(st + dsr[1] + off);
            o.da[qb] = (u32x4_t){d1[0], d1[1], d2[0], d2[1]};
        }
    };
    auto mfma_ks = [&](const Ops& o) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                acc[qb][dt] = mfma_32x32x16(o.ka[dt], o.da[qb], acc[qb][dt]);
    };

    // The second key step of a stage runs at the start of the next iteration,
    // before its barrier (zero operands at first, adding nothing).
    Ops c_ops;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) c_ops.ka[dt] = (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) c_ops.da[qb] = (u32x4_t){0u, 0u, 0u, 0u};
    auto tile = [&](const unsigned char* st) {
        Ops o0;
        read_ks(st, 0, o0);
        __builtin_amdgcn_sched_barrier(0);
        mfma_ks(o0);
        read_ks(st, 1, c_ops);
        __builtin_amdgcn_sched_barrier(0);
    };

    // the list entry (key tile, this quarter's dS entry) of iteration it + 1
    auto kt_of = [&](int it) { return ents[5 * (e0 + it / C::SPT)]; };
    auto e_of = [&](int it) { return ents[5 * (e0 + it / C::SPT) + 1 + wave]; };
    int kt_nx = n_iter > 1 ? kt_of(1) : 0, e_nx = n_iter > 1 ? e_of(1) : -1;
    auto step = [&](int it, const unsigned char* cur, unsigned char* nxt) {
        mfma_ks(c_ops);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+a"(acc[qb][dt]));
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage it have landed
        __syncthreads();
        if (it + 1 < n_iter) load(it + 1, kt_nx, e_nx, nxt);
        tile(cur);
        if (it + 2 < n_iter) {
            kt_nx = kt_of(it + 2);
            e_nx = e_of(it + 2);
        }
    };
    if (n_iter > 0) load(0, kt_of(0), e_of(0), stA);
    for (int it = 0; it < n_iter; it += 2) {   // n_iter is even
        step(it, stA, stB);
        step(it + 1, stB, stA);
    }
    mfma_ks(c_ops);

    // dq_acc (+)= scale * acc, in the layout of the recomputing dQ kernel
    // (one branch on `first` for the whole update, and all loads of a 32-row
    // block issued before its stores: per element, the branch split the
    // update into one load-wait-store round trip each)
    const bool add = !p.first;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        f32x4_t* dst = (f32x4_t*)p.dq_acc +
                       (((int64_t)b * p.Hq + h) * (p.S_pad / 32) + (qt * 8 + wave * 2 + qb)) * (8 * DH) + lane;
        f32x4_t old[C::NDT][4];
        if (add) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) old[dt][rg] = dst[(dt * 4 + rg) * 64];
        }
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4_t o = {acc[qb][dt][4 * rg] * p.scale, acc[qb][dt][4 * rg + 1] * p.scale,
                             acc[qb][dt][4 * rg + 2] * p.scale, acc[qb][dt][4 * rg + 3] * p.scale};
                if (add) o += old[dt][rg];
                dst[(dt * 4 + rg) * 64] = o;
            }
    }
}

template __global__ void bwd_dq_ds_bf16_kernel<128>(DqDsArgs);
template __global__ void bwd_dq_ds_bf16_kernel<64>(DqDsArgs);

hipError_t launch_bwd_dq_ds_bf16(const DqDsArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL(bwd_dq_ds_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL(bwd_dq_ds_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
