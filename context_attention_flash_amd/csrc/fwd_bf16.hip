// K1: one ring step of the flash forward, bf16 inputs, fp32 accumulation.
//
// One work-group = one (batch, q head, 256-row query tile), eight waves of 32
// rows (two per SIMD, so that one wave's softmax overlaps the other's MFMAs,
// and each K/V tile in LDS serves eight waves); it walks the
// step's list of 64-key tiles of block j (instagit/nanotron page, "Forward
// Pass Implementation": one flash call per ring step) with an online softmax
// (ai360xpert "Ring Attention", "Online softmax across ring steps") and ends
// with the step's epilogue: write, merge ("Numerically-Stable Output Fusion")
// or finalise the running result.
//
// Per wave (32 query rows) and key tile:
//   S^T[64 x 32] = K[64 x d] * Q^T[d x 32]   (v_mfma_f32_32x32x16_bf16)
//   so each lane owns one query column: its 32 scores are in-lane and the
//   other 32 sit in lane ^ 32 (one permlane32 swap for the row max);
//   P = exp2(S * scale*log2e - m) in fp32, rounded to bf16;
//   O^T[d x 32] += V^T[d x 64] * P^T[64 x 32]; the P^T operand is read
//   straight from the S^T accumulator registers, which hold keys
//   {0-3, 8-11} (lanes 0-31) and {4-7, 12-15} (lanes 32-63) of every 16-key
//   step; V^T comes from the gfx950 LDS transpose read ds_read_b64_tr_b16 on
//   the natural V rows, picking the key rows in that same order.
// K and V tiles are double-buffered in LDS in natural rows (buffer loads
// straight into LDS), XOR-swizzled so that 16-row operand reads and 4-row
// transpose reads are free of bank conflicts.  Each tile list holds its FULL
// tiles before its PARTIAL ones, and the kernel runs an unmasked loop and then
// a masked one.
// The running max m only moves when a tile's max exceeds it by more than 8
// (log2 units): exp2(s - m) then stays <= 256, which changes no result beyond
// rounding, and the O rescale is skipped by the whole wave in almost every
// tile.
#include <type_traits>

#include "kernel_args.h"
#include "kernel_common.h"

namespace ra {

template <int DH>
struct FwdCfg {
    static constexpr int NT = 512;
    static constexpr int BQ = DQ_BQ, BK = FWD_BK;      // 8 waves x 32 query rows, 64 keys
    static constexpr int NKS = DH / 16;        // MFMA steps over the head dim
    static constexpr int NDT = DH / 32;        // 32-row tiles of O^T
    static constexpr int ROWB = DH * 2;        // bytes of one K row
    static constexpr int KCH = DH / 8;         // 16-byte chunks per K row
    static constexpr int K_BYTES = BK * ROWB;
    static constexpr int OUT_STRIDE = ROWB + 16;          // epilogue staging row
    // a stage array also holds the output rows of two waves in the epilogue
    static constexpr int STAGE_BYTES = 64 * OUT_STRIDE > K_BYTES ? 64 * OUT_STRIDE : K_BYTES;
};

typedef short fi16x4_t __attribute__((ext_vector_type(4)));
// LDS transpose read: within each 16-lane group, result lane i, element k is
// the 16-bit value at (address of lane 4k + i/4) + 2*(i%4).
__device__ __forceinline__ u32x2_t fwd_tr16(const unsigned char* p) {
    const fi16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) fi16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, r);
}

// RING = false: one launch per ring step, over the step's tile lists, with the
// step epilogue of p.mode.  RING = true: one launch over every active step of
// the rank's share (FWD_SOLO): each query tile's list holds the key tiles of
// all steps (those that need no mask first), each entry naming its step, so
// the running max, sum and output stay in registers from one ring step to the
// next; carrying the unnormalised partial with its running max and sum across
// the steps is the log-sum-exp merge of the normalised partials, done in
// registers (the "online softmax across ring steps" of the ai360xpert page).
template <int DH, bool RING>
__global__ __launch_bounds__(512, 1) void fwd_step_bf16_kernel(FwdArgs p) {
    using C = FwdCfg<DH>;
    // K and V stages as separate objects, each access naming its stage
    // statically: the compiler can then see that the transpose reads of V
    // never overlap the loads in flight into the other stages (it would
    // otherwise wait for those loads before every transpose read).
    __shared__ __attribute__((aligned(16))) unsigned char KA[C::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char KB[C::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char VA[C::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char VB[C::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    // The work items of this work-group: one, from the block index; or, with a
    // persistent schedule (one work-group per CU), the planner's list for this
    // block, walked in order.
    const bool persistent = RING && p.pers_off != nullptr;
    const int it0 = persistent ? as_const(p.pers_off)[blockIdx.x] : 0;
    const int it1 = persistent ? as_const(p.pers_off)[blockIdx.x + 1] : 1;
    for (int it = it0; it < it1; ++it) {
    // item: work index, entries [first, end) of the work's list (relative),
    // and the part slot (-1: the whole list, whose result is final)
    int work, e_first = 0, e_end = 0x7fffffff, pslot = -1;
    if (persistent) {
        const cint_ptr item = as_const(p.pers_items) + 4 * it;
        work = item[0];
        e_first = item[1];
        e_end = item[2];
        pslot = item[3];
    } else {
        work = xcd_work_index(blockIdx.x, gridDim.x);
    }
    if (work >= p.total_work) break;
    if (it > it0) __syncthreads();  // the previous item's epilogue is done with the stages
    const int t = work % p.nqt, bh = work / p.nqt;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int qt = as_const(p.t_order)[t];
    const int hk = (h * p.Hkv) / p.Hq;
    const cint_ptr ents = as_const(p.t_ent);
    const int l0 = as_const(p.t_off)[qt], l1 = as_const(p.t_off)[qt + 1];
    const int e0 = l0 + e_first, e1 = l0 + min(l1 - l0, e_end);
    // FULL tiles in [e0, m_full), PARTIAL after
    const int m_full = min(max(as_const(p.t_mid)[qt], e0), e1);

    const int iq = qt * C::BQ + wave * 32 + l32;  // this lane's query row
    const int iqc = min(iq, p.S - 1);
    const uint16_t* qrow = (const uint16_t*)p.q + ((int64_t)(b * p.S + iqc) * p.Hq + h) * DH;
    u32x4_t qreg[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) qreg[ks] = *(const u32x4_t*)(qrow + 16 * ks + 8 * g);
    // the visible key interval [ra, rb) of this lane's row (per ring step when RING)
    int ra = 0, rb = 0;
    if (!RING) {
        ra = p.rng[2 * iq];
        rb = p.rng[2 * iq + 1];
    }

    BufTileLoader<DH, C::BK, C::NT> lk, lv;   // K and V tiles of 64 keys
    const int64_t kv_batch = (int64_t)b * p.Skv * p.Hkv * DH;
    lk.init((const uint16_t*)p.k + kv_batch, p.Skv, p.Hkv, hk, wave, lane);
    lv.init((const uint16_t*)p.v + kv_batch, p.Skv, p.Hkv, hk, wave, lane);
    // RING: the K/V buffers of the block of a plan step
    auto k_rsrc = [&](int jb) {
        return lk.rsrc_of((const uint16_t*)p.k + kv_batch + jb * p.block_elems, p.Skv, p.Hkv);
    };
    auto v_rsrc = [&](int jb) {
        return lv.rsrc_of((const uint16_t*)p.v + kv_batch + jb * p.block_elems, p.Skv, p.Hkv);
    };

    // per-lane LDS offsets: natural K reads of row l32 (+32 mt), chunk 2ks+g;
    // transpose reads of V rows {4g, 8+4g} + j/4 (+16 kk), head-dim block dt.
    const int j = lane & 15, gsel = (lane >> 4) & 1;
    int nat[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) nat[ks] = swz_off<C::KCH>(l32, 2 * ks + g);
    int trv[2][C::NDT];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int col = 32 * dt + 16 * gsel + 4 * (j & 3);
            trv[r][dt] = swz_off<C::KCH>(8 * r + 4 * g + (j >> 2), col >> 3) + (col & 7) * 2;
        }

    f32x16_t oacc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = (f32x16_t){};
    float m_run = -INFINITY, l_run = 0.f;
    const float c2 = p.scale_log2;
    constexpr float kSlack = 8.f;  // log2 units the running max may lag behind

    // Software pipeline over the step's key tiles (n of them): K runs one tile
    // ahead of V, so that S(i+1) = K(i+1) Q^T is issued on the MFMA pipe
    // while the vector ALUs work on the softmax of tile i.  Tile i sits in
    // K/V stage A when i is even, B when odd; in iteration i the wave reads K
    // of tile i+1 and V of tile i, and the threads load K of tile i+2 and V of
    // tile i+1 into the stages freed in iteration i-1.
    const int n = e1 - e0;

    // S^T = K Q^T; the K operands of step ks+1 are read while step ks runs
    auto s_tile = [&](f32x16_t (&sacc)[2], const unsigned char* Ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sacc[mt] = (f32x16_t){};
        u32x4_t ka[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) ka[0][mt] = *(const u32x4_t*)(Ks + nat[0] + mt * 32 * C::ROWB);
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            if (ks + 1 < C::NKS)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    ka[(ks + 1) & 1][mt] = *(const u32x4_t*)(Ks + nat[ks + 1] + mt * 32 * C::ROWB);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma_32x32x16(ka[ks & 1][mt], qreg[ks], sacc[mt]);
        }
    };

    // The softmax of a tile is split around the tile boundary: the row max of
    // tile i+1 (and the rescale of O it may call for) is taken at the end of
    // iteration i, right after its scores are computed, so that iteration
    // i+1 can start its exponentials at once, beside the S MFMAs of tile i+2,
    // and the MFMAs of P V run beside the next max.  The order of operations
    // on every row is unchanged.

    // mask of a tile (keys outside [a, b) are invisible) and its row max,
    // in log2 units
    auto mask_max = [&](f32x16_t (&sacc)[2], int kt, int a, int b, auto partial_tag) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        if (PARTIAL) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * C::BK + 32 * mt + (r >> 2) * 8 + g * 4 + (r & 3);
                    sacc[mt][r] = ((key >= a) & (key < b)) ? sacc[mt][r] : -INFINITY;
                }
        }
        // linear chain: the compiler fuses pairs into v_max3_f32 (built with
        // -fno-honor-nans, so no per-operand quieting is emitted)
        float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, sacc[0][r]), sacc[1][r]);
        return pair_max(mx) * c2;
    };
    // move the reference max only when the tile exceeds it by > kSlack;
    // lanes that do not move keep alpha = 1 (m_run may be -inf there); the O
    // rescale is skipped by the whole wave in almost every tile
    auto rebase = [&](float mx, bool valid) {
        const bool bump = valid & (mx > m_run + kSlack);
        const float alpha = bump ? fast_exp2(m_run - mx) : 1.f;  // 0 if m_run = -inf
        m_run = bump ? mx : m_run;
        l_run *= alpha;
        if (__builtin_amdgcn_ballot_w64(bump)) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] *= alpha;
        }
    };
    // P rounded to bf16 for P V; the row sum stays in fp32 (a sum of the
    // rounded values would cost up to 2^-9 in lse on rows with few keys)
    auto p_tile = [&](const f32x16_t (&sacc)[2], u32x4_t (&pb)[4]) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float rsum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(fmaf(sacc[mt][r], c2, -m_use));
                const float p1 = fast_exp2(fmaf(sacc[mt][r + 1], c2, -m_use));
                rsum += p0 + p1;
                pb[2 * mt + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
            }
        l_run += rsum;
    };
    // O^T += V^T P^T; the K dimension (keys) of step kk takes rows
    // 16kk + 4g + 0..3 and 16kk + 8 + 4g + 0..3, as P is held.  The V^T
    // operands of step kk+1 are read while the MFMAs of step kk run.
    auto pv_tile = [&](const u32x4_t (&pb)[4], const unsigned char* Vs) {
        u32x4_t va[2][C::NDT];
        auto read_v = [&](u32x4_t (&dst)[C::NDT], int kk) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                const u32x2_t a1 = fwd_tr16(Vs + trv[0][dt] + kk * 16 * C::ROWB);
                const u32x2_t a2 = fwd_tr16(Vs + trv[1][dt] + kk * 16 * C::ROWB);
                dst[dt] = (u32x4_t){a1[0], a1[1], a2[0], a2[1]};
            }
        };
        read_v(va[0], 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk + 1 < 4) read_v(va[(kk + 1) & 1], kk + 1);
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
                oacc[dt] = mfma_32x32x16(va[kk & 1][dt], pb[kk], oacc[dt]);
        }
    };

    // Entries of tiles i, i+1 and i+2 (0 past the list), the last one fetched
    // an iteration ahead; key tile, plan step and KV block of each.
    constexpr int KT_MASK = RING ? (1 << RING_STEP_SHIFT) - 1 : 0x7fffffff;
    // (called with n > 0 only; the load is clamped to the list so that the
    // loop needs no branch)
    auto raw_at = [&](int i) {
        const int v = ents[e0 + min(i, n - 1)];
        return i < n ? v : 0;
    };
    auto step_of = [&](int e) { return RING ? (e >> RING_STEP_SHIFT) & (RING_MAX_STEPS - 1) : 0; };
    auto blk_of = [&](int e) { return RING ? as_const(p.blk)[step_of(e)] : 0; };
    int en0 = 0, en1 = 0, en2 = 0, jb1 = 0, jb2 = 0;
    if (n > 0) {
        en0 = raw_at(0);
        en1 = raw_at(1);
        en2 = raw_at(2);
        jb1 = blk_of(en1);
        jb2 = blk_of(en2);
    }
    // RING: the interval of the lane's row in a tile's step (every key for a
    // tile that needs no mask), loaded two tiles ahead: rng1 is tile i+1's
    // (masked at the end of iteration i), the load issued in iteration i is
    // tile i+2's.
    int2 rng1 = {ra, rb};
    auto fetch_rng = [&](int e) {
        int2 r = {ra, rb};
        if (RING) {
            const int2 v = *(const int2*)(p.rng + (int64_t)step_of(e) * p.rng_stride + 2 * iq);
            r.x = e < 0 ? v.x : 0;
            r.y = e < 0 ? v.y : 0x7fffffff;
        }
        return r;
    };

    // iteration i: refill; S(i+1) on the matrix cores beside P(i); P V of
    // tile i beside the max of tile i+1, then its rebase.  S(i+1) of the last
    // tile reads a stale stage and is discarded.
    auto body = [&](int i, f32x16_t (&cur)[2], f32x16_t (&nxt)[2], const unsigned char* Kn,
                    unsigned char* Kl, const unsigned char* Vc, unsigned char* Vl,
                    auto partial_tag) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into LDS have landed
        __syncthreads();  // K(i+1) and V(i) are in LDS; the stages refilled below are free
        // unconditional: past the list the entries are 0, a valid tile that
        // nobody reads (no branch splits the region of the MFMAs below)
        int2 rng2 = rng1;
        if (RING) {
            lk.load_from(Kl, k_rsrc(jb2), en2 & KT_MASK, wave);
            lv.load_from(Vl, v_rsrc(jb1), en1 & KT_MASK, wave);
            rng2 = fetch_rng(en2);
        } else {
            lk.load(Kl, en2 & KT_MASK, wave);
            lv.load(Vl, en1 & KT_MASK, wave);
        }
        const int kt1 = en1 & KT_MASK;
        en0 = en1;
        en1 = en2;
        jb1 = jb2;
        en2 = raw_at(i + 3);
        if (RING) jb2 = blk_of(en2);
        s_tile(nxt, Kn);
        u32x4_t pb[4];
        p_tile(cur, pb);
        pv_tile(pb, Vc);
        const float mx = mask_max(nxt, kt1, rng1.x, rng1.y, partial_tag);
        rebase(mx, i + 1 < n);
        rng1 = rng2;
    };

    if (n > 0) {
        int2 rng0 = {ra, rb};
        if (RING) {
            const int jb0 = blk_of(en0);
            lk.load_from(KA, k_rsrc(jb0), en0 & KT_MASK, wave);
            lv.load_from(VA, v_rsrc(jb0), en0 & KT_MASK, wave);
            if (n > 1) lk.load_from(KB, k_rsrc(jb1), en1 & KT_MASK, wave);
            rng0 = fetch_rng(en0);
            rng1 = fetch_rng(en1);
        } else {
            lk.load(KA, en0 & KT_MASK, wave);
            lv.load(VA, en0 & KT_MASK, wave);
            if (n > 1) lk.load(KB, en1 & KT_MASK, wave);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16_t sa[2], sb[2];
        s_tile(sa, KA);
        rebase(mask_max(sa, en0 & KT_MASK, rng0.x, rng0.y, std::true_type{}), true);
        // iterations whose next tile needs no mask, in pairs; the rest mask
        // the next tile (a tile that needs none keeps every key)
        const int nF = m_full - e0;
        const int nU = nF > 1 ? (nF - 1) & ~1 : 0;
        int i = 0;
        for (; i < nU; i += 2) {
            body(i, sa, sb, KB, KA, VA, VB, std::false_type{});
            body(i + 1, sb, sa, KA, KB, VB, VA, std::false_type{});
        }
        for (; i < n; i += 2) {
            body(i, sa, sb, KB, KA, VA, VB, std::true_type{});
            if (i + 1 < n) body(i + 1, sb, sa, KA, KB, VB, VA, std::true_type{});
        }
        // the last iterations' loads (of tiles nobody reads) land before the
        // stages are reused below
        __builtin_amdgcn_s_waitcnt(0);
    }

    // ---- epilogue: normalise the step's partial and apply the step mode ----
    const float l_tot = pair_sum(l_run);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float Lj = empty ? -INFINITY : (m_run + log2f(l_tot)) * kLn2;
    const bool valid = iq < p.S;
    const int64_t lse_idx = ((int64_t)b * p.Hq + h) * p.S + iq;

    // O_j (normalised) in registers; element (dt, r) is head-dim index
    // 32*dt + 8*(r/4) + 4*g + r%4 of query row iq.
    float w_old = 0.f, w_new = inv, L_out = Lj;
    f32x4_t* orun = (f32x4_t*)p.o_run +
                    (((int64_t)b * p.Hq + h) * (p.S_pad / 32) + (qt * (C::BQ / 32) + wave)) * (8 * DH) + lane;
    if (pslot >= 0) {
        // a part of a split list: its normalised partial and lse, merged with
        // the other parts' by the part-merge kernel
        const int row = wave * 32 + l32;
        float* orow = p.part_o + ((int64_t)pslot * C::BQ + row) * DH;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4_t o = {oacc[dt][4 * rg] * inv, oacc[dt][4 * rg + 1] * inv,
                             oacc[dt][4 * rg + 2] * inv, oacc[dt][4 * rg + 3] * inv};
                *(f32x4_t*)(orow + 32 * dt + 8 * rg + 4 * g) = o;
            }
        if (g == 0) p.part_l[(int64_t)pslot * C::BQ + row] = Lj;
        continue;
    }
    const int mode = p.mode;
    if (mode == FWD_MERGE || mode == FWD_LAST) {
        const float Lr = valid ? p.lse[lse_idx] : -INFINITY;
        const float M = fmaxf(Lr, Lj);
        if (M == -INFINITY) {
            w_old = 0.f; w_new = 0.f; L_out = -INFINITY;
        } else {
            const float er = expf(Lr - M), ej = expf(Lj - M);
            const float den = er + ej;
            L_out = M + logf(den);
            w_old = er / den;
            w_new = ej * inv / den;
        }
    }

    if (mode == FWD_FIRST || mode == FWD_MERGE) {
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                f32x4_t* ptr = orun + (dt * 4 + rg) * 64;
                f32x4_t o = {oacc[dt][4 * rg] * w_new, oacc[dt][4 * rg + 1] * w_new,
                             oacc[dt][4 * rg + 2] * w_new, oacc[dt][4 * rg + 3] * w_new};
                if (mode == FWD_MERGE) o += w_old * (*ptr);
                *ptr = o;
            }
        if (valid && g == 0) p.lse[lse_idx] = L_out;
        continue;
    }
    if (mode == FWD_PARTIAL) {
        if (valid) {
            float* orow = p.o_part + ((int64_t)(b * p.S + iq) * p.Hq + h) * DH;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    f32x4_t o = {oacc[dt][4 * rg] * inv, oacc[dt][4 * rg + 1] * inv,
                                 oacc[dt][4 * rg + 2] * inv, oacc[dt][4 * rg + 3] * inv};
                    *(f32x4_t*)(orow + 32 * dt + 8 * rg + 4 * g) = o;
                }
            if (g == 0) p.lse_part[lse_idx] = Lj;
        }
        continue;
    }

    // FWD_LAST / FWD_SOLO: final bf16 output through LDS for coalesced rows.
    __syncthreads();  // every wave is done with the K/V stages
    unsigned char* st = ((wave & 3) == 0 ? KA : (wave & 3) == 1 ? KB : (wave & 3) == 2 ? VA : VB) +
                        (wave >> 2) * 32 * C::OUT_STRIDE;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4_t o = {oacc[dt][4 * rg] * w_new, oacc[dt][4 * rg + 1] * w_new,
                         oacc[dt][4 * rg + 2] * w_new, oacc[dt][4 * rg + 3] * w_new};
            if (mode == FWD_LAST) o += w_old * orun[(dt * 4 + rg) * 64];
            u32x2_t w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *(u32x2_t*)(st + l32 * C::OUT_STRIDE + (32 * dt + 8 * rg + 4 * g) * 2) = w;
        }
    if (valid && g == 0) p.lse[lse_idx] = L_out;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    constexpr int CPR = DH / 8;            // 16-byte chunks per output row
    constexpr int RPI = 64 / CPR;          // rows per wave instruction
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + lane / CPR, ch = lane % CPR;
        const int iqr = qt * C::BQ + wave * 32 + row;
        const u32x4_t val = *(const u32x4_t*)(st + row * C::OUT_STRIDE + ch * 16);
        if (iqr < p.S)
            *(u32x4_t*)((uint16_t*)p.out + ((int64_t)(b * p.S + iqr) * p.Hq + h) * DH + ch * 8) = val;
    }
    }  // work items
}

template __global__ void fwd_step_bf16_kernel<128, false>(FwdArgs);
template __global__ void fwd_step_bf16_kernel<128, true>(FwdArgs);
template __global__ void fwd_step_bf16_kernel<64, false>(FwdArgs);
template __global__ void fwd_step_bf16_kernel<64, true>(FwdArgs);

// Merge of the parts of split forward lists: one work-group per 32 query
// rows of a split list; each row's parts are folded with the log-sum-exp merge of
// "Numerically-Stable Output Fusion" (instagit/nanotron page), generalised to
// any number of parts: L = M + ln sum_k e^{L_k - M}, O = sum_k e^{L_k - L} O_k,
// M = max_k L_k; a row that sees no key in any part gets O = 0, L = -inf.
// The result is rounded to bf16 (RNE) and written with its lse, as the
// one-launch forward writes an unsplit list.
constexpr int PART_MERGE_ROWS = 32;   // rows of a split list per work-group
__global__ __launch_bounds__(256) void fwd_part_merge_kernel(PartMergeArgs p) {
    const int i = blockIdx.x / (DQ_BQ / PART_MERGE_ROWS);
    const int r0 = (blockIdx.x % (DQ_BQ / PART_MERGE_ROWS)) * PART_MERGE_ROWS;
    const int work = p.items[3 * i], slot0 = p.items[3 * i + 1], np = p.items[3 * i + 2];
    const int t = work % p.nqt, bh = work / p.nqt;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int qt = as_const(p.t_order)[t];
    const int cpr = p.d / 4;      // 4-float chunks per row
    const int rpp = 256 / cpr;    // rows per pass of the work-group
    const int c = (threadIdx.x % cpr) * 4;
    for (int r = r0 + threadIdx.x / cpr; r < r0 + PART_MERGE_ROWS; r += rpp) {
        const int iq = qt * DQ_BQ + r;
        if (iq >= p.S) break;
        float M = -INFINITY;
        for (int k = 0; k < np; ++k) M = fmaxf(M, p.part_l[(int64_t)(slot0 + k) * DQ_BQ + r]);
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
        float L = -INFINITY;
        if (M != -INFINITY) {
            float sum = 0.f;
            for (int k = 0; k < np; ++k) sum += expf(p.part_l[(int64_t)(slot0 + k) * DQ_BQ + r] - M);
            L = M + logf(sum);
            for (int k = 0; k < np; ++k) {
                const float wk = expf(p.part_l[(int64_t)(slot0 + k) * DQ_BQ + r] - L);
                o += wk * *(const f32x4_t*)(p.part_o + ((int64_t)(slot0 + k) * DQ_BQ + r) * p.d + c);
            }
        }
        const u32x2_t w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *(u32x2_t*)((uint16_t*)p.out + ((int64_t)(b * p.S + iq) * p.Hq + h) * p.d + c) = w;
        if (c == 0) p.lse[((int64_t)b * p.Hq + h) * p.S + iq] = L;
    }
}

hipError_t launch_fwd_part_merge(const PartMergeArgs& a, hipStream_t s) {
    if (a.n_items == 0) return hipSuccess;
    if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fwd_part_merge_kernel, dim3(a.n_items * (DQ_BQ / PART_MERGE_ROWS)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, hipStream_t s) {
    const int grid = a.ring && a.pers_off ? a.pers_blocks : (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128 && a.ring)
        hipLaunchKernelGGL((fwd_step_bf16_kernel<128, true>), dim3(grid), dim3(512), 0, s, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((fwd_step_bf16_kernel<128, false>), dim3(grid), dim3(512), 0, s, a);
    else if (head_dim == 64 && a.ring)
        hipLaunchKernelGGL((fwd_step_bf16_kernel<64, true>), dim3(grid), dim3(512), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL((fwd_step_bf16_kernel<64, false>), dim3(grid), dim3(512), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
