// K4: one ring step of the attention backward, bf16 operands, fp32
// accumulation (instagit/nanotron page, "Backward Pass and Gradient
// Accumulation": per step, the flash backward of (dout, q, k_j, v_j, out, lse)
// adds into dq, dk_j and dv_j).
//
// One work-group = one (batch, kv head, 128-key tile of block j); wave w owns
// keys 32w..32w+31.  It walks every query tile (64 rows) of every query head
// of the GQA group that sees its keys, and per tile computes
//   S = Q K^T and dP = dO V^T        (C layout: lane = key, 16 query rows)
//   P = exp(scale*S - lse), dS = P (dP - Delta)
//   dV^T += dO^T P,  dK^T += Q^T dS  (fp32 accumulators in registers)
//   dQ += scale * dS K               (fp32 atomics into a head-major accumulator)
// Q, dO and K live in LDS in their natural row layout only.  The transposed
// operands (dO^T, Q^T, and K as the B operand of dQ) come from the gfx950 LDS
// transpose read ds_read_b64_tr_b16: within each 16-lane group, result lane i,
// element k is the 16-bit value at (address of lane 4k + i/4) + 2*(i%4), so a
// group turns a 4-row x 16-column K-major block into MFMA operand layout.  P
// and dS feed the MFMAs straight from the accumulator registers, whose query
// order inside each 16-row group is {0-3, 8-11 | 4-7, 12-15} (lanes 0-31 |
// 32-63); the transpose reads pick their rows in that same order.  dS goes to
// LDS as dS^T [key][query] with 8-byte writes for the dQ product.  dK/dV are
// added to the caller's buffers once at the end: every key tile of a block has
// one owner per launch.
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
    static constexpr int K_BYTES = BK * ROWB;
    static constexpr int DST_ROWB = BQ * 2;         // dS^T row: 64 queries
    static constexpr int DST_BYTES = BK * DST_ROWB;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = OFF_Q + Q_BYTES;
    static constexpr int OFF_K = OFF_DO + Q_BYTES;
    static constexpr int OFF_V = OFF_K + K_BYTES;
    static constexpr int OFF_DST = OFF_V + K_BYTES;
    static constexpr int OFF_ROW = OFF_DST + DST_BYTES;  // lse2, delta, a, b per query row
    static constexpr int LDS = OFF_ROW + 4 * BQ * 4;
    static constexpr int LDT = BQ * KCH / 4;        // threads taking part in a Q/dO load
    static_assert(LDT == NT || LDT == NT / 2, "tile shape");
};

// 16-byte slot of logical chunk c in row r.  Rows of 16 chunks (256 B) and of
// 8 chunks (128 B, two rows per bank cycle) have their own XOR patterns; both
// keep 16 consecutive rows at one chunk, and 4 consecutive rows x 2 chunks,
// free of bank conflicts.
template <int NCH>
__device__ __forceinline__ int slot(int r, int c) {
    if (NCH == 16) return c ^ (((r & 7) << 1) | ((r >> 3) & 1));
    return c ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}

template <int NCH>
__device__ __forceinline__ int row_off(int r, int c) {
    return r * (NCH * 16) + (slot<NCH>(r, c) << 4);
}

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

// Global -> registers: 4 consecutive query rows x one 16-byte chunk of Q and
// dO, plus the per-row values of row tid.
template <int DH>
struct BwdTileRegs {
    u32x4_t q[4], o[4];
    float l2, dl;   // lse * log2(e) (+inf: row sees no key) and Delta
    int a, b;       // visible key interval
};

template <int DH>
__device__ __forceinline__ void bwd_load_tile(BwdTileRegs<DH>& R, const BwdArgs& p, int b, int h,
                                              int qt, int tid) {
    using C = BwdCfg<DH>;
    const int q_stride = p.Hq * DH;
    if (tid < C::LDT) {
        const uint16_t* qh = p.q + ((int64_t)b * p.S) * q_stride + h * DH;
        const uint16_t* oh = p.dout + ((int64_t)b * p.S) * q_stride + h * DH;
        const int m = tid / C::KCH, ch = tid % C::KCH;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int row = min(qt * C::BQ + 4 * m + rr, p.S - 1);
            R.q[rr] = *(const u32x4_t*)(qh + (int64_t)row * q_stride + ch * 8);
            R.o[rr] = *(const u32x4_t*)(oh + (int64_t)row * q_stride + ch * 8);
        }
    }
    if (tid < C::BQ) {
        const int iq = qt * C::BQ + tid;
        const int iqc = min(iq, p.S - 1);
        const float L = p.lse[((int64_t)b * p.Hq + h) * p.S + iqc];
        R.dl = p.delta[((int64_t)b * p.Hq + h) * p.S_pad + iqc];
        R.a = p.rng[2 * iqc];
        R.b = p.rng[2 * iqc + 1];
        R.l2 = L == -INFINITY ? INFINITY : L * kLog2e;
        if (iq >= p.S) {  // rows past the shard contribute nothing
            R.l2 = INFINITY;
            R.dl = 0.f;
            R.a = 0;
            R.b = 0;
        }
    }
}

template <int DH>
__global__ __launch_bounds__(256, 1) void bwd_step_bf16_kernel(BwdArgs p) {
    using C = BwdCfg<DH>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
    unsigned char* sQ = smem + C::OFF_Q;
    unsigned char* sDO = smem + C::OFF_DO;
    unsigned char* sK = smem + C::OFF_K;
    unsigned char* sV = smem + C::OFF_V;
    unsigned char* sDST = smem + C::OFF_DST;
    float* sL = (float*)(smem + C::OFF_ROW);
    float* sD = sL + C::BQ;
    int32_t* sA = (int32_t*)(sD + C::BQ);
    int32_t* sB = sA + C::BQ;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nkt, bh = work / p.nkt;
    const int hk = bh % p.Hkv, b = bh / p.Hkv;
    const cint_ptr ents = as_const(p.t_ent);
    const int kt = as_const(p.t_order)[t];
    const int e0 = as_const(p.t_off)[kt], e1 = as_const(p.t_off)[kt + 1];
    const int group = p.Hq / p.Hkv;

    const int kv_stride = p.Hkv * DH;
    const uint16_t* kb = p.k + (int64_t)b * p.Skv * kv_stride + hk * DH;
    const uint16_t* vb = p.v + (int64_t)b * p.Skv * kv_stride + hk * DH;
    const int key = kt * C::BK + wave * 32 + l32;   // this lane's key (C-layout column)
    const int keyc = min(key, p.Skv - 1);

    // K and V tiles of the work-group in LDS (natural rows).
    for (int idx = tid; idx < C::BK * C::KCH; idx += C::NT) {
        const int r = idx / C::KCH, ch = idx % C::KCH;
        const int64_t kr = min(kt * C::BK + r, p.Skv - 1);
        *(u32x4_t*)(sK + row_off<C::KCH>(r, ch)) = *(const u32x4_t*)(kb + kr * kv_stride + ch * 8);
        *(u32x4_t*)(sV + row_off<C::KCH>(r, ch)) = *(const u32x4_t*)(vb + kr * kv_stride + ch * 8);
    }

    f32x16_t dk_acc[C::NDT], dv_acc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        dk_acc[dt] = (f32x16_t){};
        dv_acc[dt] = (f32x16_t){};
    }
    const float c2 = p.scale_log2;
    const int n_ent = e1 - e0;
    const int n_iter = n_ent * group;

    // Per-lane LDS offsets.  Every swizzle below depends only on the low four
    // bits of the row, so moving by 16 or 32 rows is a constant offset.
    //   nat[ks]    : natural read of row l32, chunk 2ks+g (S and dP A operands)
    //   trq[r][dt] : transpose read of rows {4g, 8+4g} + j/4, head-dim block dt
    //   trd[r]     : transpose read of dS^T rows {8g, 8g+4} + j/4, query block mt_q
    //   trk[r][tw] : transpose read of K rows {8g, 8g+4} + j/4, head-dim block nt
    constexpr int TILES = 2 * C::NDT;
    constexpr int PER_WAVE = TILES / 4;
    const int mt_q = (wave * PER_WAVE) / C::NDT;
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
    int trd[2], trk[2][PER_WAVE];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int colq = 32 * mt_q + 16 * gsel + 4 * (j & 3);
        trd[r] = row_off<8>(8 * g + 4 * r + (j >> 2), colq >> 3) + (colq & 7) * 2;
#pragma unroll
        for (int tw = 0; tw < PER_WAVE; ++tw) {
            const int nt = (wave * PER_WAVE + tw) % C::NDT;
            const int cold = 32 * nt + 16 * gsel + 4 * (j & 3);
            trk[r][tw] = row_off<C::KCH>(8 * g + 4 * r + (j >> 2), cold >> 3) + (cold & 7) * 2;
        }
    }
    const int dst_w = row_off<8>(wave * 32 + l32, 0);  // dS^T row of this lane's key
    const int dst_x = slot<8>(wave * 32 + l32, 0);     // its chunk swizzle

    // Registers -> LDS: the staged query tile (natural rows) and its row values.
    auto store_tile = [&](const BwdTileRegs<DH>& T) {
        if (tid < C::LDT) {
            const int m = tid / C::KCH, ch = tid % C::KCH;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                *(u32x4_t*)(sQ + row_off<C::KCH>(4 * m + rr, ch)) = T.q[rr];
                *(u32x4_t*)(sDO + row_off<C::KCH>(4 * m + rr, ch)) = T.o[rr];
            }
        }
        if (tid < C::BQ) {
            sL[tid] = T.l2;
            sD[tid] = T.dl;
            sA[tid] = T.a;
            sB[tid] = T.b;
        }
    };

    // Loop schedule (two barriers per query tile):
    //   barrier A: tile `it` is in sQ/sDO; every wave is done with the previous dQ
    //   issue global loads of tile it+1 into registers
    //   S, dP, P, dS (-> dS^T in LDS), dV, dK
    //   barrier B: every wave is done with sQ/sDO; dS^T is complete
    //   store tile it+1 into sQ/sDO (its loads were issued before this
    //   iteration's dQ atomics, so waiting for them does not wait for those)
    //   dQ product and atomics
    BwdTileRegs<DH> R;
    if (n_iter > 0) {
        bwd_load_tile<DH>(R, p, b, hk * group, ents[e0] & 0x7fffffff, tid);
        store_tile(R);
    }
    for (int it = 0; it < n_iter; ++it) {
        const int h = hk * group + it / n_ent;
        const int ent = ents[e0 + it % n_ent];
        const int qt = ent & 0x7fffffff;
        const bool partial = ent < 0;
        // Keep the dK/dV accumulators in AGPRs across iterations (the MFMAs
        // accumulate there directly; no VALU touches them inside the loop).
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+a"(dk_acc[dt]), "+a"(dv_acc[dt]));

        __syncthreads();  // barrier A
        const bool has_next = it + 1 < n_iter;
        if (has_next)
            bwd_load_tile<DH>(R, p, b, hk * group + (it + 1) / n_ent,
                              ents[e0 + (it + 1) % n_ent] & 0x7fffffff, tid);

        // S = Q K^T and dP = dO V^T: two 32-row halves of the 64-row tile; the
        // B operands are this lane's K and V rows (key 32*wave + l32).
        f32x16_t sacc[2], pacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = (f32x16_t){};
            pacc[mt] = (f32x16_t){};
        }
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            const u32x4_t kb4 = *(const u32x4_t*)(sK + nat[ks] + wave * 32 * C::ROWB);
            const u32x4_t vb4 = *(const u32x4_t*)(sV + nat[ks] + wave * 32 * C::ROWB);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const u32x4_t qa = *(const u32x4_t*)(sQ + nat[ks] + mt * 32 * C::ROWB);
                const u32x4_t oa = *(const u32x4_t*)(sDO + nat[ks] + mt * 32 * C::ROWB);
                sacc[mt] = mfma_32x32x16(qa, kb4, sacc[mt]);
                pacc[mt] = mfma_32x32x16(oa, vb4, pacc[mt]);
            }
        }
        // P (in sacc) and dS (in pacc); element (mt, r) is query row
        // 32*mt + 8*(r/4) + 4*g + r%4.
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const f32x4_t L = *(const f32x4_t*)(sL + 32 * mt + 8 * rg + 4 * g);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[mt][4 * rg + i] = fast_exp2(fmaf(sacc[mt][4 * rg + i], c2, -L[i]));
            }
        if (partial) {  // keys outside a row's interval [a, b) are invisible
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int r0 = 32 * mt + 8 * rg + 4 * g;
                    const int4 A4 = *(const int4*)(sA + r0);
                    const int4 B4 = *(const int4*)(sB + r0);
                    const int av[4] = {A4.x, A4.y, A4.z, A4.w}, bv[4] = {B4.x, B4.y, B4.z, B4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool vis = (key >= av[i]) & (key < bv[i]);
                        sacc[mt][4 * rg + i] = vis ? sacc[mt][4 * rg + i] : 0.f;
                    }
                }
        }
        u32x4_t pb[4], db[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int r0 = 32 * mt + 8 * rg + 4 * g;
                const f32x4_t Dl = *(const f32x4_t*)(sD + r0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pacc[mt][4 * rg + i] = sacc[mt][4 * rg + i] * (pacc[mt][4 * rg + i] - Dl[i]);
                const int kk = 2 * mt + (rg >> 1), w = (rg & 1) * 2;
                pb[kk][w] = pack_bf16x2(sacc[mt][4 * rg], sacc[mt][4 * rg + 1]);
                pb[kk][w + 1] = pack_bf16x2(sacc[mt][4 * rg + 2], sacc[mt][4 * rg + 3]);
                db[kk][w] = pack_bf16x2(pacc[mt][4 * rg], pacc[mt][4 * rg + 1]);
                db[kk][w + 1] = pack_bf16x2(pacc[mt][4 * rg + 2], pacc[mt][4 * rg + 3]);
                // dS^T [key][query]: this lane's key row, queries r0..r0+3
                // (chunk r0/8 = 4mt + rg, half g)
                *(u32x2_t*)(sDST + dst_w - (dst_x << 4) + (((4 * mt + rg) ^ dst_x) << 4) + 8 * g) =
                    (u32x2_t){db[kk][w], db[kk][w + 1]};
            }
        // dV^T += dO^T P and dK^T += Q^T dS; the K dimension (queries) of step
        // kk takes rows 16kk + 4g + 0..3 and 16kk + 8 + 4g + 0..3.
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            u32x4_t oa[4], qa[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int o16 = kk * 16 * C::ROWB;
                const u32x2_t o1 = lds_tr16(sDO + trq[0][dt] + o16), o2 = lds_tr16(sDO + trq[1][dt] + o16);
                const u32x2_t q1 = lds_tr16(sQ + trq[0][dt] + o16), q2 = lds_tr16(sQ + trq[1][dt] + o16);
                oa[kk] = (u32x4_t){o1[0], o1[1], o2[0], o2[1]};
                qa[kk] = (u32x4_t){q1[0], q1[1], q2[0], q2[1]};
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                dv_acc[dt] = mfma_32x32x16(oa[kk], pb[kk], dv_acc[dt]);
                dk_acc[dt] = mfma_32x32x16(qa[kk], db[kk], dk_acc[dt]);
            }
        }
        __syncthreads();  // barrier B
        if (has_next) store_tile(R);

        // dQ[64 x DH] = dS[64 x 128] K[128 x DH]; wave tiles (mt_q, nt) of 32 x 32,
        // both operands from transpose reads (keys 16ks + 8g + 0..7 in order).
        const int rows_left = p.S - qt * C::BQ;  // >= 1
        constexpr int qs = DH;  // accumulator rows of one head are contiguous
#pragma unroll
        for (int tw = 0; tw < PER_WAVE; ++tw) {
            const int nt = (wave * PER_WAVE + tw) % C::NDT;
            f32x16_t acc = (f32x16_t){};
            u32x4_t da[C::BK / 16], ka[C::BK / 16];
#pragma unroll
            for (int ks = 0; ks < C::BK / 16; ++ks) {
                const u32x2_t d1 = lds_tr16(sDST + trd[0] + ks * 16 * C::DST_ROWB);
                const u32x2_t d2 = lds_tr16(sDST + trd[1] + ks * 16 * C::DST_ROWB);
                const u32x2_t k1 = lds_tr16(sK + trk[0][tw] + ks * 16 * C::ROWB);
                const u32x2_t k2 = lds_tr16(sK + trk[1][tw] + ks * 16 * C::ROWB);
                da[ks] = (u32x4_t){d1[0], d1[1], d2[0], d2[1]};
                ka[ks] = (u32x4_t){k1[0], k1[1], k2[0], k2[1]};
            }
#pragma unroll
            for (int ks = 0; ks < C::BK / 16; ++ks) acc = mfma_32x32x16(da[ks], ka[ks], acc);
            // acc: column d = 32*nt + l32, rows 32*mt_q + 8*(r/4) + 4*g + r%4.  Rows
            // past the shard are clamped onto the last row and add 0.
            float* dqt = p.dq + (((int64_t)b * p.Hq + h) * p.S_pad + qt * C::BQ) * DH + 32 * nt + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * mt_q + 8 * (r >> 2) + 4 * g + (r & 3);
                const bool ok = row < rows_left;
                unsafeAtomicAdd(dqt + (ok ? row : rows_left - 1) * qs, ok ? acc[r] * p.scale : 0.f);
            }
        }
    }

    // dK_j += scale * dK^T acc, dV_j += dV^T acc (this lane's key, 64 head-dim values)
    if (key < p.Skv) {
        float* dkr = p.dk + ((int64_t)b * p.Skv + key) * kv_stride + hk * DH;
        float* dvr = p.dv + ((int64_t)b * p.Skv + key) * kv_stride + hk * DH;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = 32 * dt + 8 * rg + 4 * g;
                f32x4_t x = *(f32x4_t*)(dkr + d0);
                f32x4_t y = *(f32x4_t*)(dvr + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] += p.scale * dk_acc[dt][4 * rg + i];
                    y[i] += dv_acc[dt][4 * rg + i];
                }
                *(f32x4_t*)(dkr + d0) = x;
                *(f32x4_t*)(dvr + d0) = y;
            }
    }
}

hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL(bwd_step_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL(bwd_step_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
