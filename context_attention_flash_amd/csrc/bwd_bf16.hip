// K4: one ring step of the attention backward, bf16 operands, fp32
// accumulation (instagit/nanotron page, "Backward Pass and Gradient
// Accumulation": per step, the flash backward of (dout, q, k_j, v_j, out, lse)
// adds into dq, dk_j and dv_j).  Two kernels share the step:
//
// K4a bwd_dkdv: one work-group = one (batch, kv head, 128-key tile of block
// j); wave w owns keys 32w..32w+31.  It walks every 64-row query tile of every
// query head of the GQA group that sees its keys and computes
//   S = Q K^T and dP = dO V^T        (C layout: lane = key, 16 query rows)
//   P = exp(scale*S - lse), dS = P (dP - Delta)
//   dV^T += dO^T P,  dK^T += Q^T dS  (fp32 accumulators in AGPRs)
// Q, dO, K and V live in LDS in natural rows; dO^T and Q^T come from the gfx950
// transpose read ds_read_b64_tr_b16 (within each 16-lane group, result lane i,
// element k is the 16-bit value at (address of lane 4k + i/4) + 2*(i%4)).
// P and dS feed the MFMAs straight from the accumulator registers, whose query
// order inside each 16-row group is {0-3, 8-11 | 4-7, 12-15} (lanes 0-31 |
// 32-63); the transpose reads pick their rows in that same order.  dK/dV are
// added to the caller's buffers once at the end (one owner per key tile).
//
// K4b bwd_dq: one work-group = one (batch, q head, 128-row query tile), as in
// the forward: lane = query column, Q and dO in registers, 64-key tiles of K
// and V streamed through LDS.  It recomputes S^T = K Q^T and dP^T = V dO^T and
// accumulates dQ^T += K^T dS^T (K^T from transpose reads).  Each (head, query
// tile) has one owner per launch, so dQ needs no atomics: fp32 atomics on the
// L2 run about ten times slower than plain stores, and the dQ of a key-tile
// decomposition would be bound by them.
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
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = OFF_Q + Q_BYTES;
    static constexpr int OFF_K = OFF_DO + Q_BYTES;
    static constexpr int OFF_V = OFF_K + K_BYTES;
    static constexpr int OFF_ROW = OFF_V + K_BYTES;   // lse2, delta, a, b per query row
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
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(BwdArgs p) {
    using C = BwdCfg<DH>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
    unsigned char* sQ = smem + C::OFF_Q;
    unsigned char* sDO = smem + C::OFF_DO;
    unsigned char* sK = smem + C::OFF_K;
    unsigned char* sV = smem + C::OFF_V;
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
    //   barrier A: tile `it` is in sQ/sDO
    //   issue global loads of tile it+1 into registers
    //   S, dP, P, dS, dV, dK
    //   barrier B: every wave is done with sQ/sDO
    //   store tile it+1 into sQ/sDO
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

hipError_t launch_bwd_dkdv_bf16(const BwdArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (grid == 0) return hipSuccess;
    if (head_dim == 128)
        hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
    else if (head_dim == 64)
        hipLaunchKernelGGL(bwd_dkdv_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
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
    static constexpr int BQ = FWD_BQ, BK = FWD_BK;   // 4 waves x 32 queries, 64 keys
    static constexpr int NKS = DH / 16;
    static constexpr int NDT = DH / 32;
    static constexpr int ROWB = DH * 2;
    static constexpr int KCH = DH / 8;
    static constexpr int K_BYTES = BK * ROWB;
    static constexpr int STAGE = 2 * K_BYTES;        // K and V tiles, natural rows
    static constexpr int LDS = 2 * STAGE;
    static constexpr int KLD = BK * KCH / NT;        // 16-byte chunks per thread per tensor
    static_assert(KLD >= 1, "tile shape");
};

// One 64-key tile of K or V straight from global memory into LDS
// (global_load_lds_dwordx4: the 16 bytes of lane l land at the wave-uniform
// LDS base + 16*l).  Instruction c of wave w fills LDS chunks 256c + 64w +
// lane, so the lane whose slot is physical chunk p of row r loads logical
// chunk p ^ swizzle(r).
template <int DH>
__device__ __forceinline__ void dq_load_lds(unsigned char* stage, const uint16_t* base,
                                            int kv_stride, int kt, int Skv, int wave, int lane) {
    using C = DqCfg<DH>;
#pragma unroll
    for (int c = 0; c < C::KLD; ++c) {
        const int idx = C::NT * c + 64 * wave + lane;
        const int row = idx / C::KCH, pc = idx % C::KCH;
        const int lc = slot<C::KCH>(row, pc);  // XOR swizzle: its own inverse
        const int key = min(kt * C::BK + row, Skv - 1);
        __builtin_amdgcn_global_load_lds(
            (const void*)(base + (key * kv_stride + lc * 8)),
            (__attribute__((address_space(3))) void*)(stage + (C::NT * c + 64 * wave) * 16), 16,
            0, 0);
    }
}

template <int DH>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(DqArgs p) {
    using C = DqCfg<DH>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

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

    const int iq = qt * C::BQ + wave * 32 + l32;  // this lane's query row
    const int iqc = min(iq, p.S - 1);
    const bool valid = iq < p.S;
    const int q_stride = p.Hq * DH;
    const uint16_t* qrow = p.q + ((int64_t)b * p.S + iqc) * q_stride + h * DH;
    const uint16_t* orow = p.dout + ((int64_t)b * p.S + iqc) * q_stride + h * DH;
    u32x4_t qreg[C::NKS], oreg[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        qreg[ks] = *(const u32x4_t*)(qrow + 16 * ks + 8 * g);
        oreg[ks] = *(const u32x4_t*)(orow + 16 * ks + 8 * g);
    }
    const float Lraw = p.lse[((int64_t)b * p.Hq + h) * p.S + iqc];
    const float L2 = (!valid || Lraw == -INFINITY) ? INFINITY : Lraw * kLog2e;
    const float Dl = valid ? p.delta[((int64_t)b * p.Hq + h) * p.S_pad + iqc] : 0.f;
    const int ra = p.rng[2 * iq], rb = p.rng[2 * iq + 1];

    const int kv_stride = p.Hkv * DH;
    const uint16_t* kb = p.k + (int64_t)b * p.Skv * kv_stride + hk * DH;
    const uint16_t* vb = p.v + (int64_t)b * p.Skv * kv_stride + hk * DH;

    // per-lane LDS offsets (see the dK/dV kernel)
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

    f32x16_t acc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) acc[dt] = (f32x16_t){};
    const float c2 = p.scale_log2;

    if (e0 < e1) {
        dq_load_lds<DH>(smem, kb, kv_stride, ents[e0] & 0x7fffffff, p.Skv, wave, lane);
        dq_load_lds<DH>(smem + C::K_BYTES, vb, kv_stride, ents[e0] & 0x7fffffff, p.Skv, wave, lane);
        for (int e = e0; e < e1; ++e) {
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) asm volatile("" : "+a"(acc[dt]));
            unsigned char* stage = smem + ((e - e0) & 1) * C::STAGE;
            __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
            __syncthreads();  // tile e is in LDS; the other stage is free
            if (e + 1 < e1) {
                unsigned char* nxt = smem + (((e - e0) & 1) ^ 1) * C::STAGE;
                const int ktn = ents[e + 1] & 0x7fffffff;
                dq_load_lds<DH>(nxt, kb, kv_stride, ktn, p.Skv, wave, lane);
                dq_load_lds<DH>(nxt + C::K_BYTES, vb, kv_stride, ktn, p.Skv, wave, lane);
            }
            const int ent = ents[e];
            const int kt = ent & 0x7fffffff;
            const unsigned char* Ks = stage;
            const unsigned char* Vs = stage + C::K_BYTES;

            // S^T = K Q^T and dP^T = V dO^T for the 64 keys (two 32-key halves);
            // the operands of step ks+1 are read while step ks runs
            f32x16_t sacc[2], pacc[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                sacc[mt] = (f32x16_t){};
                pacc[mt] = (f32x16_t){};
            }
            u32x4_t ka[2][2], va[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                ka[0][mt] = *(const u32x4_t*)(Ks + nat[0] + mt * 32 * C::ROWB);
                va[0][mt] = *(const u32x4_t*)(Vs + nat[0] + mt * 32 * C::ROWB);
            }
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                if (ks + 1 < C::NKS)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        ka[(ks + 1) & 1][mt] = *(const u32x4_t*)(Ks + nat[ks + 1] + mt * 32 * C::ROWB);
                        va[(ks + 1) & 1][mt] = *(const u32x4_t*)(Vs + nat[ks + 1] + mt * 32 * C::ROWB);
                    }
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    sacc[mt] = mfma_32x32x16(ka[ks & 1][mt], qreg[ks], sacc[mt]);
                    pacc[mt] = mfma_32x32x16(va[ks & 1][mt], oreg[ks], pacc[mt]);
                }
            }
            // P = exp(scale*S - lse) and dS = P (dP - Delta); element (mt, r) is key
            // 32*mt + 8*(r/4) + 4*g + r%4 of the tile.
            u32x4_t db[4];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float pv[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float pr = fast_exp2(fmaf(sacc[mt][r + u], c2, -L2));
                        if (ent < 0) {
                            const int key = kt * C::BK + 32 * mt + 8 * ((r + u) >> 2) + 4 * g + ((r + u) & 3);
                            pr = ((key >= ra) & (key < rb)) ? pr : 0.f;
                        }
                        pv[u] = pr * (pacc[mt][r + u] - Dl);
                    }
                    db[2 * mt + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(pv[0], pv[1]);
                }
            // dQ^T += K^T dS^T; the K dimension (keys) of step kk takes rows
            // 16kk + 4g + 0..3 and 16kk + 8 + 4g + 0..3, as dS is held.  The K^T
            // operands of step kk+1 are read while step kk runs.
            u32x4_t kt4[2][C::NDT];
            auto read_kt = [&](u32x4_t (&dst)[C::NDT], int kk) {
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt) {
                    const u32x2_t a1 = lds_tr16(Ks + trk[0][dt] + kk * 16 * C::ROWB);
                    const u32x2_t a2 = lds_tr16(Ks + trk[1][dt] + kk * 16 * C::ROWB);
                    dst[dt] = (u32x4_t){a1[0], a1[1], a2[0], a2[1]};
                }
            };
            read_kt(kt4[0], 0);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk + 1 < 4) read_kt(kt4[(kk + 1) & 1], kk + 1);
#pragma unroll
                for (int dt = 0; dt < C::NDT; ++dt)
                    acc[dt] = mfma_32x32x16(kt4[kk & 1][dt], db[kk], acc[dt]);
            }
        }
    }

    // dq_acc (+)= scale * acc in the accumulator layout: element (dt, r) of this
    // lane is head-dim index 32*dt + 8*(r/4) + 4*g + r%4 of query row iq.
    f32x4_t* dst = (f32x4_t*)p.dq_acc +
                   (((int64_t)b * p.Hq + h) * (p.S_pad / 32) + (qt * 4 + wave)) * (8 * DH) + lane;
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
            f32x4_t o = {acc[dt][4 * rg] * p.scale, acc[dt][4 * rg + 1] * p.scale,
                         acc[dt][4 * rg + 2] * p.scale, acc[dt][4 * rg + 3] * p.scale};
            f32x4_t* ptr = dst + (dt * 4 + rg) * 64;
            if (!p.first) o += *ptr;
            *ptr = o;
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

}  // namespace ra
