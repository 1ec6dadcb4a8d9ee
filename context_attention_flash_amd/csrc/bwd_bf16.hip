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
//   dQ += scale * dS K               (dS staged in LDS, fp32 atomics to HBM)
// P and dS feed the next MFMAs straight from the accumulator registers, so
// Q^T and dO^T are stored in LDS with the matching query order inside every
// 16-row group ({0-3, 8-11, 4-7, 12-15}).  dK/dV are added to the caller's
// fp32 buffers once at the end: every key tile of a block has one owner per
// launch, so no atomics are needed there.
#include "kernel_args.h"
#include "kernel_common.h"

namespace ra {

template <int DH>
struct BwdCfg {
    static constexpr int NT = 256;
    static constexpr int BQ = BWD_BQ, BK = BWD_BK;
    static constexpr int NKS = DH / 16;
    static constexpr int NDT = DH / 32;
    static constexpr int ROWB = DH * 2;             // natural Q/dO row (bytes)
    static constexpr int KCH = DH / 8;              // 16-byte chunks per natural row
    static constexpr int NAT_BYTES = BQ * ROWB;     // Q or dO tile, natural
    static constexpr int TR_BYTES = DH * BQ * 2;    // Q^T or dO^T tile (64 queries per row)
    static constexpr int KT_BYTES = DH * BK * 2;    // K^T of the work-group's keys
    static constexpr int DS_BYTES = BQ * BK * 2;    // dS [64 q][128 keys]
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_DO = OFF_Q + NAT_BYTES;
    static constexpr int OFF_QT = OFF_DO + NAT_BYTES;
    static constexpr int OFF_DOT = OFF_QT + TR_BYTES;
    static constexpr int OFF_KT = OFF_DOT + TR_BYTES;
    static constexpr int OFF_DS = OFF_KT + KT_BYTES;
    static constexpr int OFF_ROW = OFF_DS + DS_BYTES;  // lse2, delta, a, b per query row
    static constexpr int LDS = OFF_ROW + 4 * BQ * 4;
    static constexpr int LD = BQ * KCH / 4 / NT;       // 4-row x 16-byte loads per thread
    static_assert(BQ * KCH / 4 == NT || BQ * KCH / 4 == NT / 2, "tile shape");
    static constexpr int LDT = BQ * KCH / 4;           // threads that take part in a load
};

template <int KCH>
__device__ __forceinline__ int nat_swz(int row) {
    return KCH == 16 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int tr_swz(int d) { return (d >> 1) & 7; }
__device__ __forceinline__ int grp_slot(int m) { return m == 1 ? 2 : (m == 2 ? 1 : m); }

// Global -> registers: 4 consecutive query rows x one 16-byte chunk of Q and dO.
template <int DH>
struct BwdTileRegs {
    u32x4_t q[4], o[4];
};

template <int DH>
__device__ __forceinline__ void bwd_load_tile(BwdTileRegs<DH>& R, const uint16_t* qh,
                                              const uint16_t* oh, int64_t row_stride, int qt,
                                              int S, int tid) {
    using C = BwdCfg<DH>;
    if (tid >= C::LDT) return;
    const int m = tid / C::KCH, ch = tid % C::KCH;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = min(qt * C::BQ + 4 * m + rr, S - 1);
        R.q[rr] = *(const u32x4_t*)(qh + row * row_stride + ch * 8);
        R.o[rr] = *(const u32x4_t*)(oh + row * row_stride + ch * 8);
    }
}

// Registers -> LDS, natural rows and transposed (head dim major) copies.
template <int DH>
__device__ __forceinline__ void bwd_store_one(const u32x4_t (&x)[4], unsigned char* nat,
                                              unsigned char* tr, int tid) {
    using C = BwdCfg<DH>;
    const int m = tid / C::KCH, ch = tid % C::KCH;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int row = 4 * m + rr;
        *(u32x4_t*)(nat + row * C::ROWB + ((ch ^ nat_swz<C::KCH>(row)) << 4)) = x[rr];
    }
    const int sp = 16 * (m >> 2) + 4 * grp_slot(m & 3);  // stored position of rows 4m..4m+3
    const int chunk = sp >> 3, inner = (sp & 7) * 2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = ch * 8 + e, w = e >> 1;
        const uint32_t a0 = x[0][w], a1 = x[1][w], a2 = x[2][w], a3 = x[3][w];
        u32x2_t o;
        if (e & 1) {
            o[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            o[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
            o[0] = (a0 & 0xffffu) | (a1 << 16);
            o[1] = (a2 & 0xffffu) | (a3 << 16);
        }
        *(u32x2_t*)(tr + d * (C::BQ * 2) + ((chunk ^ tr_swz(d)) << 4) + inner) = o;
    }
}

template <int DH>
__global__ __launch_bounds__(256, 1) void bwd_step_bf16_kernel(BwdArgs p) {
    using C = BwdCfg<DH>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];
    unsigned char* sQ = smem + C::OFF_Q;
    unsigned char* sDO = smem + C::OFF_DO;
    unsigned char* sQT = smem + C::OFF_QT;
    unsigned char* sDOT = smem + C::OFF_DOT;
    unsigned char* sKT = smem + C::OFF_KT;
    unsigned char* sDS = smem + C::OFF_DS;
    float* sL = (float*)(smem + C::OFF_ROW);        // lse * log2(e) (+inf: no key visible)
    float* sD = sL + C::BQ;                         // Delta
    int32_t* sA = (int32_t*)(sD + C::BQ);           // visible key interval [a, b)
    int32_t* sB = sA + C::BQ;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nkt, bh = work / p.nkt;
    const int hk = bh % p.Hkv, b = bh / p.Hkv;
    const int kt = p.t_order[t];
    const int e0 = p.t_off[kt], e1 = p.t_off[kt + 1];
    const int group = p.Hq / p.Hkv;

    const int64_t kv_stride = (int64_t)p.Hkv * DH;
    const uint16_t* kb = p.k + (int64_t)b * p.Skv * kv_stride + hk * DH;
    const uint16_t* vb = p.v + (int64_t)b * p.Skv * kv_stride + hk * DH;
    const int key = kt * C::BK + wave * 32 + l32;   // this lane's key (C-layout column)
    const int keyc = min(key, p.Skv - 1);

    // Stationary operands: K and V rows of this lane's key (B operands of S, dP).
    u32x4_t kreg[C::NKS], vreg[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        kreg[ks] = *(const u32x4_t*)(kb + keyc * kv_stride + 16 * ks + 8 * g);
        vreg[ks] = *(const u32x4_t*)(vb + keyc * kv_stride + 16 * ks + 8 * g);
    }
    // K^T of the 128 keys in LDS (B operand of dQ = dS K): row d, keys contiguous.
    for (int idx = tid; idx < (C::BK / 4) * C::KCH; idx += C::NT) {
        const int m = idx / C::KCH, ch = idx % C::KCH;
        u32x4_t x[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int kr = min(kt * C::BK + 4 * m + rr, p.Skv - 1);
            x[rr] = *(const u32x4_t*)(kb + kr * kv_stride + ch * 8);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = ch * 8 + e, w = e >> 1;
            u32x2_t o;
            if (e & 1) {
                o[0] = (x[0][w] >> 16) | (x[1][w] & 0xffff0000u);
                o[1] = (x[2][w] >> 16) | (x[3][w] & 0xffff0000u);
            } else {
                o[0] = (x[0][w] & 0xffffu) | (x[1][w] << 16);
                o[1] = (x[2][w] & 0xffffu) | (x[3][w] << 16);
            }
            const int kp = 4 * m;  // key position in the row
            *(u32x2_t*)(sKT + d * (C::BK * 2) + (((kp >> 3) ^ (d & 15)) << 4) + (kp & 7) * 2) = o;
        }
    }

    f32x16_t dk_acc[C::NDT], dv_acc[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        dk_acc[dt] = (f32x16_t){};
        dv_acc[dt] = (f32x16_t){};
    }
    const float c2 = p.scale_log2;
    const int64_t q_stride = (int64_t)p.Hq * DH;
    const int n_ent = e1 - e0;
    const int n_iter = n_ent * group;

    BwdTileRegs<DH> R;
    if (n_iter > 0) {
        const int h0 = hk * group;
        const int qt0 = p.t_ent[e0] & 0x7fffffff;
        bwd_load_tile<DH>(R, p.q + ((int64_t)b * p.S) * q_stride + h0 * DH,
                          p.dout + ((int64_t)b * p.S) * q_stride + h0 * DH, q_stride, qt0, p.S, tid);
    }
    for (int it = 0; it < n_iter; ++it) {
        const int hh = it / n_ent, ei = e0 + it % n_ent;
        const int h = hk * group + hh;
        const int ent = p.t_ent[ei];
        const int qt = ent & 0x7fffffff;
        const bool partial = ent < 0;

        __syncthreads();  // previous iteration's readers of the Q/dO/dS stages are done
        if (tid < C::LDT) {
            bwd_store_one<DH>(R.q, sQ, sQT, tid);
            bwd_store_one<DH>(R.o, sDO, sDOT, tid);
        }
        if (tid < C::BQ) {
            const int iq = qt * C::BQ + tid;
            float l2 = INFINITY, dl = 0.f;
            int a = 0, bb = 0;
            if (iq < p.S) {
                const float L = p.lse[((int64_t)b * p.Hq + h) * p.S + iq];
                l2 = L == -INFINITY ? INFINITY : L * kLog2e;
                dl = p.delta[((int64_t)b * p.Hq + h) * p.S_pad + iq];
                a = p.rng[2 * iq];
                bb = p.rng[2 * iq + 1];
            }
            sL[tid] = l2;
            sD[tid] = dl;
            sA[tid] = a;
            sB[tid] = bb;
        }
        __syncthreads();
        if (it + 1 < n_iter) {
            const int hn = hk * group + (it + 1) / n_ent;
            const int qn = p.t_ent[e0 + (it + 1) % n_ent] & 0x7fffffff;
            bwd_load_tile<DH>(R, p.q + ((int64_t)b * p.S) * q_stride + hn * DH,
                              p.dout + ((int64_t)b * p.S) * q_stride + hn * DH, q_stride, qn, p.S,
                              tid);
        }

        // S = Q K^T and dP = dO V^T: two 32-row halves of the 64-row tile.
        f32x16_t sacc[2], pacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = (f32x16_t){};
            pacc[mt] = (f32x16_t){};
            const int row = 32 * mt + l32;
            const int sw = nat_swz<C::KCH>(row);
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                const int off = row * C::ROWB + (((2 * ks + g) ^ sw) << 4);
                sacc[mt] = mfma_32x32x16(*(const u32x4_t*)(sQ + off), kreg[ks], sacc[mt]);
                pacc[mt] = mfma_32x32x16(*(const u32x4_t*)(sDO + off), vreg[ks], pacc[mt]);
            }
        }
        // P and dS; element (mt, r) is query row 32*mt + 8*(r/4) + 4*g + r%4.
        u32x4_t pb[4], db[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int r0 = 32 * mt + 8 * rg + 4 * g;
                const f32x4_t L = *(const f32x4_t*)(sL + r0);
                const f32x4_t Dl = *(const f32x4_t*)(sD + r0);
                float pv[4], dsv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float pr = fast_exp2(fmaf(sacc[mt][4 * rg + i], c2, -L[i]));
                    if (partial) {
                        const bool vis = key >= sA[r0 + i] && key < sB[r0 + i];
                        pr = vis ? pr : 0.f;
                    }
                    pv[i] = pr;
                    dsv[i] = pr * (pacc[mt][4 * rg + i] - Dl[i]);
                }
                const int kk = 2 * mt + (rg >> 1), w = (rg & 1) * 2;
                pb[kk][w] = pack_bf16x2(pv[0], pv[1]);
                pb[kk][w + 1] = pack_bf16x2(pv[2], pv[3]);
                db[kk][w] = pack_bf16x2(dsv[0], dsv[1]);
                db[kk][w + 1] = pack_bf16x2(dsv[2], dsv[3]);
                // dS -> LDS [query][key] for the dQ product
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int qrow = r0 + i, kcol = wave * 32 + l32;
                    const uint32_t wv = db[kk][w + (i >> 1)];
                    const uint16_t hv = (i & 1) ? (uint16_t)(wv >> 16) : (uint16_t)(wv & 0xffff);
                    *(uint16_t*)(sDS + qrow * (C::BK * 2) + (((kcol >> 3) ^ (qrow & 15)) << 4) +
                                 (kcol & 7) * 2) = hv;
                }
            }
        // dV^T += dO^T P and dK^T += Q^T dS
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) {
            const int row = 32 * dt + l32;
            const int sw = tr_swz(row);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int off = row * (C::BQ * 2) + (((2 * kk + g) ^ sw) << 4);
                dv_acc[dt] = mfma_32x32x16(*(const u32x4_t*)(sDOT + off), pb[kk], dv_acc[dt]);
                dk_acc[dt] = mfma_32x32x16(*(const u32x4_t*)(sQT + off), db[kk], dk_acc[dt]);
            }
        }
        __syncthreads();  // dS of every wave is in LDS

        // dQ[64 x DH] = dS[64 x 128] K[128 x DH]; wave tiles (mt, nt) of 32 x 32.
        constexpr int TILES = 2 * C::NDT;
        constexpr int PER_WAVE = TILES / 4;
#pragma unroll
        for (int tw = 0; tw < PER_WAVE; ++tw) {
            const int tile = wave * PER_WAVE + tw;
            const int mt = tile / C::NDT, nt = tile % C::NDT;
            f32x16_t acc = (f32x16_t){};
            const int arow = 32 * mt + l32, brow = 32 * nt + l32;
#pragma unroll
            for (int ks = 0; ks < C::BK / 16; ++ks) {
                const u32x4_t a =
                    *(const u32x4_t*)(sDS + arow * (C::BK * 2) + (((2 * ks + g) ^ (arow & 15)) << 4));
                const u32x4_t bo =
                    *(const u32x4_t*)(sKT + brow * (C::BK * 2) + (((2 * ks + g) ^ (brow & 15)) << 4));
                acc = mfma_32x32x16(a, bo, acc);
            }
            // acc: column d = 32*nt + l32, rows 32*mt + 8*(r/4) + 4*g + r%4
            float* dqh = p.dq + ((int64_t)b * p.S) * q_stride + h * DH + 32 * nt + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int iq = qt * C::BQ + 32 * mt + 8 * (r >> 2) + 4 * g + (r & 3);
                if (iq < p.S) unsafeAtomicAdd(dqh + iq * q_stride, acc[r] * p.scale);
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
