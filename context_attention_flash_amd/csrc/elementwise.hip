// Memory-bound kernels of the ring step:
//   K2 lse_merge   -- the log-sum-exp merge of a partial into the running
//                     result (instagit/nanotron page, "Numerically-Stable
//                     Output Fusion"), one pass over fp32 rows;
//   K5 finalize    -- running fp32 output -> output dtype;
//   K3 bwd_pre     -- per-row values of the backward: -Delta = -rowsum(dout *
//                     out) and the lse in base 2;
//   dq_finalize    -- the dQ accumulator (kept in the MFMA accumulator layout of
//                     the dQ kernel: per 32-row group of one head,
//                     [d/32][4][64 lanes][4] floats) -> the caller's dq
//                     [B, S, Hq, d].
#include "kernel_args.h"
#include "kernel_common.h"

namespace ra {

// Rows are owned by waves: a row of c4 = d/4 float4 items is handled by a
// group of G = 2^lg lanes of ONE wave (G = the smallest power of two >= c4,
// at most 64; lane c of the group takes items c, c + G, ...), so the lanes that
// read a row's running lse and the lane that writes the merged one belong to
// the same wave, whose store cannot issue before its own loads have returned.
// Each wave walks MERGE_ITEMS groups of 64/G rows; every item's loads are
// issued (from clamped, always valid addresses) before any item is used, to
// keep enough bytes in flight, and only the stores are predicated.
constexpr int MERGE_ITEMS = 4;

__global__ __launch_bounds__(256) void lse_merge_kernel(float* __restrict__ out,
                                                        float* __restrict__ lse,
                                                        const float* __restrict__ oj,
                                                        const float* __restrict__ lj,
                                                        int64_t n_rows, int64_t S, int32_t H,
                                                        int32_t c4, int32_t lg) {
    const int lane = threadIdx.x & 63;
    const int c0 = lane & ((1 << lg) - 1), rsub = lane >> lg, rg = 64 >> lg;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    for (int cb = 0; cb < c4; cb += 1 << lg) {       // one pass unless d > 256
        const int c = cb + c0, cc = min(c, c4 - 1);
        f32x4_t o[MERGE_ITEMS], x[MERGE_ITEMS];
        float L[MERGE_ITEMS], Lj[MERGE_ITEMS];
        int64_t li[MERGE_ITEMS], item[MERGE_ITEMS];
        bool live[MERGE_ITEMS];
#pragma unroll
        for (int it = 0; it < MERGE_ITEMS; ++it) {
            const int64_t row = (wave * MERGE_ITEMS + it) * rg + rsub;   // (b, s, h)
            live[it] = row < n_rows && c < c4;
            const int64_t rw = min(row, n_rows - 1);
            const int64_t h = rw % H, bs = rw / H;
            const int64_t b = bs / S, s = bs % S;
            li[it] = (b * H + h) * S + s;
            item[it] = rw * c4 + cc;
        }
        // all loads of the pass in one group, ahead of every use
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < MERGE_ITEMS; ++it) {
            o[it] = __builtin_nontemporal_load((const f32x4_t*)out + item[it]);
            x[it] = __builtin_nontemporal_load((const f32x4_t*)oj + item[it]);
            L[it] = lse[li[it]];
            Lj[it] = lj[li[it]];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < MERGE_ITEMS; ++it) {
            const float M = fmaxf(L[it], Lj[it]);
            const bool empty = M == -INFINITY;
            const float Ms = empty ? 0.f : M;
            const float a = expf(L[it] - Ms), e = expf(Lj[it] - Ms), den = a + e;
            const float Ln = empty ? -INFINITY : Ms + logf(den);
            const float wa = empty ? 0.f : a / den, we = empty ? 0.f : e / den;
            const f32x4_t r = wa * o[it] + we * x[it];
            if (live[it]) {
                __builtin_nontemporal_store(r, (f32x4_t*)out + item[it]);
                // lane 0 of the group writes the merged lse in the row's last pass
                if (c0 == 0 && cb + (1 << lg) >= c4) lse[li[it]] = Ln;
            }
        }
    }
}

hipError_t launch_lse_merge(float* out, float* lse, const float* out_j, const float* lse_j,
                            int32_t B, int64_t S, int32_t H, int32_t d, hipStream_t s) {
    const int64_t n_rows = (int64_t)B * S * H;
    const int c4 = d / 4;
    if (n_rows == 0 || c4 == 0) return hipSuccess;
    int lg = 0;
    while ((1 << lg) < c4 && lg < 6) ++lg;
    const int64_t rows_per_block = 4LL * MERGE_ITEMS * (64 >> lg);
    const int64_t grid = (n_rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)grid), dim3(256), 0, s, out, lse, out_j,
                       lse_j, n_rows, S, H, c4, lg);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ o, void* out,
                                                       int is_bf16, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const f32x4_t x = ((const f32x4_t*)o)[i];
    if (is_bf16) {
        ((u32x2_t*)out)[i] = (u32x2_t){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    } else {
        ((f32x4_t*)out)[i] = x;
    }
}

hipError_t launch_finalize(const float* o, void* out, int is_bf16, int64_t n, hipStream_t s) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, o,
                       out, is_bf16, n4);
    return hipGetLastError();
}

// K3: one group of d/8 lanes per padded row (b, s, h), rows ordered
// [B][S_pad][Hq]; each lane reads 8 elements of dout and of out.  Writes
// -Delta = -rowsum(dout * out) and lse2 = lse * log2(e) (+inf where lse is
// -inf, i.e. the row sees no key), and 0 / +inf on the padding rows s >= S,
// so that the backward kernels need no per-row special cases.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdPreArgs a) {
    const int lanes_per_row = a.d / 8;
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = gt / lanes_per_row;
    const int c = (int)(gt % lanes_per_row);
    const int64_t rows = (int64_t)a.B * a.S_pad * a.Hq;
    const int64_t h = row % a.Hq, bs = row / a.Hq;
    const int64_t b = bs / a.S_pad, s = bs % a.S_pad;
    const bool live = row < rows && s < a.S;
    float sum = 0.f;
    if (live) {
        const int64_t src = ((b * a.S + s) * a.Hq + h) * lanes_per_row + c;
        if (BF16) {
            const u32x4_t x = *((const u32x4_t*)a.dout + src);
            const u32x4_t y = *((const u32x4_t*)a.out + src);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                sum += bf16_lo(x[w]) * bf16_lo(y[w]) + bf16_hi(x[w]) * bf16_hi(y[w]);
        } else {
            const f32x4_t* xp = (const f32x4_t*)a.dout + 2 * src;
            const f32x4_t* yp = (const f32x4_t*)a.out + 2 * src;
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const f32x4_t x = xp[w], y = yp[w];
                sum += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
            }
        }
    }
    for (int off = lanes_per_row / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (row < rows && c == 0) {
        const int64_t dst = (b * a.Hq + h) * a.S_pad + s;
        float l2 = INFINITY;
        if (live) {
            const float L = a.lse[(b * a.Hq + h) * a.S + s];
            l2 = L == -INFINITY ? INFINITY : L * kLog2e;
        }
        a.ndelta[dst] = -sum;
        a.lse2[dst] = l2;
    }
}

// One thread per 4 floats of a (b, s, h) row of the caller's dq.  Head-dim
// index dd = 4c lives in accumulator lane (s % 32) + 32 * ((dd / 4) % 2), slot
// (dd / 32) * 4 + (dd / 8) % 4 of the row group s / 32.
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ acc,
                                                          float* __restrict__ dq, int32_t S,
                                                          int32_t Hq, int32_t S_pad, int32_t d,
                                                          int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const int c4 = d / 4;
    const int64_t row = i / c4;                 // row = (b * S + s) * Hq + h
    const int dd = (int)(i % c4) * 4;
    const int64_t h = row % Hq, bs = row / Hq;
    const int64_t b = bs / S, s = bs % S;
    const int64_t grp = (b * Hq + h) * (S_pad / 32) + s / 32;
    const int lane = (int)(s % 32) + 32 * ((dd >> 2) & 1);
    const int slotidx = (dd >> 5) * 4 + ((dd >> 3) & 3);
    ((f32x4_t*)dq)[i] = ((const f32x4_t*)acc)[grp * (8 * d) + slotidx * 64 + lane];
}

hipError_t launch_dq_finalize(const float* dq_acc, float* dq, int32_t B, int32_t S, int32_t Hq,
                              int32_t S_pad, int32_t d, hipStream_t s) {
    const int64_t n4 = (int64_t)B * S * Hq * (d / 4);
    if (n4 == 0) return hipSuccess;
    hipLaunchKernelGGL(dq_finalize_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s,
                       dq_acc, dq, S, Hq, S_pad, d, n4);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdPreArgs& a, int is_bf16, hipStream_t s) {
    const int64_t threads = (int64_t)a.B * a.S_pad * a.Hq * (a.d / 8);
    if (threads == 0) return hipSuccess;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (is_bf16)
        hipLaunchKernelGGL(bwd_pre_kernel<true>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(bwd_pre_kernel<false>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ra
