// K1 (fp32 inputs): one ring step of the flash forward in fp32 on the vector
// ALUs.  Same schedule, tile lists and step epilogues as the bf16 kernel;
// one thread owns one query row of the 128-row tile, K/V tiles of 64 keys are
// staged in LDS and read as broadcasts.  The running output of this kernel
// family is a plain fp32 [B, Hq, S_pad, d] array.
#include "kernel_args.h"
#include "kernel_common.h"

namespace ra {

template <int DH>
__global__ __launch_bounds__(128) void fwd_step_f32_kernel(FwdArgs p) {
    constexpr int BK = FWD_BK;
    __shared__ __attribute__((aligned(16))) float Ks[BK * DH];
    __shared__ __attribute__((aligned(16))) float Vs[BK * DH];

    const int tid = threadIdx.x;
    const int work = xcd_work_index(blockIdx.x, gridDim.x);
    if (work >= p.total_work) return;
    const int t = work % p.nqt, bh = work / p.nqt;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int qt = p.t_order[t];
    const int hk = (h * p.Hkv) / p.Hq;
    const int e0 = p.t_off[qt], e1 = p.t_off[qt + 1];
    const int iq = qt * FWD_BQ + tid;
    const int iqc = min(iq, p.S - 1);
    const bool valid = iq < p.S;

    float q[DH], acc[DH];
    const float* qrow = (const float*)p.q + ((int64_t)(b * p.S + iqc) * p.Hq + h) * DH;
#pragma unroll
    for (int c = 0; c < DH; c += 4) {
        const f32x4_t x = *(const f32x4_t*)(qrow + c);
        q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
        acc[c] = acc[c + 1] = acc[c + 2] = acc[c + 3] = 0.f;
    }
    const int ra = p.rng[2 * iq], rb = p.rng[2 * iq + 1];
    const float scale = p.scale_log2 * kLn2;
    float m_run = -INFINITY, l_run = 0.f;

    const int64_t row_stride = (int64_t)p.Hkv * DH;
    const float* kb = (const float*)p.k + (int64_t)b * p.Skv * row_stride + hk * DH;
    const float* vb = (const float*)p.v + (int64_t)b * p.Skv * row_stride + hk * DH;

    for (int e = e0; e < e1; ++e) {
        const int ent = p.t_ent[e];
        const int kt = ent & 0x7fffffff;
        __syncthreads();
        for (int idx = tid; idx < BK * DH / 4; idx += 128) {
            const int row = idx / (DH / 4), c4 = idx % (DH / 4);
            const int key = min(kt * BK + row, p.Skv - 1);
            *(f32x4_t*)(Ks + row * DH + 4 * c4) = *(const f32x4_t*)(kb + key * row_stride + 4 * c4);
            *(f32x4_t*)(Vs + row * DH + 4 * c4) = *(const f32x4_t*)(vb + key * row_stride + 4 * c4);
        }
        __syncthreads();
        float s[BK];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < BK; ++u) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < DH; ++c) dot = fmaf(q[c], Ks[u * DH + c], dot);
            const int key = kt * BK + u;
            s[u] = (ent < 0 && (key < ra || key >= rb)) ? -INFINITY : dot * scale;
            mx = fmaxf(mx, s[u]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < DH; ++c) acc[c] *= alpha;
#pragma unroll
        for (int u = 0; u < BK; ++u) {
            const float pu = expf(s[u] - m_use);
            l_run += pu;
#pragma unroll
            for (int c = 0; c < DH; ++c) acc[c] = fmaf(pu, Vs[u * DH + c], acc[c]);
        }
    }

    const bool empty = !(l_run > 0.f);
    const float inv = empty ? 0.f : 1.f / l_run;
    const float Lj = empty ? -INFINITY : m_run + logf(l_run);
    const int64_t lse_idx = ((int64_t)b * p.Hq + h) * p.S + iq;
    float* orun = p.o_run + (((int64_t)b * p.Hq + h) * p.S_pad + iq) * DH;
    float w_old = 0.f, w_new = inv, L_out = Lj;
    const int mode = p.mode;
    if (mode == FWD_MERGE || mode == FWD_LAST) {
        const float Lr = valid ? p.lse[lse_idx] : -INFINITY;
        const float M = fmaxf(Lr, Lj);
        if (M == -INFINITY) {
            w_old = 0.f; w_new = 0.f; L_out = -INFINITY;
        } else {
            const float er = expf(Lr - M), ej = expf(Lj - M), den = er + ej;
            L_out = M + logf(den);
            w_old = er / den;
            w_new = ej * inv / den;
        }
    }
    if (!valid) {
        if (mode == FWD_FIRST || mode == FWD_MERGE)
            for (int c = 0; c < DH; ++c) orun[c] = 0.f;
        return;
    }
    float* dst;
    if (mode == FWD_FIRST || mode == FWD_MERGE) dst = orun;
    else if (mode == FWD_PARTIAL) dst = p.o_part + ((int64_t)(b * p.S + iq) * p.Hq + h) * DH;
    else dst = (float*)p.out + ((int64_t)(b * p.S + iq) * p.Hq + h) * DH;
    const bool read_old = mode == FWD_MERGE || mode == FWD_LAST;
#pragma unroll
    for (int c = 0; c < DH; c += 4) {
        f32x4_t o = {acc[c] * w_new, acc[c + 1] * w_new, acc[c + 2] * w_new, acc[c + 3] * w_new};
        if (read_old) o += w_old * *(const f32x4_t*)(orun + c);
        *(f32x4_t*)(dst + c) = o;
    }
    if (mode == FWD_PARTIAL) p.lse_part[lse_idx] = Lj;
    else p.lse[lse_idx] = L_out;
}

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, hipStream_t s) {
    const int grid = (a.total_work + 7) / 8 * 8;
    if (head_dim == 64)
        hipLaunchKernelGGL(fwd_step_f32_kernel<64>, dim3(grid), dim3(128), 0, s, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL(fwd_step_f32_kernel<128>, dim3(grid), dim3(128), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace ra
