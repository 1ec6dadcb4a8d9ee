// Measurement aid (not part of the attention path): a kernel that does
// nothing but bf16 MFMAs, to measure what the matrix cores of this GPU deliver
// when they are the only thing running, under the clocks the chip then holds.
// Built into its own library (libraprobe.so), loaded by bench.py only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int CHAINS = 4;   // independent accumulators per wave

// Each wave runs CHAINS independent chains of v_mfma_f32_32x32x16_bf16
// (32*32*16*2 flops each), iters (rounded up to a multiple of 8) MFMAs per
// chain.  One element of the A operand changes after every round of MFMAs (one
// xor), so that the matrix cores see changing data as in real use; the result
// is written out so that nothing is optimised away.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (short)(0x3c00 + ((lane * 37 + i * 11) & 0x7f));
        b[i] = (short)(0x3c00 + ((lane * 53 + i * 7) & 0x7f));
    }
    f32x16_t acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = (f32x16_t){};
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
            for (int c = 0; c < CHAINS; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
            a[k] ^= (short)((it + k) & 0x3f);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Flops one launch of ra_probe_mfma performs.
double ra_probe_mfma_flops(int32_t blocks, int32_t iters) {
    return (double)blocks * 4 /* waves */ * ((iters + 7) / 8 * 8) * CHAINS * (32.0 * 32.0 * 16.0 * 2.0);
}

// Launch `blocks` work-groups of 4 waves on `stream`; `out` must hold
// blocks * 256 floats.  Returns a hipError_t value.
int ra_probe_mfma(float* out, int32_t blocks, int32_t iters, hipStream_t stream) {
    if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
