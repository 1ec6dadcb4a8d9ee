// Measurement aids (not part of the attention path): kernels that do nothing
// but bf16 MFMAs (on nearly constant operands, and on operands with the bit
// statistics of N(0,1) data), to measure what the matrix cores of this GPU
// deliver when they are the only thing running, under the clocks the chip then
// holds; and streaming kernels (a copy, an add that reads two bytes per byte
// written, as the LSE merge does, and a read-only fold), to measure what HBM
// delivers to plain streaming kernels.  Built into their own library
// (libraprobe.so), loaded by bench.py and the tests only.
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

// The same MFMA chains on operands with the bit statistics of N(0,1) bf16
// data (random sign, exponents for magnitudes 1/8 .. 4, random mantissas), 8
// operand sets per lane, each MFMA of a chain taking the next set, so that the
// matrix cores switch about as many bits as on attention inputs.  The chip
// holds a lower clock on such data than on the nearly constant operands
// above, for the same instructions.
__global__ __launch_bounds__(256) void mfma_peak_random_kernel(float* out, int iters) {
    uint32_t x = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 0x9e3779b9u;
    auto bf16_rand = [&]() {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        const uint32_t sign = x & 0x8000u, mant = x & 0x7fu, ex = 124u + (x >> 16) % 5u;
        return (short)(sign | (ex << 7) | mant);
    };
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int sidx = 0; sidx < 8; ++sidx)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[sidx][i] = bf16_rand();
            b[sidx][i] = bf16_rand();
        }
    f32x16_t acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = (f32x16_t){};
    for (int it = 0; it < iters; it += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int c = 0; c < CHAINS; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + c) & 7], b[(k + 3 * c + 1) & 7],
                                                                 acc[c], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int STREAM_UNROLL = 8;   // independent 16-byte chunks in flight per thread

template <bool NT>
__device__ __forceinline__ f32x4_t ld16(const f32x4_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st16(f32x4_t v, f32x4_t* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Over n 16-byte chunks: dst[i] = a[i] (ADD = false, one byte read per byte
// written, like a copy) or dst[i] = a[i] + b[i] as four floats (ADD = true,
// two read per written, like the LSE merge).  Chunk i of a pass goes to
// thread i % (grid threads), so each wave instruction moves 1 KiB of
// contiguous memory; every thread keeps STREAM_UNROLL chunks in flight.
template <bool ADD, bool NT_LD, bool NT_ST>
__global__ __launch_bounds__(256) void stream_kernel(const f32x4_t* __restrict__ a,
                                                     const f32x4_t* __restrict__ b,
                                                     f32x4_t* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (STREAM_UNROLL - 1) * stride < n; i += STREAM_UNROLL * stride) {
        f32x4_t v[STREAM_UNROLL];
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = ld16<NT_LD>(a + i + u * stride);
        if constexpr (ADD) {
#pragma unroll
            for (int u = 0; u < STREAM_UNROLL; ++u) v[u] += ld16<NT_LD>(b + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; ++u) st16<NT_ST>(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) {
        if constexpr (ADD) dst[i] = a[i] + b[i];
        else dst[i] = a[i];
    }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// The xor of a chunk's four words.  The whole vector is bit-cast: this
// compiler folds a bit-cast of a single vector element (v[k]) as if every
// element were the first, which turns the xor of four of them into zero.
__device__ __forceinline__ uint32_t xor4(f32x4_t v) {
    const u32x4_t w = __builtin_bit_cast(u32x4_t, v);
    return w.x ^ w.y ^ w.z ^ w.w;
}

// Read-only streaming: each thread folds its chunks of a[0 .. n) into one
// word (the xor of their bits, so no load is optimised away) and writes it to
// out[thread] (4 bytes per thread).
template <bool NT_LD>
__global__ __launch_bounds__(256) void stream_read_kernel(const f32x4_t* __restrict__ a,
                                                          uint32_t* __restrict__ out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t x = 0;
    for (; i + (STREAM_UNROLL - 1) * stride < n; i += STREAM_UNROLL * stride) {
        f32x4_t v[STREAM_UNROLL];
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; ++u) v[u] = ld16<NT_LD>(a + i + u * stride);
#pragma unroll
        for (int u = 0; u < STREAM_UNROLL; ++u) x ^= xor4(v[u]);
    }
    for (; i < n; i += stride) x ^= xor4(ld16<NT_LD>(a + i));
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x;
}

template <bool ADD>
void launch_stream(int flags, int blocks, hipStream_t s, const f32x4_t* a, const f32x4_t* b,
                   f32x4_t* d, int64_t n) {
    switch (flags & 3) {
        case 0: hipLaunchKernelGGL((stream_kernel<ADD, false, false>), dim3(blocks), dim3(256), 0, s, a, b, d, n); break;
        case 1: hipLaunchKernelGGL((stream_kernel<ADD, true, false>), dim3(blocks), dim3(256), 0, s, a, b, d, n); break;
        case 2: hipLaunchKernelGGL((stream_kernel<ADD, false, true>), dim3(blocks), dim3(256), 0, s, a, b, d, n); break;
        default: hipLaunchKernelGGL((stream_kernel<ADD, true, true>), dim3(blocks), dim3(256), 0, s, a, b, d, n); break;
    }
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

// As ra_probe_mfma (same flops, ra_probe_mfma_flops), on operands with the
// bit statistics of N(0,1) bf16 data that change from one MFMA to the next.
int ra_probe_mfma_random(float* out, int32_t blocks, int32_t iters, hipStream_t stream) {
    if (out == nullptr || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_random_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}

// Read `bytes` bytes of a (16-byte aligned, a multiple of 16) with `blocks`
// work-groups of 256 threads on `stream`; out receives blocks * 256 uint32.
// flags bit 0: non-temporal loads.  Returns a hipError_t value.
int ra_probe_stream_read(const void* a, void* out, int64_t bytes, int32_t blocks, int32_t flags,
                         hipStream_t stream) {
    if (a == nullptr || out == nullptr || bytes < 0 || bytes % 16 != 0 || blocks <= 0 || flags < 0 ||
        flags > 1 || ((uintptr_t)a | (uintptr_t)out) % 16 != 0)
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return (int)hipSuccess;
    if (flags & 1)
        hipLaunchKernelGGL(stream_read_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                           (const f32x4_t*)a, (uint32_t*)out, bytes / 16);
    else
        hipLaunchKernelGGL(stream_read_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                           (const f32x4_t*)a, (uint32_t*)out, bytes / 16);
    return (int)hipGetLastError();
}

// dst = a (b == NULL) or dst = a + b as floats (b != NULL), over `bytes`
// bytes of device memory (every pointer 16-byte aligned, bytes a multiple of
// 16, dst overlapping neither input) with `blocks` work-groups of 256 threads
// on `stream`.  flags bit 0: non-temporal loads, bit 1: non-temporal stores.
// Returns a hipError_t value.
int ra_probe_stream(const void* a, const void* b, void* dst, int64_t bytes, int32_t blocks,
                    int32_t flags, hipStream_t stream) {
    if (a == nullptr || dst == nullptr || bytes < 0 || bytes % 16 != 0 || blocks <= 0 ||
        flags < 0 || flags > 3 || ((uintptr_t)a | (uintptr_t)b | (uintptr_t)dst) % 16 != 0)
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return (int)hipSuccess;
    const int64_t n = bytes / 16;
    if (b == nullptr)
        launch_stream<false>(flags, blocks, stream, (const f32x4_t*)a, nullptr, (f32x4_t*)dst, n);
    else
        launch_stream<true>(flags, blocks, stream, (const f32x4_t*)a, (const f32x4_t*)b, (f32x4_t*)dst, n);
    return (int)hipGetLastError();
}

}  // extern "C"
