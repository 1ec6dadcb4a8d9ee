// Device helpers shared by the HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Two fp32 -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D = A * B + C on a 32x32x16 bf16 tile.  Lane l holds, for A (32 x 16):
// row l%32, k = 8*(l/32) .. +7; for B (16 x 32): column l%32, the same k; for
// C/D: column l%32, rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap(x, x) returns
// two registers: the first holds x[l] on lanes 0-31 and x[l-32] on lanes
// 32-63, the second x[l+32] on lanes 0-31 and x[l] on lanes 32-63; combining
// the two gives the pair reduction on every lane.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                              __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                              __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Plan arrays (tile lists, orders) are never written while a kernel runs; reading
// them through the constant address space lets uniform indices use scalar
// loads, which do not wait behind outstanding vector memory operations.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;
__device__ __forceinline__ cint_ptr as_const(const int32_t* p) { return (cint_ptr)(p); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte slot of logical chunk c in row r of an LDS tile whose rows hold NCH
// chunks (16: 256-byte rows; 8: 128-byte rows, two rows per 256 bytes).  LDS
// serves 256 bytes (sixteen 16-byte bank groups) per cycle; the XOR patterns
// put on distinct bank groups both 16 consecutive rows at one chunk (the
// 16-lane phases of a ds_read_b128 operand read) and every aligned block of 4
// rows x 4 chunks (the half-wave phases of a ds_read_b64_tr_b16 transpose
// read).  Each pattern is its own inverse within a row.
template <int NCH>
__device__ __forceinline__ int swz_slot(int r, int c) {
    static_assert(NCH == 16 || NCH == 8, "row width");
    if (NCH == 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int NCH>
__device__ __forceinline__ int swz_off(int r, int c) {
    return r * (NCH * 16) + (swz_slot<NCH>(r, c) << 4);
}

// Tiles of ROWS rows x DH bf16 values (one head) of a row-major tensor
// [rows, heads, DH] copied straight into LDS by buffer loads
// (buffer_load_dwordx4 ... lds: the 16 bytes of lane l land at the
// wave-uniform LDS base + 16*l).  Instruction c of wave w fills LDS chunks
// NT*c + 64w + lane; the lane whose slot there is physical chunk p of row r
// loads logical chunk swz_slot(r, p), so the tile lands XOR-swizzled.  The
// buffer spans the tensor's `nrows` rows, so rows past the end read as zeros;
// the per-lane part of every offset is fixed and a tile moves only the scalar
// offset.  Byte offsets are 32-bit: nrows * row bytes must stay below 2^32.
template <int DH, int ROWS, int NT = 256>
struct BufTileLoader {
    static constexpr int KCH = DH / 8;
    static constexpr int NLD = ROWS * KCH / NT;   // instructions per thread per tile
    static_assert(NLD >= 1 && ROWS * KCH % NT == 0, "tile shape");
    __amdgpu_buffer_rsrc_t rsrc;
    int voff[NLD];
    int tile_bytes;   // bytes from one tile to the next
    int head_off;     // bytes from the start of a row to this head

    __device__ __forceinline__ void init(const uint16_t* base, int nrows, int heads, int head,
                                         int wave, int lane) {
        const int row_bytes = heads * DH * 2;
        tile_bytes = ROWS * row_bytes;
        head_off = head * DH * 2;
        rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrows * row_bytes, 0x00020000);
#pragma unroll
        for (int c = 0; c < NLD; ++c) {
            const int idx = NT * c + 64 * wave + lane;
            const int row = idx / KCH, pc = idx % KCH;
            voff[c] = row * row_bytes + swz_slot<KCH>(row, pc) * 16;
        }
    }
    // tile `t` (rows ROWS*t ..) of head `head` (default: the head of init)
    __device__ __forceinline__ void load(unsigned char* lds, int t, int wave, int head = -1) const {
        load_from(lds, rsrc, t, wave, head);
    }
    // the same tile of another buffer of the same shape (e.g. another KV block)
    __device__ __forceinline__ void load_from(unsigned char* lds, __amdgpu_buffer_rsrc_t r, int t,
                                              int wave, int head = -1) const {
        const int soff = t * tile_bytes + (head < 0 ? head_off : head * DH * 2);
#pragma unroll
        for (int c = 0; c < NLD; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(lds + (NT * c + 64 * wave) * 16), 16,
                voff[c], soff, 0, 0);
    }
    // buffer over the nrows rows of another tensor laid out like the first
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const uint16_t* base, int nrows,
                                                              int heads) const {
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, nrows * heads * DH * 2,
                                                 0x00020000);
    }
};

// K and V tiles of one kv head (rows = keys of a [B, Skv, Hkv, DH] block),
// loaded by a work-group of NT threads.
template <int DH, int ROWS, int NT = 256>
struct KvLoader {
    BufTileLoader<DH, ROWS, NT> lk, lv;
    __device__ __forceinline__ void init(const uint16_t* k, const uint16_t* v, int b, int Skv,
                                         int Hkv, int hk, int wave, int lane) {
        const int64_t batch = (int64_t)b * Skv * Hkv * DH;
        lk.init(k + batch, Skv, Hkv, hk, wave, lane);
        lv.init(v + batch, Skv, Hkv, hk, wave, lane);
    }
    __device__ __forceinline__ void load(unsigned char* kdst, unsigned char* vdst, int t,
                                         int wave) const {
        lk.load(kdst, t, wave);
        lv.load(vdst, t, wave);
    }
};

// Blocks of a launch are dealt to the 8 XCDs round-robin; this remaps the
// block index so that each XCD receives one contiguous range of work items
// (neighbouring items share K/V and therefore that XCD's L2).  grid % 8 == 0.
__device__ __forceinline__ int xcd_work_index(int bid, int grid) {
    return (bid & 7) * (grid >> 3) + (bid >> 3);
}

}  // namespace ra
