// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, MFMA wrappers, LDS swizzles and the relation (mask) logic.
//
// MFMA register layouts used throughout (wave64, lane = 0..63, g = lane / 32,
// c = lane % 32):
//   v_mfma_f32_32x32x16_{f16,bf16}: A (32 x 16): lane holds A[c][8g .. 8g+7];
//     B (16 x 32): lane holds B[8g .. 8g+7][c];
//   v_mfma_f32_32x32x2_f32:         A (32 x 2):  lane holds A[c][g];
//     B (2 x 32):  lane holds B[g][c];
//   both: the 32 x 32 f32 result sits in 16 registers, register r of a lane
//     holding D[8 * (r / 4) + 4 * g + (r % 4)][c].
// The contraction index is only ever paired slot-for-slot between A and B, so
// a kernel may assign any permutation of its contraction index to the slots as
// long as A and B use the same one; the kernels use that freedom to read
// operands straight from registers or in 16-byte LDS vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace osattn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// 16-bit element traits: the 8-wide operand vector and the 32x32x16 MFMA.
template <typename T> struct Half8;
template <> struct Half8<_Float16> {
    typedef f16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Half8<__bf16> {
    typedef bf16x8 vec;
    static __device__ __forceinline__ f32x16 mma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename V> __device__ __forceinline__ V zero_vec() {
    V z;
    for (int i = 0; i < (int)(sizeof(V) / sizeof(z[0])); ++i) z[i] = 0;
    return z;
}

// 16-byte global load; returns zeros when !ok (the address is not touched).
__device__ __forceinline__ u32x4 load16(const void *p, bool ok) {
    u32x4 r = {0u, 0u, 0u, 0u};
    if (ok) r = *reinterpret_cast<const u32x4 *>(p);
    return r;
}

// Row-major LDS tile of 16-byte chunks with an XOR swizzle: chunk c of row r
// lives at chunk c ^ (r & 7).  Eight consecutive rows read at the same logical
// chunk then hit eight different bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Transposed V tile (16-bit types): row = feature d, columns = key slots.
// Eight consecutive d rows map a logical chunk to eight distinct physical
// chunks, and so do rows d, d + 8, ..., d + 56 (the writer's pattern).
__device__ __forceinline__ int swz_t(int d, int chunk) { return chunk ^ ((d ^ (d >> 3)) & 7); }

// Key slot order of the transposed V tile.  Register r of an S^T accumulator
// tile holds key 8 * (r / 4) + 4 * g + (r % 4); the P.V product consumes
// registers 8h .. 8h+7, i.e. keys {16h + 4g + 0..3, 16h + 8 + 4g + 0..3}.
// Swapping bits 2 and 3 of the key index places exactly those eight keys in
// consecutive slots 16h + 8g .. 16h + 8g + 7, so one 16-byte LDS read yields
// the matching A operand.
__device__ __forceinline__ int key_slot(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Row of the 32x32 MFMA result held in register r by lane half g.
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---------------------------------------------------------------- relations
// The rows a workgroup owns and the keys they may attend, for one (head,
// sequence, tile) work item.  All bounds are global positions.
struct Span {
    int lo, hi;  // [lo, hi)
};

// Clamped sequence bounds [cu[s], cu[s+1]) within [0, n].
__device__ __forceinline__ Span seq_bounds(const int32_t *cu, int s, int n) {
    int a = cu[s], b = cu[s + 1];
    a = a < 0 ? 0 : (a > n ? n : a);
    b = b < a ? a : (b > n ? n : b);
    return {a, b};
}

}  // namespace osattn
