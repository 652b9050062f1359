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

#include <type_traits>
#include <utility>

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

// max(a, b) as v_maximum*_f32 (NaN-propagating): unlike fmaxf it needs no
// quieting of its inputs, and three-input chains fuse into v_maximum3_f32.
// The kernels' scores are finite or -inf, where the two agree.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// The value of lane l ^ 32 combined with lane l's own, through gfx950's
// v_permlane32_swap (no LDS round trip).  After swapping the upper half of
// one copy of x with the lower half of another, each lane holds x[l] in one
// result and x[l ^ 32] in the other, in an order that depends on the half;
// max and sum are symmetric in the pair.
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
// chunk then hit eight different bank groups.  (Used by the f32 kernels.)
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

// Swizzles of the 16-bit forward tiles for gfx950's 64 x 4-byte LDS banks, where
// a 16-byte-per-lane access is served 16 lanes at a time and must then touch 16
// distinct 16-byte bank groups.
//  - A row of >= 256 bytes spans all banks, so 16 consecutive rows read at one
//    logical chunk need 16 distinct physical chunks: XOR with (row & 15).
//  - A 128-byte row covers half the banks and the next row the other half, so
//    rows of equal parity must differ: XOR with ((row >> 1) & 7).
template <int ROW_BYTES>
__device__ __forceinline__ int swz_k(int row, int chunk) {
    return ROW_BYTES >= 256 ? (chunk ^ (row & 15)) : (chunk ^ ((row >> 1) & 7));
}
// Swizzle of a row-major V tile read by ds_read_b64_tr_b16: 16 lanes read four
// consecutive key rows x 32 bytes, and a wave half reads those rows x 64 bytes.
// XOR-ing the chunk index with a per-row quarter (256-byte rows) or half
// (128-byte rows, whose neighbours sit in the other bank half) puts the four
// rows' windows on disjoint banks.
template <int ROW_BYTES>
__device__ __forceinline__ int swz_vt(int row, int chunk) {
    return ROW_BYTES >= 256 ? (chunk ^ ((row & 3) << 2)) : (chunk ^ (((row >> 1) & 1) << 2));
}

// Swizzle of a 16-bit tile that is read both ways: as MFMA rows with
// ds_read_b128 (16 consecutive rows at one logical chunk) and transposed with
// ds_read_b64_tr_b16 (4 consecutive rows x 2 chunks per 16 lanes).  The XOR
// mask mixes the low row bits into different chunk bits so that both patterns
// touch distinct bank groups (checked exhaustively with a 64-bank model):
// 256-byte rows use ((row & 3) << 2) | ((row >> 2) & 3); 128-byte rows, whose
// neighbours share the bank half, use bits 1, 2, 3 of the row.
template <int ROW_BYTES>
__device__ __forceinline__ int swz_rt(int row, int chunk) {
    return ROW_BYTES >= 256
               ? (chunk ^ (((row & 3) << 2) | ((row >> 2) & 3)))
               : (chunk ^ ((((row >> 1) & 1) << 1) | ((row >> 2) & 1) | (((row >> 3) & 1) << 2)));
}

#define OSATTN_LDS __attribute__((address_space(3)))
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane 4 r + c names 4 consecutive 16-bit elements of row r (columns
// 4c .. 4c+3) of a 4 x 16 block; lane j then receives column j of that block,
// one element per row (verified on the device by a lane-layout probe).
__device__ __forceinline__ i16x4 lds_read_tr16(const void *lds_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((OSATTN_LDS i16x4 *)(lds_addr));
}

// 16 bytes per lane from a raw buffer straight into LDS: lane L writes bytes
// [lds_base + 16 L, lds_base + 16 L + 16); lds_base must be wave-uniform.
// Past-the-end chunks arrive as zeros.  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds_base, int byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (OSATTN_LDS void *)(lds_base), 16, byte_off, 0, 0, 0);
}
// The same with 4 bytes per lane: lane L writes [lds_base + 4 L, + 4).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *lds_base, int byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (OSATTN_LDS void *)(lds_base), 4, byte_off, 0, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt on the LDS/scalar counter only (vmcnt and expcnt at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier without the memory fence __syncthreads() carries (that
// fence would wait for every outstanding LDS DMA, defeating the prefetch).
// Callers order their own LDS traffic with explicit vmcnt / lgkmcnt waits;
// the empty asm keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Four f32 values rounded (RNE) to 16-bit type T and stored as 8 bytes.
template <typename T>
__device__ __forceinline__ void store4_16(T *dst, f32x4 v) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<t4 *>(dst) = __builtin_convertvector(v, t4);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0,
// which is how the kernels guard ragged tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes < 0 ? 0 : (bytes > 0x7ffffff0LL ? 0x7ffffff0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// f(integral_constant<int, I>) for I = 0, 1, ... in order.
template <typename F, int... I>
__device__ __forceinline__ void for_each_index(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

// The four words of a raw buffer resource over [base, base + bytes) (the same
// descriptor make_rsrc builds): loads at or past the end return zeros.  The
// caller passes bytes <= 0x7ffffff0.
__device__ __forceinline__ i32x4 rsrc_words(const void *base, int bytes) {
    const int n = bytes < 0 ? 0 : bytes;
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    // Wave-uniform by construction; readfirstlane lets the compiler see it,
    // so the descriptor sits in scalar registers as the instruction requires.
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(n);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from a raw buffer into LDS bytes [lds + 16 L, +16) of
// lane L; lds is wave-uniform.  Completion is counted by vmcnt only.  As
// inline assembly the copy leaves the ordering of LDS reads to the caller's
// explicit waits and barriers (the compiler would make every LDS read wait for
// every copy in flight).  The s_nop is the one wait state gfx9 requires
// between a scalar write of M0 and an LDS copy that reads it (the compiler
// inserts it for its own copies, not inside inline assembly).
__device__ __forceinline__ void dma16_asm(i32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// The same copy with 4 bytes per lane: lane L writes LDS bytes [lds + 4 L, +4).
__device__ __forceinline__ void dma4_asm(i32x4 rsrc, uint32_t lds, int voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(lds)
                 : "memory");
}

// rsrc_words over [base, base + bytes) with bytes clamped to [0, 0x7ffffff0],
// as make_rsrc clamps them.
__device__ __forceinline__ i32x4 rsrc_words64(const void *base, int64_t bytes) {
    return rsrc_words(base, bytes < 0 ? 0 : (bytes > 0x7ffffff0LL ? 0x7ffffff0 : (int)bytes));
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
