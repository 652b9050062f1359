// Backward attention kernels for gfx950 (f32, feature width 64 or 128).
//
// Method: OCANNL "Module Ir.Online_softmax", third rewrite bullet (the fused
// backward): a per-row D = sum(dO * O), then nests that recompute each pair's
// p, dp and ds = p * (dp - D) from the forward's row state (m, l) -- one over
// the query rows accumulating dQ, one over the keys accumulating dK and dV --
// each owning what it writes.  The mask and the scale act on ds only.  No
// (N_q, N_k) buffer exists at any point.
//
// Kernels, all on one stream:
//   bwd_pre   : D_i = <dO_i, O_i>, m_i log2(e), 1 / l_i             (B0)
//   bwd_dkdv  : a workgroup owns 128 keys (32 per wave, one key per lane
//               column) and scans blocks of 64 queries staged in LDS:
//               S = Q K^T, P, dV += dO^T P, dP = dO V^T, dS, dK += Q^T dS (B1)
//   bwd_dq    : a workgroup owns 128 queries (one per lane column) and scans
//               blocks of 64 keys staged in LDS:
//               S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T      (B2)
//   reduce    : sums the partial gradients of a split reduction in a fixed
//               order (no atomics, bit-reproducible).
// When a problem has too few key (or query) tiles to fill the 256 CUs, the
// dK/dV kernel splits its query range (and the dQ kernel its key range) over
// several workgroups that write f32 partial sums to the workspace.
#include "attn_device.h"

namespace osattn {

constexpr int kBThreads = 256;
constexpr int kBQ = 64;    // query block of the dK/dV scan
constexpr int kBK = 128;   // keys owned by a dK/dV workgroup
constexpr int kBRq = 128;  // queries owned by a dQ workgroup
constexpr int kBCk = 64;   // key block of the dQ scan

// ---------------------------------------------------------------- B0
template <typename T, int D>
__global__ void __launch_bounds__(kBThreads) bwd_pre_kernel(BwdParams p) {
    constexpr int PER = D / 16;  // features per thread; 16 threads per row
    const int64_t total = (int64_t)p.H * p.n_q;
    const int64_t row = (int64_t)blockIdx.x * (kBThreads / 16) + threadIdx.x / 16;
    const int sub = threadIdx.x % 16;
    float acc = 0.f;
    if (row < total) {
        const int h = (int)(row / p.n_q), i = (int)(row % p.n_q);
        const T *dorow = static_cast<const T *>(p.d_o) + (int64_t)h * p.q_sh + (int64_t)i * p.q_sn;
        const float *orow = static_cast<const float *>(p.o) + (int64_t)h * p.o_sh + (int64_t)i * p.o_sn;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            acc += (float)dorow[sub * PER + e] * orow[sub * PER + e];
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (sub == 0 && row < total) {
        p.stat_delta[row] = acc;
        p.stat_mlog2[row] = p.m[row] * kLog2e;
        p.stat_linv[row] = 1.f / p.l[row];
    }
}

struct Range {
    int lo, hi;
};

// Sequence bounds of a work item (whole axis unless varlen).
template <bool VARLEN>
__device__ __forceinline__ Range axis_bounds(const BwdParams &p, int seq, int n) {
    if (!VARLEN) return {0, n};
    const Span s = seq_bounds(p.cu, seq, n);
    return {s.lo, s.hi};
}

// Part `split` of [lo, hi) cut into `splits` pieces aligned to `blk`.
__device__ __forceinline__ Range split_range(int lo, int hi, int split, int splits, int blk) {
    const int len = hi > lo ? hi - lo : 0;
    int chunk = (len + splits - 1) / splits;
    chunk = (chunk + blk - 1) / blk * blk;
    const int a = lo + split * chunk;
    const int b = min(a + chunk, hi);
    return {a, b > a ? b : a};
}

// Store one lane's 32 x 32 transposed accumulator tiles (feature rows, one
// position column) as rows of `out` (f32), scaled.
template <int NDT>
__device__ __forceinline__ void store_rows_f32(float *rowp, const f32x16 (&acc)[NDT], int g,
                                               float scale) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v = {acc[dt][4 * j] * scale, acc[dt][4 * j + 1] * scale,
                       acc[dt][4 * j + 2] * scale, acc[dt][4 * j + 3] * scale};
            *reinterpret_cast<f32x4 *>(rowp + 32 * dt + 8 * j + 4 * g) = v;
        }
}

// Element (acc_row(r, g) + row0, 32 dt + c32) of a swizzled f32 tile of KCH
// 16-byte chunks per row, split as rowoff[r & 3] (per lane) + tile_elem (a
// compile-time constant for unrolled r, dt and row0 a multiple of 8): the
// swizzle XORs the chunk with row & 7 = 4 g + (r & 3), which leaves the 8 dt
// part of the chunk and the rows' multiple of 8 untouched.
template <int KCH>
__device__ __forceinline__ void lane_row_offsets(int (&rowoff)[4], int c32, int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        rowoff[j] = ((4 * g + j) * KCH + ((c32 >> 2) ^ (4 * g + j))) * 4 + (c32 & 3);
}
template <int KCH>
__device__ __forceinline__ constexpr int tile_elem(int row0, int r, int dt) {
    return ((row0 + 8 * (r >> 2)) * KCH + 8 * dt) * 4;
}

// ---------------------------------------------------------------- B1
template <int D, int MASK>
__global__ void __launch_bounds__(kBThreads, 1) bwd_dkdv32_kernel(BwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    constexpr int KCH = D / 4, NJ = D / 8, NQ = D / 2, NDT = D / 32;
    constexpr int LD = kBQ * KCH / kBThreads;
    static_assert(LD * kBThreads == kBQ * KCH, "");

    __shared__ u32x4 sQ[kBQ * KCH];
    __shared__ u32x4 sDO[kBQ * KCH];
    __shared__ float sM[kBQ], sLi[kBQ], sDl[kBQ];

    const int b = blockIdx.x;
    const int h = b % p.H;
    int rest = b / p.H;
    const int split = rest % p.k_splits;
    rest /= p.k_splits;
    int seq = 0;
    if (varlen) {
        seq = rest % p.num_seqs;
        rest /= p.num_seqs;
    }
    const int ktile = rest;
    const Range ks = axis_bounds<varlen>(p, seq, p.n_k);
    const Range qs_all = axis_bounds<varlen>(p, seq, p.n_q);
    const int k_lo = ks.lo + ktile * kBK;
    if (k_lo >= ks.hi) return;
    const int k_hi = min(k_lo + kBK, ks.hi);
    const int qa = causal ? max(qs_all.lo, k_lo) : qs_all.lo;
    const Range qr = split_range(qa, qs_all.hi, split, p.k_splits, kBQ);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, g = lane >> 5;
    const float *qh = static_cast<const float *>(p.q) + (int64_t)h * p.q_sh;
    const float *doh = static_cast<const float *>(p.d_o) + (int64_t)h * p.q_sh;
    const float *kh = static_cast<const float *>(p.k) + (int64_t)h * p.kv_sh;
    const float *vh = static_cast<const float *>(p.v) + (int64_t)h * p.kv_sh;
    const float *st_m = p.stat_mlog2 + (int64_t)h * p.n_q;
    const float *st_li = p.stat_linv + (int64_t)h * p.n_q;
    const float *st_d = p.stat_delta + (int64_t)h * p.n_q;

    // This lane's key (the column of every accumulator) as B operands.
    const int key = k_lo + wave * 32 + c32;
    const bool kok = key < k_hi;
    float kreg[NQ], vreg[NQ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const f32x4 a = __builtin_bit_cast(f32x4, load16(kh + (int64_t)key * p.kv_sn + (D / 2) * g + 4 * j, kok));
        const f32x4 c = __builtin_bit_cast(f32x4, load16(vh + (int64_t)key * p.kv_sn + (D / 2) * g + 4 * j, kok));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kreg[4 * j + e] = a[e];
            vreg[4 * j + e] = c[e];
        }
    }

    u32x4 qpf[LD], dopf[LD];
    float mpf = 0.f, lipf = 0.f, dpf = 0.f;
    auto gload = [&](int q0) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kBThreads, row = id / KCH, ch = id % KCH;
            const int q = q0 + row;
            const bool ok = q < qr.hi;
            qpf[i] = load16(qh + (int64_t)q * p.q_sn + ch * 4, ok);
            dopf[i] = load16(doh + (int64_t)q * p.q_sn + ch * 4, ok);
        }
        if (tid < kBQ) {
            const int q = q0 + tid;
            const bool ok = q < qr.hi;
            mpf = ok ? st_m[q] : 0.f;
            lipf = ok ? st_li[q] : 0.f;  // 0 zeroes P for rows past the range
            dpf = ok ? st_d[q] : 0.f;
        }
    };
    auto lds_store = [&]() {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kBThreads, row = id / KCH, ch = id % KCH;
            sQ[row * KCH + swz(row, ch)] = qpf[i];
            sDO[row * KCH + swz(row, ch)] = dopf[i];
        }
        if (tid < kBQ) {
            sM[tid] = mpf;
            sLi[tid] = lipf;
            sDl[tid] = dpf;
        }
    };

    f32x16 dK[NDT], dV[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        dK[dt] = zero_vec<f32x16>();
        dV[dt] = zero_vec<f32x16>();
    }
    const float c = p.scale_log2;
    const float *sQf = reinterpret_cast<const float *>(sQ);
    const float *sDOf = reinterpret_cast<const float *>(sDO);
    const int nblk = (qr.hi - qr.lo + kBQ - 1) / kBQ;
    int rowoff[4];
    lane_row_offsets<KCH>(rowoff, c32, g);

    if (nblk > 0) gload(qr.lo);
    for (int qb = 0; qb < nblk; ++qb) {
        const int q0 = qr.lo + qb * kBQ;
        __syncthreads();
        lds_store();
        __syncthreads();
        if (qb + 1 < nblk) gload(q0 + kBQ);
#pragma unroll
        for (int qs = 0; qs < kBQ / 32; ++qs) {
            // S = Q K^T: rows = queries of this sub-tile, column = this lane's key.
            f32x16 S = zero_vec<f32x16>();
            const u32x4 *qrow = &sQ[(32 * qs + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, qrow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) S = mma_f32(a[e], kreg[4 * j + e], S);
            }
            // P = exp(scale s - m) / l, zero where the pair is not admitted.
            f32x16 P;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = 32 * qs + acc_row(r, g);
                float pv = fast_exp2(fmaf(S[r], c, -sM[ql])) * sLi[ql];
                if (causal && key > q0 + ql) pv = 0.f;
                P[r] = pv;
            }
            // dV^T += dO^T P
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    dV[dt] = mma_f32(sDOf[rowoff[r & 3] + tile_elem<KCH>(32 * qs, r, dt)], P[r], dV[dt]);
            // dP = dO V^T
            f32x16 dP = zero_vec<f32x16>();
            const u32x4 *dorow = &sDO[(32 * qs + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, dorow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) dP = mma_f32(a[e], vreg[4 * j + e], dP);
            }
            // dS = P (dP - D); dK^T += Q^T dS
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = 32 * qs + acc_row(r, g);
                const float ds = P[r] * (dP[r] - sDl[ql]);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    dK[dt] = mma_f32(sQf[rowoff[r & 3] + tile_elem<KCH>(32 * qs, r, dt)], ds, dK[dt]);
            }
        }
    }

    if (!kok) return;
    if (p.k_splits == 1) {
        store_rows_f32<NDT>(static_cast<float *>(p.dk) + (int64_t)h * p.kv_sh + (int64_t)key * p.kv_sn, dK, g, p.scale);
        store_rows_f32<NDT>(static_cast<float *>(p.dv) + (int64_t)h * p.kv_sh + (int64_t)key * p.kv_sn, dV, g, 1.f);
    } else {
        const int64_t off = (((int64_t)split * p.H + h) * p.n_k + key) * D;
        store_rows_f32<NDT>(p.dk_part + off, dK, g, p.scale);
        store_rows_f32<NDT>(p.dv_part + off, dV, g, 1.f);
    }
}

// ---------------------------------------------------------------- B2
template <int D, int MASK>
__global__ void __launch_bounds__(kBThreads, 1) bwd_dq32_kernel(BwdParams p) {
    constexpr bool causal = MASK == kCausal || MASK == kVarlenCausal;
    constexpr bool varlen = MASK == kVarlen || MASK == kVarlenCausal;
    constexpr int KCH = D / 4, NJ = D / 8, NQ = D / 2, NDT = D / 32;
    constexpr int LD = kBCk * KCH / kBThreads;
    static_assert(LD * kBThreads == kBCk * KCH, "");

    __shared__ u32x4 sK[kBCk * KCH];
    __shared__ u32x4 sV[kBCk * KCH];

    const int b = blockIdx.x;
    const int h = b % p.H;
    int rest = b / p.H;
    const int split = rest % p.q_splits;
    rest /= p.q_splits;
    int seq = 0;
    if (varlen) {
        seq = rest % p.num_seqs;
        rest /= p.num_seqs;
    }
    const int qtile = causal ? (p.q_tiles - 1 - rest) : rest;
    const Range qs_all = axis_bounds<varlen>(p, seq, p.n_q);
    const Range ks_all = axis_bounds<varlen>(p, seq, p.n_k);
    const int q_lo = qs_all.lo + qtile * kBRq;
    if (q_lo >= qs_all.hi) return;
    const int q_hi = min(q_lo + kBRq, qs_all.hi);
    const int kv_hi = causal ? q_hi : ks_all.hi;
    const Range kr = split_range(ks_all.lo, kv_hi, split, p.q_splits, kBCk);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c32 = lane & 31, g = lane >> 5;
    const float *qh = static_cast<const float *>(p.q) + (int64_t)h * p.q_sh;
    const float *doh = static_cast<const float *>(p.d_o) + (int64_t)h * p.q_sh;
    const float *kh = static_cast<const float *>(p.k) + (int64_t)h * p.kv_sh;
    const float *vh = static_cast<const float *>(p.v) + (int64_t)h * p.kv_sh;

    const int qrow = q_lo + wave * 32 + c32;
    const bool qok = qrow < q_hi;
    float qreg[NQ], doreg[NQ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const f32x4 a = __builtin_bit_cast(f32x4, load16(qh + (int64_t)qrow * p.q_sn + (D / 2) * g + 4 * j, qok));
        const f32x4 c = __builtin_bit_cast(f32x4, load16(doh + (int64_t)qrow * p.q_sn + (D / 2) * g + 4 * j, qok));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qreg[4 * j + e] = a[e];
            doreg[4 * j + e] = c[e];
        }
    }
    const int64_t srow = (int64_t)h * p.n_q + qrow;
    const float mlog2 = qok ? p.stat_mlog2[srow] : 0.f;
    const float linv = qok ? p.stat_linv[srow] : 0.f;
    const float dl = qok ? p.stat_delta[srow] : 0.f;

    u32x4 kpf[LD], vpf[LD];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kBThreads, row = id / KCH, ch = id % KCH;
            const int kk = k0 + row;
            const bool ok = kk < kr.hi;
            kpf[i] = load16(kh + (int64_t)kk * p.kv_sn + ch * 4, ok);
            vpf[i] = load16(vh + (int64_t)kk * p.kv_sn + ch * 4, ok);
        }
    };
    auto lds_store = [&]() {
#pragma unroll
        for (int i = 0; i < LD; ++i) {
            const int id = tid + i * kBThreads, row = id / KCH, ch = id % KCH;
            sK[row * KCH + swz(row, ch)] = kpf[i];
            sV[row * KCH + swz(row, ch)] = vpf[i];
        }
    };

    f32x16 dQ[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dQ[dt] = zero_vec<f32x16>();
    const float c = p.scale_log2;
    const float *sKf = reinterpret_cast<const float *>(sK);
    const int nblk = (kr.hi - kr.lo + kBCk - 1) / kBCk;
    int rowoff[4];
    lane_row_offsets<KCH>(rowoff, c32, g);

    if (nblk > 0) gload(kr.lo);
    for (int kb = 0; kb < nblk; ++kb) {
        const int k0 = kr.lo + kb * kBCk;
        __syncthreads();
        lds_store();
        __syncthreads();
        if (kb + 1 < nblk) gload(k0 + kBCk);
#pragma unroll
        for (int s = 0; s < kBCk / 32; ++s) {
            f32x16 S = zero_vec<f32x16>();
            const u32x4 *krow = &sK[(32 * s + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, krow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) S = mma_f32(a[e], qreg[4 * j + e], S);
            }
            f32x16 dP = zero_vec<f32x16>();
            const u32x4 *vrow = &sV[(32 * s + c32) * KCH];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const f32x4 a = __builtin_bit_cast(f32x4, vrow[swz(c32, (D / 8) * g + j)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) dP = mma_f32(a[e], doreg[4 * j + e], dP);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kl = 32 * s + acc_row(r, g);
                const int kk = k0 + kl;
                float pv = fast_exp2(fmaf(S[r], c, -mlog2)) * linv;
                if (kk >= kr.hi || (causal && kk > qrow)) pv = 0.f;
                const float ds = pv * (dP[r] - dl);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    dQ[dt] = mma_f32(sKf[rowoff[r & 3] + tile_elem<KCH>(32 * s, r, dt)], ds, dQ[dt]);
            }
        }
    }

    if (!qok) return;
    if (p.q_splits == 1) {
        store_rows_f32<NDT>(static_cast<float *>(p.dq) + (int64_t)h * p.q_sh + (int64_t)qrow * p.q_sn, dQ, g, p.scale);
    } else {
        const int64_t off = (((int64_t)split * p.H + h) * p.n_q + qrow) * D;
        store_rows_f32<NDT>(p.dq_part + off, dQ, g, p.scale);
    }
}

// ---------------------------------------------------------------- reduce
// Up to three split reductions (dK, dV, dQ) in one launch (Reduce3): each
// thread sums one float4 of its output over the splits in a fixed order
// (deterministic), eight loads in flight.

template <int D>
__global__ void __launch_bounds__(kBThreads) reduce_parts_f32_kernel(Reduce3 q) {
    int64_t b = blockIdx.x;
    const ReduceParams &r = q.r[q.which(b)];
    const int64_t total4 = (int64_t)r.H * r.n * D / 4;
    const int64_t i4 = (int64_t)b * kBThreads + threadIdx.x;
    if (i4 >= total4) return;
    const int64_t e = i4 * 4;
    const int64_t plane = (int64_t)r.n * D;
    const int h = (int)(e / plane);
    const int64_t rem = e % plane;
    const int i = (int)(rem / D), d = (int)(rem % D);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int64_t stride = (int64_t)r.H * plane;
#pragma unroll 8  // eight partial loads in flight (SQ=8192 SK=2048 backward: 155.0 -> 153.9 us)
    for (int s = 0; s < r.splits; ++s)
        acc += *reinterpret_cast<const f32x4 *>(r.part + s * stride + e);
    *reinterpret_cast<f32x4 *>(static_cast<float *>(r.out) + (int64_t)h * r.out_sh + (int64_t)i * r.out_sn + d) = acc;
}

// ------------------------------------------------------------------ launch
template <int D, int MASK>
static void launch_bwd_mask(const BwdParams &p, int grid_k, int grid_q, hipStream_t st) {
    if (grid_k > 0)
        hipLaunchKernelGGL((bwd_dkdv32_kernel<D, MASK>), dim3(grid_k), dim3(kBThreads), 0, st, p);
    if (grid_q > 0)
        hipLaunchKernelGGL((bwd_dq32_kernel<D, MASK>), dim3(grid_q), dim3(kBThreads), 0, st, p);
}

// Adds one reduction to the combined launch.
static void add_reduce(Reduce3 &q, const float *part, void *out, int64_t sh, int64_t sn, int H,
                       int n, int d, int splits) {
    const int64_t grid = ((int64_t)H * n * d / 4 + kBThreads - 1) / kBThreads;
    if (grid <= 0) return;
    q.r[q.count] = ReduceParams{part, out, sh, sn, H, n, splits};
    q.end[q.count] = (q.count ? q.end[q.count - 1] : 0) + grid;
    ++q.count;
}

template <int D>
static void launch_bwd_width(int mask, const BwdParams &p, int grid_k, int grid_q, hipStream_t st) {
    switch (mask) {
        case kDense: launch_bwd_mask<D, kDense>(p, grid_k, grid_q, st); break;
        case kCausal: launch_bwd_mask<D, kCausal>(p, grid_k, grid_q, st); break;
        case kVarlen: launch_bwd_mask<D, kVarlen>(p, grid_k, grid_q, st); break;
        default: launch_bwd_mask<D, kVarlenCausal>(p, grid_k, grid_q, st); break;
    }
}

// Host entry used by the C ABI (arguments and workspace already validated;
// p carries the workspace views and the split plan), d = 64 or 128.
hipError_t launch_backward(int d, int mask, BwdParams p, int seqs, hipStream_t st) {
    const int64_t rows = (int64_t)p.H * p.n_q;
    const int64_t grid_pre = (rows + (kBThreads / 16) - 1) / (kBThreads / 16);
    if (d == 64)
        hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), dim3((unsigned)grid_pre), dim3(kBThreads), 0, st, p);
    else
        hipLaunchKernelGGL((bwd_pre_kernel<float, 128>), dim3((unsigned)grid_pre), dim3(kBThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid_k = (int64_t)p.H * p.k_splits * seqs * p.k_tiles;
    const int64_t grid_q = (int64_t)p.H * p.q_splits * seqs * p.q_tiles;
    if (grid_k > 0x7fffffffLL || grid_q > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (d == 64) launch_bwd_width<64>(mask, p, (int)grid_k, (int)grid_q, st);
    else launch_bwd_width<128>(mask, p, (int)grid_k, (int)grid_q, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    Reduce3 q{};
    if (p.k_splits > 1) {
        add_reduce(q, p.dk_part, p.dk, p.kv_sh, p.kv_sn, p.H, p.n_k, d, p.k_splits);
        add_reduce(q, p.dv_part, p.dv, p.kv_sh, p.kv_sn, p.H, p.n_k, d, p.k_splits);
    }
    if (p.q_splits > 1) add_reduce(q, p.dq_part, p.dq, p.q_sh, p.q_sn, p.H, p.n_q, d, p.q_splits);
    if (q.count > 0) {
        if (q.end[q.count - 1] > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)q.end[q.count - 1]);
        if (d == 64) hipLaunchKernelGGL((reduce_parts_f32_kernel<64>), grid, dim3(kBThreads), 0, st, q);
        else hipLaunchKernelGGL((reduce_parts_f32_kernel<128>), grid, dim3(kBThreads), 0, st, q);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace osattn
